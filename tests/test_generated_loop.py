"""Host checks of the generated forward tile loop (csrc/attn_fwd_loop.inc).

The loop is one inline-asm block written by csrc/gen_attn_loop.py. These CPU
tests pin what the compiler cannot check for hand-written asm: the committed
file is the generator's current output, every register the block names is one
it declares (an operand or a clobber), and every branch target exists.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "transformer_scaled_dot_mha_amd", "csrc")
sys.path.insert(0, CSRC)

import gen_attn_loop as gen  # noqa: E402


def _inc_text():
    with open(os.path.join(CSRC, "attn_fwd_loop.inc")) as f:
        return f.read()


def test_committed_loop_matches_generator():
    r = subprocess.run([sys.executable, os.path.join(CSRC, "gen_attn_loop.py"), "--check"], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr


def _split(txt):
    body = [ln.strip()[1:-3] for ln in txt.splitlines() if ln.strip().startswith('"') and ln.strip().endswith('\\n"')]
    tail = txt[txt.index('      : "+'):]
    return body, tail


def _expand(tok):
    m = re.fullmatch(r"([vas])\[(\d+):(\d+)\]", tok)
    if m:
        return {f"{m.group(1)}{i}" for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    return {tok}


def _declared(tail):
    regs = set()
    for tok in re.findall(r'"\+?\{([^}]+)\}"', tail):
        regs |= _expand(tok)
    for tok in re.findall(r'"([vs]\d+)"', tail):
        regs.add(tok)
    return regs


def _used(body):
    regs = set()
    for ln in body:
        if ln.endswith(":"):
            continue
        for tok in re.findall(r"\b[vas]\[\d+:\d+\]|\b[vas]\d+\b", ln):
            regs |= _expand(tok)
    return regs


def test_loop_names_only_declared_registers():
    for o_agpr in (False, True):
        body, tail = _split(gen.generate(o_agpr))
        undeclared = _used(body) - _declared(tail)
        assert not undeclared, sorted(undeclared)


def test_loop_branch_targets_exist():
    body, _ = _split(_inc_text())
    labels = {ln[:-1] for ln in body if ln.endswith(":")}
    targets = {ln.split()[-1] for ln in body if ln.startswith("s_cbranch") or ln.startswith("s_branch")}
    assert targets <= labels, sorted(targets - labels)
    # every step that checks a reference has its cold path and its way back
    for ln in body:
        if "_rare" in ln and ln.startswith("s_cbranch_vccnz"):
            tgt = ln.split()[-1]
            assert tgt in labels


def _operands(ln):
    """(destination registers, source registers) of one instruction."""
    parts = [p.strip() for p in ln.split(None, 1)[1].split(",")] if len(ln.split(None, 1)) > 1 else []
    regs = [set().union(*[_expand(t) for t in re.findall(r"\b[va]\[\d+:\d+\]|\b[va]\d+\b", p)] or [set()])
            for p in parts]
    if not regs:
        return set(), set()
    return regs[0], set().union(*regs[1:]) if len(regs) > 1 else set()


def test_loop_wait_states():
    """Along the straight-line text, no instruction reads a register sooner than
    gfx950 allows: 12 wait states after a 32x32x16 product and 8 after a
    16x16x32 one before a VALU read, 2 after a VALU write before a matrix-core
    read, 1 after a transcendental before a VALU read (instructions and s_nop
    lengths counted; the check restarts at each label)."""
    body, _ = _split(_inc_text())
    pending = []  # (registers written, wait states still needed, reader kind: "valu" | "mfma")
    for ln in body:
        if ln.endswith(":"):
            pending = []
            continue
        op = ln.split()[0]
        if op.startswith("s_branch") or op.startswith("s_cbranch"):
            continue
        dst, src = _operands(ln) if op.startswith("v_") else (set(), set())
        kind = "mfma" if op.startswith("v_mfma") else ("valu" if op.startswith("v_") else None)
        if kind == "mfma":
            src = src | dst  # the accumulator operand is read too
        for regs, need, reader in pending:
            if reader == kind and need > 0:
                assert not (regs & src), ln
        n = int(ln.split()[1]) + 1 if op == "s_nop" else 1
        pending = [(r, w - n, k) for r, w, k in pending if w - n > 0]
        if kind == "mfma":
            pending.append((dst, 12 if "32x32x16" in op else 8, "valu"))
        elif kind == "valu":
            pending.append((dst, 2, "mfma"))
            if op.startswith("v_exp"):
                pending.append((dst, 1, "valu"))
