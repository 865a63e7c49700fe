#!/usr/bin/env python3
"""Writes attn_fwd_loop.inc: the steady-state tile loop of the 64-row forward
attention kernel (attn_bf16.hip) as one hand-scheduled gfx950 asm block.

    python gen_attn_loop.py            # rewrite attn_fwd_loop.inc next to this file
    python gen_attn_loop.py --check    # exit 1 if the committed file differs

What the loop computes is the kernel's own unmasked tile step, unchanged
(the attention equation of "The Transformer" (hoshank.vercel.app), "The
Mathematics", over streamed key tiles with a running softmax reference): per
32-key slab and 32-query block, S^T = K Q^T on the matrix core, the bf16
weights exp2(s*c - m*c), their row sum on the matrix core (a 0/1 selector
times the weights), the reference check (row sum <= 2^8) and O^T += V^T P^T.
Only the issue order is new, and it is fixed here instead of left to the
compiler: the wavefront walks "units" u = (block, slab) in the order A0 B0 A1
B1 ..., and step u issues
    the 4 S^T products of unit u+1, each followed by one pair of unit u's
      weights (2 fma, 2 exp, 1 pack; software-pipelined by two slots),
    unit u-1's reference check and row-sum update,
    the 4 P V products of unit u-1, each followed by one more pair,
    unit u's two row-sum products,
    and this step's LDS fragment reads, tile sync and tile DMA.
So every matrix-core instruction is followed by about its own duration of
independent VALU work from the same wavefront, and no instruction waits on a
result issued less than a few slots earlier.

Registers are fixed (asm operand constraints), so the loop needs no copies:
    v[0:63]    O^T accumulators, blocks A/B x d blocks 0/1     (in/out)
    v[64:95]   Q^T fragments, blocks A/B x 4 k steps           (in)
    v[96:127]  K fragments, 2 slab buffers x 4 k steps
    v[128:159] V^T fragments, 2 slab buffers x (2 x 2)
    v[160:191] scores of block A / block B (16 each)
    v[192:207] bf16 weights of block A / block B (8 each)
    v[208:211] row-sum accumulator;  v[212:215] 0/1 selector (in)
    v216..v221 m, m*c, l of blocks A/B (in/out)
    v[222:225] K fragment LDS addresses, v226 V (in);  v227..v230 DMA offsets (in)
    v231, v232 temporaries of the rare path
    s64..s77   loop scalars (in), s[80:87] tile descriptors, s88, s89 temporaries
Wait states follow the gfx950 rules the compiler applies to the same
instructions (12 after a 32x32x16 product before a VALU read, 8 after a
16x16x32 one, 2 after a VALU write before a matrix-core read, 1 after a
transcendental); the schedule keeps producers and consumers further apart
than that, and explicit s_nop covers the few places where it does not.
"""
from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "attn_fwd_loop.inc")

# ---- register map -------------------------------------------------------
O_AGPR = False   # O^T accumulators in the accumulation registers (a0..a63) instead of v0..v63


def set_map(o_agpr=False):
    """Fix the register numbers; with o_agpr the O^T accumulators live in
    a[0:63] and every other vector register moves down by 64."""
    global O_AGPR, O, Q, KB, VB, S, PW, RS, SEL, M, MC, L, KL, VL, DK, DV, T0, T1
    O_AGPR = o_agpr
    b = -64 if o_agpr else 0
    O = {("A", 0): 0, ("A", 1): 16, ("B", 0): 32, ("B", 1): 48}
    Q = {"A": 64 + b, "B": 80 + b}
    KB = [96 + b, 112 + b]
    VB = [128 + b, 144 + b]
    S = {"A": 160 + b, "B": 176 + b}
    PW = {"A": 192 + b, "B": 200 + b}
    RS = 208 + b
    SEL = 212 + b
    M = {"A": 216 + b, "B": 217 + b}
    MC = {"A": 218 + b, "B": 219 + b}
    L = {"A": 220 + b, "B": 221 + b}
    KL = 222 + b
    VL = 226 + b
    DK = [227 + b, 228 + b]
    DV = [229 + b, 230 + b]
    T0, T1 = 231 + b, 232 + b


set_map()
S_C, S_T, S_TLAST, S_NT, S_KREM, S_KSN2, S_VSN2, S_KSTEP, S_VSTEP, S_LDSW = range(64, 74)
S_KBLO, S_KBHI, S_VBLO, S_VBHI = 74, 75, 76, 77
S_KD, S_VD = 80, 84
S_X, S_Y = 88, 89

STAGE_BYTES = 16384
ROW_BYTES = 128
MAX_SUM = "0x43800000"  # 256.0 = 2^8


def v(i):
    return f"v{i}"


def vr(i, n):
    return f"v[{i}:{i + n - 1}]"


def mfma32(d, a, b, c):
    return f"v_mfma_f32_32x32x16_bf16 {vr(d, 16)}, {vr(a, 4)}, {vr(b, 4)}, {c}"


def other(x):
    return "B" if x == "A" else "A"


class Emitter:
    def __init__(self):
        self.lines = []

    def __call__(self, *ins):
        self.lines.extend(ins)

    def label(self, name):
        self.lines.append(f"{name}:")


# ---- pieces -------------------------------------------------------------
def pair_ops(x, i, what):
    """One stage of weight pair i of block x: 'f' = scale and shift (fma),
    'e' = exp2, 'c' = pack the two weights to bf16."""
    s0, s1 = S[x] + 2 * i, S[x] + 2 * i + 1
    if what == "f":
        return [f"v_fma_f32 {v(s0)}, {v(s0)}, s{S_C}, -{v(MC[x])}",
                f"v_fma_f32 {v(s1)}, {v(s1)}, s{S_C}, -{v(MC[x])}"]
    if what == "e":
        return [f"v_exp_f32_e32 {v(s0)}, {v(s0)}", f"v_exp_f32_e32 {v(s1)}, {v(s1)}"]
    return [f"v_cvt_pk_bf16_f32 {v(PW[x] + i)}, {v(s0)}, {v(s1)}"]


def slot_pairs(x, j):
    """Weight work issued after matrix-core slot j (0..7): fma of pair j, exp
    of pair j-1, pack of pair j-2."""
    ops = []
    if j - 2 >= 0:
        ops += pair_ops(x, j - 2, "c")
    if j - 1 >= 0:
        ops += pair_ops(x, j - 1, "e")
    ops += pair_ops(x, j, "f")
    return ops


def finish_pairs(x):
    """All weight work of block x that slots 4..7 and the tail would have done
    (by the check, slots 0..3 have issued fma 0..3, exp 0..2 and pack 0..1)."""
    ops = []
    ops += pair_ops(x, 3, "e")
    for i in range(4, 8):
        ops += pair_ops(x, i, "f")
    ops += ["s_nop 1"]
    ops += pair_ops(x, 2, "c") + pair_ops(x, 3, "c")
    for i in range(4, 8):
        ops += pair_ops(x, i, "e")
    ops += ["s_nop 0"]
    for i in range(4, 8):
        ops += pair_ops(x, i, "c")
    return ops


def rowsum_mfmas(x):
    return [f"v_mfma_f32_16x16x32_bf16 {vr(RS, 4)}, {vr(SEL, 4)}, {vr(PW[x], 4)}, 0",
            f"v_mfma_f32_16x16x32_bf16 {vr(RS, 4)}, {vr(SEL, 4)}, {vr(PW[x] + 4, 4)}, {vr(RS, 4)}"]


def k_reads(kbuf, stage, slab):
    base = stage * STAGE_BYTES + slab * 32 * ROW_BYTES
    return [f"ds_read_b128 {vr(KB[kbuf] + 4 * kk, 4)}, {v(KL + kk)} offset:{base}" for kk in range(4)]


def v_reads(vbuf, stage, slab):
    ops = []
    for jj in range(2):
        for blk in range(2):
            idx = 2 * jj + blk
            base = stage * STAGE_BYTES + (32 * slab + 16 * jj) * ROW_BYTES
            ops.append(f"ds_read_b64_tr_b16 {vr(VB[vbuf] + 4 * idx, 2)}, {v(VL)} offset:{base + 64 * blk}")
            ops.append(f"ds_read_b64_tr_b16 {vr(VB[vbuf] + 4 * idx + 2, 2)}, {v(VL)} offset:"
                       f"{base + 4 * ROW_BYTES + 64 * (blk ^ 1)}")
    return ops


def oreg(i, n=16):
    return f"a[{i}:{i + n - 1}]" if O_AGPR else vr(i, n)


def pv_mfma(y, vbuf, i):
    jj, blk = i >> 1, i & 1
    o = O[(y, blk)]
    return (f"v_mfma_f32_32x32x16_bf16 {oreg(o)}, {vr(VB[vbuf] + 4 * (2 * jj + blk), 4)}, "
            f"{vr(PW[y] + 4 * jj, 4)}, {oreg(o)}")


def s_mfma(xn, kbuf, kk):
    return mfma32(S[xn], KB[kbuf] + 4 * kk, Q[xn] + 4 * kk, "0" if kk == 0 else vr(S[xn], 16))


def dma_tile(stage):
    """DMA of the next tile (4 loads per wavefront) into `stage`; the caller
    has checked that the tile exists."""
    ops = [
        f"s_min_i32 s{S_X}, s{S_KREM}, 64",
        f"s_add_i32 s{S_X}, s{S_X}, -1",
        f"s_mul_i32 s{S_Y}, s{S_X}, s{S_KSN2}",
        f"s_add_u32 s{S_KD + 2}, s{S_Y}, 0x80",
        f"s_mul_i32 s{S_Y}, s{S_X}, s{S_VSN2}",
        f"s_add_u32 s{S_VD + 2}, s{S_Y}, 0x80",
        f"s_mov_b32 s{S_KD}, s{S_KBLO}",
        f"s_and_b32 s{S_KD + 1}, s{S_KBHI}, 0xffff",
        f"s_mov_b32 s{S_KD + 3}, 0x20000",
        f"s_mov_b32 s{S_VD}, s{S_VBLO}",
        f"s_and_b32 s{S_VD + 1}, s{S_VBHI}, 0xffff",
        f"s_mov_b32 s{S_VD + 3}, 0x20000",
    ]
    base = stage * STAGE_BYTES
    for i in range(2):
        ops += [f"s_add_u32 m0, s{S_LDSW}, {base + 1024 * i}", "s_nop 0",
                f"buffer_load_dwordx4 {v(DK[i])}, s[{S_KD}:{S_KD + 3}], 0 offen lds",
                f"s_add_u32 m0, s{S_LDSW}, {base + 8192 + 1024 * i}", "s_nop 0",
                f"buffer_load_dwordx4 {v(DV[i])}, s[{S_VD}:{S_VD + 3}], 0 offen lds"]
    ops += [
        f"s_add_u32 s{S_KBLO}, s{S_KBLO}, s{S_KSTEP}",
        f"s_addc_u32 s{S_KBHI}, s{S_KBHI}, 0",
        f"s_add_u32 s{S_VBLO}, s{S_VBLO}, s{S_VSTEP}",
        f"s_addc_u32 s{S_VBHI}, s{S_VBHI}, 0",
        f"s_sub_i32 s{S_KREM}, s{S_KREM}, 64",
    ]
    return ops


def tile_sync(stage, uid):
    """Sync before the next tile's first fragment read (skipped on the last
    tile): this wavefront's DMA of tile t+1 has landed (the loads of tiles t+2
    and t+3 that exist may still be in flight), every LDS read is done, then
    all wavefronts meet; then the DMA of tile t+4 into this tile's stage."""
    return [
        f"s_sub_i32 s{S_X}, s{S_NT}, s{S_T}",
        f"s_cmp_ge_i32 s{S_X}, 4",
        f"s_cbranch_scc1 {uid}_w8",
        f"s_cmp_eq_i32 s{S_X}, 3",
        f"s_cbranch_scc1 {uid}_w4",
        "s_waitcnt vmcnt(0)",
        f"s_branch {uid}_wd",
        f"{uid}_w4:",
        "s_waitcnt vmcnt(4)",
        f"s_branch {uid}_wd",
        f"{uid}_w8:",
        "s_waitcnt vmcnt(8)",
        f"{uid}_wd:",
        "s_waitcnt lgkmcnt(0)",
        "s_barrier",
        f"s_cmp_lt_i32 s{S_X}, 5",
        f"s_cbranch_scc1 {uid}_nodma",
    ] + dma_tile(stage) + [f"{uid}_nodma:"]


def rare_fix(e, y, kbuf_prev, tmp_scores, back):
    """The reference check of block y's last unit failed: form that unit's
    scores again into `tmp_scores` (16 free registers), move the reference to
    the row maximum where it grew (rescaling O and l of those rows), form the
    unit's weights and row sum again, and return to `back`."""
    sx = tmp_scores
    e(*[mfma32(sx, KB[kbuf_prev] + 4 * kk, Q[y] + 4 * kk, "0" if kk == 0 else vr(sx, 16)) for kk in range(4)])
    e("s_nop 7", "s_nop 7")
    e(f"v_max3_f32 {v(T0)}, {v(sx)}, {v(sx + 1)}, {v(sx + 2)}")
    for r in range(3, 15, 2):
        e(f"v_max3_f32 {v(T0)}, {v(T0)}, {v(sx + r)}, {v(sx + r + 1)}")
    e(f"v_max_f32_e32 {v(T0)}, {v(T0)}, {v(sx + 15)}")
    e(f"v_mov_b32_e32 {v(T1)}, {v(T0)}", "s_nop 1",
      f"v_permlane32_swap_b32_e32 {v(T0)}, {v(T1)}", "s_nop 1",
      f"v_max_f32_e32 {v(T0)}, {v(T0)}, {v(T1)}")
    # m_new = max(m, row max); where m_new > m: alpha = (m == -inf ? 0 : exp2(m*c - m_new*c)),
    # O and l scale by alpha, m = m_new, m*c = m_new*c; elsewhere nothing changes (alpha = 1)
    p0 = PW[y]
    e(f"v_max_f32_e32 {v(T0)}, {v(M[y])}, {v(T0)}",
      f"v_mul_f32_e32 {v(T1)}, s{S_C}, {v(T0)}",
      f"v_fma_f32 {v(p0)}, -s{S_C}, {v(T0)}, {v(MC[y])}",  # m*c - m_new*c, one rounding
      f"v_exp_f32_e32 {v(p0)}, {v(p0)}",
      "s_nop 0",
      f"v_cmp_eq_f32_e32 vcc, 0xff800000, {v(M[y])}",
      f"v_cndmask_b32_e64 {v(p0)}, {v(p0)}, 0, vcc",
      f"v_cmp_gt_f32_e32 vcc, {v(T0)}, {v(M[y])}",
      f"v_cndmask_b32_e64 {v(p0)}, 1.0, {v(p0)}, vcc",
      f"v_cndmask_b32_e32 {v(M[y])}, {v(M[y])}, {v(T0)}, vcc",
      f"v_cndmask_b32_e32 {v(MC[y])}, {v(MC[y])}, {v(T1)}, vcc")
    for blk in range(2):
        for r in range(16):
            o = O[(y, blk)] + r
            if O_AGPR:
                e(f"v_accvgpr_read_b32 {v(T1)}, a{o}", "s_nop 1", f"v_mul_f32_e32 {v(T1)}, {v(T1)}, {v(p0)}",
                  f"v_accvgpr_write_b32 a{o}, {v(T1)}")
            else:
                e(f"v_mul_f32_e32 {v(o)}, {v(o)}, {v(p0)}")
    e(f"v_mul_f32_e32 {v(L[y])}, {v(L[y])}, {v(p0)}")
    # the unit's weights against the new reference
    for i in range(8):
        s0, s1 = sx + 2 * i, sx + 2 * i + 1
        e(f"v_fma_f32 {v(s0)}, {v(s0)}, s{S_C}, -{v(MC[y])}",
          f"v_fma_f32 {v(s1)}, {v(s1)}, s{S_C}, -{v(MC[y])}")
    for i in range(8):
        s0, s1 = sx + 2 * i, sx + 2 * i + 1
        e(f"v_exp_f32_e32 {v(s0)}, {v(s0)}", f"v_exp_f32_e32 {v(s1)}, {v(s1)}")
    e("s_nop 0")
    for i in range(8):
        e(f"v_cvt_pk_bf16_f32 {v(PW[y] + i)}, {v(sx + 2 * i)}, {v(sx + 2 * i + 1)}")
    e("s_nop 1")
    e(f"v_mfma_f32_16x16x32_bf16 {vr(RS, 4)}, {vr(SEL, 4)}, {vr(PW[y], 4)}, 0",
      f"v_mfma_f32_16x16x32_bf16 {vr(RS, 4)}, {vr(SEL, 4)}, {vr(PW[y] + 4, 4)}, {vr(RS, 4)}",
      "s_nop 7", "s_nop 3")
    e(f"s_branch {back}")


# unit layout inside a tile: position p -> (block of u, block/K buffer of u+1, block/V buffer of u-1)
def unit_info(p):
    x = "A" if p % 2 == 0 else "B"
    y = other(x)
    kbuf_next = {0: 0, 1: 1, 2: 1, 3: 0}[p]      # K buffer of unit u+1's slab
    vbuf_prev = {0: 1, 1: 0, 2: 0, 3: 1}[p]      # V buffer of unit u-1's slab
    kbuf_prev = {0: 1, 1: 0, 2: 0, 3: 1}[p]      # K buffer of unit u-1's slab (the rare path)
    return x, y, kbuf_next, vbuf_prev, kbuf_prev


def step(e, cold, stage, p, kind):
    """One step. kind: 'reg' (regular), 'first' (the loop's first unit: no
    unit u-1), 'last' (p = 3 of the last tile: no unit u+1, no next tile)."""
    x, y, kbuf_next, vbuf_prev, kbuf_prev = unit_info(p)
    uid = f"L%=_s{stage}p{p}{kind[0]}"
    has_prev = kind != "first"
    has_next = not (kind == "last")
    if p in (1, 3):
        e("s_waitcnt lgkmcnt(0)")
    # slots 0..3: S^T of unit u+1, weights of unit u
    for j in range(4):
        if has_next:
            e(s_mfma(y, kbuf_next, j))
        e(*slot_pairs(x, j))
    if has_prev:
        e(f"v_cmp_nge_f32_e32 vcc, {MAX_SUM}, {v(RS)}",
          f"s_cbranch_vccnz {uid}_rare")
    def loads_and_sync():
        ops = []
        if p == 0:
            ops += k_reads(1, stage, 1)
        elif p == 1:
            ops += v_reads(1, stage, 1)
        elif p == 2:
            ops += [f"s_cmp_eq_u32 s{S_T}, s{S_TLAST}", f"s_cbranch_scc1 {uid}_skip"]
            ops += tile_sync(stage, uid)
            ops += k_reads(0, (stage + 1) % 4, 0)
            ops += [f"{uid}_skip:"]
        elif p == 3 and has_next:
            ops += v_reads(0, (stage + 1) % 4, 0)
        return ops

    post = loads_and_sync()
    if has_prev:
        e(f"v_add_f32_e32 {v(L[y])}, {v(L[y])}, {v(RS)}")
    # slots 4..7: P V of unit u-1, more weights of unit u
    for j in range(4, 8):
        if has_prev:
            e(pv_mfma(y, vbuf_prev, j - 4))
        e(*slot_pairs(x, j))
        if j == 4 and p != 2:
            e(*post)  # the fragment reads go early; p = 2's sync waits until after the row sums
    # tail: last weights, then the row-sum products of unit u
    e(*pair_ops(x, 7, "e"))
    e(*pair_ops(x, 6, "c"))
    e(rowsum_mfmas(x)[0])
    e(*pair_ops(x, 7, "c"))
    e("s_nop 1")
    e(rowsum_mfmas(x)[1])
    e(f"{uid}_post:")
    if p == 2:
        e(*post)
    # cold path: the check of unit u-1 failed
    if has_prev:
        cold.label(f"{uid}_rare")
        cold(*finish_pairs(x))
        rare_fix(cold, y, kbuf_prev, S[x], f"{uid}_cont")
        cold.label(f"{uid}_cont")
        cold(f"v_add_f32_e32 {v(L[y])}, {v(L[y])}, {v(RS)}")
        for j in range(4):
            cold(pv_mfma(y, vbuf_prev, j))
        if p != 2:
            cold(*post)
        cold("s_nop 1")
        cold(*rowsum_mfmas(x))
        cold(f"s_branch {uid}_post")


def generate(o_agpr: bool = False) -> str:
    set_map(o_agpr)
    e, cold = Emitter(), Emitter()
    # ---- prologue: fragments of tile 1 slab 0, the scores of unit A of that slab
    e(*k_reads(0, 1, 0))
    e(*v_reads(0, 1, 0))
    e("s_waitcnt lgkmcnt(0)")
    for kk in range(4):
        e(s_mfma("A", 0, kk))
    e("s_nop 7", "s_nop 3")
    # first step (tile 1 is in stage 1): no unit u-1
    step(e, cold, 1, 0, "first")
    e("s_branch L%=_s1p1")
    # ---- the loop: tiles in stage order 1, 2, 3, 0
    e.label("L%=_top")
    for stage in (1, 2, 3, 0):
        for p in range(4):
            e.label(f"L%=_s{stage}p{p}")
            if p == 3:
                e(f"s_cmp_eq_u32 s{S_T}, s{S_TLAST}", f"s_cbranch_scc1 L%=_s{stage}p3l_entry")
            step(e, cold, stage, p, "reg")
        e(f"s_add_u32 s{S_T}, s{S_T}, 1")
    e("s_branch L%=_top")
    for stage in (1, 2, 3, 0):
        e.label(f"L%=_s{stage}p3l_entry")
        step(e, cold, stage, 3, "last")
        e("s_branch L%=_epi")
    # ---- epilogue: check and P V of the last unit (block B)
    e.label("L%=_epi")
    e("s_nop 7", "s_nop 3")
    e(f"v_cmp_nge_f32_e32 vcc, {MAX_SUM}, {v(RS)}", "s_cbranch_vccnz L%=_epi_rare")
    e.label("L%=_epi_cont")
    e(f"v_add_f32_e32 {v(L['B'])}, {v(L['B'])}, {v(RS)}")
    for j in range(4):
        e(pv_mfma("B", 1, j))
    e("s_nop 7", "s_nop 7", "s_nop 3")
    e("s_branch L%=_end")
    cold.label("L%=_epi_rare")
    rare_fix(cold, "B", 1, S["A"], "L%=_epi_cont")
    body = e.lines + cold.lines + ["L%=_end:"]

    clob_v = [v(i) for i in range(KB[0], RS + 4)] + [v(T0), v(T1)]
    clob_s = [f"s{i}" for i in list(range(S_KD, S_KD + 8)) + [S_X, S_Y]]
    ofile = "a" if O_AGPR else "v"

    def pin(r, n=1):
        return f"{{v{r}}}" if n == 1 else f"{{v[{r}:{r + n - 1}]}}"
    out = []
    out.append("// Generated by gen_attn_loop.py; do not edit by hand.")
    out.append("// The steady-state tile loop of attn_fwd_bf16_d64_r64 (unmasked tiles 1 .. t_last),")
    out.append("// hand-scheduled; see the generator's docstring for the schedule and register map.")
    out.append("__device__ __forceinline__ void fwd_loop_asm(f32x16& oa0, f32x16& oa1, f32x16& ob0, f32x16& ob1,")
    out.append("    float& ma, float& mb, float& mca, float& mcb, float& la, float& lb, u32x4 (&qf)[2][4],")
    out.append("    u32x4& sel, u32x4 kl, unsigned vl, unsigned dk0, unsigned dk1, unsigned dv0, unsigned dv1,")
    out.append("    float c, int t_last, int ntiles, int krem, int ksn2, int vsn2, unsigned kstep, unsigned vstep,")
    out.append("    unsigned ldsw, unsigned kb_lo, unsigned kb_hi, unsigned vb_lo, unsigned vb_hi) {")
    out.append("  int m0_dummy = 0;")
    out.append("  int t_first = 1;")
    out.append("  asm volatile(")
    for ln in body:
        out.append('      "' + ln + '\\n"')
    out.append("      : " + ", ".join(f'"+{{{ofile}[{O[k]}:{O[k] + 15}]}}"({n})' for k, n in
                                    ((("A", 0), "oa0"), (("A", 1), "oa1"), (("B", 0), "ob0"), (("B", 1), "ob1"))) + ",")
    out.append("        " + ", ".join(f'"+{pin(r)}"({n})' for r, n in ((M["A"], "ma"), (M["B"], "mb"), (MC["A"], "mca"),
                                                                       (MC["B"], "mcb"), (L["A"], "la"), (L["B"], "lb"))) + ",")
    out.append('        "+{m0}"(m0_dummy), "+{s65}"(t_first), "+{s68}"(krem), "+{s74}"(kb_lo), "+{s75}"(kb_hi),')
    out.append(f'        "+{{s76}}"(vb_lo), "+{{s77}}"(vb_hi), "+{pin(SEL, 4)}"(sel),')
    out.append("        " + ", ".join(f'"+{pin(Q["A"] + 4 * i, 4)}"(qf[{i // 4}][{i % 4}])' for i in range(8)))
    out.append(f'      : "{pin(KL, 4)}"(kl), "{pin(VL)}"(vl), "{pin(DK[0])}"(dk0), "{pin(DK[1])}"(dk1), '
               f'"{pin(DV[0])}"(dv0), "{pin(DV[1])}"(dv1),')
    out.append('        "{s64}"(c), "{s66}"(t_last), "{s67}"(ntiles), "{s69}"(ksn2), "{s70}"(vsn2), "{s71}"(kstep),')
    out.append('        "{s72}"(vstep), "{s73}"(ldsw)')
    out.append("      : " + ", ".join(f'"{r}"' for r in clob_v + clob_s) + ', "vcc", "scc", "memory");')
    out.append("}")
    return "\n".join(out) + "\n"


def main(argv):
    txt = generate()
    if "--check" in argv:
        with open(OUT) as f:
            if f.read() != txt:
                print(f"{OUT} is stale: run {os.path.basename(__file__)}", file=sys.stderr)
                return 1
        return 0
    with open(OUT, "w") as f:
        f.write(txt)
    print(f"wrote {OUT}: {txt.count(chr(10))} lines")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
