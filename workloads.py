"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws and stores numbers. It holds none of the attention
arithmetic: no products, no softmax, no masking. Both the fp64 oracle and the
HIP path receive exactly the arrays produced here, so any disagreement between
them is compute error, never input error.

Shapes follow the pages' base model (d_model = 512, h = 8, d_k = d_v = 64;
"The Transformer", hoshank.vercel.app, "The Mathematics", symbol tables under
the Attention and MultiHead equations) and the big model's head count for the
long causal case (width 1024 with 16 heads, same section). Values are unit
normal, the variance that the scale argument assumes ("32 Transformer",
ml-canon-en.vercel.app, "Why we divide by sqrt(dk)"). Projection weights are
N(0, 1/d_model) so that the projected Q, K and V stay unit variance.

Recipe, per workload: ``numpy.random.default_rng(seed)`` (PCG64), tensors drawn
in the listed order as float64 ``standard_normal``, weights multiplied by
1/sqrt(d_model), then stored as float32 (fp32 workloads) or rounded to bf16
with round-to-nearest-even (bf16 workloads).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "mha": projections + attention + W^O;  "attn": attention core only;
                         # "layer": a whole encoder layer (attention sub-layer, FFN, two residual norms);
                         # "decode": one query per (batch, head) against a K/V cache of n_k slots;
                         # "bwd": the attention backward (dQ, dK, dV for a given dO)
    dtype: str           # "f32" or "bf16": the stored type of every tensor
    batch: int
    heads: int
    n_q: int
    n_k: int
    d_k: int
    causal: bool
    seed: int
    d_model: int = 0     # mha workloads only
    oracle_rows: int = 0  # >0: the oracle checks this many sampled query positions
    kv_len_range: tuple = ()  # (lo, hi): per-batch key lengths drawn uniformly in [lo, hi] (padding mask)
    d_ff: int = 0        # layer workloads only: FFN inner width
    page_size: int = 0   # decode workloads: key slots per cache page (0: one contiguous cache per sequence)

    def kv_lengths(self):
        """Per-batch key lengths of a padded workload (None if unpadded), from
        their own generator ``default_rng(2000 + seed)`` so that the tensors'
        draws do not depend on them."""
        if not self.kv_len_range:
            return None
        lo, hi = self.kv_len_range
        return np.random.default_rng(2000 + self.seed).integers(lo, hi + 1, size=self.batch).astype(np.int32)

    def pages(self):
        """(block_table, num_pages) of a paged decode workload: page_table over
        the key lengths with its own generator seed 3000 + seed."""
        return page_table(self.kv_lengths(), self.page_size, self.n_k // self.page_size, seed=3000 + self.seed)

    @property
    def d_v(self) -> int:
        return self.d_k

    def attention_pairs(self) -> int:
        """Unmasked (query, key) pairs per (batch, head); for a padded workload,
        the mean over the batch items of their own counts times the batch
        (attention_flops uses the exact total)."""
        return self.total_pairs() // self.batch

    def total_pairs(self) -> int:
        """Unmasked (query, key) pairs summed over the batch, per head."""
        lens = self.kv_lengths()
        if lens is None:
            lens = np.full(self.batch, self.n_k)
        tot = 0
        for L in lens:
            L = int(min(max(L, 0), self.n_k))
            if self.causal:
                # query i sees keys j <= min(i, L - 1)
                tot += L * (L + 1) // 2 + (self.n_q - L) * L if L <= self.n_q else self.n_q * (self.n_q + 1) // 2
            else:
                tot += self.n_q * L
        return tot

    def attention_flops(self) -> int:
        """4 * H * d * (unmasked pairs over the batch): QK^T and PV, two flops per multiply-add."""
        return 4 * self.heads * self.d_k * self.total_pairs()

    def backward_flops(self) -> int:
        """10 * H * d * (unmasked pairs): the five products of the gradient (dV = P^T dO,
        dP = dO V^T, dQ = dS K, dK = dS^T Q, and S = Q K^T again for P), two flops per
        multiply-add -- 2.5 times the forward's count."""
        return 10 * self.heads * self.d_k * self.total_pairs()

    def projection_flops(self) -> int:
        if self.kind not in ("mha", "layer"):
            return 0
        dm = self.d_model
        rows_q = self.batch * self.n_q
        rows_k = self.batch * self.n_k
        # Q, K, V projections and the output projection W^O
        return 2 * dm * dm * (rows_q + 2 * rows_k + rows_q)

    def ffn_flops(self) -> int:
        """The FFN's two products, 2 * rows * d_model * d_ff each (biases, ReLU and norms not counted)."""
        if self.kind != "layer":
            return 0
        return 2 * 2 * self.batch * self.n_q * self.d_model * self.d_ff

    def total_flops(self) -> int:
        if self.kind == "bwd":
            return self.backward_flops()
        return self.attention_flops() + self.projection_flops() + self.ffn_flops()


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_mha_f32_b1_n128", "mha", "f32", batch=1, heads=8, n_q=128,
                 n_k=128, d_k=64, causal=False, seed=1, d_model=512),
        Workload("base_encoder_mha_bf16_b32_n512", "mha", "bf16", batch=32, heads=8,
                 n_q=512, n_k=512, d_k=64, causal=False, seed=2, d_model=512),
        Workload("decoder_causal_bf16_b16_h8_n1024", "attn", "bf16", batch=16, heads=8,
                 n_q=1024, n_k=1024, d_k=64, causal=True, seed=3),
        Workload("cross_attn_bf16_b32_h8_nq384_nk512", "attn", "bf16", batch=32, heads=8,
                 n_q=384, n_k=512, d_k=64, causal=False, seed=4),
        Workload("long_causal_bf16_b2_h16_n8192", "attn", "bf16", batch=2, heads=16,
                 n_q=8192, n_k=8192, d_k=64, causal=True, seed=5, oracle_rows=64),
        # the base encoder over a padded batch: key lengths uniform in [64, 512]
        Workload("base_encoder_padded_mha_bf16_b32_n512", "mha", "bf16", batch=32, heads=8,
                 n_q=512, n_k=512, d_k=64, causal=False, seed=6, d_model=512, kv_len_range=(64, 512)),
        # one whole encoder layer of the base model (d_ff = 2048)
        Workload("base_encoder_layer_bf16_b32_n512", "layer", "bf16", batch=32, heads=8,
                 n_q=512, n_k=512, d_k=64, causal=False, seed=7, d_model=512, d_ff=2048),
        # one decoding step of the base model (8 heads of 64) for 64 sequences against a
        # paged K/V cache of 16-slot pages, each page stored head-major (H, 16, d);
        # cached lengths uniform in [1024, 4096]
        # the backward of the long causal attention (training at long context)
        Workload("long_causal_bwd_bf16_b2_h16_n8192", "bwd", "bf16", batch=2, heads=16,
                 n_q=8192, n_k=8192, d_k=64, causal=True, seed=9, oracle_rows=64),
        Workload("decode_paged_bf16_b64_h8_kv4096", "decode", "bf16", batch=64, heads=8,
                 n_q=1, n_k=4096, d_k=64, causal=False, seed=8, kv_len_range=(1024, 4096), page_size=16),
    ]
}

# Short aliases used by command-line flags.
ALIASES = {
    "tiny": "tiny_mha_f32_b1_n128",
    "encoder": "base_encoder_mha_bf16_b32_n512",
    "decoder": "decoder_causal_bf16_b16_h8_n1024",
    "cross": "cross_attn_bf16_b32_h8_nq384_nk512",
    "long": "long_causal_bf16_b2_h16_n8192",
    "padded": "base_encoder_padded_mha_bf16_b32_n512",
    "layer": "base_encoder_layer_bf16_b32_n512",
    "decode": "decode_paged_bf16_b64_h8_kv4096",
    "bwd": "long_causal_bwd_bf16_b2_h16_n8192",
}


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


# ---------------------------------------------------------------- storage types

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (round to nearest, ties to even); return the raw uint16 bits.

    The input is first stored as float32 (the recipe above), then the upper
    16 bits are kept after adding the round-to-nearest-even bias. NaN does not
    occur in these inputs.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    # finite inputs: u + bias stays below 2^32 (the largest finite pattern is 0xFF7FFFFF)
    bias = (u >> np.uint32(16)) & np.uint32(1)
    bias += np.uint32(0x7FFF)
    bias += u
    bias >>= np.uint32(16)
    return bias.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """x rounded to the nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_bits(x))


@dataclasses.dataclass
class Stored:
    """One stored tensor: its exact value (float64) and the bits the device gets."""
    value: np.ndarray      # float64, exactly the stored value
    dtype: str             # "f32" or "bf16"
    raw: np.ndarray        # float32 array (f32) or uint16 bits (bf16), C-contiguous

    @property
    def shape(self):
        return self.value.shape


def store(x: np.ndarray, dtype: str) -> Stored:
    if dtype == "f32":
        f = np.ascontiguousarray(x, dtype=np.float32)
        return Stored(f.astype(np.float64), "f32", f)
    if dtype == "bf16":
        bits = bf16_bits(x)
        return Stored(bf16_bits_to_f32(bits).astype(np.float64), "bf16", bits)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------- generators

def make_inputs(w: Workload, *, v_ones: bool = False) -> dict[str, Stored]:
    """Draw the workload's tensors in the documented order.

    mha:  x (B, N, d_model), then W^Q, W^K, W^V, W^O, each (d_model, d_model),
          stored (in, out) so that Q = x @ W^Q. Self-attention: one x serves
          as the query, key and value input.
    layer: x (B, N, d_model), then encoder_params(d_model, d_ff, seed=100 + seed).
    attn: Q (B, H, N_q, d), K (B, H, N_k, d), V (B, H, N_k, d).
    decode: Q (B, H, d), then the logical caches K (B, H, N_k, d), V (B, H, N_k, d).
    bwd: Q, K, V as for attn, then dO (B, H, N_q, d).
    v_ones replaces V by all ones after drawing (row-sum checks); the draws
    themselves are unchanged so Q and K stay identical to the plain run.
    """
    rng = np.random.default_rng(w.seed)
    out: dict[str, Stored] = {}
    if w.kind == "layer":
        out["x"] = store(rng.standard_normal((w.batch, w.n_q, w.d_model)), w.dtype)
        out.update(encoder_params(w.d_model, w.d_ff, w.dtype, seed=100 + w.seed))
        return out
    if w.kind == "mha":
        dm = w.d_model
        out["x"] = store(rng.standard_normal((w.batch, w.n_q, dm)), w.dtype)
        s = 1.0 / math.sqrt(dm)
        for name in ("wq", "wk", "wv", "wo"):
            out[name] = store(rng.standard_normal((dm, dm)) * s, w.dtype)
        return out
    qshape = (w.batch, w.heads, w.d_k) if w.kind == "decode" else (w.batch, w.heads, w.n_q, w.d_k)
    out["q"] = store(rng.standard_normal(qshape), w.dtype)
    out["k"] = store(rng.standard_normal((w.batch, w.heads, w.n_k, w.d_k)), w.dtype)
    v = rng.standard_normal((w.batch, w.heads, w.n_k, w.d_v))
    if v_ones:
        v = np.ones_like(v)
    out["v"] = store(v, w.dtype)
    if w.kind == "bwd":
        out["do"] = store(rng.standard_normal((w.batch, w.heads, w.n_q, w.d_v)), w.dtype)
    return out


ENCODER_PARAM_NAMES = ("wq", "wk", "wv", "wo", "bq", "bk", "bv", "bo", "ln1_gamma", "ln1_beta",
                       "w1", "b1", "w2", "b2", "ln2_gamma", "ln2_beta")


def encoder_params(d_model: int, d_ff: int, dtype: str, seed: int) -> dict[str, Stored]:
    """Seeded encoder-layer parameters, drawn in ENCODER_PARAM_NAMES order from
    ``default_rng(seed)``: matrices (in, out) N(0, 1/fan_in) so activations stay
    unit variance; biases and LayerNorm shifts N(0, 0.1^2); LayerNorm scales
    1 + N(0, 0.1^2)."""
    rng = np.random.default_rng(seed)
    shapes = {"w1": (d_model, d_ff), "b1": (d_ff,), "w2": (d_ff, d_model)}
    out = {}
    for name in ENCODER_PARAM_NAMES:
        shape = shapes.get(name, (d_model, d_model) if name in ("wq", "wk", "wv", "wo") else (d_model,))
        z = rng.standard_normal(shape)
        if len(shape) == 2:
            z = z / math.sqrt(shape[0])
        elif name.endswith("gamma"):
            z = 1.0 + 0.1 * z
        else:
            z = 0.1 * z
        out[name] = store(z, dtype)
    return out


def page_table(lengths, page_size: int, max_pages: int, seed: int, spare: int = 0):
    """A shuffled page assignment for a paged cache.

    Sequence b owns ceil(lengths[b] / page_size) pages; all owned pages, plus
    `spare` unowned ones, are numbered 0..num_pages-1 in a random order drawn
    from ``default_rng(seed)`` (a permutation), so logically adjacent pages are
    physically scattered. Table entries past a sequence's own pages are -1.
    Returns (table (B, max_pages) int32, num_pages)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    need = (lengths + page_size - 1) // page_size
    if np.any(need > max_pages):
        raise ValueError("a sequence needs more pages than a table row holds")
    num_pages = int(need.sum()) + spare
    perm = np.random.default_rng(seed).permutation(num_pages).astype(np.int32)
    table = np.full((len(lengths), max_pages), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += int(n)
    return table, num_pages


def paged_pool(stored: Stored, table, lengths, page_size: int, num_pages: int, layout: str = "nhd") -> Stored:
    """Move a logical cache (B, H, N, d) into a page pool laid out by `table`
    (rows only move; slots no sequence owns stay 0): layout "nhd" gives
    (num_pages, page_size, H, d), "hnd" gives (num_pages, H, page_size, d), where
    each head's part of a page is one contiguous run. The returned Stored
    carries the raw pool only (value is None)."""
    raw = stored.raw
    B, H, N, d = raw.shape
    shape = (num_pages, page_size, H, d) if layout == "nhd" else (num_pages, H, page_size, d)
    pool = np.zeros(shape, dtype=raw.dtype)
    for b in range(B):
        n_pages = (int(lengths[b]) + page_size - 1) // page_size
        for i in range(n_pages):
            rows = raw[b, :, i * page_size:(i + 1) * page_size, :]     # (H, <=page_size, d)
            if layout == "nhd":
                pool[table[b, i], :rows.shape[1]] = rows.transpose(1, 0, 2)
            else:
                pool[table[b, i], :, :rows.shape[1]] = rows
    return Stored(None, stored.dtype, pool)


def random_tensor(shape, dtype: str, seed: int, scale: float = 1.0) -> Stored:
    """A seeded unit-normal tensor (times scale) for edge-shape tests."""
    rng = np.random.default_rng(seed)
    return store(rng.standard_normal(shape) * scale, dtype)


# Fixed edge positions checked in every sampled run of the long causal workload:
# the first rows, both sides of 64- and 128-row tile edges, the middle and the end.
EDGE_ROWS = (0, 1, 63, 64, 127, 128, 4095, 4096, 8190, 8191)


def sample_rows(w: Workload) -> np.ndarray:
    """Query positions the oracle evaluates for a sampled workload, sorted."""
    n = w.n_q
    fixed = [r for r in EDGE_ROWS if r < n]
    need = w.oracle_rows - len(fixed)
    rng = np.random.default_rng(1000 + w.seed)
    pool = np.setdiff1d(np.arange(n), np.array(fixed))
    extra = rng.choice(pool, size=max(need, 0), replace=False)
    return np.sort(np.concatenate([np.array(fixed, dtype=np.int64), extra.astype(np.int64)]))
