// Fused scaled dot-product attention forward, bf16 in/out, d_k = d_v = 64, gfx950.
//
// Computes O = softmax(scale * Q K^T (+ causal mask)) V per (batch, head)
// ("The Transformer" (hoshank.vercel.app), "The Mathematics", Attention
// equation) in one pass, without forming the score matrix in memory: the
// exact result is reached by streaming key/value tiles and keeping a running
// row maximum and row sum (the tiling idea the pages credit to FlashAttention,
// "32 Transformer", "Connections"; re-derived here for CDNA4).
//
// Three kernel forms, all with workgroups of 4 wavefronts on one (batch, head)
// and 64-key tiles staged through LDS:
//   32 query rows per wavefront (128 per workgroup): short or ragged unmasked
//     query runs. Tiles are double buffered: the next tile's global loads (raw
//     buffer loads; rows past the end read as zero) are in flight in
//     registers while the current one is used, then written to LDS, V
//     transposed ([d][key], two keys per 32-bit word).
//   32 query rows per wavefront, causal: the same tile order on tiles loaded
//     straight into a three-stage LDS ring (the 64-row form's layout), two
//     tiles ahead.
//   64 query rows per wavefront (two 32-row blocks sharing every K/V fragment
//     read; 256 per workgroup): long query runs. Tiles go straight from global
//     memory into a 4-stage LDS ring (buffer loads that write LDS) three tiles
//     ahead; the wavefront walks 32-key slabs and reads the next slab's K and
//     V fragments while the current one is computed.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, fp32 accumulate)
//   Scores are formed transposed, S^T = K Q^T: the MFMA's B operand is the
//   wavefront's Q^T (kept in registers for the whole kernel) and its A operand
//   is a 32-key slab of K read from LDS. In the 32x32 accumulator layout lane l
//   then holds column n = l % 32 (one query) and 16 rows (keys), so a query's
//   row maximum is an in-register reduction plus one exchange between lane
//   halves.
//   K rows are placed in LDS in a permuted order so that accumulator register
//   r of lane half hf holds key 16*(r/8) + 8*hf + (r%8) of its 32-key slab.
//   After conversion to bf16 those registers are, unchanged, the B operand of
//   O^T = V^T P^T (8 consecutive keys per lane), so P never goes through LDS.
//
// Softmax: exp2 with scale*log2(e) folded into one FMA. The row sum is formed
// on the matrix core from the bf16-rounded weights that the P V product uses
// (so the final 1/l normalises exactly what was multiplied by V). The
// reference maximum is moved lazily (only when weights against it would grow
// past 2^8), so the rescale of O and l is skipped on almost every slab;
// numerator and denominator always share one reference, so the result stays
// exact.
// Causal: tiles wholly above the diagonal are never loaded; per wavefront, a
// tile whose first key lies past the wavefront's last query is skipped; only
// tiles that straddle the diagonal (or the ragged end) apply per-element masks.
// Causal workgroups run heaviest query block first, with each head's blocks
// on one XCD (when the grid overflows one round of resident workgroups by at
// most a round, the 32-row causal form puts as many of the lightest levels
// first as overflow, the 64-row form the lightest quarter of its levels).
#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.h"

namespace mha {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x16 __attribute__((ext_vector_type(16)));

constexpr int kBN = 64;        // keys per tile
constexpr int kPitch = 72;     // LDS row pitch, bf16 elements (144 bytes: conflict-free 16-byte reads)
constexpr int kTile = kBN * kPitch;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBufferFlags = 0x00020000;  // raw buffer descriptor word 3 (gfx9 family: 32-bit data format)

__device__ __forceinline__ u32x4 ld16(const bf16* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Row sums of one 32-key slab's bf16 weights on the matrix core (v_dot2c
// would stall behind every MFMA in flight). The weights' registers, the B
// operand of the P V products (8 keys of one query per lane), are fed
// unchanged as the B operand of two v_mfma_f32_16x16x32_bf16 (one per 16
// keys) against a constant 0/1 selector A: lane l of that B holds column
// j = l % 16, rows 8 (l / 16) + 0..7, i.e. query 16 ((l / 16) % 2) + j, keys
// 8 (l / 32) + 0..7. Selector row m (m % 4 == 0) takes the groups whose
// query half is (m / 4) % 2, so output register 0 of lane L holds the slab's
// sum for query L % 32 in both lane halves. Products with 1 are exact and the
// accumulation is fp32, as with the dot instruction.
__device__ __forceinline__ bf16x8 rowsum_selector(int lane) {
  const unsigned one = ((lane & 3) == 0 && ((lane >> 2) & 1) == ((lane >> 4) & 1)) ? 0x3F803F80u : 0u;
  return __builtin_bit_cast(bf16x8, u32x4{one, one, one, one});
}
__device__ __forceinline__ float slab_rowsum(const unsigned (&pw)[8], const bf16x8& sel) {
  const bf16x8 p0 = __builtin_bit_cast(bf16x8, u32x4{pw[0], pw[1], pw[2], pw[3]});
  const bf16x8 p1 = __builtin_bit_cast(bf16x8, u32x4{pw[4], pw[5], pw[6], pw[7]});
  const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p0, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, p1, c, 0, 0, 0)[0];
}

// LDS row that receives key offset kappa (0..31) of a 32-key slab, so that the
// S^T accumulator register r of lane half hf maps to key 16*(r/8) + 8*hf + r%8.
// Accumulator row m = 8*(r/4) + 4*hf + r%4 in the 32x32 MFMA output layout.
__device__ __forceinline__ int key_to_lds_row(int kappa) {
  return 8 * (2 * (kappa >> 4) + ((kappa >> 2) & 1)) + 4 * ((kappa >> 3) & 1) + (kappa & 3);
}

// max(x[lane], x[lane ^ 32]) across the two half-waves (v_permlane32_swap).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}

// The reference maximum moves only when a row's weights against it would
// exceed 2^8, so the rescale of O and l is skipped on almost every tile. The
// result is exact: numerator and denominator always use the same reference.
constexpr float kMaxSlabSum = 256.0f;  // 2^8

// Running state of one 32-row query block: O^T in two 32-row d blocks.
struct RowState {
  f32x16 o0, o1;
  float m;   // reference maximum (raw score units), identical in both lane halves
  float mc;  // m * c
  float l;   // running row sum (the same in both lane halves)
};

// Softmax weights of pairs [i0, i1) of one 32-key slab (16 scores per lane)
// against the current reference, rounded to bf16.
template <bool kMasked>
__device__ __forceinline__ void slab_weights(const float (&sv)[16], unsigned (&pw)[8], float mc, float c, int i0,
                                             int i1) {
#pragma unroll
  for (int i = i0; i < i1; ++i) {
    float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], c, -mc));
    float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], c, -mc));
    if (kMasked) {
      p0 = sv[2 * i] == -INFINITY ? 0.f : p0;
      p1 = sv[2 * i + 1] == -INFINITY ? 0.f : p1;
    }
    pw[i] = pack_bf16(p0, p1);
  }
}

// Weights of pairs [i0, i1) of slab `slab` from its raw (unmasked) scores;
// on diagonal and ragged-end tiles the keys past `last` (relative to this
// lane's first key of the tile) get weight 0 by their index, so the scores
// themselves need no mask (a masked key's weight may be computed as inf or
// NaN and is then replaced).
template <bool kMasked>
__device__ __forceinline__ void slab_weights_k(const float (&sv)[16], unsigned (&pw)[8], float mc, float c, int i0,
                                               int i1, int slab, int last) {
#pragma unroll
  for (int i = i0; i < i1; ++i) {
    float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], c, -mc));
    float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], c, -mc));
    if (kMasked) {
      p0 = 32 * slab + 16 * ((2 * i) >> 3) + ((2 * i) & 7) <= last ? p0 : 0.f;
      p1 = 32 * slab + 16 * ((2 * i + 1) >> 3) + ((2 * i + 1) & 7) <= last ? p1 : 0.f;
    }
    pw[i] = pack_bf16(p0, p1);
  }
}

// Every weight is <= 2^8 while the reference holds. A weight above 2^8 (or
// an overflow) makes the row's 32-weight slab sum exceed 2^8, so one compare per
// slab detects when the reference must move; only then is the row maximum
// formed, O and l rescaled and the slab's weights recomputed. This branch is
// taken on a block's first slab and rarely after. Both kernel forms check a
// block's slab before forming that block's next weights and add its weights
// into O right after the check, so nothing computed against an older
// reference is left outside O and l when they are rescaled. The slab's scores
// are not kept for this path: `rescore` forms them again from the staged tile.
template <bool kMasked, typename Rescore>
__device__ __forceinline__ void check_reference(RowState& st, Rescore&& rescore, unsigned (&pw)[8], float ps, float c,
                                                const bf16x8& sel) {
  // an unmasked tile comes after the block's first (unmasked) slab has set the reference
  const bool bad = !(ps <= kMaxSlabSum) || (kMasked && st.m == -INFINITY);
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(bad) != 0, 0)) {
    asm volatile("" ::: "memory");  // keep a real branch, not predicated code
    // the slab's scores again (their registers are not kept for this rare path)
    float sv[16];
    rescore(sv);
    float tmax = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = __builtin_fmaxf(tmax, sv[r]);
    tmax = max_halves(tmax);
    const float m_new = __builtin_fmaxf(st.m, tmax);
    if (m_new > st.m) {
      const float mc_new = m_new * c;
      const float alpha = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.mc - mc_new);
      st.o0 *= alpha;
      st.o1 *= alpha;
      st.l *= alpha;
      st.m = m_new;
      st.mc = mc_new;
    }
    slab_weights<kMasked>(sv, pw, st.mc, c, 0, 8);
    ps = slab_rowsum(pw, sel);
  }
  st.l += ps;
}

// The reference of a block that has seen no key yet (O = 0, l = 0), from the
// row maximum of its first slab's scores: those weights are then <= 1 and the
// check after them passes without recomputing them.
__device__ __forceinline__ void first_reference(RowState& st, const float (&sv)[16], float c) {
  float tmax = sv[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) tmax = __builtin_fmaxf(tmax, sv[r]);
  tmax = max_halves(tmax);
  if (tmax > st.m) {
    st.m = tmax;
    st.mc = tmax * c;
  }
}

// One P V MFMA: 16 keys (step jj of a slab) into d block blk of O^T.
__device__ __forceinline__ void pv_one(RowState& st, const u32x4& vfrag, const unsigned (&pw)[8], int jj, int blk) {
  const bf16x8 bp = as_bf16x8(u32x4{pw[4 * jj], pw[4 * jj + 1], pw[4 * jj + 2], pw[4 * jj + 3]});
  if (blk == 0)
    st.o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vfrag), bp, st.o0, 0, 0, 0);
  else
    st.o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vfrag), bp, st.o1, 0, 0, 0);
}

__device__ __forceinline__ f32x16 qk_one(f32x16 acc, const u32x4& kfrag, const u32x4& qfrag) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kfrag), as_bf16x8(qfrag), acc, 0, 0, 0);
}

// Masked scores of one slab: keys past `last` (relative to this lane's first
// key of the tile) become -inf.
__device__ __forceinline__ void mask_slab(float (&sv)[16], const f32x16& s, int slab, int last) {
#pragma unroll
  for (int r = 0; r < 16; ++r) sv[r] = 32 * slab + 16 * (r >> 3) + (r & 7) <= last ? s[r] : -INFINITY;
}
// A slab's scores, masked (-inf past `last`) on diagonal and ragged-end tiles:
// the rare reference move takes its row maximum from them. The common path
// masks the weights instead (slab_weights_k).
template <bool kMasked>
__device__ __forceinline__ void scores_of_impl(float (&sv)[16], const f32x16& s, int slab, int last) {
  if (kMasked) {
    mask_slab(sv, s, slab, last);
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = s[r];
  }
}

// One 64-key tile for a wavefront of the 32-row form: two 32-key slabs
// (register r of a slab holds key 32*slab + 16*(r/8) + 8*hf + r%8 of the
// tile). Issue order, so that the wavefront keeps both the matrix core and the
// VALU busy: slab 0's S^T MFMAs; slab 1's S^T MFMAs each followed by a quarter
// of slab 0's softmax; slab 0's row sum and check; slab 0's P V MFMAs each
// followed by a quarter of slab 1's softmax; slab 1's row sum and check; slab
// 1's P V MFMAs. kMasked (diagonal and ragged-end tiles) runs the same order,
// with masked keys' scores set to -inf before the softmax.
template <bool kMasked, int kQB, bool kFirst = false>
__device__ __forceinline__ void attend_tile(RowState (&st)[kQB], const u32x4 (&qf)[kQB][4], const bf16* Ks,
                                            const bf16* Vt, const int (&last)[kQB], int lq, int hf, float c,
                                            const bf16x8& sel) {
  // the slab's scores; on a wavefront's first (unmasked) tile, slab 0 also
  // sets its block's reference, so that its weights need no second pass
  auto scores_of = [&](float (&sv)[16], const f32x16& s, int slab, int lst, RowState& rs) {
    scores_of_impl<false>(sv, s, slab, lst);  // masks are applied to the weights
    if (kFirst && slab == 0) first_reference(rs, sv, c);
  };
  u32x4 kf[2][4];
#pragma unroll
  for (int slab = 0; slab < 2; ++slab)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[slab][kk] = ld16(Ks + (32 * slab + lq) * kPitch + 16 * kk + 8 * hf);
  auto rescore = [&](int qb, int slab) {
    return [&, qb, slab](float (&sv)[16]) {
      f32x16 s = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) s = qk_one(s, ld16(Ks + (32 * slab + lq) * kPitch + 16 * kk + 8 * hf), qf[qb][kk]);
      scores_of_impl<kMasked>(sv, s, slab, last[qb]);
    };
  };

  {
    u32x4 vf0[2][2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) vf0[jj][blk] = ld16(Vt + (32 * blk + lq) * kPitch + 16 * jj + 8 * hf);
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) s0 = qk_one(s0, kf[0][kk], qf[0][kk]);
    float sv0[16], sv1[16];
    unsigned pw0[8], pw1[8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      s1 = qk_one(s1, kf[1][kk], qf[0][kk]);
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) scores_of(sv0, s0, 0, last[0], st[0]);
      slab_weights_k<kMasked>(sv0, pw0, st[0].mc, c, 2 * kk, 2 * kk + 2, 0, last[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    check_reference<kMasked>(st[0], rescore(0, 0), pw0, slab_rowsum(pw0, sel), c, sel);
    u32x4 vf1[2][2];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) vf1[jj][blk] = ld16(Vt + (32 * blk + lq) * kPitch + 16 * (2 + jj) + 8 * hf);
    scores_of(sv1, s1, 1, last[0], st[0]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pv_one(st[0], vf0[i >> 1][i & 1], pw0, i >> 1, i & 1);
      __builtin_amdgcn_sched_barrier(0);
      slab_weights_k<kMasked>(sv1, pw1, st[0].mc, c, 2 * i, 2 * i + 2, 1, last[0]);
      __builtin_amdgcn_sched_barrier(0);
    }
    check_reference<kMasked>(st[0], rescore(0, 1), pw1, slab_rowsum(pw1, sel), c, sel);
#pragma unroll
    for (int i = 0; i < 4; ++i) pv_one(st[0], vf1[i >> 1][i & 1], pw1, i >> 1, i & 1);
  }
}

// Pack lane's 4 values of d group g (d = 8g + 4hf + 0..3) of both lane halves
// into one 16-byte row chunk: half 0 ends with group gA = 2t, half 1 with 2t+1.
__device__ __forceinline__ u32x4 gather_row_chunk(unsigned a0, unsigned a1, unsigned b0, unsigned b1) {
  const auto x0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto x1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  return u32x4{(unsigned)x0[0], (unsigned)x1[0], (unsigned)x0[1], (unsigned)x1[1]};
}

// The 32-row form: 32 query rows per wavefront, 4 wavefronts per workgroup.
template <bool kCausal>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_d64_r32(AttnArgs a, float c, unsigned q_sign, int n_qblk) {
  constexpr int kQB = 1;
  constexpr int kRowsPerWave = 32 * kQB;
  constexpr int kRows = 4 * kRowsPerWave;  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * kTile];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int n_q = a.n_q;
  const bf16x8 sel = rowsum_selector(lane);

  // ---- workgroup -> (batch*head, query block)
  int bh, qblk;
  if (kCausal) {
    // heaviest query blocks (most key tiles) are dispatched first; workgroup i
    // goes to XCD i % 8, so XCD x takes the heads bh = x (mod 8) and all of a
    // head's query blocks share one L2
    const int BH = a.batch * a.heads;
    if ((BH & 7) == 0) {
      const int x = blockIdx.x & 7, j = blockIdx.x >> 3, bhx = BH >> 3;
      qblk = n_qblk - 1 - j / bhx;
      bh = x + 8 * (j % bhx);
    } else {
      qblk = n_qblk - 1 - (int)(blockIdx.x / BH);
      bh = (int)(blockIdx.x % BH);
    }
  } else {
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous run of logical ids so the query blocks of one (batch, head)
    // share that XCD's L2 and its K/V.
    const int total = gridDim.x, id = blockIdx.x;
    const int per = total >> 3, rem = total & 7, x = id & 7, slot = id >> 3;
    const int logical = (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
    bh = logical / n_qblk;
    qblk = logical - bh * n_qblk;
  }
  const int b = bh / a.heads, h = bh - b * a.heads;
  // keys visible to this batch item: all n_k, or its padded length
  const int n_k = a.kv_len != nullptr ? min(max(a.kv_len[b], 0), a.n_k) : a.n_k;
  const bf16* qp = static_cast<const bf16*>(a.q) + b * a.q_sb + h * a.q_sh;
  const bf16* kp = static_cast<const bf16*>(a.k) + b * a.k_sb + h * a.k_sh;
  const bf16* vp = static_cast<const bf16*>(a.v) + b * a.v_sb + h * a.v_sh;
  bf16* op = static_cast<bf16*>(a.o) + b * a.o_sb + h * a.o_sh;

  const int q_wave0 = qblk * kRows + wave * kRowsPerWave;

  // ---- this lane's slices of Q^T: d = 16*kk + 8*hf + 0..7 of query q_wave0 + 32*qb + lq
  u32x4 qf[kQB][4];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int my_q = q_wave0 + 32 * qb + lq;
    const bf16* src = qp + (int64_t)min(my_q, n_q - 1) * a.q_sn + 8 * hf;
    // loads from a clamped (always valid) row, then rows past n_q are zeroed:
    // a load under a per-lane condition would be waited for before the next
    // one is issued, serialising the opening round trips
    const unsigned keep = my_q < n_q ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[qb][kk] = (ld16(src + 16 * kk) ^ q_sign) & keep;
  }

  const int kv_end = kCausal ? min(n_k, qblk * kRows + kRows) : n_k;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // ---- cooperative staging assignment
  // K: two 16-byte chunks per thread, rows (tid/8) and (tid/8)+32, chunk tid%8
  const int k_row = tid >> 3, k_chunk = tid & 7;
  const int k_lds = key_to_lds_row(k_row);
  // V: keys 2*(tid%32) and 2*(tid%32)+1, d chunk tid/32
  const int v_key = (tid & 31) * 2, v_chunk = tid >> 5;

  // Buffer-resource loads: each thread's byte offset within a tile is fixed;
  // the tile's base moves in scalar registers, and the descriptor's record
  // count ends at the last valid key row, so rows past n_k read as zero with
  // no per-lane bounds checks.
  const int k_off[2] = {(int)(((int64_t)k_row * a.k_sn + 8 * k_chunk) * 2),
                        (int)(((int64_t)(k_row + 32) * a.k_sn + 8 * k_chunk) * 2)};
  const int v_off[2] = {(int)(((int64_t)v_key * a.v_sn + 8 * v_chunk) * 2),
                        (int)(((int64_t)(v_key + 1) * a.v_sn + 8 * v_chunk) * 2)};
  u32x4 kreg[2], vreg[2];
  auto gload = [&](int k0) {
    // record counts end at the last visible key row (none when no key is visible)
    const int valid = min(n_k - k0, kBN);
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kp + (int64_t)k0 * a.k_sn), (short)0, valid > 0 ? (int)((valid - 1) * a.k_sn * 2 + 2 * 64) : 0,
        kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(vp + (int64_t)k0 * a.v_sn), (short)0, valid > 0 ? (int)((valid - 1) * a.v_sn * 2 + 2 * 64) : 0,
        kBufferFlags);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, k_off[i], 0, 0));
      vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, v_off[i], 0, 0));
    }
  };
  auto lstore = [&](int buf) {
    bf16* Ks = smem + buf * 2 * kTile;
    bf16* Vt = Ks + kTile;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(Ks + (32 * i + k_lds) * kPitch + 8 * k_chunk) = kreg[i];
    // V^T[d][key]: word (d, key pair) = V[key][d] | V[key+1][d] << 16 (byte permutes)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned word = __builtin_amdgcn_perm(vreg[1][e >> 1], vreg[0][e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
      *reinterpret_cast<unsigned*>(Vt + (8 * v_chunk + e) * kPitch + v_key) = word;
    }
  };

  RowState st[kQB];
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    st[qb].o0 = f32x16{};
    st[qb].o1 = f32x16{};
    st[qb].m = -INFINITY;
    st[qb].mc = 0.f;
    st[qb].l = 0.f;
  }

  gload(0);
  lstore(0);
  __syncthreads();

  // Tiles before t_split are fully visible to every wavefront of the
  // workgroup (below the workgroup's first query and before the ragged end):
  // they take the unmasked path. The remaining tiles (the diagonal, the end)
  // take the masked path, or are skipped by wavefronts they lie wholly above.
  const int t_split = min(kCausal ? qblk * (kRows / kBN) : ntiles, n_k / kBN);
  const int no_mask[kQB] = {};
  int t = 0;
  if (t_split > 0) {  // the first tile sets each block's reference from its first slab
    const bool more = 1 < ntiles;
    if (more) gload(kBN);
    attend_tile<false, kQB, true>(st, qf, smem, smem + kTile, no_mask, lq, hf, c, sel);
    if (more) lstore(1);
    __syncthreads();
    t = 1;
  }
  for (; t < t_split; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) gload((t + 1) * kBN);
    const bf16* Ks = smem + (t & 1) * 2 * kTile;
    attend_tile<false, kQB>(st, qf, Ks, Ks + kTile, no_mask, lq, hf, c, sel);
    if (more) lstore((t + 1) & 1);
    __syncthreads();
  }
  for (; t < ntiles; ++t) {
    const int k0 = t * kBN;
    const bool more = t + 1 < ntiles;
    if (more) gload(k0 + kBN);
    const bf16* Ks = smem + (t & 1) * 2 * kTile;
    if (!kCausal || k0 <= q_wave0 + kRowsPerWave - 1) {  // wave-uniform
      int last[kQB];
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
        last[qb] = (kCausal ? min(n_k - 1, q_wave0 + 32 * qb + lq) : n_k - 1) - k0 - 8 * hf;
      attend_tile<true, kQB>(st, qf, Ks, Ks + kTile, last, lq, hf, c, sel);
    }
    if (more) lstore((t + 1) & 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds d = 32*blk + 8*g + 4*hf + 0..3 of its query;
  // the two halves swap groups so that each lane writes two 16-byte chunks per d block.
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int my_q = q_wave0 + 32 * qb + lq;
    const float l_tot = st[qb].l;
    // a row with no visible key (padded length 0) has l = 0: output 0, lse -inf
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    unsigned w[2][4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      w[0][g][0] = pack_bf16(st[qb].o0[4 * g] * inv, st[qb].o0[4 * g + 1] * inv);
      w[0][g][1] = pack_bf16(st[qb].o0[4 * g + 2] * inv, st[qb].o0[4 * g + 3] * inv);
      w[1][g][0] = pack_bf16(st[qb].o1[4 * g] * inv, st[qb].o1[4 * g + 1] * inv);
      w[1][g][1] = pack_bf16(st[qb].o1[4 * g + 2] * inv, st[qb].o1[4 * g + 3] * inv);
    }
    u32x4 chunk[2][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        chunk[blk][tt] =
            gather_row_chunk(w[blk][2 * tt][0], w[blk][2 * tt][1], w[blk][2 * tt + 1][0], w[blk][2 * tt + 1][1]);
    if (my_q < n_q) {
      bf16* dst = op + (int64_t)my_q * a.o_sn;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          *reinterpret_cast<u32x4*>(dst + 32 * blk + 8 * (2 * tt + hf)) = chunk[blk][tt];
      if (a.lse != nullptr && hf == 0)
        a.lse[(int64_t)bh * n_q + my_q] = l_tot > 0.f ? (st[qb].mc + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
// LDS stage: K tile (64 rows x 128 B, rows in the permuted key order), then V
// tile (64 rows x 128 B, key order); 16-byte chunk c of row R sits at chunk
// position c ^ (R & 7).
constexpr int kRowBytes = 128;
constexpr int kStageBytes = 2 * 64 * kRowBytes;
constexpr int kNStages = 4;

// fwd_loop_asm: the steady-state unmasked tile loop of the 64-row form
#include "attn_fwd_loop.inc"
struct LdsFrags {
  const char* base;  // generic pointer to the stage
  int klane[4];      // per-lane byte offsets of K fragments kk = 0..3 (slab 0)
  int vlane;         // per-lane byte offset of V transposed reads
  __device__ __forceinline__ u32x4 k(int slab, int kk) const {
    return *reinterpret_cast<const u32x4*>(base + klane[kk] + slab * 32 * kRowBytes);
  }
  __device__ __forceinline__ u32x4 v(int slab, int jj, int blk) const {
    const char* p = base + 64 * kRowBytes + vlane + (32 * slab + 16 * jj) * kRowBytes;
    const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 64 * blk));
    const v4i16 x1 =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 4 * kRowBytes + 64 * (blk ^ 1)));
    const u32x2 a = __builtin_bit_cast(u32x2, x0), b = __builtin_bit_cast(u32x2, x1);
    return u32x4{a[0], a[1], b[0], b[1]};
  }
};

__device__ __forceinline__ unsigned lds_off(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p;
}
// 16 bytes per lane from a raw buffer into LDS at lds_byte + 16 * lane (rows
// past the record end write zeros). Issued as asm so that the compiler does
// not wait for it before every LDS read; completion is awaited explicitly
// (vmcnt). The wave-uniform LDS base goes in m0 through the {m0} operand, so
// the compiler sets m0 itself and knows the register is taken.
__device__ __forceinline__ void dma16(u32x4 rsrc, int voff, unsigned lds_byte) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_byte) : "memory");
}

// ---------------------------------------------------------------------------
// 64 query rows per wavefront (blocks A and B of 32), slab-pipelined: the
// wavefront walks 32-key slabs; K and V fragments of slab g + 1 are read while
// slab g is computed, so no fragment read waits at a slab's start. Per slab:
//   A's 4 S^T MFMAs;
//   B's 4 S^T MFMAs, each followed by a quarter of A's softmax; A's row sum;
//   a quarter of B's softmax, A's check; A's 4 P V MFMAs each followed by
//     the next quarter of B's softmax (the last after them); B's row sum;
//   B's check; B's 4 P V MFMAs.
// Tiles of 64 keys (two slabs) are staged by DMA into a 4-stage LDS ring
// three tiles ahead; at tile t's sync tiles t and t + 1 are complete, so
// slab 1 of tile t can read tile t + 1's fragments.
template <bool kMasked, bool kFirst>
__device__ __forceinline__ void attend_slab(RowState (&st)[2], const u32x4 (&qf)[2][4], const LdsFrags& fr, int slab,
                                            const int (&last)[2], float c, const bf16x8& sel, const u32x4 (&kf)[4],
                                            const u32x4 (&vf)[2][2], u32x4 (&kf_nxt)[4], u32x4 (&vf_nxt)[2][2],
                                            const LdsFrags& fn, int nslab) {
  constexpr int A = 0, B = 1;
  auto rescore = [&](int qb) {
    return [&, qb](float (&sv)[16]) {
      f32x16 s = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) s = qk_one(s, fr.k(slab, kk), qf[qb][kk]);
      scores_of_impl<kMasked>(sv, s, slab, last[qb]);
    };
  };
  f32x16 sa = {}, sb = {};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) sa = qk_one(sa, kf[kk], qf[A][kk]);
  float sva[16], svb[16];
  unsigned pwa[8], pwb[8];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    sb = qk_one(sb, kf[kk], qf[B][kk]);
    __builtin_amdgcn_sched_barrier(0);
    if (kk == 0) {
      scores_of_impl<false>(sva, sa, slab, last[A]);  // masks are applied to the weights
      if (kFirst) first_reference(st[A], sva, c);
    }
    slab_weights_k<kMasked>(sva, pwa, st[A].mc, c, 2 * kk, 2 * kk + 2, slab, last[A]);
    if (kk == 1) {  // the next slab's K fragments (this slab's are used by the MFMAs above)
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) kf_nxt[k2] = fn.k(nslab, k2);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  const float psa = slab_rowsum(pwa, sel);
  scores_of_impl<false>(svb, sb, slab, last[B]);
  if (kFirst) first_reference(st[B], svb, c);
  slab_weights_k<kMasked>(svb, pwb, st[B].mc, c, 0, 2, slab, last[B]);
  __builtin_amdgcn_sched_barrier(0);
  check_reference<kMasked>(st[A], rescore(A), pwa, psa, c, sel);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pv_one(st[A], vf[j >> 1][j & 1], pwa, j >> 1, j & 1);
    __builtin_amdgcn_sched_barrier(0);
    if (j < 3) slab_weights_k<kMasked>(svb, pwb, st[B].mc, c, 2 * j + 2, 2 * j + 4, slab, last[B]);
    if (j == 1) {  // the next slab's V fragments go to the other register set
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) vf_nxt[jj][blk] = fn.v(nslab, jj, blk);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  const float psb = slab_rowsum(pwb, sel);
  check_reference<kMasked>(st[B], rescore(B), pwb, psb, c, sel);
#pragma unroll
  for (int j = 0; j < 4; ++j) pv_one(st[B], vf[j >> 1][j & 1], pwb, j >> 1, j & 1);
}

template <bool kCausal>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_d64_r64(AttnArgs a, float c, unsigned q_sign, int n_qblk, int n_light) {
  constexpr int kRowsPerWave = 64;
  constexpr int kRows = 256;
  __shared__ __attribute__((aligned(16))) char smem[kNStages * kStageBytes];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int n_q = a.n_q;
  bf16x8 sel = rowsum_selector(lane);

  int bh, qblk;
  if (kCausal) {
    // dispatch level r of the query blocks: the n_light lightest levels first,
    // then the others heaviest first (most key tiles); workgroup i goes to
    // XCD i % 8, so XCD x takes the heads bh = x (mod 8) and all of a head's
    // query blocks share one L2
    const int BH = a.batch * a.heads;
    int r;
    if ((BH & 7) == 0) {
      const int x = blockIdx.x & 7, j = blockIdx.x >> 3, bhx = BH >> 3;
      r = j / bhx;
      bh = x + 8 * (j % bhx);
    } else {
      r = (int)(blockIdx.x / BH);
      bh = (int)(blockIdx.x % BH);
    }
    qblk = r < n_light ? n_light - 1 - r : n_qblk - 1 - (r - n_light);
  } else {
    const int total = gridDim.x, id = blockIdx.x;
    const int per = total >> 3, rem = total & 7, x = id & 7, slot = id >> 3;
    const int logical = (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
    bh = logical / n_qblk;
    qblk = logical - bh * n_qblk;
  }
  const int b_ = bh / a.heads, h_ = bh - b_ * a.heads;
  const int n_k = a.kv_len != nullptr ? min(max(a.kv_len[b_], 0), a.n_k) : a.n_k;
  const bf16* qp = static_cast<const bf16*>(a.q) + b_ * a.q_sb + h_ * a.q_sh;
  const bf16* kp = static_cast<const bf16*>(a.k) + b_ * a.k_sb + h_ * a.k_sh;
  const bf16* vp = static_cast<const bf16*>(a.v) + b_ * a.v_sb + h_ * a.v_sh;
  bf16* op = static_cast<bf16*>(a.o) + b_ * a.o_sb + h_ * a.o_sh;
  const int q_wave0 = qblk * kRows + wave * kRowsPerWave;

  const int kv_end = kCausal ? min(n_k, qblk * kRows + kRows) : n_k;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto dma_tile = [&](int tile) {
    const int k0 = tile * kBN;
    const int valid = min(n_k - k0, kBN);
    const unsigned long long kb = (unsigned long long)(kp + (int64_t)k0 * a.k_sn);
    const unsigned long long vb = (unsigned long long)(vp + (int64_t)k0 * a.v_sn);
    auto uni = [](unsigned x) { return (unsigned)__builtin_amdgcn_readfirstlane((int)x); };
    const u32x4 kr = {uni((unsigned)kb), uni((unsigned)(kb >> 32) & 0xffffu),
                      uni(valid > 0 ? (unsigned)((valid - 1) * a.k_sn * 2 + 2 * 64) : 0u), (unsigned)kBufferFlags};
    const u32x4 vr = {uni((unsigned)vb), uni((unsigned)(vb >> 32) & 0xffffu),
                      uni(valid > 0 ? (unsigned)((valid - 1) * a.v_sn * 2 + 2 * 64) : 0u), (unsigned)kBufferFlags};
    const unsigned st_base = uni(lds_off(smem) + (unsigned)((tile % kNStages) * kStageBytes));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int R = 16 * wave + 8 * i + (lane >> 3);
      const int cch = (lane & 7) ^ (lane >> 3);
      const int kr5 = R & 31;
      const int key_k = (R & 32) | (kr5 & ~12) | ((kr5 >> 1) & 4) | ((kr5 << 1) & 8);
      dma16(kr, (key_k * (int)a.k_sn + 8 * cch) * 2, st_base + (unsigned)((16 * wave_u + 8 * i) * kRowBytes));
      dma16(vr, (R * (int)a.v_sn + 8 * cch) * 2, st_base + (unsigned)(64 * kRowBytes + (16 * wave_u + 8 * i) * kRowBytes));
    }
  };
  LdsFrags fr0;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) fr0.klane[kk] = lq * kRowBytes + 16 * ((2 * kk + hf) ^ (lq & 7));
  {
    const int g = lane >> 4, j = lane & 15;
    const int c_lane = 2 * (g & 1) + ((j & 3) >> 1);
    fr0.vlane = (8 * (g >> 1) + (j >> 2)) * kRowBytes + 16 * (c_lane ^ (j >> 2)) + 8 * (j & 1);
  }
  fr0.base = smem;
  auto frags_of = [&](int t) {
    LdsFrags f = fr0;
    f.base = smem + (t % kNStages) * kStageBytes;
    return f;
  };
  auto tile_sync = [&](int t) {
    if (t + 2 < ntiles)
      asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (t + 3 < ntiles) dma_tile(t + 3);
  };

  RowState st[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    st[qb].o0 = f32x16{};
    st[qb].o1 = f32x16{};
    st[qb].m = -INFINITY;
    st[qb].mc = 0.f;
    st[qb].l = 0.f;
  }
  // Opening: tiles 0 and 1 and this wavefront's Q^T slices are fetched
  // together, Q is complete before tile 2 is issued (so the wait for Q does
  // not also wait for tiles 2 and 3).
  if (ntiles > 0) dma_tile(0);
  if (ntiles > 1) dma_tile(1);
  // loads from a clamped (always valid) row, then rows past n_q are zeroed:
  // a load under a per-lane condition would be waited for before the next
  // one is issued, serialising the round trips
  u32x4 qf[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int my_q = q_wave0 + 32 * qb + lq;
    const bf16* src = qp + (int64_t)min(my_q, n_q - 1) * a.q_sn + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[qb][kk] = ld16(src + 16 * kk);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const unsigned keep = q_wave0 + 32 * qb + lq < n_q ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qf[qb][kk] = (qf[qb][kk] ^ q_sign) & keep;
      asm volatile("" : "+v"(qf[qb][kk]));  // complete here, before tile 2 is issued
    }
  }
  if (ntiles > 2) dma_tile(2);

  // fragments: set 0 for slab 0 of a tile, set 1 for slab 1
  u32x4 kf0[4], kf1[4], vf0[2][2], vf1[2][2];
  if (ntiles > 0) {
    tile_sync(0);
    const LdsFrags f = frags_of(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf0[kk] = f.k(0, kk);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) vf0[jj][blk] = f.v(0, jj, blk);
  }
  const int t_split = min(kCausal ? qblk * (kRows / kBN) : ntiles, n_k / kBN);
  const int no_mask[2] = {};
  auto tile = [&](auto masked, auto first, int t) {
    constexpr bool kM = decltype(masked)::value, kF = decltype(first)::value;
    const int k0 = t * kBN;
    int last[2] = {0, 0};
    if (kM) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        last[qb] = (kCausal ? min(n_k - 1, q_wave0 + 32 * qb + lq) : n_k - 1) - k0 - 8 * hf;
    }
    const LdsFrags fc = frags_of(t);
    // slab 1 reads the next tile's slab-0 fragments (this tile's again on the last)
    const LdsFrags fn = frags_of(t + 1 < ntiles ? t + 1 : t);
    attend_slab<kM, kF>(st, qf, fc, 0, kM ? last : no_mask, c, sel, kf0, vf0, kf1, vf1, fc, 1);
    attend_slab<kM, false>(st, qf, fc, 1, kM ? last : no_mask, c, sel, kf1, vf1, kf0, vf0, fn, 0);
  };
  using T = std::true_type;
  using F = std::false_type;
  int t = 0;
  if (t_split > 0) {
    tile(F{}, T{}, 0);
    if (1 < ntiles) tile_sync(1);
    t = 1;
  }
  if (t_split > 1) {
    // Unmasked tiles 1 .. t_split-1: the hand-scheduled loop (same arithmetic,
    // fixed issue order). On entry tiles 1 and 2 are in LDS and tiles 3 and 4
    // are requested; it requests tiles 5 .. t_split+2 itself (three ahead, as
    // tile_sync does) and leaves every wavefront past its last LDS read.
    const unsigned smem_lds = lds_off(smem);
    u32x4 kl;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kl[kk] = smem_lds + (unsigned)fr0.klane[kk];
    const unsigned vl = smem_lds + 64 * kRowBytes + (unsigned)fr0.vlane;
    unsigned dk[2], dv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int R = 16 * wave + 8 * i + (lane >> 3);
      const int cch = (lane & 7) ^ (lane >> 3);
      const int kr5 = R & 31;
      const int key_k = (R & 32) | (kr5 & ~12) | ((kr5 >> 1) & 4) | ((kr5 << 1) & 8);
      dk[i] = (unsigned)((key_k * (int)a.k_sn + 8 * cch) * 2);
      dv[i] = (unsigned)((R * (int)a.v_sn + 8 * cch) * 2);
    }
    auto uni = [](unsigned x) { return (unsigned)__builtin_amdgcn_readfirstlane((int)x); };
    const unsigned long long kb5 = (unsigned long long)kp + (unsigned long long)(5 * kBN) * a.k_sn * 2;
    const unsigned long long vb5 = (unsigned long long)vp + (unsigned long long)(5 * kBN) * a.v_sn * 2;
    u32x4 sel_u = __builtin_bit_cast(u32x4, sel);
    fwd_loop_asm(st[0].o0, st[0].o1, st[1].o0, st[1].o1, st[0].m, st[1].m, st[0].mc, st[1].mc, st[0].l, st[1].l,
                 qf, sel_u, kl, vl, dk[0], dk[1], dv[0], dv[1], c, t_split - 1, ntiles,
                 n_k - 5 * kBN, (int)uni((unsigned)(a.k_sn * 2)), (int)uni((unsigned)(a.v_sn * 2)),
                 uni((unsigned)(kBN * a.k_sn * 2)), uni((unsigned)(kBN * a.v_sn * 2)),
                 uni(smem_lds + (unsigned)(16 * wave_u * kRowBytes)), uni((unsigned)kb5), uni((unsigned)(kb5 >> 32)),
                 uni((unsigned)vb5), uni((unsigned)(vb5 >> 32)));
    // the selector comes back from the loop unchanged; using its copy keeps
    // the compiler from holding a second one across it
    sel = __builtin_bit_cast(bf16x8, sel_u);
    t = t_split;
    if (t < ntiles) tile_sync(t);
    // the next tile's slab-0 fragments (when no tile follows, these in-bounds
    // reads are not used; reading them unconditionally keeps the fragments
    // from before the loop dead across it)
    const LdsFrags f = frags_of(t);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf0[kk] = f.k(0, kk);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) vf0[jj][blk] = f.v(0, jj, blk);
  }
  for (; t < ntiles; ++t) {
    const int k0 = t * kBN;
    if (!kCausal || k0 <= q_wave0 + kRowsPerWave - 1) tile(T{}, F{}, t);  // wave-uniform
    if (t + 1 < ntiles) tile_sync(t + 1);
  }

#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int my_q = q_wave0 + 32 * qb + lq;
    const float l_tot = st[qb].l;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    unsigned w[2][4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      w[0][g][0] = pack_bf16(st[qb].o0[4 * g] * inv, st[qb].o0[4 * g + 1] * inv);
      w[0][g][1] = pack_bf16(st[qb].o0[4 * g + 2] * inv, st[qb].o0[4 * g + 3] * inv);
      w[1][g][0] = pack_bf16(st[qb].o1[4 * g] * inv, st[qb].o1[4 * g + 1] * inv);
      w[1][g][1] = pack_bf16(st[qb].o1[4 * g + 2] * inv, st[qb].o1[4 * g + 3] * inv);
    }
    u32x4 chunk[2][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        chunk[blk][tt] =
            gather_row_chunk(w[blk][2 * tt][0], w[blk][2 * tt][1], w[blk][2 * tt + 1][0], w[blk][2 * tt + 1][1]);
    if (my_q < n_q) {
      bf16* dst = op + (int64_t)my_q * a.o_sn;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          *reinterpret_cast<u32x4*>(dst + 32 * blk + 8 * (2 * tt + hf)) = chunk[blk][tt];
      if (a.lse != nullptr && hf == 0)
        a.lse[(int64_t)bh * n_q + my_q] = l_tot > 0.f ? (st[qb].mc + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// The 32-row form for causal runs: the same tile order as attend_tile (slab
// 1's S^T MFMAs between slab 0's softmax quarters, slab 0's P V MFMAs between
// slab 1's), with the tiles in the 64-row form's LDS layout, loaded straight
// into a three-stage ring two tiles ahead (48 KB: three workgroups per CU).
constexpr int kR32Stages = 3;

template <bool kMasked, bool kFirst = false>
__device__ __forceinline__ void attend_tile_f(RowState& st, const u32x4 (&qf)[4], const LdsFrags& fr, int last,
                                              float c, const bf16x8& sel) {
  u32x4 kf[2][4];
#pragma unroll
  for (int slab = 0; slab < 2; ++slab)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[slab][kk] = fr.k(slab, kk);
  auto rescore = [&](int slab) {
    return [&, slab](float (&sv)[16]) {
      f32x16 s = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) s = qk_one(s, fr.k(slab, kk), qf[kk]);
      scores_of_impl<kMasked>(sv, s, slab, last);
    };
  };
  u32x4 vf0[2][2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) vf0[jj][blk] = fr.v(0, jj, blk);
  f32x16 s0 = {}, s1 = {};
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) s0 = qk_one(s0, kf[0][kk], qf[kk]);
  float sv0[16], sv1[16];
  unsigned pw0[8], pw1[8];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    s1 = qk_one(s1, kf[1][kk], qf[kk]);
    __builtin_amdgcn_sched_barrier(0);
    if (kk == 0) {
      scores_of_impl<false>(sv0, s0, 0, last);  // masks are applied to the weights
      if (kFirst) first_reference(st, sv0, c);
    }
    slab_weights_k<kMasked>(sv0, pw0, st.mc, c, 2 * kk, 2 * kk + 2, 0, last);
    __builtin_amdgcn_sched_barrier(0);
  }
  check_reference<kMasked>(st, rescore(0), pw0, slab_rowsum(pw0, sel), c, sel);
  u32x4 vf1[2][2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) vf1[jj][blk] = fr.v(1, jj, blk);
  scores_of_impl<false>(sv1, s1, 1, last);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pv_one(st, vf0[i >> 1][i & 1], pw0, i >> 1, i & 1);
    __builtin_amdgcn_sched_barrier(0);
    slab_weights_k<kMasked>(sv1, pw1, st.mc, c, 2 * i, 2 * i + 2, 1, last);
    __builtin_amdgcn_sched_barrier(0);
  }
  check_reference<kMasked>(st, rescore(1), pw1, slab_rowsum(pw1, sel), c, sel);
#pragma unroll
  for (int i = 0; i < 4; ++i) pv_one(st, vf1[i >> 1][i & 1], pw1, i >> 1, i & 1);
}

template <bool kCausal>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_d64_r32d(AttnArgs a, float c, unsigned q_sign, int n_qblk, int n_light) {
  constexpr int kRowsPerWave = 32;
  constexpr int kRows = 128;
  __shared__ __attribute__((aligned(16))) char smem[kR32Stages * kStageBytes];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int n_q = a.n_q;
  const bf16x8 sel = rowsum_selector(lane);

  int bh, qblk;
  if (kCausal) {
    // dispatch level r of the query blocks: the n_light lightest levels
    // first (they would otherwise start in a late, partial second round of
    // workgroups, each with its own opening), then the others heaviest first
    const int BH = a.batch * a.heads;
    int r;
    if ((BH & 7) == 0) {
      const int x = blockIdx.x & 7, j = blockIdx.x >> 3, bhx = BH >> 3;
      r = j / bhx;
      bh = x + 8 * (j % bhx);
    } else {
      r = (int)(blockIdx.x / BH);
      bh = (int)(blockIdx.x % BH);
    }
    qblk = r < n_light ? n_light - 1 - r : n_qblk - 1 - (r - n_light);
  } else {
    const int total = gridDim.x, id = blockIdx.x;
    const int per = total >> 3, rem = total & 7, x = id & 7, slot = id >> 3;
    const int logical = (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
    bh = logical / n_qblk;
    qblk = logical - bh * n_qblk;
  }
  const int b_ = bh / a.heads, h_ = bh - b_ * a.heads;
  const int n_k = a.kv_len != nullptr ? min(max(a.kv_len[b_], 0), a.n_k) : a.n_k;
  const bf16* qp = static_cast<const bf16*>(a.q) + b_ * a.q_sb + h_ * a.q_sh;
  const bf16* kp = static_cast<const bf16*>(a.k) + b_ * a.k_sb + h_ * a.k_sh;
  const bf16* vp = static_cast<const bf16*>(a.v) + b_ * a.v_sb + h_ * a.v_sh;
  bf16* op = static_cast<bf16*>(a.o) + b_ * a.o_sb + h_ * a.o_sh;
  const int q_wave0 = qblk * kRows + wave * kRowsPerWave;
  const int kv_end = kCausal ? min(n_k, qblk * kRows + kRows) : n_k;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto dma_tile = [&](int tile) {
    const int k0 = tile * kBN;
    const int valid = min(n_k - k0, kBN);
    const unsigned long long kb = (unsigned long long)(kp + (int64_t)k0 * a.k_sn);
    const unsigned long long vb = (unsigned long long)(vp + (int64_t)k0 * a.v_sn);
    auto uni = [](unsigned x) { return (unsigned)__builtin_amdgcn_readfirstlane((int)x); };
    const u32x4 kr = {uni((unsigned)kb), uni((unsigned)(kb >> 32) & 0xffffu),
                      uni(valid > 0 ? (unsigned)((valid - 1) * a.k_sn * 2 + 2 * 64) : 0u), (unsigned)kBufferFlags};
    const u32x4 vr = {uni((unsigned)vb), uni((unsigned)(vb >> 32) & 0xffffu),
                      uni(valid > 0 ? (unsigned)((valid - 1) * a.v_sn * 2 + 2 * 64) : 0u), (unsigned)kBufferFlags};
    const unsigned st_base = uni(lds_off(smem) + (unsigned)((tile % kR32Stages) * kStageBytes));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int R = 16 * wave + 8 * i + (lane >> 3);
      const int cch = (lane & 7) ^ (lane >> 3);
      const int kr5 = R & 31;
      const int key_k = (R & 32) | (kr5 & ~12) | ((kr5 >> 1) & 4) | ((kr5 << 1) & 8);
      dma16(kr, (key_k * (int)a.k_sn + 8 * cch) * 2, st_base + (unsigned)((16 * wave_u + 8 * i) * kRowBytes));
      dma16(vr, (R * (int)a.v_sn + 8 * cch) * 2, st_base + (unsigned)(64 * kRowBytes + (16 * wave_u + 8 * i) * kRowBytes));
    }
  };
  LdsFrags fr0;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) fr0.klane[kk] = lq * kRowBytes + 16 * ((2 * kk + hf) ^ (lq & 7));
  {
    const int g = lane >> 4, j = lane & 15;
    const int c_lane = 2 * (g & 1) + ((j & 3) >> 1);
    fr0.vlane = (8 * (g >> 1) + (j >> 2)) * kRowBytes + 16 * (c_lane ^ (j >> 2)) + 8 * (j & 1);
  }
  fr0.base = smem;
  auto frags_of = [&](int t) {
    LdsFrags f = fr0;
    f.base = smem + (t % kR32Stages) * kStageBytes;
    return f;
  };
  // tile t has landed when at most the tiles issued after it are outstanding
  // (4 loads per tile and wavefront); the barrier also ends every read of the
  // stage that tile t + kR32Stages - 1 then reuses
  auto tile_sync = [&](int t) {
    const int ahead = min(kR32Stages - 2, ntiles - 1 - t);
    if (kR32Stages >= 4 && ahead >= 2)
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else if (kR32Stages >= 3 && ahead == 1)
      asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (t + kR32Stages - 1 < ntiles) dma_tile(t + kR32Stages - 1);
  };

  // opening: tile 0 and Q together, the rest of the lead once Q is in
  if (ntiles > 0) dma_tile(0);
  u32x4 qf[4];
  {
    const int my_q = q_wave0 + lq;
    const bf16* src = qp + (int64_t)min(my_q, n_q - 1) * a.q_sn + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = ld16(src + 16 * kk);
    const unsigned keep = my_q < n_q ? 0xffffffffu : 0u;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qf[kk] = (qf[kk] ^ q_sign) & keep;
      asm volatile("" : "+v"(qf[kk]));
    }
  }
  for (int t = 1; t < kR32Stages - 1 && t < ntiles; ++t) dma_tile(t);

  RowState st;
  st.o0 = f32x16{};
  st.o1 = f32x16{};
  st.m = -INFINITY;
  st.mc = 0.f;
  st.l = 0.f;

  const int t_split = min(kCausal ? qblk * (kRows / kBN) : ntiles, n_k / kBN);
  int t = 0;
  if (t_split > 0) {
    tile_sync(0);
    attend_tile_f<false, true>(st, qf, frags_of(0), 0, c, sel);
    t = 1;
  }
  for (; t < t_split; ++t) {
    tile_sync(t);
    attend_tile_f<false>(st, qf, frags_of(t), 0, c, sel);
  }
  for (; t < ntiles; ++t) {
    tile_sync(t);
    const int k0 = t * kBN;
    if (!kCausal || k0 <= q_wave0 + kRowsPerWave - 1) {  // wave-uniform
      const int last = (kCausal ? min(n_k - 1, q_wave0 + lq) : n_k - 1) - k0 - 8 * hf;
      attend_tile_f<true>(st, qf, frags_of(t), last, c, sel);
    }
  }

  {
    const int my_q = q_wave0 + lq;
    const float l_tot = st.l;
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    unsigned w[2][4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      w[0][g][0] = pack_bf16(st.o0[4 * g] * inv, st.o0[4 * g + 1] * inv);
      w[0][g][1] = pack_bf16(st.o0[4 * g + 2] * inv, st.o0[4 * g + 3] * inv);
      w[1][g][0] = pack_bf16(st.o1[4 * g] * inv, st.o1[4 * g + 1] * inv);
      w[1][g][1] = pack_bf16(st.o1[4 * g + 2] * inv, st.o1[4 * g + 3] * inv);
    }
    u32x4 chunk[2][2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        chunk[blk][tt] =
            gather_row_chunk(w[blk][2 * tt][0], w[blk][2 * tt][1], w[blk][2 * tt + 1][0], w[blk][2 * tt + 1][1]);
    if (my_q < n_q) {
      bf16* dst = op + (int64_t)my_q * a.o_sn;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          *reinterpret_cast<u32x4*>(dst + 32 * blk + 8 * (2 * tt + hf)) = chunk[blk][tt];
      if (a.lse != nullptr && hf == 0)
        a.lse[(int64_t)bh * n_q + my_q] = l_tot > 0.f ? (st.mc + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// Workgroups of the causal 32-row form the current device holds at once
// (occupancy x compute units), cached per device; 0 if the query fails.
static int r32d_resident() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] != 0) return cache[dev] > 0 ? cache[dev] : 0;
  int occ = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, attn_fwd_bf16_d64_r32d<true>, 256, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || occ * cus <= 0) {
    cache[dev] = -1;
    return 0;
  }
  cache[dev] = occ * cus;
  return cache[dev];
}

static void launch_r32d(const AttnArgs& a, hipStream_t stream, float c, unsigned q_sign) {
  const int n_qblk = (a.n_q + 127) / 128;
  const int BH = a.batch * a.heads;
  const int n_items = n_qblk * BH;
  // causal grids that overflow one round of resident workgroups by at most a
  // round: as many of the lightest levels as overflow go first
  int n_light = 0;
  const int resident = a.causal ? r32d_resident() : 0;
  if (resident > 0 && n_items > resident && n_items <= 2 * resident)
    n_light = min((n_items - resident + BH - 1) / BH, n_qblk);
  const dim3 grid((unsigned)n_items);
  if (a.causal)
    hipLaunchKernelGGL((attn_fwd_bf16_d64_r32d<true>), grid, dim3(256), 0, stream, a, c, q_sign, n_qblk, n_light);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_d64_r32d<false>), grid, dim3(256), 0, stream, a, c, q_sign, n_qblk, 0);
}

// Workgroups of the causal 64-row form the current device holds at once
// (occupancy x compute units), cached per device; 0 if the query fails.
static int r64_resident() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] != 0) return cache[dev] > 0 ? cache[dev] : 0;
  int occ = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, attn_fwd_bf16_d64_r64<true>, 256, 0) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || occ * cus <= 0) {
    cache[dev] = -1;
    return 0;
  }
  cache[dev] = occ * cus;
  return cache[dev];
}

static void launch_slab(const AttnArgs& a, hipStream_t stream, float c, unsigned q_sign) {
  const int n_qblk = (a.n_q + 255) / 256;
  const int n_items = n_qblk * a.batch * a.heads;
  const dim3 grid((unsigned)n_items);
  // Causal grids of more than one and at most two rounds of resident
  // workgroups: the lightest quarter of the query-block levels goes first.
  // Measured on the long causal launch (2 x 16 heads, N = 8192: 32 levels,
  // two rounds of 512): 8 levels first 253-262 against 261-269 us on two
  // boxes; the dependence on the count is not smooth (6, 7 and 10 were
  // slower than none), and grids of four rounds gained nothing.
  int n_light = 0;
  const int resident = a.causal ? r64_resident() : 0;
  if (resident > 0 && n_items > resident && n_items <= 2 * resident) n_light = n_qblk / 4;
  if (a.causal)
    hipLaunchKernelGGL((attn_fwd_bf16_d64_r64<true>), grid, dim3(256), 0, stream, a, c, q_sign, n_qblk, n_light);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_d64_r64<false>), grid, dim3(256), 0, stream, a, c, q_sign, n_qblk, 0);
}

}  // namespace

// Rows per wavefront: 64 (two 32-row blocks share every K/V fragment read;
// the slab-prefetching kernel) in 256-row workgroups, else 32. Measured on
// MI355X: 64 rows pay off for long query runs with little padding (longer K/V
// streams per workgroup: unmasked from 2048 queries, causal from 4096) and for
// unmasked runs that fill whole 256-row workgroups (the encoder launch); for
// shorter causal or ragged runs the 32-row forms' occupancy and finer causal
// split win (causal N=2048, B=8, H=8: 45.3 against 50.4 us with the causal
// 32-row form).
int attention_rows_per_wave(int n_q, bool causal) {
  const int pad256 = (n_q + 255) / 256 * 256 - n_q;
  if (!causal && n_q >= 512 && pad256 == 0) return 64;
  return (n_q >= (causal ? 4096 : 2048) && pad256 * 16 <= n_q) ? 64 : 32;
}

static void launch_rows32(const AttnArgs& a, hipStream_t stream, float c, unsigned q_sign) {
  const int n_qblk = (a.n_q + 127) / 128;
  const dim3 grid((unsigned)(n_qblk * a.batch * a.heads));
  if (a.causal)
    hipLaunchKernelGGL((attn_fwd_bf16_d64_r32<true>), grid, dim3(256), 0, stream, a, c, q_sign, n_qblk);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_d64_r32<false>), grid, dim3(256), 0, stream, a, c, q_sign, n_qblk);
}

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t stream) {
  const float kLog2e = 1.4426950408889634f;
  const float c = fabsf(a.scale) * kLog2e;
  const unsigned q_sign = a.scale < 0.f ? 0x80008000u : 0u;  // negate Q exactly: scale*s = |scale|*(-q).k
  if (attention_rows_per_wave(a.n_q, a.causal != 0) == 64)
    launch_slab(a, stream, c, q_sign);
  else if (a.causal)
    launch_r32d(a, stream, c, q_sign);
  else
    launch_rows32(a, stream, c, q_sign);
  return hipGetLastError();
}

}  // namespace mha
