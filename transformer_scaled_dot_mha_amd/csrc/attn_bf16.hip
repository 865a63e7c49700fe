// Fused scaled dot-product attention forward, bf16 in/out, d_k = d_v = 64, gfx950.
//
// Computes O = softmax(scale * Q K^T (+ causal mask)) V per (batch, head)
// ("The Transformer" (hoshank.vercel.app), "The Mathematics", Attention
// equation) in one pass, without forming the score matrix in memory: the
// exact result is reached by streaming key/value tiles and keeping a running
// row maximum and row sum (the tiling idea the pages credit to FlashAttention,
// "32 Transformer", "Connections"; re-derived here for CDNA4).
//
// Work decomposition
//   workgroup = 256 threads = 4 wavefronts of one (batch, head); each
//   wavefront owns 32 query rows, or 64 (two 32-row blocks sharing every K/V
//   fragment read) for long query runs, so a workgroup owns 128 or 256 rows.
//   key/value tiles of 64 rows are staged through LDS, double buffered, with
//   the next tile's global loads (raw buffer loads; rows past the end read as
//   zero) in flight while the current one is used.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, fp32 accumulate)
//   Scores are formed transposed, S^T = K Q^T: the MFMA's B operand is the
//   wavefront's Q^T (kept in registers for the whole kernel) and its A operand
//   is a 32-key slab of K read from LDS. In the 32x32 accumulator layout lane l
//   then holds column n = l % 32 (one query) and 16 rows (keys), so a query's
//   row maximum and row sum are in-register reductions plus one exchange
//   between lane halves.
//   K rows are written to LDS in a permuted order so that accumulator register
//   r of lane half hf holds key 16*(r/8) + 8*hf + (r%8) of its 32-key slab.
//   After conversion to bf16 those registers are, unchanged, the B operand of
//   O^T = V^T P^T (8 consecutive keys per lane), so P never goes through LDS.
//   V is transposed into LDS ([d][key]) while staging, two keys per 32-bit word.
//
// Softmax: exp2 with scale*log2(e) folded into one FMA; the row sum is
// accumulated from the bf16-rounded weights that the P V product uses, so the
// final 1/l normalises exactly what was summed. The reference maximum is
// moved lazily (only when weights against it would grow past 2^8), so the
// rescale of O and l is skipped on almost every tile; numerator and
// denominator always share one reference, so the result stays exact.
// Causal: tiles wholly above the diagonal are never loaded; per wavefront, a
// tile whose first key lies past the wavefront's last query is skipped; only
// tiles that straddle the diagonal (or the ragged end) apply per-element masks.
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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

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

// Sum of a packed bf16 pair, added to acc in fp32 (v_dot2c_f32_bf16 with (1, 1)).
__device__ __forceinline__ float add_pair(unsigned pair, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
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
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
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
  float l;   // running sum over this lane half's keys
};

// Softmax weights of pairs [i0, i1) of one 32-key slab (16 scores per lane)
// against the current reference, rounded to bf16; ps adds exactly the
// rounded values.
template <bool kMasked>
__device__ __forceinline__ void slab_weights(const float (&sv)[16], unsigned (&pw)[8], float& ps, float mc, float c,
                                             int i0, int i1) {
#pragma unroll
  for (int i = i0; i < i1; ++i) {
    float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], c, -mc));
    float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], c, -mc));
    if (kMasked) {
      p0 = sv[2 * i] == -INFINITY ? 0.f : p0;
      p1 = sv[2 * i + 1] == -INFINITY ? 0.f : p1;
    }
    pw[i] = pack_bf16(p0, p1);
    ps = add_pair(pw[i], ps);
  }
}

struct NoPending {
  __device__ void operator()() const {}
};

// Every weight is <= 2^8 while the reference holds. A weight above 2^8 (or
// an overflow) makes the lane's 16-weight sum exceed 2^8, so one compare per
// slab detects when the reference must move; only then is the row maximum
// formed, O and l rescaled and the slab's weights recomputed. This branch is
// taken on the first tile and rarely after.
// `flush_pending` adds into O the weights of an earlier slab that were
// computed against the current reference but not yet multiplied by V; it
// runs before a move, so that O is rescaled together with them (l already
// holds their sum).
template <bool kMasked, typename Pending = NoPending>
__device__ __forceinline__ void check_reference(RowState& st, const float (&sv)[16], unsigned (&pw)[8], float& ps,
                                                float c, Pending&& flush_pending = Pending{}) {
  const bool bad = !(ps <= kMaxSlabSum) || st.m == -INFINITY;
  if (__builtin_expect(__builtin_amdgcn_ballot_w64(bad) != 0, 0)) {
    asm volatile("" ::: "memory");  // keep a real branch, not predicated code
    float tmax = sv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = __builtin_fmaxf(tmax, sv[r]);
    tmax = max_halves(tmax);
    const float m_new = __builtin_fmaxf(st.m, tmax);
    if (__builtin_amdgcn_ballot_w64(m_new > st.m) != 0) flush_pending();
    if (m_new > st.m) {
      const float mc_new = m_new * c;
      const float alpha = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.mc - mc_new);
      st.o0 *= alpha;
      st.o1 *= alpha;
      st.l *= alpha;
      st.m = m_new;
      st.mc = mc_new;
    }
    ps = 0.f;
    slab_weights<kMasked>(sv, pw, ps, st.mc, c, 0, 8);
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
// The slab's scores for the softmax: masked on diagonal and ragged-end tiles.
template <bool kMasked>
__device__ __forceinline__ void scores_of_impl(float (&sv)[16], const f32x16& s, int slab, int last) {
  if (kMasked) {
    mask_slab(sv, s, slab, last);
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) sv[r] = s[r];
  }
}

// One 64-key tile for one wavefront holding kQB blocks of 32 query rows.
// Each block's tile is two 32-key slabs (register r of a slab holds key
// 32*slab + 16*(r/8) + 8*hf + r%8 of the tile). K and V fragments are read
// from LDS once and used by every block of the wavefront.
//
// Unmasked tiles are issued in a fixed order so that the wavefront keeps both
// the matrix core and the VALU busy: every MFMA is followed by a chunk of
// softmax work that does not depend on it.
//   kQB = 1: slab 0's S^T MFMAs; slab 1's S^T MFMAs each followed by a
//            quarter of slab 0's softmax; slab 0's P V MFMAs each followed by
//            a quarter of slab 1's softmax; slab 1's P V MFMAs.
//   kQB = 2: block A's S^T MFMAs; block B's eight S^T MFMAs each followed by
//            an eighth of A's softmax; A's eight P V MFMAs each followed by an
//            eighth of B's softmax; B's P V MFMAs.
// A reference move (rare) rescales that block's O and l after its earlier
// P V products, so every term matches the reference it was computed against:
// with kQB = 2 both slabs of a block are checked before its P V products, so
// a move found on slab 1 first adds slab 0's weights into O.
// kMasked (diagonal and ragged-end tiles) runs the same order, with masked
// keys' scores set to -inf before the softmax.
template <bool kMasked, int kQB, bool kFirst = false>
__device__ __forceinline__ void attend_tile(RowState (&st)[kQB], const u32x4 (&qf)[kQB][4], const bf16* Ks,
                                            const bf16* Vt, const int (&last)[kQB], int lq, int hf, float c) {
  // the slab's scores; on a wavefront's first (unmasked) tile, slab 0 also
  // sets its block's reference, so that its weights need no second pass
  auto scores_of = [&](float (&sv)[16], const f32x16& s, int slab, int lst, RowState& rs) {
    scores_of_impl<kMasked>(sv, s, slab, lst);
    if (kFirst && slab == 0) first_reference(rs, sv, c);
  };
  u32x4 kf[2][4];
#pragma unroll
  for (int slab = 0; slab < 2; ++slab)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kf[slab][kk] = ld16(Ks + (32 * slab + lq) * kPitch + 16 * kk + 8 * hf);

  if (kQB == 1) {
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
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      s1 = qk_one(s1, kf[1][kk], qf[0][kk]);
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) scores_of(sv0, s0, 0, last[0], st[0]);
      slab_weights<kMasked>(sv0, pw0, ps0, st[0].mc, c, 2 * kk, 2 * kk + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    check_reference<kMasked>(st[0], sv0, pw0, ps0, c);
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
      slab_weights<kMasked>(sv1, pw1, ps1, st[0].mc, c, 2 * i, 2 * i + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    check_reference<kMasked>(st[0], sv1, pw1, ps1, c);
#pragma unroll
    for (int i = 0; i < 4; ++i) pv_one(st[0], vf1[i >> 1][i & 1], pw1, i >> 1, i & 1);
  } else {
    // block A = 0, block B = kQB - 1
    constexpr int A = 0, B = kQB - 1;
    f32x16 sa[2] = {}, sb[2] = {};
#pragma unroll
    for (int slab = 0; slab < 2; ++slab)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) sa[slab] = qk_one(sa[slab], kf[slab][kk], qf[A][kk]);
    u32x4 vf[2][2][2];  // [slab][jj][blk]
#pragma unroll
    for (int slab = 0; slab < 2; ++slab)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
          vf[slab][jj][blk] = ld16(Vt + (32 * blk + lq) * kPitch + 16 * (2 * slab + jj) + 8 * hf);
    float sva[2][16], svb[2][16];
    unsigned pwa[2][8], pwb[2][8];
    float psa[2] = {0.f, 0.f}, psb[2] = {0.f, 0.f};
    // slab 0's weights of a block, added into O (and cleared) ahead of a
    // reference move found on its slab 1
    auto pending_a = [&] {
#pragma unroll
      for (int j = 0; j < 4; ++j) pv_one(st[A], vf[0][j >> 1][j & 1], pwa[0], j >> 1, j & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) pwa[0][j] = 0u;
    };
    auto pending_b = [&] {
#pragma unroll
      for (int j = 0; j < 4; ++j) pv_one(st[B], vf[0][j >> 1][j & 1], pwb[0], j >> 1, j & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) pwb[0][j] = 0u;
    };
    // B's S^T, each MFMA followed by a quarter slab of A's softmax
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slab = i >> 2, kk = i & 3;
      sb[slab] = qk_one(sb[slab], kf[slab][kk], qf[B][kk]);
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) scores_of(sva[slab], sa[slab], slab, last[A], st[A]);
      slab_weights<kMasked>(sva[slab], pwa[slab], psa[slab], st[A].mc, c, 2 * kk, 2 * kk + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 3) {
        if (slab == 0)
          check_reference<kMasked>(st[A], sva[0], pwa[0], psa[0], c);
        else
          check_reference<kMasked>(st[A], sva[1], pwa[1], psa[1], c, pending_a);
      }
    }
    // A's P V, each MFMA followed by a quarter slab of B's softmax
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int slab = i >> 2, jj = (i >> 1) & 1, blk = i & 1, q4 = i & 3;
      pv_one(st[A], vf[slab][jj][blk], pwa[slab], jj, blk);
      __builtin_amdgcn_sched_barrier(0);
      if (q4 == 0) scores_of(svb[slab], sb[slab], slab, last[B], st[B]);
      slab_weights<kMasked>(svb[slab], pwb[slab], psb[slab], st[B].mc, c, 2 * q4, 2 * q4 + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (q4 == 3) {
        if (slab == 0)
          check_reference<kMasked>(st[B], svb[0], pwb[0], psb[0], c);
        else
          check_reference<kMasked>(st[B], svb[1], pwb[1], psb[1], c, pending_b);
      }
    }
    // B's P V
#pragma unroll
    for (int i = 0; i < 8; ++i) pv_one(st[B], vf[i >> 2][(i >> 1) & 1][i & 1], pwb[i >> 2], (i >> 1) & 1, i & 1);
  }
}

// Pack lane's 4 values of d group g (d = 8g + 4hf + 0..3) of both lane halves
// into one 16-byte row chunk: half 0 ends with group gA = 2t, half 1 with 2t+1.
__device__ __forceinline__ u32x4 gather_row_chunk(unsigned a0, unsigned a1, unsigned b0, unsigned b1) {
  const auto x0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto x1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  return u32x4{(unsigned)x0[0], (unsigned)x1[0], (unsigned)x0[1], (unsigned)x1[1]};
}

// kQB blocks of 32 query rows per wavefront, 4 wavefronts per workgroup.
template <bool kCausal, int kQB>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_d64(AttnArgs a, float c, unsigned q_sign, int n_qblk) {
  constexpr int kRowsPerWave = 32 * kQB;
  constexpr int kRows = 4 * kRowsPerWave;  // query rows per workgroup
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * kTile];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int n_q = a.n_q;

  // ---- workgroup -> (batch*head, query block)
  int bh, qblk;
  if (kCausal) {
    // heaviest query blocks (most key tiles) are dispatched first
    const int BH = a.batch * a.heads;
    qblk = n_qblk - 1 - (int)(blockIdx.x / BH);
    bh = (int)(blockIdx.x % BH);
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
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[qb][kk] = my_q < n_q ? (ld16(src + 16 * kk) ^ q_sign) : u32x4{0, 0, 0, 0};
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
    attend_tile<false, kQB, true>(st, qf, smem, smem + kTile, no_mask, lq, hf, c);
    if (more) lstore(1);
    __syncthreads();
    t = 1;
  }
  for (; t < t_split; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) gload((t + 1) * kBN);
    const bf16* Ks = smem + (t & 1) * 2 * kTile;
    attend_tile<false, kQB>(st, qf, Ks, Ks + kTile, no_mask, lq, hf, c);
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
      attend_tile<true, kQB>(st, qf, Ks, Ks + kTile, last, lq, hf, c);
    }
    if (more) lstore((t + 1) & 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds d = 32*blk + 8*g + 4*hf + 0..3 of its query;
  // the two halves swap groups so that each lane writes two 16-byte chunks per d block.
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    const int my_q = q_wave0 + 32 * qb + lq;
    const float l_tot = sum_halves(st[qb].l);
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

}  // namespace

// Rows per wavefront: 64 (two 32-row blocks share every K/V fragment read)
// in 256-row workgroups, else 32. Measured on MI355X: 64 rows pay off for
// long query runs with little padding (longer K/V streams per workgroup) and
// for unmasked runs that fill whole 256-row workgroups (the encoder launch,
// 29 -> 27 us at N = 512); for short causal or ragged runs the 32-row form's
// finer split wins.
int attention_rows_per_wave(int n_q, bool causal) {
  const int pad256 = (n_q + 255) / 256 * 256 - n_q;
  if (!causal && n_q >= 512 && pad256 == 0) return 64;
  return (n_q >= 2048 && pad256 * 16 <= n_q) ? 64 : 32;
}

template <int kQB>
static void launch_qb(const AttnArgs& a, hipStream_t stream, float c, unsigned q_sign) {
  const int rows = 4 * 32 * kQB;
  const int n_qblk = (a.n_q + rows - 1) / rows;
  const dim3 grid((unsigned)(n_qblk * a.batch * a.heads));
  if (a.causal)
    hipLaunchKernelGGL((attn_fwd_bf16_d64<true, kQB>), grid, dim3(256), 0, stream, a, c, q_sign, n_qblk);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_d64<false, kQB>), grid, dim3(256), 0, stream, a, c, q_sign, n_qblk);
}

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t stream) {
  const float kLog2e = 1.4426950408889634f;
  const float c = fabsf(a.scale) * kLog2e;
  const unsigned q_sign = a.scale < 0.f ? 0x80008000u : 0u;  // negate Q exactly: scale*s = |scale|*(-q).k
  if (attention_rows_per_wave(a.n_q, a.causal != 0) == 64)
    launch_qb<2>(a, stream, c, q_sign);
  else
    launch_qb<1>(a, stream, c, q_sign);
  return hipGetLastError();
}

}  // namespace mha
