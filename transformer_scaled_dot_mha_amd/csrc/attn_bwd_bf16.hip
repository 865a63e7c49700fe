// Scaled dot-product attention backward, bf16 in/out, d = 64, gfx950.
//
// The gradient through the softmax that the pages give as the reason for the
// 1/sqrt(d_k) scale ("32 Transformer" (ml-canon-en.vercel.app), "Why we divide
// by sqrt(dk)"; "The Transformer" (hoshank.vercel.app), "The Breakthrough"),
// by the chain rule through O = P V, the row softmax and S = scale Q K^T:
//   dV = P^T dO,  dP = dO V^T,  dS_ij = P_ij (dP_ij - delta_i),
//   delta_i = dO_i . O_i,  dQ = scale dS K,  dK = scale dS^T Q,
// with P recomputed from the forward's log-sum-exp, P_ij = exp(scale q_i.k_j - lse_i).
//
// Two launches and no atomics (deterministic results):
//   attn_bwd_dq_bf16   workgroup = 128 query rows (4 wavefronts x 32) of one
//                      (batch, head); streams 64-key tiles of K and V. Also
//                      writes delta for the second launch.
//   attn_bwd_dkdv_bf16 workgroup = 128 key rows (4 x 32); streams 64-query
//                      tiles of Q and dO with their lse and delta.
// Each computes S and dP again (the price of having no atomics): 12 + 16
// matrix products per 32x32 block of pairs against the 20 of the gradient
// itself.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, fp32 accumulate). As in the
// forward kernel, products are arranged so that an accumulator, converted to
// bf16, is already the B operand of the next product:
//   dQ launch:  S^T = K Q^T and dP^T = V dO^T (A = K or V rows from LDS in a
//     permuted row order, B = the wavefront's Q or dO rows in registers): lane
//     l holds query l%32 and 16 keys, registers 0-7 and 8-15 being 8
//     consecutive keys each. dS^T from them is the B operand of
//     dQ^T = K^T dS^T, with K^T ([d][key]) staged in LDS.
//   dK/dV launch: S = Q K^T and dP = dO V^T (A = Q or dO rows from LDS,
//     permuted; B = the wavefront's K or V rows in registers): lane l holds
//     key l%32 and 16 queries. P and dS from them are the B operands of
//     dV^T = dO^T P and dK^T = Q^T dS, with dO^T and Q^T staged in LDS.
// P and dS are rounded to bf16 for the products (P is in the forward too);
// the exponent, the row terms and every accumulation are fp32.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "kernels.h"

namespace mha {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlk = 64;     // rows per streamed tile
constexpr int kPitch = 72;   // LDS row pitch in bf16 elements (144 bytes)
constexpr int kTileElems = kBlk * kPitch;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufferFlags = 0x00020000;  // raw buffer descriptor word 3 (32-bit data format)

__device__ __forceinline__ u32x4 ld16(const bf16* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ f32x16 mfma(f32x16 acc, const u32x4& a, const u32x4& b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
}

// LDS row of row offset kappa (0..31) of a 32-row slab: accumulator register r
// of lane half hf then holds row 16*(r/8) + 8*hf + r%8 of the slab.
__device__ __forceinline__ int perm_row(int kappa) {
  return 8 * (2 * (kappa >> 4) + ((kappa >> 2) & 1)) + 4 * ((kappa >> 3) & 1) + (kappa & 3);
}
// Slab row held by accumulator register r of lane half hf.
__device__ __forceinline__ int acc_row(int r, int hf) { return 16 * (r >> 3) + 8 * hf + (r & 7); }

__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                                  false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Lane's 4 values of d group g of both lane halves -> one 16-byte row chunk.
__device__ __forceinline__ u32x4 gather_row_chunk(unsigned a0, unsigned a1, unsigned b0, unsigned b1) {
  const auto x0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto x1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  return u32x4{(unsigned)x0[0], (unsigned)x1[0], (unsigned)x0[1], (unsigned)x1[1]};
}

// Store a 32-row x 64 block held transposed in two accumulators (lane: row
// l%32, d = 32*blk + 8*g + 4*hf + 0..3), times `mul`, as bf16 rows; a lane
// with `zero` set stores zeros whatever its accumulators hold.
__device__ __forceinline__ void store_rows(bf16* row_ptr, bool ok, const f32x16& a0, const f32x16& a1, float mul,
                                           int hf, bool zero = false) {
  unsigned w[2][4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    w[0][g][0] = zero ? 0u : pack_bf16(a0[4 * g] * mul, a0[4 * g + 1] * mul);
    w[0][g][1] = zero ? 0u : pack_bf16(a0[4 * g + 2] * mul, a0[4 * g + 3] * mul);
    w[1][g][0] = zero ? 0u : pack_bf16(a1[4 * g] * mul, a1[4 * g + 1] * mul);
    w[1][g][1] = zero ? 0u : pack_bf16(a1[4 * g + 2] * mul, a1[4 * g + 3] * mul);
  }
  u32x4 chunk[2][2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
      chunk[blk][tt] = gather_row_chunk(w[blk][2 * tt][0], w[blk][2 * tt][1], w[blk][2 * tt + 1][0],
                                        w[blk][2 * tt + 1][1]);
  if (ok) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        *reinterpret_cast<u32x4*>(row_ptr + 32 * blk + 8 * (2 * tt + hf)) = chunk[blk][tt];
  }
}

__device__ __forceinline__ float lse_base2(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// Workgroup -> (batch*head, block). Causal: the heaviest blocks first; else
// each XCD (workgroups are dealt round-robin to the 8) gets a contiguous run of
// logical ids, so the blocks of one (batch, head) share its L2.
__device__ __forceinline__ void map_block(int n_blk, int BH, bool causal, bool heavy_first_is_last, int& bh, int& blk) {
  if (causal) {
    const int r = (int)(blockIdx.x / BH);
    blk = heavy_first_is_last ? n_blk - 1 - r : r;
    bh = (int)(blockIdx.x % BH);
  } else {
    const int total = gridDim.x, id = blockIdx.x;
    const int per = total >> 3, rem = total & 7, x = id & 7, slot = id >> 3;
    const int logical = (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
    bh = logical / n_blk;
    blk = logical - bh * n_blk;
  }
}

// Pair-row staging of a 64-row tile: thread t loads rows 2*(t%32) and
// 2*(t%32)+1, 16-byte chunk t/32, through a buffer descriptor whose record
// count ends at the last valid row (rows past it read as zero).
struct PairStage {
  int row, chunk;
  int off0, off1;  // byte offsets of the two rows' chunk
  __device__ void init(int tid, int64_t row_stride) {
    row = (tid & 31) * 2;
    chunk = tid >> 5;
    off0 = (int)(((int64_t)row * row_stride + 8 * chunk) * 2);
    off1 = (int)(((int64_t)(row + 1) * row_stride + 8 * chunk) * 2);
  }
  __device__ void load(const bf16* base, int64_t row_stride, int valid, u32x4 (&r)[2]) const {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)base, (short)0, valid > 0 ? (int)((valid - 1) * row_stride * 2 + 2 * 64) : 0, kBufferFlags);
    r[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off0, 0, 0));
    r[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off1, 0, 0));
  }
  // row-major copy in permuted row order (per 32-row slab)
  __device__ void store_rows(bf16* lds, const u32x4 (&r)[2]) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int rr = row + i;
      *reinterpret_cast<u32x4*>(lds + (32 * (rr >> 5) + perm_row(rr & 31)) * kPitch + 8 * chunk) = r[i];
    }
  }
  // transposed copy [d][row], two rows per 32-bit word
  __device__ void store_transposed(bf16* lds, const u32x4 (&r)[2]) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned word = __builtin_amdgcn_perm(r[1][e >> 1], r[0][e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
      *reinterpret_cast<unsigned*>(lds + (8 * chunk + e) * kPitch + row) = word;
    }
  }
};

// ---------------------------------------------------------------- dQ and delta
template <bool kCausal>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_bf16(BwdArgs a, float c, int n_qblk) {
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 3 * kTileElems];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 31, hf = lane >> 5;
  int bh, qblk;
  map_block(n_qblk, a.batch * a.heads, kCausal, true, bh, qblk);
  const int b = bh / a.heads, h = bh - b * a.heads;
  const int n_q = a.n_q;
  const int n_k = a.kv_len != nullptr ? min(max(a.kv_len[b], 0), a.n_k) : a.n_k;
  const bf16* qp = static_cast<const bf16*>(a.q) + b * a.q_s[0] + h * a.q_s[1];
  const bf16* kp = static_cast<const bf16*>(a.k) + b * a.k_s[0] + h * a.k_s[1];
  const bf16* vp = static_cast<const bf16*>(a.v) + b * a.v_s[0] + h * a.v_s[1];
  const bf16* op = static_cast<const bf16*>(a.o) + b * a.o_s[0] + h * a.o_s[1];
  const bf16* dop = static_cast<const bf16*>(a.d_o) + b * a.do_s[0] + h * a.do_s[1];
  bf16* dqp = static_cast<bf16*>(a.dq) + b * a.dq_s[0] + h * a.dq_s[1];

  const int q_wave0 = qblk * 128 + 32 * wave;
  const int my_q = q_wave0 + lq;
  const bool row_ok = my_q < n_q;
  const int q_row = min(my_q, n_q - 1);

  // this lane's slices (d = 16*kk + 8*hf + 0..7) of its query's Q, dO and O rows
  u32x4 qf[4], dof[4];
  float delta = 0.f;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int col = 16 * kk + 8 * hf;
    qf[kk] = row_ok ? ld16(qp + (int64_t)q_row * a.q_s[2] + col) : u32x4{0, 0, 0, 0};
    dof[kk] = row_ok ? ld16(dop + (int64_t)q_row * a.do_s[2] + col) : u32x4{0, 0, 0, 0};
    const u32x4 of = row_ok ? ld16(op + (int64_t)q_row * a.o_s[2] + col) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      delta = fmaf(__builtin_bit_cast(float, dof[kk][i] << 16), __builtin_bit_cast(float, of[i] << 16), delta);
      delta = fmaf(__builtin_bit_cast(float, dof[kk][i] & 0xffff0000u), __builtin_bit_cast(float, of[i] & 0xffff0000u),
                   delta);
    }
  }
  delta = sum_halves(delta);
  const float lse2 = row_ok ? lse_base2(a.lse[(int64_t)bh * n_q + my_q]) : INFINITY;
  if (row_ok && hf == 0) a.delta[(int64_t)bh * n_q + my_q] = delta;

  f32x16 dq0 = {}, dq1 = {};
  const int kv_end = kCausal ? min(n_k, qblk * 128 + 128) : n_k;
  const int ntiles = (kv_end + kBlk - 1) / kBlk;

  PairStage ks, vs;
  ks.init(tid, a.k_s[2]);
  vs.init(tid, a.v_s[2]);
  u32x4 kr[2], vr[2];
  auto gload = [&](int k0) {
    const int valid = min(n_k - k0, kBlk);
    ks.load(kp + (int64_t)k0 * a.k_s[2], a.k_s[2], valid, kr);
    vs.load(vp + (int64_t)k0 * a.v_s[2], a.v_s[2], valid, vr);
  };
  auto lstore = [&](int buf) {
    bf16* base = smem + buf * 3 * kTileElems;
    ks.store_rows(base, kr);
    ks.store_transposed(base + kTileElems, kr);
    vs.store_rows(base + 2 * kTileElems, vr);
  };

  // One 64-key tile. Tiles that straddle the causal diagonal or hold the end
  // of the keys mask their pairs (a key past n_k is a zero row, but its
  // unmasked weight exp(-lse) can overflow); the others need no mask.
  auto tile = [&](int k0, const bf16* Ks, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    const bf16* Kt = Ks + kTileElems;
    const bf16* Vs = Ks + 2 * kTileElems;
    // keys of this lane's registers: k0 + 32*slab + acc_row(r, hf)
    const int last = (kCausal ? min(n_k - 1, my_q) : n_k - 1) - k0;
#pragma unroll
    for (int slab = 0; slab < 2; ++slab) {
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        s = mfma(s, ld16(Ks + (32 * slab + lq) * kPitch + 16 * kk + 8 * hf), qf[kk]);
        dp = mfma(dp, ld16(Vs + (32 * slab + lq) * kPitch + 16 * kk + 8 * hf), dof[kk]);
      }
      unsigned pw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float ds2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * i + e;
          float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lse2));
          if (kMasked) p = 32 * slab + acc_row(r, hf) <= last ? p : 0.f;
          ds2[e] = p * (dp[r] - delta);
        }
        pw[i] = pack_bf16(ds2[0], ds2[1]);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const u32x4 bs = u32x4{pw[4 * jj], pw[4 * jj + 1], pw[4 * jj + 2], pw[4 * jj + 3]};
        dq0 = mfma(dq0, ld16(Kt + lq * kPitch + 16 * (2 * slab + jj) + 8 * hf), bs);
        dq1 = mfma(dq1, ld16(Kt + (32 + lq) * kPitch + 16 * (2 * slab + jj) + 8 * hf), bs);
      }
    }
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  // tiles before t_split lie wholly below every query of the workgroup and
  // before the end of the keys
  const int t_split = min(kCausal ? qblk * (128 / kBlk) : ntiles, n_k / kBlk);
  int t = 0;
  for (; t < t_split; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) gload((t + 1) * kBlk);
    tile(t * kBlk, smem + (t & 1) * 3 * kTileElems, std::false_type());
    if (more) lstore((t + 1) & 1);
    __syncthreads();
  }
  for (; t < ntiles; ++t) {
    const int k0 = t * kBlk;
    const bool more = t + 1 < ntiles;
    if (more) gload(k0 + kBlk);
    if (!kCausal || k0 <= q_wave0 + 31)  // uniform over the wavefront
      tile(k0, smem + (t & 1) * 3 * kTileElems, std::true_type());
    if (more) lstore((t + 1) & 1);
    __syncthreads();
  }
  store_rows(dqp + (int64_t)q_row * a.dq_s[2], row_ok, dq0, dq1, a.scale, hf);
}

// ---------------------------------------------------------------- dK and dV
template <bool kCausal>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_bf16(BwdArgs a, float c, int n_kblk) {
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 4 * kTileElems];
  __shared__ __attribute__((aligned(16))) float s_lse[2][kBlk], s_delta[2][kBlk];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 31, hf = lane >> 5;
  int bh, kblk;
  map_block(n_kblk, a.batch * a.heads, kCausal, false, bh, kblk);
  const int b = bh / a.heads, h = bh - b * a.heads;
  const int n_q = a.n_q;
  const int n_k = a.kv_len != nullptr ? min(max(a.kv_len[b], 0), a.n_k) : a.n_k;
  const bf16* qp = static_cast<const bf16*>(a.q) + b * a.q_s[0] + h * a.q_s[1];
  const bf16* kp = static_cast<const bf16*>(a.k) + b * a.k_s[0] + h * a.k_s[1];
  const bf16* vp = static_cast<const bf16*>(a.v) + b * a.v_s[0] + h * a.v_s[1];
  const bf16* dop = static_cast<const bf16*>(a.d_o) + b * a.do_s[0] + h * a.do_s[1];
  bf16* dkp = static_cast<bf16*>(a.dk) + b * a.dk_s[0] + h * a.dk_s[1];
  bf16* dvp = static_cast<bf16*>(a.dv) + b * a.dv_s[0] + h * a.dv_s[1];
  const float* lse_row = a.lse + (int64_t)bh * n_q;
  const float* delta_row = a.delta + (int64_t)bh * n_q;

  const int k_wave0 = kblk * 128 + 32 * wave;
  const int my_k = k_wave0 + lq;
  const bool key_ok = my_k < n_k;  // keys past a padded length get zero gradients
  const int k_row = min(my_k, max(n_k, 1) - 1);

  u32x4 kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int col = 16 * kk + 8 * hf;
    kf[kk] = key_ok ? ld16(kp + (int64_t)k_row * a.k_s[2] + col) : u32x4{0, 0, 0, 0};
    vf[kk] = key_ok ? ld16(vp + (int64_t)k_row * a.v_s[2] + col) : u32x4{0, 0, 0, 0};
  }
  f32x16 dv0 = {}, dv1 = {}, dk0 = {}, dk1 = {};

  // queries before the block's first key see none of its keys under the causal mask
  const int q_begin = kCausal ? kblk * 128 : 0;
  const int n_tiles = kblk * 128 < n_k ? (n_q - q_begin + kBlk - 1) / kBlk : 0;

  PairStage qs, ds;
  qs.init(tid, a.q_s[2]);
  ds.init(tid, a.do_s[2]);
  u32x4 qr[2], dr[2];
  float lr = 0.f, dl = 0.f;
  auto gload = [&](int q0) {
    const int valid = min(n_q - q0, kBlk);
    qs.load(qp + (int64_t)q0 * a.q_s[2], a.q_s[2], valid, qr);
    ds.load(dop + (int64_t)q0 * a.do_s[2], a.do_s[2], valid, dr);
    if (tid < kBlk) {
      const int qi = q0 + tid;
      lr = qi < n_q ? lse_base2(lse_row[qi]) : INFINITY;
      dl = qi < n_q ? delta_row[qi] : 0.f;
    }
  };
  auto lstore = [&](int buf) {
    bf16* base = smem + buf * 4 * kTileElems;
    qs.store_rows(base, qr);
    qs.store_transposed(base + kTileElems, qr);
    ds.store_rows(base + 2 * kTileElems, dr);
    ds.store_transposed(base + 3 * kTileElems, dr);
    if (tid < kBlk) {
      s_lse[buf][tid] = lr;
      s_delta[buf][tid] = dl;
    }
  };

  // One 64-query tile. Keys past a padded length are zeroed at the store, and
  // queries past n_q have lse = +inf (weight 0), so only tiles that straddle
  // the causal diagonal mask pairs.
  auto tile = [&](int q0, int buf, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    const bf16* Qs = smem + buf * 4 * kTileElems;
    const bf16* Qt = Qs + kTileElems;
    const bf16* Ds = Qs + 2 * kTileElems;
    const bf16* Dt = Qs + 3 * kTileElems;
#pragma unroll
    for (int slab = 0; slab < 2; ++slab) {
      f32x16 s = {}, dp = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        s = mfma(s, ld16(Qs + (32 * slab + lq) * kPitch + 16 * kk + 8 * hf), kf[kk]);
        dp = mfma(dp, ld16(Ds + (32 * slab + lq) * kPitch + 16 * kk + 8 * hf), vf[kk]);
      }
      // lse and delta of this lane's 16 queries: two runs of 8
      float lq16[16], dq16[16];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int base = 32 * slab + 16 * half + 8 * hf;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&s_lse[buf][base]);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&s_lse[buf][base + 4]);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&s_delta[buf][base]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&s_delta[buf][base + 4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lq16[8 * half + i] = l0[i];
          lq16[8 * half + 4 + i] = l1[i];
          dq16[8 * half + i] = d0[i];
          dq16[8 * half + 4 + i] = d1[i];
        }
      }
      unsigned pp[8], pd[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float p2[2], d2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * i + e;
          float p = __builtin_amdgcn_exp2f(fmaf(s[r], c, -lq16[r]));
          if (kMasked) p = my_k <= q0 + 32 * slab + acc_row(r, hf) ? p : 0.f;
          p2[e] = p;
          d2[e] = p * (dp[r] - dq16[r]);
        }
        pp[i] = pack_bf16(p2[0], p2[1]);
        pd[i] = pack_bf16(d2[0], d2[1]);
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const u32x4 bp = u32x4{pp[4 * jj], pp[4 * jj + 1], pp[4 * jj + 2], pp[4 * jj + 3]};
        const u32x4 bd = u32x4{pd[4 * jj], pd[4 * jj + 1], pd[4 * jj + 2], pd[4 * jj + 3]};
        const int col = 16 * (2 * slab + jj) + 8 * hf;
        dv0 = mfma(dv0, ld16(Dt + lq * kPitch + col), bp);
        dv1 = mfma(dv1, ld16(Dt + (32 + lq) * kPitch + col), bp);
        dk0 = mfma(dk0, ld16(Qt + lq * kPitch + col), bd);
        dk1 = mfma(dk1, ld16(Qt + (32 + lq) * kPitch + col), bd);
      }
    }
  };

  if (n_tiles > 0) {
    gload(q_begin);
    lstore(0);
  }
  __syncthreads();
  // causal: the first two query tiles straddle the block's diagonal; from the
  // third on every query lies at or past every key of the block
  const int t_masked = kCausal ? min(n_tiles, 128 / kBlk) : 0;
  int t = 0;
  for (; t < t_masked; ++t) {
    const int q0 = q_begin + t * kBlk;
    const bool more = t + 1 < n_tiles;
    if (more) gload(q0 + kBlk);
    if (q0 + kBlk - 1 >= k_wave0) tile(q0, t & 1, std::true_type());  // uniform over the wavefront
    if (more) lstore((t + 1) & 1);
    __syncthreads();
  }
  for (; t < n_tiles; ++t) {
    const int q0 = q_begin + t * kBlk;
    const bool more = t + 1 < n_tiles;
    if (more) gload(q0 + kBlk);
    tile(q0, t & 1, std::false_type());
    if (more) lstore((t + 1) & 1);
    __syncthreads();
  }
  // keys past a padded length were never masked above (their K and V rows
  // are zero): they store exactly zero, selected, not multiplied, since
  // their unmasked weights can overflow
  const bool store_ok = my_k < a.n_k;
  const int out_row = min(my_k, a.n_k - 1);
  store_rows(dvp + (int64_t)out_row * a.dv_s[2], store_ok, dv0, dv1, 1.0f, hf, !key_ok);
  store_rows(dkp + (int64_t)out_row * a.dk_s[2], store_ok, dk0, dk1, a.scale, hf, !key_ok);
}

}  // namespace

hipError_t launch_attention_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  const float c = a.scale * kLog2e;
  const int BH = a.batch * a.heads;
  const int n_qblk = (a.n_q + 127) / 128, n_kblk = (a.n_k + 127) / 128;
  const dim3 gq((unsigned)(n_qblk * BH)), gk((unsigned)(n_kblk * BH));
  if (a.causal)
    hipLaunchKernelGGL((attn_bwd_dq_bf16<true>), gq, dim3(256), 0, stream, a, c, n_qblk);
  else
    hipLaunchKernelGGL((attn_bwd_dq_bf16<false>), gq, dim3(256), 0, stream, a, c, n_qblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.causal)
    hipLaunchKernelGGL((attn_bwd_dkdv_bf16<true>), gk, dim3(256), 0, stream, a, c, n_kblk);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_bf16<false>), gk, dim3(256), 0, stream, a, c, n_kblk);
  return hipGetLastError();
}

}  // namespace mha
