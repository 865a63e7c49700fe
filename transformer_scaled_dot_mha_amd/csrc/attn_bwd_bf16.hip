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
//                      writes -delta and lse log2(e) for the second launch.
//   attn_bwd_dkdv_bf16 workgroup = 128 key rows (4 x 32); streams 64-query
//                      tiles of Q and dO with those two rows.
// Each computes S and dP again (the price of having no atomics): 12 + 16
// matrix products per 32x32 block of pairs against the 20 of the gradient
// itself.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, fp32 accumulate). As in the
// forward kernel, products are arranged so that an accumulator, converted to
// bf16, is already the B operand of the next product:
//   dQ launch:  S^T = K Q^T and dP^T = V dO^T (A = K or V rows from LDS, rows
//     read in a permuted order, B = the wavefront's Q or dO rows in registers):
//     lane l holds query l%32 and 16 keys, registers 0-7 and 8-15 being 8
//     consecutive keys each. dS^T from them is the B operand of
//     dQ^T = K^T dS^T, the K^T operand read from K's rows with transposing
//     LDS reads.
//   dK/dV launch: S = Q K^T and dP = dO V^T (A = Q or dO rows from LDS,
//     permuted; B = the wavefront's K or V rows in registers): lane l holds
//     key l%32 and 16 queries. P and dS from them are the B operands of
//     dV^T = dO^T P and dK^T = Q^T dS (dO^T, Q^T by transposing reads).
// P and dS are rounded to bf16 for the products (P is in the forward too);
// the exponent, the row terms and every accumulation are fp32. dP starts from
// -delta as its accumulator's initial value, so that it ends as dP - delta.
//
// Staging: the streamed tiles go from global memory straight into LDS with
// buffer loads that write LDS, into a ring of four stages (each a 64-row tile
// of both streamed matrices); the loads of tile t + 3 are issued while tile t
// is processed (about two tiles of work before they are first read), and one
// wait plus barrier per tile makes the next tile visible. Rows keep
// their 128-byte layout with the 16-byte chunk c of row r at c ^ swz(r), so
// that both the row reads and the transposing reads hit distinct banks.
//
// Schedule: a wavefront's work is a sequence of units u, each a 32-row slab
// of a tile against its own 32 rows: A(u) (the S and dP products), V(u) (the
// per-element exponent and dS, VALU) and B(u) (the gradient products). VALU
// work issued right after a matrix-core instruction of the same wavefront can
// overlap it, so iteration u runs the products B(u-1) and A(u+1) with the
// element steps of V(u) spread between them, and the three steps of each
// element (x = s c - lse2; p = exp2(x); dS = p (dP - delta), pack) are
// staggered so that consecutive instructions do not wait on each other.
// The loop body covers two tiles, so that every stage offset is a constant
// within it; the tiles past the last (to an even count) read as zeros and add
// nothing.
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
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int N>
using ic = std::integral_constant<int, N>;

constexpr int kBlk = 64;                  // rows per streamed tile
constexpr int kRowB = 128;                // a streamed row in LDS: 64 bf16
constexpr int kTileB = kBlk * kRowB;      // 8 KB per tile of one matrix
constexpr int kStageB = 2 * kTileB;       // the two streamed matrices' tiles
constexpr int kStatB = kBlk * 4;          // 64 floats
constexpr int kStages = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBufferFlags = 0x00020000;  // raw buffer descriptor word 3 (32-bit data format)

__device__ __forceinline__ u32x4 ld16(const bf16* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__device__ __forceinline__ f32x16 mfma(const f32x16& acc, const u32x4& a, const u32x4& b) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc, 0, 0, 0);
}

// Row of a 32-row slab that the A operand's row kappa reads: accumulator
// register r of lane half hf then holds slab row 16*(r/8) + 8*hf + r%8
// (the map swaps bits 2 and 3, so it is its own inverse).
__device__ __forceinline__ int perm_row(int kappa) {
  return 8 * (2 * (kappa >> 4) + ((kappa >> 2) & 1)) + 4 * ((kappa >> 3) & 1) + (kappa & 3);
}

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

// ------------------------------------------------------------ staging helpers
// LDS position of 16-byte chunk c of tile row r: c ^ swz(r), with bits
// (r3, r0 ^ r2, r1): the 16 row reads of a quarter wavefront (rows
// perm_row(0..15)) and the 4-row x 64-byte transposing reads of a half
// wavefront both fall on distinct banks.
__device__ __forceinline__ int swz(int r) {
  return ((r >> 3) & 1) | (((r ^ (r >> 2)) & 1) << 1) | (((r >> 1) & 1) << 2);
}
__device__ __forceinline__ unsigned lds_addr(const void* p) { return (unsigned)(size_t)(const lds_char*)p; }
// 16 (or 4) bytes per lane from a raw buffer into LDS at lds_byte + 16 (or 4)
// times the lane; offsets past the buffer's record write zeros. The
// wave-uniform LDS base goes in m0 through the asm's {m0} operand, so the
// compiler sets m0 itself and knows the register is taken.
__device__ __forceinline__ void dma16(u32x4 rsrc, unsigned voff, unsigned lds_byte) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_byte) : "memory");
}
__device__ __forceinline__ void dma4(u32x4 rsrc, unsigned voff, unsigned lds_byte) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_byte) : "memory");
}
// Raw buffer descriptor (stride 0) over `bytes` bytes from base.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long b = (unsigned long long)base;
  return u32x4{(unsigned)__builtin_amdgcn_readfirstlane((int)(unsigned)b),
               (unsigned)__builtin_amdgcn_readfirstlane((int)((unsigned)(b >> 32) & 0xffffu)),
               (unsigned)__builtin_amdgcn_readfirstlane((int)bytes), (unsigned)kBufferFlags};
}
// Wait until at most kN of this wavefront's loads are in flight, then meet the
// workgroup (the loads are in order, so the older tiles have landed).
template <int kN>
__device__ __forceinline__ void wait_loads_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kN) : "memory");
}
__device__ __forceinline__ u32x4 lds16(const lds_char* p) { return *(const lds_u32x4*)p; }
__device__ __forceinline__ f32x4 ldsf4(const lds_char* p) { return *(const lds_f32x4*)p; }
// Two transposing reads: rows +0..3 (p0) and +4..7 (p1) of a column group.
__device__ __forceinline__ u32x4 lds_tr(const lds_char* p0, const lds_char* p1) {
  const v4i16 w0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
  const v4i16 w1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1);
  const u32x2 a0 = __builtin_bit_cast(u32x2, w0), a1 = __builtin_bit_cast(u32x2, w1);
  return u32x4{a0[0], a0[1], a1[0], a1[1]};
}

// Per-lane LDS fragment bases at stage 0.
struct Ptrs {
  const lds_char* pa[4];     // row operand: slab row perm_row(lq), chunk 2 kk + hf
  const lds_char* pt[2][2];  // transposed operand [32-column block][read]
  const lds_char* ps;        // row statistics (dK/dV launch)
};
// Row operand: the lane reads slab row perm_row(lq), 16-byte chunk 2 kk + hf.
// Transposed operand: in 16-lane group gi, lane lj reads row 8 (gi >> 1) +
// 4 rd + lj / 4 (plus the slab and 16-row step), columns 32 blk + 16 (gi & 1)
// + 4 (lj % 4) + 0..3, so that lane l receives 4 consecutive rows of column
// 32 blk + l % 32.
__device__ __forceinline__ Ptrs fragment_bases(const char* smem, int lane) {
  const int lq = lane & 31, hf = lane >> 5;
  const lds_char* lds0 = (const lds_char*)smem;
  Ptrs p;
  const int pr = perm_row(lq), sw = swz(pr);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) p.pa[kk] = lds0 + pr * kRowB + 16 * ((2 * kk + hf) ^ sw);
  const int gi = lane >> 4, lj = lane & 15;
  const int tc = 2 * (gi & 1) + ((lj & 3) >> 1);
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int tr = 8 * (gi >> 1) + 4 * rd + (lj >> 2), tsw = swz(tr);
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) p.pt[blk][rd] = lds0 + tr * kRowB + 16 * ((4 * blk + tc) ^ tsw) + 8 * (lj & 1);
  }
  p.ps = lds0 + kStages * kStageB + 32 * hf;
  return p;
}
// The bases of stage pair `pair` (stages 2 pair and 2 pair + 1).
__device__ __forceinline__ Ptrs pair_bases(const Ptrs& b, int pair) {
  Ptrs r;
  const int o = pair * 2 * kStageB, os = pair * 2 * 2 * kStatB;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) r.pa[kk] = b.pa[kk] + o;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    r.pt[blk][0] = b.pt[blk][0] + o;
    r.pt[blk][1] = b.pt[blk][1] + o;
  }
  r.ps = b.ps + os;
  return r;
}
// Row-operand fragment kk of matrix `mat` (0 or 1), slab J, stage ST.
template <int ST, int J>
__device__ __forceinline__ u32x4 row_frag(const Ptrs& P, int mat, int kk) {
  return lds16(P.pa[kk] + ST * kStageB + mat * kTileB + 32 * J * kRowB);
}
// Transposed fragment of matrix `mat`, column block blk, 16-row step jj of slab J.
template <int ST, int J>
__device__ __forceinline__ u32x4 tr_frag(const Ptrs& P, int mat, int blk, int jj) {
  const int off = ST * kStageB + mat * kTileB + (32 * J + 16 * jj) * kRowB;
  return lds_tr(P.pt[blk][0] + off, P.pt[blk][1] + off);
}

// Element step q (0..47) of a unit's 16 elements: type 0 (x = s c - lse2),
// 1 (p = exp2(x), masked) or 2 (dS, packing), in the order type 0 of element
// g, type 1 of g - 1, type 2 of g - 2 for g = 0..17.
__device__ __forceinline__ void elem_step(int q, int& type, int& r) {
  int g, t;
  if (q < 1) {
    g = 0;
    t = 0;
  } else if (q < 3) {
    g = 1;
    t = q - 1;
  } else if (q < 45) {
    g = 2 + (q - 3) / 3;
    t = (q - 3) % 3;
  } else {
    g = q < 47 ? 16 : 17;
    t = q < 47 ? q - 44 : 2;
  }
  type = t;
  r = g - t;
}

struct Unit {
  f32x16 s, dp;
};

// ---------------------------------------------------------------- dQ and delta
template <bool kCausal>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_bf16(BwdArgs a, float c, int n_qblk) {
  __shared__ __attribute__((aligned(16))) char smem[kStages * kStageB];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 31, hf = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
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
  // rows for the dK/dV launch: -delta, then lse log2(e)
  if (row_ok && hf == 0) a.delta[(int64_t)bh * n_q + my_q] = -delta;
  if (row_ok && hf == 1) a.delta[((int64_t)a.batch * a.heads + bh) * n_q + my_q] = lse2;

  f32x16 dq0 = {}, dq1 = {};
  const int kv_end = kCausal ? min(n_k, qblk * 128 + 128) : n_k;
  const int ntiles = (kv_end + kBlk - 1) / kBlk;

  if (ntiles > 0) {  // workgroup-uniform
    constexpr int kDma = 4;  // loads per wavefront per tile
    const int64_t ks2 = a.k_s[2], vs2 = a.v_s[2];
    // load i of wavefront w fills tile rows 16 w + 8 i + lane / 8, LDS
    // position lane % 8, which holds chunk (lane % 8) ^ swz(row)
    unsigned kdo[2], vdo[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 16 * wave + 8 * i + (lane >> 3);
      const int ch = (lane & 7) ^ swz(row);
      kdo[i] = (unsigned)((row * ks2 + 8 * ch) * 2);
      vdo[i] = (unsigned)((row * vs2 + 8 * ch) * 2);
    }
    const unsigned smem_lds = lds_addr(smem);
    // tile t (keys 64 t..) into stage t % 4; rows past the keys read as zero
    auto dma_tile = [&](int t) {
      const int k0 = t * kBlk;
      const int valid = max(min(n_k - k0, kBlk), 0);
      const u32x4 rk = make_rsrc(kp + (int64_t)k0 * ks2, valid > 0 ? (unsigned)(((valid - 1) * ks2 + 64) * 2) : 0u);
      const u32x4 rv = make_rsrc(vp + (int64_t)k0 * vs2, valid > 0 ? (unsigned)(((valid - 1) * vs2 + 64) * 2) : 0u);
      const unsigned sb = smem_lds + (unsigned)((t & (kStages - 1)) * kStageB);
      dma16(rk, kdo[0], sb + (unsigned)((16 * wave_u) * kRowB));
      dma16(rk, kdo[1], sb + (unsigned)((16 * wave_u + 8) * kRowB));
      dma16(rv, vdo[0], sb + (unsigned)(kTileB + (16 * wave_u) * kRowB));
      dma16(rv, vdo[1], sb + (unsigned)(kTileB + (16 * wave_u + 8) * kRowB));
    };
    const Ptrs base = fragment_bases(smem, lane);

    // dP^T starts from -delta (the lane's query): the same 16 values every unit
    f32x16 dinit;
#pragma unroll
    for (int r = 0; r < 16; ++r) dinit[r] = -delta;

    // B(u) product m (0..3): dQ^T block m & 1 over the 16-key step m >> 1
    auto b_mfma = [&](const u32x4 (&D)[2], int m, const u32x4& fr) {
      if ((m & 1) == 0)
        dq0 = mfma(dq0, fr, D[m >> 1]);
      else
        dq1 = mfma(dq1, fr, D[m >> 1]);
    };
    // A(u) product m (0..7): S^T (even m) or dP^T (odd m), d step m >> 1
    auto a_mfma = [&](Unit& U, int m, const u32x4& fr) {
      const int kk = m >> 1;
      if (m & 1)
        U.dp = mfma(kk == 0 ? dinit : U.dp, fr, dof[kk]);
      else
        U.s = mfma(kk == 0 ? f32x16{} : U.s, fr, qf[kk]);
    };
    // element steps of V(u); register r holds key 16 (r >> 3) + 8 hf + (r & 7)
    // of the slab, kept where that is <= lim (masked tiles)
    float ex[16], ep[16];
    auto el_step = [&](const Unit& U, u32x4 (&D)[2], int q, auto maskc, int lim) {
      int type, r;
      elem_step(q, type, r);
      if (type == 0) {
        ex[r] = fmaf(U.s[r], c, -lse2);
      } else if (type == 1) {
        float p = __builtin_amdgcn_exp2f(ex[r]);
        if (decltype(maskc)::value) p = 16 * (r >> 3) + (r & 7) <= lim ? p : 0.f;
        ep[r] = p;
      } else {
        ep[r] = ep[r] * U.dp[r];
        if (r & 1) D[r >> 3][(r >> 1) & 3] = pack_bf16(ep[r - 1], ep[r]);
      }
    };

    // Iteration u = (t, J): B(u-1) in slots 0-3, A(u+1) in slots 4-11, four
    // element steps of V(u) after each; fragments are read two slots ahead.
    // PB/PA/PC: bases of the stage pairs holding u-1's, u+1's and u's tiles.
    auto iter = [&](int t, auto jc, auto maskc, auto firstc, const Ptrs& PB, auto sbc, const Ptrs& PA, auto sac,
                    const Ptrs& PC, auto scc, Unit& cur, Unit& nxt, u32x4 (&D)[2], const u32x4 (&DP)[2],
                    u32x4 (&carry)[2]) {
      constexpr int J = decltype(jc)::value, JP = 1 - J, JN = 1 - J;
      constexpr int SB = decltype(sbc)::value, SA = decltype(sac)::value, SC = decltype(scc)::value;
      constexpr bool kFirst = decltype(firstc)::value;
      const int last = (kCausal ? min(n_k - 1, my_q) : n_k - 1);
      const int lim = last - (t * kBlk + 32 * J + 8 * hf);
      u32x4 fr[12];
      if (!kFirst) {
        fr[0] = carry[0];
        fr[1] = carry[1];
      }
#pragma unroll
      for (int k = 0; k < 12; ++k) {
        const int kn = k + 2;
        if (kn < 4) {
          if (!kFirst) fr[kn] = tr_frag<SB, JP>(PB, 0, kn & 1, kn >> 1);
        } else if (kn < 12) {
          fr[kn] = row_frag<SA, JN>(PA, (kn - 4) & 1, (kn - 4) >> 1);
        } else {
          carry[kn - 12] = tr_frag<SC, J>(PC, 0, (kn - 12) & 1, 0);  // B(u) of the next iteration
        }
        if (k < 4) {
          if (!kFirst) b_mfma(DP, k, fr[k]);
        } else {
          a_mfma(nxt, k - 4, fr[k]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) el_step(cur, D, 4 * k + i, maskc, lim);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    Unit X, Y;
    u32x4 DX[2], DY[2];
    u32x4 carry[2];
    const int n_eff = (max(ntiles, 2) + 1) & ~1;
    // tiles before t_split lie wholly below every query of the workgroup and
    // before the end of the keys; pairs from t_u on mask their pairs (the
    // first pair always does)
    const int t_split = min(kCausal ? qblk * (128 / kBlk) : ntiles, n_k / kBlk);
    const int t_u = max(t_split & ~1, 2);
    dma_tile(0);
    dma_tile(1);
    dma_tile(2);
    wait_loads_barrier<2 * kDma>();
#pragma unroll
    for (int m = 0; m < 8; ++m) a_mfma(X, m, row_frag<0, 0>(base, m & 1, m >> 1));

    auto pair_body = [&](int t, auto maskc, auto firstc) {
      const int pc = (t >> 1) & 1;
      const Ptrs C = pair_bases(base, pc), O = pair_bases(base, pc ^ 1);
      iter(t, ic<0>(), maskc, firstc, O, ic<1>(), C, ic<0>(), C, ic<0>(), X, Y, DX, DY, carry);
      wait_loads_barrier<kDma>();
      dma_tile(t + 3);
      iter(t, ic<1>(), maskc, std::false_type(), C, ic<0>(), C, ic<1>(), C, ic<0>(), Y, X, DY, DX, carry);
      iter(t + 1, ic<0>(), maskc, std::false_type(), C, ic<0>(), C, ic<1>(), C, ic<1>(), X, Y, DX, DY, carry);
      wait_loads_barrier<kDma>();
      dma_tile(t + 4);
      iter(t + 1, ic<1>(), maskc, std::false_type(), C, ic<1>(), O, ic<0>(), C, ic<1>(), Y, X, DY, DX, carry);
    };
    pair_body(0, std::true_type(), std::true_type());
    int t = 2;
    for (; t < t_u; t += 2) pair_body(t, std::false_type(), std::false_type());
    for (; t < n_eff; t += 2) pair_body(t, std::true_type(), std::false_type());
    // B of the last unit (tile n_eff - 1, slab 1)
    {
      const int off = ((n_eff - 1) & (kStages - 1)) * kStageB + 32 * kRowB + 16 * kRowB;
      b_mfma(DY, 0, carry[0]);
      b_mfma(DY, 1, carry[1]);
      b_mfma(DY, 2, lds_tr(base.pt[0][0] + off, base.pt[0][1] + off));
      b_mfma(DY, 3, lds_tr(base.pt[1][0] + off, base.pt[1][1] + off));
    }
  }
  store_rows(dqp + (int64_t)q_row * a.dq_s[2], row_ok, dq0, dq1, a.scale, hf);
}

// ---------------------------------------------------------------- dK and dV
template <bool kCausal>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_bf16(BwdArgs a, float c, int n_kblk) {
  __shared__ __attribute__((aligned(16))) char smem[kStages * kStageB + kStages * 2 * kStatB];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 31, hf = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
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
  const float* ndelta_row = a.delta + (int64_t)bh * n_q;  // -delta
  const float* lse2_row = a.delta + ((int64_t)a.batch * a.heads + bh) * n_q;

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

  if (n_tiles > 0) {  // workgroup-uniform
    constexpr int kDma = 5;  // loads per wavefront per tile
    const int64_t qs2 = a.q_s[2], ds2 = a.do_s[2];
    unsigned qdo[2], ddo[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 16 * wave + 8 * i + (lane >> 3);
      const int ch = (lane & 7) ^ swz(row);
      qdo[i] = (unsigned)((row * qs2 + 8 * ch) * 2);
      ddo[i] = (unsigned)((row * ds2 + 8 * ch) * 2);
    }
    const unsigned smem_lds = lds_addr(smem), stat_lds = smem_lds + kStages * kStageB;
    // the row statistics: wavefronts 0 and 2 load lse2, 1 and 3 -delta (the
    // pairs write the same bytes)
    const float* stat_src = (wave_u & 1) ? ndelta_row : lse2_row;
    // tile t (queries q_begin + 64 t..) into stage t % 4; rows past the
    // queries read as zero
    auto dma_tile = [&](int t) {
      const int q0 = q_begin + t * kBlk;
      const int valid = max(min(n_q - q0, kBlk), 0);
      const u32x4 rq = make_rsrc(qp + (int64_t)q0 * qs2, valid > 0 ? (unsigned)(((valid - 1) * qs2 + 64) * 2) : 0u);
      const u32x4 rd = make_rsrc(dop + (int64_t)q0 * ds2, valid > 0 ? (unsigned)(((valid - 1) * ds2 + 64) * 2) : 0u);
      const u32x4 rs = make_rsrc(stat_src + q0, (unsigned)(valid * 4));
      const unsigned sb = smem_lds + (unsigned)((t & (kStages - 1)) * kStageB);
      dma16(rq, qdo[0], sb + (unsigned)((16 * wave_u) * kRowB));
      dma16(rq, qdo[1], sb + (unsigned)((16 * wave_u + 8) * kRowB));
      dma16(rd, ddo[0], sb + (unsigned)(kTileB + (16 * wave_u) * kRowB));
      dma16(rd, ddo[1], sb + (unsigned)(kTileB + (16 * wave_u + 8) * kRowB));
      dma4(rs, (unsigned)(4 * lane), stat_lds + (unsigned)((t & (kStages - 1)) * 2 * kStatB + (wave_u & 1) * kStatB));
    };
    const Ptrs base = fragment_bases(smem, lane);

    // statistics chunk i: queries 16 (i >> 1) + 8 hf + 4 (i & 1) + 0..3 of slab J
    auto stat_off = [](int ST, int J, int i) { return ST * 2 * kStatB + 4 * (32 * J + 16 * (i >> 1) + 4 * (i & 1)); };
    // B(u) product m (0..7): dV^T (m % 4 < 2) or dK^T, column block m & 1,
    // 16-query step m >> 2
    auto b_mfma = [&](const u32x4 (&PP)[2], const u32x4 (&DD)[2], int m, const u32x4& fr) {
      const int jj = m >> 2, w = m & 3;
      if (w == 0) dv0 = mfma(dv0, fr, PP[jj]);
      if (w == 1) dv1 = mfma(dv1, fr, PP[jj]);
      if (w == 2) dk0 = mfma(dk0, fr, DD[jj]);
      if (w == 3) dk1 = mfma(dk1, fr, DD[jj]);
    };
    // A(u) product m (0..7): S (even m) or dP from -delta (odd m), d step m >> 1
    auto a_mfma = [&](Unit& U, int m, const u32x4& fr, const f32x16& dinit) {
      const int kk = m >> 1;
      if (m & 1)
        U.dp = mfma(kk == 0 ? dinit : U.dp, fr, vf[kk]);
      else
        U.s = mfma(kk == 0 ? f32x16{} : U.s, fr, kf[kk]);
    };
    // element steps; register r holds query 16 (r >> 3) + 8 hf + (r & 7) of
    // the slab, kept where lim <= that (masked tiles)
    float ex[16], ep[16];
    auto el_step = [&](const Unit& U, const f32x4 (&L)[4], u32x4 (&PP)[2], u32x4 (&DD)[2], int q, auto maskc,
                       int lim) {
      int type, r;
      elem_step(q, type, r);
      if (type == 0) {
        ex[r] = fmaf(U.s[r], c, -L[r >> 2][r & 3]);
      } else if (type == 1) {
        float p = __builtin_amdgcn_exp2f(ex[r]);
        if (decltype(maskc)::value) p = lim <= 16 * (r >> 3) + (r & 7) ? p : 0.f;
        ep[r] = p;
      } else {
        ex[r] = ep[r] * U.dp[r];
        if (r & 1) {
          PP[r >> 3][(r >> 1) & 3] = pack_bf16(ep[r - 1], ep[r]);
          DD[r >> 3][(r >> 1) & 3] = pack_bf16(ex[r - 1], ex[r]);
        }
      }
    };

    // Iteration u = (t, J): B(u-1) in slots 0-7, A(u+1) in slots 8-15, three
    // element steps of V(u) after each; fragments two slots ahead, lse2 of 4
    // queries at a time 4 slots ahead, the -delta start of A(u+1) in slots 3-6.
    auto iter = [&](int t, auto jc, auto maskc, auto firstc, const Ptrs& PB, auto sbc, const Ptrs& PA, auto sac,
                    const Ptrs& PC, auto scc, Unit& cur, Unit& nxt, u32x4 (&PP)[2], u32x4 (&DD)[2],
                    const u32x4 (&PPp)[2], const u32x4 (&DDp)[2], f32x4 (&L)[4], u32x4 (&carry)[2]) {
      constexpr int J = decltype(jc)::value, JP = 1 - J, JN = 1 - J;
      constexpr int SB = decltype(sbc)::value, SA = decltype(sac)::value, SC = decltype(scc)::value;
      constexpr bool kFirst = decltype(firstc)::value;
      const int lim = my_k - (q_begin + t * kBlk) - 32 * J - 8 * hf;
      u32x4 fr[16];
      f32x16 dinit;
      if (!kFirst) {
        fr[0] = carry[0];
        fr[1] = carry[1];
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int kn = k + 2;
        if (kn < 8) {
          if (!kFirst) fr[kn] = tr_frag<SB, JP>(PB, (kn & 3) < 2 ? 1 : 0, kn & 1, kn >> 2);
        } else if (kn < 16) {
          fr[kn] = row_frag<SA, JN>(PA, (kn - 8) & 1, (kn - 8) >> 1);
        } else {
          carry[kn - 16] = tr_frag<SC, J>(PC, 1, (kn - 16) & 1, 0);  // B(u) of the next iteration
        }
        if (k == 0 || k == 3 || k == 7) L[(k + 5) / 4] = ldsf4(PC.ps + stat_off(SC, J, (k + 5) / 4));
        if (k == 11) L[0] = ldsf4(PA.ps + stat_off(SA, JN, 0));
        if (k >= 3 && k < 7) {
          const f32x4 v = ldsf4(PA.ps + stat_off(SA, JN, k - 3) + kStatB);
#pragma unroll
          for (int e = 0; e < 4; ++e) dinit[4 * (k - 3) + e] = v[e];
        }
        if (k < 8) {
          if (!kFirst) b_mfma(PPp, DDp, k, fr[k]);
        } else {
          a_mfma(nxt, k - 8, fr[k], dinit);
        }
#pragma unroll
        for (int i = 0; i < 3; ++i) el_step(cur, L, PP, DD, 3 * k + i, maskc, lim);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    Unit X, Y;
    u32x4 PX[2], DX[2], PY[2], DY[2];
    f32x4 L[4];
    u32x4 carry[2];
    // Tiles past the last (to an even count of at least 2, and the loads ahead
    // of the end) read as zero rows: P = 1, dP - delta = 0, dS = 0 and
    // dO = Q = 0, so they add nothing.
    const int n_eff = (max(n_tiles, 2) + 1) & ~1;
    dma_tile(0);
    dma_tile(1);
    dma_tile(2);
    wait_loads_barrier<2 * kDma>();
    {  // A(0)
      f32x16 dinit;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4 v = ldsf4(base.ps + stat_off(0, 0, i) + kStatB);
#pragma unroll
        for (int e = 0; e < 4; ++e) dinit[4 * i + e] = v[e];
      }
#pragma unroll
      for (int m = 0; m < 8; ++m) a_mfma(X, m, row_frag<0, 0>(base, m & 1, m >> 1), dinit);
      L[0] = ldsf4(base.ps + stat_off(0, 0, 0));
    }

    // Tiles t, t + 1 (t even) at the stages of pair (t / 2) % 2. Before the
    // second iteration of each tile, the wait and barrier make the next tile
    // visible and free the stage that the tile three ahead is loaded into.
    auto pair_body = [&](int t, auto maskc, auto firstc) {
      const int pc = (t >> 1) & 1;
      const Ptrs C = pair_bases(base, pc), O = pair_bases(base, pc ^ 1);
      iter(t, ic<0>(), maskc, firstc, O, ic<1>(), C, ic<0>(), C, ic<0>(), X, Y, PX, DX, PY, DY, L, carry);
      wait_loads_barrier<kDma>();
      dma_tile(t + 3);
      iter(t, ic<1>(), maskc, std::false_type(), C, ic<0>(), C, ic<1>(), C, ic<0>(), Y, X, PY, DY, PX, DX, L, carry);
      iter(t + 1, ic<0>(), maskc, std::false_type(), C, ic<0>(), C, ic<1>(), C, ic<1>(), X, Y, PX, DX, PY, DY, L,
           carry);
      wait_loads_barrier<kDma>();
      dma_tile(t + 4);
      iter(t + 1, ic<1>(), maskc, std::false_type(), C, ic<1>(), O, ic<0>(), C, ic<1>(), Y, X, PY, DY, PX, DX, L,
           carry);
    };
    // causal: tiles 0 and 1 straddle the block's diagonal, the others lie past it
    pair_body(0, std::integral_constant<bool, kCausal>(), std::true_type());
    for (int t = 2; t < n_eff; t += 2) pair_body(t, std::false_type(), std::false_type());
    // B of the last unit (tile n_eff - 1, slab 1)
    {
      const int off = ((n_eff - 1) & (kStages - 1)) * kStageB + 32 * kRowB;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int jj = m >> 2, w = m & 3;
        const int o2 = off + (w < 2 ? kTileB : 0) + 16 * jj * kRowB;
        const u32x4 fr = m < 2 ? carry[m] : lds_tr(base.pt[w & 1][0] + o2, base.pt[w & 1][1] + o2);
        b_mfma(PY, DY, m, fr);
      }
    }
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
