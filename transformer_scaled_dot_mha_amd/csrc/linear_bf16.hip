// Projection Y = X W in bf16 with fp32 accumulation on the matrix cores, gfx950.
//
// The Q, K, V projections and the output projection W^O of multi-head
// attention ("The Transformer" (hoshank.vercel.app), "The Mathematics",
// MultiHead equation: each W is a d_model x d_k block applied on the right).
// X is (m, k) row-major, W is (k, n) row-major (in, out), Y is (m, n) row-major.
// Because head i owns columns [i*d, (i+1)*d), the row-major Y already *is* the
// head-split (batch, n, heads, d) layout; no permutation pass is needed.
//
// Tile 128 x 128 per workgroup, 32-deep k steps, double-buffered LDS.
// 4 wavefronts in a 2 x 2 arrangement, each owning 64 x 64 outputs as 2 x 2
// blocks of v_mfma_f32_32x32x16_bf16. The MFMA computes Y^T blocks
// (A operand = W^T rows, B operand = X^T columns) so that each lane ends with
// 4 consecutive output columns of one row and stores 8 contiguous bytes.
// W's k dimension is strided in memory; it is transposed into LDS while
// staging, two k rows packed per 32-bit word.
// Up to three independent problems sharing n and k run in one launch
// (grid.y selects the problem): the Q, K and V projections together.
#include <hip/hip_runtime.h>

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

constexpr int kTM = 128, kTN = 128, kTK = 32;
constexpr int kPitch = 40;  // LDS row pitch in elements (80 bytes)
constexpr int kXTile = kTM * kPitch;
constexpr int kWTile = kTN * kPitch;

__device__ __forceinline__ u32x4 ld16(const bf16* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

__global__ __launch_bounds__(256, 2) void linear_bf16_kernel(LinearArgs args, int tiles_n, int tiles_m) {
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * (kXTile + kWTile)];
  // uniform selects, not a dynamic index into the kernel arguments
  const LinearGroup g = blockIdx.y == 0 ? args.g[0] : (blockIdx.y == 1 ? args.g[1] : args.g[2]);
  const int n = args.n, kdim = args.k;

  // XCD-aware order: each XCD gets a contiguous run of tiles, n fastest, so
  // the column tiles of one row tile share an L2 (and the X tile it holds).
  const int total = gridDim.x, id = blockIdx.x;
  const int per = total >> 3, rem = total & 7, x = id & 7, slot = id >> 3;
  const int logical = (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
  const int tm = logical / tiles_n, tn = logical - tm * tiles_n;
  const int m0 = tm * kTM, n0 = tn * kTN;
  if (tm >= tiles_m || m0 >= g.m) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, hf = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const bf16* X = static_cast<const bf16*>(g.x);
  const bf16* W = static_cast<const bf16*>(g.w);
  bf16* Y = static_cast<bf16*>(g.y);

  // staging assignment: X rows tid/4 and tid/4+64, 16-byte chunk tid%4;
  // W k rows 2*(tid%16) and +1, 8-column chunk tid/16
  const int x_row = tid >> 2, x_chunk = tid & 3;
  const int w_k = (tid & 15) * 2, w_chunk = tid >> 4;

  u32x4 xr[2], wr[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = m0 + x_row + 64 * i, col = k0 + 8 * x_chunk;
      xr[i] = (row < g.m && col < kdim) ? ld16(X + (int64_t)row * g.ldx + col) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = k0 + w_k + i, col = n0 + 8 * w_chunk;
      wr[i] = (row < kdim && col < n) ? ld16(W + (int64_t)row * g.ldw + col) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
    bf16* Xs = smem + buf * (kXTile + kWTile);
    bf16* Wt = Xs + kXTile;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(Xs + (x_row + 64 * i) * kPitch + 8 * x_chunk) = xr[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned w0 = wr[0][e >> 1], w1 = wr[1][e >> 1];
      const unsigned word = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u)) : ((w0 & 0xffffu) | (w1 << 16));
      *reinterpret_cast<unsigned*>(Wt + (8 * w_chunk + e) * kPitch + w_k) = word;
    }
  };

  f32x16 acc[2][2] = {};  // [n block][m block], Y^T layout
  const int nsteps = (kdim + kTK - 1) / kTK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const bool more = s + 1 < nsteps;
    if (more) gload((s + 1) * kTK);
    const bf16* Xs = smem + (s & 1) * (kXTile + kWTile);
    const bf16* Wt = Xs + kXTile;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 xf[2], wf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        xf[i] = as_bf16x8(ld16(Xs + (64 * wm + 32 * i + lq) * kPitch + 16 * ks + 8 * hf));
        wf[i] = as_bf16x8(ld16(Wt + (64 * wn + 32 * i + lq) * kPitch + 16 * ks + 8 * hf));
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], xf[mb], acc[nb][mb], 0, 0, 0);
    }
    if (more) lstore((s + 1) & 1);
    __syncthreads();
  }

  // lane holds row m0 + 64*wm + 32*mb + lq, columns n0 + 64*wn + 32*nb + 8*q + 4*hf + 0..3
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int row = m0 + 64 * wm + 32 * mb + lq;
    if (row >= g.m) continue;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + 64 * wn + 32 * nb + 8 * q + 4 * hf;
        if (col < n) {
          const f32x16& c = acc[nb][mb];
          *reinterpret_cast<u32x2*>(Y + (int64_t)row * g.ldy + col) =
              u32x2{pack_bf16(c[4 * q], c[4 * q + 1]), pack_bf16(c[4 * q + 2], c[4 * q + 3])};
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t stream) {
  int max_m = 0;
  for (int i = 0; i < a.groups; ++i) max_m = a.g[i].m > max_m ? a.g[i].m : max_m;
  const int tiles_n = (a.n + kTN - 1) / kTN;
  const int tiles_m = (max_m + kTM - 1) / kTM;
  const dim3 grid((unsigned)(tiles_n * tiles_m), (unsigned)a.groups);
  hipLaunchKernelGGL(linear_bf16_kernel, grid, dim3(256), 0, stream, a, tiles_n, tiles_m);
  return hipGetLastError();
}

}  // namespace mha
