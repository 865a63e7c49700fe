// Projection Y = X W in fp32 (fp32 products and accumulation).
//
// The full-precision counterpart of the bf16 projection kernel, used by the
// fp32 workloads: X (m, k) row-major, W (k, n) row-major (in, out), Y (m, n)
// row-major ("The Transformer" (hoshank.vercel.app), "The Mathematics",
// MultiHead equation). 64 x 64 output tile per workgroup of 256 threads, each
// thread 4 x 4 outputs, 16-deep k steps staged through LDS. Optional epilogue:
// a bias per column and a ReLU (the FFN's max(0, x W1 + b1)).
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mha {
namespace {

constexpr int kT = 64, kK = 16;

__global__ __launch_bounds__(256) void linear_f32_kernel(LinearArgs args, int tiles_n) {
  __shared__ float Xs[kK][kT + 4];  // X tile stored k-major
  __shared__ float Ws[kK][kT];
  const LinearGroup g = blockIdx.y == 0 ? args.g[0] : (blockIdx.y == 1 ? args.g[1] : args.g[2]);
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * kT, n0 = tn * kT;
  if (m0 >= g.m) return;
  const int n = args.n, kdim = args.k;
  const float* X = static_cast<const float*>(g.x);
  const float* W = static_cast<const float*>(g.w);
  float* Y = static_cast<float*>(g.y);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < kdim; k0 += kK) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, kk = idx & 15;
      const int row = m0 + r, col = k0 + kk;
      Xs[kk][r] = (row < g.m && col < kdim) ? X[(int64_t)row * g.ldx + col] : 0.f;
      const int wk = idx >> 6, wc = idx & 63;
      Ws[wk][wc] = (k0 + wk < kdim && n0 + wc < n) ? W[(int64_t)(k0 + wk) * g.ldw + n0 + wc] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kK; ++kk) {
      float xa[4], wb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xa[i] = Xs[kk][4 * ty + i];
        wb[i] = Ws[kk][4 * tx + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xa[i], wb[j], acc[i][j]);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + 4 * ty + i;
    if (row >= g.m) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + 4 * tx + j;
      if (col < n) {
        // optional epilogue: + bias[column], then max(0, .)
        float v = acc[i][j] + (g.bias != nullptr ? static_cast<const float*>(g.bias)[col] : 0.f);
        if (args.relu) v = fmaxf(v, 0.f);
        Y[(int64_t)row * g.ldy + col] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_linear_f32(const LinearArgs& a, hipStream_t stream) {
  int max_m = 0;
  for (int i = 0; i < a.groups; ++i) max_m = a.g[i].m > max_m ? a.g[i].m : max_m;
  const int tiles_n = (a.n + kT - 1) / kT;
  const int tiles_m = (max_m + kT - 1) / kT;
  const dim3 grid((unsigned)(tiles_n * tiles_m), (unsigned)a.groups);
  hipLaunchKernelGGL(linear_f32_kernel, grid, dim3(256), 0, stream, a, tiles_n);
  return hipGetLastError();
}

}  // namespace mha
