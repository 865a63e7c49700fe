// Projection Y = X W in fp32 (fp32 products and accumulation).
//
// The full-precision counterpart of the bf16 projection kernel, used by the
// fp32 workloads: X (m, k) row-major, W (k, n) row-major (in, out), Y (m, n)
// row-major ("The Transformer" (hoshank.vercel.app), "The Mathematics",
// MultiHead equation). 64 x 64 output tile per workgroup of 256 threads, each
// thread 4 x 4 outputs, 16-deep k steps staged through LDS. Optional epilogue:
// a bias per column and a ReLU (the FFN's max(0, x W1 + b1)).
//
// Grids of fewer than 256 such tiles (a single short sequence) take a second
// form instead: 32 x 32 tiles whose sixteen wavefronts (one 1024-thread
// workgroup) each run a sixteenth of k (their own LDS chunks, the next
// chunk's loads in flight in registers), the partial tiles summed at the end
// in wavefront order, so that short problems spread over many wavefronts
// instead of long serial k loops.
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


// 32 x 32 output tile; wavefront w runs k range [w kq, (w + 1) kq) in
// 16-deep chunks staged in its own LDS region; lane (ty, tx) = (lane / 8,
// lane % 8) accumulates rows 4 ty.., columns 4 tx..
constexpr int kSW = 16;  // wavefronts per split-k workgroup, one k range each

__global__ __launch_bounds__(64 * kSW) void linear_f32_splitk(LinearArgs args, int tiles_n) {
  constexpr int kS = 32, kC = 16;
  __shared__ float Xs[kSW][kC][kS + 4];
  __shared__ float Ws[kSW][kC][kS];
  __shared__ float red[kSW][kS][kS + 1];
  const LinearGroup g = blockIdx.y == 0 ? args.g[0] : (blockIdx.y == 1 ? args.g[1] : args.g[2]);
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * kS, n0 = tn * kS;
  if (m0 >= g.m) return;  // workgroup-uniform
  const int n = args.n, kdim = args.k;
  const float* X = static_cast<const float*>(g.x);
  const float* W = static_cast<const float*>(g.w);
  float* Y = static_cast<float*>(g.y);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, tx = lane & 7, ty = lane >> 3;
  const int kq = (kdim + kSW * kC - 1) / (kSW * kC) * kC;  // each wavefront's k range, a multiple of 16
  const int kb = w * kq, ke = min(kdim, kb + kq);
  float xr[8], wr[8];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = lane + 64 * i;
      const int r = idx >> 4, kk = idx & 15, row = m0 + r, col = k0 + kk;
      xr[i] = (row < g.m && col < ke) ? X[(int64_t)row * g.ldx + col] : 0.f;
      const int wk = idx >> 5, wc = idx & 31;
      wr[i] = (k0 + wk < ke && n0 + wc < n) ? W[(int64_t)(k0 + wk) * g.ldw + n0 + wc] : 0.f;
    }
  };
  float acc[4][4] = {};
  if (kb < ke) load(kb);
  for (int k0 = kb; k0 < ke; k0 += kC) {  // wave-uniform
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = lane + 64 * i;
      Xs[w][idx & 15][idx >> 4] = xr[i];
      Ws[w][idx >> 5][idx & 31] = wr[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (k0 + kC < ke) load(k0 + kC);
#pragma unroll
    for (int kk = 0; kk < kC; ++kk) {
      float xa[4], wb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xa[i] = Xs[w][kk][4 * ty + i];
        wb[i] = Ws[w][kk][4 * tx + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(xa[i], wb[j], acc[i][j]);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // reads done before the next chunk's writes
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[w][4 * ty + i][4 * tx + j] = acc[i][j];
  __syncthreads();
  // thread t sums the kSW partials of output t (row t / 32, column t % 32), in wavefront order
  const int r = tid >> 5, cc = tid & 31, row = m0 + r, col = n0 + cc;
  if (row < g.m && col < n) {
    float v = red[0][r][cc];
#pragma unroll
    for (int q = 1; q < kSW; ++q) v += red[q][r][cc];
    // optional epilogue: + bias[column], then max(0, .)
    if (g.bias != nullptr) v += static_cast<const float*>(g.bias)[col];
    if (args.relu) v = fmaxf(v, 0.f);
    Y[(int64_t)row * g.ldy + col] = v;
  }
}
}  // namespace

hipError_t launch_linear_f32(const LinearArgs& a, hipStream_t stream) {
  int max_m = 0;
  for (int i = 0; i < a.groups; ++i) max_m = a.g[i].m > max_m ? a.g[i].m : max_m;
  const int tiles_n = (a.n + kT - 1) / kT;
  const int tiles_m = (max_m + kT - 1) / kT;
  if ((int64_t)tiles_n * tiles_m * a.groups < 256) {
    const int sn = (a.n + 31) / 32, sm = (max_m + 31) / 32;
    hipLaunchKernelGGL(linear_f32_splitk, dim3((unsigned)(sn * sm), (unsigned)a.groups), dim3(64 * kSW), 0, stream, a, sn);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(tiles_n * tiles_m), (unsigned)a.groups);
  hipLaunchKernelGGL(linear_f32_kernel, grid, dim3(256), 0, stream, a, tiles_n);
  return hipGetLastError();
}

}  // namespace mha
