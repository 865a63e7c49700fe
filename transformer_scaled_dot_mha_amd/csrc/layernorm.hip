// Residual add and LayerNorm: out = LayerNorm(x + y) * gamma + beta, per row.
//
// The wrapper around both sub-layers of an encoder layer: output =
// LayerNorm(x + Sublayer(x)) ("The Transformer" (hoshank.vercel.app), "The
// Mathematics"); each position's numbers are shifted to mean 0 and scaled to
// variance 1, then scaled and shifted by learned vectors ("The Transformer"
// (rayaq.ca), "Residuals and LayerNorm"). The variance is the population one
// (mean of squared deviations), eps is added under the square root.
//
// One wavefront per row: lane l holds 8 consecutive columns of every 512-column
// chunk (16-byte loads of bf16, 32-byte of fp32), so a 512-wide row is one
// coalesced 1 KB (bf16) read per input. The sum x + y, the mean and the
// variance (two passes over the registers, no cancellation) are fp32; the
// output is rounded to the stored type once. HBM-bound: 3 row reads/writes.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.h"

namespace mha {
namespace {

typedef __bf16 bf16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ void unpack8(u32x4 w, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// 8 values at element offset col of a row of type T, widened to fp32.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&f)[8]) {
  if constexpr (sizeof(T) == 2) {
    unpack8(*reinterpret_cast<const u32x4*>(p), f);
  } else {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = a[i];
      f[4 + i] = b[i];
    }
  }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&f)[8]) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<u32x4*>(p) =
        u32x4{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
  }
}

// kChunks 512-column chunks per row (d <= 512 * kChunks); four rows per workgroup.
template <typename T, int kChunks>
__global__ __launch_bounds__(256) void add_layernorm_kernel(AddNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;  // wave-uniform, and the kernel has no barrier
  const int d = a.d;
  const T* x = static_cast<const T*>(a.x) + (int64_t)row * d;
  const T* y = static_cast<const T*>(a.y) + (int64_t)row * d;
  const T* gamma = static_cast<const T*>(a.gamma);
  const T* beta = static_cast<const T*>(a.beta);
  T* out = static_cast<T*>(a.out) + (int64_t)row * d;

  float v[kChunks][8];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int col = 8 * (lane + 64 * c);
    if (col < d) {
      float fx[8], fy[8];
      load8(x + col, fx);
      load8(y + col, fy);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[c][i] = fx[i] + fy[i];
        sum += v[c][i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[c][i] = 0.f;
    }
  }
  const float inv_d = 1.0f / (float)d;
  const float mean = wave_sum(sum) * inv_d;
  float sq = 0.f;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    if (8 * (lane + 64 * c) < d) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float dv = v[c][i] - mean;
        sq += dv * dv;
      }
    }
  }
  const float var = wave_sum(sq) * inv_d;
  const float rstd = 1.0f / sqrtf(var + a.eps);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int col = 8 * (lane + 64 * c);
    if (col < d) {
      float g[8], bt[8], o[8];
      load8(gamma + col, g);
      load8(beta + col, bt);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = (v[c][i] - mean) * rstd * g[i] + bt[i];
      store8(out + col, o);
    }
  }
}

template <typename T>
hipError_t launch_t(const AddNormArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((a.rows + 3) / 4));
  if (a.d <= 512)
    hipLaunchKernelGGL((add_layernorm_kernel<T, 1>), grid, dim3(256), 0, stream, a);
  else if (a.d <= 1024)
    hipLaunchKernelGGL((add_layernorm_kernel<T, 2>), grid, dim3(256), 0, stream, a);
  else if (a.d <= 2048)
    hipLaunchKernelGGL((add_layernorm_kernel<T, 4>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((add_layernorm_kernel<T, 8>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_add_layernorm_bf16(const AddNormArgs& a, hipStream_t stream) { return launch_t<bf16>(a, stream); }
hipError_t launch_add_layernorm_f32(const AddNormArgs& a, hipStream_t stream) { return launch_t<float>(a, stream); }

}  // namespace mha
