// Scaled dot-product attention forward in fp32, any head width in {16, 32, 64, 128}.
//
// O = softmax(scale * Q K^T (+ causal mask)) V per (batch, head) ("The
// Transformer" (hoshank.vercel.app), "The Mathematics", Attention equation),
// computed exactly in one pass over key tiles with a running row maximum and
// row sum. This is the full-precision path (fp32 storage, fp32 products and
// accumulation, no reduced-precision matrix modes) used by the fp32 workloads;
// one thread owns one query row, and 32-key tiles of K and V are staged in
// LDS and read by every thread of the workgroup (broadcast reads).
#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.h"

namespace mha {
namespace {

constexpr int kRows = 64;  // query rows per workgroup (one wavefront)
constexpr int kKeys = 32;  // keys per tile

template <int D, bool kCausal>
__global__ __launch_bounds__(kRows) void attn_fwd_f32(AttnArgs a, float c, float q_sign, int n_qblk) {
  __shared__ float Ks[kKeys][D];
  __shared__ float Vs[kKeys][D];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / n_qblk;
  const int qb = blockIdx.x - bh * n_qblk;
  const int b = bh / a.heads, h = bh - b * a.heads;
  const float* qp = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh;
  const float* kp = static_cast<const float*>(a.k) + b * a.k_sb + h * a.k_sh;
  const float* vp = static_cast<const float*>(a.v) + b * a.v_sb + h * a.v_sh;
  float* op = static_cast<float*>(a.o) + b * a.o_sb + h * a.o_sh;
  const int n_q = a.n_q;
  // keys visible to this batch item: all n_k, or its padded length
  const int n_k = a.kv_len != nullptr ? min(max(a.kv_len[b], 0), a.n_k) : a.n_k;
  const int my_q = qb * kRows + tid;

  float qr[D], acc[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    qr[t] = my_q < n_q ? q_sign * qp[(int64_t)my_q * a.q_sn + t] : 0.f;
    acc[t] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const int kv_end = kCausal ? min(n_k, qb * kRows + kRows) : n_k;

  for (int k0 = 0; k0 < kv_end; k0 += kKeys) {
    __syncthreads();
    for (int idx = tid; idx < kKeys * D; idx += kRows) {
      const int r = idx / D, col = idx - r * D;
      const int key = k0 + r;
      Ks[r][col] = key < n_k ? kp[(int64_t)key * a.k_sn + col] : 0.f;
      Vs[r][col] = key < n_k ? vp[(int64_t)key * a.v_sn + col] : 0.f;
    }
    __syncthreads();
    float s[kKeys];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < D; ++t) dot = fmaf(qr[t], Ks[j][t], dot);
      const int key = k0 + j;
      const bool ok = key < n_k && (!kCausal || key <= my_q);
      s[j] = ok ? dot : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m_run, tmax);
    const float mc = (m_new == -INFINITY ? 0.f : m_new) * c;
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2f(fmaf(m_run, c, -mc));
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < D; ++t) acc[t] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = s[j] == -INFINITY ? 0.f : exp2f(fmaf(s[j], c, -mc));
      l_run += p;
#pragma unroll
      for (int t = 0; t < D; ++t) acc[t] = fmaf(p, Vs[j][t], acc[t]);
    }
  }
  if (my_q < n_q) {
    // a row with no visible key (padded length 0) has l = 0: output 0, lse -inf
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* dst = op + (int64_t)my_q * a.o_sn;
#pragma unroll
    for (int t = 0; t < D; ++t) dst[t] = acc[t] * inv;
    if (a.lse != nullptr)
      a.lse[(int64_t)bh * n_q + my_q] = l_run > 0.f ? m_run * (c / 1.4426950408889634f) + logf(l_run) : -INFINITY;
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  const float c = fabsf(a.scale) * 1.4426950408889634f;
  const float q_sign = a.scale < 0.f ? -1.f : 1.f;
  const int n_qblk = (a.n_q + kRows - 1) / kRows;
  const dim3 grid((unsigned)(n_qblk * a.batch * a.heads));
  if (a.causal)
    hipLaunchKernelGGL((attn_fwd_f32<D, true>), grid, dim3(kRows), 0, stream, a, c, q_sign, n_qblk);
  else
    hipLaunchKernelGGL((attn_fwd_f32<D, false>), grid, dim3(kRows), 0, stream, a, c, q_sign, n_qblk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 16: return launch_d<16>(a, stream);
    case 32: return launch_d<32>(a, stream);
    case 64: return launch_d<64>(a, stream);
    case 128: return launch_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mha
