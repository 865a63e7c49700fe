// Scaled dot-product attention forward in fp32, any head width in {16, 32, 64, 128}.
//
// O = softmax(scale * Q K^T (+ causal mask)) V per (batch, head) ("The
// Transformer" (hoshank.vercel.app), "The Mathematics", Attention equation),
// computed exactly in one pass over key tiles with a running row maximum and
// row sum. This is the full-precision path (fp32 storage, fp32 products and
// accumulation, no reduced-precision matrix modes) used by the fp32 workloads.
//
// A workgroup of 4 wavefronts owns 16 query rows of one (batch, head); four
// lanes share a row, each holding a quarter of its d values (the partial dot
// products are summed across the four lanes with DPP quad permutes). The
// wavefronts split the key tiles between them (tile i goes to wavefront
// i % 4), each staging its own tiles in its own LDS region, and the four
// partial (max, sum, O) states of a row are merged at the end. Small problems
// (a single 128-token sequence) then run on many wavefronts instead of a few
// long serial loops.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.h"

namespace mha {
namespace {

constexpr int kRows = 16;  // query rows per workgroup (four lanes per row, four wavefronts)

// x summed over the four lanes of its quad (DPP quad permutes 1,0,3,2 and 2,3,0,1)
__device__ __forceinline__ float quad_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  return x;
}

template <int D, bool kCausal>
__global__ __launch_bounds__(256) void attn_fwd_f32(AttnArgs a, float c, float q_sign, int n_qblk) {
  constexpr int kKeys = D <= 64 ? 32 : 16;  // keys per tile
  constexpr int kPart = D / 4;              // d values per lane
  constexpr int kTile = kKeys * D;          // floats per K (or V) tile
  static_assert(4 * 16 * (D + 2) <= 4 * 2 * kTile, "the merge fits in the tiles' LDS");
  __shared__ __attribute__((aligned(16))) float smem[4 * 2 * kTile];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane >> 2, part = lane & 3;
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
  const int q0 = qb * kRows;
  const int my_q = q0 + r;

  // Loads go to clamped (always valid) rows and out-of-range values are
  // zeroed afterwards: a load under a per-lane condition would be waited for
  // before the next one is issued.
  float q[kPart], acc[kPart];
  {
    const float* src = qp + (int64_t)min(my_q, n_q - 1) * a.q_sn + part * kPart;
    float4 v[kPart / 4];
#pragma unroll
    for (int t = 0; t < kPart; t += 4) v[t / 4] = *reinterpret_cast<const float4*>(src + t);
    const bool row_ok = my_q < n_q;
#pragma unroll
    for (int t = 0; t < kPart; t += 4) {
      q[t] = row_ok ? q_sign * v[t / 4].x : 0.f;
      q[t + 1] = row_ok ? q_sign * v[t / 4].y : 0.f;
      q[t + 2] = row_ok ? q_sign * v[t / 4].z : 0.f;
      q[t + 3] = row_ok ? q_sign * v[t / 4].w : 0.f;
    }
  }
#pragma unroll
  for (int t = 0; t < kPart; ++t) acc[t] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int kv_end = kCausal ? min(n_k, q0 + kRows) : n_k;
  const int ntile = (kv_end + kKeys - 1) / kKeys;
  float* Ks = smem + wave * 2 * kTile;
  float* Vs = Ks + kTile;

#pragma unroll 1
  for (int ti = wave; ti < ntile; ti += 4) {  // wave-uniform
    const int k0 = ti * kKeys;
    // this wavefront's tile (only its own lanes read it, so no barrier)
    constexpr int kLoads = kTile / 4 / 64;  // float4 loads of K (and of V) per lane
    constexpr int kGroup = kLoads < 4 ? kLoads : 4;
#pragma unroll
    for (int u0 = 0; u0 < kLoads; u0 += kGroup) {  // groups of loads in flight together
      float4 kv[kGroup], vv[kGroup];
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        const int i = lane + 64 * (u0 + u);
        const int key = i / (D / 4), c4 = 4 * (i - key * (D / 4));
        const int row = min(k0 + key, n_k - 1);  // n_k >= 1 here: the tile holds a visible key
        kv[u] = *reinterpret_cast<const float4*>(kp + (int64_t)row * a.k_sn + c4);
        vv[u] = *reinterpret_cast<const float4*>(vp + (int64_t)row * a.v_sn + c4);
      }
#pragma unroll
      for (int u = 0; u < kGroup; ++u) {
        const int i = lane + 64 * (u0 + u);
        const int key = i / (D / 4), c4 = 4 * (i - key * (D / 4));
        const bool in = k0 + key < n_k;
        // component selects (a select of whole float4 structs goes through scratch memory)
        const float4 kz = {in ? kv[u].x : 0.f, in ? kv[u].y : 0.f, in ? kv[u].z : 0.f, in ? kv[u].w : 0.f};
        const float4 vz = {in ? vv[u].x : 0.f, in ? vv[u].y : 0.f, in ? vv[u].z : 0.f, in ? vv[u].w : 0.f};
        *reinterpret_cast<float4*>(Ks + key * D + c4) = kz;
        *reinterpret_cast<float4*>(Vs + key * D + c4) = vz;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    float s[kKeys];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < kPart; ++t) dot = fmaf(q[t], Ks[j * D + part * kPart + t], dot);
      dot = quad_sum(dot);
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
    for (int t = 0; t < kPart; ++t) acc[t] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = s[j] == -INFINITY ? 0.f : exp2f(fmaf(s[j], c, -mc));
      l_run += p;
#pragma unroll
      for (int t = 0; t < kPart; ++t) acc[t] = fmaf(p, Vs[j * D + part * kPart + t], acc[t]);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // reads done before the next tile's writes
  }

  // merge the four wavefronts' states of each row: [wave][row][D + 2]
  __syncthreads();
  float* red = smem + (wave * kRows + r) * (D + 2);
#pragma unroll
  for (int t = 0; t < kPart; ++t) red[part * kPart + t] = acc[t];
  if (part == 0) {
    red[D] = m_run;
    red[D + 1] = l_run;
  }
  __syncthreads();
  if (wave == 0) {
    float mw[4], lw[4], m_all = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float* rw = smem + (w * kRows + r) * (D + 2);
      mw[w] = rw[D];
      lw[w] = rw[D + 1];
      m_all = fmaxf(m_all, mw[w]);
    }
    const float mc = (m_all == -INFINITY ? 0.f : m_all) * c;
    float wt[4], l_all = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wt[w] = mw[w] == -INFINITY ? 0.f : exp2f(fmaf(mw[w], c, -mc));
      l_all = fmaf(wt[w], lw[w], l_all);
    }
    if (my_q < n_q) {
      // a row with no visible key (padded length 0) has l = 0: output 0, lse -inf
      const float inv = l_all > 0.f ? 1.0f / l_all : 0.f;
      float* dst = op + (int64_t)my_q * a.o_sn + part * kPart;
#pragma unroll
      for (int t = 0; t < kPart; ++t) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) o = fmaf(wt[w], smem[(w * kRows + r) * (D + 2) + part * kPart + t], o);
        dst[t] = o * inv;
      }
      if (a.lse != nullptr && part == 0)
        a.lse[(int64_t)bh * n_q + my_q] =
            l_all > 0.f ? m_all * (c / 1.4426950408889634f) + logf(l_all) : -INFINITY;
    }
  }
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
  const float c = fabsf(a.scale) * 1.4426950408889634f;
  const float q_sign = a.scale < 0.f ? -1.f : 1.f;
  const int n_qblk = (a.n_q + kRows - 1) / kRows;
  const dim3 grid((unsigned)(n_qblk * a.batch * a.heads));
  if (a.causal)
    hipLaunchKernelGGL((attn_fwd_f32<D, true>), grid, dim3(256), 0, stream, a, c, q_sign, n_qblk);
  else
    hipLaunchKernelGGL((attn_fwd_f32<D, false>), grid, dim3(256), 0, stream, a, c, q_sign, n_qblk);
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
