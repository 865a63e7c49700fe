// Scaled dot-product attention backward in fp32, head width in {16, 32, 64, 128}.
//
// The gradient that flows back through the softmax -- the quantity the pages
// protect with the 1/sqrt(d_k) scale ("32 Transformer" (ml-canon-en.vercel.app),
// "Why we divide by sqrt(dk)"; "The Transformer" (hoshank.vercel.app), "The
// Breakthrough") -- by the chain rule through O = P V, the row softmax and
// S = scale Q K^T:
//   dV = P^T dO,  dP = dO V^T,  dS_ij = P_ij (dP_ij - delta_i),
//   delta_i = sum_j P_ij dP_ij = dO_i . O_i,  dQ = scale dS K,  dK = scale dS^T Q.
// P is recomputed from the forward's log-sum-exp: P_ij = exp(scale q_i.k_j - lse_i),
// zero for masked keys and for rows with no visible key (lse = -inf).
//
// Full-precision path (fp32 storage and arithmetic). Two launches, no atomics:
//   attn_bwd_dq_f32   one thread per query row: delta_i, then dQ over key tiles;
//   attn_bwd_dkdv_f32 one thread per key row: dK and dV over query tiles.
// Tiles of 32 rows are staged in LDS and read by the whole workgroup. At
// d = 128 a row is shared by two lanes (lane and lane + 32), each holding half
// of its columns; their partial dot products are summed with one exchange, so
// the per-thread rows fit the register file.
#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.h"

namespace mha {
namespace {

constexpr int kRows = 64;  // rows per workgroup (one wavefront)
constexpr int kTile = 32;  // rows per staged tile
constexpr float kLog2e = 1.4426950408889634f;

// lse in base 2, with rows that have no visible key mapped to +inf so that
// exp2(s - lse2) is exactly 0 for them.
__device__ __forceinline__ float lse_base2(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// Lanes per row and the columns each lane owns.
template <int D>
struct Split {
  static constexpr int kLanes = D == 128 ? 2 : 1;
  static constexpr int kCols = D / kLanes;
  static constexpr int kRowsPerBlock = kRows / kLanes;
};

template <int kLanes>
__device__ __forceinline__ float row_sum(float x) {
  if (kLanes == 2) x += __shfl_xor(x, 32, 64);
  return x;
}

template <int D, bool kCausal>
__global__ __launch_bounds__(kRows) void attn_bwd_dq_f32(BwdArgs a, float c, int n_qblk) {
  typedef Split<D> S;
  constexpr int DH = S::kCols;
  __shared__ float Ks[kTile][D];
  __shared__ float Vs[kTile][D];
  const int tid = threadIdx.x;
  const int row = tid % S::kRowsPerBlock, c0 = (tid / S::kRowsPerBlock) * DH;
  const int bh = blockIdx.x / n_qblk;
  const int qb = blockIdx.x - bh * n_qblk;
  const int b = bh / a.heads, h = bh - b * a.heads;
  const float* qp = static_cast<const float*>(a.q) + b * a.q_s[0] + h * a.q_s[1];
  const float* kp = static_cast<const float*>(a.k) + b * a.k_s[0] + h * a.k_s[1];
  const float* vp = static_cast<const float*>(a.v) + b * a.v_s[0] + h * a.v_s[1];
  const float* op = static_cast<const float*>(a.o) + b * a.o_s[0] + h * a.o_s[1];
  const float* dop = static_cast<const float*>(a.d_o) + b * a.do_s[0] + h * a.do_s[1];
  float* dqp = static_cast<float*>(a.dq) + b * a.dq_s[0] + h * a.dq_s[1];
  const int n_q = a.n_q;
  const int n_k = a.kv_len != nullptr ? min(max(a.kv_len[b], 0), a.n_k) : a.n_k;
  const int my_q = qb * S::kRowsPerBlock + row;
  const bool row_ok = my_q < n_q;

  float qr[DH], dor[DH], dq[DH];
  float delta = 0.f;
#pragma unroll
  for (int t = 0; t < DH; ++t) {
    qr[t] = row_ok ? qp[(int64_t)my_q * a.q_s[2] + c0 + t] : 0.f;
    dor[t] = row_ok ? dop[(int64_t)my_q * a.do_s[2] + c0 + t] : 0.f;
    delta = fmaf(dor[t], row_ok ? op[(int64_t)my_q * a.o_s[2] + c0 + t] : 0.f, delta);
    dq[t] = 0.f;
  }
  delta = row_sum<S::kLanes>(delta);
  const float lse2 = row_ok ? lse_base2(a.lse[(int64_t)bh * n_q + my_q]) : INFINITY;
  if (row_ok && c0 == 0) a.delta[(int64_t)bh * n_q + my_q] = delta;

  const int kv_end = kCausal ? min(n_k, (qb + 1) * S::kRowsPerBlock) : n_k;
  for (int k0 = 0; k0 < kv_end; k0 += kTile) {
    __syncthreads();
    for (int idx = tid; idx < kTile * D; idx += kRows) {
      const int r = idx / D, col = idx - r * D;
      const int key = k0 + r;
      Ks[r][col] = key < n_k ? kp[(int64_t)key * a.k_s[2] + col] : 0.f;
      Vs[r][col] = key < n_k ? vp[(int64_t)key * a.v_s[2] + col] : 0.f;
    }
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j < kTile; ++j) {
      const int key = k0 + j;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int t = 0; t < DH; ++t) {
        s = fmaf(qr[t], Ks[j][c0 + t], s);
        dp = fmaf(dor[t], Vs[j][c0 + t], dp);
      }
      s = row_sum<S::kLanes>(s);
      dp = row_sum<S::kLanes>(dp);
      const bool ok = key < n_k && (!kCausal || key <= my_q);
      const float p = ok ? exp2f(fmaf(s, c, -lse2)) : 0.f;
      const float ds = p * (dp - delta);
#pragma unroll
      for (int t = 0; t < DH; ++t) dq[t] = fmaf(ds, Ks[j][c0 + t], dq[t]);
    }
  }
  if (row_ok) {
    float* dst = dqp + (int64_t)my_q * a.dq_s[2] + c0;
#pragma unroll
    for (int t = 0; t < DH; ++t) dst[t] = dq[t] * a.scale;
  }
}

template <int D, bool kCausal>
__global__ __launch_bounds__(kRows) void attn_bwd_dkdv_f32(BwdArgs a, float c, int n_kblk) {
  typedef Split<D> S;
  constexpr int DH = S::kCols;
  __shared__ float Qs[kTile][D];
  __shared__ float Ds[kTile][D];
  __shared__ float Ls[kTile], Dl[kTile];
  const int tid = threadIdx.x;
  const int row = tid % S::kRowsPerBlock, c0 = (tid / S::kRowsPerBlock) * DH;
  const int bh = blockIdx.x / n_kblk;
  const int kb = blockIdx.x - bh * n_kblk;
  const int b = bh / a.heads, h = bh - b * a.heads;
  const float* qp = static_cast<const float*>(a.q) + b * a.q_s[0] + h * a.q_s[1];
  const float* kp = static_cast<const float*>(a.k) + b * a.k_s[0] + h * a.k_s[1];
  const float* vp = static_cast<const float*>(a.v) + b * a.v_s[0] + h * a.v_s[1];
  const float* dop = static_cast<const float*>(a.d_o) + b * a.do_s[0] + h * a.do_s[1];
  float* dkp = static_cast<float*>(a.dk) + b * a.dk_s[0] + h * a.dk_s[1];
  float* dvp = static_cast<float*>(a.dv) + b * a.dv_s[0] + h * a.dv_s[1];
  const int n_q = a.n_q;
  const int n_k = a.kv_len != nullptr ? min(max(a.kv_len[b], 0), a.n_k) : a.n_k;
  const int k_first = kb * S::kRowsPerBlock;
  const int my_k = k_first + row;
  const bool key_ok = my_k < n_k;  // keys past a padded length get zero gradients

  float kr[DH], vr[DH], dk[DH], dv[DH];
#pragma unroll
  for (int t = 0; t < DH; ++t) {
    kr[t] = key_ok ? kp[(int64_t)my_k * a.k_s[2] + c0 + t] : 0.f;
    vr[t] = key_ok ? vp[(int64_t)my_k * a.v_s[2] + c0 + t] : 0.f;
    dk[t] = 0.f;
    dv[t] = 0.f;
  }
  // queries before the block's first key see none of its keys under the causal mask
  const int q_begin = kCausal ? k_first / kTile * kTile : 0;
  const int q_end = k_first < n_k ? n_q : 0;
  for (int q0 = q_begin; q0 < q_end; q0 += kTile) {
    __syncthreads();
    for (int idx = tid; idx < kTile * D; idx += kRows) {
      const int r = idx / D, col = idx - r * D;
      const int qi = q0 + r;
      Qs[r][col] = qi < n_q ? qp[(int64_t)qi * a.q_s[2] + col] : 0.f;
      Ds[r][col] = qi < n_q ? dop[(int64_t)qi * a.do_s[2] + col] : 0.f;
    }
    if (tid < kTile) {
      const int qi = q0 + tid;
      Ls[tid] = qi < n_q ? lse_base2(a.lse[(int64_t)bh * n_q + qi]) : INFINITY;
      Dl[tid] = qi < n_q ? a.delta[(int64_t)bh * n_q + qi] : 0.f;
    }
    __syncthreads();
#pragma unroll 1
    for (int i = 0; i < kTile; ++i) {
      const int qi = q0 + i;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int t = 0; t < DH; ++t) {
        s = fmaf(Qs[i][c0 + t], kr[t], s);
        dp = fmaf(Ds[i][c0 + t], vr[t], dp);
      }
      s = row_sum<S::kLanes>(s);
      dp = row_sum<S::kLanes>(dp);
      const bool ok = key_ok && qi < n_q && (!kCausal || my_k <= qi);
      const float p = ok ? exp2f(fmaf(s, c, -Ls[i])) : 0.f;
      const float ds = p * (dp - Dl[i]);
#pragma unroll
      for (int t = 0; t < DH; ++t) {
        dv[t] = fmaf(p, Ds[i][c0 + t], dv[t]);
        dk[t] = fmaf(ds, Qs[i][c0 + t], dk[t]);
      }
    }
  }
  if (my_k < a.n_k) {
    float* dkd = dkp + (int64_t)my_k * a.dk_s[2] + c0;
    float* dvd = dvp + (int64_t)my_k * a.dv_s[2] + c0;
#pragma unroll
    for (int t = 0; t < DH; ++t) {
      dkd[t] = dk[t] * a.scale;
      dvd[t] = dv[t];
    }
  }
}

template <int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t stream) {
  const float c = a.scale * kLog2e;
  constexpr int rows = Split<D>::kRowsPerBlock;
  const int n_qblk = (a.n_q + rows - 1) / rows;
  const int n_kblk = (a.n_k + rows - 1) / rows;
  const dim3 gq((unsigned)(n_qblk * a.batch * a.heads)), gk((unsigned)(n_kblk * a.batch * a.heads));
  if (a.causal)
    hipLaunchKernelGGL((attn_bwd_dq_f32<D, true>), gq, dim3(kRows), 0, stream, a, c, n_qblk);
  else
    hipLaunchKernelGGL((attn_bwd_dq_f32<D, false>), gq, dim3(kRows), 0, stream, a, c, n_qblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.causal)
    hipLaunchKernelGGL((attn_bwd_dkdv_f32<D, true>), gk, dim3(kRows), 0, stream, a, c, n_kblk);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_f32<D, false>), gk, dim3(kRows), 0, stream, a, c, n_kblk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention_bwd_f32(const BwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 16: return launch_d<16>(a, stream);
    case 32: return launch_d<32>(a, stream);
    case 64: return launch_d<64>(a, stream);
    case 128: return launch_d<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mha
