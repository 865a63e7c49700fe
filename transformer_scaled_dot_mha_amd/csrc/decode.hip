// One decoding step against a key/value cache.
//
// A decoder generates left to right, its masked self-attention covering the
// tokens generated so far ("How Transformers Work" (worksonmygpu.com), "What
// changed since 2017"; "The Transformer" (hoshank.vercel.app), "The
// Breakthrough"): the newest position's query attends to every key up to and
// including its own, the last row of causal attention ("The Transformer"
// (rayaq.ca), "Masks: who may look at whom"). Keys and values of earlier
// positions are kept in a cache. "How Transformers Work" names PagedAttention
// as how they are stored when serving but gives no layout; here the cache may
// be kept in fixed-size pages reached through a per-sequence page table.
//
//   o[b,h,:] = sum_{j < len_b} softmax_j(scale * q[b,h,:] . K_j) V_j
//
// With one query row there is no matrix product to feed the matrix cores: per
// key, d multiply-adds for the score and d for the output against 2 d stored
// elements read once. The kernel is bound by HBM bandwidth; it is written for
// coalesced 16-byte loads and many loads in flight, on the vector ALUs.
//
// Split over keys. Workgroup (bh, s) takes keys [256 s, 256 s + 256) of one
// (batch, head) and writes its partial softmax state (max, sum, unnormalised
// output) to the workspace; a second, small launch merges the splits of each
// (batch, head). A sequence of one split, or of none, is finished by the split
// kernel itself. (Merging in the split kernel, by the last split to finish,
// needs a release fence per workgroup, which on this chip writes back the
// whole L2 and costs far more than the second launch.) Inside a workgroup each wavefront owns 64 keys; a key's d elements
// are spread over d / 8 (bf16) or d / 4 (fp32) lanes, one 16-byte load each,
// so one load instruction of a wavefront reads several whole key rows. Each
// lane group keeps its own running max, sum and output slice (online softmax
// in base 2, scale * log2(e) folded into q), then the groups and the
// wavefronts are merged by rescaling to the common max.
//
// Cache addressing. Element e of head h of key j of sequence b is at
//   page * page_stride + slot * row_stride + h * head_stride + e
// with (page, slot) = (table[b][j / page_size], j % page_size) when a page
// table is given and (b, j) otherwise. The row offsets of a workgroup's 256
// keys are computed once into LDS. A table entry outside [0, num_pages) is
// never dereferenced: that split reports NaN, and the merge turns the
// sequence's output and lse into NaN.
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

constexpr int kChunk = kDecodeChunk;  // keys per workgroup
constexpr int kWaves = 4;
constexpr int kKeysPerWave = kChunk / kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16 bytes of T, widened to fp32.
template <typename T>
struct Vec16;
template <>
struct Vec16<bf16> {
  static constexpr int n = 8;
  typedef u32x4 raw;
  static __device__ __forceinline__ void widen(raw w, float (&f)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Vec16<float> {
  static constexpr int n = 4;
  typedef f32x4 raw;
  static __device__ __forceinline__ void widen(raw w, float (&f)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = w[i];
  }
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Fold state (m2, l2, o2) into (m, l, o): both rescaled to the larger max.
// A state with no key has m = -inf and l = o = 0 and leaves the other as is.
template <int kN>
__device__ __forceinline__ void merge_state(float& m, float& l, float (&o)[kN], float m2, float l2,
                                            const float (&o2)[kN]) {
  const float mn = fmaxf(m, m2);
  const float base = mn == -INFINITY ? 0.f : mn;
  const float a1 = exp2_fast(m - base);
  const float a2 = exp2_fast(m2 - base);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int i = 0; i < kN; ++i) o[i] = o[i] * a1 + o2[i] * a2;
  m = mn;
}

template <typename T>
__device__ __forceinline__ T to_elem(float x);
template <>
__device__ __forceinline__ bf16 to_elem<bf16>(float x) {
  return (bf16)x;
}
template <>
__device__ __forceinline__ float to_elem<float>(float x) {
  return x;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int x = 32; x > 0; x >>= 1) v = fmaxf(v, __shfl_xor(v, x, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int x = 32; x > 0; x >>= 1) v += __shfl_xor(v, x, 64);
  return v;
}

// One wavefront combines the ns >= 2 split states of (batch, head) bh,
// normalises and writes o and lse. The loads are issued together so the
// wavefront waits for memory about twice (the length, then the rest): the split states one per lane and the
// first kRows split output rows up front; splits past 64 or kRows (caches
// longer than 16384 or 4096 keys) take further rounds.
template <typename T, int D>
__device__ void merge_splits(const DecodeArgs& a, int bh, int ns, int lane) {
  constexpr int kE = (D + 63) / 64;  // output elements per lane
  constexpr int kRows = 16;          // split rows loaded up front
  const float* ml = a.part_ml + (int64_t)bh * a.splits * 2;
  const float* po = a.part_o + (int64_t)bh * a.splits * D;

  float pre[kRows][kE];
#pragma unroll
  for (int j = 0; j < kRows; ++j) {
#pragma unroll
    for (int e = 0; e < kE; ++e)
      pre[j][e] = (j < ns && lane + 64 * e < D) ? po[(int64_t)j * D + lane + 64 * e] : 0.f;
  }
  float m0 = -INFINITY, l0 = 0.f;  // this lane's split of the first 64
  if (lane < ns) {
    m0 = ml[2 * lane];
    l0 = ml[2 * lane + 1];
  }
  float mx = m0;
  bool nan = m0 != m0;
  for (int s = 64 + lane; s < ns; s += 64) {
    const float ms = ml[2 * s];
    nan |= ms != ms;
    mx = fmaxf(mx, ms);
  }
  mx = wave_max(mx);
  nan = __any(nan);

  float lsum = 0.f;
  float acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
  if (!nan) {
    const float f0 = lane < ns ? exp2_fast(m0 - mx) : 0.f;
    lsum = f0 * l0;
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      const float fj = __shfl(f0, j, 64);  // 0 for j >= ns
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[e] += fj * pre[j][e];
    }
    // splits kRows.. (rare: caches longer than kRows * kChunk keys)
    for (int s0 = 0; s0 < ns; s0 += 64) {
      const int s = s0 + lane;
      float f = s0 == 0 ? f0 : 0.f;
      if (s0 > 0 && s < ns) {
        f = exp2_fast(ml[2 * s] - mx);
        lsum += f * ml[2 * s + 1];
      }
      const int first = s0 == 0 ? kRows : 0;
      const int cnt = min(64, ns - s0);
      for (int j = first; j < cnt; ++j) {
        const float fj = __shfl(f, j, 64);
#pragma unroll
        for (int e = 0; e < kE; ++e)
          if (lane + 64 * e < D) acc[e] += fj * po[(int64_t)(s0 + j) * D + lane + 64 * e];
      }
    }
    lsum = wave_sum(lsum);
  }
  float scale_out, lse;
  if (nan) {
    scale_out = NAN;
    lse = NAN;
  } else {
    scale_out = 1.0f / lsum;
    lse = (mx + __log2f(lsum)) * kLn2;
  }
  T* out = static_cast<T*>(a.o) + (int64_t)bh * D;
#pragma unroll
  for (int e = 0; e < kE; ++e)
    if (lane + 64 * e < D) out[lane + 64 * e] = to_elem<T>(nan ? NAN : acc[e] * scale_out);
  if (a.lse != nullptr && lane == 0) a.lse[bh] = lse;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  typedef Vec16<T> V;
  constexpr int kV = V::n;                 // elements per 16-byte load
  constexpr int kLpk = D / kV;             // lanes per key
  constexpr int kKpl = 64 / kLpk;          // keys per wavefront load
  constexpr int kU = kKeysPerWave / kKpl < 8 ? kKeysPerWave / kKpl : 8;  // loads per iteration
  constexpr int kKpi = kU * kKpl;          // keys per iteration
  constexpr int kIters = kKeysPerWave / kKpi;
  static_assert(D % kV == 0 && kLpk <= 64 && 64 % kLpk == 0, "head width");
  static_assert(kKeysPerWave % kKpi == 0, "iteration tiling");

  __shared__ int64_t s_off[kChunk];
  __shared__ float s_m[kWaves], s_l[kWaves];
  __shared__ float s_o[kWaves][D];

  const int bh = blockIdx.x;
  const int split = blockIdx.y;
  const int b = bh / a.heads;
  const int h = bh - b * a.heads;
  const int len = min(max(a.kv_len[b], 0), a.max_len);
  const int key0 = split * kChunk;
  const int tid = threadIdx.x;
  if (key0 >= len) {  // uniform over the workgroup, before any barrier
    if (len == 0 && split == 0) {  // an empty cache: no softmax, o = 0 and lse = -inf
      if (tid < D) static_cast<T*>(a.o)[(int64_t)bh * D + tid] = to_elem<T>(0.f);
      if (a.lse != nullptr && tid == 0) a.lse[bh] = -INFINITY;
    }
    return;
  }

  const int lane = tid & 63;
  const int wave = tid >> 6;

  // Row offset (elements, without the head term) of each of the chunk's keys.
  // Keys past len reuse the chunk's first row, which is valid; their scores
  // are masked below.
  int bad = 0;
#pragma unroll
  for (int t = tid; t < kChunk; t += 256) {
    const int j = key0 + t < len ? key0 + t : key0;
    int64_t off;
    if (a.block_table != nullptr) {
      int page = a.block_table[(int64_t)b * a.max_pages + j / a.page_size];
      if (page < 0 || page >= a.num_pages) {
        bad = 1;
        page = 0;
      }
      off = (int64_t)page * a.page_stride + (int64_t)(j % a.page_size) * a.row_stride;
    } else {
      off = (int64_t)b * a.page_stride + (int64_t)j * a.row_stride;
    }
    s_off[t] = off;
  }
  const int any_bad = __syncthreads_or(bad);

  const int g = lane / kLpk;  // key within a load
  const int c = lane % kLpk;  // 16-byte slice of the row
  float qf[kV];
  {
    const T* qp = static_cast<const T*>(a.q) + (int64_t)bh * D + c * kV;
    V::widen(*reinterpret_cast<const typename V::raw*>(qp), qf);
    const float qs = a.scale * kLog2e;
#pragma unroll
    for (int i = 0; i < kV; ++i) qf[i] *= qs;
  }
  const T* kb = static_cast<const T*>(a.k) + (int64_t)h * a.head_stride + c * kV;
  const T* vb = static_cast<const T*>(a.v) + (int64_t)h * a.head_stride + c * kV;

  float m = -INFINITY, l = 0.f;
  float o[kV];
#pragma unroll
  for (int i = 0; i < kV; ++i) o[i] = 0.f;

  if (!any_bad) {
#pragma unroll 1
    for (int it = 0; it < kIters; ++it) {
      const int ib = wave * kKeysPerWave + it * kKpi;  // chunk-local first key
      if (key0 + ib >= len) break;                     // uniform over the wavefront
      // each cached row is read once per step: nontemporal loads keep it from
      // displacing reusable lines in the caches
      typename V::raw kr[kU], vr[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        kr[u] = __builtin_nontemporal_load(reinterpret_cast<const typename V::raw*>(kb + s_off[ib + u * kKpl + g]));
#pragma unroll
      for (int u = 0; u < kU; ++u)
        vr[u] = __builtin_nontemporal_load(reinterpret_cast<const typename V::raw*>(vb + s_off[ib + u * kKpl + g]));

      float s[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float kf[kV];
        V::widen(kr[u], kf);
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < kV; ++i) acc = __builtin_fmaf(qf[i], kf[i], acc);
        s[u] = acc;
      }
#pragma unroll
      for (int x = 1; x < kLpk; x <<= 1) {
#pragma unroll
        for (int u = 0; u < kU; ++u) s[u] += __shfl_xor(s[u], x, 64);
      }
      float mx = m;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (key0 + ib + u * kKpl + g >= len) s[u] = -INFINITY;
        mx = fmaxf(mx, s[u]);
      }
      const float base = mx == -INFINITY ? 0.f : mx;
      const float alpha = exp2_fast(m - base);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < kV; ++i) o[i] *= alpha;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const float p = exp2_fast(s[u] - base);
        float vf[kV];
        V::widen(vr[u], vf);
        l += p;
#pragma unroll
        for (int i = 0; i < kV; ++i) o[i] = __builtin_fmaf(p, vf[i], o[i]);
      }
      m = mx;
    }
  }

  // lane groups of the wavefront -> one state per slice c
#pragma unroll
  for (int x = kLpk; x < 64; x <<= 1) {
    float o2[kV];
#pragma unroll
    for (int i = 0; i < kV; ++i) o2[i] = __shfl_xor(o[i], x, 64);
    const float m2 = __shfl_xor(m, x, 64);
    const float l2 = __shfl_xor(l, x, 64);
    merge_state(m, l, o, m2, l2, o2);
  }
  if (lane < kLpk) {
#pragma unroll
    for (int i = 0; i < kV; ++i) s_o[wave][lane * kV + i] = o[i];
    if (lane == 0) {
      s_m[wave] = m;
      s_l[wave] = l;
    }
  }
  __syncthreads();

  // wavefronts -> the split's state; a sequence of one split is final here
  const int ns = (len + kChunk - 1) / kChunk;
  if (tid < D) {
    float mw = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mw = fmaxf(mw, s_m[w]);
    const float base = mw == -INFINITY ? 0.f : mw;
    float lw = 0.f, ow = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = exp2_fast(s_m[w] - base);
      lw += s_l[w] * f;
      ow += s_o[w][tid] * f;
    }
    if (ns == 1) {
      static_cast<T*>(a.o)[(int64_t)bh * D + tid] = to_elem<T>(any_bad ? NAN : ow / lw);
      if (a.lse != nullptr && tid == 0) a.lse[bh] = any_bad ? NAN : (mw + __log2f(lw)) * kLn2;
    } else {
      const int64_t part = (int64_t)bh * a.splits + split;
      a.part_o[part * D + tid] = ow;
      if (tid == 0) {
        a.part_ml[2 * part] = any_bad ? NAN : mw;
        a.part_ml[2 * part + 1] = any_bad ? NAN : lw;
      }
    }
  }
}

// One wavefront per (batch, head) of two or more splits (the others were
// finished by the split kernel): merge_splits.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= a.batch * a.heads) return;  // uniform over the wavefront; no barrier follows
  const int len = min(max(a.kv_len[bh / a.heads], 0), a.max_len);
  const int ns = (len + kChunk - 1) / kChunk;
  if (ns < 2) return;
  merge_splits<T, D>(a, bh, ns, lane);
}

template <typename T, int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  const int bhs = a.batch * a.heads;
  hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(bhs, a.splits), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((bhs + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 16: return launch_decode_d<T, 16>(a, stream);
    case 32: return launch_decode_d<T, 32>(a, stream);
    case 64: return launch_decode_d<T, 64>(a, stream);
    case 128: return launch_decode_d<T, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) { return launch_decode<bf16>(a, stream); }
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream) { return launch_decode<float>(a, stream); }

}  // namespace mha
