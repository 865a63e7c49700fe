// Fused scaled dot-product attention forward, bf16 in/out, d_k = d_v = 64, gfx950.
//
// Computes O = softmax(scale * Q K^T (+ causal mask)) V per (batch, head)
// ("The Transformer" (hoshank.vercel.app), "The Mathematics", Attention
// equation) in one pass, without forming the score matrix in memory: the
// exact result is reached by streaming key/value tiles and keeping a running
// row maximum and row sum (the tiling idea the pages credit to FlashAttention,
// "32 Transformer", "Connections"; re-derived here for CDNA4).
//
// Work decomposition
//   workgroup = 256 threads = 4 wavefronts; it owns 128 query rows of one
//   (batch, head); each wavefront owns 32 of them.
//   key/value tiles of 64 rows are staged through LDS, double buffered, with
//   the next tile's global loads in flight while the current one is used.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, fp32 accumulate)
//   Scores are formed transposed, S^T = K Q^T: the MFMA's B operand is the
//   wavefront's Q^T (kept in registers for the whole kernel) and its A operand
//   is a 32-key slab of K read from LDS. In the 32x32 accumulator layout lane l
//   then holds column n = l % 32 (one query) and 16 rows (keys), so a query's
//   row maximum and row sum are in-register reductions plus one exchange
//   between lane halves.
//   K rows are written to LDS in a permuted order so that accumulator register
//   r of lane half hf holds key 16*(r/8) + 8*hf + (r%8) of its 32-key slab.
//   After conversion to bf16 those registers are, unchanged, the B operand of
//   O^T = V^T P^T (8 consecutive keys per lane), so P never goes through LDS.
//   V is transposed into LDS ([d][key]) while staging, two keys per 32-bit word.
//
// Softmax: exp2 with scale*log2(e) folded into one FMA; the row sum is
// accumulated from the bf16-rounded weights that the P V product uses, so the
// final 1/l normalises exactly what was summed.
// Causal: tiles wholly above the diagonal are never loaded; per wavefront, a
// tile whose first key lies past the wavefront's last query is skipped; only
// tiles that straddle the diagonal (or the ragged end) apply per-element masks.
#include <hip/hip_runtime.h>
#include <math.h>

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

constexpr int kD = 64;         // head width handled by this kernel
constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kPitch = 72;     // LDS row pitch, bf16 elements (144 bytes: conflict-free 16-byte reads)
constexpr int kTile = kBN * kPitch;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ u32x4 ld16(const bf16* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Sum of a packed bf16 pair, added to acc in fp32 (v_dot2c_f32_bf16 with (1, 1)).
__device__ __forceinline__ float add_pair(unsigned pair, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}

// LDS row that receives key offset kappa (0..31) of a 32-key slab, so that the
// S^T accumulator register r of lane half hf maps to key 16*(r/8) + 8*hf + r%8.
// Accumulator row m = 8*(r/4) + 4*hf + r%4 in the 32x32 MFMA output layout.
__device__ __forceinline__ int key_to_lds_row(int kappa) {
  return 8 * (2 * (kappa >> 4) + ((kappa >> 2) & 1)) + 4 * ((kappa >> 3) & 1) + (kappa & 3);
}

template <bool kCausal>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_d64(AttnArgs a, float c, unsigned q_sign,
                                                            int n_qblk) {
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * 2 * kTile];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lq = lane & 31;
  const int hf = lane >> 5;
  const int n_q = a.n_q, n_k = a.n_k;

  // ---- workgroup -> (batch*head, query block)
  int bh, qblk;
  if (kCausal) {
    // heaviest query blocks (most key tiles) are dispatched first
    const int BH = a.batch * a.heads;
    qblk = n_qblk - 1 - (int)(blockIdx.x / BH);
    bh = (int)(blockIdx.x % BH);
  } else {
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous run of logical ids so the query blocks of one (batch, head)
    // share that XCD's L2 and its K/V.
    const int total = gridDim.x, id = blockIdx.x;
    const int per = total >> 3, rem = total & 7, x = id & 7, slot = id >> 3;
    const int logical = (x < rem) ? x * (per + 1) + slot : rem * (per + 1) + (x - rem) * per + slot;
    bh = logical / n_qblk;
    qblk = logical - bh * n_qblk;
  }
  const int b = bh / a.heads, h = bh - b * a.heads;
  const bf16* qp = static_cast<const bf16*>(a.q) + b * a.q_sb + h * a.q_sh;
  const bf16* kp = static_cast<const bf16*>(a.k) + b * a.k_sb + h * a.k_sh;
  const bf16* vp = static_cast<const bf16*>(a.v) + b * a.v_sb + h * a.v_sh;
  bf16* op = static_cast<bf16*>(a.o) + b * a.o_sb + h * a.o_sh;

  const int q_wave0 = qblk * kBM + wave * 32;
  const int my_q = q_wave0 + lq;

  // ---- this lane's slice of Q^T: d = 16*kk + 8*hf + 0..7 of query my_q
  u32x4 qf[4];
  if (my_q < n_q) {
    const bf16* src = qp + (int64_t)my_q * a.q_sn + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = ld16(src + 16 * kk) ^ q_sign;
  } else {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qf[kk] = u32x4{0, 0, 0, 0};
  }

  const int kv_end = kCausal ? min(n_k, qblk * kBM + kBM) : n_k;
  const int ntiles = (kv_end + kBN - 1) / kBN;

  // ---- cooperative staging assignment
  // K: two 16-byte chunks per thread, rows (tid/8) and (tid/8)+32, chunk tid%8
  const int k_row = tid >> 3, k_chunk = tid & 7;
  const int k_lds = key_to_lds_row(k_row);
  // V: keys 2*(tid%32) and 2*(tid%32)+1, d chunk tid/32
  const int v_key = (tid & 31) * 2, v_chunk = tid >> 5;

  u32x4 kreg[2], vreg[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = k0 + k_row + 32 * i;
      kreg[i] = key < n_k ? ld16(kp + (int64_t)key * a.k_sn + 8 * k_chunk) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = k0 + v_key + i;
      vreg[i] = key < n_k ? ld16(vp + (int64_t)key * a.v_sn + 8 * v_chunk) : u32x4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
    bf16* Ks = smem + buf * 2 * kTile;
    bf16* Vt = Ks + kTile;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4*>(Ks + (32 * i + k_lds) * kPitch + 8 * k_chunk) = kreg[i];
    // V^T[d][key]: word (d, key pair) = V[key][d] | V[key+1][d] << 16
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned w0 = vreg[0][e >> 1], w1 = vreg[1][e >> 1];
      const unsigned word = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u)) : ((w0 & 0xffffu) | (w1 << 16));
      *reinterpret_cast<unsigned*>(Vt + (8 * v_chunk + e) * kPitch + v_key) = word;
    }
  };

  f32x16 o0 = {}, o1 = {};   // O^T, d rows 0..31 and 32..63, column = query lq
  float m_run = -INFINITY;   // running max of raw scores (same in both lane halves)
  float l_run = 0.f;         // running sum over this lane half's keys

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * kBN;
    const bool more = t + 1 < ntiles;
    if (more) gload(k0 + kBN);
    const bf16* Ks = smem + (t & 1) * 2 * kTile;
    const bf16* Vt = Ks + kTile;

    if (!kCausal || k0 <= q_wave0 + 31) {
      // ---- S^T = K Q^T for two 32-key slabs
      f32x16 s0 = {}, s1 = {};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 bq = as_bf16x8(qf[kk]);
        const bf16x8 a0 = as_bf16x8(ld16(Ks + lq * kPitch + 16 * kk + 8 * hf));
        const bf16x8 a1 = as_bf16x8(ld16(Ks + (32 + lq) * kPitch + 16 * kk + 8 * hf));
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, bq, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, bq, s1, 0, 0, 0);
      }
      float sv[32];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sv[r] = s0[r];
        sv[16 + r] = s1[r];
      }
      // key of sv[i]: k0 + 16*(i/8) + 8*hf + i%8
      const bool need_mask = (k0 + kBN > n_k) || (kCausal && k0 + kBN - 1 > q_wave0);
      unsigned visible = 0xffffffffu;
      if (need_mask) {
        visible = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int key = k0 + 16 * (i >> 3) + 8 * hf + (i & 7);
          const bool ok = key < n_k && (!kCausal || key <= my_q);
          visible |= (ok ? 1u : 0u) << i;
          sv[i] = ok ? sv[i] : -INFINITY;
        }
      }
      float tmax = sv[0];
#pragma unroll
      for (int i = 1; i < 32; ++i) tmax = __builtin_fmaxf(tmax, sv[i]);
      tmax = __builtin_fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = __builtin_fmaxf(m_run, tmax);
      const float mc = (m_new == -INFINITY ? 0.f : m_new) * c;
      const float alpha = (m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(m_run, c, -mc));
      m_run = m_new;

      // ---- weights, rounded to bf16; the row sum uses the rounded values
      unsigned pw[16];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], c, -mc));
        float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], c, -mc));
        if (need_mask) {
          p0 = (visible >> (2 * i)) & 1u ? p0 : 0.f;
          p1 = (visible >> (2 * i + 1)) & 1u ? p1 : 0.f;
        }
        pw[i] = pack_bf16(p0, p1);
        psum = add_pair(pw[i], psum);
      }
      l_run = __builtin_fmaf(l_run, alpha, psum);
      o0 *= alpha;
      o1 *= alpha;

      // ---- O^T += V^T P^T, four 16-key steps
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 bp = as_bf16x8(u32x4{pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]});
        const bf16x8 v0 = as_bf16x8(ld16(Vt + lq * kPitch + 16 * j + 8 * hf));
        const bf16x8 v1 = as_bf16x8(ld16(Vt + (32 + lq) * kPitch + 16 * j + 8 * hf));
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, bp, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, bp, o1, 0, 0, 0);
      }
    }
    if (more) lstore((t + 1) & 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds d = 32*blk + 8*g + 4*hf + 0..3 of query my_q
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (my_q < n_q) {
    const float inv = 1.0f / l_tot;
    bf16* dst = op + (int64_t)my_q * a.o_sn + 4 * hf;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      *reinterpret_cast<u32x2*>(dst + 8 * g) =
          u32x2{pack_bf16(o0[4 * g] * inv, o0[4 * g + 1] * inv), pack_bf16(o0[4 * g + 2] * inv, o0[4 * g + 3] * inv)};
      *reinterpret_cast<u32x2*>(dst + 32 + 8 * g) =
          u32x2{pack_bf16(o1[4 * g] * inv, o1[4 * g + 1] * inv), pack_bf16(o1[4 * g + 2] * inv, o1[4 * g + 3] * inv)};
    }
    if (a.lse != nullptr && hf == 0) a.lse[(int64_t)bh * n_q + my_q] = (m_run * c + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t stream) {
  const float kLog2e = 1.4426950408889634f;
  const float c = fabsf(a.scale) * kLog2e;
  const unsigned q_sign = a.scale < 0.f ? 0x80008000u : 0u;  // negate Q exactly: scale*s = |scale|*(-q).k
  const int n_qblk = (a.n_q + kBM - 1) / kBM;
  const dim3 grid((unsigned)(n_qblk * a.batch * a.heads));
  if (a.causal)
    hipLaunchKernelGGL(attn_fwd_bf16_d64<true>, grid, dim3(256), 0, stream, a, c, q_sign, n_qblk);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_d64<false>, grid, dim3(256), 0, stream, a, c, q_sign, n_qblk);
  return hipGetLastError();
}

}  // namespace mha
