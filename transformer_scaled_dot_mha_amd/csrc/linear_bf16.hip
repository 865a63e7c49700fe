// Projection Y = X W in bf16 with fp32 accumulation on the matrix cores, gfx950.
//
// The Q, K, V projections and the output projection W^O of multi-head
// attention ("The Transformer" (hoshank.vercel.app), "The Mathematics",
// MultiHead equation: each W is a d_model x d_k block applied on the right).
// X is (m, k) row-major, W is (k, n) row-major (in, out), Y is (m, n) row-major.
// Because head i owns columns [i*d, (i+1)*d), the row-major Y already *is* the
// head-split (batch, n, heads, d) layout; no permutation pass is needed.
//
// Tile 256 x 128 per workgroup of 4 wavefronts (128 x 128 for launches too
// small to give every CU two workgroups); wavefront w owns rows
// 64*w .. +63 and all 128 columns as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16,
// so every fragment read from LDS feeds two or four MFMAs (0.75 KB of LDS
// reads per MFMA; a 64 x 64 wavefront tile would need 1 KB, the LDS's whole
// rate at full MFMA issue). The MFMA computes Y^T blocks: its A operand is a
// 32 x 16 slice of W^T, its B operand a 16 x 32 slice of X^T, and each lane
// ends with 4 consecutive columns of one row.
// X and W are staged through LDS in 32-deep k chunks, double buffered (60 KB),
// with the next chunk's global loads in flight during the MFMAs; two
// workgroups share a CU, so one computes while the other waits on its loads.
// X rows are copied as they are (coalesced 16-byte loads, 80-byte LDS rows for
// conflict-free fragment reads); W is read row-major and transposed while it
// is written (two k values per column, 4 bytes), so every fragment is one
// 16-byte read.
// Raw buffer loads bound every read: rows past m, k past the last column and
// rows of W past k read as zero, with no per-lane bounds branches.
// Up to three independent problems sharing n and k run in one launch (the Q,
// K and V projections); the workgroup order puts the column tiles and groups
// of one row tile on one XCD, so that a self-attention X row tile is fetched
// from HBM once.
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

constexpr int kTN = 128, kTK = 32;
constexpr int kPitch = 40;  // LDS row pitch in elements (80 bytes: conflict-free 16-byte reads)
constexpr int kWTile = kTN * kPitch;
constexpr int kBufferFlags = 0x00020000;  // raw buffer descriptor word 3 (gfx9 family: 32-bit data format)
constexpr unsigned kOutOfRange = 0x80000000u;  // byte offset past any record count: the load returns zero

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// Pack a lane's 4 values of column group g (columns 8g + 4hf + 0..3) of both
// lane halves into one 16-byte row chunk: half 0 ends with group 2t, half 1
// with group 2t + 1.
__device__ __forceinline__ u32x4 gather_row_chunk(unsigned a0, unsigned a1, unsigned b0, unsigned b1) {
  const auto x0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto x1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  return u32x4{(unsigned)x0[0], (unsigned)x1[0], (unsigned)x0[1], (unsigned)x1[1]};
}

// kTM = 256: wavefront w owns rows 64w..+63 and all 128 columns (4 x 2 MFMA
// blocks). kTM = 128, for launches too small to give every CU two
// workgroups: wavefronts form 2 x 2, each 64 rows x 64 columns (2 x 2 blocks).
template <int kTM>
__global__ __launch_bounds__(256, 2) void linear_bf16_kernel(LinearArgs args, int tiles_n, int tiles_m) {
  constexpr int kWM = kTM / 64;         // wavefronts along m
  constexpr int kWC = 128 / (4 / kWM);  // columns per wavefront
  constexpr int kNB = kWC / 32;         // 32-column MFMA blocks per wavefront
  constexpr int kXLoads = kTM / 64;     // 16-byte X loads per thread per chunk
  constexpr int kXTile = kTM * kPitch;
  constexpr int kStage = kXTile + kWTile;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * kStage];
  const int n = args.n, kdim = args.k, groups = args.groups;

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs; each XCD
  // gets a contiguous run of logical ids, ordered (row tile, group, column
  // tile) with the column tile fastest.
  const int total = gridDim.x, id = blockIdx.x;
  const int per = total >> 3, rem = total & 7, xcd = id & 7, slot = id >> 3;
  const int logical = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int tn = logical % tiles_n;
  const int rest = logical / tiles_n;
  const int gi = rest % groups, tm = rest / groups;
  const LinearGroup g = gi == 0 ? args.g[0] : (gi == 1 ? args.g[1] : args.g[2]);
  const int m0 = tm * kTM, n0 = tn * kTN;
  if (tm >= tiles_m || m0 >= g.m) return;  // workgroup-uniform

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lq = lane & 31, hf = lane >> 5;
  const int wrow = 64 * (wave % kWM), wcol = kWC * (wave / kWM);
  const bf16* X = static_cast<const bf16*>(g.x) + (int64_t)m0 * g.ldx;
  const bf16* W = static_cast<const bf16*>(g.w) + n0;
  bf16* Y = static_cast<bf16*>(g.y);
  const int valid_m = min(kTM, g.m - m0);
  const int valid_n = min(kTN, n - n0);

  // X staging: 16-byte chunk tid%4 of rows tid/4 + 64*i
  const int x_c = tid & 3, x_r = tid >> 2;
  // W staging: k rows 2*(tid%16) + 0..1, 8-column chunk tid/16
  const int w_q = tid & 15, w_c = tid >> 4;
  const unsigned w_off = (unsigned)(((int64_t)(2 * w_q) * g.ldw + 8 * w_c) * 2);

  u32x4 xr[kXLoads], wr[2];
  auto gload = [&](int k0) {
    const int cols = min(kTK, kdim - k0);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(X + k0), (short)0, (int)(((int64_t)(valid_m - 1) * g.ldx + cols) * 2), kBufferFlags);
    // k past the last column would read the next row's values: force zero
    const unsigned xo = 8 * x_c < cols ? (unsigned)(((int64_t)x_r * g.ldx + 8 * x_c) * 2) : kOutOfRange;
    const unsigned xstep = (unsigned)(64 * g.ldx * 2);
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) xr[i] = bload(rx, xo == kOutOfRange ? kOutOfRange : xo + i * xstep);
    const int rows = min(kTK, kdim - k0);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + (int64_t)k0 * g.ldw), (short)0, (int)(((int64_t)(rows - 1) * g.ldw + valid_n) * 2), kBufferFlags);
#pragma unroll
    for (int i = 0; i < 2; ++i) wr[i] = bload(rw, w_off + (unsigned)(i * g.ldw * 2));
  };
  auto lstore = [&](int buf) {
    bf16* Xs = smem + buf * kStage;
    bf16* Wt = Xs + kXTile;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) *reinterpret_cast<u32x4*>(Xs + (x_r + 64 * i) * kPitch + 8 * x_c) = xr[i];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned sel = (e & 1) ? 0x07060302u : 0x05040100u;
      *reinterpret_cast<unsigned*>(Wt + (8 * w_c + e) * kPitch + 2 * w_q) =
          __builtin_amdgcn_perm(wr[1][e >> 1], wr[0][e >> 1], sel);
    }
  };

  f32x16 acc[kNB][2] = {};  // [n block][m block], Y^T layout
  auto compute = [&](int buf) {
    const bf16* Xs = smem + buf * kStage;
    const bf16* Wt = Xs + kXTile;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 xf[2], wf[kNB];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        xf[mb] = *reinterpret_cast<const u32x4*>(Xs + (wrow + 32 * mb + lq) * kPitch + 16 * s + 8 * hf);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        wf[nb] = *reinterpret_cast<const u32x4*>(Wt + (wcol + 32 * nb + lq) * kPitch + 16 * s + 8 * hf);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wf[nb]), as_bf16x8(xf[mb]), acc[nb][mb],
                                                                0, 0, 0);
    }
  };

  const int nchunks = (kdim + kTK - 1) / kTK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) gload((c + 1) * kTK);
    compute(c & 1);
    if (more) lstore((c + 1) & 1);
    __syncthreads();
  }

  // lane holds row wrow + 32*mb + lq and columns wcol + 32*nb + 8*q + 4*hf + 0..3;
  // the two halves swap groups so that each lane writes 16-byte row chunks.
  // Optional epilogue: + bias[column], then max(0, .), in fp32 before rounding.
  const bf16* Bias = static_cast<const bf16*>(g.bias);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int row = wrow + 32 * mb + lq;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
      f32x16 v = acc[nb][mb];
      if (Bias != nullptr) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // columns 32*nb + 8*q + 4*hf + 0..3 lie in one 8-column chunk: all valid or none
          if (wcol + 32 * nb + 8 * q < valid_n) {
            const u32x2 bw = *reinterpret_cast<const u32x2*>(Bias + n0 + wcol + 32 * nb + 8 * q + 4 * hf);
            v[4 * q] += __builtin_bit_cast(float, bw[0] << 16);
            v[4 * q + 1] += __builtin_bit_cast(float, bw[0] & 0xffff0000u);
            v[4 * q + 2] += __builtin_bit_cast(float, bw[1] << 16);
            v[4 * q + 3] += __builtin_bit_cast(float, bw[1] & 0xffff0000u);
          }
        }
      }
      if (args.relu) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = __builtin_fmaxf(v[r], 0.f);
      }
      unsigned w[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[q][0] = pack_bf16(v[4 * q], v[4 * q + 1]);
        w[q][1] = pack_bf16(v[4 * q + 2], v[4 * q + 3]);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const u32x4 chunk = gather_row_chunk(w[2 * t][0], w[2 * t][1], w[2 * t + 1][0], w[2 * t + 1][1]);
        const int col = wcol + 32 * nb + 16 * t + 8 * hf;
        if (row < valid_m && col < valid_n)
          *reinterpret_cast<u32x4*>(Y + (int64_t)(m0 + row) * g.ldy + n0 + col) = chunk;
      }
    }
  }
}

}  // namespace

hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t stream) {
  int max_m = 0;
  for (int i = 0; i < a.groups; ++i) max_m = a.g[i].m > max_m ? a.g[i].m : max_m;
  const int tiles_n = (a.n + kTN - 1) / kTN;
  // 256-row tiles unless that leaves CUs without a second workgroup (2 per CU on 256 CUs)
  const int64_t big = (int64_t)tiles_n * ((max_m + 255) / 256) * a.groups;
  if (big >= 512) {
    const int tiles_m = (max_m + 255) / 256;
    hipLaunchKernelGGL((linear_bf16_kernel<256>), dim3((unsigned)big), dim3(256), 0, stream, a, tiles_n, tiles_m);
  } else {
    const int tiles_m = (max_m + 127) / 128;
    const dim3 grid((unsigned)(tiles_n * tiles_m * a.groups));
    hipLaunchKernelGGL((linear_bf16_kernel<128>), grid, dim3(256), 0, stream, a, tiles_n, tiles_m);
  }
  return hipGetLastError();
}

}  // namespace mha
