// Projection Y = X W in bf16 with fp32 accumulation on the matrix cores, gfx950.
//
// The Q, K, V projections and the output projection W^O of multi-head
// attention ("The Transformer" (hoshank.vercel.app), "The Mathematics",
// MultiHead equation: each W is a d_model x d_k block applied on the right),
// and the two FFN products of the encoder layer (same page, FFN equation).
// X is (m, k) row-major, W is (k, n) row-major (in, out), Y is (m, n) row-major.
// Because head i owns columns [i*d, (i+1)*d), the row-major Y already *is* the
// head-split (batch, n, heads, d) layout; no permutation pass is needed.
//
// Tile kTM x 128 per workgroup of 4 wavefronts: kTM = 256 (wavefront w owns
// rows 64w..+63 and all 128 columns, 2 x 4 blocks of v_mfma_f32_32x32x16_bf16),
// kTM = 128 (wavefronts 2 x 2, each 64 x 64) or, for grids smaller than the
// CU count, kTM = 64 (each wavefront 64 rows x 32 columns). The MFMA computes Y^T
// blocks: its A operand is a 32 x 16 slice of W^T, its B operand a 16 x 32
// slice of X^T, and each lane ends with 4 consecutive columns of one row.
//
// Staging: 32-deep k chunks go straight from global memory into LDS with
// buffer loads that write LDS (no staging registers, no VALU), into two
// stages: chunk c + 1 loads while chunk c is multiplied; one barrier per
// chunk. Two stages keep the 128-row tile at 32 KB of LDS, so five workgroups
// share a CU (96 VGPRs), and more resident workgroups hide the load latency
// better than a deeper ring with fewer of them. The loads are issued from
// inline asm and awaited with explicit vmcnt waits. X rows keep their layout (64-byte rows, the 16-byte chunk c
// of row r stored at position c ^ ((r >> 2) & 3), so that the 16-byte
// fragment reads of 16 consecutive rows hit distinct banks); W rows keep
// theirs (256-byte rows, chunk c of k-row r at c ^ (r & 15)) and the W^T
// fragments are read with the transposing LDS load ds_read_b64_tr_b16.
// Buffer records bound every read: rows past m and rows of W past k read as
// zero, and so do X chunks past the last column (out-of-range offset).
//
// Up to three independent problems sharing n and k run in one launch (the Q,
// K and V projections); the workgroup order puts the column tiles and groups
// of one row tile on one XCD, so that a self-attention X row tile is fetched
// from HBM once. The tile height is the one whose workgroup count fills whole
// rounds of 512 workgroups best, 128 on ties: at these sizes the kernel is
// bound by load latency rather than by the matrix cores, and the smaller tile
// keeps more workgroups in flight (five per CU against two for the 256-row
// tile, by LDS).
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
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kTN = 128, kTK = 32;
constexpr int kXRow = kTK * 2;  // 64-byte X rows in LDS (one k chunk of an m row)
constexpr int kWRow = kTN * 2;  // 256-byte W rows in LDS (the tile's n columns of a k row)
constexpr int kNStages = 2;     // LDS stages: chunk c is read while c + 1 loads
constexpr int kBufferFlags = 0x00020000;       // raw buffer descriptor word 3 (gfx9 family: 32-bit data format)
constexpr unsigned kOutOfRange = 0x80000000u;  // byte offset past any record count: the load returns zero

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}
// Pack a lane's 4 values of column group g (columns 8g + 4hf + 0..3) of both
// lane halves into one 16-byte row chunk: half 0 ends with group 2t, half 1
// with group 2t + 1.
__device__ __forceinline__ u32x4 gather_row_chunk(unsigned a0, unsigned a1, unsigned b0, unsigned b1) {
  const auto x0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto x1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  return u32x4{(unsigned)x0[0], (unsigned)x1[0], (unsigned)x0[1], (unsigned)x1[1]};
}
// LDS byte address of a shared-memory pointer.
__device__ __forceinline__ unsigned lds_off(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p;
}
// 16 bytes per lane from a raw buffer into LDS at lds_byte + 16 * lane;
// offsets past the record write zeros. The wave-uniform LDS base goes in m0
// through the asm's {m0} operand, so the compiler sets m0 itself and knows
// the register is taken.
__device__ __forceinline__ void dma16(u32x4 rsrc, unsigned voff, unsigned lds_byte) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_byte) : "memory");
}
// Raw buffer descriptor (stride 0) over `bytes` bytes from base.
__device__ __forceinline__ u32x4 make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long b = (unsigned long long)base;
  return u32x4{(unsigned)b, (unsigned)(b >> 32) & 0xffffu, bytes, (unsigned)kBufferFlags};
}

// kTM = 256: wavefront w owns rows 64w..+63 and all 128 columns (2 x 4 MFMA
// blocks). kTM = 128: wavefronts form 2 x 2, each 64 rows x 64 columns.
// kTM = 64: wavefront w owns all 64 rows and columns 32w..+31.
// LDS stage: X tile (kTM rows x 64 B), then W tile (32 k-rows x 256 B).
// kPair: a 4-stage ring, two chunks loaded and multiplied per barrier (for
// grids of at most two workgroups per CU, where the deeper ring costs no
// residency).
template <int kTM, bool kPair = false>
__global__ __launch_bounds__(256, 2) void linear_bf16_kernel(LinearArgs args, int tiles_n, int tiles_m) {
  constexpr int kWM = kTM / 64;         // wavefronts along m
  constexpr int kWC = 128 / (4 / kWM);  // columns per wavefront
  constexpr int kNB = kWC / 32;         // 32-column MFMA blocks per wavefront
  constexpr int kXBytes = kTM * kXRow;
  constexpr int kStageBytes = kXBytes + kTK * kWRow;
  constexpr int kStages = kPair ? 4 : kNStages;
  constexpr int kXDma = kTM / 64;  // X loads per wavefront per chunk (16 rows of 64 B each)
  constexpr int kWDma = 2;         // W loads per wavefront per chunk (4 rows of 256 B each)
  // the stages, and afterwards the output tile, 128 rows of 256 bytes at a
  // time (the 256-row tile goes out in two passes, so that its LDS stays at
  // the two stages' 48 KB and three workgroups share a CU)
  constexpr int kEpiRows = kTM < 128 ? kTM : 128;
  constexpr int kSmem = kStages * kStageBytes > kEpiRows * kWRow ? kStages * kStageBytes : kEpiRows * kWRow;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
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
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int wrow = 64 * (wave % kWM), wcol = kWC * (wave / kWM);
  const bf16* X = static_cast<const bf16*>(g.x) + (int64_t)m0 * g.ldx;
  const bf16* W = static_cast<const bf16*>(g.w) + n0;
  bf16* Y = static_cast<bf16*>(g.y);
  const int valid_m = min(kTM, g.m - m0);
  const int valid_n = min(kTN, n - n0);
  const int ldx = (int)g.ldx, ldw = (int)g.ldw;

  const unsigned smem_base = lds_off(smem);
  // Per-lane load offsets, the same for every chunk (the chunk moves the buffer
  // base). Load i of wavefront w fills X rows (kTM/4) w + 16 i + 0..15, lane l
  // LDS position (row l/4, slot l%4), which holds chunk (l%4) ^ ((row >> 2) & 3);
  // W load i fills k-rows 8w + 4i + 0..3, lane l slot l%16 of row l/16, which
  // holds chunk (l%16) ^ (row & 15).
  unsigned xdo[kXDma], wdo[kWDma];
  int xch[kXDma];
#pragma unroll
  for (int i = 0; i < kXDma; ++i) {
    const int row = (kTM / 4) * wave + 16 * i + (lane >> 2);
    xch[i] = (lane & 3) ^ ((row >> 2) & 3);
    xdo[i] = (unsigned)((row * ldx + 8 * xch[i]) * 2);
  }
#pragma unroll
  for (int i = 0; i < kWDma; ++i) {
    const int kr = 8 * wave + 4 * i + (lane >> 4);
    wdo[i] = (unsigned)((kr * ldw + 8 * ((lane & 15) ^ (kr & 15))) * 2);
  }
  // loads of k chunk c into stage c % 3 (X chunks past the last column read zero)
  auto dma_chunk = [&](int c) {
    const int k0 = c * kTK;
    const int cols = min(kTK, kdim - k0);
    const u32x4 rx = make_rsrc(X + k0, (unsigned)(((valid_m - 1) * ldx + cols) * 2));
    const u32x4 rw = make_rsrc(W + (int64_t)k0 * ldw, (unsigned)(((cols - 1) * ldw + valid_n) * 2));
    const unsigned sb = smem_base + (unsigned)((c % kStages) * kStageBytes);
    const bool full = cols == kTK;  // workgroup-uniform
#pragma unroll
    for (int i = 0; i < kXDma; ++i) {
      // (an arithmetic select: a select between the two values compiled to a
      // select of addresses into the offset array, which then stayed in memory)
      const unsigned off = xdo[i] | ((full || 8 * xch[i] < cols) ? 0u : kOutOfRange);
      dma16(rx, off, sb + (unsigned)(((kTM / 4) * wave_u + 16 * i) * kXRow));
    }
#pragma unroll
    for (int i = 0; i < kWDma; ++i) dma16(rw, wdo[i], sb + (unsigned)(kXBytes + (8 * wave_u + 4 * i) * kWRow));
  };
  // Per-lane fragment offsets within a stage. X (B operand, k step s): row
  // wrow + 32 mb + lq, chunk 2s + hf. W^T (A operand) through two transposing
  // reads: in each 16-lane group gi (lane j), read r addresses k-row
  // 16 s + 8 (gi >> 1) + 4 r + j / 4, columns 32 nb + 16 (gi & 1) + 4 (j % 4) + 0..3,
  // so lane l receives 4 consecutive k of column 32 nb + l % 32; with the
  // swizzle the position's bit 2 is (nb & 1) ^ r and bit 3 (nb >> 1) ^ (gi >> 1).
  unsigned xoff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) xoff[s] = (unsigned)((wrow + lq) * kXRow + 16 * ((2 * s + hf) ^ ((lq >> 2) & 3)));
  // (the 128-byte half h = nb >> 1 is added where it is used: an array indexed
  // by a wavefront-dependent block number was kept in memory by the compiler)
  unsigned woff_base;
  int wsel;
  {
    const int gi = lane >> 4, j = lane & 15;
    const int c_lane = 2 * (gi & 1) + ((j & 3) >> 1);
    const int kr_lane = 8 * (gi >> 1) + (j >> 2);
    woff_base = (unsigned)(kXBytes + kr_lane * kWRow + 16 * (c_lane ^ (j >> 2)) + 8 * (j & 1));
    wsel = gi >> 1;
  }

  f32x16 acc[kNB][2] = {};  // [n block][m block], Y^T layout
  auto compute = [&](int c) {
    const unsigned sb = smem_base + (unsigned)((c % kStages) * kStageBytes);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4 xf[2], wf[kNB];
      const lds_char* xp = (const lds_char*)(size_t)(sb + xoff[s]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) xf[mb] = *(const __attribute__((address_space(3))) u32x4*)(xp + 32 * mb * kXRow);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const int col_nb = wcol / 32 + nb;  // 32-column block within the tile
        const lds_char* wp = (const lds_char*)(size_t)(sb + woff_base + 128u * (unsigned)(((col_nb >> 1) ^ wsel) & 1));
        const v4i16 w0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(wp + 16 * s * kWRow + 64 * (col_nb & 1)));
        const v4i16 w1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(wp + 16 * s * kWRow + 4 * kWRow + 64 * ((col_nb & 1) ^ 1)));
        const u32x2 a0 = __builtin_bit_cast(u32x2, w0), a1 = __builtin_bit_cast(u32x2, w1);
        wf[nb] = u32x4{a0[0], a0[1], a1[0], a1[1]};
      }
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(wf[nb]), as_bf16x8(xf[mb]), acc[nb][mb], 0, 0, 0);
    }
  };

  // Chunk c: wait for its loads, barrier (which also ends every read of the
  // stage chunk c + 1 reuses), start the loads of chunk c + 1, multiply.
  const int nchunks = (kdim + kTK - 1) / kTK;
  if constexpr (!kPair) {
    dma_chunk(0);
    for (int c = 0; c < nchunks; ++c) {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (c + 1 < nchunks) dma_chunk(c + 1);
      compute(c);
    }
  } else {
    // chunks c and c + 1 per barrier; the barrier also ends every read of the
    // stages that chunks c + 2 and c + 3 reuse
    dma_chunk(0);
    if (1 < nchunks) dma_chunk(1);
    for (int c = 0; c < nchunks; c += 2) {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (c + 2 < nchunks) dma_chunk(c + 2);
      if (c + 3 < nchunks) dma_chunk(c + 3);
      compute(c);
      if (c + 1 < nchunks) compute(c + 1);
    }
  }

  // Epilogue. A lane holds row wrow + 32*mb + lq and columns wcol + 32*nb +
  // 8*q + 4*hf + 0..3; the two halves swap groups so that each lane has whole
  // 16-byte row chunks. Optional: + bias[column], then max(0, .), in fp32
  // before rounding. The tile goes through LDS (the stages are free by now:
  // kTM rows of 256 bytes, chunk c of row r at c ^ (r & 15), conflict-free
  // both ways) so that the global stores write whole rows: 16 lanes per
  // 256-byte row, where the accumulator layout would have each store
  // instruction touch 32 rows with 32 bytes each.
  const bf16* Bias = static_cast<const bf16*>(g.bias);
  unsigned w[kNB][2][4][2];  // packed bf16 outputs: [n block][m block][group][pair]
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
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
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[nb][mb][q][0] = pack_bf16(v[4 * q], v[4 * q + 1]);
        w[nb][mb][q][1] = pack_bf16(v[4 * q + 2], v[4 * q + 3]);
      }
    }
  }
  constexpr int kPasses = kTM / kEpiRows;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    __syncthreads();  // every wavefront is done reading the stages (or the previous pass's rows)
    if (wrow / kEpiRows == pass) {  // wave-uniform
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int row = wrow - kEpiRows * pass + 32 * mb + lq;
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const u32x4 chunk = gather_row_chunk(w[nb][mb][2 * t][0], w[nb][mb][2 * t][1], w[nb][mb][2 * t + 1][0],
                                                 w[nb][mb][2 * t + 1][1]);
            const int c = (wcol + 32 * nb + 16 * t + 8 * hf) >> 3;
            *reinterpret_cast<u32x4*>(smem + row * kWRow + 16 * (c ^ (row & 15))) = chunk;
          }
      }
    }
    __syncthreads();
    const int c = tid & 15;
#pragma unroll
    for (int i = 0; i < kEpiRows / 16; ++i) {
      const int r = (tid >> 4) + 16 * i, gr = kEpiRows * pass + r;
      if (gr < valid_m && 8 * c < valid_n)
        *reinterpret_cast<u32x4*>(Y + (int64_t)(m0 + gr) * g.ldy + n0 + 8 * c) =
            *reinterpret_cast<const u32x4*>(smem + r * kWRow + 16 * (c ^ (r & 15)));
    }
  }
}
}  // namespace

hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t stream) {
  int max_m = 0;
  for (int i = 0; i < a.groups; ++i) max_m = a.g[i].m > max_m ? a.g[i].m : max_m;
  const int tiles_n = (a.n + kTN - 1) / kTN;
  // the tile height whose workgroup count fills whole rounds of resident
  // workgroups best: the 256-row tile (48 KB of LDS, 164 VGPRs) is resident
  // three per CU, 768 per round, the 128-row tile (32 KB, 95 VGPRs) five per
  // CU, 1280 per round; ties go to the 128-row tile
  const int64_t big = (int64_t)tiles_n * ((max_m + 255) / 256) * a.groups;
  const int64_t small = (int64_t)tiles_n * ((max_m + 127) / 128) * a.groups;
  auto fill = [](int64_t wgs, int64_t round) { return (double)wgs / (double)(((wgs + round - 1) / round) * round); };
  if (small < 256) {
    // fewer 128-row workgroups than CUs: 64-row tiles put twice as many in
    // flight (128 x 512 x 512 x 3: 6.8 against 8.0 us; 1000 x 264 x 200 x 2:
    // 5.5 against 7.1)
    const int tiles_m = (max_m + 63) / 64;
    const dim3 grid((unsigned)(tiles_n * tiles_m * a.groups));
    hipLaunchKernelGGL((linear_bf16_kernel<64>), grid, dim3(256), 0, stream, a, tiles_n, tiles_m);
  } else if (big >= 768 && fill(big, 768) > fill(small, 1280)) {
    const int tiles_m = (max_m + 255) / 256;
    hipLaunchKernelGGL((linear_bf16_kernel<256>), dim3((unsigned)big), dim3(256), 0, stream, a, tiles_n, tiles_m);
  } else if (small <= 512) {
    // at most two workgroups per CU: the 4-stage ring costs no residency
    const int tiles_m = (max_m + 127) / 128;
    const dim3 grid((unsigned)(tiles_n * tiles_m * a.groups));
    hipLaunchKernelGGL((linear_bf16_kernel<128, true>), grid, dim3(256), 0, stream, a, tiles_n, tiles_m);
  } else {
    const int tiles_m = (max_m + 127) / 128;
    const dim3 grid((unsigned)(tiles_n * tiles_m * a.groups));
    hipLaunchKernelGGL((linear_bf16_kernel<128>), grid, dim3(256), 0, stream, a, tiles_n, tiles_m);
  }
  return hipGetLastError();
}
}  // namespace mha
