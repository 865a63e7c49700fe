// Internal launchers between the C-ABI front end and the HIP kernels.
// Arguments arrive here already validated; each launcher only enqueues.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mha {

// One attention problem over all (batch, head) pairs. Strides in elements.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // nullable, (batch, heads, n_q) contiguous
  // nullable, device (batch) int32: keys at or past kv_len[b] are masked for
  // batch item b (clamped to [0, n_k] in the kernels)
  const int* kv_len;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int batch, heads, n_q, n_k, d;
  int causal;
  float scale;
};

// Up to three independent projections Y_g = X_g W_g sharing n and k, done in
// one launch (the grid's z index selects the group).
struct LinearGroup {
  const void* x;
  const void* w;
  void* y;
  int m;
  int64_t ldx, ldw, ldy;
  const void* bias;  // nullable, (n) of the element type: added to every row
};
struct LinearArgs {
  LinearGroup g[3];
  int groups;
  int n, k;
  int relu;  // 1: max(0, .) after the bias
};

// out[r, :] = LayerNorm(x[r, :] + y[r, :]) * gamma + beta over d columns, rows
// contiguous (leading dimension d); statistics in fp32.
struct AddNormArgs {
  const void* x;
  const void* y;
  const void* gamma;
  const void* beta;
  void* out;
  int rows, d;
  float eps;
};

// Attention backward over all (batch, head) pairs: dQ, dK, dV from Q, K, V,
// the forward output O, its gradient dO and the forward's log-sum-exp.
// Strides in elements ({batch, head, row}, last dimension contiguous).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* d_o;
  const float* lse;  // (batch, heads, n_q) contiguous, natural log; -inf: row with no visible key
  void* dq;
  void* dk;
  void* dv;
  float* delta;      // workspace (batch, heads, n_q): rowsum(dO * O), written by the dQ launch
  const int* kv_len;  // nullable, as in AttnArgs
  int64_t q_s[3], k_s[3], v_s[3], o_s[3], do_s[3], dq_s[3], dk_s[3], dv_s[3];
  int batch, heads, n_q, n_k, d;
  int causal;
  float scale;
};

// One decoding step: query (batch, heads, d) against the first kv_len[b] keys
// and values of a cache (see decode.hip for the addressing). Strides in
// elements. Partial softmax states of the key splits go to part_ml / part_o
// and a second launch merges them.
constexpr int kDecodeChunk = 256;  // keys per split
struct DecodeArgs {
  const void* q;  // (batch, heads, d) contiguous
  const void* k;
  const void* v;
  const int* kv_len;       // (batch), clamped to [0, max_len]
  const int* block_table;  // nullable, (batch, max_pages)
  int page_size, max_pages, num_pages, max_len;
  int64_t page_stride, row_stride, head_stride;
  void* o;       // (batch, heads, d) contiguous
  float* lse;    // nullable, (batch, heads)
  float* part_ml;  // (batch * heads, splits, 2): running max (base 2) and sum
  float* part_o;   // (batch * heads, splits, d): unnormalised output
  int batch, heads, d, splits;
  float scale;
};

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t stream);
hipError_t launch_linear_bf16(const LinearArgs& a, hipStream_t stream);
hipError_t launch_linear_f32(const LinearArgs& a, hipStream_t stream);
hipError_t launch_add_layernorm_bf16(const AddNormArgs& a, hipStream_t stream);
hipError_t launch_add_layernorm_f32(const AddNormArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
// Two launches on `stream`: dQ (and delta), then dK and dV.
hipError_t launch_attention_bwd_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_attention_bwd_f32(const BwdArgs& a, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeArgs& a, hipStream_t stream);

}  // namespace mha

// Shared by the sources of the library's entry points (they need the status
// type of the public header).
#include "mha.h"
namespace mha {
mha_status report_error(mha_status s, const char* msg);
// Defined in noalloc.hip: the current device's fixed workspace array of
// mha_forward_noalloc (its device address, looked up once per device) and
// its size.
mha_status noalloc_scratch(void** ptr, size_t* bytes);

}  // namespace mha
