// C-ABI front end of libmha.so: argument validation, workspace layout,
// kernel dispatch, status codes and thread-local error text.
//
// Every check runs before the first HIP runtime call, so a bad argument is
// reported on a machine without a GPU. No C++ exception leaves this file.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "kernels.h"
#include "mha.h"

namespace {

thread_local std::string g_last_error;

mha_status fail(mha_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

mha_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MHA_OK;
  return fail(MHA_ERR_HIP, "%s: %s (hip error %d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Element multiple that keeps every 16-byte vector access aligned.
int vec_elems(mha_dtype t) { return t == MHA_BF16 ? 8 : 4; }
size_t elem_bytes(mha_dtype t) { return t == MHA_BF16 ? 2 : 4; }
bool valid_dtype(int t) { return t == MHA_F32 || t == MHA_BF16; }
bool f32_head_width(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

constexpr size_t kAlign = 256;
constexpr int64_t kMaxLdX = (int64_t)1 << 21;  // elements
constexpr int64_t kMaxLdW = (int64_t)1 << 23;
// Attention tiles are read through buffer descriptors whose record count
// (bytes, 32-bit) spans up to 64 rows of the row stride.
constexpr int64_t kMaxRowStride = (int64_t)1 << 24;  // elements
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace regions of mha_forward: Q, K, V, concatenated heads.
struct WsLayout {
  size_t q, k, v, o, total;
};

bool ws_layout(int batch, int n_q, int n_k, int d_model, mha_dtype t, WsLayout* w) {
  const unsigned __int128 e = elem_bytes(t);
  const unsigned __int128 rq = (unsigned __int128)batch * n_q * d_model * e;
  const unsigned __int128 rk = (unsigned __int128)batch * n_k * d_model * e;
  const unsigned __int128 tot = 2 * (rq + kAlign) + 2 * (rk + kAlign);
  if (tot > ((unsigned __int128)1 << 62)) return false;
  w->q = 0;
  w->k = round_up((size_t)rq);
  w->v = w->k + round_up((size_t)rk);
  w->o = w->v + round_up((size_t)rk);
  w->total = w->o + round_up((size_t)rq);
  return true;
}

mha_status check_head_width(mha_dtype dtype, int d_k, int d_v) {
  if (d_k != d_v) return fail(MHA_ERR_UNSUPPORTED, "d_k (%d) != d_v (%d) is not supported", d_k, d_v);
  if (dtype == MHA_BF16 && d_k != 64)
    return fail(MHA_ERR_UNSUPPORTED, "bf16 attention supports d_k = 64 only (got %d)", d_k);
  if (dtype == MHA_F32 && !f32_head_width(d_k))
    return fail(MHA_ERR_UNSUPPORTED, "f32 attention supports d_k in {16, 32, 64, 128} (got %d)", d_k);
  return MHA_OK;
}

mha_status validate_attention(const void* q, const void* k, const void* v, void* o, int batch,
                              int heads, int n_q, int n_k, int d_k, int d_v, const int64_t* qs,
                              const int64_t* ks, const int64_t* vs, const int64_t* os, int dtype,
                              int causal, float scale) {
  if (!q || !k || !v || !o) return fail(MHA_ERR_INVALID_ARG, "q, k, v and o must be non-null");
  if (!qs || !ks || !vs || !os) return fail(MHA_ERR_INVALID_ARG, "stride arrays must be non-null");
  if (batch < 1 || heads < 1 || n_q < 1 || n_k < 1 || d_k < 1 || d_v < 1)
    return fail(MHA_ERR_INVALID_ARG, "sizes must be >= 1 (batch=%d heads=%d n_q=%d n_k=%d d_k=%d d_v=%d)",
                batch, heads, n_q, n_k, d_k, d_v);
  if (!valid_dtype(dtype)) return fail(MHA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (causal != 0 && causal != 1) return fail(MHA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (causal && n_q != n_k)
    return fail(MHA_ERR_INVALID_ARG, "the causal mask is defined for n_q == n_k (got %d and %d)", n_q, n_k);
  if (!isfinite(scale)) return fail(MHA_ERR_INVALID_ARG, "scale must be finite");
  mha_status s = check_head_width((mha_dtype)dtype, d_k, d_v);
  if (s != MHA_OK) return s;
  const int vec = vec_elems((mha_dtype)dtype);
  const void* ptrs[4] = {q, k, v, o};
  const char* names[4] = {"q", "k", "v", "o"};
  const int64_t* strides[4] = {qs, ks, vs, os};
  for (int t = 0; t < 4; ++t) {
    if (!aligned16(ptrs[t])) return fail(MHA_ERR_INVALID_ARG, "%s must be 16-byte aligned", names[t]);
    for (int i = 0; i < 3; ++i) {
      if (strides[t][i] < 0) return fail(MHA_ERR_INVALID_ARG, "%s stride %d is negative", names[t], i);
      if (strides[t][i] % vec)
        return fail(MHA_ERR_INVALID_ARG, "%s stride %d (%lld) must be a multiple of %d elements", names[t],
                    i, (long long)strides[t][i], vec);
    }
    if (strides[t][2] > kMaxRowStride)
      return fail(MHA_ERR_UNSUPPORTED, "%s row stride (%lld) exceeds %lld elements", names[t],
                  (long long)strides[t][2], (long long)kMaxRowStride);
  }
  // grid: one workgroup per (batch, head, 64- or 128-row query block)
  const int64_t blocks = (int64_t)batch * heads * ((n_q + 63) / 64);
  if (blocks > INT32_MAX) return fail(MHA_ERR_UNSUPPORTED, "too many (batch, head, query block) triples");
  return MHA_OK;
}

mha::AttnArgs attn_args(const void* q, const void* k, const void* v, void* o, float* lse, const int* kv_len,
                        int batch, int heads, int n_q, int n_k, int d, const int64_t* qs, const int64_t* ks,
                        const int64_t* vs, const int64_t* os, int causal, float scale) {
  mha::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.kv_len = kv_len;
  a.q_sb = qs[0], a.q_sh = qs[1], a.q_sn = qs[2];
  a.k_sb = ks[0], a.k_sh = ks[1], a.k_sn = ks[2];
  a.v_sb = vs[0], a.v_sh = vs[1], a.v_sn = vs[2];
  a.o_sb = os[0], a.o_sh = os[1], a.o_sn = os[2];
  a.batch = batch, a.heads = heads, a.n_q = n_q, a.n_k = n_k, a.d = d;
  a.causal = causal;
  a.scale = scale;
  return a;
}

mha_status run_attention(const mha::AttnArgs& a, mha_dtype dtype, hipStream_t stream) {
  hipError_t e = dtype == MHA_BF16 ? mha::launch_attention_bf16(a, stream) : mha::launch_attention_f32(a, stream);
  return hip_status(e, "attention launch");
}

mha_status validate_linear(const void* x, const void* w, void* y, int m, int n, int k, int64_t ldx,
                           int64_t ldw, int64_t ldy, int dtype) {
  if (!x || !w || !y) return fail(MHA_ERR_INVALID_ARG, "x, w and y must be non-null");
  if (m < 1 || n < 1 || k < 1) return fail(MHA_ERR_INVALID_ARG, "sizes must be >= 1 (m=%d n=%d k=%d)", m, n, k);
  if (!valid_dtype(dtype)) return fail(MHA_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (ldx < k || ldw < n || ldy < n)
    return fail(MHA_ERR_INVALID_ARG, "leading dimensions too small (ldx=%lld ldw=%lld ldy=%lld)", (long long)ldx,
                (long long)ldw, (long long)ldy);
  const int vec = vec_elems((mha_dtype)dtype);
  if (k % vec || n % vec || ldx % vec || ldw % vec || ldy % vec)
    return fail(MHA_ERR_INVALID_ARG, "k, n and leading dimensions must be multiples of %d", vec);
  if (!aligned16(x) || !aligned16(w) || !aligned16(y))
    return fail(MHA_ERR_INVALID_ARG, "x, w and y must be 16-byte aligned");
  const int64_t tiles = (int64_t)((m + 63) / 64) * ((n + 63) / 64);
  if (tiles > INT32_MAX) return fail(MHA_ERR_UNSUPPORTED, "problem too large for one launch");
  // the bf16 kernel addresses a 256-row slice of X and a 32-row slice of W
  // with 32-bit byte offsets
  if (ldx > kMaxLdX || ldw > kMaxLdW)
    return fail(MHA_ERR_UNSUPPORTED, "leading dimension too large (ldx=%lld, at most %lld; ldw=%lld, at most %lld)",
                (long long)ldx, (long long)kMaxLdX, (long long)ldw, (long long)kMaxLdW);
  return MHA_OK;
}

mha_status run_linear(const mha::LinearArgs& a, mha_dtype dtype, hipStream_t stream) {
  hipError_t e = dtype == MHA_BF16 ? mha::launch_linear_bf16(a, stream) : mha::launch_linear_f32(a, stream);
  return hip_status(e, "projection launch");
}

mha_status attention_impl(const void* q, const void* k, const void* v, void* o, int batch, int heads, int n_q,
                          int n_k, int d_k, int d_v, const int64_t* q_strides, const int64_t* k_strides,
                          const int64_t* v_strides, const int64_t* o_strides, mha_dtype dtype, int causal, float scale,
                          const int32_t* kv_len, float* lse, void* stream) {
  mha_status s = validate_attention(q, k, v, o, batch, heads, n_q, n_k, d_k, d_v, q_strides, k_strides, v_strides,
                                    o_strides, (int)dtype, causal, scale);
  if (s != MHA_OK) return s;
  if (lse && !aligned16(lse)) return fail(MHA_ERR_INVALID_ARG, "lse must be 16-byte aligned");
  const mha::AttnArgs a = attn_args(q, k, v, o, lse, kv_len, batch, heads, n_q, n_k, d_k, q_strides, k_strides,
                                    v_strides, o_strides, causal, scale);
  return run_attention(a, dtype, static_cast<hipStream_t>(stream));
}

// Projection biases of the attention module (all null for the bias-free
// MultiHead of the pages' equation).
struct MhaBiases {
  const void *q = nullptr, *k = nullptr, *v = nullptr, *o = nullptr;
};

mha_status mha_impl(const void* xq, const void* xk, const void* xv, const void* wq, const void* wk, const void* wv,
                    const void* wo, void* out, void* workspace, size_t workspace_bytes, int batch, int n_q, int n_k,
                    int d_model, int heads, mha_dtype dtype, int causal, const int32_t* kv_len, void* stream,
                    const MhaBiases& bias = MhaBiases()) {
  if (!xq || !xk || !xv || !wq || !wk || !wv || !wo || !out)
    return fail(MHA_ERR_INVALID_ARG, "inputs, weights and out must be non-null");
  if (!workspace) return fail(MHA_ERR_INVALID_ARG, "workspace must be non-null");
  if (batch < 1 || n_q < 1 || n_k < 1 || d_model < 1 || heads < 1)
    return fail(MHA_ERR_INVALID_ARG, "sizes must be >= 1 (batch=%d n_q=%d n_k=%d d_model=%d heads=%d)", batch,
                n_q, n_k, d_model, heads);
  if (!valid_dtype((int)dtype)) return fail(MHA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (d_model % heads)
    return fail(MHA_ERR_INVALID_ARG, "d_model (%d) must be divisible by heads (%d)", d_model, heads);
  if (causal != 0 && causal != 1) return fail(MHA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (causal && n_q != n_k)
    return fail(MHA_ERR_INVALID_ARG, "the causal mask is defined for n_q == n_k (got %d and %d)", n_q, n_k);
  if (d_model > kMaxLdX) return fail(MHA_ERR_UNSUPPORTED, "d_model (%d) too large, at most %lld", d_model, (long long)kMaxLdX);
  const int d = d_model / heads;
  mha_status s = check_head_width(dtype, d, d);
  if (s != MHA_OK) return s;
  const void* ptrs[9] = {xq, xk, xv, wq, wk, wv, wo, out, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return fail(MHA_ERR_INVALID_ARG, "every pointer must be 16-byte aligned");
  WsLayout w;
  if (!ws_layout(batch, n_q, n_k, d_model, dtype, &w))
    return fail(MHA_ERR_UNSUPPORTED, "workspace size overflows");
  if (workspace_bytes < w.total)
    return fail(MHA_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, w.total);
  const int64_t rows_q = (int64_t)batch * n_q, rows_k = (int64_t)batch * n_k;
  if (rows_q > INT32_MAX || rows_k > INT32_MAX) return fail(MHA_ERR_UNSUPPORTED, "batch * sequence too large");
  if ((int64_t)batch * heads * ((n_q + 63) / 64) > INT32_MAX)
    return fail(MHA_ERR_UNSUPPORTED, "too many (batch, head, query block) triples");

  char* ws = static_cast<char*>(workspace);
  void* qw = ws + w.q;
  void* kw = ws + w.k;
  void* vw = ws + w.v;
  void* ow = ws + w.o;
  hipStream_t st = static_cast<hipStream_t>(stream);

  // (1) Q, K, V projections in one grouped launch; row-major (rows, d_model)
  //     is already the head-split (batch, n, heads, d) layout.
  mha::LinearArgs lin = {};
  lin.g[0] = mha::LinearGroup{xq, wq, qw, (int)rows_q, d_model, d_model, d_model, bias.q};
  lin.g[1] = mha::LinearGroup{xk, wk, kw, (int)rows_k, d_model, d_model, d_model, bias.k};
  lin.g[2] = mha::LinearGroup{xv, wv, vw, (int)rows_k, d_model, d_model, d_model, bias.v};
  lin.groups = 3;
  lin.n = d_model;
  lin.k = d_model;
  s = run_linear(lin, dtype, st);
  if (s != MHA_OK) return s;

  // (2) attention over the strided head views; the output lands directly in
  //     the concatenated (batch, n_q, heads * d) layout.
  const int64_t qs[3] = {(int64_t)n_q * d_model, d, d_model};
  const int64_t kvs[3] = {(int64_t)n_k * d_model, d, d_model};
  const mha::AttnArgs a = attn_args(qw, kw, vw, ow, nullptr, kv_len, batch, heads, n_q, n_k, d, qs, kvs, kvs, qs,
                                    causal, 1.0f / sqrtf((float)d));
  s = run_attention(a, dtype, st);
  if (s != MHA_OK) return s;

  // (3) output projection W^O
  mha::LinearArgs out_lin = {};
  out_lin.g[0] = mha::LinearGroup{ow, wo, out, (int)rows_q, d_model, d_model, d_model, bias.o};
  out_lin.groups = 1;
  out_lin.n = d_model;
  out_lin.k = d_model;
  return run_linear(out_lin, dtype, st);
}

constexpr int kMaxNormWidth = 4096;  // the residual + LayerNorm kernel holds a row in one wavefront

bool enc_ws_layout(int batch, int n, int d_model, int d_ff, mha_dtype t, WsLayout* w, size_t* ffh, size_t* total) {
  if (!ws_layout(batch, n, n, d_model, t, w)) return false;
  const unsigned __int128 rf = (unsigned __int128)batch * n * d_ff * elem_bytes(t);
  if (rf > ((unsigned __int128)1 << 60)) return false;
  *ffh = w->total;
  *total = w->total + round_up((size_t)rf);
  return true;
}

mha_status run_add_norm(const mha::AddNormArgs& a, mha_dtype dtype, hipStream_t stream) {
  hipError_t e = dtype == MHA_BF16 ? mha::launch_add_layernorm_bf16(a, stream) : mha::launch_add_layernorm_f32(a, stream);
  return hip_status(e, "layer norm launch");
}

mha_status encoder_layer_impl(const void* x, const mha_encoder_weights* wts, void* out, void* workspace,
                              size_t workspace_bytes, int batch, int n, int d_model, int heads, int d_ff, float eps,
                              mha_dtype dtype, int causal, const int32_t* kv_len, void* stream) {
  if (!x || !out || !wts) return fail(MHA_ERR_INVALID_ARG, "x, weights and out must be non-null");
  const void* ptrs[16] = {wts->wq, wts->wk, wts->wv, wts->wo, wts->bq, wts->bk, wts->bv, wts->bo,
                          wts->ln1_gamma, wts->ln1_beta, wts->w1, wts->b1, wts->w2, wts->b2, wts->ln2_gamma,
                          wts->ln2_beta};
  for (const void* p : ptrs) {
    if (!p) return fail(MHA_ERR_INVALID_ARG, "every weight, bias and norm parameter must be non-null");
    if (!aligned16(p)) return fail(MHA_ERR_INVALID_ARG, "every weight, bias and norm parameter must be 16-byte aligned");
  }
  if (!valid_dtype((int)dtype)) return fail(MHA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (batch < 1 || n < 1 || d_model < 1 || heads < 1 || d_ff < 1)
    return fail(MHA_ERR_INVALID_ARG, "sizes must be >= 1 (batch=%d n=%d d_model=%d heads=%d d_ff=%d)", batch, n,
                d_model, heads, d_ff);
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(MHA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const int vec = vec_elems(dtype);
  if (d_model % vec || d_ff % vec)
    return fail(MHA_ERR_INVALID_ARG, "d_model and d_ff must be multiples of %d", vec);
  if (d_model > kMaxNormWidth)
    return fail(MHA_ERR_UNSUPPORTED, "d_model (%d) above %d: one row must fit the LayerNorm wavefront", d_model,
                kMaxNormWidth);
  if (d_ff > kMaxLdX) return fail(MHA_ERR_UNSUPPORTED, "d_ff (%d) too large, at most %lld", d_ff, (long long)kMaxLdX);
  WsLayout w;
  size_t ffh_off = 0, total = 0;
  if (!enc_ws_layout(batch, n, d_model, d_ff, dtype, &w, &ffh_off, &total))
    return fail(MHA_ERR_UNSUPPORTED, "workspace size overflows");
  if (workspace && workspace_bytes < total)
    return fail(MHA_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, total);
  if ((int64_t)batch * n > INT32_MAX) return fail(MHA_ERR_UNSUPPORTED, "batch * sequence too large");
  const int rows = batch * n;
  char* ws = static_cast<char*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);

  // (1) attention sub-layer with biases; its output t1 lands in the Q region
  //     (Q is dead once the attention launch has read it)
  void* t1 = ws ? ws + w.q : nullptr;
  MhaBiases b;
  b.q = wts->bq, b.k = wts->bk, b.v = wts->bv, b.o = wts->bo;
  mha_status s = mha_impl(x, x, x, wts->wq, wts->wk, wts->wv, wts->wo, t1, workspace, workspace_bytes, batch, n, n,
                          d_model, heads, dtype, causal, kv_len, stream, b);
  if (s != MHA_OK) return s;
  // the attention launch reads Q before W^O writes t1 into its region: same stream, in order

  // (2) h = LayerNorm(x + t1), into the K region
  void* h = ws + w.k;
  s = run_add_norm(mha::AddNormArgs{x, t1, wts->ln1_gamma, wts->ln1_beta, h, rows, d_model, eps}, dtype, st);
  if (s != MHA_OK) return s;

  // (3) FFN: hidden = max(0, h W1 + b1), then t2 = hidden W2 + b2 into the V region
  void* hid = ws + ffh_off;
  mha::LinearArgs l1 = {};
  l1.g[0] = mha::LinearGroup{h, wts->w1, hid, rows, d_model, d_ff, d_ff, wts->b1};
  l1.groups = 1, l1.n = d_ff, l1.k = d_model, l1.relu = 1;
  s = run_linear(l1, dtype, st);
  if (s != MHA_OK) return s;
  void* t2 = ws + w.v;
  mha::LinearArgs l2 = {};
  l2.g[0] = mha::LinearGroup{hid, wts->w2, t2, rows, d_ff, d_model, d_model, wts->b2};
  l2.groups = 1, l2.n = d_model, l2.k = d_ff;
  s = run_linear(l2, dtype, st);
  if (s != MHA_OK) return s;

  // (4) out = LayerNorm(h + t2)
  return run_add_norm(mha::AddNormArgs{h, t2, wts->ln2_gamma, wts->ln2_beta, out, rows, d_model, eps}, dtype, st);
}

// Decode workspace: per (batch, head, split) the running max and sum, then
// the unnormalised output row, both fp32.
struct DecodeWs {
  size_t ml, o, total;
};

bool decode_ws_layout(int batch, int heads, int d, int max_len, DecodeWs* w) {
  const int64_t splits = ((int64_t)max_len + mha::kDecodeChunk - 1) / mha::kDecodeChunk;
  const unsigned __int128 parts = (unsigned __int128)batch * heads * splits;
  const unsigned __int128 tot = parts * (2 + d) * 4 + 2 * kAlign;
  if (tot > ((unsigned __int128)1 << 62)) return false;
  w->ml = 0;
  w->o = round_up((size_t)(parts * 2 * 4));
  w->total = w->o + round_up((size_t)(parts * d * 4));
  return true;
}

mha_status decode_impl(const void* q, const mha_kv_cache* cache, const int32_t* kv_len, void* o, float* lse,
                       void* workspace, size_t workspace_bytes, int batch, int heads, int d, mha_dtype dtype,
                       float scale, void* stream) {
  if (!q || !cache || !kv_len || !o || !workspace)
    return fail(MHA_ERR_INVALID_ARG, "q, cache, kv_len, o and workspace must be non-null");
  if (!cache->k || !cache->v) return fail(MHA_ERR_INVALID_ARG, "cache->k and cache->v must be non-null");
  if (batch < 1 || heads < 1 || d < 1 || cache->max_len < 1)
    return fail(MHA_ERR_INVALID_ARG, "sizes must be >= 1 (batch=%d heads=%d d=%d max_len=%d)", batch, heads, d,
                cache->max_len);
  if (!valid_dtype(dtype)) return fail(MHA_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (!isfinite(scale)) return fail(MHA_ERR_INVALID_ARG, "scale must be finite");
  if (!f32_head_width(d))
    return fail(MHA_ERR_UNSUPPORTED, "decode supports d in {16, 32, 64, 128} (got %d)", d);
  const int vec = vec_elems(dtype);
  const int64_t strides[3] = {cache->page_stride, cache->row_stride, cache->head_stride};
  const char* names[3] = {"page_stride", "row_stride", "head_stride"};
  for (int i = 0; i < 3; ++i) {
    if (strides[i] < 0) return fail(MHA_ERR_INVALID_ARG, "cache %s is negative", names[i]);
    if (strides[i] % vec)
      return fail(MHA_ERR_INVALID_ARG, "cache %s (%lld) must be a multiple of %d elements", names[i],
                  (long long)strides[i], vec);
  }
  if (!aligned16(q) || !aligned16(cache->k) || !aligned16(cache->v) || !aligned16(o) || !aligned16(workspace))
    return fail(MHA_ERR_INVALID_ARG, "q, cache->k, cache->v, o and workspace must be 16-byte aligned");
  if (!aligned4(kv_len) || (lse && !aligned4(lse)))
    return fail(MHA_ERR_INVALID_ARG, "kv_len and lse must be 4-byte aligned");
  if (cache->block_table) {
    if (!aligned4(cache->block_table)) return fail(MHA_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
    if (cache->page_size < 1 || cache->max_pages < 1 || cache->num_pages < 1)
      return fail(MHA_ERR_INVALID_ARG, "page_size, max_pages and num_pages must be >= 1 with a block table");
    if ((int64_t)cache->page_size * cache->max_pages < cache->max_len)
      return fail(MHA_ERR_INVALID_ARG, "max_len (%d) exceeds page_size * max_pages (%lld)", cache->max_len,
                  (long long)cache->page_size * cache->max_pages);
  }
  const int64_t bhs = (int64_t)batch * heads;
  const int64_t splits = ((int64_t)cache->max_len + mha::kDecodeChunk - 1) / mha::kDecodeChunk;
  if (bhs > INT32_MAX || splits > 65535)
    return fail(MHA_ERR_UNSUPPORTED, "too many (batch, head) pairs or max_len too large for one launch");
  DecodeWs ws;
  if (!decode_ws_layout(batch, heads, d, cache->max_len, &ws)) return fail(MHA_ERR_INVALID_ARG, "sizes overflow");
  if (workspace_bytes < ws.total)
    return fail(MHA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, ws.total);

  mha::DecodeArgs a = {};
  a.q = q;
  a.k = cache->k;
  a.v = cache->v;
  a.kv_len = kv_len;
  a.block_table = cache->block_table;
  a.page_size = cache->page_size;
  a.max_pages = cache->max_pages;
  a.num_pages = cache->num_pages;
  a.max_len = cache->max_len;
  a.page_stride = cache->page_stride;
  a.row_stride = cache->row_stride;
  a.head_stride = cache->head_stride;
  a.o = o;
  a.lse = lse;
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.ml);
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.o);
  a.batch = batch;
  a.heads = heads;
  a.d = d;
  a.splits = (int)splits;
  a.scale = scale;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = dtype == MHA_BF16 ? mha::launch_decode_bf16(a, st) : mha::launch_decode_f32(a, st);
  return hip_status(e, "decode launch");
}

mha_status backward_impl(const void* q, const void* k, const void* v, const void* o, const void* d_o, const float* lse,
                         void* dq, void* dk, void* dv, int batch, int heads, int n_q, int n_k, int d,
                         const int64_t* q_strides, const int64_t* k_strides, const int64_t* v_strides,
                         const int64_t* o_strides, const int64_t* do_strides, const int64_t* dq_strides,
                         const int64_t* dk_strides, const int64_t* dv_strides, mha_dtype dtype, int causal,
                         float scale, const int32_t* kv_len, void* workspace, size_t workspace_bytes, void* stream) {
  // the forward's rules cover q, k, v and o; then the gradient tensors
  mha_status s = validate_attention(q, k, v, const_cast<void*>(o), batch, heads, n_q, n_k, d, d, q_strides, k_strides,
                                    v_strides, o_strides, (int)dtype, causal, scale);
  if (s != MHA_OK) return s;
  if (!d_o || !dq || !dk || !dv || !lse || !workspace)
    return fail(MHA_ERR_INVALID_ARG, "d_o, dq, dk, dv, lse and workspace must be non-null");
  if (!do_strides || !dq_strides || !dk_strides || !dv_strides)
    return fail(MHA_ERR_INVALID_ARG, "stride arrays must be non-null");
  const int vec = vec_elems(dtype);
  const void* ptrs[4] = {d_o, dq, dk, dv};
  const char* names[4] = {"d_o", "dq", "dk", "dv"};
  const int64_t* strides[4] = {do_strides, dq_strides, dk_strides, dv_strides};
  for (int t = 0; t < 4; ++t) {
    if (!aligned16(ptrs[t])) return fail(MHA_ERR_INVALID_ARG, "%s must be 16-byte aligned", names[t]);
    for (int i = 0; i < 3; ++i) {
      if (strides[t][i] < 0) return fail(MHA_ERR_INVALID_ARG, "%s stride %d is negative", names[t], i);
      if (strides[t][i] % vec)
        return fail(MHA_ERR_INVALID_ARG, "%s stride %d (%lld) must be a multiple of %d elements", names[t], i,
                    (long long)strides[t][i], vec);
    }
    if (strides[t][2] > kMaxRowStride)
      return fail(MHA_ERR_UNSUPPORTED, "%s row stride (%lld) exceeds %lld elements", names[t],
                  (long long)strides[t][2], (long long)kMaxRowStride);
  }
  if (!aligned16(lse) || !aligned16(workspace)) return fail(MHA_ERR_INVALID_ARG, "lse and workspace must be 16-byte aligned");
  if (kv_len && !aligned4(kv_len)) return fail(MHA_ERR_INVALID_ARG, "kv_len must be 4-byte aligned");
  // two fp32 rows per query: -delta and lse log2(e) (the fp32 path uses the first for delta)
  const size_t need = round_up((size_t)batch * heads * n_q * 8);
  if (workspace_bytes < need)
    return fail(MHA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  const int64_t kblocks = (int64_t)batch * heads * ((n_k + 63) / 64);
  if (kblocks > INT32_MAX) return fail(MHA_ERR_UNSUPPORTED, "too many (batch, head, key block) triples");

  mha::BwdArgs a = {};
  a.q = q, a.k = k, a.v = v, a.o = o, a.d_o = d_o, a.lse = lse;
  a.dq = dq, a.dk = dk, a.dv = dv;
  a.delta = static_cast<float*>(workspace);
  a.kv_len = kv_len;
  for (int i = 0; i < 3; ++i) {
    a.q_s[i] = q_strides[i], a.k_s[i] = k_strides[i], a.v_s[i] = v_strides[i], a.o_s[i] = o_strides[i];
    a.do_s[i] = do_strides[i], a.dq_s[i] = dq_strides[i], a.dk_s[i] = dk_strides[i], a.dv_s[i] = dv_strides[i];
  }
  a.batch = batch, a.heads = heads, a.n_q = n_q, a.n_k = n_k, a.d = d;
  a.causal = causal;
  a.scale = scale;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = dtype == MHA_BF16 ? mha::launch_attention_bwd_bf16(a, st) : mha::launch_attention_bwd_f32(a, st);
  return hip_status(e, "attention backward launch");
}

}  // namespace

namespace mha {
// The thread-local error text, for sources other than this one.
mha_status report_error(mha_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace mha

extern "C" {

const char* mha_status_string(mha_status s) {
  switch (s) {
    case MHA_OK: return "MHA_OK";
    case MHA_ERR_INVALID_ARG: return "MHA_ERR_INVALID_ARG";
    case MHA_ERR_UNSUPPORTED: return "MHA_ERR_UNSUPPORTED";
    case MHA_ERR_WORKSPACE: return "MHA_ERR_WORKSPACE";
    case MHA_ERR_HIP: return "MHA_ERR_HIP";
  }
  return "MHA_ERR_UNKNOWN";
}

const char* mha_last_error(void) { return g_last_error.c_str(); }

int mha_version(void) { return 401; }

mha_status attention_forward(const void* q, const void* k, const void* v, void* o, int batch, int heads,
                             int n_q, int n_k, int d_k, int d_v, const int64_t q_strides[3],
                             const int64_t k_strides[3], const int64_t v_strides[3],
                             const int64_t o_strides[3], mha_dtype dtype, int causal, float scale, float* lse,
                             void* stream) {
  try {
    return attention_impl(q, k, v, o, batch, heads, n_q, n_k, d_k, d_v, q_strides, k_strides, v_strides, o_strides,
                          dtype, causal, scale, nullptr, lse, stream);
  } catch (...) {
    return fail(MHA_ERR_HIP, "internal error in attention_forward");
  }
}

mha_status attention_forward_padded(const void* q, const void* k, const void* v, void* o, int batch, int heads,
                                    int n_q, int n_k, int d_k, int d_v, const int64_t q_strides[3],
                                    const int64_t k_strides[3], const int64_t v_strides[3],
                                    const int64_t o_strides[3], mha_dtype dtype, int causal, float scale,
                                    const int32_t* kv_len, float* lse, void* stream) {
  try {
    if (!kv_len) return fail(MHA_ERR_INVALID_ARG, "kv_len must be non-null (use attention_forward for no padding)");
    if (!aligned4(kv_len)) return fail(MHA_ERR_INVALID_ARG, "kv_len must be 4-byte aligned");
    return attention_impl(q, k, v, o, batch, heads, n_q, n_k, d_k, d_v, q_strides, k_strides, v_strides, o_strides,
                          dtype, causal, scale, kv_len, lse, stream);
  } catch (...) {
    return fail(MHA_ERR_HIP, "internal error in attention_forward_padded");
  }
}

mha_status linear_forward(const void* x, const void* w, void* y, int m, int n, int k, int64_t ldx, int64_t ldw,
                          int64_t ldy, mha_dtype dtype, void* stream) {
  try {
    mha_status s = validate_linear(x, w, y, m, n, k, ldx, ldw, ldy, (int)dtype);
    if (s != MHA_OK) return s;
    mha::LinearArgs a = {};
    a.g[0] = mha::LinearGroup{x, w, y, m, ldx, ldw, ldy};
    a.groups = 1;
    a.n = n;
    a.k = k;
    return run_linear(a, dtype, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(MHA_ERR_HIP, "internal error in linear_forward");
  }
}

mha_status linear_forward_grouped(const void* const* x, const void* const* w, void* const* y, const int* m,
                                  int groups, int n, int k, const int64_t* ldx, const int64_t* ldw,
                                  const int64_t* ldy, mha_dtype dtype, void* stream) {
  try {
    if (!x || !w || !y || !m || !ldx || !ldw || !ldy)
      return fail(MHA_ERR_INVALID_ARG, "x, w, y, m, ldx, ldw and ldy must be non-null arrays");
    if (groups < 1 || groups > 3) return fail(MHA_ERR_INVALID_ARG, "groups must be 1, 2 or 3 (got %d)", groups);
    mha::LinearArgs a = {};
    int max_m = 0;
    for (int g = 0; g < groups; ++g) {
      mha_status s = validate_linear(x[g], w[g], y[g], m[g], n, k, ldx[g], ldw[g], ldy[g], (int)dtype);
      if (s != MHA_OK) return s;
      a.g[g] = mha::LinearGroup{x[g], w[g], y[g], m[g], ldx[g], ldw[g], ldy[g]};
      max_m = m[g] > max_m ? m[g] : max_m;
    }
    const int64_t tiles = (int64_t)groups * ((max_m + 63) / 64) * ((n + 63) / 64);
    if (tiles > INT32_MAX) return fail(MHA_ERR_UNSUPPORTED, "problem too large for one launch");
    a.groups = groups;
    a.n = n;
    a.k = k;
    return run_linear(a, dtype, static_cast<hipStream_t>(stream));
  } catch (...) {
    return fail(MHA_ERR_HIP, "internal error in linear_forward_grouped");
  }
}

size_t mha_forward_workspace_size(int batch, int n_q, int n_k, int d_model, int heads, mha_dtype dtype) {
  if (batch < 1 || n_q < 1 || n_k < 1 || d_model < 1 || heads < 1 || !valid_dtype((int)dtype)) return 0;
  WsLayout w;
  if (!ws_layout(batch, n_q, n_k, d_model, dtype, &w)) return 0;
  return w.total;
}

mha_status mha_forward(const void* xq, const void* xk, const void* xv, const void* wq, const void* wk,
                       const void* wv, const void* wo, void* out, void* workspace, size_t workspace_bytes,
                       int batch, int n_q, int n_k, int d_model, int heads, mha_dtype dtype, int causal,
                       void* stream) {
  try {
    return mha_impl(xq, xk, xv, wq, wk, wv, wo, out, workspace, workspace_bytes, batch, n_q, n_k, d_model, heads,
                    dtype, causal, nullptr, stream);
  } catch (...) {
    return fail(MHA_ERR_HIP, "internal error in mha_forward");
  }
}

mha_status mha_forward_noalloc(const void* xq, const void* xk, const void* xv, const void* wq, const void* wk,
                               const void* wv, const void* wo, void* out, int batch, int n_q, int n_k, int d_model,
                               int heads, mha_dtype dtype, int causal, void* stream) {
  try {
    // size checks first, before any HIP call
    const size_t need = mha_forward_workspace_size(batch, n_q, n_k, d_model, heads, dtype);
    if (need == 0) return fail(MHA_ERR_INVALID_ARG, "invalid sizes or dtype (the workspace size is undefined)");
    if (need > MHA_NOALLOC_MAX_WORKSPACE)
      return fail(MHA_ERR_UNSUPPORTED,
                  "problem needs a %zu-byte workspace, more than mha_forward_noalloc's fixed 128 MiB; call "
                  "mha_forward with a workspace instead",
                  need);
    // the rest of mha_forward's validation runs before its first launch; only
    // the lookup of this device's array precedes it, so reject bad pointers first
    if (!xq || !xk || !xv || !wq || !wk || !wv || !wo || !out)
      return fail(MHA_ERR_INVALID_ARG, "inputs, weights and out must be non-null");
    void* ws = nullptr;
    size_t ws_bytes = 0;
    const mha_status s = mha::noalloc_scratch(&ws, &ws_bytes);
    if (s != MHA_OK) return s;
    return mha_impl(xq, xk, xv, wq, wk, wv, wo, out, ws, ws_bytes, batch, n_q, n_k, d_model, heads, dtype, causal,
                    nullptr, stream);
  } catch (...) {
    return fail(MHA_ERR_HIP, "internal error in mha_forward_noalloc");
  }
}

mha_status mha_forward_padded(const void* xq, const void* xk, const void* xv, const void* wq, const void* wk,
                              const void* wv, const void* wo, void* out, void* workspace, size_t workspace_bytes,
                              int batch, int n_q, int n_k, int d_model, int heads, mha_dtype dtype, int causal,
                              const int32_t* kv_len, void* stream) {
  try {
    if (!kv_len) return fail(MHA_ERR_INVALID_ARG, "kv_len must be non-null (use mha_forward for no padding)");
    if (!aligned4(kv_len)) return fail(MHA_ERR_INVALID_ARG, "kv_len must be 4-byte aligned");
    return mha_impl(xq, xk, xv, wq, wk, wv, wo, out, workspace, workspace_bytes, batch, n_q, n_k, d_model, heads,
                    dtype, causal, kv_len, stream);
  } catch (...) {
    return fail(MHA_ERR_HIP, "internal error in mha_forward_padded");
  }
}

size_t encoder_layer_workspace_size(int batch, int n, int d_model, int heads, int d_ff, mha_dtype dtype) {
  if (batch < 1 || n < 1 || d_model < 1 || heads < 1 || d_ff < 1 || !valid_dtype((int)dtype)) return 0;
  WsLayout w;
  size_t ffh = 0, total = 0;
  if (!enc_ws_layout(batch, n, d_model, d_ff, dtype, &w, &ffh, &total)) return 0;
  return total;
}

mha_status encoder_layer_forward(const void* x, const mha_encoder_weights* weights, void* out, void* workspace,
                                 size_t workspace_bytes, int batch, int n, int d_model, int heads, int d_ff, float eps,
                                 mha_dtype dtype, int causal, const int32_t* kv_len, void* stream) {
  try {
    if (kv_len && !aligned4(kv_len)) return fail(MHA_ERR_INVALID_ARG, "kv_len must be 4-byte aligned");
    if (!workspace) return fail(MHA_ERR_INVALID_ARG, "workspace must be non-null");
    return encoder_layer_impl(x, weights, out, workspace, workspace_bytes, batch, n, d_model, heads, d_ff, eps, dtype,
                              causal, kv_len, stream);
  } catch (...) {
    return fail(MHA_ERR_HIP, "internal error in encoder_layer_forward");
  }
}

size_t attention_decode_workspace_size(int batch, int heads, int d, int max_len) {
  if (batch < 1 || heads < 1 || d < 1 || max_len < 1) return 0;
  DecodeWs ws;
  if (!decode_ws_layout(batch, heads, d, max_len, &ws)) return 0;
  return ws.total;
}

mha_status attention_decode(const void* q, const mha_kv_cache* cache, const int32_t* kv_len, void* o, float* lse,
                            void* workspace, size_t workspace_bytes, int batch, int heads, int d, mha_dtype dtype,
                            float scale, void* stream) {
  try {
    return decode_impl(q, cache, kv_len, o, lse, workspace, workspace_bytes, batch, heads, d, dtype, scale, stream);
  } catch (...) {
    return fail(MHA_ERR_HIP, "internal error in attention_decode");
  }
}

size_t attention_backward_workspace_size(int batch, int heads, int n_q) {
  if (batch < 1 || heads < 1 || n_q < 1) return 0;
  const unsigned __int128 bytes = (unsigned __int128)batch * heads * n_q * 8;
  if (bytes > ((unsigned __int128)1 << 62)) return 0;
  return round_up((size_t)bytes);
}

mha_status attention_backward(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                              const float* lse, void* dq, void* dk, void* dv, int batch, int heads, int n_q, int n_k,
                              int d, const int64_t q_strides[3], const int64_t k_strides[3],
                              const int64_t v_strides[3], const int64_t o_strides[3], const int64_t do_strides[3],
                              const int64_t dq_strides[3], const int64_t dk_strides[3], const int64_t dv_strides[3],
                              mha_dtype dtype, int causal, float scale, const int32_t* kv_len, void* workspace,
                              size_t workspace_bytes, void* stream) {
  try {
    return backward_impl(q, k, v, o, d_o, lse, dq, dk, dv, batch, heads, n_q, n_k, d, q_strides, k_strides, v_strides,
                         o_strides, do_strides, dq_strides, dk_strides, dv_strides, dtype, causal, scale, kv_len,
                         workspace, workspace_bytes, stream);
  } catch (...) {
    return fail(MHA_ERR_HIP, "internal error in attention_backward");
  }
}

}  // extern "C"
