/*
 * mha.h -- C ABI of libmha.so: multi-head scaled dot-product attention,
 * forward pass, on AMD Instinct MI355X (gfx950).
 *
 * What is computed (the pages' statement of the problem):
 *   Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V, softmax over each row
 *     -- "The Transformer" (hoshank.vercel.app), "The Mathematics", Attention
 *     equation; "How Transformers Work" (worksonmygpu.com), "Scaled
 *     dot-product attention".
 *   MultiHead(Q, K, V) = Concat(head_1 .. head_h) W^O,
 *   head_i = Attention(Q W_i^Q, K W_i^K, V W_i^V)
 *     -- same page, MultiHead equation; "32 Transformer"
 *     (ml-canon-en.vercel.app), "PyTorch Implementation".
 *   Causal mask: key j is blocked for query i when j > i (diagonal kept), by
 *     adding -inf to the score before the softmax, so blocked keys weigh
 *     exactly 0 -- "The Transformer" (rayaq.ca), "Masks: who may look at whom".
 *   Key-padding mask: keys at or past a batch item's length are blocked for
 *     every query of that item the same way -- same section (padding masks,
 *     one row per batch item). Given as a number of valid keys per item, so
 *     there is no boolean polarity to get wrong.
 *
 * Conventions shared by every entry point
 *   - Every data pointer is DEVICE memory owned by the caller. The library
 *     never allocates, frees or retains device memory and keeps no state
 *     between calls.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream). MHA_OK means "validated and enqueued"; faults during execution
 *     surface at the caller's next synchronisation.
 *   - All argument validation happens before any HIP runtime call, so invalid
 *     arguments are reported without touching a device.
 *   - No C++ exception crosses this boundary. On a non-OK status,
 *     mha_last_error() returns a thread-local description.
 *   - Element types: MHA_F32 = IEEE binary32; MHA_BF16 = bfloat16. In bf16
 *     mode products accumulate in fp32, the softmax runs in fp32, the
 *     attention weights are rounded to bf16 (nearest-even) for the P V
 *     product, and every stored tensor (outputs and mha_forward's
 *     intermediates) is rounded to bf16 (nearest-even).
 *   - Output buffers must not overlap any input buffer.
 */
#ifndef MHA_H
#define MHA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mha_status {
  MHA_OK = 0,
  MHA_ERR_INVALID_ARG = 1, /* null pointer, size < 1, bad stride/alignment, causal with n_q != n_k, ... */
  MHA_ERR_UNSUPPORTED = 2, /* valid request outside what this build implements (e.g. d_k != 64 in bf16) */
  MHA_ERR_WORKSPACE = 3,   /* workspace smaller than mha_forward_workspace_size() */
  MHA_ERR_HIP = 4          /* the HIP runtime rejected a launch */
} mha_status;

typedef enum mha_dtype { MHA_F32 = 0, MHA_BF16 = 1 } mha_dtype;

/*
 * attention_forward -- scaled dot-product attention for every (batch, head).
 *
 *   O[b,h,i,:] = sum_j P[b,h,i,j] V[b,h,j,:],
 *   P[b,h,i,:] = softmax_j( scale * Q[b,h,i,:] . K[b,h,j,:]  (+ causal mask) )
 *
 * q: (batch, heads, n_q, d_k)   k: (batch, heads, n_k, d_k)
 * v: (batch, heads, n_k, d_v)   o: (batch, heads, n_q, d_v)   all of `dtype`
 *   Each tensor is addressed through its own element strides
 *   {batch, head, row}; the last dimension is contiguous (stride 1). So the
 *   head split and concat of multi-head attention are pure stride choices:
 *   a (batch, n, heads*d) buffer is passed with strides {n*heads*d, d, heads*d}.
 * causal: 0 = no mask (encoder self-attention, cross-attention);
 *   1 = key j blocked for query i when j > i (requires n_q == n_k).
 * scale: multiplies the scores before the softmax; 1/sqrt(d_k) gives the
 *   pages' attention, other values act as an inverse temperature ("The
 *   Transformer" (rayaq.ca), "Worked example"). Must be finite; 0 gives
 *   uniform weights over the visible keys.
 * lse: NULL, or fp32 (batch, heads, n_q) contiguous: on return
 *   lse[b,h,i] = log sum_j exp(scale * q_i . k_j) over the visible keys.
 *
 * Supported in this build: d_k == d_v; bf16 needs d_k == 64 (both page model
 *   sizes use 64); f32 accepts d_k in {16, 32, 64, 128}. Otherwise
 *   MHA_ERR_UNSUPPORTED.
 * Alignment: base pointers 16-byte aligned; every stride a multiple of
 *   8 elements (bf16) or 4 elements (f32). Otherwise MHA_ERR_INVALID_ARG.
 *   Row strides above 2^24 elements are MHA_ERR_UNSUPPORTED.
 */
mha_status attention_forward(const void* q, const void* k, const void* v, void* o,
                             int batch, int heads, int n_q, int n_k, int d_k, int d_v,
                             const int64_t q_strides[3], const int64_t k_strides[3],
                             const int64_t v_strides[3], const int64_t o_strides[3],
                             mha_dtype dtype, int causal, float scale, float* lse,
                             void* stream);

/*
 * attention_forward_padded -- attention_forward with a key-padding mask.
 *
 * kv_len: DEVICE pointer to `batch` int32 values, 4-byte aligned, owned by the
 *   caller and read by the kernels (not on the host). Key j is blocked for
 *   every query and head of batch item b when j >= kv_len[b]; values are
 *   clamped to [0, n_k]. Combined with causal = 1, query i sees keys
 *   j <= min(i, kv_len[b] - 1).
 * A row with no visible key (kv_len[b] == 0) has no softmax: its output is 0
 *   and its lse is -inf (the pages leave such rows undefined).
 * Every other argument, rule and status is that of attention_forward; a NULL
 *   kv_len is MHA_ERR_INVALID_ARG (call attention_forward instead).
 * Work and traffic shrink with the lengths: key tiles past kv_len[b] are
 *   never loaded.
 */
mha_status attention_forward_padded(const void* q, const void* k, const void* v, void* o,
                                    int batch, int heads, int n_q, int n_k, int d_k, int d_v,
                                    const int64_t q_strides[3], const int64_t k_strides[3],
                                    const int64_t v_strides[3], const int64_t o_strides[3],
                                    mha_dtype dtype, int causal, float scale, const int32_t* kv_len,
                                    float* lse, void* stream);

/*
 * linear_forward -- one projection, Y = X W (no bias), the building block of
 * the Q/K/V projections and of W^O ("The Transformer" (hoshank.vercel.app),
 * "The Mathematics": W_i^Q etc. are d_model x d_k matrices applied on the
 * right; "32 Transformer", "PyTorch Implementation": Q = x @ Wq).
 *
 * x: (m, k) row-major with leading dimension ldx; w: (k, n) row-major (in, out)
 * with leading dimension ldw; y: (m, n) row-major with leading dimension ldy.
 * fp32 accumulation; y rounded to `dtype`.
 * Alignment: base pointers 16-byte aligned; k, n and the leading dimensions
 *   multiples of 8 (bf16) or 4 (f32); otherwise MHA_ERR_INVALID_ARG.
 */
mha_status linear_forward(const void* x, const void* w, void* y, int m, int n, int k,
                          int64_t ldx, int64_t ldw, int64_t ldy, mha_dtype dtype, void* stream);

/*
 * linear_forward_grouped -- up to three independent projections Y_g = X_g W_g
 * that share n and k, in ONE launch: the launch mha_forward makes for the
 * Q, K and V projections ("The Transformer" (hoshank.vercel.app), "The
 * Mathematics", MultiHead equation: one d_model x d_k block per head of each
 * of W^Q, W^K, W^V, applied on the right).
 *
 * x, w, y, m, ldx, ldw, ldy: host arrays of `groups` entries (1 <= groups <= 3);
 *   entry g describes problem g exactly as linear_forward's arguments do
 *   (x[g] (m[g], k), w[g] (k, n), y[g] (m[g], n), row-major, device pointers
 *   owned by the caller). The host arrays are read during the call only.
 * Every rule and status of linear_forward applies to each problem; a groups
 *   value outside [1, 3] or a NULL array is MHA_ERR_INVALID_ARG.
 */
mha_status linear_forward_grouped(const void* const* x, const void* const* w, void* const* y,
                                  const int* m, int groups, int n, int k, const int64_t* ldx,
                                  const int64_t* ldw, const int64_t* ldy, mha_dtype dtype,
                                  void* stream);

/*
 * mha_forward_workspace_size -- bytes of device workspace mha_forward needs:
 * room for the projected Q (batch*n_q x d_model), K and V (batch*n_k x
 * d_model each) and the concatenated head outputs (batch*n_q x d_model), in
 * `dtype`, each region 256-byte aligned. Returns 0 for invalid sizes.
 */
size_t mha_forward_workspace_size(int batch, int n_q, int n_k, int d_model, int heads,
                                  mha_dtype dtype);

/*
 * mha_forward -- multi-head attention, bias-free:
 *   out = Concat_i( Attention(Xq W^Q_i, Xk W^K_i, Xv W^V_i) ) W^O,
 *   scale 1/sqrt(d_model / heads); head i owns columns [i*d, (i+1)*d) of each
 *   projection and rows [i*d, (i+1)*d) of W^O.
 *
 * xq: (batch, n_q, d_model); xk, xv: (batch, n_k, d_model), all contiguous.
 *   Self-attention passes the same pointer three times; encoder-decoder
 *   cross-attention passes the decoder state as xq and the encoder memory as
 *   xk and xv ("The Transformer" (rayaq.ca), "The decoder stack").
 * wq, wk, wv, wo: (d_model, d_model) row-major, stored (in, out) so Q = X W^Q.
 * out: (batch, n_q, d_model).
 * workspace: device memory of at least mha_forward_workspace_size() bytes,
 *   16-byte aligned, owned by the caller; its contents are scratch (the
 *   projected Q, K, V and the concatenated heads are left there on return).
 * causal: as in attention_forward (requires n_q == n_k).
 * d_model % heads must be 0 (MHA_ERR_INVALID_ARG otherwise); the head width
 *   d_model/heads follows attention_forward's support rules.
 * Launches: one grouped projection for Q, K and V, one attention, one W^O
 *   projection, all on `stream`.
 */
mha_status mha_forward(const void* xq, const void* xk, const void* xv, const void* wq,
                       const void* wk, const void* wv, const void* wo, void* out,
                       void* workspace, size_t workspace_bytes, int batch, int n_q, int n_k,
                       int d_model, int heads, mha_dtype dtype, int causal, void* stream);

/*
 * mha_forward_padded -- mha_forward with a key-padding mask on the xk/xv
 * sequence (encoder self-attention over a padded batch, or cross-attention to
 * a padded encoder memory; "The Transformer" (rayaq.ca), "Masks: who may look
 * at whom"). kv_len is as in attention_forward_padded: a device array of
 * `batch` int32 key lengths, clamped to [0, n_k]. Output rows of an item with
 * length 0 are 0 W^O = 0. A NULL kv_len is MHA_ERR_INVALID_ARG.
 * The projections still run over all n_k rows; only the attention skips the
 * padded keys.
 */
mha_status mha_forward_padded(const void* xq, const void* xk, const void* xv, const void* wq,
                              const void* wk, const void* wv, const void* wo, void* out,
                              void* workspace, size_t workspace_bytes, int batch, int n_q, int n_k,
                              int d_model, int heads, mha_dtype dtype, int causal,
                              const int32_t* kv_len, void* stream);

/*
 * mha_forward_noalloc -- mha_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): the same computation, arguments and rules, minus the
 * workspace. The library keeps the intermediates (Q, K, V, the concatenated
 * heads) in a fixed device array of MHA_NOALLOC_MAX_WORKSPACE bytes, one per
 * GPU, held from the library's load on that GPU until the process ends. The
 * call allocates nothing.
 * A problem whose mha_forward_workspace_size exceeds the array is rejected
 *   with MHA_ERR_UNSUPPORTED before any HIP call (use mha_forward there).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 *   (different streams or threads without ordering between them) race and
 *   give undefined results. Calls ordered on one stream are safe.
 */
#define MHA_NOALLOC_MAX_WORKSPACE ((size_t)128 << 20)
mha_status mha_forward_noalloc(const void* xq, const void* xk, const void* xv, const void* wq,
                               const void* wk, const void* wv, const void* wo, void* out, int batch,
                               int n_q, int n_k, int d_model, int heads, mha_dtype dtype, int causal,
                               void* stream);

/*
 * encoder_layer_forward -- one Transformer encoder layer, post-norm, inference:
 *   h   = LayerNorm(x + MultiHead(x, x, x))            (attention with biases)
 *   out = LayerNorm(h + FFN(h)),  FFN(h) = max(0, h W1 + b1) W2 + b2
 *   -- "The Transformer" (hoshank.vercel.app), "The Mathematics": the FFN
 *   equation and output = LayerNorm(x + Sublayer(x)) around both sub-layers;
 *   "The Transformer" (rayaq.ca), "Residuals and LayerNorm" and "In PyTorch"
 *   (the EncoderLayer forward in eval mode: no dropout).
 * LayerNorm: per position, subtract the mean, divide by sqrt(population
 *   variance + eps), then multiply by gamma and add beta. The pages print no
 *   eps; 1e-5 is the default of the module their code uses.
 * x, out: (batch, n, d_model) contiguous, of `dtype`. `weights` is a HOST
 *   pointer to a struct of DEVICE pointers, every one non-null, 16-byte
 *   aligned, of `dtype`, stored (in, out):
 *     wq, wk, wv, wo (d_model, d_model); bq, bk, bv, bo (d_model);
 *     ln1_gamma, ln1_beta (d_model); w1 (d_model, d_ff); b1 (d_ff);
 *     w2 (d_ff, d_model); b2 (d_model); ln2_gamma, ln2_beta (d_model).
 * workspace: device memory of at least encoder_layer_workspace_size() bytes;
 *   scratch owned by the caller.
 * causal, kv_len: masks of the self-attention, as in mha_forward and
 *   mha_forward_padded (kv_len may be NULL: no padding).
 * bf16: every stored tensor (the sub-layer outputs, h, the FFN hidden layer,
 *   out) is rounded to bf16; the residual sums, the LayerNorm statistics and
 *   every accumulation are fp32.
 * Limits: d_model/heads follows attention_forward's head-width rules;
 *   d_model and d_ff multiples of 8 (bf16) or 4 (f32); d_model <= 4096
 *   (MHA_ERR_UNSUPPORTED above); eps finite and >= 0.
 * Launches, all on `stream`: Q/K/V projections, attention, W^O, residual +
 *   LayerNorm, W1 with bias and ReLU, W2 with bias, residual + LayerNorm.
 */
typedef struct mha_encoder_weights {
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const void* bq;
  const void* bk;
  const void* bv;
  const void* bo;
  const void* ln1_gamma;
  const void* ln1_beta;
  const void* w1;
  const void* b1;
  const void* w2;
  const void* b2;
  const void* ln2_gamma;
  const void* ln2_beta;
} mha_encoder_weights;

size_t encoder_layer_workspace_size(int batch, int n, int d_model, int heads, int d_ff, mha_dtype dtype);

mha_status encoder_layer_forward(const void* x, const mha_encoder_weights* weights, void* out,
                                 void* workspace, size_t workspace_bytes, int batch, int n, int d_model,
                                 int heads, int d_ff, float eps, mha_dtype dtype, int causal,
                                 const int32_t* kv_len, void* stream);

/*
 * attention_backward -- gradients of attention_forward with respect to Q, K
 * and V, given the gradient dO of a loss with respect to the output:
 *   dV = P^T dO,   dP = dO V^T,   dS_ij = P_ij (dP_ij - delta_i),
 *   delta_i = sum_j P_ij dP_ij = dO_i . O_i,
 *   dQ = scale dS K,   dK = scale dS^T Q,
 * the chain rule through O = P V, the row softmax (Jacobian
 * diag(P_i) - P_i P_i^T) and S = scale Q K^T. Masked scores are constants, so
 * masked pairs pass no gradient. The pages give this gradient as the reason
 * for the 1/sqrt(d_k) scale: a saturated softmax passes almost none ("32
 * Transformer" (ml-canon-en.vercel.app), "Why we divide by sqrt(dk)"; "How
 * Transformers Work" (worksonmygpu.com), "Scaled dot-product attention",
 * step 2; "The Transformer" (hoshank.vercel.app), "The Breakthrough").
 *
 * q, k, v, o, d_o: as attention_forward's q, k, v, o (o is the forward's
 *   output for these inputs, d_o has o's shape); dq, dk, dv: outputs of the
 *   shapes of q, k, v. Each tensor has its own {batch, head, row} element
 *   strides; last dimension contiguous. All device memory, of `dtype`.
 * lse: DEVICE fp32 (batch, heads, n_q), 16-byte aligned: the log-sum-exp that
 *   attention_forward / attention_forward_padded returned for the same q, k,
 *   scale, causal flag and kv_len. P is recomputed from it exactly
 *   (P_ij = exp(scale q_i.k_j - lse_i)); an lse that does not belong to these
 *   inputs gives meaningless gradients (not detected). -inf marks a row with
 *   no visible key: it passes no gradient.
 * causal, scale, kv_len: as in attention_forward_padded (kv_len may be NULL).
 *   Keys at or past kv_len[b] get dK = dV = 0.
 * workspace: DEVICE scratch of at least attention_backward_workspace_size()
 *   bytes (two fp32 values per query row, written by the first launch and
 *   read by the second: delta, and for bf16 the row's lse times log2(e)),
 *   16-byte aligned.
 * Supported: as attention_forward (bf16: d = 64; f32: d in {16, 32, 64, 128}).
 * bf16: P and dS are rounded to bf16 for the matrix products (as P is in the
 *   forward), every accumulation is fp32, and dq, dk, dv are rounded once.
 * Launches, both on `stream`: dQ with delta (a workgroup per query block),
 *   then dK and dV (a workgroup per key block); no atomics, so the result is
 *   deterministic.
 * Outputs must not overlap any input.
 */
size_t attention_backward_workspace_size(int batch, int heads, int n_q);

mha_status attention_backward(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                              const float* lse, void* dq, void* dk, void* dv, int batch, int heads, int n_q,
                              int n_k, int d, const int64_t q_strides[3], const int64_t k_strides[3],
                              const int64_t v_strides[3], const int64_t o_strides[3],
                              const int64_t do_strides[3], const int64_t dq_strides[3],
                              const int64_t dk_strides[3], const int64_t dv_strides[3], mha_dtype dtype,
                              int causal, float scale, const int32_t* kv_len, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * attention_decode -- one decoding step against a key/value cache: for every
 * (batch, head) the newest position's query attends to the first kv_len[b]
 * cached keys and values,
 *   o[b,h,:] = sum_{j < kv_len[b]} softmax_j( scale * q[b,h,:] . K[b,h,j,:] ) V[b,h,j,:].
 * This is the last row of causal attention over the sequence so far: a
 * decoder generates left to right and its masked self-attention covers the
 * tokens generated so far ("How Transformers Work" (worksonmygpu.com), "What
 * changed since 2017"; "The Transformer" (hoshank.vercel.app), "The
 * Breakthrough"; the mask: "The Transformer" (rayaq.ca), "Masks: who may look
 * at whom"). The same page names PagedAttention as how K and V are stored
 * when serving; the pages give no layout, so the cache here may be kept in
 * fixed-size pages reached through a per-sequence page table (a reading).
 *
 * q, o: (batch, heads, d) contiguous, of `dtype`, device memory.
 * cache: HOST pointer to an mha_kv_cache describing two DEVICE pools, k and
 *   v, of identical geometry. Element e of head h at (page, slot) is at
 *     page * page_stride + slot * row_stride + h * head_stride + e
 *   (element strides, non-negative, multiples of 8 (bf16) or 4 (f32); the
 *   last dimension contiguous). Key j of sequence b is at
 *     (page, slot) = (block_table[b * max_pages + j / page_size], j % page_size)
 *   when block_table (DEVICE, int32, (batch, max_pages)) is non-NULL, and at
 *   (page, slot) = (b, j) otherwise, so a plain (batch, max_len, heads, d)
 *   cache has strides {max_len*heads*d, heads*d, d} and a (batch, heads,
 *   max_len, d) one {heads*max_len*d, d, max_len*d}. page_size, max_pages
 *   and num_pages are read only with a block table.
 *   max_len: capacity of one sequence in keys (<= page_size * max_pages with
 *   a table); kv_len values are clamped to [0, max_len].
 *   A table entry read for a key below kv_len[b] that lies outside
 *   [0, num_pages) is not dereferenced: that (batch item, head)'s o and lse
 *   become NaN. Entries for keys at or past kv_len[b] are never read.
 * kv_len: DEVICE, `batch` int32. A length of 0 gives o = 0 and lse = -inf.
 * lse: NULL, or DEVICE fp32 (batch, heads): natural-log sum of exp(scores).
 * scale: multiplies the scores (1/sqrt(d) for the pages' attention); finite.
 * workspace: DEVICE scratch of at least attention_decode_workspace_size()
 *   bytes, 16-byte aligned, owned by the caller (partial softmax states of
 *   the key splits); no initial contents needed. Calls that overlap on one
 *   workspace race.
 * Supported: d in {16, 32, 64, 128}, bf16 or f32 (MHA_ERR_UNSUPPORTED
 *   otherwise); max_len <= 16776960 (65535 splits of 256 keys).
 * bf16: scores, softmax and the weighted sum are fp32 (no rounding of the
 *   weights); o is rounded to bf16 once.
 * Launches, both on `stream`: a workgroup per (batch, head, 256-key split)
 *   that holds a key (a sequence of one split, or of none, is finished
 *   there), then one merge of the splits per (batch, head).
 */
typedef struct mha_kv_cache {
  const void* k;
  const void* v;
  const int32_t* block_table;
  int64_t page_stride;
  int64_t row_stride;
  int64_t head_stride;
  int32_t page_size;
  int32_t max_pages;
  int32_t num_pages;
  int32_t max_len;
} mha_kv_cache;

size_t attention_decode_workspace_size(int batch, int heads, int d, int max_len);

mha_status attention_decode(const void* q, const mha_kv_cache* cache, const int32_t* kv_len, void* o,
                            float* lse, void* workspace, size_t workspace_bytes, int batch, int heads,
                            int d, mha_dtype dtype, float scale, void* stream);

/* Static English name of a status code (never NULL). */
const char* mha_status_string(mha_status status);

/* Thread-local detail text for the most recent non-OK status returned on the
 * calling thread ("" if none). Valid until the next call on this thread. */
const char* mha_last_error(void);

/* ABI version of this library: major * 10000 + minor * 100 + patch. */
int mha_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H */
