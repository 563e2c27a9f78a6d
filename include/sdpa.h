/*
 * sdpa.h — fused scaled dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * Computes, for every batch b and query head hq (KV head g = hq / (h_q / h_kv)):
 *
 *     S   = attn_scale * Q K^T                  (first matmul, then the scale)
 *     S_ij = -inf where causal and j > i         (top-left aligned causal mask)
 *     O   = softmax_rows(S) V
 *     LSE_i = ln sum_j exp(S_ij)                (the per-row softmax statistics)
 *
 * and its exact gradient (dQ, dK, dV) given dO. dK/dV of a KV head are summed
 * over the query heads that share it (GQA / MQA).
 *
 * Sources: the formula and its four steps are those of the JAX attention
 * codelab ("Speed up attention on GPU with cuDNN and TransformerEngine"),
 * step 1; the causal mask its step 7; KV-head sharing its step 9; FP8 E4M3
 * inputs its step 10. The scale applied to the first matmul's output, the
 * causal-mask lowering and the ``stats`` output come from the cuDNN 9 blog
 * ("Accelerating Transformers with NVIDIA cuDNN 9"), "SDPA as a cuDNN graph"
 * (Figure 4) and "SDPA usage". The strided logical (b, h, s, d) tensors with a
 * BSHD physical layout, the io/compute dtype split and the
 * execute(pointers, workspace) flow come from "Using cuDNN in Python".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a caller-owned DEVICE pointer. The library never
 *    allocates, frees or retains caller memory.
 *  - Tensors are logical (b, h, s, d). Each has a 4-entry stride array, in
 *    ELEMENTS, in that logical order; the d stride must be 1. BSHD is
 *    (s*h*d, d, h*d, 1), BHSD is (h*s*d, s*d, d, 1); any other strides with
 *    a unit d stride are accepted.
 *  - Alignment: every pointer must be 16-byte aligned and the b, h and s
 *    strides must be multiples of 16 bytes' worth of elements; otherwise
 *    SDPA_ERR_NOT_SUPPORTED (no silent slow path).
 *  - Calls are asynchronous on `stream` (0 = the null stream) and return
 *    after the kernels are enqueued; the caller synchronises.
 *  - Validation happens before anything is enqueued. On an error nothing is
 *    launched, the status is returned and sdpa_last_error() describes it.
 *  - Calls are thread-safe: the only state is thread-local (the error string
 *    and the optional timing events of sdpa_set_timing_events).
 *  - b == 0 or s_q == 0 is an empty problem: sdpa_fwd enqueues nothing; sdpa_bwd
 *    writes zeros to dK and dV (no query attends to them) and nothing else.
 *  - attn_scale must be finite and > 0 (the pages use 1/sqrt(d)).
 *  - Causal alignment of sdpa_fwd / sdpa_bwd is top-left: query i sees keys
 *    0..i, also when s_q != s_kv; every query row therefore sees at least
 *    key 0. sdpa_fwd_ex / sdpa_bwd_ex add bottom-right alignment and the
 *    padding mask (per-batch valid lengths).
 */
#ifndef SDPA_H_
#define SDPA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SDPA_F32 = 0,
  SDPA_F16 = 1,
  SDPA_BF16 = 2,
  SDPA_FP8_E4M3 = 3, /* OCP e4m3fn: 4 exponent bits, 3 mantissa bits, max 448, no inf */
  SDPA_FP8_E5M2 = 4  /* OCP e5m2: 5 exponent bits, 2 mantissa bits, max 57344, inf (gradients) */
} sdpa_dtype_t;

typedef enum {
  SDPA_OK = 0,
  SDPA_ERR_INVALID_ARGUMENT = 1,   /* NULL pointer, bad size, h_q % h_kv != 0, d stride != 1, ... */
  SDPA_ERR_NOT_SUPPORTED = 2,      /* valid, but no kernel for this dtype / d / alignment */
  SDPA_ERR_WORKSPACE_TOO_SMALL = 3,
  SDPA_ERR_HIP = 4                 /* the HIP runtime reported an error at launch */
} sdpa_status_t;

/*
 * Attention mask of sdpa_fwd_ex / sdpa_bwd_ex. The cuDNN 9 blog's SDPA node
 * call ("SDPA usage") lists the causal flag next to use_padding_mask with
 * per-batch seq_len_q / seq_len_kv; where the causal diagonal sits when the
 * query and key ranges differ is not on the pages, so both placements exist:
 *   SDPA_MASK_CAUSAL               top-left: key j visible to row i iff j <= i
 *   SDPA_MASK_CAUSAL_BOTTOM_RIGHT  key j visible to row i iff j <= i + (lk - lq),
 *                                  lq / lk the batch element's valid lengths
 *                                  (the last valid row sees every valid key)
 */
typedef enum {
  SDPA_MASK_NONE = 0,
  SDPA_MASK_CAUSAL = 1,
  SDPA_MASK_CAUSAL_BOTTOM_RIGHT = 2
} sdpa_mask_t;

/*
 * Score modifiers of sdpa_fwd_ex / sdpa_bwd_ex: the SDPA node's `bias` and
 * `use_alibi_mask` options in the cuDNN 9 blog's "SDPA usage" call (the pages
 * give no semantics; both are added to the scaled scores before the mask):
 *     S_ij = attn_scale * q_i . k_j + bias[b][h][i][j] - alibi_slopes[h] * |i + off - j|
 * with off the causal diagonal offset (lk - lq for SDPA_MASK_CAUSAL_BOTTOM_RIGHT,
 * else 0). Either member may be NULL. The bias is a constant: the backward
 * forms no gradient for it.
 *   alibi_slopes  device fp32 [h_q], 4-byte aligned (the ALiBi paper's slopes are
 *                 2^(-8 (h+1) / h_q) for h_q a power of two).
 *   bias          device tensor, logical [b][h_q][s_q][s_kv], 16-byte aligned.
 *   bias_dtype    SDPA_F32, or the io dtype (F16 / BF16 inputs).
 *   bias_stride   element strides in (b, h, s_q, s_kv) order; the s_kv stride
 *                 must be 1; 0 broadcasts over b or h; the s_q stride must be a
 *                 multiple of 16 bytes' worth of elements.
 * Not supported with FP8 inputs, and dropout not with F32 inputs
 * (SDPA_ERR_NOT_SUPPORTED); the split-KV forward path is not taken when
 * modifiers are present.
 */
typedef struct {
  const float* alibi_slopes;
  const void* bias;
  sdpa_dtype_t bias_dtype;
  int64_t bias_stride[4];
  /* Dropout of the attention weights (the node's `dropout` option; BF16 / F16
   * only): O = (P * Z) V with P the softmax of the modified, masked scores and
   * Z from a counter-based Philox4x32-10 stream (Salmon et al., SC 2011):
   * element (i, j) of query-head slot b * h_q + h takes byte (j mod 4) of word
   * (i mod 4) of Philox4x32-10(counter = (j / 4, i / 4, slot, dropout_offset),
   * key = (seed mod 2^32, seed / 2^32)); it is kept iff the byte is below
   * k8 = round((1 - dropout_p) * 256) (ties to even), and kept weights are
   * scaled by 256 / k8. LSE is that of the undropped weights. The backward
   * regenerates the same Z from the same three values. dropout_p in [0, 1];
   * 0 disables. Advance dropout_offset between calls for a fresh mask. */
  float dropout_p;
  uint64_t dropout_seed;
  uint32_t dropout_offset;
} sdpa_score_mod_t;

/*
 * Per-tensor fp8 factors (JAX attention codelab, step 10: per-tensor scaling
 * recipe). A real input value is x = e4m3(code) * descale_x. Inside the kernel
 * the softmax weights P (all in [0, 1]) are quantised as e4m3(P * scale_p)
 * before the second matmul and the result is multiplied back by descale_p.
 * The usual choice is scale_p = 448, descale_p = 1/448; scale_p must be <= 448
 * (SDPA_ERR_INVALID_ARGUMENT otherwise).
 */
typedef struct {
  float descale_q;
  float descale_k;
  float descale_v;
  float scale_p;
  float descale_p;
} sdpa_fp8_scales_t;

/*
 * Forward: O (and optionally LSE) from Q, K, V.
 *
 * Defined by the SDPA node call of the cuDNN 9 blog's "SDPA usage" section
 * (q, k, v, attn_scale, is_inference, use_causal_mask in; o and stats out),
 * computing the formula of the JAX attention codelab, step 1, with its step 7
 * causal mask; the tensors are described by dims and strides and executed on
 * caller pointers as in "Using cuDNN in Python" (graph build, then execute).
 * Ownership: every pointer stays the caller's; nothing is allocated. Errors:
 * invalid arguments and unsupported combinations are reported before any
 * launch (status + sdpa_last_error()); a launch failure returns SDPA_ERR_HIP.
 *
 *   q       [b, h_q,  s_q,  d] in_dtype, strides q_stride
 *   k, v    [b, h_kv, s_kv, d] in_dtype, strides k_stride / v_stride
 *   o       [b, h_q,  s_q,  d] out_dtype, strides o_stride (written)
 *   lse     fp32 [b][h_q][s_q], contiguous, natural log (written); NULL means
 *           inference mode (the cuDNN node's is_inference): no statistics.
 *   fp8     required iff in_dtype == SDPA_FP8_E4M3, else must be NULL.
 *
 * Supported (in_dtype -> out_dtype, d):
 *   F32 -> F32, d in {64, 128}
 *   F16 -> F16, BF16 -> BF16, d in {64, 128}
 *   FP8_E4M3 -> BF16, d in {128, 256}
 * causal in {0, 1} for all of them; any h_q multiple of h_kv.
 */
sdpa_status_t sdpa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                       int b, int h_q, int h_kv, int s_q, int s_kv, int d,
                       const int64_t q_stride[4], const int64_t k_stride[4],
                       const int64_t v_stride[4], const int64_t o_stride[4],
                       float attn_scale, int causal,
                       sdpa_dtype_t in_dtype, sdpa_dtype_t out_dtype,
                       const sdpa_fp8_scales_t* fp8, hipStream_t stream);

/*
 * Forward with an explicit mask and the padding mask (the cuDNN 9 blog's
 * SDPA node options use_padding_mask / seq_len_q / seq_len_kv, "SDPA usage").
 * Same arguments and support matrix as sdpa_fwd, with `causal` replaced by:
 *   mask        an sdpa_mask_t (SDPA_ERR_INVALID_ARGUMENT otherwise).
 *   seq_len_q   device int32 [b], 4-byte aligned, or NULL (every batch element
 *               has s_q rows): batch element i uses only its first
 *               seq_len_q[i] query rows.
 *   seq_len_kv  device int32 [b] or NULL (= s_kv): batch element i uses only
 *               its first seq_len_kv[i] keys; K/V rows past it are never read.
 * The lengths are read by the kernels (no host synchronisation); values are
 * clamped to [0, s_q] and [0, s_kv]. A query row that sees no key (a row at or
 * past seq_len_q[i], or under bottom-right alignment a row above the shifted
 * diagonal) gets O = 0 and LSE = -inf.
 *   mod         optional score modifiers (bias tensor, ALiBi slopes); NULL = none.
 *   workspace, workspace_bytes  optional device scratch for the split-KV
 *               path (see sdpa_fwd_workspace_size); NULL / 0 allowed.
 * sdpa_fwd(..., causal, ...) equals sdpa_fwd_ex(..., causal ? SDPA_MASK_CAUSAL
 * : SDPA_MASK_NONE, NULL, NULL, NULL, ..., NULL, 0, stream).
 */
sdpa_status_t sdpa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                          int b, int h_q, int h_kv, int s_q, int s_kv, int d,
                          const int64_t q_stride[4], const int64_t k_stride[4],
                          const int64_t v_stride[4], const int64_t o_stride[4],
                          float attn_scale, sdpa_mask_t mask,
                          const int32_t* seq_len_q, const int32_t* seq_len_kv,
                          const sdpa_score_mod_t* mod,
                          sdpa_dtype_t in_dtype, sdpa_dtype_t out_dtype,
                          const sdpa_fp8_scales_t* fp8,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sdpa_fwd_ex without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). Same arguments, support matrix and results as
 * sdpa_fwd_ex minus the workspace pair; it calls no hipMalloc / hipFree and
 * no allocating routine. Where sdpa_fwd_ex would take the split-KV path with a
 * workspace (see sdpa_fwd_workspace_size), this entry point takes it with a
 * static scratch array of 64 MiB that the library holds on each GPU it runs
 * on until the process ends; a shape whose split-KV partials need more than
 * that returns SDPA_ERR_NOT_SUPPORTED before anything is launched. The scratch
 * is shared by every call on a GPU and keeps the last call's contents (each
 * call overwrites every partial it reads), so calls on one GPU that overlap
 * in time (concurrent streams, or host threads) race: serialise them.
 */
sdpa_status_t sdpa_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                               int b, int h_q, int h_kv, int s_q, int s_kv, int d,
                               const int64_t q_stride[4], const int64_t k_stride[4],
                               const int64_t v_stride[4], const int64_t o_stride[4],
                               float attn_scale, sdpa_mask_t mask,
                               const int32_t* seq_len_q, const int32_t* seq_len_kv,
                               const sdpa_score_mod_t* mod,
                               sdpa_dtype_t in_dtype, sdpa_dtype_t out_dtype,
                               const sdpa_fp8_scales_t* fp8, hipStream_t stream);

/*
 * Bytes of device workspace that sdpa_fwd_ex's split-KV path needs for this
 * shape; 0 when the shape does not take it, or takes it without a workspace.
 *
 * The JAX attention codelab (step 9) motivates GQA / MQA by the KV-cache
 * memory of inference. For few query rows against many keys (s_q <= 64,
 * s_kv >= 512, ceil(s_q * h_q / h_kv / 32) <= h_q / h_kv; BF16 / F16,
 * d in {64, 128}) the forward groups every query head of a KV head and every
 * query position into shared row blocks, so each K/V byte is read once, and
 * splits the key range over many workgroups; per-split fp32 partials
 * (O / l and LSE) are merged by a second kernel. sdpa_fwd_ex takes that path
 * when the workspace is given (workspace_bytes >= this size, 16-byte aligned)
 * or when this size is 0; with workspace == NULL it runs the row-block kernel
 * instead (same results within rounding). The split changes only the order in
 * which each row's softmax sums are associated.
 */
size_t sdpa_fwd_workspace_size(int b, int h_q, int h_kv, int s_q, int s_kv, int d,
                               sdpa_dtype_t in_dtype);

/*
 * Bytes of device workspace sdpa_bwd needs for this problem (16-byte aligned
 * use): the workspace query of "Using cuDNN in Python" (get_workspace_size(),
 * then a caller-allocated buffer handed to execute). Pure host arithmetic; no
 * error state (invalid shapes give 0). 0 is a valid answer only for empty
 * problems. The same size serves sdpa_bwd_fp8 (dtype SDPA_FP8_E4M3): both hold
 * the fp32 row statistic D and, for grouped-query shapes split over several
 * workgroups, the fp32 dK / dV partials.
 */
size_t sdpa_bwd_workspace_size(int b, int h_q, int h_kv, int s_q, int s_kv, int d,
                               int causal, sdpa_dtype_t dtype);

/*
 * Backward: dQ, dK, dV of L = sum(O * dO).
 *
 * The cuDNN 9 blog shows the fused forward + backward ("SDPA performance",
 * Figure 2) and a backward graph with the forward's flexibility ("SDPA as a
 * cuDNN graph"); it does not print the backward's formulas, so this is the
 * exact gradient of sdpa_fwd's result, recomputing the weights from the
 * forward's stats (LSE), with dK / dV summed over each KV head's query-head
 * group (JAX attention codelab, step 9). It runs in the execute(pointers,
 * workspace) flow of "Using cuDNN in Python": the caller queries
 * sdpa_bwd_workspace_size and owns the workspace. Errors as for sdpa_fwd;
 * SDPA_ERR_WORKSPACE_TOO_SMALL when the workspace is short.
 *
 *   q, k, v, o, dout   as in sdpa_fwd (o is the forward's output, dout is dL/dO,
 *                      same layout rules); dtype BF16 or F16 for all of them.
 *   lse                the forward's LSE (fp32 [b][h_q][s_q], contiguous); required.
 *   dq                 [b, h_q, s_q, d]  (written)
 *   dk, dv             [b, h_kv, s_kv, d] (written; summed over each KV head's
 *                      query-head group)
 *   workspace          device buffer of at least sdpa_bwd_workspace_size(...)
 *                      bytes, 16-byte aligned; its contents are scratch.
 * Supported: BF16 and F16, d in {64, 128}, causal in {0, 1}.
 */
sdpa_status_t sdpa_bwd(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse,
                       void* dq, void* dk, void* dv,
                       int b, int h_q, int h_kv, int s_q, int s_kv, int d,
                       const int64_t q_stride[4], const int64_t k_stride[4],
                       const int64_t v_stride[4], const int64_t o_stride[4],
                       const int64_t do_stride[4], const int64_t dq_stride[4],
                       const int64_t dk_stride[4], const int64_t dv_stride[4],
                       float attn_scale, int causal, sdpa_dtype_t dtype,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward with an explicit mask and the padding mask; the arguments of
 * sdpa_bwd with `causal` replaced by mask / seq_len_q / seq_len_kv, which must
 * be those of the forward that produced o and lse (same meaning and clamping as
 * in sdpa_fwd_ex). Rows that see no key (LSE = -inf) take no part: their dQ is
 * 0 and they add nothing to dK, dV; keys at or past seq_len_kv[i] get
 * dK = dV = 0; dQ rows at or past seq_len_q[i] are 0. `mod` must be the
 * forward's (it changes P). The workspace size is that of
 * sdpa_bwd_workspace_size for the same shape.
 */
sdpa_status_t sdpa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse,
                          void* dq, void* dk, void* dv,
                          int b, int h_q, int h_kv, int s_q, int s_kv, int d,
                          const int64_t q_stride[4], const int64_t k_stride[4],
                          const int64_t v_stride[4], const int64_t o_stride[4],
                          const int64_t do_stride[4], const int64_t dq_stride[4],
                          const int64_t dk_stride[4], const int64_t dv_stride[4],
                          float attn_scale, sdpa_mask_t mask,
                          const int32_t* seq_len_q, const int32_t* seq_len_kv,
                          const sdpa_score_mod_t* mod,
                          sdpa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Factors of the fp8 backward (JAX attention codelab, step 10: per-tensor
 * scaling, HYBRID format). Inputs: real value = fp8 code * descale (all
 * finite and > 0). The two products whose left operand the kernels quantise
 * themselves take a scale: P (softmax weights, <= 1) goes to e4m3 as
 * P * scale_p, with 0 < scale_p <= 448 (448 uses the whole range); dS (the
 * score gradient) goes to ds_dtype as dS * scale_ds, saturated to the
 * format's largest finite value (448 for e4m3, 57344 for e5m2). The recipe's
 * delayed scaling derives such scales from a history of per-tensor absolute
 * maxima; amax_ds, when not NULL, is a device float that receives
 * max(*amax_ds, max |dS|) over this call (dS before scaling and saturation),
 * which the caller feeds into that history (it must hold a value >= 0, e.g. 0,
 * before the call). */
typedef struct {
  float descale_q;
  float descale_k;
  float descale_v;
  float descale_do;
  float scale_p;           /* e4m3 scale of P; (0, 448] */
  float scale_ds;          /* scale of dS; finite, > 0 */
  sdpa_dtype_t ds_dtype;   /* SDPA_FP8_E4M3 or SDPA_FP8_E5M2 */
  float* amax_ds;          /* optional device float (4-byte aligned), or NULL */
} sdpa_fp8_bwd_scales_t;

/*
 * FP8 backward: dQ, dK, dV of L = sum(O * dO) for the fp8 forward, in the
 * HYBRID format of the JAX attention codelab (step 10): tensors in e4m3 for
 * the forward pass, the gradient dO in e5m2 for the backward pass, each with a
 * per-tensor scale. The gradients are those of sdpa_bwd (the exact
 * chain-rule backward from the forward's LSE), with all five matrix products
 * on fp8 operands and fp32 accumulation: S = Q K^T and dP = dO V^T on the
 * codes; dV = P^T dO with P in e4m3 (scale_p); dK = dS^T Q and dQ = dS K with
 * dS in ds_dtype (scale_ds). The factors of each product are applied to its
 * fp32 result.
 *
 *   q, k, v     e4m3 codes, [b, h, s, d] with strides as in sdpa_fwd (the
 *               forward's inputs); values q * descale_q etc.
 *   o           the fp8 forward's BF16 output; lse its fp32 LSE (required).
 *   dout        dO codes in do_dtype (SDPA_FP8_E5M2, or SDPA_FP8_E4M3),
 *               value dout * descale_do.
 *   dq, dk, dv  BF16 gradients with respect to the real-valued q, k, v.
 *   mask, seq_len_q, seq_len_kv  as in sdpa_bwd_ex (those of the forward).
 *   scales      the factors above (required).
 *   workspace   at least sdpa_bwd_workspace_size(..., SDPA_FP8_E4M3) bytes,
 *               16-byte aligned; scratch.
 * Supported: d in {64, 128}; no score modifiers. Errors as for sdpa_bwd;
 * SDPA_ERR_INVALID_ARGUMENT for factors out of range.
 */
sdpa_status_t sdpa_bwd_fp8(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse,
                           void* dq, void* dk, void* dv,
                           int b, int h_q, int h_kv, int s_q, int s_kv, int d,
                           const int64_t q_stride[4], const int64_t k_stride[4],
                           const int64_t v_stride[4], const int64_t o_stride[4],
                           const int64_t do_stride[4], const int64_t dq_stride[4],
                           const int64_t dk_stride[4], const int64_t dv_stride[4],
                           float attn_scale, sdpa_mask_t mask,
                           const int32_t* seq_len_q, const int32_t* seq_len_kv,
                           sdpa_dtype_t do_dtype, const sdpa_fp8_bwd_scales_t* scales,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The standard ALiBi slopes for h_q heads, written to host memory
 * `slopes_host` (h_q floats; copy them to the device for
 * sdpa_score_mod_t.alibi_slopes). The cuDNN 9 blog's SDPA node call ("SDPA
 * usage") lists `use_alibi_mask` without its slopes; these are the ALiBi
 * paper's (Press, Smith, Lewis, "Train Short, Test Long: Attention with
 * Linear Biases"): for h_q a power of two the geometric sequence
 * 2^(-8 (i + 1) / h_q), i = 0 .. h_q - 1; otherwise the slopes of the largest
 * power of two n < h_q, followed by the first h_q - n even-indexed slopes
 * (i = 0, 2, 4, ...) of the 2n-head sequence. Host-only: no device call.
 * Returns SDPA_ERR_INVALID_ARGUMENT for h_q < 1 or slopes_host == NULL.
 */
sdpa_status_t sdpa_alibi_slopes(int h_q, float* slopes_host);

/*
 * Timing hook (diagnostics only; GPU-time-only reporting as in the cuDNN 9
 * blog's "SDPA performance" section). Registers `n` caller-created HIP events
 * (n = 0 or events = NULL disables) that this thread's following sdpa_fwd /
 * sdpa_bwd calls record on their stream at kernel boundaries:
 *   sdpa_fwd: events[0] before its kernel, events[1] after it (n >= 2);
 *   sdpa_bwd: events[0] before the dQ kernel (which also forms
 *             D = rowsum(dO * O)), events[1] after it, events[2] after the
 *             dK/dV kernel and its split reduction (n >= 3); sdpa_bwd_fp8
 *             records the same three after its widening kernels.
 * The library does not own the events. Returns SDPA_ERR_INVALID_ARGUMENT for
 * n < 0, n > 8, or events == NULL with n > 0.
 */
sdpa_status_t sdpa_set_timing_events(hipEvent_t* events, int n);

/*
 * Diagnostics: sustained matrix-core rate probe, the measured denominator
 * beside the published dense peaks that the "% of MFMA peak" of the cuDNN 9
 * blog's forward and forward + backward figures ("SDPA performance") is
 * quoted against. Enqueues `blocks` workgroups of 4 waves on `stream`; every
 * wave issues `iters` rounds of 8 independent MFMAs:
 *   SDPA_BF16      v_mfma_f32_32x32x16_bf16          (32768 flops each)
 *   SDPA_FP8_E4M3  v_mfma_scale_f32_32x32x64_f8f6f4  (131072 flops each)
 * so one launch performs blocks * 4 * iters * 8 MFMAs; the caller times it
 * (events on the stream). stamps: caller-owned device uint64 [4 * blocks],
 * 16-byte aligned (written): per workgroup, the shader cycle counter at the
 * start and end of its loop, then the 100 MHz real-time counter at the same
 * two points (their ratio gives the shader clock under full matrix load).
 * Errors: SDPA_ERR_INVALID_ARGUMENT for another dtype, blocks or iters < 1,
 * or stamps NULL / misaligned; SDPA_ERR_HIP for a launch failure.
 */
sdpa_status_t sdpa_mfma_probe(sdpa_dtype_t dtype, int blocks, int iters, uint64_t* stamps, hipStream_t stream);

/*
 * Message describing this thread's most recent failed call ("" after a
 * success): the programmatic last-error string of the cuDNN 9 blog's
 * "Improved error reporting" section (cudnnGetLastErrorString). The string is
 * owned by the library and valid until this thread's next call.
 */
const char* sdpa_last_error(void);

/*
 * Static name of a status code (the categorised error codes of the cuDNN 9
 * blog's "Improved error reporting"); "SDPA_ERR_UNKNOWN" for other values.
 */
const char* sdpa_status_string(sdpa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_H_ */
