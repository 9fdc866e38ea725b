/*
 * lightning_attn.h -- C ABI of the MI355X (gfx950) Lightning Attention library.
 *
 * The layer (blog "Diving into MiniMax01 405B MoE", section "Hybrid Modeling",
 * 7/8 Linear Attention (Lightning Attention-2), Mechanism steps 1-4):
 *     q~, k~, v~ = SiLU(q), SiLU(k), SiLU(v)                   (step 2)
 *     y_t        = q~_t S_t,  S_t = S_0 + sum_{u<=t} k~_u^T v~_u  (step 3, causal)
 *     out_t      = y_t / sqrt(mean_{h,d} y_t^2 + eps) * w * sigmoid(gate_t)   (step 4)
 * with no 1/sqrt(d) scale, no decay and no normaliser.  The model card
 * ("2. Model Architecture") fixes 64 heads of dimension 128.  y is computed
 * blockwise: a masked intra-block product (Q~ K~^T (.) M) V~ plus an
 * inter-block product Q~ S against a running fp32 state, the O(d^2)-per-token
 * right product of Mechanism step 3.
 *
 * Conventions shared by every call
 *   - Layout: activations token-major, element (t, h, d) at ((t*H)+h)*D + d;
 *     norm weight [H*D] indexed h*D + d; states [nseq][H][D][D] fp32 with
 *     state[i][j] = sum k~_i v~_j (row = key dimension, column = value dim).
 *   - q, k, v, gate, norm_weight and out share one dtype (la_dtype).  The
 *     state is always fp32.  Arithmetic is fp32 (bf16 MFMA operands with fp32
 *     accumulation for bf16 inputs); out is rounded to the input dtype.
 *   - All pointers are device pointers (hipMalloc'd or from a framework
 *     allocator) and must be 16-byte aligned.  The caller owns all memory;
 *     the library allocates nothing and keeps no global mutable state (but
 *     a per-device cache of the CU count and, for the layer call, one
 *     hipBLASLt handle per device), so calls are reentrant and thread-safe.
 *   - Work is enqueued asynchronously on `stream`; calls do not synchronize.
 *   - Errors: arguments are validated on the host before any HIP call; on a
 *     validation error nothing is enqueued.  A launch failure reported by
 *     hipGetLastError returns LA_ERR_HIP.  Device-side conditions (invalid
 *     cu_seqlens values, a cross-workgroup wait that gave up) leave `out`
 *     unspecified and are recorded in the workspace, readable with
 *     lightning_attn_workspace_status.  Non-finite inputs are not checked.
 *     `out` must not alias an input.
 */
#ifndef LIGHTNING_ATTN_H
#define LIGHTNING_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_API __attribute__((visibility("default")))

typedef enum {
    LA_OK = 0,
    LA_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
    LA_ERR_BAD_SHAPE = 2,          /* a size is negative / zero where not allowed / inconsistent */
    LA_ERR_UNSUPPORTED = 3,        /* head_dim, block, chunk or dtype outside the supported set */
    LA_ERR_MISALIGNED = 4,         /* a pointer is not 16-byte aligned */
    LA_ERR_WORKSPACE_TOO_SMALL = 5,/* workspace_bytes below the matching *_workspace_size() */
    LA_ERR_HIP = 6,                /* the HIP runtime reported an error while enqueueing */
    LA_ERR_SCRATCH_TOO_SMALL = 7   /* sizes exceed the fixed scratch of lightning_attn_decode_noalloc */
} la_status;

typedef enum { LA_DTYPE_F32 = 0, LA_DTYPE_BF16 = 1 } la_dtype;

/* GEMM kernels of lightning_attn_layer_prefill: the library's own bf16 MFMA
 * kernel, or hipBLASLt (kept as the baseline the former is timed against). */
typedef enum { LA_GEMM_MFMA = 0, LA_GEMM_HIPBLASLT = 1 } la_gemm;

/* Human-readable text for a status code (static storage, never NULL). */
LA_API const char* lightning_attn_status_string(la_status s);

/*
 * Device-side status of the last call that used `workspace`.  Some conditions
 * can only be seen by the kernels, after the call has returned LA_OK: they
 * are recorded in a header at the start of the workspace of every prefill,
 * state, backward, layer and softmax-prefill call, and that call's `out` (or
 * gradients, or final states) is then unspecified.  This call copies the
 * header to the host after the work already enqueued on `stream` has
 * finished (it synchronizes `stream`):
 *   status[0]  error: 0 = ok;
 *              1 = cu_seqlens inconsistent (cu[0] != 0, a decreasing entry,
 *                  or cu[nseq] != total_tokens); nothing was processed;
 *              2 = chunk table overflow (cannot happen with a workspace of
 *                  the size the *_workspace_size call returns);
 *              3 = a cross-workgroup wait of the fused prefill walk gave up
 *                  (about a second of polling): the workgroups of one chunk
 *                  could not all run at once, e.g. because other work held
 *                  compute units on a concurrent stream
 *   status[1]  error 3: the wait that gave up first (1 = group sums of the
 *              RMSNorm exchange, 4 = the norm factors), else 0
 *   status[2], status[3]  error 3: its chunk and head, else 0
 *   workspace: the same pointer and its size (at least 64 bytes: the header);
 *              status: host int32[4].
 * Not meaningful for the decode calls (their workspaces have no header: the
 * softmax decode reports its per-sequence status words itself).
 */
LA_API la_status lightning_attn_workspace_status(const void* workspace, size_t workspace_bytes,
                                                 int32_t* status, hipStream_t stream);

/*
 * Supported shapes: head_dim in {16, 32, 64, 128}; block in {16, 32, 64} and
 * block <= chunk; heads >= 1.  bf16 with head_dim 128 and block 64 runs the
 * MFMA kernels, whose walk fuses the RMSNorm across heads and therefore needs
 * the workgroups of all heads of a chunk resident at once (one per compute
 * unit): with more heads than the device has compute units, and for every
 * other supported combination, the fp32 vector-ALU kernels run instead (same
 * results up to rounding; the workspace size follows that choice).
 *
 * chunk_tokens: the sequence is cut into chunks of this many tokens that are
 * processed in parallel (the running state entering each chunk is an
 * exclusive prefix sum of per-chunk states).  0 lets the library choose (about
 * one (chunk, head) work item per compute unit, at most 8192 tokens); a
 * positive value must be a multiple of `block`; negative values return
 * LA_ERR_BAD_SHAPE (workspace size 0).  The result does not depend on it
 * beyond rounding.
 *
 * Workspace bytes needed by a prefill over `total_tokens` tokens in `nseq`
 * sequences (a batch of B rows of N tokens is nseq = B, total = B*N).
 * Returns 0 for unsupported arguments.
 */
LA_API size_t lightning_attn_prefill_workspace_size(int64_t total_tokens, int nseq, int heads,
                                             int head_dim, int block, int chunk_tokens,
                                             la_dtype dtype);

/*
 * Causal prefill of `batch` independent rows of `seqlen` tokens.
 *   q, k, v, gate, out: [batch][seqlen][heads][head_dim]
 *   norm_weight:        [heads*head_dim]
 *   initial_state:      [batch][heads][head_dim][head_dim] fp32, or NULL (zeros)
 *   final_state:        same shape, or NULL (not written); may alias initial_state
 *   eps:                RMSNorm epsilon (added to the mean of squares), >= 0
 * seqlen may be 0 (nothing is written except final_state = initial_state).
 */
LA_API la_status lightning_attn_prefill(const void* q, const void* k, const void* v, const void* gate,
                                 const void* norm_weight, void* out, const float* initial_state,
                                 float* final_state, int batch, int64_t seqlen, int heads,
                                 int head_dim, int block, int chunk_tokens, float eps,
                                 la_dtype dtype, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Causal prefill of `nseq` sequences packed back to back (varlen): sequence s
 * owns tokens [cu_seqlens[s], cu_seqlens[s+1]) and starts from its own state
 * (initial_state[s], or zeros); no token attends across a boundary.
 *   q, k, v, gate, out: [total_tokens][heads][head_dim]
 *   cu_seqlens:         device int32 [nseq+1]: cu[0] = 0, nondecreasing,
 *                       cu[nseq] = total_tokens (empty sequences allowed)
 *   initial_state / final_state: [nseq][heads][head_dim][head_dim] fp32 or NULL
 */
LA_API la_status lightning_attn_prefill_varlen(const void* q, const void* k, const void* v,
                                        const void* gate, const void* norm_weight, void* out,
                                        const int32_t* cu_seqlens, int nseq, int64_t total_tokens,
                                        const float* initial_state, float* final_state, int heads,
                                        int head_dim, int block, int chunk_tokens, float eps,
                                        la_dtype dtype, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/*
 * Final states only: for each sequence, initial_state (or zeros) plus the sum
 * over its tokens of k~^T v~ -- the running state of Mechanism step 3 after
 * the sequence's last token -- without computing any output.  This is the
 * first pass of a prefill split along the sequence (the sequence-parallel
 * scheme the MiniMax-Text-01 summary page lists as LASP+): every part's state
 * sum, then an exclusive prefix over the parts (by the caller), then
 * lightning_attn_prefill of each part with its prefix as initial_state.
 * q, gate and the norm weight are not read.
 *   k, v:          [batch][seqlen][heads][head_dim], or packed [total][heads]
 *                  [head_dim] with device cu_seqlens int32 [nseq+1] (as for
 *                  lightning_attn_prefill_varlen)
 *   initial_state: [nseq][heads][head_dim][head_dim] fp32, or NULL (zeros)
 *   final_state:   same shape, required; may alias initial_state
 * chunk_tokens: as for the prefill (0 = automatic); negative values return
 * LA_ERR_BAD_SHAPE.
 * Shapes, dtypes and errors as for the prefill.
 */
LA_API size_t lightning_attn_state_workspace_size(int64_t total_tokens, int nseq, int heads,
                                                  int head_dim, int block, int chunk_tokens,
                                                  la_dtype dtype);
LA_API la_status lightning_attn_state(const void* k, const void* v, const float* initial_state,
                                      float* final_state, int batch, int64_t seqlen, int heads,
                                      int head_dim, int block, int chunk_tokens, la_dtype dtype,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream);
LA_API la_status lightning_attn_state_varlen(const void* k, const void* v,
                                             const int32_t* cu_seqlens, int nseq,
                                             int64_t total_tokens, const float* initial_state,
                                             float* final_state, int heads, int head_dim,
                                             int block, int chunk_tokens, la_dtype dtype,
                                             void* workspace, size_t workspace_bytes,
                                             hipStream_t stream);

/*
 * Backward pass: gradients of a prefill (same inputs, same eps) for a loss L
 * given dL/dout and, optionally, dL/d(final state).  By the chain rule
 * through Mechanism steps 4, 3, 2 in reverse:
 *     a = dout * w * sigmoid(gate),  yhat = y * r  (y, r as in the forward)
 *     dy    = r * (a - yhat * mean_{h,d}(a * yhat))            per token
 *     dgate = dout * yhat * w * sigmoid(gate) * (1 - sigmoid(gate))
 *     dw    = sum over tokens of dout * yhat * sigmoid(gate)
 *     dS_t  = dS_final + sum_{u >= t} q~_u^T dy_u              (dL/dS_t)
 *     dq = (dy_t S_t^T) * SiLU'(q),  dk = (v~_t dS_t^T) * SiLU'(k),
 *     dv = (k~_t dS_t) * SiLU'(v),   dS0 = dS at the sequence's first token
 * with SiLU'(x) = sigmoid(x) (1 + x (1 - sigmoid(x))).  y is recomputed.
 *   q, k, v, gate, dout, dq, dk, dv, dgate: [batch][seqlen][heads][head_dim]
 *                    (or packed [total][heads][head_dim] with cu_seqlens)
 *   norm_weight:     [heads*head_dim], dtype of the activations
 *   dweight:         [heads*head_dim] fp32, required
 *   initial_state:   [nseq][heads][head_dim][head_dim] fp32 or NULL (zeros)
 *   d_final_state:   same shape, or NULL (no gradient reaches the final state)
 *   d_initial_state: same shape, or NULL (not written)
 * Two paths, chosen by dtype and head_dim:
 *   - bf16 with head_dim 128: the walks run on bf16 MFMA with fp32
 *     accumulation and an fp32 running state; SiLU is applied to q, k, v as
 *     they are loaded (no copies of q~, k~, v~), and the recomputed y and dy
 *     are kept in bf16 (4 bytes per element of q in the workspace).  Every
 *     gradient, dweight and d_initial_state included, is therefore at bf16
 *     accuracy.
 *   - any other supported shape: fp32 vector-ALU kernels; the workspace holds
 *     fp32 q~, k~, v~, y and dy (20 bytes per element of q).
 * Both also keep two fp32 states per chunk and head in the workspace.
 * chunk_tokens: 0 = automatic, or
 * a multiple of `block` (the result does not depend on it beyond rounding).
 * heads * head_dim must be at most 32768 (else the workspace size is 0 and
 * the call returns LA_ERR_UNSUPPORTED).  Outputs must not alias inputs.
 * Errors as for the prefill.
 */
LA_API size_t lightning_attn_backward_workspace_size(int64_t total_tokens, int nseq, int heads,
                                                     int head_dim, int block, int chunk_tokens,
                                                     la_dtype dtype);
LA_API la_status lightning_attn_backward(const void* q, const void* k, const void* v,
                                         const void* gate, const void* norm_weight,
                                         const void* dout, const float* initial_state,
                                         const float* d_final_state, void* dq, void* dk, void* dv,
                                         void* dgate, float* dweight, float* d_initial_state,
                                         int batch, int64_t seqlen, int heads, int head_dim,
                                         int block, int chunk_tokens, float eps, la_dtype dtype,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);
LA_API la_status lightning_attn_backward_varlen(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    const void* dout, const int32_t* cu_seqlens, int nseq, int64_t total_tokens,
    const float* initial_state, const float* d_final_state, void* dq, void* dk, void* dv,
    void* dgate, float* dweight, float* d_initial_state, int heads, int head_dim, int block,
    int chunk_tokens, float eps, la_dtype dtype, void* workspace, size_t workspace_bytes,
    hipStream_t stream);

/*
 * Activations saved by a prefill for its backward pass (training: the
 * forward runs first anyway).  The backward above recomputes y = q~ S, the
 * attention output before the norm, and the states S entering the chunks,
 * from q, k, v: one pass of chunk sums of k~^T v~, a scan, and one walk.  A
 * prefill can keep both instead, and the backward then starts from them:
 *   saved: y, the dtype of q, [total_tokens][heads][head_dim], then (16-byte
 *          aligned) the fp32 state entering every chunk,
 *          [max_chunks][heads][head_dim][head_dim] (the initial state
 *          included), in the chunk layout both calls derive from the same
 *          (total_tokens, nseq, heads, head_dim, block, chunk_tokens).
 * The prefill's outputs are the same bits as lightning_attn_prefill's; the
 * backward's gradients are those of lightning_attn_backward (y read instead
 * of recomputed: the same bf16 values up to the rounding of the last bit).
 * The buffer is owned by the caller, written by the prefill and only read by
 * the backward, which must get the same q, k, v, gate, norm_weight, eps,
 * initial_state, chunk_tokens and shapes as the prefill that wrote it.
 * Only the fused bf16 MFMA path saves (bf16, head_dim 128, block 64, heads at
 * most the device's compute units): elsewhere lightning_attn_saved_size
 * returns 0 and the calls return LA_ERR_UNSUPPORTED.  A buffer smaller than
 * lightning_attn_saved_size returns LA_ERR_WORKSPACE_TOO_SMALL; a null one
 * LA_ERR_NULL_POINTER.  Other arguments, workspaces and errors as for
 * lightning_attn_prefill(_varlen) and lightning_attn_backward(_varlen).
 */
LA_API size_t lightning_attn_saved_size(int64_t total_tokens, int nseq, int heads, int head_dim,
                                        int block, int chunk_tokens, la_dtype dtype);
LA_API la_status lightning_attn_prefill_save(const void* q, const void* k, const void* v,
                                             const void* gate, const void* norm_weight, void* out,
                                             const float* initial_state, float* final_state,
                                             int batch, int64_t seqlen, int heads, int head_dim,
                                             int block, int chunk_tokens, float eps,
                                             la_dtype dtype, void* saved, size_t saved_bytes,
                                             void* workspace, size_t workspace_bytes,
                                             hipStream_t stream);
LA_API la_status lightning_attn_prefill_varlen_save(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    void* out, const int32_t* cu_seqlens, int nseq, int64_t total_tokens,
    const float* initial_state, float* final_state, int heads, int head_dim, int block,
    int chunk_tokens, float eps, la_dtype dtype, void* saved, size_t saved_bytes,
    void* workspace, size_t workspace_bytes, hipStream_t stream);
LA_API la_status lightning_attn_backward_saved(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    const void* dout, const float* initial_state, const float* d_final_state, void* dq, void* dk,
    void* dv, void* dgate, float* dweight, float* d_initial_state, int batch, int64_t seqlen,
    int heads, int head_dim, int block, int chunk_tokens, float eps, la_dtype dtype,
    const void* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
    hipStream_t stream);
LA_API la_status lightning_attn_backward_varlen_saved(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    const void* dout, const int32_t* cu_seqlens, int nseq, int64_t total_tokens,
    const float* initial_state, const float* d_final_state, void* dq, void* dk, void* dv,
    void* dgate, float* dweight, float* d_initial_state, int heads, int head_dim, int block,
    int chunk_tokens, float eps, la_dtype dtype, const void* saved, size_t saved_bytes,
    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The whole layer on a batch of B rows of N tokens, with the projections on
 * either side of the attention (Mechanism step 1: q, k, v and the gate are
 * linear maps of the layer input; the output is mapped back to the hidden
 * size):
 *     q~, k~, v~ = SiLU(x Wq), SiLU(x Wk), SiLU(x Wv);  g = x Wg
 *     out        = (RMSNorm(q~ S) * w * sigmoid(g)) Wo  (as lightning_attn_prefill)
 * The four input projections and the output projection are bf16 GEMMs with
 * fp32 accumulation; `gemm` picks the kernels:
 *   LA_GEMM_MFMA       the library's bf16 MFMA GEMM: the four input
 *                      projections in one launch, SiLU on q, k, v and the
 *                      logistic function on the gate applied to the fp32
 *                      accumulators before the one rounding to bf16 (the
 *                      attention then reads activated operands and multiplies
 *                      by the stored sigmoid(gate)); then the output GEMM.
 *                      Needs hidden % 64 == 0.
 *   LA_GEMM_HIPBLASLT  hipBLASLt, one call per projection, SiLU in the q, k, v
 *                      epilogues, the gate's sigmoid applied by the attention
 *                      (as in lightning_attn_prefill); the baseline.
 *   x:           [batch][seqlen][hidden] bf16
 *   w_qkvg:      [4][hidden][heads*head_dim] bf16 (Wq, Wk, Wv, Wg; y = x W)
 *   norm_weight: [heads*head_dim] bf16
 *   w_out:       [heads*head_dim][hidden] bf16
 *   out:         [batch][seqlen][hidden] bf16
 *   initial_state / final_state: as for lightning_attn_prefill
 * bf16 only, head_dim 128, and heads at most the device's compute units (the
 * attention runs the fused MFMA walk; LA_ERR_UNSUPPORTED and a workspace size
 * of 0 otherwise).  With LA_GEMM_HIPBLASLT the first call on a device
 * creates that device's hipBLASLt handle, and each shape's matmul
 * description and chosen algorithm are kept, until the process ends; the
 * hipBLASLt GEMMs use a slice of the caller's workspace.
 */
LA_API size_t lightning_attn_layer_workspace_size(int64_t total_tokens, int nseq, int hidden,
                                                  int heads, int head_dim);
LA_API la_status lightning_attn_layer_prefill(const void* x, const void* w_qkvg,
                                              const void* norm_weight, const void* w_out,
                                              void* out, const float* initial_state,
                                              float* final_state, int batch, int64_t seqlen,
                                              int hidden, int heads, int head_dim, la_gemm gemm,
                                              float eps, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream);

/*
 * The hybrid's softmax attention layer (one after every seven Lightning
 * layers: "Diving into MiniMax01 405B MoE", section "Hybrid Modeling", 1/8
 * Softmax Attention; the model card, "2. Model Architecture", Positional
 * Encoding: rotary embedding on half of the head dimension, base frequency
 * 10,000,000).  Per sequence and head, with pos counted from 0 in every
 * sequence:
 *     q^_t = rope(q_t, t), k^_u = rope(k_u, u): features (2i, 2i+1), i <
 *            rope_dim / 2, turned by the angle pos * rope_base^(-2i / rope_dim);
 *            features >= rope_dim unchanged
 *     out_t = sum_{u <= t} softmax_u(scale * <q^_t, k^_u>) v_u      (causal)
 * as many key/value heads as query heads.
 *   q, k, v, out: [batch][seqlen][heads][head_dim] bf16, or packed
 *                 [total_tokens][heads][head_dim] with device cu_seqlens int32
 *                 [nseq+1] (as for lightning_attn_prefill_varlen)
 *   rope_dim:     rotated features, a multiple of 8 in 0..head_dim (the model:
 *                 head_dim / 2 = 64); rope_base > 0 (the model: 1e7)
 *   scale:        logit scale > 0 (usually 1 / sqrt(head_dim))
 * bf16 and head_dim 128 only (LA_ERR_UNSUPPORTED otherwise).  The workspace
 * holds the query-tile plan and, when rope_dim > 0, the rotated k
 * (total_tokens x heads x head_dim bf16).
 */
LA_API size_t lightning_attn_softmax_workspace_size(int64_t total_tokens, int nseq, int heads,
                                                    int head_dim, int rope_dim);
LA_API la_status lightning_attn_softmax_prefill(const void* q, const void* k, const void* v,
                                                void* out, int batch, int64_t seqlen, int heads,
                                                int head_dim, int rope_dim, double rope_base,
                                                float scale, la_dtype dtype, void* workspace,
                                                size_t workspace_bytes, hipStream_t stream);
LA_API la_status lightning_attn_softmax_prefill_varlen(
    const void* q, const void* k, const void* v, void* out, const int32_t* cu_seqlens, int nseq,
    int64_t total_tokens, int heads, int head_dim, int rope_dim, double rope_base, float scale,
    la_dtype dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step of the softmax layer against a KV cache (cached generation:
 * each new token attends over the keys and values of the tokens before it).
 * For every sequence s with L = cache_len[s] tokens cached:
 *     k_cache[s][L] = rope(k[s], L), v_cache[s][L] = v[s]      (appended)
 *     out[s] = sum_{u <= L} softmax_u(scale <rope(q[s], L), k_cache[s][u]>) v_cache[s][u]
 * with rope and scale as for lightning_attn_softmax_prefill (the cache holds
 * rotated keys, rounded to bf16).  cache_len is not changed: the caller
 * advances it (L + 1) before the next step.
 *   q, k, v, out:     [nseq][heads][head_dim] bf16, the new token of each sequence
 *   k_cache, v_cache: [nseq][heads][max_len][head_dim] bf16 (head-major: the keys of
 *                     one sequence and head are contiguous), updated in place at slot L
 *   cache_len:        device int32 [nseq]; each 0 <= L < max_len.  A sequence whose L
 *                     is outside that range is skipped (its cache and out are left
 *                     untouched) and marked 1 in the workspace's first nseq int32
 *                     words (0 for the others), written on every call.
 * bf16 and head_dim 128 only.  Work: the cached keys and values are read once
 * (split over ranges of 768 keys, then combined).
 */
LA_API size_t lightning_attn_softmax_decode_workspace_size(int nseq, int max_len, int heads,
                                                           int head_dim);
LA_API la_status lightning_attn_softmax_decode(const void* q, const void* k, const void* v,
                                               void* k_cache, void* v_cache,
                                               const int32_t* cache_len, void* out, int nseq,
                                               int max_len, int heads, int head_dim, int rope_dim,
                                               double rope_base, float scale, la_dtype dtype,
                                               void* workspace, size_t workspace_bytes,
                                               hipStream_t stream);

/* Workspace bytes needed by lightning_attn_decode. */
LA_API size_t lightning_attn_decode_workspace_size(int nseq, int heads, int head_dim);

/*
 * One decode step: each of `nseq` sequences receives one token; its state is
 * read, updated in place (S += k~^T v~) and used for y = q~ S (the new token
 * included), then out = RMSNorm(y) * w * sigmoid(gate) over the heads*head_dim
 * values of the token.
 *   q, k, v, gate, out: [nseq][heads][head_dim]
 *   state:              [nseq][heads][head_dim][head_dim] fp32, updated in place
 */
LA_API la_status lightning_attn_decode(const void* q, const void* k, const void* v, const void* gate,
                                const void* norm_weight, void* out, float* state, int nseq,
                                int heads, int head_dim, float eps, la_dtype dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * lightning_attn_decode without a workspace and without any allocation, for
 * callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as lightning_attn_decode.  The
 * two-kernel decode path (fewer sequences than the device has compute units,
 * or heads * head_dim above the per-sequence kernel's LDS limit) keeps y and
 * the per-head sums of squares in a fixed device array of the library, 4 MiB
 * + 64 KiB per GPU, held from the library's load until the process ends:
 * shapes whose lightning_attn_decode_workspace_size exceeds it return
 * LA_ERR_SCRATCH_TOO_SMALL with nothing enqueued (e.g. 128 sequences x 64
 * heads x 128 fit; 255 sequences do not).  The other shapes use no scratch.
 * The array's device address is looked up on the first call on each device.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (concurrent streams, threads) race and must be serialised by the
 * caller.  Nothing is carried from one call to the next.
 */
LA_API la_status lightning_attn_decode_noalloc(const void* q, const void* k, const void* v,
                                               const void* gate, const void* norm_weight,
                                               void* out, float* state, int nseq, int heads,
                                               int head_dim, float eps, la_dtype dtype,
                                               hipStream_t stream);

/*
 * Instrumented variants, for attributing time to the kernels of one call.
 * They behave exactly like lightning_attn_prefill / lightning_attn_decode and
 * additionally record events[0] on `stream` before the first kernel and
 * events[i] after the i-th kernel; the kernels of a call are named by
 * lightning_attn_prefill_stage_name / lightning_attn_decode_stage_name.
 * events: caller-created hipEvent_t handles, n_events >= stage count + 1
 * (LA_ERR_BAD_SHAPE otherwise; NULL events with n_events = 0 records none).
 */
LA_API int lightning_attn_prefill_stage_count(void);
LA_API const char* lightning_attn_prefill_stage_name(int stage); /* NULL if out of range */
LA_API int lightning_attn_decode_stage_count(void);
LA_API const char* lightning_attn_decode_stage_name(int stage);  /* NULL if out of range */

LA_API la_status lightning_attn_prefill_profiled(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    void* out, const float* initial_state, float* final_state, int batch, int64_t seqlen,
    int heads, int head_dim, int block, int chunk_tokens, float eps, la_dtype dtype,
    void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
    int n_events);

LA_API la_status lightning_attn_decode_profiled(
    const void* q, const void* k, const void* v, const void* gate, const void* norm_weight,
    void* out, float* state, int nseq, int heads, int head_dim, float eps, la_dtype dtype,
    void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events,
    int n_events);

#ifdef __cplusplus
}
#endif

#endif /* LIGHTNING_ATTN_H */
