/*
 * libsdpa: exact scaled dot-product attention for AMD MI355X (gfx950): the
 * forward pass (batched, packed variable-length, and against a paged
 * key/value cache) and its gradients (batched and packed).
 *
 * The operation (exactref.ai, "scaled_dot_product_attention", sections
 * "Arguments" and "Full specification"): for query (..., L, E), key (..., S, E)
 * and value (..., S, Ev)
 *
 *     out = softmax(scale * Q K^T + mask) V     over the key axis
 *     lse = log(sum_j exp(scale * q.k_j + mask_j))   per query row
 *
 * with scale = 1/sqrt(E) unless given, the mask added after scaling, a causal
 * option that keeps key j for query i only when j <= i (counted from the
 * top-left corner), and grouped-query heads where query head h reads key/value
 * head h / (Hq / Hkv).  A row with no kept key has output 0 and lse -inf.  The
 * output has the inputs' dtype, rounded to nearest-even; lse is float32.
 *
 * Entry points: sdpa_fwd (+ _workspace_size), sdpa_fwd_noalloc, sdpa_fwd_varlen,
 * sdpa_fwd_paged (+ _workspace_size), sdpa_fwd_paged_varlen, sdpa_bwd
 * (+ _workspace_size), sdpa_bwd_varlen (+ _workspace_size), sdpa_last_error,
 * sdpa_abi_version.
 *
 * Conventions for every entry point
 *  - All data pointers are DEVICE pointers (HIP global memory) owned by the
 *    caller; the library allocates nothing, keeps no state beyond its code
 *    objects and a per-thread error string, and never frees caller memory.
 *  - Sizes and strides are in ELEMENTS.  The last dimension of q, k, v, out and
 *    a mask must have stride 1.  bf16/fp16 tensors need 16-byte aligned base
 *    pointers and row strides that are multiples of 8 elements; fp32 tensors
 *    16-byte aligned bases and row strides that are multiples of 4.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means the
 *    default stream).  Inputs must stay alive and unmodified, and outputs must
 *    not be read, until the stream reaches that point.  out and lse must not
 *    overlap any input.
 *  - Argument errors are detected on the host before anything is enqueued:
 *    the call returns a non-zero status and sdpa_last_error() describes it.
 *    No C++ exception crosses this interface.
 *  - Head dims supported by the kernels: E and Ev each in {64, 96, 128}.
 *    E != Ev (value rows of another width than query/key rows, which the
 *    operation allows) is handled for bf16/fp16 inputs by sdpa_fwd (with or
 *    without attn_mask) and sdpa_fwd_varlen; the paged entry points and the
 *    backward need E == Ev.
 *    sdpa_fwd also takes E == Ev any multiple of 8 from 8 to 128 for
 *    bf16/fp16 inputs without attn_mask (single-pass kernel only).
 *    E = 0 (an empty score sum) is valid for the operation but not handled by
 *    the kernels: it returns SDPA_ERR_UNSUPPORTED.
 */
#ifndef SDPA_H
#define SDPA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SDPA_OK = 0,
    SDPA_ERR_INVALID_ARGUMENT = 1, /* shapes, dropout, GQA ratio, mask, workspace */
    SDPA_ERR_UNSUPPORTED = 2,      /* valid operation outside what the kernels cover */
    SDPA_ERR_DEVICE = 3            /* a HIP runtime error while enqueueing */
} sdpa_status;

typedef enum {
    SDPA_F32 = 0,
    SDPA_F16 = 1,
    SDPA_BF16 = 2,
    SDPA_BOOL = 3 /* one byte per element, non-zero keeps the key */
} sdpa_dtype;

/* A strided 4-D device tensor.  size[] and stride[] are in elements. */
typedef struct {
    void* data;
    int64_t size[4];
    int64_t stride[4];
} sdpa_tensor4;

/*
 * sdpa_fwd -- batched attention forward.
 *
 *   dtype      element type of q, k, v and out: SDPA_BF16, SDPA_F16 or SDPA_F32.
 *   q          (B, Hq,  L, E)
 *   k          (B, Hkv, S, E)
 *   v          (B, Hkv, S, Ev)
 *   attn_mask  NULL, or a (B|1, Hq|1, L|1, S) tensor broadcast over size-1
 *              dims (stride 0 is fine).  mask_dtype SDPA_BOOL: non-zero keeps
 *              the key (False removes it).  mask_dtype SDPA_F32: added to the
 *              scaled scores, -inf removes the key (exactref.ai "Arguments").
 *              The logit is formed as one fp32 fused multiply-add.
 *   dropout_p  must be 0 (a random dropout has no exact reference); any other
 *              value returns SDPA_ERR_INVALID_ARGUMENT.
 *   is_causal  non-zero keeps key j for query i only when j <= i; combined with
 *              attn_mask the kept set is the intersection.
 *   scale      NULL for 1/sqrt(E), else the factor on the scores (any finite
 *              value, negative and 0 included).
 *   enable_gqa non-zero allows Hkv < Hq with Hq % Hkv == 0; query head h then
 *              reads key/value head h / (Hq / Hkv).  Without it Hq == Hkv.
 *   out        (B, Hq, L, Ev), dtype.
 *   lse        (B, Hq, L, 1), float32 (size[3] == 1, stride[3] ignored).
 *   workspace, workspace_bytes
 *              device scratch for the split-KV decode path (partial outputs
 *              and their lse).  Query the size with sdpa_fwd_workspace_size;
 *              may be NULL/0 when that size is 0.
 *   num_splits 0: the library picks the kernel and the split count.
 *              -1: force the single-pass (prefill) kernel.
 *              k >= 1: the split-KV decode kernel with k splits of the keys
 *              (SDPA_ERR_UNSUPPORTED when the call is not eligible for it:
 *              it needs no mask, no causal flag, bf16/fp16 and L*Hq/Hkv <= 16).
 *   stream     hipStream_t or NULL.
 */
sdpa_status sdpa_fwd(sdpa_dtype dtype,
                     const sdpa_tensor4* q, const sdpa_tensor4* k, const sdpa_tensor4* v,
                     const sdpa_tensor4* attn_mask, sdpa_dtype mask_dtype,
                     double dropout_p, int is_causal, const double* scale, int enable_gqa,
                     const sdpa_tensor4* out, const sdpa_tensor4* lse,
                     void* workspace, size_t workspace_bytes, int num_splits,
                     void* stream);

/*
 * sdpa_fwd_workspace_size -- bytes of workspace sdpa_fwd needs for the same
 * arguments (0 when the single-pass kernel is chosen).  Writes *bytes; runs on
 * the host only.
 */
sdpa_status sdpa_fwd_workspace_size(sdpa_dtype dtype,
                                    const sdpa_tensor4* q, const sdpa_tensor4* k,
                                    const sdpa_tensor4* v,
                                    const sdpa_tensor4* attn_mask, int is_causal,
                                    int enable_gqa, int num_splits, size_t* bytes);

/*
 * sdpa_fwd_noalloc -- sdpa_fwd for callers that cannot allocate device memory
 * while they run (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as sdpa_fwd without the
 * workspace: the scratch memory the split-KV decode needs (its per-split
 * partial outputs and logsumexps) comes from a device array inside the
 * library, SDPA_NOALLOC_SCRATCH_BYTES on each device, which the library holds
 * until the process ends.  Nothing is allocated or freed by the call.
 *
 *   - A call whose sdpa_fwd_workspace_size exceeds SDPA_NOALLOC_SCRATCH_BYTES
 *     returns SDPA_ERR_UNSUPPORTED before anything is launched (fewer
 *     num_splits, or sdpa_fwd with a workspace, lift it); for the decode
 *     workload B=64, Hq=32, Hkv=8, S=32768, E=128 the automatic split count
 *     needs about 4.2 MB.
 *   - The array of the device current at the call is used (looked up on the
 *     first call on that device); stream must belong to that device.
 *   - Calls on one device share its array: calls that overlap on one device
 *     (other streams, other threads) race and must be serialised by the
 *     caller.  Each call writes every partial it reads, so nothing carries
 *     over from one call to the next.
 */
#define SDPA_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
sdpa_status sdpa_fwd_noalloc(sdpa_dtype dtype,
                             const sdpa_tensor4* q, const sdpa_tensor4* k, const sdpa_tensor4* v,
                             const sdpa_tensor4* attn_mask, sdpa_dtype mask_dtype,
                             double dropout_p, int is_causal, const double* scale, int enable_gqa,
                             const sdpa_tensor4* out, const sdpa_tensor4* lse, int num_splits,
                             void* stream);

/*
 * sdpa_fwd_varlen -- packed variable-length attention with a block-diagonal
 * mask (insureai360 xFormers tutorial, section 4: BlockDiagonalMask and
 * BlockDiagonalCausalMask over sequences concatenated along the token axis).
 *
 *   q    packed (total_q, Hq,  E): element (t, h, e) at q + t*q_stride_tok + h*q_stride_head + e
 *   k    packed (total_k, Hkv, E)
 *   v    packed (total_k, Hkv, Ev)
 *   cu_seqlens_q, cu_seqlens_k
 *        DEVICE int32 arrays of n_seqs + 1 non-decreasing offsets starting at
 *        0: segment s holds tokens [cu[s], cu[s+1]).  Query segment s attends
 *        only to key segment s; with is_causal, key j of the segment is kept
 *        for query i of the segment when j <= i (local indices).
 *   max_seqlen_q, max_seqlen_k
 *        upper bounds of the segment lengths, which the caller must keep: they
 *        size the launch.  If a segment is longer anyway, its query rows
 *        beyond max_seqlen_q are not computed (left unwritten) and its keys
 *        beyond max_seqlen_k are not attended, in sdpa_fwd_varlen and
 *        sdpa_bwd_varlen alike; offsets are clamped to [0, total] on the
 *        device, so bad offsets never read or write out of bounds.
 *   out  packed (total_q, Hq, Ev), dtype
 *   lse  (Hq, total_q) float32: element (h, t) at lse + h*lse_stride_head + t
 *
 * The other arguments mean what they mean for sdpa_fwd.  Tokens of q outside
 * every segment are left unwritten.
 */
sdpa_status sdpa_fwd_varlen(sdpa_dtype dtype,
                            const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                            const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                            const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int32_t n_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            int32_t Hq, int32_t Hkv, int32_t E, int32_t Ev,
                            int64_t total_q, int64_t total_k,
                            double dropout_p, int is_causal, const double* scale,
                            int enable_gqa,
                            void* out, int64_t o_stride_tok, int64_t o_stride_head,
                            float* lse, int64_t lse_stride_head,
                            void* stream);

/*
 * sdpa_fwd_paged -- attention of new query rows against a paged key/value
 * cache: the cached keys of a sequence live in fixed-size pages of a shared
 * pool, listed in order by the sequence's row of a block table.  This is the
 * serving layout behind the paged KV cache and PagedAttention that the
 * hourtab.com "xFormers developer on retainer" page names in its "Related
 * retainer posts" (FlashInfer, vLLM), where sequences of a batch read pages
 * outside their own allocation; the decode it serves is the memory-bound
 * generation step of the khchao.com NN Lab page, "Arithmetic Intensity of
 * Autoregressive Decoding".  Decode steps (L * Hq / Hkv
 * <= 16 rows per cache head) run the split-KV kernel and its merge; longer
 * chunks of new rows (chunked prefill) run the single-pass kernel, which reads
 * the pages itself and needs no workspace.
 *
 *   dtype       SDPA_BF16 or SDPA_F16.
 *   q           (B, Hq, L, E): the new rows of each sequence (the same L for
 *               every sequence).
 *   k_cache     (n_pages, Hkv, page_size, E), v_cache (n_pages, Hkv, page_size, Ev):
 *               the page pool; page_size a power of two >= 16; E == Ev in
 *               {64, 96, 128}.
 *   block_table DEVICE int32, B rows of bt_stride entries; entry (b, j) is the
 *               page holding keys j*page_size .. (j+1)*page_size - 1 of sequence
 *               b; max_blocks entries per row are valid.
 *   seq_lens    DEVICE int32 (B): keys cached for each sequence (the new rows'
 *               own keys included); clamped to max_seq_len and to
 *               max_blocks * page_size on the device.
 *   max_seq_len host upper bound of seq_lens (sizes the launch).
 *   is_causal   non-zero: new row i (0-based of L) is position n - L + i of its
 *               sequence (n its cached length) and keeps key j iff
 *               j <= n - L + i (bottom-right alignment); with L = 1 it keeps
 *               every cached key.
 *   scale, enable_gqa, out (B, Hq, L, Ev), lse (B, Hq, L, 1) float32,
 *   workspace (size from sdpa_fwd_paged_workspace_size; 0 bytes, and NULL
 *   allowed, for chunked prefill), num_splits (0 auto, k >= 1 splits; only
 *   with L * Hq / Hkv <= 16, else SDPA_ERR_UNSUPPORTED) and stream: as for
 *   sdpa_fwd.
 *
 * A table entry outside [0, n_pages) for a kept key is never dereferenced:
 * the rows that would read it come out NaN (output and lse) instead of
 * silently using other memory.
 */
sdpa_status sdpa_fwd_paged(sdpa_dtype dtype, const sdpa_tensor4* q,
                           const sdpa_tensor4* k_cache, const sdpa_tensor4* v_cache,
                           const int32_t* block_table, int64_t bt_stride, int32_t max_blocks,
                           const int32_t* seq_lens, int32_t max_seq_len,
                           int is_causal, const double* scale, int enable_gqa,
                           const sdpa_tensor4* out, const sdpa_tensor4* lse,
                           void* workspace, size_t workspace_bytes, int num_splits, void* stream);

/* Workspace bytes sdpa_fwd_paged needs for these shapes (host only). */
sdpa_status sdpa_fwd_paged_workspace_size(sdpa_dtype dtype, const sdpa_tensor4* q,
                                          const sdpa_tensor4* k_cache, const sdpa_tensor4* v_cache,
                                          int32_t max_seq_len, int enable_gqa, int num_splits,
                                          size_t* bytes);

/*
 * sdpa_fwd_paged_varlen -- packed new rows of several sequences, each its own
 * number of rows, against the paged cache of sdpa_fwd_paged (chunked prefill
 * of requests with different chunk lengths); no workspace.
 *
 *   dtype       SDPA_BF16 or SDPA_F16.
 *   q           packed (total_q, Hq, E), token and head strides in elements
 *               (multiples of 8, unit last stride, 16-byte aligned base);
 *               sequence b's rows are tokens cu_seqlens_q[b] ..
 *               cu_seqlens_q[b + 1] - 1 (DEVICE int32, n_seqs + 1 offsets;
 *               max_seqlen_q must bound every count).
 *   k_cache, v_cache, block_table, bt_stride, max_blocks, seq_lens,
 *   max_seq_len  as for sdpa_fwd_paged (one table row and one length per
 *               sequence); E == Ev in {64, 96, 128}.
 *   is_causal   row r of sequence b is position n_b - L_b + r of it (L_b its
 *               row count, n_b its cached length) and keeps key j iff
 *               j <= n_b - L_b + r.
 *   scale, enable_gqa   as for sdpa_fwd.
 *   out         packed (total_q, Hq, Ev) with token and head strides; lse
 *               (Hq, total_q) float32 with head stride lse_stride_head.
 *               Tokens outside every sequence are not written.
 * Table entries outside the pool: as for sdpa_fwd_paged (the rows that keep
 * such a key come out NaN).
 */
sdpa_status sdpa_fwd_paged_varlen(sdpa_dtype dtype, const void* q, int64_t q_stride_tok,
                                  int64_t q_stride_head, const int32_t* cu_seqlens_q, int32_t n_seqs,
                                  int32_t max_seqlen_q, int64_t total_q, int32_t Hq,
                                  const sdpa_tensor4* k_cache, const sdpa_tensor4* v_cache,
                                  const int32_t* block_table, int64_t bt_stride, int32_t max_blocks,
                                  const int32_t* seq_lens, int32_t max_seq_len, int is_causal,
                                  const double* scale, int enable_gqa, void* out, int64_t o_stride_tok,
                                  int64_t o_stride_head, float* lse, int64_t lse_stride_head, void* stream);

/*
 * sdpa_bwd -- gradients of batched attention (exactref.ai
 * "scaled_dot_product_attention.backward").  With P the attention weights of
 * the forward, dP = dout V^T, D_i = sum_j P_ij dP_ij and dS = P * (dP - D):
 *
 *     dv = P^T dout,   dq = scale * dS K,   dk = scale * dS^T Q,
 *
 * dk and dv summed over the query heads that share a key/value head.  P is
 * recomputed from q, k and the forward's lse; D from the forward output
 * (D_i = dout_i . out_i, the definition's sum up to the rounding of out).
 *
 *   dtype      SDPA_BF16, SDPA_F16 or SDPA_F32.
 *   q, k, v    as for sdpa_fwd (head dims E and Ev multiples of 8 up to 128).
 *              bf16/fp16 with E == Ev in {64, 96, 128} run the matrix-core
 *              kernels; every other call the vector-ALU ones (fp32 arithmetic).
 *   attn_mask, mask_dtype
 *              as for sdpa_fwd (NULL, or a float32 bias / bool keep mask
 *              broadcastable to (B, Hq, L, S), key stride 1).  The mask gets
 *              no gradient.
 *   out, lse   the results of sdpa_fwd for the same q, k, v, attn_mask,
 *              is_causal, scale and enable_gqa: out (B, Hq, L, Ev) dtype,
 *              lse (B, Hq, L, 1) float32.  A row with no kept key (lse -inf)
 *              contributes nothing.
 *   dout       (B, Hq, L, Ev), dtype: gradient of the loss with respect to out.
 *   is_causal, scale, enable_gqa   as for sdpa_fwd.
 *   dq         (B, Hq, L, E), dk (B, Hkv, S, E), dv (B, Hkv, S, Ev), dtype;
 *              written completely (rows no query reaches get 0), rounded to
 *              nearest-even.  They must not alias any input.
 *   workspace, workspace_bytes
 *              device scratch owned by the caller, of at least
 *              B * Hq * L * 4 + 256 bytes (the per-row D in float32).  With
 *              sdpa_bwd_workspace_size() bytes, where that size also holds a
 *              16-bit dS^T of B * Hq * S * (L rounded up to 128) elements
 *              (matrix-core calls, at most 2 GiB of it), the dK/dV kernel
 *              stores dS and dq = scale dS K takes one matrix product per
 *              (query, key) pair; with less, dq recomputes S and dP (three
 *              products).  Both give the same values.
 *   stream     hipStream_t or NULL; the call is asynchronous on it.
 *
 * Errors as for sdpa_fwd: argument problems are found on the host before any
 * launch; every tensor needs unit last stride, a 16-byte aligned base and
 * strides that are multiples of 16 bytes (else SDPA_ERR_UNSUPPORTED).
 */
sdpa_status sdpa_bwd(sdpa_dtype dtype,
                     const sdpa_tensor4* q, const sdpa_tensor4* k, const sdpa_tensor4* v,
                     const sdpa_tensor4* attn_mask, sdpa_dtype mask_dtype,
                     const sdpa_tensor4* out, const sdpa_tensor4* lse, const sdpa_tensor4* dout,
                     int is_causal, const double* scale, int enable_gqa,
                     const sdpa_tensor4* dq, const sdpa_tensor4* dk, const sdpa_tensor4* dv,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_bwd_varlen -- gradients of packed variable-length attention (the
 * block-diagonal mask of sdpa_fwd_varlen), as sdpa_bwd computes them for each
 * segment on its own.
 *
 *   q, k, v, out, dout  packed (total, heads, head dim) tensors of dtype
 *               (SDPA_BF16 or SDPA_F16) with token and head strides in
 *               elements (multiples of 8, unit last stride, 16-byte aligned):
 *               q, out, dout over total_q tokens and Hq heads, k, v over
 *               total_k tokens and Hkv heads; out and lse from sdpa_fwd_varlen
 *               with the same arguments; lse (Hq, total_q) float32 with head
 *               stride lse_stride_head.
 *   cu_seqlens_q, cu_seqlens_k, n_seqs, max_seqlen_q, max_seqlen_k, Hq, Hkv,
 *   E, Ev, total_q, total_k, is_causal, scale, enable_gqa
 *               as for sdpa_fwd_varlen (DEVICE offsets; the maxima must bound
 *               every segment's length: longer segments are cut to them);
 *               E == Ev in {64, 96, 128}.
 *   dq (total_q, Hq, E), dk (total_k, Hkv, E), dv (total_k, Hkv, Ev)
 *               written for every token of a segment (tokens outside all
 *               segments are not written); dk, dv summed over the query heads
 *               of each key/value head.  They must not alias any input.
 *   workspace   at least Hq * total_q * 4 + 256 bytes
 *               (sdpa_bwd_varlen_workspace_size), owned by the caller.
 */
sdpa_status sdpa_bwd_varlen(sdpa_dtype dtype, const void* q, int64_t q_stride_tok, int64_t q_stride_head,
                            const void* k, int64_t k_stride_tok, int64_t k_stride_head,
                            const void* v, int64_t v_stride_tok, int64_t v_stride_head,
                            const void* out, int64_t o_stride_tok, int64_t o_stride_head,
                            const float* lse, int64_t lse_stride_head,
                            const void* dout, int64_t do_stride_tok, int64_t do_stride_head,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t n_seqs,
                            int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv,
                            int32_t E, int32_t Ev, int64_t total_q, int64_t total_k, int is_causal,
                            const double* scale, int enable_gqa,
                            void* dq, int64_t dq_stride_tok, int64_t dq_stride_head,
                            void* dk, int64_t dk_stride_tok, int64_t dk_stride_head,
                            void* dv, int64_t dv_stride_tok, int64_t dv_stride_head,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes sdpa_bwd_varlen needs (Hq * total_q float32 values plus
 * alignment).  Host only. */
sdpa_status sdpa_bwd_varlen_workspace_size(int32_t Hq, int64_t total_q, size_t* bytes);

/*
 * sdpa_bwd_workspace_size -- bytes of workspace for sdpa_bwd's faster
 * schedule on these shapes: B * Hq * L float32 values plus alignment, and for
 * matrix-core calls whose dS^T takes at most 2 GiB, that dS^T buffer too
 * (sdpa_bwd runs the recomputing schedule when given less, down to
 * B * Hq * L * 4 + 256 bytes).  Host only.
 */
sdpa_status sdpa_bwd_workspace_size(sdpa_dtype dtype,
                                    const sdpa_tensor4* q, const sdpa_tensor4* k,
                                    const sdpa_tensor4* v, int enable_gqa, size_t* bytes);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* sdpa_last_error(void);

/* Interface version, bumped when a signature or a meaning above changes (5:
 * sdpa_fwd_noalloc; head dims 0..128 in steps of 8 and Ev != E on every path;
 * fp32 gradients). */
int sdpa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_H */
