/*
 * rel_attn.h - C ABI of librelattn.so: paged, variable-length, grouped-query
 * attention with a per-token relative-position bias, for AMD Instinct MI355X
 * (gfx950).
 *
 * The operation is the one documented for `inkling_fa4_rel_attention`
 * (docs.vllm.ai API page of `vllm.models.inkling.nvidia.ops.fa4_rel_attention`,
 * signature and docstring), with the bias rule of the `score_mod_rel_bias`
 * device function (prhub.com.cn report on vLLM PR #48858, "key source
 * snippets"):
 *
 *   request b owns packed query rows t = cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   (S_b of them) and L_b = cache_seqlens[b] keys; query i of the request sits
 *   at absolute position p = i + L_b - S_b; logical key j lives at
 *   cache[block_table[b][j / block_size]][j % block_size][kv_head];
 *   query head h reads KV head h / (num_heads / num_kv_heads);
 *   score(j) = softmax_scale * <q[t][h], k_j> + bias, where
 *   bias = rel_logits[t][h][p - j] if 0 <= p - j < rel_extent, else 0;
 *   visible keys: j < L_b, j <= p if causal, p - window_left <= j <= p +
 *   window_right for each window side that is >= 0 ((-1,-1) = no window);
 *   out[t][h] = softmax over the visible keys applied to their V rows
 *   (zeros if no key is visible).
 *
 * All tensors are dense, row-major and contiguous, and live in device memory
 * owned by the caller; the library keeps no pointer after a call returns.
 * Calls are asynchronous on the given HIP stream, never synchronise the host,
 * never allocate and never read device data on the host, so they can be
 * captured in a HIP graph.
 */
#ifndef REL_ATTN_H
#define REL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types (q, key_cache, value_cache, rel_logits and out share one) */
#define REL_ATTN_FP32 0
#define REL_ATTN_BF16 1

/* return codes */
#define REL_ATTN_OK 0
#define REL_ATTN_EINVAL (-1)        /* NULL pointer, negative size, heads not divisible, ... */
#define REL_ATTN_EUNSUPPORTED (-2)  /* dtype / head_dim / block_size outside the supported set */
#define REL_ATTN_EWORKSPACE (-3)    /* workspace missing or too small for num_splits > 1 */
#define REL_ATTN_ELAUNCH (-4)       /* the HIP runtime rejected a kernel launch */

/*
 * rel_attn_num_splits - how many pieces to cut each request's key range into
 * (split-KV), for a call with the given shape.
 *
 * Same inputs as `inkling_fa4_num_splits` (docs.vllm.ai, same module); local
 * (sliding-window) calls are not split, as on that page. The constants are
 * chosen for 256 compute units:
 *   - decode-shaped calls (max_query_len * num_heads / num_kv_heads <= 16):
 *     the decode kernel shares the batch's keys evenly among one round of
 *     workgroups (4 or 8 KV heads each) and cuts a request into at most this many
 *     pieces; the count leaves room for requests of unequal length, and
 *     pieces hold at least 256 keys (max_kv_len / 256 + 1 at most);
 *   - other calls: work units (requests x KV heads x 64-row query tiles)
 *     are split until the launch has about 1024 workgroups, keeping at
 *     least 256 keys per split.
 * A call with one split still spreads a decode-shaped request's keys over
 * the device: with fewer than 1024 (request, KV head) pairs, the waves of
 * one workgroup per pair share its key range and merge in LDS.
 *
 * is_local:      non-zero when either window side is >= 0.
 * batch_size:    number of requests (>= 1).
 * max_query_len: longest query length in the batch (>= 1).
 * num_heads, num_kv_heads: query / KV heads; num_heads % num_kv_heads == 0.
 * max_kv_len:    longest KV length in the batch (>= 0).
 *
 * Returns a split count in [1, 512], or REL_ATTN_EINVAL. Host only; touches
 * no device.
 */
int rel_attn_num_splits(int is_local, int batch_size, int max_query_len, int num_heads,
                        int num_kv_heads, int max_kv_len);

/*
 * rel_attn_workspace_bytes - size of the fp32 split-KV workspace that
 * rel_attn_fwd needs: num_splits * num_tokens * num_heads * (head_dim + 1) * 4
 * bytes when num_splits > 1, else 0. Returns 0 for invalid arguments, and
 * SIZE_MAX when the size does not fit in size_t (no workspace is then
 * accepted: the calls return REL_ATTN_EWORKSPACE).
 */
size_t rel_attn_workspace_bytes(int num_splits, int num_tokens, int num_heads, int head_dim);

/*
 * rel_attn_fwd - one attention call (the docs.vllm.ai `inkling_fa4_rel_attention`
 * operation with return_lse=False; `out` is the output tensor).
 *
 * Device pointers (caller-owned, contiguous):
 *   q            [num_tokens][num_heads][head_dim]                    dtype
 *   key_cache    [num_blocks][block_size][num_kv_heads][head_dim]      dtype
 *   value_cache  [num_blocks][block_size][num_kv_heads][head_dim]      dtype
 *   block_table  [batch_size][max_blocks_per_seq]                      int32
 *                entries 0 .. ceil(L_b / block_size)-1 must be page ids in
 *                [0, num_blocks); later entries are never read.
 *   cache_seqlens [batch_size]                                         int32 (L_b)
 *   cu_seqlens_q [batch_size + 1], cu_seqlens_q[0] = 0,
 *                cu_seqlens_q[batch_size] = num_tokens                 int32
 *   rel_logits   [num_tokens][num_heads][rel_extent]                   dtype
 *                (may be NULL when rel_extent == 0)
 *   out          [num_tokens][num_heads][head_dim]                     dtype (written)
 *   workspace    >= rel_attn_workspace_bytes(num_splits, ...) bytes of device
 *                memory, 16-byte aligned; only needed when num_splits > 1. Its
 *                contents are scratch (not kept between calls).
 *
 * Scalars:
 *   dtype        REL_ATTN_FP32 or REL_ATTN_BF16.
 *   max_seqlen_q upper bound on every S_b (any bound >= the true maximum, e.g.
 *                a power of two, is valid; it only sizes the launch grid).
 *   head_dim     64 or 128.
 *   block_size   any value >= 1.
 *   num_heads    multiple of num_kv_heads; num_heads / num_kv_heads <= 16.
 *   rel_extent   >= 0; 0 means no bias.
 *   softmax_scale multiplies q.k (the bias is added unscaled).
 *   causal       0 or 1; window_left / window_right: -1 = unbounded side.
 *   num_splits   1..512: the key range of a query tile (of a request, in
 *                decode-shaped calls) is cut into at most this many pieces
 *                whose partial results are merged with log-sum-exp. The
 *                result does not depend on it beyond rounding.
 *   stream       hipStream_t to enqueue on (NULL = default stream).
 *
 * Workspace query: with workspace == NULL and workspace_needed != NULL the
 * call stores the required size in *workspace_needed and returns 0 without
 * launching anything. Otherwise, when workspace_needed != NULL, the required
 * size is stored there as well.
 *
 * Errors: every argument check runs on the host before any launch, and a
 * failed check launches nothing. Device data is not validated (that would
 * need a host synchronisation): a page id outside [0, num_blocks) is clamped
 * into range, and a request with L_b < S_b yields zeros for the rows whose
 * position is negative.
 * Returns REL_ATTN_OK, or one of the negative codes above.
 *
 * It is rel_attn_fwd_splits followed, when num_splits > 1, by
 * rel_attn_combine on the same stream.
 */
int rel_attn_fwd(const void* q, const void* key_cache, const void* value_cache,
                 const int32_t* block_table, const int32_t* cache_seqlens,
                 const int32_t* cu_seqlens_q, const void* rel_logits, void* out, int dtype,
                 int num_tokens, int batch_size, int max_seqlen_q, int max_blocks_per_seq,
                 int num_heads, int num_kv_heads, int head_dim, int num_blocks, int block_size,
                 int rel_extent, float softmax_scale, int causal, int window_left,
                 int window_right, int num_splits, void* workspace, size_t workspace_bytes,
                 size_t* workspace_needed, void* stream);

/*
 * rel_attn_fwd_splits - the attention stage of rel_attn_fwd alone: same
 * arguments, same checks, same return codes.
 *
 * With num_splits == 1 it is rel_attn_fwd (the result goes to `out`). With
 * num_splits > 1 it leaves `out` untouched and writes, for every split slot
 * k, token t and head h, the normalised partial output over the keys of
 * piece k and its log-sum-exp into the workspace, laid out as
 *   float o[num_splits][num_tokens][num_heads][head_dim], followed by
 *   float lse[num_splits][num_tokens][num_heads]
 * where lse is the natural-log log-sum-exp of the scores (softmax_scale * q.k
 * + bias) of the piece's visible keys, -inf for a slot with none. Every lse
 * entry is written; o entries of a slot whose lse is -inf are unspecified.
 * rel_attn_combine then produces `out`.
 * This is the split-KV scheme behind the num_splits argument of the
 * docs.vllm.ai `inkling_fa4_rel_attention` / `inkling_fa4_num_splits` pages.
 */
int rel_attn_fwd_splits(const void* q, const void* key_cache, const void* value_cache,
                        const int32_t* block_table, const int32_t* cache_seqlens,
                        const int32_t* cu_seqlens_q, const void* rel_logits, void* out, int dtype,
                        int num_tokens, int batch_size, int max_seqlen_q, int max_blocks_per_seq,
                        int num_heads, int num_kv_heads, int head_dim, int num_blocks,
                        int block_size, int rel_extent, float softmax_scale, int causal,
                        int window_left, int window_right, int num_splits, void* workspace,
                        size_t workspace_bytes, size_t* workspace_needed, void* stream);

/*
 * rel_attn_fwd_lse - rel_attn_fwd that also returns each row's log-sum-exp
 * (the docs.vllm.ai `inkling_fa4_rel_attention` operation with
 * return_lse=True): same arguments plus
 *   lse   [num_tokens][num_heads] float32, device, caller-owned: the natural
 *         log of sum_j exp(softmax_scale * q.k_j + bias_j) over the row's
 *         visible keys, -inf for a row with none.
 * The log-sum-exps come out of the split merge, so the call always runs
 * split: num_splits 1 is taken as 2, and the workspace (and
 * *workspace_needed) are those of rel_attn_workspace_bytes(max(num_splits, 2),
 * ...). Returns what rel_attn_fwd returns; REL_ATTN_EINVAL also for a NULL
 * lse in a call that launches (not for a workspace query or an empty call).
 * Asynchronous; allocates nothing.
 */
int rel_attn_fwd_lse(const void* q, const void* key_cache, const void* value_cache,
                     const int32_t* block_table, const int32_t* cache_seqlens,
                     const int32_t* cu_seqlens_q, const void* rel_logits, void* out, float* lse,
                     int dtype, int num_tokens, int batch_size, int max_seqlen_q,
                     int max_blocks_per_seq, int num_heads, int num_kv_heads, int head_dim,
                     int num_blocks, int block_size, int rel_extent, float softmax_scale,
                     int causal, int window_left, int window_right, int num_splits,
                     void* workspace, size_t workspace_bytes, size_t* workspace_needed,
                     void* stream);

/*
 * rel_attn_fwd_noalloc - rel_attn_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Same arguments as rel_attn_fwd without
 * the three workspace ones; same checks, same return codes, same results.
 *
 * With num_splits > 1 the split partials go to a static device array of
 * rel_attn_noalloc_scratch_bytes() bytes (32 MiB) that the library keeps on
 * every GPU it runs on until the process ends, not to a caller workspace. A
 * call whose workspace (rel_attn_workspace_bytes) exceeds that size returns
 * REL_ATTN_EWORKSPACE and launches nothing. The call never allocates or frees
 * device memory. Every argument check runs before any device is touched.
 *
 * All calls on one GPU share that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero): calls that overlap on one
 * GPU (on different streams, or graphs replayed at the same time) race and
 * give wrong results, so serialise them. The stream must belong to the
 * current device (REL_ATTN_EINVAL otherwise). The first split call on a
 * device looks up the array's address there (hipGetSymbolAddress) and keeps
 * it; make that first call outside graph capture.
 */
int rel_attn_fwd_noalloc(const void* q, const void* key_cache, const void* value_cache,
                         const int32_t* block_table, const int32_t* cache_seqlens,
                         const int32_t* cu_seqlens_q, const void* rel_logits, void* out, int dtype,
                         int num_tokens, int batch_size, int max_seqlen_q, int max_blocks_per_seq,
                         int num_heads, int num_kv_heads, int head_dim, int num_blocks,
                         int block_size, int rel_extent, float softmax_scale, int causal,
                         int window_left, int window_right, int num_splits, void* stream);

/* rel_attn_noalloc_scratch_bytes - size in bytes of the static scratch array
 * of rel_attn_fwd_noalloc (the largest split workspace it accepts). Host only. */
size_t rel_attn_noalloc_scratch_bytes(void);

/*
 * rel_attn_combine - merge the per-split partial results that
 * rel_attn_fwd_splits left in `workspace` (layout above) into `out`
 * [num_tokens][num_heads][head_dim] of type dtype:
 *   out = sum_k exp(lse_k - LSE) * o_k,  LSE = log sum_k exp(lse_k),
 * zeros where every lse_k is -inf.
 *
 * workspace: device memory, >= rel_attn_workspace_bytes(num_splits, ...)
 *            bytes, 16-byte aligned, read only.
 * num_splits: 2..512 (with one split there is nothing to merge).
 * head_dim:  64 or 128. stream: hipStream_t (NULL = default stream).
 * Returns REL_ATTN_OK, REL_ATTN_EINVAL (bad size, NULL out with
 * num_tokens > 0, misaligned workspace), REL_ATTN_EUNSUPPORTED (dtype,
 * head_dim), REL_ATTN_EWORKSPACE (workspace NULL or too small) or
 * REL_ATTN_ELAUNCH. Asynchronous; allocates nothing.
 */
int rel_attn_combine(const void* workspace, size_t workspace_bytes, void* out, int dtype,
                     int num_tokens, int num_heads, int head_dim, int num_splits, void* stream);

/* rel_attn_strerror - static description of a return code (never NULL). */
const char* rel_attn_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* REL_ATTN_H */
