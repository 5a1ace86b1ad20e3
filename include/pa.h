/*
 * pa.h - C ABI of the MI355X (gfx950) paged KV-cache varlen attention library
 * (libpa.so).
 *
 * The library implements the per-layer attention step of a paged KV cache:
 *
 *   pa_write_kv  scatter this step's new K/V rows into their physical slots of
 *                one global pool of 16-token blocks;
 *   pa_attend    varlen causal attention of every query token of a mixed batch
 *                (chunked-prefill chunks and single-token decodes together, one
 *                call) over each request's cached + new tokens, read through
 *                its block table;
 *   pa_write_kv_plan  the scatter and attention's work plan of a step in one
 *                launch (then pa_attend_planned + pa_attend_merge per layer).
 *
 * Where the operations are defined:
 *   - "vLLM v1 Deep Dive" (supercharleszhu.github.io), Part 3 Runtime, Aside "KV
 *     cache and prefix caching": the pool of fixed-size blocks; slot_mapping
 *     gives, per new token of the flattened batch, the slot
 *     block_id * block_size + offset that its K/V is written to; attention
 *     takes the per-request block tables, seq_lens and query_start_loc and,
 *     in one launch, gives a prefill query a causal mask over its cached
 *     prefix + new tokens and a decode query all of its blocks.
 *   - Same page, Step 4c "Mixed batches": query_start_loc is the prefix sum of
 *     per-request scheduled token counts over the flattened batch.
 *   - "vLLM: An Exhaustive Technical Study for Kernel Engineers" (anthony-chaudhary.github.io) section 2.1: the
 *     block table maps logical block index to physical block id; the write
 *     slot is block number * block_size + block offset.  Section 2.4: query
 *     heads that share one KV head are processed together (GQA).
 *   - "Inside the vLLM Engine" (rohitghumare.com), "A memory problem wearing a
 *     throughput costume": 16-token blocks, ceil(N/16) blocks for N tokens.
 *
 * Semantics (readings where the pages are silent):
 *   - Attention of query token t (head h) of request b is
 *       out = sum_j softmax_j(scale * q.K_j) V_j   over keys j = 0 .. p,
 *     where seq_lens[b] = L counts cached + new tokens, the request's
 *     Q = query_start_loc[b+1] - query_start_loc[b] new tokens are its last Q
 *     positions, and query i of the request sits at p = L - Q + i.
 *   - Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   - pa_write_kv is called before pa_attend for the same step, so the new
 *     tokens' K/V are in the pool when attention reads them.
 *
 * Data types: q, k, v, out and the pools are bf16 (IEEE binary32 truncated to
 * its upper 16 bits).  Attention computes in fp32 with bf16 MFMA operands and
 * rounds the output to bf16 (nearest even).
 *
 * KV pool layout (the pages leave it open; this library fixes it):
 *   k_cache and v_cache are two separate arrays of
 *     num_blocks x num_kv_heads tiles, each tile 16 * head_dim bf16;
 *   tile (block n, kv head g) starts at element (n * num_kv_heads + g) * 16 * D.
 *   Inside a tile, for token slot t in [0,16) and dim d in [0,D), H = D/2:
 *     K(t, d) is at ((d / 8) * 16 + t) * 8 + d % 8
 *     V(t, d) is at ((((d % H) / 16 * 2 + d / H) * 4 + t / 4) * 16 + d % 16)
 *                   * 4 + t % 4
 *   (K: 8-dim chunks of all 16 tokens; V: runs of 4 consecutive tokens of
 *   one dim, 64 runs - 16 dims x 4 token groups - per 512-byte region.)
 *   Only pa_write_kv, pa_attend and pa_gather_kv are meant to touch the
 *   pools.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE memory that the caller allocates, owns
 *     and keeps alive until the call's work on `stream` has finished.  The
 *     library never allocates, frees or keeps pointers across calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     pa_write_kv, pa_attend and pa_gather_kv only enqueue work: no host
 *     synchronisation, no device allocation.
 *   - Host-side argument errors (NULL pointer, negative size, unsupported
 *     head_dim / block shape, num_q_heads not a multiple of num_kv_heads, too
 *     small workspace) are detected before anything is enqueued and returned
 *     as a pa_status; pa_last_error() then holds a message.
 *   - Metadata CONTENT (block ids, slots, lengths) is not checked on the fast
 *     path: invalid content is a caller error whose output is undefined.  The
 *     kernels still never read or write outside the buffers whose sizes they
 *     are given (out-of-range block ids and slots are clamped or skipped, and
 *     requests with inconsistent lengths are skipped).  pa_validate_metadata
 *     reports such content errors.
 *   - Launch failures return PA_ERR_HIP with the HIP error text in
 *     pa_last_error().
 *   - Thread safety: the library holds no mutable global state except a
 *     per-device cache of the compute-unit count and the thread-local error
 *     string; calls from several host threads are safe.  Calls that share a
 *     workspace must be ordered on one stream.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1
#define PA_BLOCK_SIZE 16

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL                    */
  PA_ERR_SHAPE = 2,       /* a size is negative or sizes are inconsistent  */
  PA_ERR_UNSUPPORTED = 3, /* head_dim not 64/128, group size > 16, ...     */
  PA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required    */
  PA_ERR_METADATA = 5,    /* pa_validate_metadata found invalid content    */
  PA_ERR_HIP = 6          /* a HIP runtime call or launch failed           */
} pa_status;

/* Library ABI version (PA_ABI_VERSION). */
int pa_abi_version(void);

/* Static text for a status code. */
const char *pa_status_string(int status);

/* Message of the last failed call on this host thread ("" if none). */
const char *pa_last_error(void);

/*
 * pa_write_kv - scatter new K/V rows into the pool ("reshape and cache").
 *
 * For every token i in [0, num_tokens) with s = slot_mapping[i] >= 0:
 *   for every kv head g and dim d,
 *     K(block s/16, head g, slot s%16, d) = k[i*k_token_stride + g*D + d]
 *     V(block s/16, head g, slot s%16, d) = v[i*v_token_stride + g*D + d]
 * as exact bit copies.  Tokens with s < 0 are skipped (padding); slots
 * >= num_blocks*16 are skipped too (caller error).  Two tokens with the same
 * slot race (caller error).  Every other pool element is left unchanged.
 *
 *   k, v            device bf16, row i at k + i*k_token_stride (elements),
 *                   num_kv_heads*head_dim contiguous elements per row
 *   k_token_stride, v_token_stride   >= num_kv_heads*head_dim
 *   slot_mapping    device int64 [num_tokens]
 *   k_cache, v_cache device bf16 pools, num_blocks tiles per kv head (layout
 *                   above)
 *   head_dim        64 or 128
 *
 * Source: "vLLM v1 Deep Dive", Aside "KV cache and prefix caching" (slot_mapping,
 * the phase-agnostic scatter); "vLLM: An Exhaustive Technical Study" section 2.1.
 */
pa_status pa_write_kv(const void *k, const void *v, int64_t k_token_stride,
                      int64_t v_token_stride, const int64_t *slot_mapping,
                      int64_t num_tokens, int32_t num_kv_heads,
                      int32_t head_dim, void *k_cache, void *v_cache,
                      int64_t num_blocks, void *stream);

/*
 * pa_write_kv_fp8 - pa_write_kv into 8-bit pools (fp8 E4M3 KV cache).
 *
 * Same slots, skips and races as pa_write_kv; each element x (bf16, widened
 * exactly to fp32) is stored as the E4M3 code of the fp32 quotient
 * x / k_scale (x / v_scale for V): round to nearest, ties to the even
 * mantissa; magnitudes at or above 448 and infinities saturate to +-448;
 * NaN -> 0x7f.  E4M3 is the OCP 8-bit format (sign, 4 exponent bits with
 * bias 7, 3 mantissa bits, no infinities, S.1111.111 = NaN), the one gfx950
 * converts in hardware.  A code stands for decode(code) * scale.
 *
 *   k_cache, v_cache device uint8 pools of num_blocks * num_kv_heads tiles,
 *                   each 16 * head_dim bytes; tile (n, g) at byte
 *                   (n * num_kv_heads + g) * 16 * D, and inside it, H = D/2:
 *     K(t, d), d = 32c + 8q + j, c = 2p + h:     ((p*4 + q)*16 + t)*16 + h*8 + j
 *     V(t, d), d = dh*H + 16c + r, c = 2p + cc:  ((p*4 + t/4)*16 + r)*16
 *                                                 + (2cc + dh)*4 + t%4
 *   k_scale, v_scale one fp32 scale per pool, finite and > 0 (PA_ERR_SHAPE
 *                   otherwise)
 *   other arguments as for pa_write_kv.
 *
 * Source: "vLLM: An Exhaustive Technical Study", section 2.8 (the KV-cache
 * quantisation axis: fp8 E4M3 with an fp32 scale per tensor), with the slot
 * semantics of pa_write_kv.
 */
pa_status pa_write_kv_fp8(const void *k, const void *v, int64_t k_token_stride,
                          int64_t v_token_stride, const int64_t *slot_mapping,
                          int64_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, float k_scale, float v_scale,
                          void *k_cache, void *v_cache, int64_t num_blocks,
                          void *stream);

/*
 * pa_attend_workspace_size - bytes of device workspace pa_attend needs for a
 * batch within these bounds (work list, per-token split records and split-K
 * partial results).  Returns 0 for invalid arguments.
 */
size_t pa_attend_workspace_size(int32_t num_seqs, int64_t num_q_tokens,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_query_len,
                                int32_t max_seq_len);

/*
 * pa_attend - paged varlen causal attention over a mixed batch.
 *
 *   q                device bf16 [num_q_tokens][num_q_heads][head_dim],
 *                    rows of request b at query_start_loc[b] ..
 *                    query_start_loc[b+1]-1
 *   k_cache, v_cache device bf16 pools (layout above), num_blocks blocks;
 *                    num_blocks * num_kv_heads < 2^32 (PA_ERR_SHAPE otherwise)
 *   block_tables     device int32 [num_seqs][max_blocks_per_seq]; entry j of
 *                    row b is the physical block of logical tokens
 *                    16j .. 16j+15 of request b; entries past ceil(L_b/16) are
 *                    never read.  Several rows may name the same block
 *                    (shared prefix blocks are read-only here).
 *   seq_lens         device int32 [num_seqs], L_b = cached + new tokens
 *   query_start_loc  device int32 [num_seqs+1], 0 = qsl[0] <= qsl[1] <= ...,
 *                    qsl[num_seqs] = num_q_tokens; 0 <= Q_b <= L_b
 *   max_query_len, max_seq_len  host-side upper bounds of Q_b and L_b (used
 *                    for workspace sizing; requests beyond them are skipped)
 *   scale            softmax scale (e.g. 1/sqrt(head_dim)), finite and > 0
 *                    (PA_ERR_SHAPE otherwise)
 *   out              device bf16 [num_q_tokens][num_q_heads][head_dim]
 *   workspace        device buffer of >= pa_attend_workspace_size(...) bytes,
 *                    256-byte aligned; contents need no initialisation and
 *                    hold the work plan and split-K partials after the call.
 *                    Calls that overlap in time must use distinct workspaces.
 *   num_q_heads % num_kv_heads == 0, num_q_heads/num_kv_heads <= 16,
 *   head_dim 64 or 128.
 *
 * The reduction order of every output depends only on that request's own
 * (Q_b, L_b) and the logical positions of its keys: outputs are bitwise
 * independent of physical block ids, of block sharing and of the rest of the
 * batch.
 *
 * Source: "vLLM v1 Deep Dive", Step 4c and the Aside "KV cache and prefix caching";
 * "vLLM: An Exhaustive Technical Study" sections 2.1 and 2.4.
 */
pa_status pa_attend(const void *q, const void *k_cache, const void *v_cache,
                    int64_t num_blocks, const int32_t *block_tables,
                    int32_t max_blocks_per_seq, const int32_t *seq_lens,
                    const int32_t *query_start_loc, int32_t num_seqs,
                    int64_t num_q_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim,
                    int32_t max_query_len, int32_t max_seq_len, float scale,
                    void *out, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * pa_attend_noalloc - pa_attend for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments, results and errors as pa_attend,
 * without the workspace.  Its work plan and split-K partials live in a
 * static device array of PA_NOALLOC_SCRATCH_BYTES (64 MiB) inside the
 * library, one per device, allocated with the library's code when it is
 * loaded on the device and held until the process ends.  The call allocates
 * and frees nothing.
 *
 * Limit: batches whose pa_attend_workspace_size(...) exceeds
 * PA_NOALLOC_SCRATCH_BYTES are rejected with PA_ERR_WORKSPACE before
 * anything is enqueued (e.g. 64 decodes of up to 4096 tokens with 32 q heads
 * of 128 dims need 11.3 MiB; 16 x 32768-token decodes with 64 q heads, 44 MiB;
 * a 2048-token mixed step, more than the limit: use pa_attend there).
 *
 * Every call on a device shares that device's array, and the array keeps
 * the last call's plan and partials: calls that overlap in time on one
 * device (several streams, several host threads) race and give undefined
 * outputs; order them on one stream.  Nothing in the array needs to start
 * at zero: each call's plan kernel writes the header and queue counters its
 * attention kernel reads.
 */
#define PA_NOALLOC_SCRATCH_BYTES (((size_t)64) << 20)

pa_status pa_attend_noalloc(const void *q, const void *k_cache, const void *v_cache,
                            int64_t num_blocks, const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *seq_lens,
                            const int32_t *query_start_loc, int32_t num_seqs,
                            int64_t num_q_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_query_len, int32_t max_seq_len, float scale,
                            void *out, void *stream);

/*
 * pa_attend_plan, pa_attend_planned, pa_attend_merge - pa_attend in three
 * calls, so that one plan serves every layer of a forward step (the metadata
 * is the same for all layers; "vLLM v1 Deep Dive", Step 4c: the runner builds
 * query_start_loc and the block tables once per step), and so that each
 * kernel can be timed on its own.
 *
 * pa_attend_plan enqueues the work-plan kernel: it reads the metadata and
 * writes the work list into `workspace`.  pa_attend_planned enqueues the
 * attention kernel over the plan found in `workspace`: it writes `out` for
 * every query row whose keys were not split, and fp32 partial results into
 * the workspace for the others.  pa_attend_merge enqueues the merge kernel
 * that combines those partials into `out`; it must follow every
 * pa_attend_planned on the same stream, before the workspace is reused.
 * When max_seq_len is at most 384 (no request's keys are split at any
 * length the batch allows) there are no partials and pa_attend_merge
 * launches nothing.
 * Arguments mean the same as for pa_attend.  Between the calls the workspace
 * and the metadata arrays must not change, and every size argument must be
 * passed with the same value to all three; a plan made for other sizes is
 * detected on the device and the attention kernel then writes nothing (out
 * keeps its contents).  pa_attend == plan + planned + merge.
 */
pa_status pa_attend_plan(const int32_t *block_tables,
                         int32_t max_blocks_per_seq, const int32_t *seq_lens,
                         const int32_t *query_start_loc, int32_t num_seqs,
                         int64_t num_q_tokens, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim,
                         int32_t max_query_len, int32_t max_seq_len,
                         void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * pa_attend_plan_fp8 - pa_attend_plan for attention over 8-bit pools
 * (pa_attend_planned_fp8).  Same arguments, checks and errors.  A plain
 * plan of either call is valid for either pool type; this one, for batches
 * of decodes only (max_query_len at most 16 / (num_q_heads / num_kv_heads)),
 * splits requests of up to 8192 keys into ranges of 384 keys instead of 512:
 * 8-bit units read half the bytes, and the shorter ranges balance the launch
 * better.  pa_attend_fp8 and pa_write_kv_plan_fp8 plan the same way.
 */
pa_status pa_attend_plan_fp8(const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *seq_lens,
                             const int32_t *query_start_loc, int32_t num_seqs,
                             int64_t num_q_tokens, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim,
                             int32_t max_query_len, int32_t max_seq_len,
                             void *workspace, size_t workspace_bytes,
                             void *stream);

pa_status pa_attend_planned(const void *q, const void *k_cache,
                            const void *v_cache, int64_t num_blocks,
                            const int32_t *block_tables,
                            int32_t max_blocks_per_seq,
                            const int32_t *seq_lens,
                            const int32_t *query_start_loc, int32_t num_seqs,
                            int64_t num_q_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_query_len, int32_t max_seq_len,
                            float scale, void *out, void *workspace,
                            size_t workspace_bytes, void *stream);

pa_status pa_attend_merge(int32_t num_seqs, int64_t num_q_tokens,
                          int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t max_query_len,
                          int32_t max_seq_len, void *out, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * pa_attend_fp8, pa_attend_planned_fp8 - pa_attend and pa_attend_planned
 * over 8-bit pools written by pa_write_kv_fp8.
 *
 * Same arguments and results as the bf16 calls, with k_cache and v_cache the
 * uint8 pools (layout with pa_write_kv_fp8) and two more scalars: a K code
 * stands for decode(code) * k_scale, a V code for decode(code) * v_scale
 * (decode: the E4M3 value; k_scale, v_scale finite and > 0, PA_ERR_SHAPE
 * otherwise).  Codes are widened to bf16 exactly (every E4M3 value is a
 * bf16 value) before the same fp32-accumulating MFMAs as the bf16 path;
 * k_scale joins the softmax scale and v_scale the output normalisation.
 * The work plan (pa_attend_plan) and the merge (pa_attend_merge) are the
 * bf16 path's: the split partials already carry v_scale.
 *
 * Source: "vLLM: An Exhaustive Technical Study", section 2.8 (fp8 E4M3
 * KV cache, one fp32 scale per tensor), with the attention of pa_attend.
 */
pa_status pa_attend_fp8(const void *q, const void *k_cache, const void *v_cache,
                        int64_t num_blocks, const int32_t *block_tables,
                        int32_t max_blocks_per_seq, const int32_t *seq_lens,
                        const int32_t *query_start_loc, int32_t num_seqs,
                        int64_t num_q_tokens, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim,
                        int32_t max_query_len, int32_t max_seq_len, float scale,
                        float k_scale, float v_scale, void *out, void *workspace,
                        size_t workspace_bytes, void *stream);

pa_status pa_attend_planned_fp8(const void *q, const void *k_cache,
                                const void *v_cache, int64_t num_blocks,
                                const int32_t *block_tables,
                                int32_t max_blocks_per_seq,
                                const int32_t *seq_lens,
                                const int32_t *query_start_loc, int32_t num_seqs,
                                int64_t num_q_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_query_len, int32_t max_seq_len,
                                float scale, float k_scale, float v_scale,
                                void *out, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * Shared-prefix (cascade) attention: pa_attend for a batch whose requests all
 * begin with the same common_prefix_len keys.  The prefix is attended once
 * for every query token of the batch (tiles of consecutive query tokens of
 * all requests against the prefix's blocks, read once instead of once per
 * request) and each request's own keys separately; the two results of every
 * row are combined by the split-K merge (log-sum-exp renormalisation).
 * Source: "vLLM: An Exhaustive Technical Study", section 2.3 (cascade
 * attention: the shared prefix computed once, merged with each request's
 * suffix by log-sum-exp renormalisation; metadata common_prefix_len).
 *
 * Result: the same attention as pa_attend (one more split point per row, so
 * equal up to fp32 rounding order, within the same tolerance of the exact
 * result).  The reduction order of a row depends only on its request's
 * (Q_b, L_b), its logical key positions and common_prefix_len.
 *
 * Requirements on the batch (content; check with pa_validate_cascade_host):
 *   - every request b holds the prefix and queries only past it:
 *     seq_lens[b] - Q_b >= common_prefix_len (requests that break this are
 *     skipped: their rows are not written, PA_OK is still returned);
 *   - the prefix's whole blocks are the same in every table: the prefix is
 *     read through request 0's row.
 * The library shares the largest multiple of 32 keys not above
 * common_prefix_len (0: plain pa_attend through the shared-prefix path);
 * 0 <= common_prefix_len <= max_seq_len (PA_ERR_SHAPE otherwise).
 *
 * pa_attend_cascade_workspace_size - workspace bytes of the shared-prefix
 *   calls (the pa_attend workspace plus a prefix section for up to 8 prefix
 *   key ranges per query token).  0 for invalid arguments.
 * pa_attend_cascade, pa_attend_cascade_fp8 - plan + attention + merge, over
 *   bf16 or 8-bit pools (arguments as pa_attend / pa_attend_fp8 plus
 *   common_prefix_len).
 * pa_attend_plan_cascade, pa_attend_planned_cascade(_fp8),
 *   pa_attend_merge_cascade - the same in three calls, as pa_attend_plan,
 *   pa_attend_planned(_fp8) and pa_attend_merge (one plan for every layer).
 *   A shared-prefix plan is run only by these calls and a plain plan only by
 *   the plain ones (the other kind is detected on the device and nothing is
 *   written).
 * All of them: workspace >= pa_attend_cascade_workspace_size(...) bytes
 * (PA_ERR_WORKSPACE otherwise); other arguments and errors as pa_attend.
 */
size_t pa_attend_cascade_workspace_size(int32_t num_seqs, int64_t num_q_tokens,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t max_query_len,
                                        int32_t max_seq_len);

pa_status pa_attend_cascade(const void *q, const void *k_cache,
                            const void *v_cache, int64_t num_blocks,
                            const int32_t *block_tables,
                            int32_t max_blocks_per_seq, const int32_t *seq_lens,
                            const int32_t *query_start_loc, int32_t num_seqs,
                            int64_t num_q_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_query_len, int32_t max_seq_len,
                            int32_t common_prefix_len, float scale, void *out,
                            void *workspace, size_t workspace_bytes,
                            void *stream);

pa_status pa_attend_cascade_fp8(const void *q, const void *k_cache,
                                const void *v_cache, int64_t num_blocks,
                                const int32_t *block_tables,
                                int32_t max_blocks_per_seq,
                                const int32_t *seq_lens,
                                const int32_t *query_start_loc, int32_t num_seqs,
                                int64_t num_q_tokens, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_query_len, int32_t max_seq_len,
                                int32_t common_prefix_len, float scale,
                                float k_scale, float v_scale, void *out,
                                void *workspace, size_t workspace_bytes,
                                void *stream);

pa_status pa_attend_plan_cascade(const int32_t *block_tables,
                                 int32_t max_blocks_per_seq,
                                 const int32_t *seq_lens,
                                 const int32_t *query_start_loc, int32_t num_seqs,
                                 int64_t num_q_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 int32_t max_query_len, int32_t max_seq_len,
                                 int32_t common_prefix_len, void *workspace,
                                 size_t workspace_bytes, void *stream);

pa_status pa_attend_planned_cascade(const void *q, const void *k_cache,
                                    const void *v_cache, int64_t num_blocks,
                                    const int32_t *block_tables,
                                    int32_t max_blocks_per_seq,
                                    const int32_t *seq_lens,
                                    const int32_t *query_start_loc,
                                    int32_t num_seqs, int64_t num_q_tokens,
                                    int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_query_len,
                                    int32_t max_seq_len, float scale, void *out,
                                    void *workspace, size_t workspace_bytes,
                                    void *stream);

pa_status pa_attend_planned_cascade_fp8(
    const void *q, const void *k_cache, const void *v_cache, int64_t num_blocks,
    const int32_t *block_tables, int32_t max_blocks_per_seq,
    const int32_t *seq_lens, const int32_t *query_start_loc, int32_t num_seqs,
    int64_t num_q_tokens, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t max_query_len, int32_t max_seq_len, float scale,
    float k_scale, float v_scale, void *out, void *workspace,
    size_t workspace_bytes, void *stream);

pa_status pa_attend_merge_cascade(int32_t num_seqs, int64_t num_q_tokens,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_query_len,
                                  int32_t max_seq_len, void *out, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * pa_write_kv_plan, pa_write_kv_plan_fp8 - pa_write_kv (pa_write_kv_fp8) and
 * pa_attend_plan (pa_attend_plan_cascade) of the same step in one launch.
 *
 * A step scatters its new K/V and plans its attention before the first
 * layer's attention runs ("vLLM v1 Deep Dive", Step 4c: the runner prepares
 * the step's metadata once; "vLLM: An Exhaustive Technical Study" section
 * 2.1: the new tokens are cached before attention reads them).  The two do
 * not depend on each other: one workgroup of the launch writes the plan
 * while the others scatter, saving one kernel launch per step.
 *
 * Arguments: the scatter's (k, v, strides, slot_mapping, num_new_tokens,
 * the scales for the 8-bit variant, k_cache, v_cache, num_blocks) exactly
 * as pa_write_kv / pa_write_kv_fp8 take them, num_new_tokens in the place of
 * num_tokens; then the plan's, exactly as pa_attend_plan takes them.
 * num_kv_heads and head_dim serve both.  common_prefix_len < 0: a plain plan
 * (workspace >= pa_attend_workspace_size(...)), run by pa_attend_planned(_fp8);
 * common_prefix_len >= 0: a shared-prefix plan as pa_attend_plan_cascade
 * makes it (workspace >= pa_attend_cascade_workspace_size(...)), run by
 * pa_attend_planned_cascade(_fp8).
 *
 * Results, skips and races: those of the two calls it replaces; the call
 * checks both argument sets first and enqueues nothing if either is
 * invalid (the errors of pa_write_kv(_fp8) and pa_attend_plan(_cascade)).
 * With num_new_tokens == 0 it is the plan alone; with nothing to plan
 * (num_seqs == 0 or num_q_tokens == 0) it is the scatter alone.
 */
pa_status pa_write_kv_plan(const void *k, const void *v, int64_t k_token_stride,
                           int64_t v_token_stride, const int64_t *slot_mapping,
                           int64_t num_new_tokens, void *k_cache, void *v_cache,
                           int64_t num_blocks, const int32_t *block_tables,
                           int32_t max_blocks_per_seq, const int32_t *seq_lens,
                           const int32_t *query_start_loc, int32_t num_seqs,
                           int64_t num_q_tokens, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_query_len, int32_t max_seq_len,
                           int32_t common_prefix_len, void *workspace,
                           size_t workspace_bytes, void *stream);

pa_status pa_write_kv_plan_fp8(const void *k, const void *v, int64_t k_token_stride,
                               int64_t v_token_stride, const int64_t *slot_mapping,
                               int64_t num_new_tokens, float k_scale, float v_scale,
                               void *k_cache, void *v_cache, int64_t num_blocks,
                               const int32_t *block_tables, int32_t max_blocks_per_seq,
                               const int32_t *seq_lens, const int32_t *query_start_loc,
                               int32_t num_seqs, int64_t num_q_tokens,
                               int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_query_len,
                               int32_t max_seq_len, int32_t common_prefix_len,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * pa_validate_cascade_host - host check of the shared-prefix requirements
 * above on HOST arrays: PA_ERR_METADATA (detail in pa_last_error()) when a
 * request has seq_lens[b] - Q_b < common_prefix_len, or when one of the
 * first common_prefix_len / 16 block-table entries of a request differs from
 * request 0's (or the row is shorter than that).
 */
pa_status pa_validate_cascade_host(const int32_t *block_tables,
                                   int32_t max_blocks_per_seq,
                                   const int32_t *seq_lens,
                                   const int32_t *query_start_loc,
                                   int32_t num_seqs, int32_t common_prefix_len);

/*
 * pa_copy_blocks - the block copy of copy-on-write: for each pair
 * (src, dst) = (block_mapping[2i], block_mapping[2i+1]), copy every byte of
 * block src to block dst in both pools (all kv heads, K and V).
 *
 *   k_cache, v_cache  device pools of num_blocks blocks: bf16 pools
 *                     (elem_bytes 2, pa_write_kv) or 8-bit pools (elem_bytes
 *                     1, pa_write_kv_fp8); one block is
 *                     num_kv_heads * 16 * head_dim * elem_bytes bytes
 *   block_mapping     device int64 [num_pairs][2]
 * A pair naming a block outside [0, num_blocks), or the same block twice, is
 * skipped.  A block that is the destination of one pair and the source of
 * another in the same call, or the destination of two pairs, gives undefined
 * contents.  Asynchronous on `stream`; call it before writing the step's new
 * tokens into the copies.
 *
 * Source: "vLLM: An Exhaustive Technical Study", section 2.1 (blocks shared
 * by reference count, a block duplicated when a request writes into one whose
 * count is above 1).
 */
pa_status pa_copy_blocks(void *k_cache, void *v_cache, int64_t num_blocks,
                         int32_t num_kv_heads, int32_t head_dim, int32_t elem_bytes,
                         const int64_t *block_mapping, int64_t num_pairs,
                         void *stream);

/*
 * pa_expand_block_tables - pools with larger blocks.  A block of
 * block_size = R * 16 tokens (R = 1, 2, 4, ...) is stored as R consecutive
 * 16-token blocks of the pool: block n holds the 16-token blocks
 * n*R .. n*R + R-1, so a pool of N such blocks is a pool of N*R 16-token
 * blocks, and slot_mapping values (n * block_size + offset) are the same
 * numbers for pa_write_kv.  This call turns block tables of block_size-token
 * ids into the 16-token tables pa_attend reads:
 *   out[b][j] = block_tables[b][j / R] * R + j % R,  j < max_blocks_per_seq * R
 * (entries < 0 stay -1).  out: device int32 [num_seqs][max_blocks_per_seq * R].
 * (8-token blocks have calls of their own: pa_write_kv_bs, pa_attend_bs.)
 *
 * Source: "vLLM: An Exhaustive Technical Study", section 2.1 (block sizes 8,
 * 16, 32 and larger per platform; the write slot is
 * block number * block_size + offset).
 */
pa_status pa_expand_block_tables(const int32_t *block_tables, int32_t num_seqs,
                                 int32_t max_blocks_per_seq, int32_t block_size,
                                 int32_t *out, void *stream);

/*
 * Multi-head latent attention (MLA) over a paged latent cache.
 *
 * Source: "vLLM: An Exhaustive Technical Study", section 2.4 (the MLA
 * paragraph): one low-rank latent vector cached per token, shared by every
 * query head and attended MQA-style in decode; 512 latent + 64 decoupled
 * rotary dims = 576 cached values per token; blocks of 64 tokens.
 * Reading: a query head supplies a 576-dim query (its latent-space part
 * and its rotary part); its score of token j is scale * (query . cached vector
 * j), and its output is the softmax-weighted sum of the first 512 (latent)
 * dims of the cached vectors -- the up- and output projections around this
 * step are the caller's.  Causal as pa_attend: query i of a request's Q new
 * tokens sits at L - Q + i and sees tokens 0 .. L - Q + i.
 *
 * Cache: bf16, num_blocks blocks of 64 * 576 elements; token t (0..63), dim d
 * of a block sit at element (((t / 16) * 18 + d / 32) * 16 + t % 16) * 32 + d % 32.
 * slot = block * 64 + offset.
 *
 * pa_mla_write_kv - scatter kv (device bf16, row i of 576 values at
 *   kv + i * kv_token_stride elements; stride a multiple of 8) into the cache
 *   at slot_mapping[i] (device int64; < 0 or >= num_blocks * 64: skipped).
 * pa_mla_workspace_size - workspace bytes of pa_mla_decode (per-token
 *   records and the partial results of query tokens whose keys are cut
 *   between workgroups: at most two groups of tokens per workgroup), enough
 *   for either of the decode's two forms (one query token per work item, or
 *   groups of 128 / num_q_heads consecutive tokens of a request for 16, 32
 *   and 64 heads when the batch averages 4 or more query tokens per
 *   request); 0 for invalid arguments.
 * pa_mla_decode - q device bf16 [num_q_tokens][num_q_heads][576], out device
 *   bf16 [num_q_tokens][num_q_heads][512]; block_tables of 64-token block ids
 *   [num_seqs][max_blocks_per_seq]; seq_lens, query_start_loc as pa_attend;
 *   num_q_heads a multiple of 16, at most 128, max_seq_len at most 262144,
 *   num_seqs at most 131072, num_q_tokens below 2^25 and num_blocks at most
 *   2^29 (PA_ERR_UNSUPPORTED otherwise); query_start_loc non-decreasing;
 *   workspace >= pa_mla_workspace_size(...) bytes, 256-byte aligned.  A
 *   request whose metadata is out of bounds is skipped (its rows unwritten).
 *   Two launches: the decode, then (when keys of a token can be cut between
 *   workgroups) the fold of the pieces; calls sharing a workspace must be
 *   ordered (one stream).
 */
#define PA_MLA_BLOCK_SIZE 64
#define PA_MLA_DIM 576
#define PA_MLA_LATENT 512

size_t pa_mla_workspace_size(int64_t num_q_tokens, int32_t num_q_heads,
                             int32_t max_seq_len);

pa_status pa_mla_write_kv(const void *kv, int64_t kv_token_stride,
                          const int64_t *slot_mapping, int64_t num_tokens, void *cache,
                          int64_t num_blocks, void *stream);

pa_status pa_mla_decode(const void *q, const void *cache, int64_t num_blocks,
                        const int32_t *block_tables, int32_t max_blocks_per_seq,
                        const int32_t *seq_lens, const int32_t *query_start_loc,
                        int32_t num_seqs, int64_t num_q_tokens, int32_t num_q_heads,
                        int32_t max_seq_len, float scale, void *out, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * pa_gather_kv - logical gather through the block tables (a checking aid).
 *
 * Writes k_out/v_out, device bf16 [sum_b L_b][num_kv_heads][head_dim]: row
 * kv_start[b] + j holds token j < L_b of request b, read from block
 * block_tables[b][j/16], slot j%16.  kv_start: device int64 [num_seqs+1],
 * prefix sum of seq_lens; total_rows = kv_start[num_seqs].
 *
 * Source: "Deep Dive - vLLM" (leetllm.com), "The historical idea: page KV
 * memory" (a kernel follows the table to load the right physical blocks);
 * "vLLM: An Exhaustive Technical Study" section 2.1.
 */
pa_status pa_gather_kv(const void *k_cache, const void *v_cache,
                       int64_t num_blocks, const int32_t *block_tables,
                       int32_t max_blocks_per_seq, const int32_t *seq_lens,
                       const int64_t *kv_start, int32_t num_seqs,
                       int64_t total_rows, int32_t num_kv_heads,
                       int32_t head_dim, void *k_out, void *v_out,
                       void *stream);

/*
 * Pools of 8-token blocks (bf16): pa_write_kv_bs, pa_attend_bs,
 * pa_gather_kv_bs.
 *
 * The pages offer block sizes 8, 16 and 32 ("vLLM: An Exhaustive Technical
 * Study", section 2.1, the --block-size choices; the write slot is
 * block number * block_size + offset).  These calls take block_size = 8 or
 * 16; with 16 they are pa_write_kv, pa_attend and pa_gather_kv (larger
 * blocks: 16-token pools and pa_expand_block_tables).  With 8, a pool is
 * num_blocks x num_kv_heads tiles of 8 * head_dim bf16, tile (n, g) at
 * element (n * num_kv_heads + g) * 8 * D, and inside it, H = D/2:
 *     K(t, d) at ((d / 8) * 8 + t) * 8 + d % 8
 *     V(t, d) at ((((d % H) / 16 * 2 + d / H) * 2 + t / 4) * 16 + d % 16)
 *                * 4 + t % 4
 * (the 16-token tile's formulas with 8 token slots); slot s is offset s % 8
 * of block s / 8, and entry j of a block-table row names the block of
 * tokens 8j .. 8j+7 (ceil(L_b / 8) entries used).  Attention gathers each
 * 16-key step from two 8-token blocks; results are identical to pa_attend's
 * over the same tokens in 16-token blocks (same work decomposition, same
 * reduction order).  Arguments, workspace (pa_attend_workspace_size), checks
 * and errors otherwise as the block-size-16 calls; a block_size other than
 * 8 or 16 is PA_ERR_UNSUPPORTED.  8-bit pools of 8-token blocks are not
 * supported.
 */
pa_status pa_write_kv_bs(const void *k, const void *v, int64_t k_token_stride,
                         int64_t v_token_stride, const int64_t *slot_mapping,
                         int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                         void *k_cache, void *v_cache, int64_t num_blocks,
                         int32_t block_size, void *stream);

pa_status pa_attend_bs(const void *q, const void *k_cache, const void *v_cache,
                       int64_t num_blocks, int32_t block_size,
                       const int32_t *block_tables, int32_t max_blocks_per_seq,
                       const int32_t *seq_lens, const int32_t *query_start_loc,
                       int32_t num_seqs, int64_t num_q_tokens, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                       int32_t max_seq_len, float scale, void *out, void *workspace,
                       size_t workspace_bytes, void *stream);

pa_status pa_gather_kv_bs(const void *k_cache, const void *v_cache, int64_t num_blocks,
                          int32_t block_size, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *seq_lens,
                          const int64_t *kv_start, int32_t num_seqs, int64_t total_rows,
                          int32_t num_kv_heads, int32_t head_dim, void *k_out,
                          void *v_out, void *stream);

/*
 * pa_validate_metadata_host - check the CONTENT of one step's metadata, all
 * pointers HOST memory.  Returns PA_OK or PA_ERR_METADATA (message in
 * pa_last_error()) for: query_start_loc not starting at 0, decreasing, or not
 * ending at num_q_tokens; Q_b > L_b or L_b < 0; L_b > max_seq_len or
 * Q_b > max_query_len; ceil(L_b/16) > max_blocks_per_seq; a used block-table
 * entry outside [0, num_blocks); a slot >= num_blocks*16; two tokens with the
 * same slot.  slot_mapping may be NULL (num_slots ignored).
 */
pa_status pa_validate_metadata_host(const int32_t *block_tables,
                                    int32_t max_blocks_per_seq,
                                    const int32_t *seq_lens,
                                    const int32_t *query_start_loc,
                                    int32_t num_seqs, int64_t num_q_tokens,
                                    int32_t max_query_len, int32_t max_seq_len,
                                    int64_t num_blocks,
                                    const int64_t *slot_mapping,
                                    int64_t num_slots);

/*
 * pa_validate_metadata - the same checks on DEVICE metadata.  Synchronous:
 * copies the arrays to host memory (blocking hipMemcpy) first.
 */
pa_status pa_validate_metadata(const int32_t *block_tables,
                               int32_t max_blocks_per_seq,
                               const int32_t *seq_lens,
                               const int32_t *query_start_loc,
                               int32_t num_seqs, int64_t num_q_tokens,
                               int32_t max_query_len, int32_t max_seq_len,
                               int64_t num_blocks, const int64_t *slot_mapping,
                               int64_t num_slots);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
