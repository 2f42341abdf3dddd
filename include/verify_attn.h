/*
 * verify_attn.h -- C ABI of the MI355X (gfx950) MLA speculative-decoding
 * verify-attention library (libverify_attn.so).
 *
 * The operation (page "The Build That Bridged Design and Deployment:
 * Compiling the Custom sm_120 Verify Kernel", section "What This Build
 * Achieves: The paged+bf16 Kernel"; page "The Build That Unlocked 3-6x
 * Decode Speedup", section "The Context: A Custom Kernel for an Unsupported
 * Architecture"):
 *
 *   For every sequence b, query position i and head h, attend with the
 *   576-d query q[b][i][h] over the KV positions of sequence b. Position j
 *   of sequence b lives in pool slot kv_indices[off_b + j] (page_size 1),
 *   where off_b = sum_{b' < b} (prefix_lens[b'] + Q). The first
 *   prefix_lens[b] positions (the prefix) are visible to every query; the
 *   last Q positions are the speculative tail, and tail position t is
 *   visible to query i iff tree_mask[b][i][t] != 0. Keys are the whole
 *   576-d bf16 latent rows, values their first 512 dims, scores are
 *   scale * (q . k), and
 *       lse[b][i][h] = ln sum_{visible j} exp(score_j)
 *       out[b][i][h] = sum_{visible j} exp(score_j - lse) * value_j.
 *   A query with no visible position gets out = 0 and lse = -inf.
 *
 * The KV range of each sequence is split into chunks that run on separate
 * workgroups (flash-decode with online softmax over KV tiles); a second
 * kernel merges the chunk partials by log-sum-exp (the KV split whose count
 * the pages call NSPLIT: page "The Build That Unlocked 3-6x Decode Speedup", section "The
 * Context: A Custom Kernel for an Unsupported Architecture"; page "The Build
 * Script Edit: How a Single Line of Infrastructure Unlocked Custom CUDA
 * Kernels on sm_120", section "Context: The Long Road to a Custom sm_120
 * Kernel").
 *
 * Conventions for every entry point:
 *  - Device pointers are caller-owned device memory; the library allocates
 *    nothing and never frees caller memory.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Work is enqueued asynchronously; no entry point synchronises, reads
 *    device data on the host or allocates.
 *  - Return value: VA_OK (0) or a negative va_status. On error nothing has
 *    been enqueued (argument errors) or the launch failed (VA_EHIP);
 *    verify_attn_last_error() then describes it. No C++ exception crosses
 *    this interface.
 *  - Results are deterministic: identical inputs give bitwise-identical
 *    outputs (no floating-point atomics, fixed reduction order).
 */
#ifndef VERIFY_ATTN_H
#define VERIFY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VA_LATENT_DIM 576 /* key width: one compressed latent row, bf16 */
#define VA_VALUE_DIM 512  /* value width: the leading dims of the same row */
#define VA_MAX_Q 64       /* verify positions per sequence supported */

typedef enum {
  VA_OK = 0,
  VA_EINVAL = -1, /* bad pointer, alignment or dimension; nothing enqueued */
  VA_ENOSPC = -2, /* workspace smaller than verify_attn_workspace_size() */
  VA_EHIP = -3    /* the HIP runtime reported an error for a launch */
} va_status;

/*
 * Not on the pages: added because the caller owns all device memory. Bytes
 * of device workspace verify_attn() needs for these sizes on the current HIP
 * device (the split plan depends on its compute-unit count): the chunk
 * offsets, and the per-chunk partial outputs and log-sum-exps that the merge
 * folds. Returns 0 if the sizes are invalid.
 */
size_t verify_attn_workspace_size(int B, int Q, int H, int64_t total_kv);

/*
 * Verify attention (see the top of this file for the definition).
 *
 *  q           bf16 [B][Q][H][576], contiguous, 16-byte aligned.
 *  kv_pool     bf16 [num_slots][576], row stride 1152 bytes, 16-byte aligned.
 *  kv_indices  int32 [total_kv]: sequence b owns entries off_b .. off_b +
 *              prefix_lens[b] + Q - 1, its prefix slots in position order
 *              followed by the Q tail slots in query order. An entry outside
 *              [0, num_slots) is read as an all-zero row (never a fault).
 *  prefix_lens int32 [B] on the device, each >= 0 (a negative value counts as 0).
 *  tree_mask   uint8 [B][Q][Q]; [b][i][t] != 0 iff query i sees tail position t
 *              (normally the diagonal is set: a query sees its own draft token).
 *  scale       multiplies q . k (in fp32, on the fp32 dot product).
 *  out         fp32 [B][Q][H][512], 16-byte aligned (written).
 *  lse         fp32 [B][Q][H], natural log (written).
 *  B >= 1, 1 <= Q <= 64, H >= 1, num_slots >= 1,
 *  total_kv = sum_b (prefix_lens[b] + Q), with B*Q <= total_kv < 2^31.
 *  workspace   device memory of at least verify_attn_workspace_size(B, Q, H,
 *              total_kv) bytes, 256-byte aligned; its contents on entry do
 *              not matter and are scratch afterwards.
 *
 * Device-side preconditions that the host cannot check: the prefix_lens
 * sum must match total_kv (positions past total_kv are treated as absent),
 * inputs must be finite, and value elements must lie within the finite
 * fp16 range (|v| < 65504): the probability-times-value product takes its
 * operands in fp16 and each chunk's normalised partial output is kept in
 * fp16, so a larger value becomes inf or NaN without an error. The absolute
 * error grows with the values (fp16 rounding is relative to magnitude).
 */
int verify_attn(const void* q, const void* kv_pool, const int32_t* kv_indices,
                const int32_t* prefix_lens, const uint8_t* tree_mask, float scale,
                float* out, float* lse, int B, int Q, int H, int64_t num_slots,
                int64_t total_kv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * computation as verify_attn(), with the same arguments except the
 * workspace. It uses a fixed device scratch of VA_NOALLOC_SCRATCH_BYTES that
 * the library holds on each device it runs on until the process ends, and
 * calls no allocating routine. Sizes whose workspace
 * (verify_attn_workspace_size) exceeds that scratch are rejected with
 * VA_ENOSPC before anything is enqueued. Every call on a device shares that
 * device's scratch: calls that may overlap on one device (different streams,
 * different threads) race and must be ordered by the caller. Results equal
 * verify_attn()'s bit for bit.
 */
#define VA_NOALLOC_SCRATCH_BYTES (64u << 20)
int verify_attn_noalloc(const void* q, const void* kv_pool, const int32_t* kv_indices,
                        const int32_t* prefix_lens, const uint8_t* tree_mask, float scale,
                        float* out, float* lse, int B, int Q, int H, int64_t num_slots,
                        int64_t total_kv, void* stream);

/*
 * Not on the pages: added because a C ABI carries no exceptions.
 * Thread-local description of the last error on this thread ("" if none).
 */
const char* verify_attn_last_error(void);

/*
 * KV-cache defragmentation (page "The Build That Unlocked 3-6x Decode
 * Speedup", sections "The Context: A Custom Kernel for an Unsupported
 * Architecture" and "The Broader Significance", where it is named as the step
 * after the verify kernel; the pages give no more, and this is the plainest
 * reading). For j = 0 .. n-1:
 *     dst_pool[dst_base + j] = src_pool[kv_indices[j]]   (an all-zero row if
 *                                                          the slot is outside
 *                                                          [0, num_slots))
 *     new_indices[j]         = dst_base + j
 * Other destination rows are not touched. verify_attn() over (dst_pool,
 * new_indices) then equals verify_attn() over (src_pool, kv_indices) bit for
 * bit, and its gather reads consecutive rows.
 *
 *  src_pool    bf16 [num_slots][576], 16-byte aligned (read).
 *  kv_indices  int32 [n] (read).
 *  dst_pool    bf16 [dst_slots][576], 16-byte aligned (rows dst_base ..
 *              dst_base + n - 1 written).
 *  new_indices int32 [n] (written); may not alias kv_indices.
 *  0 <= n <= 2^31 - 1; 0 <= dst_base <= dst_slots - n; dst_base + n - 1 must
 *  fit in int32.
 * The destination run must not overlap any row the source indices name (the
 * host cannot check this; dst_pool may be src_pool when the run lies in free
 * slots). Returns VA_OK, VA_EINVAL (nothing enqueued) or VA_EHIP.
 */
int verify_attn_kv_defrag(const void* src_pool, const int32_t* kv_indices, int64_t n, int64_t num_slots,
                          void* dst_pool, int64_t dst_base, int64_t dst_slots, int32_t* new_indices,
                          void* stream);

/*
 * Draft-tree acceptance (the tree_accept kernel source listed next to the
 * verify kernels, page "The Build That Unlocked 3-6x Decode Speedup", section
 * "Why This Build Was Different"; page "The Build Script Edit: How a Single
 * Line of Infrastructure Unlocked Custom CUDA Kernels on sm_120", section
 * "Input Knowledge Required"; the pages give only the name, and this is the
 * plainest reading of greedy tree speculative decoding). For every sequence
 * b, node 0 is the root (the last accepted token) and node i >= 1 has parent
 * parents[b][i] < i and draft token draft_tokens[b][i]; target_tokens[b][i]
 * is the target model's choice after the path root -> i. Starting at the
 * root, the walk steps to the smallest-index child c of the current node
 * with draft_tokens[b][c] == target_tokens[b][current] until no child
 * matches.
 *
 *  parents, draft_tokens, target_tokens  int32 [B][Q] (read).
 *  accept_len   int32 [B] (written): accepted draft tokens (path length - 1).
 *  accepted     int32 [B][Q] (written): the path's node indices, root first,
 *               then -1.
 *  bonus_token  int32 [B] (written): target_tokens at the last accepted node.
 *  B >= 1, 1 <= Q <= 64. A malformed tree (parents[i] >= i) cannot hang the
 *  walk: only children with a larger index than the current node count.
 * Returns VA_OK, VA_EINVAL (nothing enqueued) or VA_EHIP.
 */
int verify_attn_tree_accept(const int32_t* parents, const int32_t* draft_tokens, const int32_t* target_tokens,
                            int B, int Q, int32_t* accept_len, int32_t* accepted, int32_t* bonus_token,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_ATTN_H */
