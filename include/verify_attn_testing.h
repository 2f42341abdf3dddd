/*
 * verify_attn_testing.h -- test and measurement entry points of
 * libverify_attn.so. None of these is on the pages: they were added so that
 * the gather order can be compared bit for bit, the chunk plan inspected and
 * forced, and the split kernel timed on its own. A production caller needs
 * only include/verify_attn.h.
 *
 * The conventions of include/verify_attn.h apply (caller-owned device memory,
 * asynchronous on `stream`, va_status return codes, thread-local
 * verify_attn_last_error()). Nothing here keeps state between calls: every
 * option is an argument of the call it applies to.
 */
#ifndef VERIFY_ATTN_TESTING_H
#define VERIFY_ATTN_TESTING_H

#include <stddef.h>
#include <stdint.h>

#include "verify_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Per-call options of verify_attn_ex().
 *  chunk_keys         0: the automatic chunk plan (what verify_attn() does);
 *                     > 0: every chunk holds this many keys (rounded up to a
 *                     multiple of 32), for tests that put chunk boundaries at
 *                     chosen places and for tuning sweeps.
 *  split_start_event  hipEvent_t (as void*) recorded on the stream right before
 *                     the split kernel, the call's first launch; NULL: none.
 *  split_stop_event   hipEvent_t recorded right after the split kernel; NULL:
 *                     none. The pair times the split kernel alone; the start
 *                     event with one the caller records after the call times
 *                     the whole call from its first kernel.
 */
typedef struct {
  int32_t chunk_keys;
  void* split_start_event;
  void* split_stop_event;
} va_test_options;

/*
 * verify_attn() with per-call options (opts may be NULL: the same as
 * verify_attn()). The workspace must hold verify_attn_workspace_size_ex()
 * bytes for the same chunk_keys. A negative chunk_keys gives VA_EINVAL.
 */
int verify_attn_ex(const void* q, const void* kv_pool, const int32_t* kv_indices,
                   const int32_t* prefix_lens, const uint8_t* tree_mask, float scale,
                   float* out, float* lse, int B, int Q, int H, int64_t num_slots,
                   int64_t total_kv, void* workspace, size_t workspace_bytes, void* stream,
                   const va_test_options* opts);

/* Workspace bytes for verify_attn_ex() with this chunk_keys (0 if invalid). */
size_t verify_attn_workspace_size_ex(int B, int Q, int H, int64_t total_kv, int32_t chunk_keys);

/*
 * The split plan verify_attn_ex() would use for these sizes and this
 * chunk_keys (0 = automatic) on the current device: the keys per chunk (with
 * chunk_keys = 0, the keys per column at which the columns fill the grid; the
 * device then cuts the batch's key tiles into equal columns from the actual
 * prefix lengths when there are fewer sequences than columns, and into
 * chunks of this length otherwise), the capacity of the workspace in pieces
 * (one partial each), row tiles per sequence (128 query-head rows each) and
 * the split-kernel grid size. Any output pointer may be NULL. Returns VA_OK
 * or VA_EINVAL.
 */
int verify_attn_query_plan(int B, int Q, int H, int64_t total_kv, int32_t chunk_keys_in,
                           int32_t* chunk_keys, int32_t* max_chunks, int32_t* row_tiles,
                           int32_t* grid);

/*
 * Runs the split kernel's own slot copy and gather routines (kv_indices ->
 * LDS slot ring -> 16-byte direct-to-LDS loads -> LDS tile) for positions
 * 0..n-1 and copies each tile back out in position order, so that the gather
 * can be compared bit-exactly with kv_pool[kv_indices[j]]. rows_out is bf16
 * [n][576], 16-byte aligned. Slots outside [0, num_slots) produce zero rows,
 * as in verify_attn(). 0 <= n <= 2^35.
 */
int verify_attn_debug_gather(const void* kv_pool, const int32_t* kv_indices, int64_t n,
                             int64_t num_slots, void* rows_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VERIFY_ATTN_TESTING_H */
