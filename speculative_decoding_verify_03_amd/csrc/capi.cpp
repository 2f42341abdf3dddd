// C-ABI shim of libverify_attn.so: argument validation, the split plan,
// workspace carving and the two launches of a call (split kernel, then merge
// kernel). The ABI is declared in include/verify_attn.h and, for tests and
// measurement, include/verify_attn_testing.h. No entry point allocates,
// synchronises or reads device memory on the host, and none keeps state
// between calls other than a per-device cache of the compute-unit count (and,
// for verify_attn_noalloc, the fixed device scratch and its address).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "va_internal.hpp"
#include "verify_attn.h"
#include "verify_attn_testing.h"

static_assert(VA_NOALLOC_SCRATCH_BYTES == va::kNoAllocScratchBytes, "scratch size in the header");

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_cu_count[64];

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return VA_OK;
}

// Compute units of the current device (cached per device ordinal).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool dims_ok(int B, int Q, int H, int64_t total_kv) {
  if (B < 1 || Q < 1 || Q > VA_MAX_Q || H < 1) return false;
  if ((int64_t)Q * H > (1 << 24)) return false;
  if (total_kv < (int64_t)B * Q || total_kv > (int64_t)INT32_MAX - VA_MAX_Q) return false;
  return true;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// The split plan. Workgroups are (column, 128-row tile) pairs and one
// workgroup fills a compute unit (8 waves, ~159 KiB of LDS), so the batch
// gets a budget of floor(CUs / row_tiles) columns. With fewer sequences than
// that (and at most kPlanThreads) the split kernel cuts the batch's key tiles
// into at most that many equal columns, one piece per sequence a column
// meets; otherwise, and with a forced chunk length (chunk_keys > 0, tests and
// tuning only), every column is one chunk of ideal_keys keys.
bool make_plan(int B, int Q, int H, int64_t total_kv, int ncu, int32_t chunk_keys, va::Plan* p) {
  if (!dims_ok(B, Q, H, total_kv)) return false;
  const int64_t R = (int64_t)Q * H;
  p->row_tiles = (int32_t)((R + va::kRowsPerWG - 1) / va::kRowsPerWG);
  int64_t target = ncu / p->row_tiles;
  if (target < 1) target = 1;
  int64_t ideal = (total_kv + target - 1) / target;
  const int32_t ov = chunk_keys > 0 ? chunk_keys : 0;
  if (ov > 0) ideal = ov;
  if (ideal < va::kMinChunk && ov <= 0) ideal = va::kMinChunk;
  ideal = (ideal + va::kUnit - 1) / va::kUnit * va::kUnit;
  p->target = ov > 0 ? 0 : (int32_t)target;   // a forced length is used as is
  p->ideal_keys = (int32_t)ideal;
  // Workgroups: the row tiles of every column, rounded up to whole groups of
  // 8 columns (the XCD mapping): at most one column per ideal keys, plus one
  // per sequence (the chunk plan's count), at most ceil((total_kv + Q) / ideal)
  // for a batch of one sequence, and at most `target` under the column plan
  // (a budget above B, at most kPlanThreads sequences), which uses no more
  // columns than are launched. Launching no workgroup beyond these bounds
  // matters because a surplus workgroup only gets a compute unit once a
  // working one has finished, and then adds its own start-up to the end of
  // the launch.
  const bool columns = p->target > B && B <= va::kPlanThreads;
  const int64_t chunk_bound = total_kv / ideal + B + 1;
  int64_t live = chunk_bound;
  if (B == 1) live = std::min<int64_t>(live, (total_kv + Q + ideal - 1) / ideal);
  if (columns) live = std::min<int64_t>(live, p->target);
  const int64_t launched = (live + 7) / 8 * 8;
  const int64_t grid = launched * p->row_tiles;
  if (grid > INT32_MAX) return false;
  p->grid = (int32_t)grid;
  // Partial buffers: a sequence of N_b keys takes ceil(N_b / ideal) chunks,
  // so the chunk plan never needs more than total_kv / ideal + B of them; the
  // column plan's pieces are at most its columns + B - 1.
  int64_t max_chunks = chunk_bound;
  if (columns) max_chunks = std::max<int64_t>(max_chunks, launched + B);
  if (max_chunks > INT32_MAX / 8) return false;
  p->max_chunks = (int32_t)max_chunks;
  size_t off = 0;
  p->off_chunk = off;
  off += sizeof(int32_t) * (size_t)(B + 1);
  off = align_up(off, 256);
  p->off_lse = off;
  off += sizeof(float) * (size_t)max_chunks * (size_t)R;
  off = align_up(off, 256);
  p->off_o = off;
  off += sizeof(uint16_t) * (size_t)max_chunks * (size_t)R * va::kValue;   // fp16 partial outputs
  p->bytes = align_up(off, 256);
  return true;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Host-side checks of a verify call's arguments other than the workspace;
// fills the plan. Returns VA_OK or the status to report.
int check_verify_args(const void* q, const void* kv_pool, const int32_t* kv_indices, const int32_t* prefix_lens,
                      const uint8_t* tree_mask, float scale, const float* out, const float* lse, int B, int Q,
                      int H, int64_t num_slots, int64_t total_kv, int32_t chunk_keys, va::Plan* p) {
  if (!q || !kv_pool || !kv_indices || !prefix_lens || !tree_mask || !out || !lse)
    return fail(VA_EINVAL, "null pointer argument");
  if (!aligned(q, 16) || !aligned(kv_pool, 16) || !aligned(out, 16))
    return fail(VA_EINVAL, "q, kv_pool and out must be 16-byte aligned");
  if (!aligned(kv_indices, 4) || !aligned(prefix_lens, 4) || !aligned(lse, 4))
    return fail(VA_EINVAL, "kv_indices, prefix_lens and lse must be 4-byte aligned");
  if (!dims_ok(B, Q, H, total_kv))
    return fail(VA_EINVAL, "bad sizes: B=%d Q=%d H=%d total_kv=%lld (need B>=1, 1<=Q<=%d, H>=1, "
                "B*Q <= total_kv < 2^31)", B, Q, H, (long long)total_kv, VA_MAX_Q);
  if (num_slots < 1 || num_slots > INT64_MAX / va::kRowBytes)
    return fail(VA_EINVAL, "bad num_slots %lld", (long long)num_slots);
  if (!std::isfinite(scale)) return fail(VA_EINVAL, "scale must be finite");
  if (chunk_keys < 0) return fail(VA_EINVAL, "bad chunk_keys %d", chunk_keys);
  if (!make_plan(B, Q, H, total_kv, cu_count(), chunk_keys, p)) return fail(VA_EINVAL, "sizes too large to plan");
  return VA_OK;
}

// The two launches of a call, on a checked plan and a workspace of at least
// p.bytes bytes (256-byte aligned). ev0 / ev1 (may be null) are recorded right
// before and after the split kernel.
int launch_verify(const void* q, const void* kv_pool, const int32_t* kv_indices, const int32_t* prefix_lens,
                  const uint8_t* tree_mask, float scale, float* out, float* lse, int B, int Q, int H,
                  int64_t num_slots, int64_t total_kv, const va::Plan& p, char* ws, hipStream_t st,
                  hipEvent_t ev0, hipEvent_t ev1) {
  auto* chunk_off = reinterpret_cast<int32_t*>(ws + p.off_chunk);
  auto* part_lse = reinterpret_cast<float*>(ws + p.off_lse);
  auto* part_o = reinterpret_cast<_Float16*>(ws + p.off_o);
  hipError_t e = hipSuccess;

  va::SplitArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.kv_pool = static_cast<const char*>(kv_pool);
  a.kv_indices = kv_indices;
  a.prefix_lens = prefix_lens;
  a.tree_mask = tree_mask;
  a.chunk_off = chunk_off;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.num_slots = num_slots;
  a.total_kv = total_kv;
  a.B = B;
  a.Q = Q;
  a.H = H;
  a.R = Q * H;
  a.row_tiles = p.row_tiles;
  a.ideal_keys = p.ideal_keys;
  a.target = p.target;
  a.max_chunks = p.max_chunks;
  a.c_log2 = scale * 1.4426950408889634f;
  if (ev0 != nullptr && (e = hipEventRecord(ev0, st)) != hipSuccess)
    return fail(VA_EHIP, "event record: %s", hipGetErrorString(e));
  e = va::launch_split(a, p.grid, st);
  if (e != hipSuccess) return fail(VA_EHIP, "split launch: %s", hipGetErrorString(e));
  if (ev1 != nullptr && (e = hipEventRecord(ev1, st)) != hipSuccess)
    return fail(VA_EHIP, "event record: %s", hipGetErrorString(e));

  e = va::launch_merge(part_o, part_lse, chunk_off, out, lse, B, Q * H, p.max_chunks, st);
  if (e != hipSuccess) return fail(VA_EHIP, "merge launch: %s", hipGetErrorString(e));
  return ok();
}

int verify_with_workspace(const void* q, const void* kv_pool, const int32_t* kv_indices,
                          const int32_t* prefix_lens, const uint8_t* tree_mask, float scale, float* out,
                          float* lse, int B, int Q, int H, int64_t num_slots, int64_t total_kv, void* workspace,
                          size_t workspace_bytes, void* stream, int32_t chunk_keys, hipEvent_t ev0,
                          hipEvent_t ev1) {
  try {
    va::Plan p;
    const int rc = check_verify_args(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, out, lse, B, Q, H,
                                     num_slots, total_kv, chunk_keys, &p);
    if (rc != VA_OK) return rc;
    if (!workspace) return fail(VA_EINVAL, "null pointer argument");
    if (!aligned(workspace, 256)) return fail(VA_EINVAL, "workspace must be 256-byte aligned");
    if (workspace_bytes < p.bytes)
      return fail(VA_ENOSPC, "workspace of %zu bytes < %zu needed", workspace_bytes, p.bytes);
    return launch_verify(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, out, lse, B, Q, H, num_slots,
                         total_kv, p, static_cast<char*>(workspace), static_cast<hipStream_t>(stream), ev0, ev1);
  } catch (...) {
    return fail(VA_EHIP, "unexpected C++ exception");
  }
}

}  // namespace

extern "C" {

size_t verify_attn_workspace_size(int B, int Q, int H, int64_t total_kv) {
  return verify_attn_workspace_size_ex(B, Q, H, total_kv, 0);
}

size_t verify_attn_workspace_size_ex(int B, int Q, int H, int64_t total_kv, int32_t chunk_keys) {
  va::Plan p;
  if (chunk_keys < 0 || !make_plan(B, Q, H, total_kv, cu_count(), chunk_keys, &p)) return 0;
  return p.bytes;
}

int verify_attn_query_plan(int B, int Q, int H, int64_t total_kv, int32_t chunk_keys_in, int32_t* chunk_keys,
                           int32_t* max_chunks, int32_t* row_tiles, int32_t* grid) {
  va::Plan p;
  if (chunk_keys_in < 0 || !make_plan(B, Q, H, total_kv, cu_count(), chunk_keys_in, &p))
    return fail(VA_EINVAL, "invalid sizes");
  if (chunk_keys) *chunk_keys = p.ideal_keys;
  if (max_chunks) *max_chunks = p.max_chunks;
  if (row_tiles) *row_tiles = p.row_tiles;
  if (grid) *grid = p.grid;
  return ok();
}

const char* verify_attn_last_error(void) { return g_last_error.c_str(); }

int verify_attn(const void* q, const void* kv_pool, const int32_t* kv_indices,
                const int32_t* prefix_lens, const uint8_t* tree_mask, float scale, float* out,
                float* lse, int B, int Q, int H, int64_t num_slots, int64_t total_kv,
                void* workspace, size_t workspace_bytes, void* stream) {
  return verify_with_workspace(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, out, lse, B, Q, H,
                               num_slots, total_kv, workspace, workspace_bytes, stream, 0, nullptr, nullptr);
}

int verify_attn_noalloc(const void* q, const void* kv_pool, const int32_t* kv_indices,
                        const int32_t* prefix_lens, const uint8_t* tree_mask, float scale, float* out,
                        float* lse, int B, int Q, int H, int64_t num_slots, int64_t total_kv, void* stream) {
  try {
    va::Plan p;
    const int rc = check_verify_args(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, out, lse, B, Q, H,
                                     num_slots, total_kv, 0, &p);
    if (rc != VA_OK) return rc;
    if (p.bytes > va::kNoAllocScratchBytes)
      return fail(VA_ENOSPC, "these sizes need %zu bytes of scratch; the allocation-free entry point has a "
                  "fixed %zu (use verify_attn with a workspace)", p.bytes, va::kNoAllocScratchBytes);
    void* ws = nullptr;
    const hipError_t e = va::noalloc_scratch(&ws);
    if (e != hipSuccess) return fail(VA_EHIP, "scratch lookup: %s", hipGetErrorString(e));
    return launch_verify(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, out, lse, B, Q, H, num_slots,
                         total_kv, p, static_cast<char*>(ws), static_cast<hipStream_t>(stream), nullptr, nullptr);
  } catch (...) {
    return fail(VA_EHIP, "unexpected C++ exception");
  }
}

int verify_attn_ex(const void* q, const void* kv_pool, const int32_t* kv_indices, const int32_t* prefix_lens,
                   const uint8_t* tree_mask, float scale, float* out, float* lse, int B, int Q, int H,
                   int64_t num_slots, int64_t total_kv, void* workspace, size_t workspace_bytes, void* stream,
                   const va_test_options* opts) {
  const int32_t ck = opts ? opts->chunk_keys : 0;
  hipEvent_t e0 = opts ? static_cast<hipEvent_t>(opts->split_start_event) : nullptr;
  hipEvent_t e1 = opts ? static_cast<hipEvent_t>(opts->split_stop_event) : nullptr;
  return verify_with_workspace(q, kv_pool, kv_indices, prefix_lens, tree_mask, scale, out, lse, B, Q, H,
                               num_slots, total_kv, workspace, workspace_bytes, stream, ck, e0, e1);
}

int verify_attn_debug_gather(const void* kv_pool, const int32_t* kv_indices, int64_t n,
                             int64_t num_slots, void* rows_out, void* stream) {
  try {
    if (n < 0 || n > (int64_t)INT32_MAX * 16) return fail(VA_EINVAL, "bad n %lld", (long long)n);
    if (n == 0) return ok();
    if (!kv_pool || !kv_indices || !rows_out) return fail(VA_EINVAL, "null pointer argument");
    if (!aligned(kv_pool, 16) || !aligned(rows_out, 16) || !aligned(kv_indices, 4))
      return fail(VA_EINVAL, "kv_pool/rows_out must be 16-byte and kv_indices 4-byte aligned");
    if (num_slots < 1 || num_slots > INT64_MAX / va::kRowBytes)
      return fail(VA_EINVAL, "bad num_slots %lld", (long long)num_slots);
    hipError_t e = va::launch_debug_gather(kv_pool, kv_indices, n, num_slots, rows_out,
                                           static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(VA_EHIP, "debug gather launch: %s", hipGetErrorString(e));
    return ok();
  } catch (...) {
    return fail(VA_EHIP, "unexpected C++ exception");
  }
}

int verify_attn_kv_defrag(const void* src_pool, const int32_t* kv_indices, int64_t n, int64_t num_slots,
                          void* dst_pool, int64_t dst_base, int64_t dst_slots, int32_t* new_indices,
                          void* stream) {
  try {
    if (n < 0 || n > (int64_t)INT32_MAX) return fail(VA_EINVAL, "bad n %lld", (long long)n);
    if (n == 0) return ok();
    if (!src_pool || !kv_indices || !dst_pool || !new_indices) return fail(VA_EINVAL, "null pointer argument");
    if (!aligned(src_pool, 16) || !aligned(dst_pool, 16) || !aligned(kv_indices, 4) || !aligned(new_indices, 4))
      return fail(VA_EINVAL, "pools must be 16-byte and index arrays 4-byte aligned");
    if (num_slots < 1 || num_slots > INT64_MAX / va::kRowBytes)
      return fail(VA_EINVAL, "bad num_slots %lld", (long long)num_slots);
    if (dst_slots < 1 || dst_slots > INT64_MAX / va::kRowBytes)
      return fail(VA_EINVAL, "bad dst_slots %lld", (long long)dst_slots);
    if (dst_base < 0 || dst_base > dst_slots - n || dst_base + n - 1 > (int64_t)INT32_MAX)
      return fail(VA_EINVAL, "destination run [%lld, %lld) outside [0, %lld) or past int32 slots",
                  (long long)dst_base, (long long)(dst_base + n), (long long)dst_slots);
    hipError_t e = va::launch_defrag(src_pool, kv_indices, n, num_slots, dst_pool, dst_base, new_indices,
                                     static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(VA_EHIP, "defrag launch: %s", hipGetErrorString(e));
    return ok();
  } catch (...) {
    return fail(VA_EHIP, "unexpected C++ exception");
  }
}

int verify_attn_tree_accept(const int32_t* parents, const int32_t* draft_tokens, const int32_t* target_tokens,
                            int B, int Q, int32_t* accept_len, int32_t* accepted, int32_t* bonus_token,
                            void* stream) {
  try {
    if (B < 1 || Q < 1 || Q > VA_MAX_Q) return fail(VA_EINVAL, "bad B=%d or Q=%d", B, Q);
    if (!parents || !draft_tokens || !target_tokens || !accept_len || !accepted || !bonus_token)
      return fail(VA_EINVAL, "null pointer argument");
    if (!aligned(parents, 4) || !aligned(draft_tokens, 4) || !aligned(target_tokens, 4) ||
        !aligned(accept_len, 4) || !aligned(accepted, 4) || !aligned(bonus_token, 4))
      return fail(VA_EINVAL, "arrays must be 4-byte aligned");
    hipError_t e = va::launch_tree_accept(parents, draft_tokens, target_tokens, B, Q, accept_len, accepted,
                                          bonus_token, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(VA_EHIP, "tree accept launch: %s", hipGetErrorString(e));
    return ok();
  } catch (...) {
    return fail(VA_EHIP, "unexpected C++ exception");
  }
}

}  // extern "C"
