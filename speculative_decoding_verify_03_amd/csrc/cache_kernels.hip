// HIP kernels for the steps next to verify attention on gfx950 (MI355X):
// KV-cache defragmentation and draft-tree acceptance.
//
// Defragmentation (page "The Build That Unlocked 3-6x Decode Speedup",
// sections "The Context: A Custom Kernel for an Unsupported Architecture" and
// "The Broader Significance", where it is named as the next step): the rows
// a position list points to are copied in position order into a contiguous
// destination run and the index table is rewritten, so a later verify call
// gathers consecutive rows.
//
// Tree acceptance (the tree_accept kernel source listed next to the verify
// kernels on the same page, section "Why This Build Was Different"): a
// greedy walk of the draft tree from the root, stepping to the smallest
// child whose draft token equals the target's choice at the current node.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "va_internal.hpp"

namespace va {

typedef unsigned u32x4c __attribute__((ext_vector_type(4)));

constexpr int kRowChunks = kRowBytes / 16;   // 72 sixteen-byte chunks per latent row
constexpr int kDefragThreads = 256;
constexpr int kDefragRows = 32;              // positions per workgroup
constexpr int kDefragPerThread = kDefragRows * kRowChunks / kDefragThreads;   // 9 chunks in flight
static_assert(kDefragRows * kRowChunks % kDefragThreads == 0, "defrag chunk split");

// ---------------------------------------------------------------------------
// Defragmentation: one workgroup copies 32 positions. Their 32 slot indices
// are read once (one coalesced load) into LDS, and the new indices written;
// then chunk t of the workgroup's 32 * 72 chunks is chunk t % 72 of position
// t / 72, thread i taking chunks i + 256k. Consecutive threads take
// consecutive chunks, so a wave reads and writes whole 1152-byte rows with
// 16-byte accesses, and each thread has all nine of its loads in flight
// before its stores. Source rows and the destination run are touched once,
// so both go around the caches' normal replacement (nontemporal).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kDefragThreads) defrag_kernel(const u32x4c* __restrict__ src,
                                                                const int32_t* __restrict__ kv_indices,
                                                                int64_t n, int64_t num_slots,
                                                                u32x4c* __restrict__ dst, int64_t dst_base,
                                                                int32_t* __restrict__ new_indices) {
  __shared__ int32_t s_slot[kDefragRows];
  const int64_t row0 = (int64_t)blockIdx.x * kDefragRows;
  const int tid = threadIdx.x;
  if (tid < kDefragRows) {
    const int64_t j = row0 + tid;
    int32_t slot = -1;
    if (j < n) {
      slot = kv_indices[j];
      new_indices[j] = (int32_t)(dst_base + j);
    }
    s_slot[tid] = (slot >= 0 && slot < num_slots) ? slot : -1;
  }
  __syncthreads();
  u32x4c v[kDefragPerThread];
#pragma unroll
  for (int i = 0; i < kDefragPerThread; ++i) {
    const int t = tid + i * kDefragThreads;
    const int r = t / kRowChunks;
    const int c = t - r * kRowChunks;
    const int32_t slot = s_slot[r];
    v[i] = u32x4c{0, 0, 0, 0};
    if (row0 + r < n && slot >= 0) v[i] = __builtin_nontemporal_load(&src[(int64_t)slot * kRowChunks + c]);
  }
#pragma unroll
  for (int i = 0; i < kDefragPerThread; ++i) {
    const int t = tid + i * kDefragThreads;
    const int r = t / kRowChunks;
    const int c = t - r * kRowChunks;
    if (row0 + r < n) __builtin_nontemporal_store(v[i], &dst[(dst_base + row0 + r) * kRowChunks + c]);
  }
}

// ---------------------------------------------------------------------------
// Tree acceptance: one wave per sequence, lane i holds node i (Q <= 64). At
// each step the lanes whose node is a child of the current node (with a
// larger index, which every well-formed tree satisfies and which bounds the
// walk at Q - 1 steps) and whose draft token equals the target's choice at
// the current node vote; the lowest voting lane is the next node.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) tree_accept_kernel(const int32_t* __restrict__ parents,
                                                         const int32_t* __restrict__ draft,
                                                         const int32_t* __restrict__ target, int Q,
                                                         int32_t* __restrict__ accept_len,
                                                         int32_t* __restrict__ accepted,
                                                         int32_t* __restrict__ bonus) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int64_t row = (int64_t)b * Q;
  const bool node = lane < Q;
  const int32_t par = node ? parents[row + lane] : -2;
  const int32_t tok = node ? draft[row + lane] : 0;
  int cur = 0;
  int len = 0;
  int32_t my_path = lane == 0 ? 0 : -1;   // entry `lane` of the accepted path
  for (int step = 1; step < Q; ++step) {
    const int32_t want = target[row + cur];
    const bool vote = node && lane > cur && par == cur && tok == want;
    const uint64_t m = __ballot(vote);
    if (m == 0) break;
    cur = __builtin_ctzll(m);
    len = step;
    if (lane == step) my_path = cur;
  }
  if (node) accepted[row + lane] = lane <= len ? my_path : -1;
  if (lane == 0) {
    accept_len[b] = len;
    bonus[b] = target[row + cur];
  }
}

hipError_t launch_defrag(const void* src_pool, const int32_t* kv_indices, int64_t n, int64_t num_slots,
                         void* dst_pool, int64_t dst_base, int32_t* new_indices, hipStream_t stream) {
  const int64_t grid = (n + kDefragRows - 1) / kDefragRows;
  hipLaunchKernelGGL(defrag_kernel, dim3((unsigned)grid), dim3(kDefragThreads), 0, stream,
                     static_cast<const u32x4c*>(src_pool), kv_indices, n, num_slots,
                     static_cast<u32x4c*>(dst_pool), dst_base, new_indices);
  return hipGetLastError();
}

hipError_t launch_tree_accept(const int32_t* parents, const int32_t* draft, const int32_t* target, int B,
                              int Q, int32_t* accept_len, int32_t* accepted, int32_t* bonus,
                              hipStream_t stream) {
  hipLaunchKernelGGL(tree_accept_kernel, dim3((unsigned)B), dim3(64), 0, stream, parents, draft, target, Q,
                     accept_len, accepted, bonus);
  return hipGetLastError();
}

}  // namespace va
