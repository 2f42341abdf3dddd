// Internal interface between the C-ABI shim (capi.cpp) and the HIP kernels
// (verify_attn_kernels.hip). Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace va {

constexpr int kLatent = 576;           // key width (bf16 elements per latent row)
constexpr int kValue = 512;            // value width (leading dims of the row)
constexpr int kRowBytes = kLatent * 2; // 1152 bytes per pool row
constexpr int kUnit = 32;              // keys per LDS tile
constexpr int kRowsPerBlock = 32;      // query-head rows of one 32x32 MFMA score block
constexpr int kRowBlocksPerWG = 4;     // score blocks per workgroup (one per wave pair)
constexpr int kRowsPerWG = kRowsPerBlock * kRowBlocksPerWG;  // 128 rows per row tile
constexpr int kMinChunk = 128;         // smallest chunk worth a workgroup (keys): four tiles
constexpr int kPlanThreads = 512;      // threads of the split workgroup, which plans the pieces: the
                                       // column plan runs for batches of at most this many sequences

// Host-side split plan (the split kernel plans the pieces from the sequence
// lengths: equal columns of the batch's key tiles, at most `target` of them,
// when there are fewer sequences than that, else chunks of ideal_keys keys).
struct Plan {
  int32_t row_tiles;    // ceil(Q*H / 128)
  int32_t target;       // column budget over the whole batch; 0 = chunks of ideal_keys as is
  int32_t ideal_keys;   // keys per column that would hit `target` exactly (multiple of 32)
  int32_t max_chunks;   // capacity of the partial buffers (pieces)
  int32_t grid;         // split-kernel workgroups
  size_t off_chunk;     // workspace byte offsets

  size_t off_lse;
  size_t off_o;
  size_t bytes;         // total workspace bytes
};

struct SplitArgs {
  const uint16_t* q;
  const char* kv_pool;
  const int32_t* kv_indices;
  const int32_t* prefix_lens;
  const uint8_t* tree_mask;
  int32_t* chunk_off;      // written by workgroup 0: [B + 1] piece offsets for the merge
  _Float16* part_o;       // [max_chunks][R][512] fp16, normalised (O / l)
  float* part_lse;
  int64_t num_slots;
  int64_t total_kv;
  int32_t B, Q, H, R, row_tiles;
  int32_t ideal_keys, target, max_chunks;   // chunk plan inputs (see Plan)
  float c_log2;  // scale * log2(e)
};

hipError_t launch_split(const SplitArgs& a, int grid, hipStream_t stream);
// Size of the allocation-free entry point's fixed device scratch, and its
// device address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);
// The merge: the one-wave-per-row form when the partial buffers hold at most
// kMergeFewPerSeq chunks per sequence on average, the slice form when they hold
// at least kMergeSlicePerSeq (few rows, many chunks: the 8-head shape), else
// the chunk-lane form.
constexpr int kMergeFewPerSeq = 16;
constexpr int kMergeSlicePerSeq = 64;
hipError_t launch_merge(const _Float16* part_o, const float* part_lse, const int32_t* chunk_off,
                        float* out, float* lse, int B, int R, int max_chunks, hipStream_t stream);
hipError_t launch_debug_gather(const void* kv_pool, const int32_t* kv_indices, int64_t n,
                               int64_t num_slots, void* rows_out, hipStream_t stream);
hipError_t launch_defrag(const void* src_pool, const int32_t* kv_indices, int64_t n, int64_t num_slots,
                         void* dst_pool, int64_t dst_base, int32_t* new_indices, hipStream_t stream);
hipError_t launch_tree_accept(const int32_t* parents, const int32_t* draft, const int32_t* target, int B,
                              int Q, int32_t* accept_len, int32_t* accepted, int32_t* bonus,
                              hipStream_t stream);

}  // namespace va
