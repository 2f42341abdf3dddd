// HIP kernels for MLA speculative-decoding verify attention on gfx950 (MI355X).
//
// Method (page "The Build That Unlocked 3-6x Decode Speedup", section "The
// Context: A Custom Kernel for an Unsupported Architecture"; page "The Build
// That Bridged Design and Deployment: Compiling the Custom sm_120 Verify
// Kernel", section "What This Build Achieves: The paged+bf16 Kernel"):
// flash-decode. The KV positions of the batch are cut into pieces (whole
// columns of the batch's key tiles, one piece per sequence a column meets);
// every (column, 128-row tile) pair is one workgroup that streams its pieces
// through LDS in 32-key tiles with an online softmax, leaving one partial per
// piece, and a second kernel merges each sequence's partials by log-sum-exp.
//
// gfx950 mapping, per workgroup (8 waves, two per SIMD, 128 query-head rows):
//  * gather: every 32-key tile is brought into LDS with 16-byte direct
//    global->LDS loads through kv_indices (page_size 1, 1152-byte rows), one
//    whole 128-byte line per 8 lanes, all issued by one half of the waves; a
//    3-slot ring holds the tile being applied, the next one, and one in flight;
//  * scores: S^T = K Q^T on MFMA 32x32x16 bf16. K comes from LDS (A operand);
//    each pair of waves keeps its 32 query rows resident in VGPRs (B operand),
//    split by latent dims. All heads and verify positions of the tile share
//    every latent row that is loaded;
//  * softmax: one wave per pair owns it; each lane owns one row, so the running
//    max needs one cross-half exchange per tile; rescaling is lazy (only when
//    a row max grows by more than 2^8);
//  * values: O^T += V^T P^T on MFMA 32x32x16 fp16. P^T is the score
//    accumulator layout itself (published through LDS), V^T is read from the
//    same LDS tile with the gfx950 transpose read ds_read_b64_tr_b16 and
//    converted bf16 -> fp16 in registers. P is fp16 (not bf16) for accuracy:
//    fp16 keeps 11 significant bits against bf16's 8;
//  * partials: each piece leaves O / l in fp16 (bounded by the largest |value|
//    of the piece) and its lse in fp32; the merge folds them in fp32.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "va_internal.hpp"

namespace va {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kChunks = kRowBytes / 16;          // 72 chunk columns per row
constexpr int kTileBytes = kUnit * kRowBytes;    // 36864 bytes per tile
constexpr int kKSteps = kLatent / 16;            // 36 MFMA k-steps over the latent
constexpr int kDvBlocks = kValue / 32;           // 16 value blocks of 32 dims
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;             // log2 headroom before O is rescaled

// An all-zero latent row: the gather source for absent positions, so LDS
// never holds anything but finite data and a masked key contributes 0 * 0.
__device__ __attribute__((aligned(16))) uint32_t g_zero_row[kRowBytes / 4] = {0};

// Byte offset of (16-byte chunk c, key k) inside one LDS tile. The tile is
// 36 regions of 1 KiB, one per (group of 8 keys, 128-byte line of the row);
// inside a region, key k%8 owns 8 slots and chunk c%8 sits at slot
// (c%8) ^ ((k >> 1) & 7). The xor spreads both the score reads (32 keys, one
// chunk) and the value transpose reads over all banks.
__host__ __device__ constexpr int tile_offset(int chunk, int key) {
  return ((key >> 3) * 9 + (chunk >> 3)) * 1024 + ((key & 7) * 8 + ((chunk & 7) ^ ((key >> 1) & 7))) * 16;
}

// The gather is line-granular and done by four waves, nine load instructions
// each per tile. One instruction fills one 1 KiB region (key group kg, line L):
// lane l fetches, of key 8kg + l/8, the 16-byte chunk of line L that lands in
// slot l%8 of the region, so every instruction moves 8 whole 128-byte lines.
// Gather wave j owns key group j: all nine lines of keys 8j .. 8j + 7, so each
// lane needs the pool slot of one key only. In the split kernel a tile slot is
// refilled while other waves may still be reading the slot's previous tile
// unless every read of that tile ends before the refill's phase barrier; the
// check after the split kernel's layout constants proves, over the tables
// below and the phase in which each wave reads its value lines, that no
// refill overwrites a region another wave still reads.
constexpr int kGatherWaves = kUnit / 8;
constexpr int kGatherLoads = kRowBytes / 128;   // 9 load instructions per wave and tile
constexpr int kKeyGroups = kUnit / 8;           // 4 groups of 8 keys per tile
static_assert(kGatherWaves == kKeyGroups, "one gather wave per key group");

__host__ __device__ constexpr int gather_kg(int j, int k) { return j + 0 * k; }
__host__ __device__ constexpr int gather_line(int j, int k) { return k + 0 * j; }
__host__ __device__ constexpr bool gather_lines_in_order() {
  for (int j = 0; j < kKeyGroups; ++j)
    for (int k = 0; k < kGatherLoads; ++k)
      if (gather_line(j, k) != k) return false;
  return kGatherLoads == 9;
}
// Line of a tile whose value operands wave w reads (its 64 value dims are
// chunks 8w .. 8w + 7; see value_chunk).
__host__ __device__ constexpr int value_line(int w) { return w; }
// Value chunk read by lane (g = lane/16, s = lane%16) of wave w for value
// block d of that wave.
__host__ __device__ constexpr int value_chunk(int w, int d, int g, int s) {
  return 8 * value_line(w) + 4 * d + 2 * (g & 1) + ((s & 3) >> 1);
}

// Score A operand: A-row n of a 32x32x16 block holds key arow_key(n) (bits 2
// and 3 of n swapped), so that the score accumulator element i of lane
// (n + 32h) is key 16*(i/8) + 8h + (i%8), the B-operand layout of P. K-step ks
// of dim half p reads chunk 2(18p + ks) + h; within the 1 KiB region of a key
// group and line, the swizzle of tile_offset only flips slot bits (4..6) of
// the offset, so k-steps j = 0..3 follow from k-step 0 by an XOR (and, in dim
// half 1, k-steps 2 and 3 lie in the next region); k-step j + 4q adds q KiB.
__host__ __device__ constexpr int arow_key(int n) { return (n & ~12) | ((n & 4) << 1) | ((n & 8) >> 1); }
__host__ __device__ constexpr int score_koff(int a0, int j, int p) {
  return (a0 ^ (32 * j)) + ((p == 1 && j >= 2) ? 1024 : 0);
}
// Value transpose read (hf, d) from read (0, 0): key 4hf further (+512 bytes)
// flips slot bit 1, value block d flips slot bit 2.
__host__ __device__ constexpr int value_off(int t00, int hf, int d) { return ((t00 + 512 * hf) ^ (32 * hf)) ^ (64 * d); }
// Both derivations reproduce tile_offset for every lane, wave and dim half.
// (Tile bases are multiples of 1 KiB, so the XORs may act on absolute LDS
// addresses as well as on offsets.)
__host__ __device__ constexpr bool lane_offsets_ok() {
  for (int p = 0; p < 2; ++p)
    for (int lane = 0; lane < 64; ++lane) {
      const int nn = lane & 31, hh = lane >> 5;
      const int a0 = tile_offset(36 * p + hh, arow_key(nn));
      for (int j = 0; j < 4; ++j)
        for (int q = 0; q < 5; ++q) {
          if (4 * q + j >= 18) continue;
          if (tile_offset(2 * (18 * p + 4 * q + j) + hh, arow_key(nn)) != score_koff(a0, j, p) + 1024 * q) return false;
        }
    }
  for (int w = 0; w < 8; ++w)
    for (int lane = 0; lane < 64; ++lane) {
      const int g = lane >> 4, s = lane & 15, hh = lane >> 5;
      const int t00 = tile_offset(value_chunk(w, 0, g, s), 8 * hh + (s >> 2)) + (s & 1) * 8;
      for (int hf = 0; hf < 2; ++hf)
        for (int d = 0; d < 2; ++d)
          for (int t = 0; t < 2; ++t)
            if (tile_offset(value_chunk(w, d, g, s), 16 * t + 8 * hh + 4 * hf + (s >> 2)) + (s & 1) * 8 !=
                value_off(t00, hf, d) + 18432 * t)
              return false;
    }
  return (kUnit * kRowBytes) % 1024 == 0;
}
static_assert(lane_offsets_ok(), "derived LDS operand offsets differ from tile_offset");

struct GatherLane {
  int key;   // key of the tile this lane fetches
  int coff;  // byte offset of its chunk inside a 128-byte line
  int kg;    // key group (region row)
};

__device__ __forceinline__ GatherLane gather_lane(int gw, int lane) {
  GatherLane g;
  g.kg = gather_kg(gw, 0);
  g.key = 8 * g.kg + (lane >> 3);
  g.coff = ((lane & 7) ^ ((g.key >> 1) & 7)) * 16;
  return g;
}

// Direct-to-LDS loads, written out in asm. (Issued through the builtin, an LDS
// DMA anywhere in a wave's code makes the compiler wait for every LDS read of
// that wave with lgkmcnt(0), draining the operand reads queued ahead of each
// MFMA.) M0 carries the wave-uniform LDS destination and is restored after
// the load. The loads write LDS only, so no register is left pending; their
// completion is awaited with explicit vmcnt waits, and the compiler's own
// vmcnt waits only grow stricter for not counting them.
// The nine lines of one key group in one block: line L reads gaddr + 128 L
// into lds_dst + 1024 L. The instruction offset (128 L) is added to the
// global and to the LDS address alike, so M0 advances by 1024 - 128 per line
// and the lane's address register serves all nine loads. (An SALU write of M0
// needs one wait state before an LDS DMA reads it: the s_nop after each.)
__device__ __forceinline__ void lds_dma16_nt_lines9(const char* gaddr, LDS_AS char* lds_dst) {
  const unsigned lb = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_dst);
  unsigned saved;
  asm volatile("s_mov_b32 %0, m0\n\t"
               "s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt\n\t"
               "s_add_u32 m0, m0, 0x380\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:128 nt\n\t"
               "s_add_u32 m0, m0, 0x380\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:256 nt\n\t"
               "s_add_u32 m0, m0, 0x380\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:384 nt\n\t"
               "s_add_u32 m0, m0, 0x380\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:512 nt\n\t"
               "s_add_u32 m0, m0, 0x380\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:640 nt\n\t"
               "s_add_u32 m0, m0, 0x380\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:768 nt\n\t"
               "s_add_u32 m0, m0, 0x380\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:896 nt\n\t"
               "s_add_u32 m0, m0, 0x380\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off offset:1024 nt\n\t"
               "s_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(gaddr), "s"(lb) : "memory", "scc");
}
__device__ __forceinline__ void lds_dma4(const void* gaddr, LDS_AS char* lds_dst) {
  const unsigned lb = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_dst);
  unsigned saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(gaddr), "s"(lb) : "memory");
}

// Issue this wave's share of one tile gather (exactly kGatherLoads load
// instructions, regions as in gather_kg / gather_line). `slot` is the pool row
// of the lane's key (any out-of-range value for an absent position: the zero
// row). The loads carry the nontemporal cache policy (nt): a workgroup reads
// each row once, and with it one CU sustains about twice the gather rate it
// reaches under the default policy.
__device__ __forceinline__ void issue_tile_gather(const char* kv_pool, int64_t num_slots, int32_t slot,
                                                  LDS_AS char* tile, const GatherLane& gl) {
  const char* row = (slot >= 0 && slot < num_slots) ? kv_pool + (int64_t)slot * kRowBytes
                                                    : reinterpret_cast<const char*>(g_zero_row);
  row += gl.coff;
  static_assert(gather_lines_in_order(), "lds_dma16_nt_lines9 issues lines 0..8 in order");
  lds_dma16_nt_lines9(row, tile + gl.kg * 9 * 1024);
}

__device__ __forceinline__ LDS_AS char* lds_cast(char* p) { return (LDS_AS char*)(p); }

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// x of lane l ^ 32 (the other half of the wave); `addr` = 4 (l ^ 32).
__device__ __forceinline__ float swap_halves(float x, int addr) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(x)));
}


// The lane id, re-derived where it is used: as a volatile asm result it cannot
// be hoisted out of a loop, so per-lane addresses built from it are
// recomputed in place instead of occupying registers across the loop.
// A wave-uniform 64-bit value, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// bf16 x 4 (as raw bits, two per dword) -> fp16 x 4; exact for |v| in the
// fp16 normal range.
__device__ __forceinline__ void bf16x4_to_f16(u32x2 v, f16x8& dst, int base) {
  const unsigned lo = v[0];
  const unsigned hi = v[1];
  const float a0 = __builtin_bit_cast(float, lo << 16);
  const float a1 = __builtin_bit_cast(float, lo & 0xffff0000u);
  const float a2 = __builtin_bit_cast(float, hi << 16);
  const float a3 = __builtin_bit_cast(float, hi & 0xffff0000u);
  dst[base + 0] = (_Float16)a0;
  dst[base + 1] = (_Float16)a1;
  dst[base + 2] = (_Float16)a2;
  dst[base + 3] = (_Float16)a3;
}

// ---------------------------------------------------------------------------
// Split plans, computed by every split workgroup at its start (identically,
// from prefix_lens alone). Sequence b has N_b = clamped prefix + Q keys, and
// its positions start at the running sum of N. Under either plan it owns the
// partials [chunk_off[b], chunk_off[b+1]), which workgroup 0 writes for the
// merge.
//
// Column plan (a chunk budget, target > 0, above the number of sequences, and
// at most 512 sequences): the batch's 32-key tiles are laid end to end,
// sequence after sequence, each sequence's tiles preceded by kSeqUnits units
// that stand for what starting a piece costs (a prologue and an epilogue),
// and this axis is cut into columns of ceil(U / C) units (U the axis length,
// C = min(target, max_chunks - B + 1, launched columns)), one per workgroup
// of each row tile. A column runs one piece per sequence whose tiles it
// meets, so the workgroups end within about a tile of each other whatever the
// sequences' lengths. There are at most C + B - 1 pieces, which the partial
// buffers hold.
//
// Chunk plan (otherwise): one chunk length L = ideal_keys for the batch;
// sequence b owns ceil(N_b / L) chunks, and chunk c is workgroup c's piece.
// ---------------------------------------------------------------------------

// What one workgroup (one column of row tiles) does: nseg pieces, each a key
// range of one sequence with a partial of its own. The first piece is given in
// full; under the column plan (below) the next one, if any, is always the next
// sequence from its first key, with partial index c + 1.
struct ChunkPlan {
  int64_t sbase;    // first position of the first piece's sequence
  int64_t P;        // its clamped prefix length
  int64_t kstart;   // the piece's keys [kstart, kend) within its sequence
  int64_t kend;
  int64_t ubase;    // column plan: axis unit where that sequence's tiles start
  int64_t uend;     // column plan: axis unit where the column ends
  int32_t b;        // the piece's sequence
  int32_t c;        // its partial index
  int32_t nseg;     // pieces of this workgroup (0: nothing to do)
};

// Sum over the kPlanThreads threads of the workgroup; every thread gets the total.
// `red` holds 8 int64 in LDS.
__device__ __forceinline__ int64_t block_sum(int64_t v, LDS_AS int64_t* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();   // readers of the previous sum are done
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int64_t t = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) t += red[w];
  return t;
}

// Inclusive prefix sum over the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_scan(T v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  return v;
}

// All kPlanThreads threads call this with the same c. `scratch` is 256 bytes of LDS
// that nothing else uses until the workgroup's next barrier after the call.
// The workgroup that gets write_offsets stores chunk_off[0..B] for the merge.
__device__ ChunkPlan chunk_plan(const SplitArgs& a, int c, bool write_offsets, LDS_AS char* scratch) {
  LDS_AS int64_t* red = reinterpret_cast<LDS_AS int64_t*>(scratch);        // 8 sums
  LDS_AS int64_t* wn = red + 8;                                            // 8 wave totals of N
  LDS_AS int32_t* wc = reinterpret_cast<LDS_AS int32_t*>(red + 16);        // 8 wave totals of chunks
  LDS_AS int64_t* own = red + 20;                                          // b, coff, sbase, P of chunk c
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.B;
  auto keys_of = [&](int i) -> int64_t {
    int64_t pl = a.prefix_lens[i];
    pl = pl < 0 ? 0 : (pl > a.total_kv ? a.total_kv : pl);
    return pl + a.Q;
  };
  if (tid == 0) own[0] = -1;

  const int64_t L = a.ideal_keys;

  // Running sums over the batch, kPlanThreads sequences per pass.
  int64_t carry_n = 0;
  int32_t carry_c = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int i = base + tid;
    const int64_t nb = i < B ? keys_of(i) : 0;
    const int32_t cb = i < B ? (int32_t)((nb + L - 1) / L) : 0;
    int64_t in_n = wave_scan(nb, lane);
    int32_t in_c = wave_scan(cb, lane);
    __syncthreads();   // readers of the previous pass's totals are done
    if (lane == 63) {
      wn[wave] = in_n;
      wc[wave] = in_c;
    }
    __syncthreads();
    int64_t tot_n = 0;
    int32_t tot_c = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      if (w < wave) {
        in_n += wn[w];
        in_c += wc[w];
      }
      tot_n += wn[w];
      tot_c += wc[w];
    }
    const int32_t ex_c = carry_c + in_c - cb;
    const int64_t ex_n = carry_n + in_n - nb;
    if (i < B && ex_c <= c && c < ex_c + cb) {
      own[0] = i;
      own[1] = ex_c;
      own[2] = ex_n;
      own[3] = nb - a.Q;
    }
    if (write_offsets && i < B) a.chunk_off[i] = ex_c < a.max_chunks ? ex_c : a.max_chunks;
    carry_n += tot_n;
    carry_c += tot_c;
  }
  if (write_offsets && tid == 0) a.chunk_off[B] = carry_c < a.max_chunks ? carry_c : a.max_chunks;
  __syncthreads();
  ChunkPlan cp;
  const int32_t total = carry_c < a.max_chunks ? carry_c : a.max_chunks;
  cp.b = (int32_t)own[0];
  cp.c = c;
  cp.nseg = c < total ? 1 : 0;
  cp.sbase = own[2];
  cp.P = own[3];
  cp.kstart = (int64_t)(c - (int32_t)own[1]) * L;
  cp.kend = cp.kstart + L;
  cp.ubase = cp.uend = 0;
  return cp;
}

// Axis units that stand for starting a piece: about what a second prologue and
// epilogue cost a workgroup, in 32-key tiles of its loop.
constexpr int kSeqUnits = 3;

// Inclusive prefix sum over the 64 lanes of a wave through DPP moves (no LDS
// round trips): three shifts by 1-3 lanes and two by 4 and 8 within each row
// of 16 lanes, then the broadcasts of lanes 15 and 31 into the rows after
// them. Lanes a move does not reach take 0.
__device__ __forceinline__ int32_t wave_scan_dpp(int32_t x) {
  int32_t s = x;
  s += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  s += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  s += __builtin_amdgcn_update_dpp(0, x, 0x113, 0xf, 0xf, false);   // row_shr:3
  s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xf, 0xe, false);   // row_shr:4, lanes 4-15 of a row
  s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xf, 0xc, false);   // row_shr:8, lanes 8-15 of a row
  s += __builtin_amdgcn_update_dpp(0, s, 0x142, 0xa, 0xf, false);   // row_bcast:15, rows 1 and 3
  s += __builtin_amdgcn_update_dpp(0, s, 0x143, 0xc, 0xf, false);   // row_bcast:31, rows 2 and 3
  return s;
}

// The column plan for column g (see above). All kPlanThreads threads call it
// with the same g; `scratch` is 512 bytes of LDS that nothing else uses until
// the workgroup's next barrier after the call. Requires 0 < B <= kPlanThreads
// and target > B. Running sums of keys and axis units are 64-bit (prefix
// lengths need not add up to total_kv); a column's units and its pieces fit
// in 32 bits.
__device__ ChunkPlan column_plan(const SplitArgs& a, int g, bool write_offsets, LDS_AS char* scratch) {
  int C = a.max_chunks - a.B + 1;                   // pieces fit the partial buffers
  if (C > a.target) C = a.target;                   // one wave of workgroups
  const int launched = (int)(gridDim.x / a.row_tiles);
  if (C > launched) C = launched;                   // every column has its workgroups
  if (C < 1) C = 1;
  if (a.B == 1) {
    // One sequence: the same rule in closed form, with no scans and no
    // barriers (its tiles start at unit kSeqUnits; the axis ends after them).
    int64_t pl = a.prefix_lens[0];
    pl = pl < 0 ? 0 : (pl > a.total_kv ? a.total_kv : pl);
    const int64_t U = kSeqUnits + (pl + a.Q + kUnit - 1) / kUnit;
    const int64_t W = (U + C - 1) / C;
    const int64_t cs = kSeqUnits / W, ce = (U - 1) / W;
    if (write_offsets && threadIdx.x == 0) {
      a.chunk_off[0] = 0;
      a.chunk_off[1] = (int32_t)(ce - cs + 1);
    }
    ChunkPlan cp;
    const bool meets = cs <= g && g <= ce;
    cp.b = 0;
    cp.c = (int32_t)(g - cs);
    cp.nseg = meets ? 1 : 0;
    cp.sbase = 0;
    cp.P = pl;
    cp.ubase = kSeqUnits;
    const int64_t lo = (int64_t)g * W;
    cp.uend = lo + W < U ? lo + W : U;
    cp.kstart = ((lo > cp.ubase ? lo : cp.ubase) - cp.ubase) * kUnit;
    cp.kend = (cp.uend - cp.ubase) * kUnit;
    return cp;
  }
  LDS_AS int64_t* wu = reinterpret_cast<LDS_AS int64_t*>(scratch);   // 8 wave totals of units
  LDS_AS int64_t* wn = wu + 8;                                       // 8 wave totals of keys
  LDS_AS int32_t* wp = reinterpret_cast<LDS_AS int32_t*>(wu + 16);   // 8 wave totals of pieces
  LDS_AS int32_t* wm = wp + 8;                                       // 8 wave counts of pieces of column g
  LDS_AS int64_t* own = wu + 24;                                     // the column's first piece
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.B;
  const bool mine = tid < B;   // thread b holds sequence b
  int64_t nb = 0;
  if (mine) {
    int64_t pl = a.prefix_lens[tid];
    pl = pl < 0 ? 0 : (pl > a.total_kv ? a.total_kv : pl);
    nb = pl + a.Q;
  }
  const int64_t tb = (nb + kUnit - 1) / kUnit;   // tiles
  const int64_t ub = mine ? kSeqUnits + tb : 0;   // axis units

  // Inclusive scans of units and keys over the batch (one pass: B <= 512).
  int64_t in_u = wave_scan(ub, lane);
  int64_t in_n = wave_scan(nb, lane);
  if (tid == 0) own[0] = -1;
  if (lane == 63) {
    wu[wave] = in_u;
    wn[wave] = in_n;
  }
  __syncthreads();
  int64_t U = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    if (w < wave) {
      in_u += wu[w];
      in_n += wn[w];
    }
    U += wu[w];
  }
  const int64_t ta = in_u - tb;   // first tile unit of sequence tid; its tiles end at in_u
  const int64_t sb = in_n - nb;   // its first position

  // Columns: column j covers units [j W, min((j + 1) W, U)) with W =
  // ceil(U / C), so unit x lies in column x / W.
  const int64_t W = (U + C - 1) / C;                // uniform: one division
  const bool small = U < ((int64_t)1 << 31);        // always, when the lengths fit the array
  auto col = [&](int64_t x) -> int32_t {
    return small ? (int32_t)((uint32_t)x / (uint32_t)W) : (int32_t)(x / W);
  };
  const int32_t cs = mine ? col(ta) : 0;
  const int32_t ce = mine ? col(in_u - 1) : -1;
  const int32_t np = ce - cs + 1;   // pieces of sequence tid (0 for no sequence)
  // The column's pieces: the sequences whose tiles meet it, which are
  // consecutive; the first is the one whose predecessor's tiles end before it.
  const bool meets = mine && cs <= g && g <= ce;
  int32_t in_p = wave_scan_dpp(np);
  const int32_t wave_meets = (int32_t)__builtin_popcountll(__ballot(meets));   // all lanes take part
  if (lane == 63) wp[wave] = in_p;
  if (lane == 0) wm[wave] = wave_meets;
  __syncthreads();
  int32_t total = 0, nseg = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    if (w < wave) in_p += wp[w];
    total += wp[w];
    nseg += wm[w];
  }
  const int32_t off = in_p - np;
  if (write_offsets && mine) a.chunk_off[tid] = off < a.max_chunks ? off : a.max_chunks;
  if (write_offsets && tid == 0) a.chunk_off[B] = total < a.max_chunks ? total : a.max_chunks;

  const bool first = meets && (tid == 0 || col(ta - kSeqUnits - 1) < g);
  if (first) {
    own[0] = tid;
    own[1] = off + (g - cs);
    own[2] = sb;
    own[3] = nb - a.Q;
    own[4] = ta;
  }
  __syncthreads();
  ChunkPlan cp;
  cp.b = (int32_t)own[0];
  cp.c = (int32_t)own[1];
  cp.sbase = own[2];
  cp.P = own[3];
  cp.ubase = own[4];
  const int64_t lo = (int64_t)g * W;
  cp.uend = lo + W < U ? lo + W : U;
  cp.kstart = ((lo > cp.ubase ? lo : cp.ubase) - cp.ubase) * kUnit;
  cp.kend = (cp.uend - cp.ubase) * kUnit;
  // Bounds that hold by construction, kept so that no piece can index past
  // the sequences or the partial buffers.
  int32_t ns = cp.b < 0 ? 0 : nseg;
  if (cp.b + ns > B) ns = B - cp.b;
  if (cp.c + ns > a.max_chunks) ns = a.max_chunks - cp.c;
  cp.nseg = ns > 0 ? ns : 0;
  return cp;
}

// ---------------------------------------------------------------------------
// Split kernel: one workgroup per (column, 128-row tile).
//
// 8 waves, two per SIMD. Waves j and j+4 (same SIMD) form pair j and own
// query-head rows [32j, 32j + 32) of the tile for the scores: wave half
// p = wave / 4 computes the partial S^T over latent dims [288p, 288p + 288).
// The odd half hands its partial block to the even half through LDS; the even
// wave sums the two, runs the masked online softmax for the pair's 32 rows and
// publishes P (fp16), the rescale factors and a rescale flag in LDS.
// For the values every wave owns a 64-dim slice [64w, 64w + 64) of O^T for all
// 128 rows, so each value element is transposed and converted only once per
// workgroup and tile.
// ---------------------------------------------------------------------------
constexpr int kSplitWaves = 8;
constexpr int kSplitThreads = kSplitWaves * 64;
static_assert(kSplitThreads == kPlanThreads, "the split plan runs on the split workgroup");
constexpr int kRingS = 3;                               // tiles resident in LDS
constexpr int kPairs = 4;
constexpr int kHalfKSteps = kKSteps / 2;                // 18 k-steps per wave
constexpr int kRowBlocks = kRowsPerWG / 32;             // 4 blocks of 32 rows
constexpr int kWaveDvBlocks = kDvBlocks / kSplitWaves;  // 2 value blocks (64 dims) per wave
constexpr int kXchgBytes = 64 * 16 * 4;                 // one 32x32 fp32 score block
constexpr int kPBytes = 2 * 64 * 16;                    // one pair's P: two 16-key k-steps of f16x8
constexpr int kRegKSteps = 16;                          // query k-steps held in VGPRs
constexpr int kLdsKSteps = kHalfKSteps - kRegKSteps;    // the rest are re-read from LDS
constexpr int kQParkBytes = kLdsKSteps * 64 * 16;       // per wave
constexpr int kOffXchg = kRingS * kTileBytes;                      // 110592: partial-score hand-over
constexpr int kOffP = kOffXchg + kPairs * kXchgBytes;              // 126976: P, two tile parities
constexpr int kOffAlpha = kOffP + 2 * kPairs * kPBytes;            // 143360: rescale factors, two parities
constexpr int kOffFlag = kOffAlpha + 2 * kRowsPerWG * 4;           // 144384: rescale flags, two parities
constexpr int kOffSlots = kOffFlag + 64;                           // 144448: slot-index ring
constexpr int kSlotRing = 8;                                       // 256 bytes per tile
constexpr int kGatherAhead = 3;                                    // tile u+3 is gathered while tile u is applied
constexpr int kSlotAhead = 5;                                      // slot copy distance, tiles
constexpr int kOffQPark = kOffSlots + kSlotRing * 256;             // 146496
constexpr int kOffPlan = kOffQPark + kSplitWaves * kQParkBytes;    // 162880: the column's first piece
constexpr int kSplitLds = kOffPlan + 64;                             // 162944
static_assert(kSplitLds <= 160 * 1024, "split kernel LDS budget");
// A slot copy issued in phase X of iteration v lands before the barrier that
// ends phase X of iteration v+1; gathers read it kGatherAhead tiles ahead of
// their tile.
static_assert(kSlotAhead - 2 >= kGatherAhead, "slot copy distance");
static_assert(kSlotRing > kSlotAhead && kGatherAhead == kRingS, "ring sizes");
// Epilogue staging: one 32-row block of a wave's 64 dims in fp16, rows padded
// to 144 bytes (a multiple of 16, for the 16-byte read-back), per wave, inside
// the tile ring.
constexpr int kStageRow = kWaveDvBlocks * 32 * 2 + 16;
constexpr int kStageBytes = 32 * kStageRow;
static_assert(kSplitWaves * kStageBytes <= kOffXchg, "epilogue staging fits in the tile ring");

// The refill of a tile slot (gather of tile u + 3 in phase X of iteration u)
// must not overwrite a region that a wave still reads. The last reads of tile
// u are the value reads: wave w reads line value_line(w) of every key group,
// before the barrier that opens phase X (both halves; see the schedule in the
// split kernel) unless values_read_in_phase_x(w) says otherwise; both halves
// read tile u's score operands (lines 0..8) one iteration earlier. Gather wave
// j (wave 4 + j) issues its loads after its own value reads are complete, so
// each region it writes must be one that no other wave reads after the
// barrier; and the four gather waves together must write every region
// exactly once. Both are checked here over the same tables the gather and the
// value reads use. (Letting the odd waves read their values in phase X, with
// each gather wave writing all nine lines of its key group, fails the check:
// a refill would overwrite value lines that other odd waves still read.)
__host__ __device__ constexpr bool values_read_in_phase_x(int wave) { return wave < 0; }
__host__ __device__ constexpr bool read_after_phase_barrier(int wave, int line) {
  return values_read_in_phase_x(wave) && value_line(wave) == line;
}
__host__ __device__ constexpr bool gather_ownership_ok() {
  int cover[kKeyGroups][kGatherLoads] = {};
  for (int j = 0; j < kGatherWaves; ++j)
    for (int k = 0; k < kGatherLoads; ++k) {
      const int kg = gather_kg(j, k), L = gather_line(j, k);
      if (kg < 0 || kg >= kKeyGroups || L < 0 || L >= kGatherLoads) return false;
      ++cover[kg][L];
      for (int w = 0; w < kSplitWaves; ++w)
        if (w != kSplitWaves / 2 + j && read_after_phase_barrier(w, L)) return false;
    }
  for (int kg = 0; kg < kKeyGroups; ++kg)
    for (int L = 0; L < kGatherLoads; ++L)
      if (cover[kg][L] != 1) return false;
  // every value chunk a wave reads lies in its value line
  for (int w = 0; w < kSplitWaves; ++w)
    for (int d = 0; d < kWaveDvBlocks; ++d)
      for (int g = 0; g < 4; ++g)
        for (int s = 0; s < 16; ++s)
          if (value_chunk(w, d, g, s) / 8 != value_line(w)) return false;
  return true;
}
static_assert(gather_ownership_ok(), "a tile refill may overwrite a region another wave still reads");

template <int V>
struct IntC {
  static constexpr int value = V;
};

__global__ void __launch_bounds__(kSplitThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
split_kernel(SplitArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kSplitLds];
  LDS_AS char* lds = lds_cast(smem);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Lane-derived values are re-derived from fresh_lane() for each piece (the
  // loop over pieces below), so that nothing computed from them is hoisted out
  // of that loop and kept live through all of it.
  int lane = tid & 63;
  int n = lane & 31;   // row of this lane within a 32-row block
  int h = lane >> 5;   // k-half of the MFMA operands
  int swap_addr = (lane ^ 32) << 2;   // LDS permute address of the lane in the other half
  const int pair = wave & 3;
  const int p = wave >> 2;   // 0: even half (softmax owner), 1: odd half

  // Workgroup -> (column, row tile). Consecutive ids go round-robin to the 8
  // XCDs, so all row tiles of one column share an XCD and its L2.
  const int wg = blockIdx.x;
  const int xcd = wg & 7;
  const int y = wg >> 3;
  const int rt = y % a.row_tiles;
  const int g = (y / a.row_tiles) * 8 + xcd;
  // (P region of LDS as scratch: first written by the softmax of tile 0,
  // after several barriers.)
  const bool columns = a.target > a.B && a.B <= kPlanThreads;   // uniform across the launch
  const ChunkPlan cp = columns ? column_plan(a, g, wg == 0, lds + kOffP) : chunk_plan(a, g, wg == 0, lds + kOffP);
  if (cp.nseg == 0) return;   // uniform across the workgroup
  // The first piece's description stays in LDS for the later pieces (read
  // there, after the barriers of the first piece), so that it does not occupy
  // registers through the loop over pieces.
  LDS_AS int64_t* plan_st = reinterpret_cast<LDS_AS int64_t*>(lds + kOffPlan);
  if (tid == 0) {
    plan_st[0] = cp.b;
    plan_st[1] = cp.c;
    plan_st[2] = cp.sbase;
    plan_st[3] = cp.ubase;
    plan_st[4] = cp.uend;
    plan_st[5] = cp.nseg;
  }
  // The current piece (see ChunkPlan); set for each piece below.
  int b = __builtin_amdgcn_readfirstlane(cp.b);
  int c = __builtin_amdgcn_readfirstlane(cp.c);
  int64_t P = uniform64(cp.P);
  int64_t sbase = uniform64(cp.sbase);
  int64_t kstart = uniform64(cp.kstart);
  int64_t kend = uniform64(cp.kend);
  int nunits = 0;

  // Score rows of this lane (pair block) and its query's tail-visibility bits.
  auto row_of_lane = [&]() { return rt * kRowsPerWG + pair * 32 + n; };
  bool row_ok = row_of_lane() < a.R;
  int rr = row_ok ? row_of_lane() : 0;
  // Tail-visibility bits of the lane's query (even half; all ones elsewhere).
  // The first 16 positions are 16 unconditional byte loads (indices clamped
  // into the row), so they cost one memory round trip, not one each. Only a
  // piece that reaches the tail (kend > P) consults them, and only such a
  // piece loads them: at the start of a launch the byte loads add about two
  // microseconds to every workgroup that issues them.
  uint64_t tbits = ~0ull;
  auto load_mask = [&]() {
    // (the divisor goes through an opaque move, so that the division's setup
    // is not hoisted out of the loop over pieces and kept live through it)
    int heads;
    asm volatile("s_mov_b32 %0, %1" : "=s"(heads) : "s"(a.H));
    const uint8_t* mrow = a.tree_mask + ((int64_t)b * a.Q + rr / heads) * a.Q;
    uint64_t bits = 0;
    for (int t0 = 0; t0 < a.Q; t0 += 16) {
      uint32_t mb[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) mb[j] = mrow[t0 + j < a.Q ? t0 + j : a.Q - 1];
#pragma unroll
      for (int j = 0; j < 16; ++j) bits |= (uint64_t)((t0 + j < a.Q) & (mb[j] != 0)) << (t0 + j);
    }
    tbits = row_ok ? bits : ~0ull;
  };

  // Resident queries: for k-step ks of this wave's dim half, lane (n + 32h)
  // holds dims 288p + 16ks + 8h .. +7 of row n (zeros for padding rows). The
  // last kLdsKSteps k-steps are parked in LDS to stay within 256 VGPRs.
  // Loading and placing are separate steps, so that a wave can have other
  // loads in flight with the queries.
  bf16x8 qf[kRegKSteps];
  LDS_AS char* my_q;
  auto load_q = [&](u32x4 (&qv)[kHalfKSteps]) {
    const u32x4* qrow = reinterpret_cast<const u32x4*>(a.q + ((int64_t)b * a.R + rr) * kLatent) +
                        p * (kHalfKSteps * 2) + h;
#pragma unroll
    for (int ks = 0; ks < kHalfKSteps; ++ks) qv[ks] = qrow[2 * ks];
  };
  auto place_q = [&](const u32x4 (&qv)[kHalfKSteps]) {
#pragma unroll
    for (int ks = 0; ks < kHalfKSteps; ++ks) {
      const u32x4 vz = row_ok ? qv[ks] : u32x4{0, 0, 0, 0};
      if (ks < kRegKSteps) qf[ks] = __builtin_bit_cast(bf16x8, vz);
      else *reinterpret_cast<LDS_AS u32x4*>(my_q + (ks - kRegKSteps) * 1024) = vz;
    }
  };

  // Lane-constant LDS offsets, recomputed where they are used (from
  // fresh_lane(), so they do not occupy registers across the loop).
  // Score A operand: A-row n holds key swap_bits23(n), so that the score
  // accumulator element i of lane (n + 32h) is key 16*(i/8) + 8h + (i%8).
  // Its k-step ks of this wave reads chunk 2(18p + ks) + h; a_off[j] is the
  // address for ks = j, and ks = j + 4q adds q KiB.
  // Only the offset of k-step 0 is computed; the others follow by score_koff
  // (lane_offsets_ok).
  auto score_offsets = [&](LDS_AS const char* tile, unsigned (&a_addr)[4]) {
    const int fl = fresh_lane();
    const int a0 = tile_offset(2 * kHalfKSteps * p + (fl >> 5), arow_key(fl & 31));
#pragma unroll
    for (int j = 0; j < 4; ++j) a_addr[j] = (unsigned)(uintptr_t)tile + (unsigned)score_koff(a0, j, p);
  };
  // Value transpose reads: group g = lane/16, s = lane%16 supplies the address
  // of V[key 16t + 8h + 4hf + s/4][dv 32db + 16(g%2) + 4(s%4) .. +3] for this
  // wave's blocks db = 2w + d; key 16t adds 18 KiB (t is an immediate). Only
  // the offset for (hf, d) = (0, 0) is computed; the others follow by
  // value_off (lane_offsets_ok).
  auto value_offsets = [&](LDS_AS const char* tile, unsigned (&tr_addr)[2][2]) {
    const int fl = fresh_lane();
    const int g = fl >> 4, s = fl & 15, hh = fl >> 5;
    const int t00 = tile_offset(value_chunk(wave, 0, g, s), 8 * hh + (s >> 2)) + (s & 1) * 8;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int d = 0; d < 2; ++d) tr_addr[hf][d] = (unsigned)(uintptr_t)tile + (unsigned)value_off(t00, hf, d);
  };
  LDS_AS char* xchg;   // lds + kOffXchg + pair * kXchgBytes + lane * 16, + k * 1024
  LDS_AS char* pbuf;   // lds + kOffP + lane * 16, + rb * kPBytes + t * 1024
  LDS_AS char* abuf = lds + kOffAlpha;
  LDS_AS char* fbuf = lds + kOffFlag;

  // Gather bookkeeping (see gather_lane): the odd half (waves 4-7) issues all
  // direct-to-LDS loads, nine per wave and tile; lane l always fetches the
  // same key of a tile. The even half issues none inside the loop, so its
  // LDS reads never wait on them.
  // (The per-lane gather fields are re-derived from fresh_lane() at each use,
  // so they do not occupy registers across the loop.)
  auto glane = [&]() { return gather_lane(wave - kSplitWaves / 2, fresh_lane()); };
  // Slot indices travel through LDS like the latent rows: wave 4 copies the
  // 32 kv_indices entries of tile v into ring entry v % 8 with one
  // direct-to-LDS dword load (lanes 32-63 duplicate lanes 0-31), kSlotAhead
  // tiles ahead, so that the vmcnt waits that cover the gathers cover them
  // too. (A register load would make the compiler wait for it with a vmcnt
  // that also drains the gathers issued after it.)
  LDS_AS char* slot_ring = lds + kOffSlots;
  auto tile_key_ok = [&](int v, int gkey) -> bool { return kstart + (int64_t)v * kUnit + gkey < kend; };
  auto load_slots_to_lds = [&](int v) {
    if (wave == 4) {
      int64_t gpos = sbase + kstart + (int64_t)v * kUnit + (fresh_lane() & 31);
      gpos = gpos < a.total_kv ? gpos : a.total_kv - 1;
      gpos = gpos < 0 ? 0 : gpos;
      lds_dma4(a.kv_indices + gpos, slot_ring + (v % kSlotRing) * 256);
    }
  };
  auto read_slot = [&](int v) -> int32_t {
    const int gkey = glane().key;
    const int32_t sl = *reinterpret_cast<LDS_AS const int32_t*>(slot_ring + (v % kSlotRing) * 256 + gkey * 4);
    return tile_key_ok(v, gkey) ? sl : -1;
  };
  auto load_slot = [&](int v) -> int32_t {
    const int64_t pos = kstart + (int64_t)v * kUnit + glane().key;
    int64_t gpos = sbase + pos;   // inside [0, total_kv) for pos < kend; clamped all the same
    gpos = gpos < 0 ? 0 : (gpos >= a.total_kv ? a.total_kv - 1 : gpos);
    return pos < kend ? a.kv_indices[gpos] : -1;
  };
  auto issue = [&](int32_t slot, LDS_AS char* tile) { issue_tile_gather(a.kv_pool, a.num_slots, slot, tile, glane()); };

  // Online-softmax state of the pair's rows (log2 domain; kept by the even
  // half) and this wave's output accumulators O^T: [row block][value block].
  float m_ref = -INFINITY;
  float l_sum = 0.f;  // partial: this lane's half of the keys
  f32x16 o[kRowBlocks][kWaveDvBlocks];
#pragma unroll
  for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
    for (int db = 0; db < kWaveDvBlocks; ++db) o[rb][db] = f32x16{};

  // P, rescale factors and rescale flags are double-buffered by tile parity:
  // the odd half applies tile u-1 while the even half publishes tile u.
  auto pbuf_of = [&](int v) { return pbuf + (v & 1) * (kPairs * kPBytes); };
  auto abuf_of = [&](int v) { return abuf + (v & 1) * (kRowsPerWG * 4); };
  auto fbuf_of = [&](int v) { return fbuf + (v & 1) * 16; };
  // O^T *= alpha(v) when some row's running max grew in tile v (rare); rows
  // whose max did not grow carry alpha = 1.
  auto rescale = [&](int v) {
    const uint32_t flags = *reinterpret_cast<LDS_AS const uint32_t*>(fbuf_of(v));   // one byte per pair
    if (flags) {
#pragma unroll
      for (int rb = 0; rb < kRowBlocks; ++rb) {
        const float al = *reinterpret_cast<LDS_AS const float*>(abuf_of(v) + (rb * 32 + n) * 4);
#pragma unroll
        for (int db = 0; db < kWaveDvBlocks; ++db) o[rb][db] *= al;
      }
    }
  };
  // O^T += V(v)^T P(v)^T for this wave's 64 dims and all 128 rows.
  auto apply_values = [&](int v, const f16x8 (&va)[kWaveDvBlocks][2]) {
    // MFMA pair i (of 8) takes P(row block i % 4, key step i / 4). The P
    // operands stream through a ring of three reads: the read for pair i+3 is
    // issued right after pair i, two pairs of MFMAs ahead of its use.
    // Consecutive MFMAs write different accumulators.
    constexpr int kPRing = 3;
    auto pread = [&](int i) {
      return *reinterpret_cast<LDS_AS const f16x8*>(pbuf_of(v) + (i % kRowBlocks) * kPBytes + (i / kRowBlocks) * 1024);
    };
    f16x8 pq[kPRing];
    pq[0] = pread(0);
    pq[1] = pread(1);
    // O^T *= alpha(v) first; the flag read queues behind the first P reads,
    // so they arrive in one LDS round trip.
    rescale(v);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 2; i < kPRing; ++i) pq[i] = pread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * kRowBlocks; ++i) {
      const int rb = i % kRowBlocks, t = i / kRowBlocks;
#pragma unroll
      for (int db = 0; db < kWaveDvBlocks; ++db)
        o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[db][t], pq[i % kPRing], o[rb][db], 0, 0, 0);
      if (i + kPRing < 2 * kRowBlocks) pq[i % kPRing] = pread(i + kPRing);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- partial scores S^T of one tile over this wave's 288 dims. The K
  // operands (and parked queries) are read kDepth k-steps ahead of their MFMA;
  // the scheduling barriers keep the compiler from sinking each read next to
  // its use, which would expose one LDS round trip per MFMA.
  auto scores = [&](LDS_AS const char* tile) -> f32x16 {
    f32x16 acc = f32x16{};
    unsigned a_addr[4];
    score_offsets(tile, a_addr);
    constexpr int kDepth = 4;    // K reads in flight
    constexpr int kQDepth = 2;   // parked-query reads in flight
    auto kload = [&](int ks) {
      return *reinterpret_cast<LDS_AS const bf16x8*>((uintptr_t)(a_addr[ks & 3] + (ks >> 2) * 1024));
    };
    auto qpark = [&](int ks) {
      return *reinterpret_cast<LDS_AS const bf16x8*>(my_q + (ks - kRegKSteps) * 1024);
    };
    bf16x8 kb[kDepth], qb[kQDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) kb[i] = kload(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kHalfKSteps; ++ks) {
      const bf16x8 kc = kb[ks % kDepth];
      const bf16x8 qc = ks < kRegKSteps ? qf[ks < kRegKSteps ? ks : 0] : qb[ks % kQDepth];
      if (ks + kDepth < kHalfKSteps) kb[ks % kDepth] = kload(ks + kDepth);
      if (ks + kQDepth >= kRegKSteps && ks + kQDepth < kHalfKSteps) qb[ks % kQDepth] = qpark(ks + kQDepth);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc, qc, acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
  };
  // The odd half hands its partial block to the even half of its pair.
  auto write_xchg = [&](const f32x16& sa) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<LDS_AS f32x4*>(xchg + k * 1024) = f32x4{sa[4 * k], sa[4 * k + 1], sa[4 * k + 2], sa[4 * k + 3]};
  };
  // ---- even half: full scores of tile u, mask, running max, lazy rescale,
  // probabilities; publishes P(u), the rescale factors and the rescale flag.
  auto softmax = [&](int u, const f32x16& sa) {
    float x[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 d = *reinterpret_cast<LDS_AS const f32x4*>(xchg + k * 1024);
      x[4 * k] = (sa[4 * k] + d[0]) * a.c_log2;
      x[4 * k + 1] = (sa[4 * k + 1] + d[1]) * a.c_log2;
      x[4 * k + 2] = (sa[4 * k + 2] + d[2]) * a.c_log2;
      x[4 * k + 3] = (sa[4 * k + 3] + d[3]) * a.c_log2;
    }
    const int64_t ustart = kstart + (int64_t)u * kUnit;
    if (ustart + kUnit > P || ustart + kUnit > kend) {
      // Positions relative to the tile start fit in 32 bits (a chunk is at
      // most 2^31 keys). Branch-free selects: a short-circuit form of this
      // test was compiled into control flow that dropped the -inf store for
      // hidden tail keys.
      const int rel0 = (int)(ustart - P);
      const int end0 = (int)(kend - ustart);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 16 * (i >> 3) + 8 * h + (i & 7);
        const int rel = rel0 + kk;
        const unsigned tail_bit = (unsigned)(tbits >> (unsigned)(rel & 63)) & 1u;
        const unsigned vis = (unsigned)(kk < end0) & ((unsigned)(rel < 0) | tail_bit);
        x[i] = vis ? x[i] : -INFINITY;
      }
    }
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, x[i]);
    mx = fmaxf(mx, swap_halves(mx, swap_addr));
    const bool grow = mx > m_ref + kLazyRescale;  // false while the row has seen nothing
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - mx) : 1.f;  // exp2(-inf) = 0
    if (grow) m_ref = mx;
    l_sum *= alpha;
    const float mref_safe = m_ref == -INFINITY ? 0.f : m_ref;
    f16x8 p0, p1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float e0 = __builtin_amdgcn_exp2f(x[j] - mref_safe);
      const float e1 = __builtin_amdgcn_exp2f(x[8 + j] - mref_safe);
      l_sum += e0 + e1;
      p0[j] = (_Float16)e0;
      p1[j] = (_Float16)e1;
    }
    *reinterpret_cast<LDS_AS f16x8*>(pbuf_of(u) + pair * kPBytes) = p0;
    *reinterpret_cast<LDS_AS f16x8*>(pbuf_of(u) + pair * kPBytes + 1024) = p1;
    const int any_grow = __ballot(grow) != 0;  // wave-wide: taken before any lane is masked off
    if (h == 0) *reinterpret_cast<LDS_AS float*>(abuf_of(u) + (pair * 32 + n) * 4) = alpha;
    if (fresh_lane() == 0) *reinterpret_cast<LDS_AS uint8_t*>(fbuf_of(u) + pair) = (uint8_t)any_grow;
  };
  // ---- this wave's value operands of one tile: V^T for its two 32-dim
  // blocks and both 16-key steps, transposed and converted to fp16.
  // The transpose reads are compiler builtins, so their waits are counted
  // like any other LDS read (the direct-to-LDS loads, being asm, do not make
  // the compiler fence them).
  auto read_values = [&](LDS_AS const char* tile, f16x8 (&va)[kWaveDvBlocks][2]) {
    u32x2 v[kWaveDvBlocks][2][2];   // [d][t][hf]
    unsigned tr_addr[2][2];
    value_offsets(tile, tr_addr);
    const unsigned a00 = tr_addr[0][0];
    const unsigned a10 = tr_addr[1][0];
    const unsigned a01 = tr_addr[0][1];
    const unsigned a11 = tr_addr[1][1];
    auto tr = [&](unsigned addr) {
      const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(uintptr_t)addr);
      return __builtin_bit_cast(u32x2, r);
    };
    v[0][0][0] = tr(a00);
    v[0][0][1] = tr(a10);
    v[0][1][0] = tr(a00 + 18432);
    v[0][1][1] = tr(a10 + 18432);
    v[1][0][0] = tr(a01);
    v[1][0][1] = tr(a11);
    v[1][1][0] = tr(a01 + 18432);
    v[1][1][1] = tr(a11 + 18432);
#pragma unroll
    for (int db = 0; db < kWaveDvBlocks; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x4_to_f16(v[db][t][0], va[db][t], 0);
        bf16x4_to_f16(v[db][t][1], va[db][t], 4);
      }
  };

  // One half's pipeline (PP = p). Each iteration u has two phases, each
  // closed by a barrier, and the two waves of a SIMD take turns on its matrix
  // core:
  //   phase Y: the even wave runs the softmax of tile u (vector ALU) while the
  //            odd wave applies tile u-1 to its values and computes its
  //            partial scores of tile u+1 (34 MFMAs); both then read their
  //            value operands of tile u, the last reads of tile u;
  //   phase X: the even wave applies tile u and computes its partial scores
  //            of tile u+1 (34 MFMAs) while the odd wave hands over its
  //            partial scores, issues the gather of tile u+3 into tile u's
  //            slot (nobody reads it after the barrier that opens phase X),
  //            and waits for tile u+2.
  // (With the odd wave's value reads in phase X, where it has slack, the
  // split kernel ran 2% faster, but its gather then overwrote value lines that
  // other odd waves could still be reading; see gather_ownership_ok.)
  // P, the rescale factors and flags are double-buffered by tile parity, as
  // the odd half reads those of tile u-1 while the even half writes tile u's.
  auto run = [&](auto pc) {
    constexpr int PP = decltype(pc)::value;
    if (nunits == 0) return;   // uniform across the workgroup

    // Prologue. Odd half: pool rows of tiles 0-2 and the queries, loaded
    // together (one memory round trip); then the gathers of tiles 0-2 and
    // slot copies of tiles 3..kSlotAhead-1, in the order that gives the loop
    // its vmcnt counts; then wait for everything but tile 2. (The queries are
    // placed before the gathers go out: the compiler orders any use of a
    // register load after every direct-to-LDS load issued behind it.) Even
    // half: queries and mask row.
    u32x4 qv[kHalfKSteps];
    if constexpr (PP == 1) {
      const int32_t s0 = load_slot(0);
      const int32_t s1 = load_slot(1);
      const int32_t s2 = load_slot(2);
      load_q(qv);
      place_q(qv);
      issue(s0, lds);
      issue(s1, lds + kTileBytes);
      for (int v = kGatherAhead; v < kSlotAhead; ++v) load_slots_to_lds(v);
      issue(s2, lds + 2 * kTileBytes);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kGatherLoads) : "memory");
    } else {
      load_q(qv);
      if (kend > P) load_mask();   // uniform across the workgroup
      place_q(qv);
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    f32x16 sa = scores(lds);   // tile 0, both halves
    if constexpr (PP == 1) write_xchg(sa);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    f16x8 vheld[kWaveDvBlocks][2];   // odd half: values of the previous tile
#pragma unroll
    for (int db = 0; db < kWaveDvBlocks; ++db) vheld[db][0] = vheld[db][1] = f16x8{};

    for (int u = 0; u < nunits; ++u) {
      LDS_AS char* tile = lds + (u % kRingS) * kTileBytes;
      LDS_AS char* next = lds + ((u + 1) % kRingS) * kTileBytes;
      const bool more = u + 1 < nunits;

      // ---- phase Y
      if constexpr (PP == 0) {
        softmax(u, sa);
      } else {
        // The wave feeding the matrix core raises its issue priority for
        // its MFMA stretch, so that the other wave of its SIMD yields to
        // its operand reads.
        __builtin_amdgcn_s_setprio(1);
        if (u > 0) apply_values(u - 1, vheld);
        // (the else branch keeps the old block from living on through the MFMAs)
        if (more) sa = scores(next);
        else sa = f32x16{};
        __builtin_amdgcn_s_setprio(0);
      }
      constexpr bool kValuesInX = values_read_in_phase_x(PP * kSplitWaves / 2);
      static_assert(!values_read_in_phase_x(0), "the even half applies tile u in phase X");
      f16x8 va[kWaveDvBlocks][2];
      if constexpr (!kValuesInX) read_values(tile, va);
      if constexpr (PP == 0) {
        // The even wave converts its values before the barrier: its phase Y
        // has slack, its phase X does not. (The odd wave's conversion is left
        // to the compiler, which sinks it into phase X, where the odd wave
        // has slack.)
#pragma unroll
        for (int db = 0; db < kWaveDvBlocks; ++db) asm volatile("" ::"v"(va[db][0]), "v"(va[db][1]));
      }
      // P/alpha/flag stores of the even half are complete before the barrier
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

      // ---- phase X
      if constexpr (PP == 0) {
        __builtin_amdgcn_s_setprio(1);   // as in the odd half's phase Y
        apply_values(u, va);
        // Unconditional (after the last tile this reads a landed tile of zero
        // rows and the result is dropped): a conditional update keeps the old
        // block live through the MFMAs, and the registers do not allow it.
        sa = scores(next);
        __builtin_amdgcn_s_setprio(0);
        asm volatile("s_barrier" ::: "memory");
      } else {
        if constexpr (kValuesInX) {
          read_values(tile, vheld);
        } else {
#pragma unroll
          for (int db = 0; db < kWaveDvBlocks; ++db) {
            vheld[db][0] = va[db][0];
            vheld[db][1] = va[db][1];
          }
        }
        if (more) write_xchg(sa);
        load_slots_to_lds(u + kSlotAhead);
        const int32_t slot = read_slot(u + kGatherAhead);
        // The refill of tile u's slot with tile u + 3 may overwrite only what
        // nobody reads any more (gather_ownership_ok): after the barrier that
        // opened this phase, at most this wave's own value reads.
        if constexpr (kValuesInX) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue(slot, tile);
        // Tile u+2 has landed once no more than the loads issued after it are
        // outstanding: this phase's slot copy (wave 4) and its nine gather
        // loads. (The compiler does not track direct-to-LDS loads, so the wait
        // is explicit; the barrier is issued by hand so that it does not drain
        // tile u+3.)
        if (wave == 4) asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(kGatherLoads + 1) : "memory");
        else asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(kGatherLoads) : "memory");
      }
    }
    // the odd half's value update of the last tile
    if constexpr (PP == 1) {
      apply_values(nunits - 1, vheld);
    }
  };
  for (int piece = 0;;) {
    if (piece > 0) {
      // Piece `piece` of the column (column plan): sequence b0 + piece from
      // its first key; its tiles start past those of the pieces before it.
      const int b0 = __builtin_amdgcn_readfirstlane((int)plan_st[0]);
      int64_t sb = uniform64(plan_st[2]);
      int64_t ub = uniform64(plan_st[3]);
      for (int j = 0; j < piece; ++j) {
        int64_t pl = a.prefix_lens[b0 + j];
        pl = pl < 0 ? 0 : (pl > a.total_kv ? a.total_kv : pl);
        sb += pl + a.Q;
        ub += (pl + a.Q + kUnit - 1) / kUnit + kSeqUnits;
      }
      b = b0 + piece;
      c = __builtin_amdgcn_readfirstlane((int)plan_st[1]) + piece;
      sbase = sb;
      int64_t pl = a.prefix_lens[b];
      pl = pl < 0 ? 0 : (pl > a.total_kv ? a.total_kv : pl);
      P = uniform64(pl);
      kstart = 0;
      kend = uniform64((uniform64(plan_st[4]) - ub) * kUnit);
    }
    lane = fresh_lane();
    n = lane & 31;
    h = lane >> 5;
    swap_addr = (lane ^ 32) << 2;
    row_ok = row_of_lane() < a.R;
    rr = row_ok ? row_of_lane() : 0;
    my_q = lds + kOffQPark + wave * kQParkBytes + lane * 16;
    xchg = lds + kOffXchg + pair * kXchgBytes + lane * 16;
    pbuf = lds + kOffP + lane * 16;
    if (kend > P + a.Q) kend = P + a.Q;
    if (kend > a.total_kv - sbase) kend = a.total_kv - sbase;  // positions past the array are absent
    nunits = kend > kstart ? (int)((kend - kstart + kUnit - 1) / kUnit) : 0;
    tbits = ~0ull;
    m_ref = -INFINITY;
    l_sum = 0.f;
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb)
#pragma unroll
      for (int db = 0; db < kWaveDvBlocks; ++db) o[rb][db] = f32x16{};

  if (p == 0) run(IntC<0>{});
  else run(IntC<1>{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the trailing gathers and slot copies

  // ---- epilogue: the even halves publish 1/l per row (reusing the alpha
  // slots) and write lse; every wave normalises and writes its 64 dims.
  {
    // (lane values re-derived, as elsewhere in the loop over pieces)
    const int efl = fresh_lane();
    const int en = efl & 31, eh = efl >> 5;
    const float l_tot = l_sum + swap_halves(l_sum, (efl ^ 32) << 2);
    const bool live = l_tot > 0.f;
    asm volatile("s_barrier" ::: "memory");  // all waves are past their last alpha read
    if (p == 0) {
      if (eh == 0) *reinterpret_cast<LDS_AS float*>(abuf + (pair * 32 + en) * 4) = live ? 1.f / l_tot : 0.f;
      const float lse_v = live ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
      // the row index is re-derived here rather than kept live through the loop
      const int r2 = rt * kRowsPerWG + pair * 32 + en;
      if (r2 < a.R && eh == 0) a.part_lse[(int64_t)c * a.R + r2] = lse_v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // The normalised block is rounded to fp16 (|O / l| is at most the largest
    // |value| in the chunk, which the fp16 value operands already bound) and
    // goes out through a wave-private LDS staging area (the tile ring is free
    // now): written in the accumulator layout, read back row-major, so that
    // every store instruction writes eight rows of 128 contiguous bytes
    // (whole lines) instead of 8-byte pieces of 32 rows.
    LDS_AS char* stg = lds + wave * kStageBytes;
#pragma unroll
    for (int rb = 0; rb < kRowBlocks; ++rb) {
      const float inv = *reinterpret_cast<LDS_AS const float*>(abuf + (rb * 32 + en) * 4);
#pragma unroll
      for (int db = 0; db < kWaveDvBlocks; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          f16x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = (_Float16)(o[rb][db][4 * qd + e] * inv);
          *reinterpret_cast<LDS_AS f16x4*>(stg + en * kStageRow + (db * 32 + 8 * qd + 4 * eh) * 2) = hv;
        }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int fl = fresh_lane();
        const int row = 8 * k + (fl >> 3);
        const int ch = fl & 7;
        const u32x4 v = *reinterpret_cast<LDS_AS const u32x4*>(stg + row * kStageRow + ch * 16);
        const int rw = rt * kRowsPerWG + rb * 32 + row;
        if (rw < a.R)
          *reinterpret_cast<u32x4*>(a.part_o + ((int64_t)c * a.R + rw) * kValue + wave * kWaveDvBlocks * 32 + ch * 8) = v;
      }
    }
  }

    if (++piece >= __builtin_amdgcn_readfirstlane((int)plan_st[5])) break;
    // Every wave is done with the epilogue's LDS (staging in the tile ring, the
    // 1/l slots) before the next prologue refills the ring.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// Chunk range [c0, c1) of sequence b for the merges, clamped to the partial
// buffers' capacity. The split kernel writes offsets inside it; the clamp keeps
// every partial read in bounds whatever the offsets hold.
__device__ __forceinline__ int2 chunk_range(const int32_t* __restrict__ chunk_off, int b, int max_chunks) {
  int c0 = chunk_off[b], c1 = chunk_off[b + 1];
  c0 = c0 < 0 ? 0 : (c0 > max_chunks ? max_chunks : c0);
  c1 = c1 < c0 ? c0 : (c1 > max_chunks ? max_chunks : c1);
  return int2{c0, c1};
}

// ---------------------------------------------------------------------------
// Merge: lse = ln sum_s exp(lse_s); out = sum_s exp(lse_s - lse) O_s.
// One 256-thread workgroup per (row, quarter of the 512 value dims): thread
// t handles 4 dims (t % 32) of the quarter for chunks c0 + (t / 32) + 8k, so
// each wave reads two whole 256-byte fp16 row segments per step and the chunks
// of a row are spread over 8 lanes. Each lane folds its chunks in one pass
// with a running maximum (the log2 domain; earlier terms are rescaled when it
// grows), loading the next four chunks while it folds the current four; an
// LDS step then combines the 8 lanes.
// ---------------------------------------------------------------------------
constexpr int kMergeLanes = 8;   // chunk lanes per workgroup
constexpr int kMergeBatch = 4;   // chunks per lane and load batch

__global__ void __launch_bounds__(256) merge_kernel(const _Float16* __restrict__ part_o,
                                                    const float* __restrict__ part_lse,
                                                    const int32_t* __restrict__ chunk_off,
                                                    float* __restrict__ out, float* __restrict__ lse,
                                                    int B, int R, int max_chunks) {
  __shared__ f32x4 s_acc[kMergeLanes][32];
  __shared__ float s_m[kMergeLanes];
  __shared__ float s_w[kMergeLanes];
  const int64_t grow = (int64_t)(blockIdx.x >> 2);
  const int qd = blockIdx.x & 3;
  if (grow >= (int64_t)B * R) return;
  const int b = (int)(grow / R);
  const int r = (int)(grow - (int64_t)b * R);
  const int t = threadIdx.x;
  const int dl = t & 31, cl = t >> 5;
  const int2 cr = chunk_range(chunk_off, b, max_chunks);
  const int c0 = cr.x, c1 = cr.y;
  float* orow = out + grow * kValue + qd * 128 + 4 * dl;
  if (c1 <= c0) {   // no chunk (only when the partial buffers ran out)
    if (cl == 0) *reinterpret_cast<f32x4*>(orow) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t == 0 && qd == 0) lse[grow] = -INFINITY;
    return;
  }

  // Running maximum m (log2 units), weight sum and weighted sum of this
  // lane's chunks. Chunks that are empty for the row (lse_s = -inf) weigh 0.
  float m = -INFINITY, ws = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const _Float16* obase = part_o + (int64_t)r * kValue + qd * 128 + 4 * dl;
  // Batch of chunks cs + 8k; positions past the row's last chunk load that
  // chunk again and count as empty.
  auto load = [&](int cs, float (&l)[kMergeBatch], f32x4 (&v)[kMergeBatch]) {
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int ck = cs + k * kMergeLanes;
      const int64_t cc = ck < c1 ? ck : c1 - 1;
      l[k] = part_lse[cc * R + r];
      const f16x4 hv = *reinterpret_cast<const f16x4*>(obase + cc * R * kValue);
      v[k] = f32x4{(float)hv[0], (float)hv[1], (float)hv[2], (float)hv[3]};
      if (ck >= c1) l[k] = -INFINITY;
    }
  };
  auto fold = [&](const float (&l)[kMergeBatch], const f32x4 (&v)[kMergeBatch]) {
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float lt = l[k] * kLog2e;
      const float mn = fmaxf(m, lt);
      if (mn > -INFINITY) {
        const float sc = __builtin_amdgcn_exp2f(m - mn);   // 0 while nothing was folded
        const float w = __builtin_amdgcn_exp2f(lt - mn);   // 0 for an empty chunk
        acc = acc * sc + w * v[k];
        ws = ws * sc + w;
        m = mn;
      }
    }
  };
  float la[kMergeBatch], lb[kMergeBatch];
  f32x4 va[kMergeBatch], vb[kMergeBatch];
  constexpr int kStep = kMergeBatch * kMergeLanes;
  int c = c0 + cl;
  load(c, la, va);
  for (; c < c1; c += 2 * kStep) {
    if (c + kStep < c1) load(c + kStep, lb, vb);
    fold(la, va);
    if (c + kStep >= c1) break;
    if (c + 2 * kStep < c1) load(c + 2 * kStep, la, va);
    fold(lb, vb);
  }

  s_acc[cl][dl] = acc;
  if (dl == 0) {
    s_m[cl] = m;
    s_w[cl] = ws;
  }
  __syncthreads();
  if (cl == 0) {
    float M = s_m[0];
#pragma unroll
    for (int k = 1; k < kMergeLanes; ++k) M = fmaxf(M, s_m[k]);
    if (!(M > -INFINITY)) {   // nothing visible in any chunk
      *reinterpret_cast<f32x4*>(orow) = f32x4{0.f, 0.f, 0.f, 0.f};
      if (dl == 0 && qd == 0) lse[grow] = -INFINITY;
      return;
    }
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float wt = 0.f;
#pragma unroll
    for (int k = 0; k < kMergeLanes; ++k) {
      const float sc = __builtin_amdgcn_exp2f(s_m[k] - M);   // 0 for a lane with no visible chunk
      tot += sc * s_acc[k][dl];
      wt += sc * s_w[k];
    }
    *reinterpret_cast<f32x4*>(orow) = tot * (1.f / wt);
    if (dl == 0 && qd == 0) lse[grow] = (M + __builtin_amdgcn_logf(wt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Merge for sequences with many chunks: one 256-thread workgroup per (row,
// 64-dim slice of the 512 value dims), so that each 128-byte line of a chunk's
// partial row is read by exactly one workgroup and there are eight workgroups
// per row. Thread t takes 8 dims (one 16-byte load per chunk) and chunk lane
// t / 8 of 32: chunks c0 + lane + 32k, loaded eight at a time before any is
// folded, so that every thread keeps several independent loads in flight (the
// merge is bound by memory latency, not by its arithmetic). Each lane folds its
// chunks with a running maximum (log2 domain); an LDS step combines the 32
// lanes.
// ---------------------------------------------------------------------------
constexpr int kSliceLanes = 32;   // chunk lanes per workgroup
constexpr int kSliceBatch = 8;    // chunks per lane and load batch
constexpr int kSlices = kValue / 64;

__global__ void __launch_bounds__(256) merge_slice_kernel(const _Float16* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          const int32_t* __restrict__ chunk_off,
                                                          float* __restrict__ out, float* __restrict__ lse,
                                                          int B, int R, int max_chunks) {
  __shared__ float s_acc[kSliceLanes][64];
  __shared__ float s_m[kSliceLanes];
  __shared__ float s_w[kSliceLanes];
  const int64_t grow = (int64_t)(blockIdx.x / kSlices);
  const int slice = blockIdx.x % kSlices;
  if (grow >= (int64_t)B * R) return;
  const int b = (int)(grow / R);
  const int r = (int)(grow - (int64_t)b * R);
  const int t = threadIdx.x;
  const int dl = t & 7, cl = t >> 3;
  const int2 cr = chunk_range(chunk_off, b, max_chunks);
  const int c0 = cr.x, c1 = cr.y;
  const _Float16* obase = part_o + (int64_t)r * kValue + slice * 64 + dl * 8;
  float m = -INFINITY, ws = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int cs = c0 + cl; cs < c1; cs += kSliceLanes * kSliceBatch) {
    float l[kSliceBatch];
    f16x8 v[kSliceBatch];
#pragma unroll
    for (int k = 0; k < kSliceBatch; ++k) {
      const int ck = cs + k * kSliceLanes;
      l[k] = -INFINITY;   // past the row's last chunk: no load, weight 0
      v[k] = f16x8{};
      if (ck < c1) {
        l[k] = part_lse[(int64_t)ck * R + r] * kLog2e;
        v[k] = *reinterpret_cast<const f16x8*>(obase + (int64_t)ck * R * kValue);
      }
    }
    float mb = m;
#pragma unroll
    for (int k = 0; k < kSliceBatch; ++k) mb = fmaxf(mb, l[k]);
    if (mb > -INFINITY) {
      const float sc = __builtin_amdgcn_exp2f(m - mb);   // 0 while nothing was folded
      ws *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= sc;
#pragma unroll
      for (int k = 0; k < kSliceBatch; ++k) {
        const float w = __builtin_amdgcn_exp2f(l[k] - mb);   // 0 for an empty chunk
        ws += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w * (float)v[k][e];
      }
      m = mb;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_acc[cl][dl * 8 + e] = acc[e];
  if (dl == 0) {
    s_m[cl] = m;
    s_w[cl] = ws;
  }
  __syncthreads();
  if (t < 64) {
    float M = s_m[0];
#pragma unroll
    for (int k = 1; k < kSliceLanes; ++k) M = fmaxf(M, s_m[k]);
    float* orow = out + grow * kValue + slice * 64 + t;
    if (!(M > -INFINITY)) {   // no chunk, or nothing visible in any chunk
      *orow = 0.f;
      if (t == 0 && slice == 0) lse[grow] = -INFINITY;
      return;
    }
    float tot = 0.f, wt = 0.f;
#pragma unroll
    for (int k = 0; k < kSliceLanes; ++k) {
      const float sc = __builtin_amdgcn_exp2f(s_m[k] - M);   // 0 for a lane with no visible chunk
      tot += sc * s_acc[k][t];
      wt += sc * s_w[k];
    }
    *orow = tot * (1.f / wt);
    if (t == 0 && slice == 0) lse[grow] = (M + __builtin_amdgcn_logf(wt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Merge for batches whose sequences have few chunks each: one wave per (row,
// half of the 512 value dims), lane l holding 4 dims, with no cross-lane
// step. The wave loads the partials of up to eight chunks at once and folds
// them with a running maximum (log2 domain), batch after batch, so any number
// of chunks is handled; with few chunks per row this keeps every loaded byte
// useful and the grid small, where the chunk-lane merge above would leave
// most of its lanes idle.
// ---------------------------------------------------------------------------
constexpr int kFewBatch = 8;

__global__ void __launch_bounds__(256) merge_few_kernel(const _Float16* __restrict__ part_o,
                                                        const float* __restrict__ part_lse,
                                                        const int32_t* __restrict__ chunk_off,
                                                        float* __restrict__ out, float* __restrict__ lse,
                                                        int B, int R, int max_chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (row, half)
  if (item >= (int64_t)B * R * 2) return;   // uniform per wave
  const int64_t grow = item >> 1;
  const int half = (int)(item & 1);
  const int b = (int)(grow / R);
  const int r = (int)(grow - (int64_t)b * R);
  const int2 cr = chunk_range(chunk_off, b, max_chunks);
  const int c0 = cr.x, c1 = cr.y;
  float* orow = out + grow * kValue + half * 256 + 4 * lane;
  const _Float16* obase = part_o + (int64_t)r * kValue + half * 256 + 4 * lane;
  float m = -INFINITY, ws = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int cs = c0; cs < c1; cs += kFewBatch) {
    float l[kFewBatch];
    f16x4 v[kFewBatch];
#pragma unroll
    for (int k = 0; k < kFewBatch; ++k) {
      const int ck = cs + k;
      const int64_t cc = ck < c1 ? ck : c1 - 1;   // past the row's last chunk: reload it, weigh 0
      l[k] = ck < c1 ? part_lse[cc * R + r] * kLog2e : -INFINITY;
      v[k] = *reinterpret_cast<const f16x4*>(obase + cc * R * kValue);
    }
    float mb = m;
#pragma unroll
    for (int k = 0; k < kFewBatch; ++k) mb = fmaxf(mb, l[k]);
    if (mb > -INFINITY) {
      const float sc = __builtin_amdgcn_exp2f(m - mb);   // 0 while nothing was folded
      acc *= sc;
      ws *= sc;
#pragma unroll
      for (int k = 0; k < kFewBatch; ++k) {
        const float w = __builtin_amdgcn_exp2f(l[k] - mb);   // 0 for an empty chunk
        acc += w * f32x4{(float)v[k][0], (float)v[k][1], (float)v[k][2], (float)v[k][3]};
        ws += w;
      }
      m = mb;
    }
  }
  if (!(m > -INFINITY)) {   // no chunk, or nothing visible in any chunk
    *reinterpret_cast<f32x4*>(orow) = f32x4{0.f, 0.f, 0.f, 0.f};
    if (lane == 0 && half == 0) lse[grow] = -INFINITY;
    return;
  }
  *reinterpret_cast<f32x4*>(orow) = acc * (1.f / ws);
  if (lane == 0 && half == 0) lse[grow] = (m + __builtin_amdgcn_logf(ws)) * kLn2;
}

// ---------------------------------------------------------------------------
// Debug gather: the split kernel's slot copy and gather routines for one
// tile per workgroup (wave 0 copies the 32 slot indices into LDS, each of the
// four waves reads its lanes' slots back and issues its share of the gather),
// copied back out in position order.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kGatherWaves * 64) debug_gather_kernel(const char* __restrict__ kv_pool,
                                                                         const int32_t* __restrict__ kv_indices,
                                                                         int64_t n, int64_t num_slots,
                                                                         u32x4* __restrict__ rows_out) {
  __shared__ __attribute__((aligned(1024))) char smem[kTileBytes + 256];
  LDS_AS char* lds = lds_cast(smem);
  LDS_AS char* ring = lds + kTileBytes;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ustart = (int64_t)blockIdx.x * kUnit;
  if (wave == 0) {
    int64_t pos = ustart + (lane & 31);
    pos = pos < n ? pos : n - 1;
    lds_dma4(kv_indices + pos, ring);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();
  const GatherLane gl = gather_lane(wave, lane);
  const int32_t sl = *reinterpret_cast<LDS_AS const int32_t*>(ring + gl.key * 4);
  issue_tile_gather(kv_pool, num_slots, ustart + gl.key < n ? sl : -1, lds, gl);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int p = tid; p < kUnit * kChunks; p += kGatherWaves * 64) {
    const int key = p / kChunks, ch = p - key * kChunks;
    if (ustart + key < n)
      rows_out[(ustart + key) * kChunks + ch] =
          *reinterpret_cast<LDS_AS const u32x4*>(lds + tile_offset(ch, key));
  }
}

// ---------------------------------------------------------------------------
// Fixed scratch for the allocation-free entry point: the same workspace
// layout as a caller-owned workspace (chunk offsets, partial lse values,
// fp16 partial outputs), in a device array of fixed size that each device
// holds from the library's load until the process ends. Every call on a
// device shares that device's copy (calls that overlap on one device race);
// nothing in it has to start at zero, since every call writes what it reads.
// In host code `scratch` names a host-side stand-in, never the device array:
// its device address is looked up once per device and used instead.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with device `dev` current
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_split(const SplitArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(split_kernel, dim3(grid), dim3(kSplitThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const _Float16* part_o, const float* part_lse, const int32_t* chunk_off,
                        float* out, float* lse, int B, int R, int max_chunks, hipStream_t stream) {
  const int64_t rows = (int64_t)B * R;
  if (max_chunks <= kMergeFewPerSeq * B) {   // few chunks per sequence on average
    hipLaunchKernelGGL(merge_few_kernel, dim3((unsigned)((rows * 2 + 3) / 4)), dim3(256), 0, stream, part_o,
                       part_lse, chunk_off, out, lse, B, R, max_chunks);
  } else if (max_chunks >= kMergeSlicePerSeq * B) {   // many chunks per sequence
    hipLaunchKernelGGL(merge_slice_kernel, dim3((unsigned)(rows * kSlices)), dim3(256), 0, stream, part_o,
                       part_lse, chunk_off, out, lse, B, R, max_chunks);
  } else {
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)(rows * 4)), dim3(256), 0, stream, part_o,
                       part_lse, chunk_off, out, lse, B, R, max_chunks);
  }
  return hipGetLastError();
}

hipError_t launch_debug_gather(const void* kv_pool, const int32_t* kv_indices, int64_t n,
                               int64_t num_slots, void* rows_out, hipStream_t stream) {
  const int64_t tiles = (n + kUnit - 1) / kUnit;
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(debug_gather_kernel, dim3((unsigned)tiles), dim3(kGatherWaves * 64), 0, stream,
                     static_cast<const char*>(kv_pool), kv_indices, n, num_slots,
                     static_cast<u32x4*>(rows_out));
  return hipGetLastError();
}

}  // namespace va
