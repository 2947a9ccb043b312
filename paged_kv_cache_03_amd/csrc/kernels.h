// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Longest partition a decode workgroup handles, in blocks (512 tokens).
constexpr int kMaxPartitionBlocks = 32;

struct PartArgs {
  const _Float16* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  _Float16* out;
  float* ws_ml;        // [B][H][max_parts][2]: running max (log2 units), running sum
  float* ws_acc;       // [B][H][max_parts][D]: unnormalised weighted sums
  float scale_log2;    // scale * log2(e)
  int B, H;
  int max_blocks;      // table row length
  int ctx_limit;       // contexts are clamped to this (host's max_context_len)
  int num_blocks;
  int part_blocks;     // partition length in blocks
  int max_parts;       // partitions of the longest sequence
  int head_groups;     // H / waves_per_group
  int waves_per_group;
  bool keep_cached;    // normal cache policy for the tiles (blocks shared)
};

struct MergeArgs {
  const float* ws_ml;
  const float* ws_acc;
  const int32_t* context_lens;
  _Float16* out;
  int B, H;
  int ctx_limit;
  int part_blocks;
  int max_parts;
};

// Flat strategy: every workgroup takes one of `nr` equal ranges of the
// lined-up blocks of all sequences (see pa_decode_flat.hip).
#ifndef PKV_FLAT_GRID
#define PKV_FLAT_GRID 512
#endif
#ifndef PKV_FLAT_TILES
#define PKV_FLAT_TILES 3
#endif
#ifndef PKV_FLAT_WAVES
#define PKV_FLAT_WAVES 4
#endif
// Waves (heads) per flat workgroup.
constexpr int kFlatMaxWaves = PKV_FLAT_WAVES;
// Cache-policy bits of the K/V tile loads by default: non-temporal (NT) on
// gfx950, i.e. tiles stream through the caches with low retention (batch 200:
// 347 -> 313 us).  Callers whose tables share blocks ask for the normal
// policy instead, so that shared blocks are found in L2 (shared 1024-token
// prefix: 169 -> 134 us).
constexpr int kStreamPolicy = 2;
constexpr int kCachedPolicy = 0;
// Workgroups of 4 waves resident at once (256 CUs x 2 at the flat kernel's
// register use) and tiles in each wave's load ring.
constexpr int kFlatGridTarget = PKV_FLAT_GRID;
constexpr int kFlatTiles = PKV_FLAT_TILES;
constexpr int kFlatMaxLdsBytes = 32 * 1024;  // per workgroup, so LDS never limits residency

struct FlatArgs {
  const _Float16* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  _Float16* out;
  float* ws_ml;        // [H][nr][2 pieces][2]: running max (log2 units), running sum
  float* ws_acc;       // [H][nr][2 pieces][D]: unnormalised weighted sums
  int* ws_seq;         // [B + 1]: first position of each sequence, then T
  float scale_log2;
  int B, H;
  int max_blocks;
  int ctx_limit;
  int num_blocks;
  int head_groups;
  int waves_per_group;
  int nr;              // ranges (workgroups) per head group
  int max_chunk;       // longest range, in blocks (LDS sizing)
  bool keep_cached;    // normal cache policy for the tiles (blocks shared)
  // Contiguous layout instead of a block pool: sequence b's token t is row
  // b * row_tokens + t of k_pool / v_pool ([rows][H][D]); no block tables.
  bool contig;
  int row_tokens;
  const int32_t* capacity;   // contiguous: tokens each sequence may read (or null)
  // Append fused into the decode (or null): [B][H][D] keys / values of each
  // sequence's new token, written to its last position (context_lens[b] - 1)
  // in the pools before that position is read.
  const _Float16* k_new;
  const _Float16* v_new;
  int heads_per_item;           // heads of one query group per work item (>= 1)
};

// Grouped decode (pa_decode_grouped.hip): groups of up to kGroupMaxMembers
// sequences sharing leading blocks; one MFMA column per member; the groups'
// positions lined up and cut into equal ranges.
constexpr int kGroupMaxMembers = 16;
constexpr int kGroupWaves = 4;             // waves (heads) per workgroup
constexpr int kGroupTiles = 3;             // tiles in each wave's load ring
#ifndef PKV_GROUP_GRID
#define PKV_GROUP_GRID 512
#endif
constexpr int kGroupGridTarget = PKV_GROUP_GRID;   // workgroups (ranges x head groups) at least
constexpr int kGroupMaxLdsBytes = 44 * 1024;       // dynamic LDS: contexts, group offsets, range staging
                                                   // (with the 16 KiB V staging: under 64 KiB)

struct GroupArgs {
  const _Float16* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* group_offsets;  // [G + 1]: group g = sequences [off[g], off[g+1])
  const int32_t* group_shared;   // [G]: leading blocks the members share
  _Float16* out;
  int* ws_map;         // [B]: group * 16 + member of each sequence, -1 if it is in no group
  int* ws_gpos;        // [G + 1]: first position of each group, then the total
  float* ws_ml;        // [H][nr][2 pieces][group_size][2]: running max (log2 units), sum
  float* ws_acc;       // [H][nr][2 pieces][group_size][D]: unnormalised weighted sums
  float scale_log2;
  int B, H, G;
  int max_blocks;
  int ctx_limit;
  int num_blocks;
  int group_size;      // members decoded per group (1..kGroupMaxMembers)
  int head_groups;     // ceil(H / kGroupWaves)
  int nr;              // ranges per head group
  int max_chunk;       // longest range, in positions (LDS sizing)
  int t_cap;           // positions the ranges can hold: nr * max_chunk (at most INT_MAX)
  bool keep_cached;
};

// Prefill (pa_prefill.hip): work items of (128 query rows, a few heads),
// one workgroup at a time.
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 4
#endif
constexpr int kPrefillWaves = PKV_PREFILL_WAVES;   // waves per workgroup, 32 query rows each
constexpr int kPrefillRows = 32 * kPrefillWaves;
constexpr int kPrefillMaxLdsBytes = 32 * 1024;
constexpr int kPrefillSlotsPerCU = 2;      // resident workgroups per CU (two waves per SIMD)
// heads per item: as many as keep about this many items per resident
// workgroup (enough for the dispatch to balance items of unequal length)
constexpr int kPrefillItemsPerSlot = 8;
constexpr int kPrefillMaxHeadsPerItem = 8;

struct PrefillArgs {
  const _Float16* q;            // [num_rows][H][D]
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;   // [B + 1]: sequence b's rows are [qs[b], qs[b+1])
  _Float16* out;                // [num_rows][H][D]
  float scale_log2;
  int B, H;
  int num_rows;
  int max_blocks;
  int ctx_limit;
  int num_blocks;
  // the append fused into the prefill (pkv_pa_prefill_append): the new
  // tokens' keys and values, [num_rows][H][D] like q; null otherwise
  const _Float16* k_new;
  const _Float16* v_new;
  int heads_per_item;           // heads of one query group per work item (>= 1)
};

struct AppendArgs {
  const void* k;
  const void* v;
  const int32_t* slots;
  void* k_pool;
  void* v_pool;
  int T, H, D;
  int num_blocks;
};

constexpr int kMaxCowLayers = 32;  // per launch; more layers take more launches

struct CowArgs {
  void* k[kMaxCowLayers];
  void* v[kMaxCowLayers];
  const int32_t* pairs;
  long long block_bytes;
  int n_pairs;
  int layers;
  int num_blocks;
};

hipError_t launch_pa_decode(const PartArgs& part, int D, int grid_part, int threads,
                            hipStream_t stream);
hipError_t launch_pa_decode_flat(const FlatArgs& a, int D, int threads, hipStream_t stream);
size_t flat_lds_bytes(int B, int max_chunk);
hipError_t launch_hbm_copy_probe(const void* src, void* dst, long long n16, int grid,
                                 hipStream_t stream);
hipError_t launch_hbm_read_probe(const void* buf, long long n16, uint32_t* sink, int grid,
                                 hipStream_t stream);
hipError_t launch_hbm_gather_probe(const void* buf, const int32_t* order, long long n_chunks,
                                   int log_kib, uint32_t* sink, int grid, hipStream_t stream);
hipError_t launch_pa_decode_grouped(const GroupArgs& a, int D, hipStream_t stream);
size_t grouped_lds_bytes(int B, int G, int max_chunk);
hipError_t launch_pa_prefill(const PrefillArgs& a, int D, int grid, int max_blocks_used,
                             hipStream_t stream);
hipError_t launch_pa_prefill_append(const PrefillArgs& a, int D, int grid, int max_blocks_used,
                                    hipStream_t stream);
size_t prefill_lds_bytes(int B, int max_blocks_used);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_cow_copy(const CowArgs& a, hipStream_t stream);

}  // namespace pkv
