// C ABI of libpagedkv: argument checks (all on the host, before any HIP
// call), partition choice, workspace sizing and launches.  Declarations and
// the contract of every entry point are in include/pagedkv.h.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "kernels.h"
#include "pagedkv.h"

namespace {

constexpr int kAbiVersion = 2;
constexpr int kBlockTokens = PKV_BLOCK_TOKENS;
constexpr size_t kWsAlign = 256;
// Enough workgroups to keep all 256 CUs busy several times over.
constexpr long long kTargetWorkgroups = 2048;
constexpr int kDefaultMaxPartitionTokens = 256;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }
bool head_dim_ok(int32_t D) { return D == 64 || D == 128; }
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int waves_per_group(int32_t H) { return (H % 4 == 0) ? 4 : (H % 2 == 0) ? 2 : 1; }
// Heads per workgroup of the flat strategy: the largest power of two up to
// kFlatMaxWaves that divides H.
int flat_waves_per_group(int32_t H) {
  int w = pkv::kFlatMaxWaves;
  while (w > 1 && H % w) w /= 2;
  return w;
}

int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

// Largest partition (<= 256 tokens) that still gives enough workgroups for
// the longest context; short batches are split finer so they fill the GPU.
int32_t choose_partition(int32_t B, int32_t H, int32_t max_ctx) {
  const long long groups = (long long)B * (H / waves_per_group(H));
  int32_t part = kDefaultMaxPartitionTokens;
  while (part > kBlockTokens && groups * ceil_div(max_ctx, part) < kTargetWorkgroups) part /= 2;
  return part;
}

bool partition_ok(int32_t part) {
  return part == 0 || (part > 0 && part % kBlockTokens == 0 &&
                       part <= pkv::kMaxPartitionBlocks * kBlockTokens);
}

// How one decode call runs: the flat strategy by default (when its LDS
// staging fits), the partitioned one for an explicit partition length or
// very large batches.  A pure function of the shape.
struct Plan {
  bool flat = false;
  int32_t part = 0;        // partitioned: tokens per partition
  int32_t max_parts = 0;   // partitioned: partitions of the longest context
  int32_t nr = 0;          // flat: ranges per head group
  int32_t max_chunk = 0;   // flat: blocks in the longest range
  size_t ml_bytes = 0;     // workspace: (m, l) area, 256-byte aligned
  size_t seq_offset = 0;   // flat: byte offset of the sequence offsets
  size_t total = 0;        // workspace bytes
};

Plan make_plan(int32_t B, int32_t H, int32_t D, int32_t max_ctx, int32_t partition_tokens) {
  Plan p;
  const long long max_blocks = ceil_div(max_ctx, kBlockTokens);
  if (partition_tokens == 0 && B > 0) {
    const int32_t groups = H / flat_waves_per_group(H);
    const int32_t nr = pkv::kFlatGridTarget / groups > 0 ? pkv::kFlatGridTarget / groups : 1;
    const long long t_max = (long long)B * max_blocks;
    const long long chunk = (t_max + nr - 1) / nr;
    if (pkv::flat_lds_bytes(B, (int)(chunk < (1 << 24) ? chunk : (1 << 24))) <=
        (size_t)pkv::kFlatMaxLdsBytes) {
      p.flat = true;
      p.nr = nr;
      p.max_chunk = (int32_t)chunk;
      const size_t pieces = (size_t)H * nr * 2;
      p.ml_bytes = round_up(pieces * 2 * sizeof(float), kWsAlign);
      p.seq_offset = p.ml_bytes + round_up(pieces * D * sizeof(float), kWsAlign);
      p.total = p.seq_offset + (size_t)(B + 1) * sizeof(int32_t);
      return p;
    }
  }
  p.part = partition_tokens ? partition_tokens : choose_partition(B, H, max_ctx);
  p.max_parts = max_ctx > 0 ? ceil_div(max_ctx, p.part) : 0;
  if (p.max_parts > 1) {
    const size_t rows = (size_t)B * H * p.max_parts;
    p.ml_bytes = round_up(rows * 2 * sizeof(float), kWsAlign);
    p.total = p.ml_bytes + rows * D * sizeof(float);
  }
  return p;
}

bool decode_shape_ok(int32_t B, int32_t H, int32_t D, int32_t max_ctx) {
  return B >= 0 && H > 0 && head_dim_ok(D) && max_ctx >= 0 && max_ctx <= (1 << 24) &&
         (long long)B * H <= (1LL << 26);
}

// Grouped decode: workspace = per-sequence map (group, member), the groups'
// first positions, then (m, l) and acc of every (head, range, piece, member
// slot).  The ranges are sized without looking at device data: all groups
// together have at most B * ceil(max_ctx / 16) positions (a group's are at
// most its members' blocks), cut into nr ranges of at most max_chunk.
struct GroupPlan {
  int32_t nr = 0;          // ranges per head group
  int32_t max_chunk = 0;   // longest range, in positions
  size_t map_bytes = 0;    // workspace: per-sequence map, then group offsets, (m, l), acc
  size_t gpos_bytes = 0;
  size_t ml_bytes = 0;
  size_t total = 0;
};

// Positions of all groups at most B * ceil(max_ctx / 16); the grid asks for
// kGroupGridTarget workgroups, more ranges if a range's staging would not
// fit LDS.  Returns nr = 0 when even single-position ranges would not.
GroupPlan make_group_plan(int32_t B, int32_t H, int32_t D, int32_t max_ctx, int32_t G,
                          int32_t group_size) {
  GroupPlan p;
  const long long hg = (H + pkv::kGroupWaves - 1) / pkv::kGroupWaves;
  const long long t_max = (long long)B * ceil_div(max_ctx, kBlockTokens);
  // LDS: B context lengths, G + 1 group offsets, 4 ints a position
  const long long cap = ((long long)pkv::kGroupMaxLdsBytes / 4 - B - G - 1) / 4;   // positions
  if (cap <= 0) return p;
  long long nr = pkv::kGroupGridTarget / hg > 0 ? pkv::kGroupGridTarget / hg : 1;
  if ((t_max + nr - 1) / nr > cap) nr = (t_max + cap - 1) / cap;
  if (nr * hg >= (1LL << 31)) return p;
  p.nr = (int32_t)nr;
  p.max_chunk = (int32_t)((t_max + nr - 1) / nr);
  const size_t pieces = (size_t)H * nr * 2 * group_size;
  p.map_bytes = round_up((size_t)B * sizeof(int32_t), kWsAlign);
  p.gpos_bytes = round_up(((size_t)G + 1) * sizeof(int32_t), kWsAlign);
  p.ml_bytes = round_up(pieces * 2 * sizeof(float), kWsAlign);
  p.total = p.map_bytes + p.gpos_bytes + p.ml_bytes + pieces * D * sizeof(float);
  return p;
}

bool group_shape_ok(int32_t B, int32_t H, int32_t D, int32_t max_ctx, int32_t G,
                    int32_t group_size) {
  return decode_shape_ok(B, H, D, max_ctx) && G >= 0 && group_size >= 1 &&
         group_size <= pkv::kGroupMaxMembers && (long long)B * H * D * 2 < (1LL << 32) &&
         (long long)B * ceil_div(max_ctx, kBlockTokens) < (1LL << 31) &&
         make_group_plan(B, H, D, max_ctx, G, group_size).nr > 0;
}

}  // namespace

// Scratch of pkv_pa_decode_append_noalloc: one copy per GPU, held until the
// process ends.  In host code `scratch` only names the symbol; kernels get
// the device address that device_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on
// the first call on that device (with it current) and kept.
hipError_t device_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int32_t pkv_abi_version(void) { return kAbiVersion; }

const char* pkv_status_string(int code) {
  switch (code) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL_PTR: return "a required pointer is NULL";
    case PKV_ERR_BAD_SHAPE: return "invalid size or shape";
    case PKV_ERR_MISALIGNED: return "pointer not aligned (16 bytes for data, 4 for int32 arrays, 256 for workspace)";
    case PKV_ERR_UNSUPPORTED: return "unsupported block size (only 16 tokens per block)";
    case PKV_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than pkv_pa_decode_workspace_size";
    case PKV_ERR_HIP: return "HIP runtime error at launch";
    case PKV_ERR_SCRATCH_TOO_SMALL:
      return "shape needs more than the fixed scratch buffer (PKV_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int32_t pkv_pa_decode_default_partition(int32_t B, int32_t H, int32_t D, int32_t max_context_len) {
  if (!decode_shape_ok(B, H, D, max_context_len)) return 0;
  const Plan p = make_plan(B, H, D, max_context_len, 0);
  return p.flat ? 0 : p.part;
}

size_t pkv_pa_decode_workspace_size_ex(int32_t B, int32_t H, int32_t D, int32_t max_context_len,
                                       int32_t partition_tokens) {
  if (!decode_shape_ok(B, H, D, max_context_len) || !partition_ok(partition_tokens)) return 0;
  return make_plan(B, H, D, max_context_len, partition_tokens).total;
}

size_t pkv_pa_decode_workspace_size(int32_t B, int32_t H, int32_t D, int32_t max_context_len) {
  return pkv_pa_decode_workspace_size_ex(B, H, D, max_context_len, 0);
}

namespace {

// pkv_pa_decode_ex, and with k_new / v_new the decode with the fused append
// (flat strategy only).
int decode_impl(const void* q, const void* k_pool, const void* v_pool,
                const int32_t* block_tables, int32_t max_blocks_per_seq,
                const int32_t* context_lens, int32_t max_context_len, int32_t B, int32_t H,
                int32_t D, int32_t block_size, int32_t num_blocks, float scale, void* out,
                void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                uint32_t flags, const void* k_new, const void* v_new, void* stream,
                bool use_scratch = false) {
  const bool append = k_new != nullptr || v_new != nullptr;
  if (block_size != kBlockTokens) return PKV_ERR_UNSUPPORTED;
  if (flags & ~(uint32_t)PKV_DECODE_KEEP_KV_CACHED) return PKV_ERR_BAD_SHAPE;
  const bool keep_cached = (flags & PKV_DECODE_KEEP_KV_CACHED) != 0;
  if (!decode_shape_ok(B, H, D, max_context_len) || !partition_ok(partition_tokens))
    return PKV_ERR_BAD_SHAPE;
  if (B == 0) return PKV_OK;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      (long long)max_blocks_per_seq * kBlockTokens < max_context_len)
    return PKV_ERR_BAD_SHAPE;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out) return PKV_ERR_NULL_PTR;
  if (append && (!k_new || !v_new)) return PKV_ERR_NULL_PTR;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PKV_ERR_MISALIGNED;
  if (append && (!aligned(k_new, 16) || !aligned(v_new, 16))) return PKV_ERR_MISALIGNED;

  const Plan plan = make_plan(B, H, D, max_context_len, partition_tokens);
  if (append && !plan.flat) return PKV_ERR_UNSUPPORTED;
  if (use_scratch) {                   // the library's array instead of a workspace
    if (plan.total > PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH_TOO_SMALL;
    if (device_scratch(&workspace) != hipSuccess) return PKV_ERR_HIP;
    workspace_bytes = PKV_NOALLOC_SCRATCH_BYTES;
  }
  if (plan.total > 0) {
    if (!workspace) return PKV_ERR_NULL_PTR;
    if (!aligned(workspace, kWsAlign)) return PKV_ERR_MISALIGNED;
    if (workspace_bytes < plan.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  }
  const int wpg = waves_per_group(H);
  float* ws_ml = plan.total ? static_cast<float*>(workspace) : nullptr;
  float* ws_acc =
      plan.total ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ml_bytes) : nullptr;
  hipError_t e;
  if (plan.flat) {
    const int fw = flat_waves_per_group(H);
    pkv::FlatArgs a;
    a.q = static_cast<const _Float16*>(q);
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = static_cast<_Float16*>(out);
    a.ws_ml = ws_ml;
    a.ws_acc = ws_acc;
    a.ws_seq = reinterpret_cast<int*>(static_cast<char*>(workspace) + plan.seq_offset);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.B = B;
    a.H = H;
    a.max_blocks = max_blocks_per_seq;
    a.ctx_limit = max_context_len;
    a.num_blocks = num_blocks;
    a.head_groups = H / fw;
    a.waves_per_group = fw;
    a.nr = plan.nr;
    a.max_chunk = plan.max_chunk;
    a.keep_cached = keep_cached;
    a.contig = false;
    a.row_tokens = 0;
    a.capacity = nullptr;
    a.k_new = static_cast<const _Float16*>(k_new);
    a.v_new = static_cast<const _Float16*>(v_new);
    e = pkv::launch_pa_decode_flat(a, D, fw * 64, static_cast<hipStream_t>(stream));
  } else {
    const long long grid = (long long)B * (H / wpg) * (plan.max_parts > 0 ? plan.max_parts : 1);
    if (grid >= (1LL << 31)) return PKV_ERR_BAD_SHAPE;
    pkv::PartArgs a;
    a.q = static_cast<const _Float16*>(q);
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = static_cast<_Float16*>(out);
    a.ws_ml = ws_ml;
    a.ws_acc = ws_acc;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.B = B;
    a.H = H;
    a.max_blocks = max_blocks_per_seq;
    a.ctx_limit = max_context_len;
    a.num_blocks = num_blocks;
    a.part_blocks = plan.part / kBlockTokens;
    a.max_parts = plan.max_parts;
    a.head_groups = H / wpg;
    a.waves_per_group = wpg;
    a.keep_cached = keep_cached;
    e = pkv::launch_pa_decode(a, D, (int)grid, wpg * 64, static_cast<hipStream_t>(stream));
  }
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

int pkv_pa_decode_ex(const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, int32_t B, int32_t H,
                     int32_t D, int32_t block_size, int32_t num_blocks, float scale, void* out,
                     void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                     uint32_t flags, void* stream) {
  return decode_impl(q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, B, H, D, block_size, num_blocks, scale, out, workspace,
                     workspace_bytes, partition_tokens, flags, nullptr, nullptr, stream);
}

int pkv_pa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_pool,
                         void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t max_context_len, int32_t B,
                         int32_t H, int32_t D, int32_t block_size, int32_t num_blocks, float scale,
                         void* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                         void* stream) {
  if (!k_new || !v_new) return PKV_ERR_NULL_PTR;
  return decode_impl(q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, B, H, D, block_size, num_blocks, scale, out, workspace,
                     workspace_bytes, 0, flags, k_new, v_new, stream);
}

int pkv_pa_decode_append_noalloc(const void* q, const void* k_new, const void* v_new,
                                 void* k_pool, void* v_pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t max_context_len, int32_t B, int32_t H, int32_t D,
                                 int32_t block_size, int32_t num_blocks, float scale, void* out,
                                 uint32_t flags, void* stream) {
  if (!k_new || !v_new) return PKV_ERR_NULL_PTR;
  return decode_impl(q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                     max_context_len, B, H, D, block_size, num_blocks, scale, out, nullptr, 0, 0,
                     flags, k_new, v_new, stream, true);
}

int pkv_pa_decode(const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, int32_t max_context_len, int32_t B, int32_t H,
                  int32_t D, int32_t block_size, int32_t num_blocks, float scale, void* out,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return pkv_pa_decode_ex(q, k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens,
                          max_context_len, B, H, D, block_size, num_blocks, scale, out, workspace,
                          workspace_bytes, 0, 0u, stream);
}

size_t pkv_contig_decode_workspace_size(int32_t B, int32_t H, int32_t D,
                                        int32_t max_context_len) {
  if (!decode_shape_ok(B, H, D, max_context_len) || B == 0) return 0;
  const Plan p = make_plan(B, H, D, max_context_len, 0);
  return p.flat ? p.total : 0;
}

int pkv_contig_decode(const void* q, const void* k_buf, const void* v_buf, int32_t row_tokens,
                      const int32_t* context_lens, const int32_t* capacity,
                      int32_t max_context_len, int32_t B, int32_t H, int32_t D, float scale,
                      void* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                      void* stream) {
  if (flags != 0) return PKV_ERR_BAD_SHAPE;
  if (!decode_shape_ok(B, H, D, max_context_len)) return PKV_ERR_BAD_SHAPE;
  if (B == 0) return PKV_OK;
  if (row_tokens <= 0 || row_tokens % kBlockTokens || row_tokens < max_context_len ||
      (long long)B * (row_tokens / kBlockTokens) >= (1LL << 31) ||
      (long long)H * D * 2 * kBlockTokens >= (1LL << 31))
    return PKV_ERR_BAD_SHAPE;
  const Plan plan = make_plan(B, H, D, max_context_len, 0);
  if (!plan.flat) return PKV_ERR_UNSUPPORTED;
  if (!q || !k_buf || !v_buf || !context_lens || !out || !workspace) return PKV_ERR_NULL_PTR;
  if (!aligned(q, 16) || !aligned(k_buf, 16) || !aligned(v_buf, 16) || !aligned(out, 16) ||
      !aligned(context_lens, 4) || !aligned(capacity, 4) || !aligned(workspace, kWsAlign))
    return PKV_ERR_MISALIGNED;
  if (workspace_bytes < plan.total) return PKV_ERR_WORKSPACE_TOO_SMALL;
  const int fw = flat_waves_per_group(H);
  pkv::FlatArgs a;
  a.q = static_cast<const _Float16*>(q);
  a.k_pool = k_buf;
  a.v_pool = v_buf;
  a.block_tables = nullptr;
  a.context_lens = context_lens;
  a.out = static_cast<_Float16*>(out);
  a.ws_ml = static_cast<float*>(workspace);
  a.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ml_bytes);
  a.ws_seq = reinterpret_cast<int*>(static_cast<char*>(workspace) + plan.seq_offset);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.B = B;
  a.H = H;
  a.max_blocks = row_tokens / kBlockTokens;
  a.ctx_limit = max_context_len;
  a.num_blocks = B * (row_tokens / kBlockTokens);
  a.head_groups = H / fw;
  a.waves_per_group = fw;
  a.nr = plan.nr;
  a.max_chunk = plan.max_chunk;
  a.keep_cached = false;
  a.contig = true;
  a.row_tokens = row_tokens;
  a.capacity = capacity;
  a.k_new = nullptr;
  a.v_new = nullptr;
  const hipError_t e = pkv::launch_pa_decode_flat(a, D, fw * 64, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

size_t pkv_pa_decode_grouped_workspace_size(int32_t B, int32_t H, int32_t D,
                                            int32_t max_context_len, int32_t num_groups,
                                            int32_t group_size) {
  if (!group_shape_ok(B, H, D, max_context_len, num_groups, group_size) || B == 0) return 0;
  return make_group_plan(B, H, D, max_context_len, num_groups, group_size).total;
}

int pkv_pa_decode_grouped(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len,
                          const int32_t* group_offsets, const int32_t* group_shared_blocks,
                          int32_t num_groups, int32_t group_size, int32_t B, int32_t H,
                          int32_t D, int32_t block_size, int32_t num_blocks, float scale,
                          void* out, void* workspace, size_t workspace_bytes, uint32_t flags,
                          void* stream) {
  if (block_size != kBlockTokens) return PKV_ERR_UNSUPPORTED;
  if (flags & ~(uint32_t)PKV_DECODE_KEEP_KV_CACHED) return PKV_ERR_BAD_SHAPE;
  if (!group_shape_ok(B, H, D, max_context_len, num_groups, group_size)) return PKV_ERR_BAD_SHAPE;
  if (B == 0) return PKV_OK;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      (long long)max_blocks_per_seq * kBlockTokens < max_context_len)
    return PKV_ERR_BAD_SHAPE;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out) return PKV_ERR_NULL_PTR;
  if (num_groups > 0 && (!group_offsets || !group_shared_blocks)) return PKV_ERR_NULL_PTR;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(group_offsets, 4) ||
      !aligned(group_shared_blocks, 4))
    return PKV_ERR_MISALIGNED;
  const GroupPlan plan = make_group_plan(B, H, D, max_context_len, num_groups, group_size);
  if (!workspace) return PKV_ERR_NULL_PTR;
  if (!aligned(workspace, kWsAlign)) return PKV_ERR_MISALIGNED;
  if (workspace_bytes < plan.total) return PKV_ERR_WORKSPACE_TOO_SMALL;

  pkv::GroupArgs a;
  a.q = static_cast<const _Float16*>(q);
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.group_offsets = group_offsets;
  a.group_shared = group_shared_blocks;
  a.out = static_cast<_Float16*>(out);
  char* ws = static_cast<char*>(workspace);
  a.ws_map = reinterpret_cast<int*>(ws);
  a.ws_gpos = reinterpret_cast<int*>(ws + plan.map_bytes);
  a.ws_ml = reinterpret_cast<float*>(ws + plan.map_bytes + plan.gpos_bytes);
  a.ws_acc = reinterpret_cast<float*>(ws + plan.map_bytes + plan.gpos_bytes + plan.ml_bytes);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.B = B;
  a.H = H;
  a.G = num_groups;
  a.max_blocks = max_blocks_per_seq;
  a.ctx_limit = max_context_len;
  a.num_blocks = num_blocks;
  a.group_size = group_size;
  a.head_groups = (H + pkv::kGroupWaves - 1) / pkv::kGroupWaves;
  a.nr = plan.nr;
  a.max_chunk = plan.max_chunk;
  const long long t_cap = (long long)plan.nr * plan.max_chunk;
  a.t_cap = (int)(t_cap < 0x7fffffffLL ? t_cap : 0x7fffffffLL);
  a.keep_cached = (flags & PKV_DECODE_KEEP_KV_CACHED) != 0;
  const hipError_t e = pkv::launch_pa_decode_grouped(a, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

namespace {

// pkv_pa_prefill and pkv_pa_prefill_append: k_new / v_new are null for the
// former, the new tokens' rows for the latter.
int prefill_call(const void* q, const void* k_new, const void* v_new, const void* k_pool,
                 const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* context_lens, int32_t max_context_len,
                 const int32_t* query_start, int32_t num_query_rows, int32_t B, int32_t H,
                 int32_t D, int32_t block_size, int32_t num_blocks, float scale, void* out,
                 uint32_t flags, void* stream, bool append) {
  if (block_size != kBlockTokens) return PKV_ERR_UNSUPPORTED;
  // flags: 0, or bits 8..15 = 1 + log2(heads per item), at most 8 heads
  const uint32_t hcode = (flags >> 8) & 0xffu;
  if ((flags & ~0xff00u) != 0 || hcode > 4) return PKV_ERR_BAD_SHAPE;
  if (!decode_shape_ok(B, H, D, max_context_len) || num_query_rows < 0 ||
      (long long)num_query_rows * H * D * 2 >= (1LL << 32))
    return PKV_ERR_BAD_SHAPE;
  if (B == 0 || num_query_rows == 0) return PKV_OK;
  if (num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      (long long)max_blocks_per_seq * kBlockTokens < max_context_len)
    return PKV_ERR_BAD_SHAPE;
  const int32_t blocks_used = ceil_div(max_context_len, kBlockTokens);
  if (pkv::prefill_lds_bytes(B, blocks_used) > (size_t)pkv::kPrefillMaxLdsBytes)
    return PKV_ERR_BAD_SHAPE;
  // query groups: sum over sequences of ceil(n_b / R) <= num_query_rows / R + B, R = kPrefillRows
  const long long bound = ((long long)ceil_div(num_query_rows, pkv::kPrefillRows) + B) * H;
  if (bound >= (1LL << 31)) return PKV_ERR_BAD_SHAPE;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start || !out ||
      (append && (!k_new || !v_new)))
    return PKV_ERR_NULL_PTR;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4) ||
      (append && (!aligned(k_new, 16) || !aligned(v_new, 16))))
    return PKV_ERR_MISALIGNED;
  pkv::PrefillArgs a;
  a.q = static_cast<const _Float16*>(q);
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.out = static_cast<_Float16*>(out);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.B = B;
  a.H = H;
  a.num_rows = num_query_rows;
  a.max_blocks = max_blocks_per_seq;
  a.ctx_limit = max_context_len;
  a.num_blocks = num_blocks;
  a.k_new = append ? static_cast<const _Float16*>(k_new) : nullptr;
  a.v_new = append ? static_cast<const _Float16*>(v_new) : nullptr;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return PKV_ERR_HIP;
  const long long slots = (long long)cus * pkv::kPrefillSlotsPerCU;   // resident workgroups
  // Heads per item: the largest power of two (up to kPrefillMaxHeadsPerItem)
  // that leaves about kPrefillItemsPerSlot items per resident workgroup,
  // with the query groups estimated halfway between their bounds
  // (ceil(rows / R) and that plus B).
  const long long groups_est = ceil_div(num_query_rows, pkv::kPrefillRows) + B / 2;
  int hpi = 1;
  while (2 * hpi <= H && 2 * hpi <= pkv::kPrefillMaxHeadsPerItem &&
         groups_est * ceil_div(H, 2 * hpi) >= pkv::kPrefillItemsPerSlot * slots)
    hpi *= 2;
  if (hcode != 0) hpi = 1 << (hcode - 1);
  if (hpi > H) hpi = H;
  a.heads_per_item = hpi;
  // The items run in a grid-stride loop over at most eight workgroups per
  // resident slot: few enough that no workgroup is launched only to find no
  // item, enough that the hardware's dispatch still balances items of
  // unequal length; a multiple of 8, so item i stays on XCD i % 8.
  const long long items_bound = bound / H * ceil_div(H, hpi);
  const long long grid_cap = slots * 8;
  const int grid = (int)(items_bound < grid_cap ? items_bound : grid_cap);
  const hipError_t e =
      append ? pkv::launch_pa_prefill_append(a, D, grid, blocks_used, static_cast<hipStream_t>(stream))
             : pkv::launch_pa_prefill(a, D, grid, blocks_used, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

int pkv_pa_prefill(const void* q, const void* k_pool, const void* v_pool,
                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* context_lens, int32_t max_context_len,
                   const int32_t* query_start, int32_t num_query_rows, int32_t B, int32_t H,
                   int32_t D, int32_t block_size, int32_t num_blocks, float scale, void* out,
                   uint32_t flags, void* stream) {
  return prefill_call(q, nullptr, nullptr, k_pool, v_pool, block_tables, max_blocks_per_seq,
                      context_lens, max_context_len, query_start, num_query_rows, B, H, D,
                      block_size, num_blocks, scale, out, flags, stream, false);
}

int pkv_pa_prefill_append(const void* q, const void* k_new, const void* v_new, void* k_pool,
                          void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len,
                          const int32_t* query_start, int32_t num_query_rows, int32_t B,
                          int32_t H, int32_t D, int32_t block_size, int32_t num_blocks,
                          float scale, void* out, uint32_t flags, void* stream) {
  return prefill_call(q, k_new, v_new, k_pool, v_pool, block_tables, max_blocks_per_seq,
                      context_lens, max_context_len, query_start, num_query_rows, B, H, D,
                      block_size, num_blocks, scale, out, flags, stream, true);
}

int pkv_kv_append(const void* k, const void* v, const int32_t* slot_mapping, int32_t T,
                  void* k_pool, void* v_pool, int32_t num_blocks, int32_t H, int32_t D,
                  int32_t block_size, void* stream) {
  if (block_size != kBlockTokens) return PKV_ERR_UNSUPPORTED;
  if (T < 0 || H <= 0 || !head_dim_ok(D) || num_blocks <= 0) return PKV_ERR_BAD_SHAPE;
  if (T == 0) return PKV_OK;
  if (((long long)T + 15) / 16 * 16 * H * (D / 8) >= (1LL << 31) * 256LL) return PKV_ERR_BAD_SHAPE;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return PKV_ERR_NULL_PTR;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(slot_mapping, 4))
    return PKV_ERR_MISALIGNED;
  pkv::AppendArgs a;
  a.k = k;
  a.v = v;
  a.slots = slot_mapping;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.T = T;
  a.H = H;
  a.D = D;
  a.num_blocks = num_blocks;
  const hipError_t e = pkv::launch_kv_append(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_cow_copy_blocks(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                        const int32_t* src_dst_pairs, int32_t n_pairs, int32_t num_blocks,
                        int64_t block_bytes, void* stream) {
  if (num_layers <= 0 || n_pairs < 0 || num_blocks <= 0 || block_bytes <= 0 || block_bytes % 16)
    return PKV_ERR_BAD_SHAPE;
  if (n_pairs == 0) return PKV_OK;
  if ((long long)n_pairs * 2 * pkv::kMaxCowLayers >= (1LL << 31)) return PKV_ERR_BAD_SHAPE;
  if (!k_pools || !v_pools || !src_dst_pairs) return PKV_ERR_NULL_PTR;
  for (int32_t l = 0; l < num_layers; ++l) {
    if (!k_pools[l] || !v_pools[l]) return PKV_ERR_NULL_PTR;
    if (!aligned(k_pools[l], 16) || !aligned(v_pools[l], 16)) return PKV_ERR_MISALIGNED;
  }
  if (!aligned(src_dst_pairs, 4)) return PKV_ERR_MISALIGNED;
  for (int32_t l0 = 0; l0 < num_layers; l0 += pkv::kMaxCowLayers) {
    pkv::CowArgs a;
    memset(&a, 0, sizeof(a));
    a.layers = num_layers - l0 < pkv::kMaxCowLayers ? num_layers - l0 : pkv::kMaxCowLayers;
    for (int i = 0; i < a.layers; ++i) {
      a.k[i] = k_pools[l0 + i];
      a.v[i] = v_pools[l0 + i];
    }
    a.pairs = src_dst_pairs;
    a.block_bytes = block_bytes;
    a.n_pairs = n_pairs;
    a.num_blocks = num_blocks;
    const hipError_t e = pkv::launch_cow_copy(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return PKV_ERR_HIP;
  }
  return PKV_OK;
}

int pkv_hbm_read_probe(const void* buf, size_t bytes, void* sink, int32_t workgroups,
                       void* stream) {
  if (bytes == 0 || bytes % 16 || workgroups <= 0) return PKV_ERR_BAD_SHAPE;
  if (!buf || !sink) return PKV_ERR_NULL_PTR;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return PKV_ERR_MISALIGNED;
  const hipError_t e = pkv::launch_hbm_read_probe(buf, (long long)(bytes / 16),
                                                  static_cast<uint32_t*>(sink), workgroups,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_hbm_copy_probe(const void* src, void* dst, size_t bytes, int32_t workgroups,
                       void* stream) {
  if (bytes == 0 || bytes % 16 || workgroups <= 0) return PKV_ERR_BAD_SHAPE;
  if (!src || !dst) return PKV_ERR_NULL_PTR;
  if (!aligned(src, 16) || !aligned(dst, 16)) return PKV_ERR_MISALIGNED;
  const hipError_t e = pkv::launch_hbm_copy_probe(src, dst, (long long)(bytes / 16), workgroups,
                                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int pkv_hbm_gather_probe(const void* buf, size_t bytes, const int32_t* chunk_order,
                         int32_t chunk_bytes, void* sink, int32_t workgroups, void* stream) {
  int log_kib = -1;
  for (int k = 0; k <= 10; ++k)
    if (chunk_bytes == (1 << (10 + k))) log_kib = k;
  if (bytes == 0 || log_kib < 0 || bytes % (size_t)chunk_bytes || workgroups <= 0)
    return PKV_ERR_BAD_SHAPE;
  if (!buf || !chunk_order || !sink) return PKV_ERR_NULL_PTR;
  if (!aligned(buf, 16) || !aligned(chunk_order, 4) || !aligned(sink, 4)) return PKV_ERR_MISALIGNED;
  const hipError_t e = pkv::launch_hbm_gather_probe(
      buf, chunk_order, (long long)(bytes / (size_t)chunk_bytes), log_kib,
      static_cast<uint32_t*>(sink), workgroups, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
