// Paged prefill for gfx950 (MI355X): the new tokens of every sequence (a
// prompt, or a chunk of one, already appended to its pages) attend causally
// over the sequence's block-paged KV cache.
//
// "PagedAttention" (e-fortepiano.pl), "Formulació matemàtica": causal
// self-attention computed block by block over the paged cache; a query
// token sees the tokens up to and including its own position.  Query row i
// of sequence b (n_b rows) sits at position ctx_b - n_b + i.
//
// Work: a workgroup takes 128 consecutive query rows of one sequence for
// one head; each of its 4 waves serves 32 of them.  The workgroup streams
// the blocks up to the one holding its last row's position once: every
// (block, head) tile of K and V is fetched by the workgroup's threads
// together (16 bytes each), copied straight from memory into one of four
// LDS pair slots (buffer_load ... lds) or, with the append fused in,
// through a register ring of four tiles into one of three (V slots past the
// context zeroed, V token slots swizzled against bank conflicts); after
// every pair of tiles a barrier, then each wave consumes the pair (32
// tokens), its score products issued one pair ahead of its softmax, on the
// v_mfma_f32_32x32x16_f16 matrix instruction, whose lane l holds row l%32
// and k slots 8*(l/32) .. +7 of A, the same of B (column l%32), and C rows
// 8*(r/4) + 4*(l/32) + r%4 of column l%32 in its register r:
//  * scores S^T (32 tokens x 32 queries) = K . Q^T, one MFMA per 16 dims:
//    lane l reads the 16 bytes of token l%32 (tile (l%32)/16), dims
//    16i + 8*(l/32) .. +7 from LDS as its A operand; the queries are the B
//    operand, loaded once;
//  * online softmax per query column: a query's 32 scores sit in lanes c and
//    c + 32 (16 each), combined with one permlane32 swap; the weights are
//    rounded to fp16 once and the running sum uses the rounded weights;
//  * O^T (D x 32 queries) += V^T . P^T, per 32 output dims one MFMA per tile:
//    its k slot 8h + e (h = l/32) is token 4h + e%4 + 8*(e/4) of the tile,
//    which is exactly score registers 8kk .. 8kk+7 (kk = the tile), so P^T
//    is the score result itself; V^T comes from two transpose reads (tokens
//    4h .. 4h+3 and 8+4h .. 8+4h+3).
// Blocks past a row's position are exact no-ops for it (causal mask per
// element), so a row's result does not depend on the rows it shares a
// workgroup with.  Workgroups take (query group, head group) items in a
// grid-stride loop: an item covers a few consecutive heads of one query
// group, and its tile pipeline runs straight through them (the next head's
// queries are loaded while the last pair of the current one is in flight,
// a finished head's rows are written at the next step), so the set-up of an
// item and the fill of its pipeline are paid once per head group.  Item i
// serves head group i % G (G head groups), and with a grid that is a
// multiple of 8 it runs on XCD i % 8 (one XCD per head group when G is a
// multiple of 8).  Within a sequence the groups that reach furthest come
// first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "pa_common.h"
#include "pa_mfma.h"

namespace pkv {
namespace {

using namespace dev;

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// s_waitcnt operand for "at most n vector memory operations outstanding"
// (gfx9 encoding: vmcnt bits 3:0 and 15:14; expcnt and lgkmcnt at their
// maxima, so they do not wait)
constexpr unsigned waitcnt_vm(unsigned n) {
  return (n & 0xfu) | ((n >> 4) << 14) | (0x7u << 4) | (0xfu << 8);
}

// LDS slot of V unit u = g * 16 + token (8 dims of dim group g of one
// token): the token index is XOR-ed with 4 * (g % 4), so that the 16 lanes
// of a transpose read, which take tokens t0 .. t0+3 (t0 % 4 == 0) of dim
// groups g0 and g0 + 1 (and the next 16 lanes g0 + 2, g0 + 3), meet 16
// distinct 16-byte slots of the LDS banks; writes of whole rows of 16
// tokens stay conflict-free (a permutation inside a row).
__device__ __forceinline__ int v_slot(int u) { return u ^ (4 * ((u >> 4) & 3)); }

// Slack of the reference maximum, in log2 units: weights stay below 2^8
// (exact in fp16's range; the fp32 sums have room to spare).
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ int rows_of(const PrefillArgs& a, int b) {
  return max(0, a.query_start[b + 1] - a.query_start[b]);
}

__device__ __forceinline__ int groups_of(const PrefillArgs& a, int b) {
  return (rows_of(a, b) + kPrefillRows - 1) / kPrefillRows;
}

// s_group[b] = first query group of sequence b over the batch, s_group[B] =
// total.  All threads take part; ends with a barrier.
__device__ void group_prefix(const PrefillArgs& a, int* s_group, int* s_wave) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int per = (a.B + nt - 1) / nt;
  const int lo = min(a.B, tid * per);
  const int hi = min(a.B, lo + per);
  int own = 0;
  for (int b = lo; b < hi; ++b) own += groups_of(a, b);
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  int incl = own;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  int run = incl - own;
  for (int w = 0; w < wave; ++w) run += s_wave[w];
  for (int b = lo; b < hi; ++b) {
    s_group[b] = run;
    run += groups_of(a, b);
  }
  if (tid == nt - 1) s_group[a.B] = run;
  __syncthreads();
}

// The sequence of query group t: the largest b < B with s_group[b] <= t.
// The whole wave searches, 64 candidates a round (one LDS read each and a
// ballot): the answer stays in [lo, lo + len), where s_group[lo] <= t, and
// since s_group does not decrease, the candidates that pass form a prefix
// of the lanes.  B <= 4096 takes at most two rounds.  Uniform result; every
// lane of the wave must be active.
__device__ __forceinline__ int seq_of_group(const int* s_group, int B, int t) {
  const int lane = threadIdx.x % kWave;
  int lo = 0, len = B;
  while (len > 1) {
    const int step = (len + kWave - 1) / kWave;
    const int c = lo + step * lane;
    const bool pass = c < lo + len && s_group[min(c, lo + len - 1)] <= t;
    const uint64_t m = __ballot(pass);
    const int k = 63 - __clzll(m | 1ull);                // the last lane that passes
    const int c0 = lo + step * k;
    len = min(step, lo + len - c0);
    lo = c0;
  }
  return __builtin_amdgcn_readfirstlane(lo);
}

// Two waves per SIMD (two workgroups per CU): the register budget that
// allows fits the kernel without spilling.
//
// kAppend: the append of the new tokens is fused in.  Blocks whose tokens
// are all new are read from the caller's rows (a.k_new / a.v_new) instead
// of the pools; blocks with cached tokens (the one the new tokens start in
// included, whose new tokens a separate kernel writes first) come from the
// pools.  The source is one choice per tile, taken with selects, and the
// item whose query rows hold a block's first token writes that block to
// the pools as it stages it (a store with an empty range for the other
// tiles), so the load ring keeps its fixed shape.
template <int D, bool kAppend, bool kMulti>
__global__ __launch_bounds__(64 * kPrefillWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void pa_prefill_kernel(PrefillArgs a) {
  typedef float f16x16 __attribute__((ext_vector_type(16)));
  typedef short s4v __attribute__((ext_vector_type(4)));
  typedef short s8v __attribute__((ext_vector_type(8)));
  constexpr int kQK = D / 16;                           // score MFMAs (16 dims each)
  constexpr int kSl = D / 32;                           // output slices of 32 dims
  constexpr int kTile = D * kBlockTokens * 2;           // bytes of one K (or V) tile
  constexpr int kTileUnits = kTile / 16;                // 16-byte units of one tile
  constexpr int kThreads = 64 * kPrefillWaves;
  constexpr int kLoaders = 2 * kTileUnits < kThreads ? 2 * kTileUnits : kThreads;
  constexpr int kUnits = 2 * kTileUnits / kLoaders;     // 16-byte units per loading thread
  constexpr int R = 4;                                  // register ring: two pairs of tiles
  constexpr int kSlots = 3;                             // LDS pair slots
  static_assert(kUnits >= 1 && kLoaders % kWave == 0, "tile split; whole loading waves");
  // Without the append, tiles go from HBM straight into LDS (no register
  // ring); with it, through registers, since the item that owns an all-new
  // block also writes it to the pools.
  constexpr bool kDma = !kAppend;
  static_assert(!kDma || kLoaders == kThreads, "every thread copies a share of each pair");
  extern __shared__ __attribute__((aligned(16))) int smem[];
  __shared__ int s_wave[kPrefillWaves];
  // register-ring staging: three pair slots, each its K tile then V tile
  __shared__ u4v s_kv[kDma ? 1 : 2 * kSlots][kDma ? 1 : 2 * kTileUnits];
  // direct staging: four pair slots as four arrays, so that the compiler
  // tells them apart when it places waits before LDS reads (a read of one
  // slot does not wait for copies still landing in another)
  __shared__ u4v s_d0[kDma ? 2 : 1][kDma ? 2 * kTileUnits : 1];
  __shared__ u4v s_d1[kDma ? 2 : 1][kDma ? 2 * kTileUnits : 1];
  __shared__ u4v s_d2[kDma ? 2 : 1][kDma ? 2 * kTileUnits : 1];
  __shared__ u4v s_d3[kDma ? 2 : 1][kDma ? 2 * kTileUnits : 1];
  int* s_group = smem;                                  // B + 1
  // block ids of the sequence, 8-byte aligned with one spare entry, so that
  // the two ids of a pair of blocks are read together
  int* s_ids = smem + ((a.B + 2) & ~1);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int col = lane % 32;                            // query column of this lane
  const int hf = lane / 32;                             // k-slot half of this lane

  group_prefix(a, s_group, s_wave);
  // Items (query group, head group), longest-reaching groups first, in a
  // grid-stride loop: the prefix above is computed once per workgroup for
  // its few items, and no workgroup is launched only to find none.  An item
  // covers heads h0 .. h0 + nh - 1 of its query group: the sequence's
  // parameters and block ids are set up once, and the tile pipeline runs on
  // across the head boundaries as over one sequence of nh * npairs pairs.
  const int hpi = a.heads_per_item;
  const int hgroups = (a.H + hpi - 1) / hpi;
  const int items = s_group[a.B] * hgroups;
  // An item's sequence, the first blockDim.x entries of its block table and
  // its lengths.  With direct staging they are loaded one item ahead, while
  // the item before waits for its first copies, so that their latency is
  // not paid at the item's start.  Entries past the item's blocks are not
  // used.  nx_len: lane 0 holds the sequence's first query row, lane 1 the
  // end of its rows, the other lanes its context length (one vector load).
  // Every path through an item issues these loads once and waits for them
  // with the item's first copies, so that the compiler's wait for them at
  // the next item's start leaves the item's output stores in flight.
  const int cap = min(a.max_blocks, (a.ctx_limit + kBlockTokens - 1) / kBlockTokens);
  int nx_b = 0, nx_id = 0, nx_len = 0;
  // (past the last item, the last item's again: the loads are issued on
  // every path, so the compiler's count of the loads in flight stays exact)
  auto load_item = [&](int it) {
    nx_b = seq_of_group(s_group, a.B, max(0, min(it, items - 1)) / hgroups);
    nx_id = tid < cap ? a.block_tables[(size_t)nx_b * a.max_blocks + tid] : 0;
    const int lane = tid % kWave;
    nx_len = lane < 2 ? a.query_start[nx_b + lane] : a.context_lens[nx_b];
  };
  if constexpr (kDma) {
    load_item(blockIdx.x);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    // (the register ring loads its item's at the start: loaded one item
    // ahead there, its loop compiles to a slower schedule)
    if constexpr (!kDma) load_item(item);
    const int gt = item / hgroups;
    const int h0 = (item - gt * hgroups) * hpi;
    const int nh = kMulti ? min(hpi, a.H - h0) : 1;
    // (the item's parameters are the same for every lane: taken as uniform,
    // so that they live in scalar registers)
    const int b = nx_b;
    const int id_first = nx_id;
    const int qs_b = __builtin_amdgcn_readlane(nx_len, 0);
    const int n = max(0, __builtin_amdgcn_readlane(nx_len, 1) - qs_b);
    const int kq = (n + kPrefillRows - 1) / kPrefillRows - 1 -
                   (gt - __builtin_amdgcn_readfirstlane(s_group[b]));   // furthest-reaching first
    const int ctx = clampi(__builtin_amdgcn_readlane(nx_len, 2), 0, a.ctx_limit);
    const int row0 = kPrefillRows * kq;
    const int grows = min(kPrefillRows, n - row0);
    const int p_group = ctx - n + row0;                   // position of the group's first row
    const int p_last = min(p_group + grows - 1, ctx - 1);
    const int nblk = p_last >= 0 ? p_last / kBlockTokens + 1 : 0;
    // fused append: position of the sequence's first new token, and the
    // first block whose tokens are all new
    const int bnd = ctx - n;
    const int jn = kAppend ? (max(bnd, 0) + kBlockTokens - 1) / kBlockTokens : 0x7fffffff;

    // Block ids, clamped into the pool for reading.  With the append, an
    // entry outside the pool also sets bit 31, so the block is never written.
    // The entry after the last block is block 0 (read with the last pair).
    // (the entries past the first blockDim.x are loaded here, in a loop of
    // their own, so that the compiler's wait for them stays inside it)
    auto put_id = [&](int j, int id) {
      const int in_pool = clampi(id, 0, a.num_blocks - 1);
      s_ids[j] = kAppend && in_pool != id ? (int)((uint32_t)in_pool | 0x80000000u) : in_pool;
    };
    if (tid <= nblk) put_id(tid, tid == nblk ? 0 : id_first);
    for (int j = tid + blockDim.x; j <= nblk; j += blockDim.x)
      put_id(j, j == nblk ? 0 : a.block_tables[(size_t)b * a.max_blocks + j]);
    __syncthreads();

    // this lane's query row: wave w serves rows row0 + 32w ..; a wave with no
    // row skips the arithmetic (it still loads, stages and meets the barriers)
    const bool wave_rows = 32 * wave < grows;
    const int wrow = 32 * wave + col;
    const int qrow = qs_b + row0 + wrow;
    const bool row_ok = wrow < grows && qrow >= 0 && qrow < a.num_rows;
    const int p_q = p_group + wrow;
    const rsrc_t qr = make_rsrc(a.q, (uint32_t)((size_t)a.num_rows * a.H * D * 2));
    const uint32_t qrow_off = (uint32_t)(((size_t)qrow * a.H * D + 8 * hf) * 2);
    h8v qb[kQK];                                          // B operands: dims 16i + 8hf ..
    // the queries of head h (no row: past the resource, reads 0)
    auto load_q = [&](int h) {
      const uint32_t off = row_ok ? qrow_off + (uint32_t)(h * D * 2) : 0xFFFFFFF0u;
  #pragma unroll
      for (int i = 0; i < kQK; ++i)
        qb[i] = as_h8(__builtin_amdgcn_raw_buffer_load_b128(qr, off + (row_ok ? i * 32 : 0), 0, 0));
    };
    // The scores are taken as (sign(scale) q) . k (an exact negation), so that
    // their maximum is the maximum of the scaled scores; weights are then
    // exp2(s * |scale log2 e| - m) with one fused multiply-add.
    // (a zero scale is taken as the smallest normal float: the weights are
    // then exactly 1, and a masked score's -inf times it stays -inf)
    const float sabs = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
    auto sign_q = [&]() {
      if (a.scale_log2 < 0.0f) {
  #pragma unroll
        for (int i = 0; i < kQK; ++i) qb[i] = -qb[i];
      }
    };
    const int p_wave = p_group + 32 * wave;               // position of the wave's first row
    // Causality per wave: a pair of blocks that starts past the wave's last
    // row is masked for all its rows (an exact no-op), so the wave skips its
    // arithmetic and leaves the matrix core to the other workgroup on its
    // SIMD.  need(pp): pair pp of a head is not all masked for this wave
    // (uniform per wave; false from some pp on).
    const int p_wlast = p_group + min(32 * wave + 31, grows - 1);
    auto need = [&](int pp) { return wave_rows && 2 * kBlockTokens * pp <= p_wlast; };

    float m = kNegInf, l = 0.0f;        // reference maximum (scaled, log2); sum over this lane's tokens
    f16x16 acc[kSl];
  #pragma unroll
    for (int s = 0; s < kSl; ++s)
  #pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][r] = 0.0f;

    // Output rows of head h from the sums, which then restart for the next
    // head.  Rows at a negative position (more queries than cached tokens)
    // are zero.  Lane l holds dims 32s + 8q + 4hf .. +3 (q < 4) of its row;
    // the two lanes of a row swap halves (one permlane32 swap per dword) so
    // that each writes 16 contiguous bytes: of dims 32s + 16p .. +15, the
    // lane with hf = 0 writes the first 8, the other the last 8.  Half as
    // many store instructions and write requests as 8-byte pieces.  A lane
    // without a row stores past the buffer's range (dropped).
    const rsrc_t outr = make_rsrc(a.out, (uint32_t)((size_t)a.num_rows * a.H * D * 2));
    auto finish = [&](int h) {
      auto sw = __builtin_amdgcn_permlane32_swap(as_u32(l), as_u32(l), false, false);
      const float lt = as_f32(sw[0]) + as_f32(sw[1]);
      const float inv = row_ok && p_q >= 0 && lt > 0.0f ? 1.0f / lt : 0.0f;
      const uint32_t ob =
          row_ok ? (uint32_t)((((size_t)qrow * a.H + h) * D + 8 * hf) * 2) : 0xFFFFFFF0u;
  #pragma unroll
      for (int s = 0; s < kSl; ++s)
  #pragma unroll
        for (int p = 0; p < 2; ++p) {
          h4v lo, hi;                                     // dims 32s + 16p + 4hf, + 8
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            lo[r] = (_Float16)(acc[s][8 * p + r] * inv);
            hi[r] = (_Float16)(acc[s][8 * p + 4 + r] * inv);
          }
          typedef uint32_t u2v __attribute__((ext_vector_type(2)));
          const u2v lo2 = __builtin_bit_cast(u2v, lo), hi2 = __builtin_bit_cast(u2v, hi);
          // lanes 32.. take the hf = 0 partner's hi, lanes .. 31 the partner's lo
          auto x0 = __builtin_amdgcn_permlane32_swap(lo2[0], hi2[0], false, false);
          auto x1 = __builtin_amdgcn_permlane32_swap(lo2[1], hi2[1], false, false);
          const u4v o = {x0[0], x1[0], x0[1], x1[1]};
          __builtin_amdgcn_raw_buffer_store_b128(
                o, outr, row_ok ? ob + (uint32_t)((32 * s + 16 * p) * 2) : 0xFFFFFFF0u, 0, 0);
        }
      m = kNegInf;
      l = 0.0f;
  #pragma unroll
      for (int s = 0; s < kSl; ++s)
  #pragma unroll
        for (int r = 0; r < 16; ++r) acc[s][r] = 0.0f;
    };

    // head h0 + hl of block id: pool offset id * block_stride + hl * kTile
    const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)h0 * kTile;
    const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)h0 * kTile;
    const size_t block_stride = (size_t)a.H * kTile;
    // The tile pair is 2 * kTileUnits 16-byte units; the first kLoaders
    // threads load them, unit u = tid + kLoaders * k (K for u < kTileUnits,
    // V after).  kTileUnits and kLoaders are multiples of 64, so the choice
    // of K or V is uniform per wave and the buffer resource stays in scalar
    // registers.
    const bool loader = wave * kWave < kLoaders;        // uniform per wave
    auto unit_is_v = [&](int k) { return wave * kWave + kLoaders * k >= kTileUnits; };
    const uint32_t unit_off = (uint32_t)(tid % kTileUnits) * 16u;
    // Rows source (fused append): a thread holds the same unit of a tile
    // read from the caller's rows as of a pool tile, u_r = 16 g_r + t_r
    // (token t_r, dims 8 g_r .. +7), so both stage into the same LDS slot
    // without bank conflicts; in the rows, 4 lanes of a wave read 64
    // consecutive bytes of each of 16 token rows.  row_r is the row of
    // token t_r of block 0.
    const int u_r = tid % kTileUnits;
    const int t_r = u_r % kBlockTokens;
    const int g_r = u_r / kBlockTokens;
    const int row_r = qs_b - bnd + t_r;
    const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
    const uint32_t rows_total = (uint32_t)a.num_rows * row_bytes;
    // byte offset of token t_r of block 0, head h0 (modulo 2^32: row_r may
    // be negative, the rows of the tokens that exist are not)
    const uint32_t row_base = (uint32_t)row_r * row_bytes + (uint32_t)((h0 * D + 8 * g_r) * 2);
    // Token t_r of block j exists if it lies inside the context; tiles at or
    // past nblk read as zeros.  With query_start inside [0, num_rows] its row
    // is one of the sequence's; the buffer bounds keep any other row inside
    // the caller's rows.
    auto row_off = [&](int j, int hl) {
      return j < nblk && t_r < ctx - kBlockTokens * j
                 ? row_base + (uint32_t)(hl * D * 2) + (uint32_t)j * (uint32_t)kBlockTokens * row_bytes
                 : 0xFFFFFFF0u;
    };
    if (nblk > 0) {
      const int npairs = (nblk + 1) / 2;                  // pairs of blocks per head
      const int nv = nh * npairs;                         // pairs over the item's heads
      // (head, pair) cursors run through the item's pairs in order
      auto advance = [&](int& hl, int& pp) {
        if constexpr (kMulti) {
          if (++pp == npairs) {
            pp = 0;
            ++hl;
          }
        } else {
          ++pp;                                           // one head: past npairs reads zeros
        }
      };
      // V token slots past the context must hold zeros (their weight is 0,
      // and 0 times stale data could be NaN).  Only the last block can be
      // partial: there the lanes of those tokens read past the resource,
      // which returns zeros, so the staging copies every unit as loaded.
      const int v_last = ctx - (nblk - 1) * kBlockTokens;   // valid tokens of the last block
      const uint32_t v_off_last =
          (int)((tid % kTileUnits) % kBlockTokens) < v_last ? unit_off : 0x7FFFFFF0u;
      // Block j of head h0 + hl (hl >= nh: past the item, reads zeros).  o
      // returns the tile's pool offset; with the append its bit 0 is set
      // when the table entry lies outside the pool (offsets are multiples of
      // 16, so bit 0 is free).
      auto fetch = [&](u4v (&r)[kUnits], size_t& o, int j, int hl) {
        const bool live = !kMulti || hl < nh;             // uniform
        const int jj = min(j, nblk - 1);
        const uint32_t bytes = live && j < nblk && loader ? kTile : 0u;
        const int raw = __builtin_amdgcn_readfirstlane(s_ids[jj]);
        o = (size_t)(raw & 0x7fffffff) * block_stride + (size_t)hl * kTile;
        const bool rows = kAppend && j >= jn;             // uniform
        const uint32_t roff = kAppend ? row_off(live ? j : nblk, hl) : 0u;
  #pragma unroll
        for (int k = 0; k < kUnits; ++k) {
          const uint32_t off = unit_is_v(k) && j == nblk - 1 ? v_off_last : unit_off;
          const char* pool = (unit_is_v(k) ? vbase : kbase) + o;
          if constexpr (kAppend) {
            const char* src = rows ? reinterpret_cast<const char*>(unit_is_v(k) ? a.v_new : a.k_new)
                                   : pool;
            r[k] = __builtin_amdgcn_raw_buffer_load_b128(
                make_rsrc(src, rows ? rows_total : bytes), rows ? roff : off, 0, 0);
          } else {
            r[k] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(pool, bytes), off, 0, 0);
          }
        }
        if constexpr (kAppend) o |= (size_t)(raw < 0);
      };
      // Stage block j of head h0 + hl (pool offset o) into pair slot half
      // st.  With the append, a tile read from the rows also goes to its
      // pool block when this item owns the block (its rows hold the block's
      // first token): the store is issued for every tile, with an empty
      // range when the item does not own it, so the ring's wait counts stay
      // fixed.
      auto stage = [&](const u4v (&r)[kUnits], int st, int j, int hl, size_t o) {
        if (!loader) return;                              // uniform per wave
        const int u = tid % kTileUnits;
  #pragma unroll
        for (int k = 0; k < kUnits; ++k)
          s_kv[st][unit_is_v(k) ? kTileUnits + v_slot(u) : u] = r[k];
        if constexpr (kAppend) {
          // a block whose table entry lies outside the pool is not written
          const bool own = j >= jn && hl < nh && j < nblk && !(o & 1) &&
                           (kBlockTokens * j - bnd) / kPrefillRows == kq;
          const size_t ob = o & ~(size_t)1;
          const uint32_t woff = t_r < ctx - kBlockTokens * j ? (uint32_t)u_r * 16u : 0xFFFFFFF0u;
  #pragma unroll
          for (int k = 0; k < kUnits; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(
                r[k], make_rsrc(const_cast<char*>((unit_is_v(k) ? vbase : kbase) + ob),
                                own ? kTile : 0u),
                woff, 0, 0);
        }
      };
      // transpose reads (offsets in halves inside a V tile): lane i = l%16 of
      // its 16-lane group addresses dims 8*g + 4*(i%2) .. +3 of token
      // 4hf + i/4 (lo) and of token 8 + 4hf + i/4 (hi), g = 2*(col/16) +
      // (i%4)/2 (+ 4 per slice of 32 dims), at the swizzled slots
      const int qi = lane % 16;
      const int g0 = 2 * (col / 16) + (qi & 3) / 2;
      const int tr_lo = v_slot(g0 * kBlockTokens + 4 * hf + (qi >> 2)) * 8 + 4 * (qi & 1);
      const int tr_hi = v_slot(g0 * kBlockTokens + 8 + 4 * hf + (qi >> 2)) * 8 + 4 * (qi & 1);
      // this lane's K row: token col of the pair (tile col / 16), dims 16i + 8hf ..
      const int k_unit = hf * kBlockTokens + col % 16;    // + 2i * 16 per MFMA

      // Score products of the pair whose tiles are at blk_a and blk_b:
      // S^T (32 tokens x 32 queries), register r = token 8*(r/4) + 4*hf + r%4.
      auto scores = [&](const u4v* blk_a, const u4v* blk_b) {
        f16x16 sc;
  #pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 0.0f;
        const u4v* kt = col < 16 ? blk_a : blk_b;
        u4v kr[kQK];                                      // A operands: token col of the pair
  #pragma unroll
        for (int i = 0; i < kQK; ++i) kr[i] = kt[k_unit + 2 * i * kBlockTokens];
  #pragma unroll
        for (int i = 0; i < kQK; ++i)
          sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(kr[i]), qb[i], sc, 0, 0, 0);
        return sc;
      };

      // Softmax of pair pp of a head (blocks 2 pp, 2 pp + 1), first part:
      // mask the scores (masked ones become -inf), raise the reference
      // maximum if needed (rescaling the sums), return the reference for the
      // weights.  All the branches of the step are here, so that the rest of
      // the step and the next pair's score products share one basic block.
      auto prep = [&](f16x16& sc, int pp) {
        const int j = 2 * pp;
        const int t0 = j * kBlockTokens;
        // A pair wholly at or before the wave's first row (hence inside the
        // context and visible to every row of the wave) needs no mask.
        const bool full = t0 + 2 * kBlockTokens - 1 <= p_wave;   // uniform per wave
        if (!full) {
          const int va = j < nblk ? min(kBlockTokens, ctx - t0) : 0;
          const int vb = j + 1 < nblk ? min(kBlockTokens, ctx - t0 - kBlockTokens) : 0;
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tk = 8 * (r / 4) + 4 * hf + r % 4;
            const bool live =
                row_ok & (tk % kBlockTokens < (tk < kBlockTokens ? va : vb)) & (t0 + tk <= p_q);
            sc[r] = live ? sc[r] : kNegInf;
          }
        }
        float mx = kNegInf;
  #pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
        auto sw = __builtin_amdgcn_permlane32_swap(as_u32(mx), as_u32(mx), false, false);
        mx = fmaxf(as_f32(sw[0]), as_f32(sw[1]));
        // The reference maximum m moves only when the pair's maximum exceeds it
        // by more than kRescaleSlack, so the weights stay below 2^kRescaleSlack
        // and the accumulators are rescaled rarely.  Both lanes of a row take
        // the same decision.
        const float mxs = mx == kNegInf ? kNegInf : mx * sabs;
        if (mxs > m + kRescaleSlack) {
          const float alpha = __builtin_amdgcn_exp2f(m - mxs);   // m = -inf: 0
  #pragma unroll
          for (int s = 0; s < kSl; ++s) acc[s] = acc[s] * alpha;
          l *= alpha;
          m = mxs;
        }
        return m == kNegInf ? 0.0f : m;
      };

      // Second part: the fp16 weights (exp2(s |scale log2 e| - mref); a
      // masked score gives exp2(-inf) = 0), their running sum, and the value
      // products of the pair whose tiles are at blk_a and blk_b.
      auto weights_pv = [&](const f16x16& sc, float mref, const u4v* blk_a, const u4v* blk_b) {
        h8v pb[2];
  #pragma unroll
        for (int r = 0; r < 16; ++r)
          pb[r / 8][r % 8] = (_Float16)__builtin_amdgcn_exp2f(fmaf(sc[r], sabs, -mref));
        // running sum of the rounded weights, two per instruction
        typedef _Float16 h2v __attribute__((ext_vector_type(2)));
        const h2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  #pragma unroll
        for (int kk = 0; kk < 2; ++kk)
  #pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const h2v two = {pb[kk][e], pb[kk][e + 1]};
            l = __builtin_amdgcn_fdot2(two, ones, l, false);
          }
  #pragma unroll
        for (int s = 0; s < kSl; ++s) {
  #pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            const _Float16* vt = reinterpret_cast<const _Float16*>((kk ? blk_b : blk_a) + kTileUnits);
            const int off = s * 4 * kBlockTokens * 8;       // 4 dim groups per slice
            const s4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s4v*)(vt + off + tr_lo));
            const s4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s4v*)(vt + off + tr_hi));
            const s8v both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8v, both), pb[kk],
                                                            acc[s], 0, 0, 0);
          }
        }
      };

      // Head boundaries inside the pipeline.  With the computed pair at
      // (head ch, pair cp) of the item:
      //  * when cp == 0 and ch > 0, head ch - 1 is complete: its rows are
      //    written and the sums restart, before this pair's softmax;
      //  * the queries of head ch + 1 are loaded into qb right after the
      //    score products of head ch's last pair were issued (one step
      //    before that pair's softmax), so they are in registers by the time
      //    the first pair of head ch + 1 needs them.
      // next_is_last: the pair after (ch, cp) is the last pair of its head.
      auto next_is_last = [&](int cp) { return npairs == 1 || cp + 2 == npairs; };

      // Software pipeline over pairs of blocks.  Pair p lives in LDS pair
      // slot p % 3; its two tiles come through a register ring of four tiles
      // (two pairs), fetched two pairs before they are staged.  Iteration p
      // stages pair p + 1 and refetches its ring tiles for pair p + 3, meets
      // the barrier, takes the branching part of pair p's softmax, then issues
      // the score products of pair p + 1 in one basic block with the weights
      // and value products of pair p, which do not depend on them.
      // The slot staged in iteration p was last read in iteration p - 2, which
      // every wave finished before the barrier of iteration p - 1.  The loop
      // runs whole rounds of two pairs with no exit in its body; a pair past
      // the item's last one is all masked (an exact no-op).
      if constexpr (!kDma) {
      u4v ring[R][kUnits];
      size_t ring_o[R];                                   // pool offsets of the ring's tiles
      int ring_j[R], ring_h[R];                           // (block, head) of the ring's tiles
      int fh = 0, fp = 0;                                 // the pair fetched next
      // ring tile r takes block hb of pair (fh, fp); the pair advances after hb = 1
      auto fetch_tile = [&](int r, int hb) {
        ring_j[r] = 2 * fp + hb;
        ring_h[r] = fh;
        fetch(ring[r], ring_o[r], 2 * fp + hb, fh);
        if (hb) advance(fh, fp);
      };
      auto stage_tile = [&](int r, int st) { stage(ring[r], st, ring_j[r], ring_h[r], ring_o[r]); };
  #pragma unroll
      for (int r = 0; r < R; ++r) fetch_tile(r, r % 2);
      // the queries after the first tiles, whose latency the item's start
      // waits out (the compiler waits for them before the first products)
      load_q(h0);
      sign_q();
      stage_tile(0, 0);
      stage_tile(1, 1);
      fetch_tile(0, 0);
      fetch_tile(1, 1);
      __syncthreads();
      // The two halves of a round alternate the score registers (sc_a holds
      // pair p's scores on entry), so no copy joins them.
      f16x16 sc_a = {}, sc_b = {};
      if (need(0)) sc_a = scores(s_kv[0], s_kv[1]);
      if constexpr (kMulti) {
        if (wave_rows && npairs == 1 && nh > 1) load_q(h0 + 1);
      }
      int ch = 0, cp = 0;                                 // the pair computed now
      int sl = 0;                                         // its pair slot
      auto half = [&](int u, f16x16& cur, f16x16& next) {
        const int sn = sl == kSlots - 1 ? 0 : sl + 1;
        const int ra = (2 * (u + 1)) % R;                 // ring tiles of the pair staged now
        if constexpr (kMulti) {
          if (cp == 0 && ch > 0 && ch < nh && wave_rows) finish(h0 + ch - 1);
        }
        stage_tile(ra, 2 * sn);
        fetch_tile(ra, 0);
        stage_tile(ra + 1, 2 * sn + 1);
        fetch_tile(ra + 1, 1);
        __syncthreads();
        if constexpr (kMulti) {
          if (wave_rows) {                                // uniform per wave
            // a new head starts with the next pair: its first pair is needed
            // even where this head's last pairs are not
            const bool cur_last = cp == npairs - 1;
            const bool head_next = cur_last && ch + 1 < nh;
            const bool need_cur = ch < nh && need(cp);
            float mref = 0.0f;
            if (need_cur) mref = prep(cur, cp);
            if (head_next) sign_q();
            if (need_cur || head_next) next = scores(s_kv[2 * sn], s_kv[2 * sn + 1]);
            if (next_is_last(cp) && (cur_last ? ch + 1 : ch) + 1 < nh)
              load_q(h0 + (cur_last ? ch + 1 : ch) + 1);
            if (need_cur) weights_pv(cur, mref, s_kv[2 * sl], s_kv[2 * sl + 1]);
          }
        } else {
          if (need(cp)) {                                 // uniform per wave
            const float mref = prep(cur, cp);
            next = scores(s_kv[2 * sn], s_kv[2 * sn + 1]);
            weights_pv(cur, mref, s_kv[2 * sl], s_kv[2 * sl + 1]);
          }
        }
        advance(ch, cp);
        sl = sn;
      };
      for (int v = 0; v < nv; v += 2) {
        half(0, sc_a, sc_b);
        half(1, sc_b, sc_a);
      }
      } else {
      // Direct staging.  Pair q goes from HBM (or L2) straight into slot q % 4
      // (buffer_load ... lds: lane l's 16 bytes land at the slot position
      // the wave's base names + 16 l, a load past the buffer range writes
      // zeros).  Iteration i meets the barrier once this wave's copies of
      // pair i + 1 are complete (those of pair i + 2 stay in flight), so
      // after it every wave's are, and every wave has finished iteration
      // i - 1: slot (i + 3) % 4, last read there, takes pair i + 3, two
      // iterations ahead of its use.  The loop runs whole rounds of four
      // pairs, so each slot is a fixed array in the unrolled body.  (The
      // barrier is written out: __syncthreads would also wait for the copies
      // still in flight.)  Each wave meets exactly one barrier per iteration.
      //
      // Over several heads, the copies of a step are issued after its score
      // products and after the next head's query loads (when that step
      // issues them), and the step ends waiting for all but its own copies
      // (what the next barrier waits for anyway): so the query loads are
      // complete by the next step, and the compiler, which cannot tell the
      // steps that issue them, places no wait for them in the others.
      int fh = 0, fp = 0;                                 // the pair copied next
      auto dma = [&](u4v (*slot)[2 * kTileUnits]) {
        const bool live = !kMulti || fh < nh;             // uniform
        // both ids of the pair in one LDS read (a pair past the end reads the
        // last one again; the spare entry after the blocks holds pool block 0,
        // and copies past the blocks have an empty range)
        const int j0 = 2 * min(fp, (nblk - 1) / 2);
        const int ids[2] = {s_ids[j0], s_ids[j0 + 1]};
  #pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int j = 2 * fp + hb;
          const uint32_t bytes = live && j < nblk ? kTile : 0u;
          const int id = __builtin_amdgcn_readfirstlane(ids[hb]);
          const size_t o = (size_t)id * block_stride + (size_t)fh * kTile;
  #pragma unroll
          for (int k = 0; k < kUnits; ++k) {
            // this wave's 64 consecutive slot positions of copy k: K units
            // p0 .. p0+63, or V positions p0 .. p0+63, which hold V units
            // v_slot(p0 + lane) (the swizzle is its own inverse)
            const int wbase = wave * kWave + kLoaders * k;   // uniform
            const bool isv = wbase >= kTileUnits;             // uniform
            const int p0 = isv ? wbase - kTileUnits : wbase;
            const int src = isv ? v_slot(p0 + lane) : p0 + lane;
            // V tokens past the context of the last block load as zeros
            const bool zero = isv && j == nblk - 1 && src % kBlockTokens >= v_last;
            const uint32_t off = zero ? 0x7FFFFFF0u : (uint32_t)src * 16u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                make_rsrc((isv ? vbase : kbase) + o, bytes),
                (__attribute__((address_space(3))) void*)&slot[hb][(isv ? kTileUnits : 0) + p0],
                16, off, 0, 0, 0);
          }
        }
        advance(fh, fp);
      };
      static_assert(2 * kUnits == 4 || 2 * kUnits == 2, "copies per pair");
      dma(s_d0);
      dma(s_d1);
      dma(s_d2);
      // the queries after the first copies (issued first, the copies would
      // queue behind them); the wait below covers both
      load_q(h0);
      load_item(item + gridDim.x);                        // the next item's, while these land
      sign_q();
      // The first three pairs complete (issued together, they land close
      // together; the compiler would place this wait before the first LDS
      // read on its own, since it does not tell the copies issued here
      // apart).
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      asm volatile("s_barrier" ::: "memory");
      f16x16 sc_a = {}, sc_b = {};
      if (need(0)) sc_a = scores(s_d0[0], s_d0[1]);
      if constexpr (kMulti) {
        // one pair per head: the next head's queries now
        if (wave_rows && npairs == 1 && nh > 1) {
          load_q(h0 + 1);
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
      }
      int ch = 0, cp = 0;                                 // the pair computed now
      auto quarter = [&](u4v (*cur_slot)[2 * kTileUnits], u4v (*next_slot)[2 * kTileUnits],
                         u4v (*free_slot)[2 * kTileUnits], f16x16& cur, f16x16& next) {
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * kUnits) : "memory");
        if constexpr (!kMulti) {
          dma(free_slot);
          if (need(cp)) {                                 // uniform per wave
            const float mref = prep(cur, cp);
            next = scores(next_slot[0], next_slot[1]);
            weights_pv(cur, mref, cur_slot[0], cur_slot[1]);
          }
        } else {
          if (cp == 0 && ch > 0 && wave_rows) finish(h0 + ch - 1);
          const bool cur_last = cp == npairs - 1;
          const bool head_next = cur_last && ch + 1 < nh;
          const bool need_cur = need(cp);
          const bool qnew = wave_rows && next_is_last(cp) && (cur_last ? ch + 1 : ch) + 1 < nh;
          float mref = 0.0f;
          if (wave_rows) {                                // uniform per wave
            if (need_cur) mref = prep(cur, cp);
            if (head_next) sign_q();
            if (need_cur || head_next) next = scores(next_slot[0], next_slot[1]);
            if (qnew) load_q(h0 + (cur_last ? ch + 1 : ch) + 1);
          }
          dma(free_slot);
          if (need_cur) weights_pv(cur, mref, cur_slot[0], cur_slot[1]);
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kUnits));
        }
        advance(ch, cp);
      };
      // (uniform exits after the last pair: the copies still in flight for
      // pairs past the end write zeros and are waited for at the item's
      // closing barrier)
      for (int v = 0; v < nv; v += 4) {
        quarter(s_d0, s_d1, s_d3, sc_a, sc_b);
        if (v + 1 >= nv) break;
        quarter(s_d1, s_d2, s_d0, sc_b, sc_a);
        if (v + 2 >= nv) break;
        quarter(s_d2, s_d3, s_d1, sc_a, sc_b);
        if (v + 3 >= nv) break;
        quarter(s_d3, s_d0, s_d2, sc_b, sc_a);
      }
      }
      finish(h0 + nh - 1);
    } else {
      // no token to attend: every head's rows are zero
      if constexpr (kDma) {
        load_item(item + gridDim.x);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      }
      for (int hl = 0; hl < nh; ++hl) finish(h0 + hl);
    }

    __syncthreads();                                    // LDS staging is reused by the next item
  }
}

// Fused append, first part: the new tokens that share a block with cached
// tokens (from the sequence's first new position up to the next block
// boundary) are written to the pools here, before the prefill kernel reads
// that block from the pools.  One workgroup per sequence; a sequence whose
// new tokens start on a block boundary (a prompt, a block-aligned chunk)
// has nothing to do.
template <int D>
__global__ __launch_bounds__(256) void prefill_boundary_append_kernel(PrefillArgs a) {
  constexpr int G = D / 8;                                // 16-byte units per head row
  const int b = blockIdx.x;
  const int n = rows_of(a, b);
  const int ctx = clampi(a.context_lens[b], 0, a.ctx_limit);
  const int bnd = ctx - n;                                // first new position
  if (n == 0 || bnd <= 0 || bnd % kBlockTokens == 0) return;
  const int cnt = min(kBlockTokens - bnd % kBlockTokens, n);
  const int id = a.block_tables[(size_t)b * a.max_blocks + bnd / kBlockTokens];
  if ((unsigned)id >= (unsigned)a.num_blocks) return;   // outside the pool: nothing written
  const int units = cnt * a.H * G;
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int g = u % G;
    const int hh = (u / G) % a.H;
    const int i = u / (G * a.H);
    const int row = a.query_start[b] + i;
    if (row < 0 || row >= a.num_rows) continue;
    const int t = (bnd + i) % kBlockTokens;
    const size_t src = ((size_t)row * a.H + hh) * D + 8 * g;
    const size_t dst = ((((size_t)id * a.H + hh) * G + g) * kBlockTokens + t) * 8;
    *reinterpret_cast<u4v*>(static_cast<_Float16*>(const_cast<void*>(a.k_pool)) + dst) =
        *reinterpret_cast<const u4v*>(a.k_new + src);
    *reinterpret_cast<u4v*>(static_cast<_Float16*>(const_cast<void*>(a.v_pool)) + dst) =
        *reinterpret_cast<const u4v*>(a.v_new + src);
  }
}

}  // namespace

size_t prefill_lds_bytes(int B, int max_blocks_used) {
  return (size_t)(((B + 2) & ~1) + max_blocks_used + 1) * sizeof(int);
}

namespace {

template <bool kAppend>
void launch_prefill_kernel(const PrefillArgs& a, int D, int grid, size_t lds, hipStream_t stream) {
  const int threads = kWave * kPrefillWaves;
  const bool multi = a.heads_per_item > 1;
  if (D == 128) {
    if (multi)
      hipLaunchKernelGGL((pa_prefill_kernel<128, kAppend, true>), dim3(grid), dim3(threads), lds,
                         stream, a);
    else
      hipLaunchKernelGGL((pa_prefill_kernel<128, kAppend, false>), dim3(grid), dim3(threads), lds,
                         stream, a);
  } else {
    if (multi)
      hipLaunchKernelGGL((pa_prefill_kernel<64, kAppend, true>), dim3(grid), dim3(threads), lds,
                         stream, a);
    else
      hipLaunchKernelGGL((pa_prefill_kernel<64, kAppend, false>), dim3(grid), dim3(threads), lds,
                         stream, a);
  }
}

}  // namespace

hipError_t launch_pa_prefill(const PrefillArgs& a, int D, int grid, int max_blocks_used,
                             hipStream_t stream) {
  launch_prefill_kernel<false>(a, D, grid, prefill_lds_bytes(a.B, max_blocks_used), stream);
  return hipGetLastError();
}

hipError_t launch_pa_prefill_append(const PrefillArgs& a, int D, int grid, int max_blocks_used,
                                    hipStream_t stream) {
  if (D == 128)
    hipLaunchKernelGGL((prefill_boundary_append_kernel<128>), dim3(a.B), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_boundary_append_kernel<64>), dim3(a.B), dim3(256), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_prefill_kernel<true>(a, D, grid, prefill_lds_bytes(a.B, max_blocks_used), stream);
  return hipGetLastError();
}

}  // namespace pkv
