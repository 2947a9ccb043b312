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
// together (16 bytes each) through a register ring of four tiles and stored
// into one of three LDS pair slots (V slots past the context zeroed, V
// token slots swizzled against bank conflicts); after every second tile a
// barrier, then each wave consumes the pair (32 tokens), its score products
// issued one pair ahead of its softmax, on the
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
// workgroup with.  Workgroups take (query group, head) items in a
// grid-stride loop; item i serves head i % H, and with a grid that is a
// multiple of 8 it runs on XCD i % 8 (one XCD per head when H is a multiple
// of 8).  Within a sequence the groups that reach furthest come first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "pa_common.h"
#include "pa_mfma.h"

namespace pkv {
namespace {

using namespace dev;

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

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

__device__ __forceinline__ int seq_of_group(const int* s_group, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_group[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
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
template <int D, bool kAppend>
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
  extern __shared__ int smem[];
  __shared__ int s_wave[kPrefillWaves];
  __shared__ u4v s_kv[2 * kSlots][2 * kTileUnits];     // tile stage: K tile, then V tile
  int* s_group = smem;                                  // B + 1
  int* s_ids = smem + a.B + 1;                          // block ids of the sequence

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int col = lane % 32;                            // query column of this lane
  const int hf = lane / 32;                             // k-slot half of this lane

  group_prefix(a, s_group, s_wave);
  // Items (query group, head), longest-reaching groups first, in a
  // grid-stride loop: the prefix above is computed once per workgroup for
  // its few items, and no workgroup is launched only to find none.
  const int items = s_group[a.B] * a.H;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int gt = item / a.H;
    const int h = item % a.H;
    const int b = seq_of_group(s_group, a.B, gt);
    const int n = rows_of(a, b);
    const int kq = groups_of(a, b) - 1 - (gt - s_group[b]);   // furthest-reaching group first
    const int ctx = clampi(a.context_lens[b], 0, a.ctx_limit);
    const int row0 = kPrefillRows * kq;
    const int grows = min(kPrefillRows, n - row0);
    const int p_group = ctx - n + row0;                   // position of the group's first row
    const int p_last = min(p_group + grows - 1, ctx - 1);
    const int nblk = p_last >= 0 ? p_last / kBlockTokens + 1 : 0;
    // fused append: position of the sequence's first new token, and the
    // first block whose tokens are all new
    const int bnd = ctx - n;
    const int jn = kAppend ? (max(bnd, 0) + kBlockTokens - 1) / kBlockTokens : 0x7fffffff;

    for (int j = tid; j < nblk; j += blockDim.x) {
      const int id = a.block_tables[(size_t)b * a.max_blocks + j];
      s_ids[j] = clampi(id, 0, a.num_blocks - 1);
    }
    __syncthreads();

    // this lane's query row: wave w serves rows row0 + 32w ..; a wave with no
    // row skips the arithmetic (it still loads, stages and meets the barriers)
    const bool wave_rows = 32 * wave < grows;
    const int wrow = 32 * wave + col;
    const int qrow = a.query_start[b] + row0 + wrow;
    const bool row_ok = wrow < grows && qrow >= 0 && qrow < a.num_rows;
    const int p_q = p_group + wrow;
    const rsrc_t qr = make_rsrc(a.q, (uint32_t)((size_t)a.num_rows * a.H * D * 2));
    const uint32_t qoff = row_ok ? (uint32_t)((((size_t)qrow * a.H + h) * D + 8 * hf) * 2)
                                 : 0xFFFFFFF0u;           // past the resource: reads 0
    h8v qb[kQK];                                          // B operands: dims 16i + 8hf ..
  #pragma unroll
    for (int i = 0; i < kQK; ++i)
      qb[i] = as_h8(__builtin_amdgcn_raw_buffer_load_b128(qr, qoff + (row_ok ? i * 32 : 0), 0, 0));
    // keep the query loads ahead of the ring's first tiles (every step reads them)
    __builtin_amdgcn_sched_barrier(0);
    // The scores are taken as (sign(scale) q) . k (an exact negation), so that
    // their maximum is the maximum of the scaled scores; weights are then
    // exp2(s * |scale log2 e| - m) with one fused multiply-add.
    // (a zero scale is taken as the smallest normal float: the weights are
    // then exactly 1, and a masked score's -inf times it stays -inf)
    const float sabs = fmaxf(fabsf(a.scale_log2), 1.17549435e-38f);
    if (a.scale_log2 < 0.0f) {
  #pragma unroll
      for (int i = 0; i < kQK; ++i) qb[i] = -qb[i];
    }
    const int p_wave = p_group + 32 * wave;               // position of the wave's first row

    float m = kNegInf, l = 0.0f;        // reference maximum (scaled, log2); sum over this lane's tokens
    f16x16 acc[kSl];
  #pragma unroll
    for (int s = 0; s < kSl; ++s)
  #pragma unroll
      for (int r = 0; r < 16; ++r) acc[s][r] = 0.0f;

    const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)h * kTile;
    const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)h * kTile;
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
    const int row_r = a.query_start[b] - bnd + t_r;
    const uint32_t row_bytes = (uint32_t)(a.H * D * 2);
    const uint32_t rows_total = (uint32_t)a.num_rows * row_bytes;
    // byte offset of token t_r of block 0 (modulo 2^32: row_r may be
    // negative, the rows of the tokens that exist are not)
    const uint32_t row_base = (uint32_t)row_r * row_bytes + (uint32_t)((h * D + 8 * g_r) * 2);
    // Token t_r of block j exists if it lies inside the context; tiles at or
    // past nblk read as zeros.  With query_start inside [0, num_rows] its row
    // is one of the sequence's; the buffer bounds keep any other row inside
    // the caller's rows.
    auto row_off = [&](int j) {
      return j < nblk && t_r < ctx - kBlockTokens * j
                 ? row_base + (uint32_t)j * (uint32_t)kBlockTokens * row_bytes
                 : 0xFFFFFFF0u;
    };
    if (nblk > 0) {
      // V token slots past the context must hold zeros (their weight is 0,
      // and 0 times stale data could be NaN).  Only the last block can be
      // partial: there the lanes of those tokens read past the resource,
      // which returns zeros, so the staging copies every unit as loaded.
      const int v_last = ctx - (nblk - 1) * kBlockTokens;   // valid tokens of the last block
      const uint32_t v_off_last =
          (int)((tid % kTileUnits) % kBlockTokens) < v_last ? unit_off : 0x7FFFFFF0u;
      auto fetch = [&](u4v (&r)[kUnits], size_t& o, int j) {
        const int jj = min(j, nblk - 1);
        const uint32_t bytes = j < nblk && loader ? kTile : 0u;
        o = (size_t)__builtin_amdgcn_readfirstlane(s_ids[jj]) * block_stride;
        const bool rows = kAppend && j >= jn;             // uniform
        const uint32_t roff = kAppend ? row_off(j) : 0u;
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
      };
      // Stage block j's tiles (pool offset o) into pair slot half st.  With
      // the append, a tile read from the rows also goes to its pool
      // block when this item owns the block (its rows hold the block's first
      // token): the store is issued for every tile, with an empty range when
      // the item does not own it, so the ring's wait counts stay fixed.
      auto stage = [&](const u4v (&r)[kUnits], int st, int j, size_t o) {
        if (!loader) return;                              // uniform per wave
        const int u = tid % kTileUnits;
        const bool rows = kAppend && j >= jn;             // uniform
  #pragma unroll
        for (int k = 0; k < kUnits; ++k)
          s_kv[st][unit_is_v(k) ? kTileUnits + v_slot(u) : u] = r[k];
        if constexpr (kAppend) {
          const bool own = rows && j < nblk && (kBlockTokens * j - bnd) / kPrefillRows == kq;
          const uint32_t woff = t_r < ctx - kBlockTokens * j ? (uint32_t)u_r * 16u : 0xFFFFFFF0u;
  #pragma unroll
          for (int k = 0; k < kUnits; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(
                r[k], make_rsrc(const_cast<char*>((unit_is_v(k) ? vbase : kbase) + o),
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

      // Score products of the pair in pair slot sl (tiles 2 sl, 2 sl + 1):
      // S^T (32 tokens x 32 queries), register r = token 8*(r/4) + 4*hf + r%4.
      auto scores = [&](int sl) {
        f16x16 sc;
  #pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = 0.0f;
        const u4v* kt = s_kv[2 * sl + col / 16];
        u4v kr[kQK];                                      // A operands: token col of the pair
  #pragma unroll
        for (int i = 0; i < kQK; ++i) kr[i] = kt[k_unit + 2 * i * kBlockTokens];
  #pragma unroll
        for (int i = 0; i < kQK; ++i)
          sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(kr[i]), qb[i], sc, 0, 0, 0);
        return sc;
      };

      // Softmax of pair pp (blocks 2 pp, 2 pp + 1), first part: mask the
      // scores (masked ones become -inf), raise the reference maximum if
      // needed (rescaling the sums), return the reference for the weights.
      // All the branches of the step are here, so that the rest of the step
      // and the next pair's score products share one basic block.
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
      // products of the pair in pair slot sl.
      auto weights_pv = [&](const f16x16& sc, float mref, int sl) {
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
            const _Float16* vt = reinterpret_cast<const _Float16*>(&s_kv[2 * sl + kk][kTileUnits]);
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

      // Software pipeline over pairs of blocks.  Pair p lives in LDS pair
      // slot p % 3; its two tiles come through a register ring of four tiles
      // (two pairs), fetched two pairs before they are staged.  Iteration p
      // stages pair p + 1 and refetches its ring tiles for pair p + 3, meets
      // the barrier, takes the branching part of pair p's softmax, then issues
      // the score products of pair p + 1 in one basic block with the weights
      // and value products of pair p, which do not depend on them.
      // The slot staged in iteration p was last read in iteration p - 2, which
      // every wave finished before the barrier of iteration p - 1.  Pairs past
      // the last block see valid = 0 (exact no-ops), so the loop runs whole
      // rounds of two pairs with no exit in its body.
      u4v ring[R][kUnits];
      size_t ring_o[R];                                   // pool offsets of the ring's blocks
  #pragma unroll
      for (int r = 0; r < R; ++r) fetch(ring[r], ring_o[r], r);
      stage(ring[0], 0, 0, ring_o[0]);
      stage(ring[1], 1, 1, ring_o[1]);
      fetch(ring[0], ring_o[0], 4);
      fetch(ring[1], ring_o[1], 5);
      __syncthreads();
      // The two halves of a round alternate the score registers (sc_a holds
      // pair p's scores on entry), so no copy joins them.
      f16x16 sc_a = {}, sc_b = {};
      if (wave_rows) sc_a = scores(0);
      const int npairs = (nblk + 1) / 2;
      int sl = 0;                                         // pair slot of pair p
      auto half = [&](int p, int u, f16x16& cur, f16x16& next) {
        const int pn = p + u + 1;                         // the pair staged now
        const int sn = sl == kSlots - 1 ? 0 : sl + 1;
        const int ra = (2 * (u + 1)) % R;                 // its ring tiles
        stage(ring[ra], 2 * sn, 2 * pn, ring_o[ra]);
        fetch(ring[ra], ring_o[ra], 2 * pn + R);
        stage(ring[ra + 1], 2 * sn + 1, 2 * pn + 1, ring_o[ra + 1]);
        fetch(ring[ra + 1], ring_o[ra + 1], 2 * pn + 1 + R);
        __syncthreads();
        if (wave_rows) {                                  // uniform per wave
          const float mref = prep(cur, p + u);
          next = scores(sn);
          weights_pv(cur, mref, sl);
        }
        sl = sn;
      };
      for (int p = 0; p < npairs; p += 2) {
        half(p, 0, sc_a, sc_b);
        half(p, 1, sc_b, sc_a);
      }

    }

    // rows at a negative position (more queries than cached tokens) are zero;
    // lane l holds dims 32s + 8q + 4hf .. +3 (q < 4) of its row
    auto sw = __builtin_amdgcn_permlane32_swap(as_u32(l), as_u32(l), false, false);
    l = as_f32(sw[0]) + as_f32(sw[1]);
    if (row_ok) {
      const float inv = p_q >= 0 && l > 0.0f ? 1.0f / l : 0.0f;
      _Float16* orow = a.out + ((size_t)qrow * a.H + h) * D + 4 * hf;
  #pragma unroll
      for (int s = 0; s < kSl; ++s)
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          h4v o;
  #pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = (_Float16)(acc[s][4 * q + r] * inv);
          *reinterpret_cast<h4v*>(orow + 32 * s + 8 * q) = o;
        }
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
  const int id = clampi(a.block_tables[(size_t)b * a.max_blocks + bnd / kBlockTokens], 0,
                        a.num_blocks - 1);
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
  return (size_t)(B + 1 + max_blocks_used) * sizeof(int);
}

hipError_t launch_pa_prefill(const PrefillArgs& a, int D, int grid, int max_blocks_used,
                             hipStream_t stream) {
  const size_t lds = prefill_lds_bytes(a.B, max_blocks_used);
  const int threads = kWave * kPrefillWaves;
  if (D == 128)
    hipLaunchKernelGGL((pa_prefill_kernel<128, false>), dim3(grid), dim3(threads), lds, stream, a);
  else
    hipLaunchKernelGGL((pa_prefill_kernel<64, false>), dim3(grid), dim3(threads), lds, stream, a);
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
  const size_t lds = prefill_lds_bytes(a.B, max_blocks_used);
  const int threads = kWave * kPrefillWaves;
  if (D == 128)
    hipLaunchKernelGGL((pa_prefill_kernel<128, true>), dim3(grid), dim3(threads), lds, stream, a);
  else
    hipLaunchKernelGGL((pa_prefill_kernel<64, true>), dim3(grid), dim3(threads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
