// PagedAttention decode for gfx950 (MI355X): the flat strategy (default).
//
// Same result as the partitioned strategy ("PagedAttention", e-fortepiano.pl,
// "Formulació matemàtica": attention computed block by block), organised for
// a steady stream of loads:
//
//  * For one head, line up every block of every sequence, sequence after
//    sequence: positions 0 .. T-1, with sequence b owning [S_b, S_{b+1}).
//  * The grid is sized to what the GPU holds at once.  Each workgroup serves
//    one head group and one of NR equal, contiguous ranges of positions.
//    Workgroup i runs on XCD i % 8.  When blocks are shared between
//    sequences (the normal cache policy), workgroup i serves head group
//    i % G and range i / G, so a head group stays on one XCD (with G == 8)
//    and its shared blocks are found in that XCD's L2.  When tiles stream
//    (non-temporal), each XCD serves every head group and every eighth
//    range, which spreads each XCD's reads over the whole pool (1% faster
//    at batch 200).  Every wave of the workgroup (one per head) streams
//    through the whole range: no wave starts over at a partition boundary,
//    and the ranges differ in length by at most one block.
//  * A wave keeps a ring of kFlatTiles tiles in registers: while it works
//    on one block the next ones are in flight.  The prefetch runs straight
//    across sequence boundaries.
//  * At each sequence boundary inside the range the running (m, l, acc) is
//    closed: a sequence wholly inside the range is written as the final
//    output; a sequence cut by the range's start or end leaves a partial
//    result, at most two per wave ("head piece" = the range's first
//    sequence begun earlier, "tail piece" = its last sequence going on
//    later).  A second kernel merges the pieces of each cut sequence in
//    ascending position order and writes zero rows for empty sequences; the
//    sequence offsets it needs are published by workgroup 0.
//
// Block ids of the workgroup's range are staged once in LDS (one gather for
// all its waves), each with its count of tokens in use; the per-sequence
// block offsets come from a prefix sum of the context lengths, computed in
// LDS by every workgroup.  The ring's loads past the end of the range
// address a zero-size buffer resource, so they fetch nothing.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "pa_common.h"

namespace pkv {
namespace {

using namespace dev;

__device__ __forceinline__ int clamp_ctx(int ctx, int limit) { return min(max(ctx, 0), limit); }


// s_start[b] = blocks of the sequences before b (b <= B; s_start[B] = T);
// s_tail[b] (if given) = tokens used in sequence b's last block.  All
// threads of the workgroup take part; ends with a barrier.
__device__ __forceinline__ int seq_ctx(const int32_t* ctx_lens, const int32_t* capacity, int b,
                                       int ctx_limit) {
  const int ctx = clamp_ctx(ctx_lens[b], ctx_limit);
  return capacity ? min(ctx, max(capacity[b], 0)) : ctx;
}

__device__ void block_prefix(const int32_t* ctx_lens, const int32_t* capacity, int B,
                             int ctx_limit, int* s_start, int* s_tail, int* s_wave) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int per = (B + nt - 1) / nt;
  const int lo = min(B, tid * per);
  const int hi = min(B, lo + per);
  int own = 0;
  for (int b = lo; b < hi; ++b)
    own += (seq_ctx(ctx_lens, capacity, b, ctx_limit) + kBlockTokens - 1) / kBlockTokens;
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
    const int ctx = seq_ctx(ctx_lens, capacity, b, ctx_limit);
    const int nb = (ctx + kBlockTokens - 1) / kBlockTokens;
    s_start[b] = run;
    if (s_tail) s_tail[b] = ctx - (nb - 1) * kBlockTokens;
    run += nb;
  }
  if (tid == nt - 1) s_start[B] = run;
  __syncthreads();
}

// The sequence holding position s (0 <= s < T): the largest b with
// s_start[b] <= s, which skips empty sequences.
__device__ __forceinline__ int seq_of(const int* s_start, int B, int s) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_start[mid] <= s) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// One dword of the query row (b, h) per lane; lanes past the row read 0.
template <int D>
__device__ __forceinline__ uint32_t load_q_dword(const _Float16* q, size_t row,
                                                 uint32_t lane_off4) {
  return __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(q + row * D, D * 2), lane_off4, 0, 0);
}

// Spread a row held one dword per lane into this lane's groups 4*i + row
// (16 bytes each), through the wave's own 256-byte LDS slot.  The wave's LDS
// operations run in order, so no barrier is needed; the wavefront-scope
// fences (no instruction) tell the compiler that lanes read what other lanes
// wrote, so it neither moves the reads past the writes nor reuses a lane's
// earlier read of the slot (lanes at or past D/2 write nothing).
template <int D>
__device__ __forceinline__ void distribute_q(u4v (&q)[Geometry<D>::kLoads], uint32_t qn, int row,
                                             int lane, uint32_t* slot) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  if (lane < D / 2) slot[lane] = qn;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const u4v* rows = reinterpret_cast<const u4v*>(slot);
#pragma unroll
  for (int i = 0; i < Geometry<D>::kLoads; ++i) q[i] = rows[4 * i + row];
}

// This lane's kOut output values (consecutive dims) as fp16 / fp32.
template <int kOut>
__device__ __forceinline__ void store_out(rsrc_t r, uint32_t off, const float (&val)[kOut],
                                          float inv) {
  if constexpr (kOut == 2) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 v = {(_Float16)(val[0] * inv), (_Float16)(val[1] * inv)};
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
  } else {
    const _Float16 v = (_Float16)(val[0] * inv);
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, v), r, off, 0, 0);
  }
}
template <int kOut>
__device__ __forceinline__ void store_acc(rsrc_t r, uint32_t off, const float (&val)[kOut]) {
  if constexpr (kOut == 2) {
    typedef uint32_t u2v __attribute__((ext_vector_type(2)));
    const u2v v = {as_u32(val[0]), as_u32(val[1])};
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(as_u32(val[0]), r, off, 0, 0);
  }
}

template <int D, int kPolicy, bool kContig, bool kAppend>
__global__ __launch_bounds__(64 * kFlatMaxWaves) void pa_decode_flat_kernel(FlatArgs a) {
  static_assert(!(kContig && kAppend), "the append is for the block pool");
  constexpr int kAcc = Geometry<D>::kAcc;
  constexpr int kTile = Geometry<D>::kTileBytes;
  constexpr int kOut = Geometry<D>::kOutPerLane;
  extern __shared__ int smem[];
  __shared__ int s_wave[kFlatMaxWaves];
  __shared__ uint32_t s_q[kFlatMaxWaves][kWave];   // per-wave query staging
  int* s_start = smem;                 // B + 1
  int* s_tail = smem + a.B + 1;        // B
  int* s_ids = smem + 2 * a.B + 1;     // max_chunk block ids

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int token = lane % kBlockTokens;
  const int row = lane / kBlockTokens;
  // workgroup -> (head group g, range r); both mappings are one-to-one
  // over the grid (head_groups * nr workgroups)
  const bool spread = kPolicy == kStreamPolicy && a.nr % 8 == 0;
  const int g = spread ? (blockIdx.x / 8) % a.head_groups : blockIdx.x % a.head_groups;
  const int r = spread ? (blockIdx.x / 8 / a.head_groups) * 8 + blockIdx.x % 8
                       : blockIdx.x / a.head_groups;
  const int h = g * a.waves_per_group + wave;

  block_prefix(a.context_lens, kContig ? a.capacity : nullptr, a.B, a.ctx_limit, s_start, s_tail,
               s_wave);
  if (blockIdx.x == 0) {               // offsets for the merge kernel
    for (int i = tid; i <= a.B; i += blockDim.x) a.ws_seq[i] = s_start[i];
  }
  const int T = s_start[a.B];
  const int chunk = (T + a.nr - 1) / a.nr;
  const int c0 = min(T, r * chunk);
  const int c1 = min(T, c0 + chunk);
  if (c0 >= c1) return;                // uniform for the workgroup

  // Physical block id of every position of the range.
  // Physical block id of every position of the range; in the contiguous
  // layout, the index of the sequence's 16-row group instead.
  for (int s = c0 + tid; s < c1; s += blockDim.x) {
    const int b = seq_of(s_start, a.B, s);
    if (kContig) {
      s_ids[s - c0] = b * (a.row_tokens / kBlockTokens) + (s - s_start[b]);
    } else {
      const int id = a.block_tables[(size_t)b * a.max_blocks + (s - s_start[b])];
      s_ids[s - c0] = min(max(id, 0), a.num_blocks - 1);
    }
  }
  __syncthreads();

  // Paged: tile (block, h) at (block * H + h) * kTile, lane l at l * 16.
  // Contiguous: row r at r * H * D * 2, head h at h * D * 2, lane l at its
  // token's row plus its 16-byte dim group; a tile spans 16 rows.
  const size_t row_bytes = (size_t)a.H * D * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)h * (kContig ? D * 2 : kTile);
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)h * (kContig ? D * 2 : kTile);
  const size_t block_stride = kContig ? kBlockTokens * row_bytes : (size_t)a.H * kTile;
  const uint32_t lane_off = kContig ? (uint32_t)(token * row_bytes) + row * 16u : lane * 16u;
  const uint32_t tile_span = kContig ? (uint32_t)((kBlockTokens - 1) * row_bytes + D * 2) : kTile;
  // Past the range's end the load ring still issues its loads (so the load
  // counters stay exact) but through a zero-size resource: they return 0
  // without touching memory.
  auto fetch = [&](Tile<D>& t, int s) {
    const int j = min(s, c1 - 1) - c0;
    const uint32_t bytes = s < c1 ? tile_span : 0u;
    const size_t o = (size_t)__builtin_amdgcn_readfirstlane(s_ids[j]) * block_stride;
    load_tile<D, kPolicy, kContig ? 64 : 1024>(t, make_rsrc(kbase + o, bytes),
                                                make_rsrc(vbase + o, bytes), lane_off);
  };

  // Current segment: sequence b, positions [seg_lo, seg_hi) of its
  // [seq_lo, seq_hi).  All wave-uniform.
  int b = seq_of(s_start, a.B, c0);
  int seq_lo = s_start[b];
  int seq_hi = s_start[b + 1];
  int seg_lo = c0;
  int seg_hi = min(c1, seq_hi);
  int tail = s_tail[b];

  const uint32_t lane_off4 = lane * 4u;
  u4v q[Geometry<D>::kLoads];
  distribute_q<D>(q, load_q_dword<D>(a.q, (size_t)b * a.H + h, lane_off4), row, lane,
                  s_q[wave]);
  int b_next = b;
  uint32_t qn = 0;
  if (seg_hi < c1) {                   // the next segment's query, one segment ahead
    b_next = seq_of(s_start, a.B, seg_hi);
    qn = load_q_dword<D>(a.q, (size_t)b_next * a.H + h, lane_off4);
  }
  // Per-lane byte offsets of this lane's output values (fixed for the wave;
  // see reduce_rows), and of the (m, l) pair written by lane 0.
  const int d0 = (4 * ((token * kOut) / 8) + row) * 8 + (token * kOut) % 8;
  const uint32_t out_off = d0 * 2u;
  const uint32_t acc_off = d0 * 4u;

  // With the append: the new token of the current segment's sequence (its
  // last position, token tail - 1 of its last block), one dword per lane
  // like the query, loaded when the segment opens if the segment ends the
  // sequence.  At the last block it replaces the tile's slot in registers;
  // the merge kernel writes it to the pools after this kernel.
  uint32_t knew = 0, vnew = 0;
  auto load_new = [&]() {
    if constexpr (kAppend) {
      const uint32_t bytes = seg_hi == seq_hi ? D * 2u : 0u;
      const size_t nrow = ((size_t)b * a.H + h) * D;
      knew = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.k_new + nrow, bytes), lane_off4, 0, 0);
      vnew = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.v_new + nrow, bytes), lane_off4, 0, 0);
    }
  };
  load_new();

  float m = kNegInf, l = 0.0f;
  float acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = 0.0f;

  auto step = [&](Tile<D>& t, int s) {
    if constexpr (kAppend) {
      if (s == seq_hi - 1) {           // uniform: the sequence's last block
        // the new rows in the tile's lane layout (load i of lane l: dims
        // 8 * (l / 16 + 4 i) .. +7), through the wave's query slot
        u4v kn[Geometry<D>::kLoads], vn[Geometry<D>::kLoads];
        distribute_q<D>(kn, knew, row, lane, s_q[wave]);
        distribute_q<D>(vn, vnew, row, lane, s_q[wave]);
        const bool mine = token == tail - 1;
#pragma unroll
        for (int i = 0; i < Geometry<D>::kLoads; ++i) {
          t.k[i] = mine ? kn[i] : t.k[i];
          t.v[i] = mine ? vn[i] : t.v[i];
        }
      }
    }
    // one code path for every block: only a sequence's last block can be
    // partially filled, the others pass valid = 16
    consume<D, true>(t, q, a.scale_log2, token, s == seq_hi - 1 ? tail : kBlockTokens, m, l, acc);
    if (s != seg_hi - 1) return;
    // close the segment
    float val[kOut];
    reduce_rows<D>(l, acc, token, row, val);
    if (seg_lo == seq_lo && seg_hi == seq_hi) {
      const rsrc_t orow = make_rsrc(a.out + ((size_t)b * a.H + h) * D, D * 2);
      const float inv = 1.0f / l;
      store_out<kOut>(orow, out_off, val, inv);
    } else {
      const size_t piece = ((size_t)h * a.nr + r) * 2 + (seg_lo > seq_lo ? 0 : 1);
      store_acc<kOut>(make_rsrc(a.ws_acc + piece * D, D * 4), acc_off, val);
      // (m, l) as one 8-byte store; only lane 0 is inside the 8-byte resource
      typedef uint32_t u2v __attribute__((ext_vector_type(2)));
      const u2v ml = {as_u32(m), as_u32(l)};
      __builtin_amdgcn_raw_buffer_store_b64(ml, make_rsrc(a.ws_ml + piece * 2, 8), lane * 8u, 0, 0);
    }
    if (seg_hi < c1) {                 // open the next one
      b = b_next;
      seq_lo = s_start[b];
      seq_hi = s_start[b + 1];
      seg_lo = seg_hi;
      seg_hi = min(c1, seq_hi);
      tail = s_tail[b];
      distribute_q<D>(q, qn, row, lane, s_q[wave]);
      if (seg_hi < c1) {
        b_next = seq_of(s_start, a.B, seg_hi);
        qn = load_q_dword<D>(a.q, (size_t)b_next * a.H + h, lane_off4);
      }
      load_new();                      // (after the query loads: no load drain in the loop)
      m = kNegInf;
      l = 0.0f;
#pragma unroll
      for (int j = 0; j < kAcc; ++j) acc[j] = 0.0f;
    }
  };

  // kFlatTiles tiles in rotation: while one is consumed the next
  // kFlatTiles - 1 are in flight; every iteration issues the same loads.
  Tile<D> t[kFlatTiles];
#pragma unroll
  for (int k = 0; k + 1 < kFlatTiles; ++k) fetch(t[k], c0 + k);
  // Exits jump out of the unrolled body, so no skipped step ever flows
  // back into the loop head (that would make the compiler drain every load).
  int s = c0;
  for (;;) {
#pragma unroll
    for (int k = 0; k < kFlatTiles; ++k) {
      fetch(t[(k + kFlatTiles - 1) % kFlatTiles], s + kFlatTiles - 1);
      step(t[k], s);
      if (++s >= c1) goto done;
    }
  }
done:;
}

// One wave per (sequence, head), four per workgroup.  With the fused
// append, first write the sequence's new token to the pools.  Zero row for
// an empty sequence; for a sequence cut across ranges, merge its pieces
// (weights exp2(m_r - M)) in ascending range order; otherwise nothing (the
// decode kernel wrote the row).  Sequence offsets come from the decode kernel
// (ws_seq), so no prefix sum is redone here.
template <int D>
__global__ __launch_bounds__(256) void pa_decode_flat_merge_kernel(FlatArgs a) {
  constexpr int kPer = D / kWave;
  const int lane = threadIdx.x % kWave;
  const int bh = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (bh >= a.B * a.H) return;
  const int b = bh / a.H;
  const int h = bh % a.H;
  _Float16* orow = a.out + (size_t)bh * D;
  const int T = a.ws_seq[a.B];
  const int S = a.ws_seq[b];
  const int E = a.ws_seq[b + 1];
  if (a.k_new != nullptr) {
    // the fused append: the new token (already used by the decode kernel)
    // goes to the sequence's last position t, slot t % 16 of its last block;
    // lanes 0 .. D/8-1 write K, the next D/8 lanes V, 16 bytes each.  The
    // loads are issued unconditionally, ahead of the merge's own.
    const int ctx = clamp_ctx(a.context_lens[b], a.ctx_limit);
    const int t = max(ctx - 1, 0);
    const int id = a.block_tables[(size_t)b * a.max_blocks + t / kBlockTokens];
    const int g = lane % (D / 8);
    const bool is_v = lane >= D / 8;
    const u4v row_new =
        reinterpret_cast<const u4v*>((is_v ? a.v_new : a.k_new) + (size_t)bh * D)[g];
    // a table entry outside the pool writes nothing, as in kv_append
    if (ctx > 0 && lane < 2 * (D / 8) && (unsigned)id < (unsigned)a.num_blocks) {
      const size_t blk = (size_t)id;
      u4v* dst = reinterpret_cast<u4v*>(const_cast<void*>(is_v ? a.v_pool : a.k_pool));
      dst[((blk * a.H + h) * (D / 8) + g) * kBlockTokens + t % kBlockTokens] = row_new;
    }
  }
  if (E == S) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) orow[lane * kPer + k] = (_Float16)0.0f;
    return;
  }
  const int chunk = (T + a.nr - 1) / a.nr;
  const int r0 = S / chunk;
  const int r1 = (E - 1) / chunk;
  if (r0 == r1) return;                // written whole by the decode kernel
  auto piece = [&](int rr) {
    return ((size_t)h * a.nr + rr) * 2 + (rr * chunk > S ? 0 : 1);
  };
  float mx = kNegInf;
#pragma unroll 4
  for (int rr = r0; rr <= r1; ++rr) mx = fmaxf(mx, a.ws_ml[piece(rr) * 2]);
  float den = 0.0f;
  float num[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) num[k] = 0.0f;
#pragma unroll 4
  for (int rr = r0; rr <= r1; ++rr) {
    const size_t p = piece(rr);
    const float w = exp2f(a.ws_ml[p * 2] - mx);
    den = fmaf(w, a.ws_ml[p * 2 + 1], den);
#pragma unroll
    for (int k = 0; k < kPer; ++k) num[k] = fmaf(w, a.ws_acc[p * D + lane * kPer + k], num[k]);
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int k = 0; k < kPer; ++k) orow[lane * kPer + k] = (_Float16)(num[k] * inv);
}

}  // namespace

size_t flat_lds_bytes(int B, int max_chunk) {
  return (size_t)(2 * B + 1 + max_chunk) * sizeof(int);
}

hipError_t launch_pa_decode_flat(const FlatArgs& a, int D, int threads, hipStream_t stream) {
  const size_t lds = flat_lds_bytes(a.B, a.max_chunk);
  const int grid = a.head_groups * a.nr;
  const bool append = a.k_new != nullptr;
#define PKV_FLAT_LAUNCH(DD, POL, CONTIG, APPEND)                                              \
  hipLaunchKernelGGL((pa_decode_flat_kernel<DD, POL, CONTIG, APPEND>), dim3(grid), dim3(threads), \
                     lds, stream, a)
  const int pol = a.keep_cached ? kCachedPolicy : kStreamPolicy;
  if (a.contig) {
    if (D == 128) PKV_FLAT_LAUNCH(128, kStreamPolicy, true, false);
    else PKV_FLAT_LAUNCH(64, kStreamPolicy, true, false);
  } else if (D == 128) {
    if (pol == kStreamPolicy) {
      if (append) PKV_FLAT_LAUNCH(128, kStreamPolicy, false, true);
      else PKV_FLAT_LAUNCH(128, kStreamPolicy, false, false);
    } else {
      if (append) PKV_FLAT_LAUNCH(128, kCachedPolicy, false, true);
      else PKV_FLAT_LAUNCH(128, kCachedPolicy, false, false);
    }
  } else {
    if (pol == kStreamPolicy) {
      if (append) PKV_FLAT_LAUNCH(64, kStreamPolicy, false, true);
      else PKV_FLAT_LAUNCH(64, kStreamPolicy, false, false);
    } else {
      if (append) PKV_FLAT_LAUNCH(64, kCachedPolicy, false, true);
      else PKV_FLAT_LAUNCH(64, kCachedPolicy, false, false);
    }
  }
#undef PKV_FLAT_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int merge_grid = (a.B * a.H + 3) / 4;
  if (D == 128)
    hipLaunchKernelGGL(pa_decode_flat_merge_kernel<128>, dim3(merge_grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(pa_decode_flat_merge_kernel<64>, dim3(merge_grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
