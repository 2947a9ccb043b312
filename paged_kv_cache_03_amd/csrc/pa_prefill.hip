// Paged prefill for gfx950 (MI355X): the new tokens of every sequence (a
// prompt, or a chunk of one, already appended to its pages) attend causally
// over the sequence's block-paged KV cache.
//
// "PagedAttention" (e-fortepiano.pl), "Formulació matemàtica": causal
// self-attention computed block by block over the paged cache; a query
// token sees the tokens up to and including its own position.  Query row i
// of sequence b (n_b rows) sits at position ctx_b - n_b + i.
//
// Work: a workgroup takes one tile of 16 consecutive query rows of one
// sequence for 4 heads (one wave per head).  It stages the block ids the
// tile needs (blocks 0 .. the one holding its last position) in LDS, and
// each wave streams those blocks through a 3-tile load ring.  Per block the
// 16 x 16 scores and the P.V product run on the matrix cores (pa_mfma.h)
// with the causal mask applied per (token, query) element.  No partial
// results: every wave writes its 16 output rows.  Workgroup i serves head
// group i % G (one XCD per head group with G = 8), and within a sequence the
// tiles that reach furthest (the longest) are dispatched first.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "pa_common.h"
#include "pa_mfma.h"

namespace pkv {
namespace {

using namespace dev;

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

__device__ __forceinline__ int rows_of(const PrefillArgs& a, int b) {
  return max(0, a.query_start[b + 1] - a.query_start[b]);
}

// s_tile[b] = first query tile of sequence b over the batch, s_tile[B] =
// total.  All threads take part; ends with a barrier.
__device__ void tile_prefix(const PrefillArgs& a, int* s_tile, int* s_wave) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int per = (a.B + nt - 1) / nt;
  const int lo = min(a.B, tid * per);
  const int hi = min(a.B, lo + per);
  int own = 0;
  for (int b = lo; b < hi; ++b) own += (rows_of(a, b) + 15) / 16;
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
    s_tile[b] = run;
    run += (rows_of(a, b) + 15) / 16;
  }
  if (tid == nt - 1) s_tile[a.B] = run;
  __syncthreads();
}

__device__ __forceinline__ int seq_of_tile(const int* s_tile, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tile[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int D, int kPolicy>
__global__ __launch_bounds__(64 * kPrefillWaves) void pa_prefill_kernel(PrefillArgs a) {
  constexpr int kK = D / 32;
  constexpr int kS = D / 16;
  constexpr int kTile = D * kBlockTokens * 2;
  extern __shared__ int smem[];
  __shared__ int s_wave[kPrefillWaves];
  __shared__ u4v s_v[kPrefillWaves][kK * kWave];   // each wave's V tile, as loaded
  int* s_tile = smem;                  // B + 1
  int* s_ids = smem + a.B + 1;         // block ids of the tile's sequence

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int qc = lane % 16;
  const int tg = lane / 16;

  tile_prefix(a, s_tile, s_wave);
  const int gt = blockIdx.x / a.head_groups;
  const int hg = blockIdx.x % a.head_groups;
  if (gt >= s_tile[a.B]) return;       // uniform for the workgroup
  const int b = seq_of_tile(s_tile, a.B, gt);
  const int n = rows_of(a, b);
  const int ntiles = (n + 15) / 16;
  const int k = ntiles - 1 - (gt - s_tile[b]);     // furthest-reaching tile first
  const int ctx = clampi(a.context_lens[b], 0, a.ctx_limit);
  const int row0 = 16 * k;
  const int rows = min(16, n - row0);
  const int p_first = ctx - n + row0;  // position of the tile's first row
  const int p_last = min(p_first + rows - 1, ctx - 1);
  const int nblk = p_last >= 0 ? p_last / kBlockTokens + 1 : 0;
  const int h = hg * kPrefillWaves + wave;
  const int qrow0 = a.query_start[b] + row0;

  for (int j = tid; j < nblk; j += blockDim.x) {
    const int id = a.block_tables[(size_t)b * a.max_blocks + j];
    s_ids[j] = clampi(id, 0, a.num_blocks - 1);
  }
  __syncthreads();
  if (h >= a.H) return;

  // this lane's query row and position (rows past the tile or the output
  // array attend to nothing)
  const int qrow = qrow0 + qc;
  const bool row_ok = qc < rows && qrow >= 0 && qrow < a.num_rows;
  const int p_q = p_first + qc;
  const rsrc_t qr = make_rsrc(a.q, (uint32_t)((size_t)a.num_rows * a.H * D * 2));
  const uint32_t qoff = row_ok ? (uint32_t)((((size_t)qrow * a.H + h) * D + 8 * tg) * 2)
                               : 0xFFFFFFF0u;   // past the resource: reads 0
  h8v qb[kK];
#pragma unroll
  for (int i = 0; i < kK; ++i)
    qb[i] = as_h8(__builtin_amdgcn_raw_buffer_load_b128(qr, qoff + (row_ok ? i * 64 : 0), 0, 0));
  // keep the query loads ahead of the ring's first tiles (every step reads them)
  __builtin_amdgcn_sched_barrier(0);

  float m = kNegInf, l = 0.0f;
  f4v acc[kS];
#pragma unroll
  for (int s = 0; s < kS; ++s) acc[s] = f4v{0.0f, 0.0f, 0.0f, 0.0f};

  if (nblk > 0) {
    const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)h * kTile;
    const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)h * kTile;
    const size_t block_stride = (size_t)a.H * kTile;
    const uint32_t lane_off = lane * 16u;
    u4v* const sv = s_v[wave];
    const _Float16* const svh = reinterpret_cast<const _Float16*>(sv);
    auto fetch = [&](MTile<D>& t, int j) {
      const int jj = min(j, nblk - 1);
      const uint32_t bytes = j < nblk ? kTile : 0u;
      const size_t o = (size_t)__builtin_amdgcn_readfirstlane(s_ids[jj]) * block_stride;
      mfma_fetch<D, kPolicy>(t, make_rsrc(kbase + o, bytes), make_rsrc(vbase + o, bytes),
                             lane_off);
    };
    // Steps past the last block see valid = 0 (an exact no-op), so the ring
    // runs whole rounds with no exit in its body.
    auto step = [&](const MTile<D>& t, int j) {
      const int valid = j < nblk ? min(kBlockTokens, ctx - j * kBlockTokens) : 0;
      const int t0 = j * kBlockTokens;
      mfma_update<D>(t, qb, a.scale_log2, valid,
                     [&](int tok) { return row_ok && tok < valid && t0 + tok <= p_q; },
                     m, l, acc, sv, svh, lane);
    };
    MTile<D> t[kPrefillTiles];
#pragma unroll
    for (int r = 0; r + 1 < kPrefillTiles; ++r) fetch(t[r], r);
    for (int j = 0; j < nblk; j += kPrefillTiles) {
#pragma unroll
      for (int r = 0; r < kPrefillTiles; ++r) {
        fetch(t[(r + kPrefillTiles - 1) % kPrefillTiles], j + r + kPrefillTiles - 1);
        step(t[r], j + r);
      }
    }
  }

  // rows at a negative position (more queries than cached tokens) are zero
  l = cross_row_sum(l);
  if (row_ok) {
    const float inv = p_q >= 0 && l > 0.0f ? 1.0f / l : 0.0f;
    _Float16* orow = a.out + ((size_t)qrow * a.H + h) * D + 4 * tg;
#pragma unroll
    for (int s = 0; s < kS; ++s) {
      h4v o;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = (_Float16)(acc[s][r] * inv);
      *reinterpret_cast<h4v*>(orow + 16 * s) = o;
    }
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
    hipLaunchKernelGGL((pa_prefill_kernel<128, kCachedPolicy>), dim3(grid), dim3(threads), lds, stream, a);
  else
    hipLaunchKernelGGL((pa_prefill_kernel<64, kCachedPolicy>), dim3(grid), dim3(threads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
