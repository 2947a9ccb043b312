// Paged prefill for gfx950 (MI355X): the new tokens of every sequence (a
// prompt, or a chunk of one, already appended to its pages) attend causally
// over the sequence's block-paged KV cache.
//
// "PagedAttention" (e-fortepiano.pl), "Formulació matemàtica": causal
// self-attention computed block by block over the paged cache; a query
// token sees the tokens up to and including its own position.  Query row i
// of sequence b (n_b rows) sits at position ctx_b - n_b + i.
//
// Work: a workgroup takes 64 consecutive query rows of one sequence for one
// head; each of its 4 waves serves 16 of them, one MFMA column per row.
// The workgroup streams the blocks up to the one holding its last row's
// position once: every (block, head) tile of K and V is fetched by all 256
// threads together (32 bytes each) through a register ring of kPrefillTiles
// tiles and stored into one of four LDS stages (V slots past the context
// zeroed); after every second tile a barrier, then all 4 waves consume the
// pair: K as the scores' A operands, V through the transpose read, and the
// P.V product over 32 tokens at once on the full-rate 16x16x32 MFMA
// (pa_mfma.h).
// Blocks past a row's position are exact no-ops for it (causal mask per
// element), so a row's result does not depend on the rows it shares a
// workgroup with.  Workgroup i serves head i % H (one XCD per head when H is
// a multiple of 8), and within a sequence the groups that reach furthest
// are dispatched first.

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

template <int D>
__global__ __launch_bounds__(64 * kPrefillWaves) void pa_prefill_kernel(PrefillArgs a) {
  constexpr int kK = D / 32;
  constexpr int kS = D / 16;
  constexpr int kTile = D * kBlockTokens * 2;           // bytes of one K (or V) tile
  constexpr int kTileUnits = kTile / 16;                // 16-byte units of one tile
  constexpr int kUnits = 2 * kTileUnits / (64 * kPrefillWaves);   // per thread: K and V
  constexpr int R = kPrefillTiles;
  static_assert(kUnits >= 1 && R == 4, "tile split; four stages, consumed in pairs");
  extern __shared__ int smem[];
  __shared__ int s_wave[kPrefillWaves];
  __shared__ u4v s_kv[R][2 * kTileUnits];               // stage: K tile, then V tile
  int* s_group = smem;                                  // B + 1
  int* s_ids = smem + a.B + 1;                          // block ids of the sequence

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int qc = lane % 16;

  group_prefix(a, s_group, s_wave);
  const int gt = blockIdx.x / a.H;
  const int h = blockIdx.x % a.H;
  if (gt >= s_group[a.B]) return;                       // uniform for the workgroup
  const int b = seq_of_group(s_group, a.B, gt);
  const int n = rows_of(a, b);
  const int kq = groups_of(a, b) - 1 - (gt - s_group[b]);   // furthest-reaching group first
  const int ctx = clampi(a.context_lens[b], 0, a.ctx_limit);
  const int row0 = kPrefillRows * kq;
  const int grows = min(kPrefillRows, n - row0);
  const int p_group = ctx - n + row0;                   // position of the group's first row
  const int p_last = min(p_group + grows - 1, ctx - 1);
  const int nblk = p_last >= 0 ? p_last / kBlockTokens + 1 : 0;

  for (int j = tid; j < nblk; j += blockDim.x) {
    const int id = a.block_tables[(size_t)b * a.max_blocks + j];
    s_ids[j] = clampi(id, 0, a.num_blocks - 1);
  }
  __syncthreads();

  // this lane's query row: wave w serves rows row0 + 16w ..
  const int wrow = 16 * wave + qc;
  const int qrow = a.query_start[b] + row0 + wrow;
  const bool row_ok = wrow < grows && qrow >= 0 && qrow < a.num_rows;
  const int p_q = p_group + wrow;
  const int tg = lane / 16;
  const rsrc_t qr = make_rsrc(a.q, (uint32_t)((size_t)a.num_rows * a.H * D * 2));
  const uint32_t qoff = row_ok ? (uint32_t)((((size_t)qrow * a.H + h) * D + 8 * tg) * 2)
                               : 0xFFFFFFF0u;           // past the resource: reads 0
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
    // The tile pair is 2 * kTileUnits 16-byte units, unit u = tid + 256 * k
    // (K for u < kTileUnits, V after).  With two units per thread, unit 0 is
    // K and unit 1 is V; with one, waves 0-1 take K and waves 2-3 take V:
    // either way the choice is uniform per wave, so the buffer resource stays
    // in scalar registers.
    auto unit_is_v = [&](int k) { return kUnits == 2 ? k == 1 : wave >= kPrefillWaves / 2; };
    const uint32_t unit_off = (uint32_t)(tid % kTileUnits) * 16u;
    auto fetch = [&](u4v (&r)[kUnits], int j) {
      const int jj = min(j, nblk - 1);
      const uint32_t bytes = j < nblk ? kTile : 0u;
      const size_t o = (size_t)__builtin_amdgcn_readfirstlane(s_ids[jj]) * block_stride;
#pragma unroll
      for (int k = 0; k < kUnits; ++k)
        r[k] = __builtin_amdgcn_raw_buffer_load_b128(
            make_rsrc((unit_is_v(k) ? vbase : kbase) + o, bytes), unit_off, 0, 0);
    };
    auto stage = [&](const u4v (&r)[kUnits], int st, int j) {
      const int valid = j < nblk ? min(kBlockTokens, ctx - j * kBlockTokens) : 0;
#pragma unroll
      for (int k = 0; k < kUnits; ++k) {
        u4v w = r[k];
        // a V unit holds 8 dims of token (tid % kTileUnits) % 16
        const bool zero = unit_is_v(k) && (tid % kTileUnits) % kBlockTokens >= valid;
        w.x = zero ? 0u : w.x;
        w.y = zero ? 0u : w.y;
        w.z = zero ? 0u : w.z;
        w.w = zero ? 0u : w.w;
        s_kv[st][(unit_is_v(k) ? kTileUnits : 0) + tid % kTileUnits] = w;
      }
    };
    // two tiles per step: j and j + 1 from stages sa and sa + 1
    auto compute = [&](int sa, int j) {
      const int va = j < nblk ? min(kBlockTokens, ctx - j * kBlockTokens) : 0;
      const int vb = j + 1 < nblk ? min(kBlockTokens, ctx - (j + 1) * kBlockTokens) : 0;
      const int t0 = j * kBlockTokens;
      u4v ka[kK], kb[kK];
#pragma unroll
      for (int i = 0; i < kK; ++i) {
        ka[i] = s_kv[sa][i * kWave + lane];
        kb[i] = s_kv[sa + 1][i * kWave + lane];
      }
      mfma_update_pair<D>(
          ka, kb, qb, a.scale_log2,
          [&](int tok) { return row_ok && tok < va && t0 + tok <= p_q; },
          [&](int tok) { return row_ok && tok < vb && t0 + kBlockTokens + tok <= p_q; },
          m, l, acc, reinterpret_cast<const _Float16*>(&s_kv[sa][kTileUnits]),
          reinterpret_cast<const _Float16*>(&s_kv[sa + 1][kTileUnits]), lane);
    };
    // R tiles in flight, four LDS stages: tiles j0 .. j0+3 of a round go to
    // stages 0 .. 3, a barrier after each pair, then the pair is consumed.
    // Steps past the last block see valid = 0 (exact no-ops), so the loop
    // runs whole rounds with no exit in its body.
    u4v ring[R][kUnits];
#pragma unroll
    for (int r = 0; r + 1 < R; ++r) fetch(ring[r], r);
    for (int j = 0; j < nblk; j += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        fetch(ring[(r + R - 1) % R], j + r + R - 1);
        stage(ring[r], r, j + r);
        if (r % 2 == 1) {
          __syncthreads();
          compute(r - 1, j + r - 1);
        }
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
    hipLaunchKernelGGL((pa_prefill_kernel<128>), dim3(grid), dim3(threads), lds, stream, a);
  else
    hipLaunchKernelGGL((pa_prefill_kernel<64>), dim3(grid), dim3(threads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
