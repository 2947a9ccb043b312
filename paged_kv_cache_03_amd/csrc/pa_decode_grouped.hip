// PagedAttention decode for groups of sequences that share leading blocks
// (the branches of parallel sampling or beam search, requests forked from
// one prompt), for gfx950 (MI355X).
//
// "PagedAttention" (e-fortepiano.pl), section "Descripció": physical blocks
// are shared between requests or decoding branches through the block
// tables.  Each branch still attends to its own sequence, so the result is
// that of the single-query decode; what changes is that a block shared by n
// branches is read from HBM once, for all n queries, instead of n times.
//
// Work: group g has n <= 16 members (consecutive sequences) whose first P
// logical blocks are the same physical blocks.  Its "positions" are the P
// shared blocks (all n queries attend) followed by each member's private
// blocks (only that member's query attends).  The positions of a group are
// cut into near-equal partitions, whose length each call chooses from the
// total so that the items fill whole rounds of the resident workgroups; a
// workgroup takes (partition, head group) items in a grid-stride loop, one
// wave per head, and stages the item's block ids and masks in LDS.
//
// Per 16-token tile the arithmetic is two small dense contractions on the
// matrix cores, one MFMA column per member (pa_mfma.h).
// Each item ends with one partial result (m, l, acc[D]) per member; a merge
// kernel combines a member's partials in partition order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "pa_common.h"
#include "pa_mfma.h"

namespace pkv {
namespace {

using namespace dev;

constexpr int kInfoShared = 0;        // member field of a shared position

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return min(max(x, lo), hi); }

// Group g's members [lo, lo + n) and its position count; every bound the
// contract states is applied here, so device data cannot push an index out
// of range.
struct GroupShape {
  int lo, n, shared, npos;
};

__device__ GroupShape group_shape(const GroupArgs& a, int g) {
  GroupShape s;
  s.lo = clampi(a.group_offsets[g], 0, a.B);
  const int hi = clampi(a.group_offsets[g + 1], 0, a.B);
  s.n = clampi(hi - s.lo, 0, a.group_size);
  int sum_nb = 0, min_full = 1 << 30;
  for (int k = 0; k < s.n; ++k) {
    const int ctx = clampi(a.context_lens[s.lo + k], 0, a.ctx_limit);
    sum_nb += (ctx + kBlockTokens - 1) / kBlockTokens;
    min_full = min(min_full, ctx / kBlockTokens);
  }
  s.shared = s.n ? clampi(a.group_shared[g], 0, min_full) : 0;
  s.npos = s.n ? sum_nb - (s.n - 1) * s.shared : 0;
  return s;
}

__device__ __forceinline__ int group_parts(int npos, int part_blocks) {
  return (npos + part_blocks - 1) / part_blocks;
}

// Partition length for this call, from the total number of positions:
// items (partitions x head groups) are taken by the resident workgroups in
// rounds, and a nearly empty last round costs as much as a full one.  For
// R rounds the shortest length that keeps the items within R x slots is
// ceil(hg * total / (R * slots - hg * G)) (a group's partitions are at most
// npos / part + 1); take the R whose rounds are shortest overall, counting
// an item's set-up as kGroupItemCost positions.  At least min_part (the
// workspace is sized for it), at most kMaxGroupPartBlocks (LDS staging).
__device__ int choose_part(long long total, int hg, int G, int slots, int min_part) {
  int best = kMaxGroupPartBlocks;
  long long best_cost = -1;
  for (int R = 1; R <= 16; ++R) {
    const long long room = (long long)R * slots - (long long)hg * G;
    if (room <= 0) continue;
    const long long part = max((long long)min_part, ((long long)hg * total + room - 1) / room);
    if (part > kMaxGroupPartBlocks) continue;
    const long long cost = R * (part + kGroupItemCost);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = (int)part;
    }
  }
  return best;
}

// s_part[g] = first partition of group g over all groups, s_part[G] = total;
// returns the partition length.  All threads take part; ends with a barrier.
__device__ int partition_prefix(const GroupArgs& a, int* s_part, int* s_wave) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int per = (a.G + nt - 1) / nt;
  const int lo = min(a.G, tid * per);
  const int hi = min(a.G, lo + per);
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  // total positions over all groups, then the partition length
  int pos = 0;
  for (int g = lo; g < hi; ++g) {
    s_part[g] = group_shape(a, g).npos;   // positions first, partitions below
    pos += s_part[g];
  }
#pragma unroll
  for (int d = kWave / 2; d >= 1; d >>= 1) pos += __shfl_xor(pos, d, kWave);
  if (lane == 0) s_wave[wave] = pos;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < nt / kWave; ++w) total += s_wave[w];
  const int part = choose_part(total, a.head_groups, a.G, a.slots, a.part_blocks);
  __syncthreads();                     // s_wave is reused below
  int own = 0;
  for (int g = lo; g < hi; ++g) {
    const int np = group_parts(s_part[g], part);
    s_part[g] = np;                    // counts first, offsets below
    own += np;
  }
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
  for (int g = lo; g < hi; ++g) {
    const int np = s_part[g];
    s_part[g] = run;
    run += np;
  }
  if (tid == nt - 1) s_part[a.G] = run;
  __syncthreads();
  return part;
}

// The group holding global partition gp: the largest g < G with
// s_part[g] <= gp (which skips groups without partitions).
__device__ __forceinline__ int group_of(const int* s_part, int G, int gp) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_part[mid] <= gp) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int D, int kPolicy>
__global__ __launch_bounds__(64 * kGroupWaves) void pa_decode_grouped_kernel(GroupArgs a) {
  constexpr int kK = D / 32;           // score MFMAs (k = 32 dims each); also 16-byte loads
  constexpr int kS = D / 16;           // P.V MFMAs (16 output dims each)
  constexpr int kTile = D * kBlockTokens * 2;
  extern __shared__ int smem[];
  __shared__ int s_wave[kGroupWaves];
  __shared__ int s_id[kMaxGroupPartBlocks];
  __shared__ int s_info[kMaxGroupPartBlocks];
  __shared__ int s_mem_nb[kGroupMaxMembers];
  __shared__ int s_mem_tail[kGroupMaxMembers];
  __shared__ int s_mem_start[kGroupMaxMembers];
  __shared__ u4v s_v[kGroupWaves][kK * kWave];   // each wave's V tile, as loaded
  int* s_part = smem;                  // G + 1

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int qc = lane % 16;            // query column (member) of this lane
  const int tg = lane / 16;            // token / dim quarter of this lane

  partition_prefix(a, s_part, s_wave);   // (the items' lengths follow from s_part)
  const int total_parts = min(s_part[a.G], a.max_parts);
  if (blockIdx.x == 0) {
    // per-sequence map for the merge: (first partition, partitions * 16 + member)
    for (int b = tid; b < a.B; b += blockDim.x) {
      a.ws_map[2 * b] = -1;
      a.ws_map[2 * b + 1] = 0;
    }
    __syncthreads();
    for (int g = tid; g < a.G; g += blockDim.x) {
      const int first = s_part[g];
      const int np = min(s_part[g + 1], total_parts) - min(first, total_parts);
      if (np <= 0) continue;
      const GroupShape gs = group_shape(a, g);
      for (int k = 0; k < gs.n; ++k) {
        a.ws_map[2 * (gs.lo + k)] = first;
        a.ws_map[2 * (gs.lo + k) + 1] = np * kGroupMaxMembers + k;
      }
    }
  }

  const size_t block_stride = (size_t)a.H * kTile;
  const uint32_t lane_off = lane * 16u;
  u4v* const sv = s_v[wave];
  const _Float16* const svh = reinterpret_cast<const _Float16*>(sv);
  const int items = total_parts * a.head_groups;

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int gp = item / a.head_groups;
    const int hg = item % a.head_groups;
    const int g = group_of(s_part, a.G, gp);
    const int part = gp - s_part[g];
    const int nparts = s_part[g + 1] - s_part[g];
    const GroupShape gs = group_shape(a, g);
    const int plen = (gs.npos + nparts - 1) / nparts;
    const int p0 = part * plen;
    const int cnt = max(0, min(gs.npos, p0 + plen) - p0);
    const int h = hg * kGroupWaves + wave;

    // members' private runs: member k owns positions [start_k, start_k + nb_k - shared)
    if (tid < kWave) {
      const bool live = lane < gs.n;
      const int ctx = live ? clampi(a.context_lens[gs.lo + lane], 0, a.ctx_limit) : 0;
      const int nb = (ctx + kBlockTokens - 1) / kBlockTokens;
      const int own = live ? nb - gs.shared : 0;
      int incl = own;
#pragma unroll
      for (int d = 1; d < kGroupMaxMembers; d <<= 1) {
        const int y = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += y;
      }
      if (lane < kGroupMaxMembers) {
        s_mem_nb[lane] = nb;
        s_mem_tail[lane] = ctx - (nb - 1) * kBlockTokens;
        s_mem_start[lane] = gs.shared + incl - own;
      }
    }
    __syncthreads();
    for (int i = tid; i < cnt; i += blockDim.x) {
      const int pos = p0 + i;
      int row, j, member, valid;
      if (pos < gs.shared) {
        row = gs.lo;
        j = pos;
        member = kInfoShared;
        valid = kBlockTokens;
      } else {
        int k = 0;                     // last member whose run starts at or before pos
        for (int kk = 1; kk < gs.n; ++kk) k = s_mem_start[kk] <= pos ? kk : k;
        row = gs.lo + k;
        j = gs.shared + pos - s_mem_start[k];
        member = k + 1;
        valid = j == s_mem_nb[k] - 1 ? s_mem_tail[k] : kBlockTokens;
      }
      const int id = a.block_tables[(size_t)row * a.max_blocks + j];
      s_id[i] = clampi(id, 0, a.num_blocks - 1);
      s_info[i] = member | (valid << 8);
    }
    __syncthreads();

    // cnt > 0 for every partition ((parts - 1) * plen < npos); an empty item
    // would still write empty partials (m = -inf, l = 0, acc = 0), in the
    // branch after this one.  Entering the ring only with cnt > 0 keeps the
    // compiled loop in the shape the load counters need.
    if (h < a.H && cnt > 0) {
      // queries as the B operand: lane l holds member l%16's dims 32i + 8*(l/16) .. +7
      const rsrc_t qr = make_rsrc(a.q, (uint32_t)((size_t)a.B * a.H * D * 2));
      const uint32_t qoff = qc < gs.n
          ? (uint32_t)((((size_t)(gs.lo + qc) * a.H + h) * D + 8 * tg) * 2)
          : 0xFFFFFFF0u;               // past the resource: reads 0
      h8v qb[kK];
#pragma unroll
      for (int i = 0; i < kK; ++i)
        qb[i] = as_h8(__builtin_amdgcn_raw_buffer_load_b128(qr, qoff + (qc < gs.n ? i * 64 : 0), 0, 0));
      // Keep the query loads ahead of the ring's first tiles: every step
      // reads the queries, so if they were issued after the tiles, the wait
      // for them would hold back one tile in every round of the ring.
      __builtin_amdgcn_sched_barrier(0);

      const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)h * kTile;
      const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)h * kTile;
      auto fetch = [&](MTile<D>& t, int jpos) {
        const int jj = min(jpos, cnt - 1);
        const uint32_t bytes = jpos < cnt ? kTile : 0u;
        const size_t o = (size_t)__builtin_amdgcn_readfirstlane(s_id[jj]) * block_stride;
        mfma_fetch<D, kPolicy>(t, make_rsrc(kbase + o, bytes), make_rsrc(vbase + o, bytes),
                               lane_off);
      };

      float m = kNegInf, l = 0.0f;     // for query qc; l over this lane's tokens only
      f4v acc[kS];
#pragma unroll
      for (int s = 0; s < kS; ++s) acc[s] = f4v{0.0f, 0.0f, 0.0f, 0.0f};

      // A step past the last position (jpos >= cnt) sees valid = 0: every
      // score is -inf, alpha = 1 and every weight and value 0, so it changes
      // nothing; that keeps the ring loop free of exits in its body (an exit
      // there lets the compiler sink the prefetches down to their use).
      auto step = [&](const MTile<D>& t, int jpos) {
        const int info = jpos < cnt ? __builtin_amdgcn_readfirstlane(s_info[jpos]) : 0;
        const int member = info & 0xff;
        const int valid = info >> 8;
        const bool qok = qc < gs.n && (member == kInfoShared || qc == member - 1);
        mfma_update<D>(t, qb, a.scale_log2, valid, [&](int tok) { return qok && tok < valid; },
                       m, l, acc, sv, svh, lane);
      };

      MTile<D> t[kGroupTiles];
#pragma unroll
      for (int k = 0; k + 1 < kGroupTiles; ++k) fetch(t[k], k);
      for (int jpos = 0; jpos < cnt; jpos += kGroupTiles) {
#pragma unroll
        for (int k = 0; k < kGroupTiles; ++k) {
          fetch(t[(k + kGroupTiles - 1) % kGroupTiles], jpos + k + kGroupTiles - 1);
          step(t[k], jpos + k);
        }
      }
      // one partial per member: (m, l) and acc for dims 16s + 4*tg + r
      l = cross_row_sum(l);
      if (qc < gs.n) {
        const size_t piece = ((size_t)(s_part[g] + part) * a.group_size + qc) * a.H + h;
        if (tg == 0) {
          a.ws_ml[piece * 2] = m;
          a.ws_ml[piece * 2 + 1] = l;
        }
        f4v* dst = reinterpret_cast<f4v*>(a.ws_acc + piece * D);
#pragma unroll
        for (int s = 0; s < kS; ++s) dst[4 * s + tg] = acc[s];
      }
    } else if (h < a.H && qc < gs.n) {
      const size_t piece = ((size_t)(s_part[g] + part) * a.group_size + qc) * a.H + h;
      if (tg == 0) {
        a.ws_ml[piece * 2] = kNegInf;
        a.ws_ml[piece * 2 + 1] = 0.0f;
      }
      f4v* dst = reinterpret_cast<f4v*>(a.ws_acc + piece * D);
#pragma unroll
      for (int s = 0; s < kS; ++s) dst[4 * s + tg] = f4v{0.0f, 0.0f, 0.0f, 0.0f};
    }
    __syncthreads();                   // LDS staging is reused by the next item
  }
}

// One wave per (sequence, head): combine the member's partials in partition
// order (weights exp2(m_p - M)); zero row for a sequence that is not
// decoded or has no tokens.
template <int D>
__global__ __launch_bounds__(256) void pa_decode_grouped_merge_kernel(GroupArgs a) {
  constexpr int kPer = D / kWave;
  const int lane = threadIdx.x % kWave;
  const int bh = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (bh >= a.B * a.H) return;
  const int b = bh / a.H;
  const int h = bh % a.H;
  _Float16* orow = a.out + (size_t)bh * D;
  const int first = a.ws_map[2 * b];
  const int np = first < 0 ? 0 : min(a.ws_map[2 * b + 1] / kGroupMaxMembers, a.max_parts - first);
  const int k = a.ws_map[2 * b + 1] % kGroupMaxMembers;
  auto piece = [&](int p) { return ((size_t)(first + p) * a.group_size + k) * a.H + h; };
  float mx = kNegInf;
  for (int p = 0; p < np; ++p) mx = fmaxf(mx, a.ws_ml[piece(p) * 2]);
  if (mx == kNegInf) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) orow[lane * kPer + e] = (_Float16)0.0f;
    return;
  }
  float den = 0.0f;
  float num[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) num[e] = 0.0f;
  for (int p = 0; p < np; ++p) {
    const size_t pc = piece(p);
    const float w = exp2f(a.ws_ml[pc * 2] - mx);
    den = fmaf(w, a.ws_ml[pc * 2 + 1], den);
#pragma unroll
    for (int e = 0; e < kPer; ++e) num[e] = fmaf(w, a.ws_acc[pc * D + lane * kPer + e], num[e]);
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int e = 0; e < kPer; ++e) orow[lane * kPer + e] = (_Float16)(num[e] * inv);
}

}  // namespace

size_t grouped_lds_bytes(int G) { return (size_t)(G + 1) * sizeof(int); }

hipError_t launch_pa_decode_grouped(const GroupArgs& a, int D, int grid, hipStream_t stream) {
  const size_t lds = grouped_lds_bytes(a.G);
  const int threads = kWave * kGroupWaves;
  if (grid > 0) {
    if (D == 128 && !a.keep_cached)
      hipLaunchKernelGGL((pa_decode_grouped_kernel<128, kStreamPolicy>), dim3(grid), dim3(threads), lds, stream, a);
    else if (D == 128)
      hipLaunchKernelGGL((pa_decode_grouped_kernel<128, kCachedPolicy>), dim3(grid), dim3(threads), lds, stream, a);
    else if (!a.keep_cached)
      hipLaunchKernelGGL((pa_decode_grouped_kernel<64, kStreamPolicy>), dim3(grid), dim3(threads), lds, stream, a);
    else
      hipLaunchKernelGGL((pa_decode_grouped_kernel<64, kCachedPolicy>), dim3(grid), dim3(threads), lds, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int merge_grid = (a.B * a.H + 3) / 4;
  if (D == 128)
    hipLaunchKernelGGL(pa_decode_grouped_merge_kernel<128>, dim3(merge_grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(pa_decode_grouped_merge_kernel<64>, dim3(merge_grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
