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
// blocks (only that member's query attends).  The positions of all groups
// are lined up, group after group, and cut into equal ranges, as the flat
// decode does with sequences: workgroup i serves head group i % HG and the
// (i / HG)-th range, one wave per head.  The workgroup stages its range's
// block ids and masks in LDS; each wave takes the range's groups in turn,
// loads the group's queries and streams the group's positions in the range
// with a ring of tiles.  A group wholly inside the range
// writes its members' output rows; a group cut by the range's start or end
// leaves one partial result per member (at most two per wave), which a
// merge kernel combines in range order.
//
// Per 16-token tile the arithmetic is two small dense contractions on the
// matrix cores, one MFMA column per member (pa_mfma.h).

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

// Group g's members [lo, lo + n), its shared block count and position
// count; every bound the contract states is applied here, so device data
// cannot push an index out of range.
struct GroupShape {
  int lo, n, shared, npos;
};

__device__ __forceinline__ void group_members(const GroupArgs& a, int g, int& lo, int& n) {
  lo = clampi(a.group_offsets[g], 0, a.B);
  const int hi = clampi(a.group_offsets[g + 1], 0, a.B);
  n = clampi(hi - lo, 0, a.group_size);
}

// s_ctx: every sequence's context length, clamped to [0, ctx_limit],
// staged in LDS once per workgroup (one load per thread), so that the
// member loops below read LDS rather than a chain of dependent global
// loads.
__device__ GroupShape group_shape(const GroupArgs& a, const int* s_ctx, int g) {
  GroupShape s;
  group_members(a, g, s.lo, s.n);
  int sum_nb = 0, min_full = 1 << 30;
  for (int k = 0; k < s.n; ++k) {
    const int ctx = s_ctx[s.lo + k];
    sum_nb += (ctx + kBlockTokens - 1) / kBlockTokens;
    min_full = min(min_full, ctx / kBlockTokens);
  }
  s.shared = s.n ? clampi(a.group_shared[g], 0, min_full) : 0;
  s.npos = s.n ? sum_nb - (s.n - 1) * s.shared : 0;
  return s;
}

// Position pos (< npos) of a group: the table row and logical block it
// reads, its member field (0 = shared, k + 1 = member k's private block) and
// its tokens in use.
struct PosInfo {
  int row, j, member, valid;
};

__device__ PosInfo position_info(const int* s_ctx, const GroupShape& gs, int pos) {
  if (pos < gs.shared) return {gs.lo, pos, kInfoShared, kBlockTokens};
  int start = gs.shared;               // member k's private blocks start here
  for (int k = 0; k < gs.n; ++k) {
    const int ctx = s_ctx[gs.lo + k];
    const int nb = (ctx + kBlockTokens - 1) / kBlockTokens;
    const int own = nb - gs.shared;
    if (pos < start + own) {
      const int j = gs.shared + pos - start;
      const int valid = j == nb - 1 ? ctx - (nb - 1) * kBlockTokens : kBlockTokens;
      return {gs.lo + k, j, k + 1, valid};
    }
    start += own;
  }
  return {gs.lo, 0, kInfoShared, 0};   // not reached for pos < npos
}

// s_gpos[g] = first position of group g over all groups, s_gpos[G] = total,
// each clamped to a.t_cap (the ranges' capacity): the groups' members are
// disjoint under the contract, so the total stays below it, but overlapping
// groups in device data must not push a range past its LDS staging.  All
// threads take part; ends with a barrier.
__device__ void position_prefix(const GroupArgs& a, const int* s_ctx, int* s_gpos,
                                long long* s_wave) {
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const int per = (a.G + nt - 1) / nt;
  const int lo = min(a.G, tid * per);
  const int hi = min(a.G, lo + per);
  long long own = 0;
  for (int g = lo; g < hi; ++g) {
    const int np = group_shape(a, s_ctx, g).npos;
    s_gpos[g] = np;                    // counts first, offsets below
    own += np;
  }
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  long long incl = own;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const long long y = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  long long run = incl - own;
  for (int w = 0; w < wave; ++w) run += s_wave[w];
  for (int g = lo; g < hi; ++g) {
    const int np = s_gpos[g];
    s_gpos[g] = (int)min(run, (long long)a.t_cap);
    run += np;
  }
  if (tid == nt - 1) s_gpos[a.G] = (int)min(run, (long long)a.t_cap);
  __syncthreads();
}

// The group holding position s (0 <= s < total): the largest g with
// s_gpos[g] <= s, which skips groups without positions.
__device__ __forceinline__ int group_of(const int* s_gpos, int G, int s) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_gpos[mid] <= s) lo = mid;
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
  __shared__ long long s_wave[kGroupWaves];
  __shared__ u4v s_v[kGroupWaves][kK * kWave];   // each wave's V tile, as loaded
  int* s_ctx = smem;                   // B: context lengths, clamped
  int* s_gpos = s_ctx + a.B;           // G + 1
  int* s_id = s_gpos + a.G + 1;        // max_chunk: block id of each position of the range
  int* s_info = s_id + a.max_chunk;    // max_chunk: member | valid << 8
  int* s_grp = s_info + a.max_chunk;   // max_chunk: group of each position
  int* s_mem = s_grp + a.max_chunk;    // max_chunk: its first member * 32 + member count

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int qc = lane % 16;            // query column (member) of this lane
  const int tg = lane / 16;            // token / dim quarter of this lane
  const int hg = blockIdx.x % a.head_groups;
  const int r = blockIdx.x / a.head_groups;
  const int h = hg * kGroupWaves + wave;

  for (int b = tid; b < a.B; b += blockDim.x) s_ctx[b] = clampi(a.context_lens[b], 0, a.ctx_limit);
  __syncthreads();
  position_prefix(a, s_ctx, s_gpos, s_wave);
  if (blockIdx.x == 0) {
    // group offsets and the per-sequence map (group * 16 + member, or -1)
    // for the merge
    for (int i = tid; i <= a.G; i += blockDim.x) a.ws_gpos[i] = s_gpos[i];
    for (int b = tid; b < a.B; b += blockDim.x) a.ws_map[b] = -1;
    __syncthreads();
    for (int g = tid; g < a.G; g += blockDim.x) {
      int lo, n;
      group_members(a, g, lo, n);
      for (int k = 0; k < n; ++k) a.ws_map[lo + k] = g * kGroupMaxMembers + k;
    }
  }
  const int T = s_gpos[a.G];
  const int chunk = (T + a.nr - 1) / a.nr;
  const int c0 = min(T, r * chunk);
  const int c1 = min(T, c0 + chunk);
  if (c0 >= c1) return;                // uniform for the workgroup
  const int cnt = c1 - c0;

  for (int i = tid; i < cnt; i += blockDim.x) {
    const int s = c0 + i;
    const int g = group_of(s_gpos, a.G, s);
    const GroupShape gs = group_shape(a, s_ctx, g);
    const PosInfo pi = position_info(s_ctx, gs, s - s_gpos[g]);
    const int id = a.block_tables[(size_t)pi.row * a.max_blocks + pi.j];
    s_id[i] = clampi(id, 0, a.num_blocks - 1);
    s_info[i] = pi.member | (pi.valid << 8);
    s_grp[i] = g;
    s_mem[i] = gs.lo * 32 + gs.n;
  }
  __syncthreads();
  if (h >= a.H) return;                // uniform per wave; no barrier follows

  const size_t block_stride = (size_t)a.H * kTile;
  const uint32_t lane_off = lane * 16u;
  u4v* const sv = s_v[wave];
  const _Float16* const svh = reinterpret_cast<const _Float16*>(sv);
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + (size_t)h * kTile;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + (size_t)h * kTile;
  const rsrc_t qr = make_rsrc(a.q, (uint32_t)((size_t)a.B * a.H * D * 2));

  // The range in segments, one per group it touches: for each, the
  // group's queries, a ring over the segment's positions, then its output
  // rows (a group wholly inside the range) or one partial per member.  The
  // ring does not run across a group boundary: the queries change there.
  for (int sg = 0; sg < cnt;) {        // uniform
    const int g = __builtin_amdgcn_readfirstlane(s_grp[sg]);
    const int gstart = s_gpos[g];
    const int gend = s_gpos[g + 1];
    const int mem = __builtin_amdgcn_readfirstlane(s_mem[sg]);
    const int lo = mem >> 5;
    const int n = mem & 31;
    const int seg_lo = c0 + sg;
    const int seg_hi = min(c1, gend);
    const int scnt = seg_hi - seg_lo;  // >= 1

    // queries as the B operand: lane l holds member l%16's dims 32i + 8*(l/16) .. +7
    const uint32_t qoff = qc < n ? (uint32_t)((((size_t)(lo + qc) * a.H + h) * D + 8 * tg) * 2)
                                 : 0xFFFFFFF0u;      // past the resource: reads 0
    h8v qb[kK];
#pragma unroll
    for (int i = 0; i < kK; ++i)
      qb[i] = as_h8(__builtin_amdgcn_raw_buffer_load_b128(qr, qoff + (qc < n ? i * 64 : 0), 0, 0));
    // Keep the query loads ahead of the ring's first tiles: every step reads
    // the queries, so if they were issued after the tiles, the wait for them
    // would hold back one tile in every round of the ring.
    __builtin_amdgcn_sched_barrier(0);

    // V tokens at or past the position's valid count load as zeros
    auto fetch = [&](MTile<D>& t, int j) {
      const int jj = sg + min(j, scnt - 1);
      const uint32_t bytes = j < scnt ? kTile : 0u;
      const size_t o = (size_t)__builtin_amdgcn_readfirstlane(s_id[jj]) * block_stride;
      const int valid = __builtin_amdgcn_readfirstlane(s_info[jj]) >> 8;
      const uint32_t v_off = lane % kBlockTokens < valid ? lane_off : 0xFFFFF000u;
      mfma_fetch<D, kPolicy>(t, make_rsrc(kbase + o, bytes), make_rsrc(vbase + o, bytes),
                             lane_off, v_off);
    };

    float m = kNegInf, l = 0.0f;       // for query qc; l over this lane's tokens only
    f4v acc[kS];
#pragma unroll
    for (int s = 0; s < kS; ++s) acc[s] = f4v{0.0f, 0.0f, 0.0f, 0.0f};

    // A step past the segment's end (j >= scnt) sees valid = 0: every score
    // is -inf, alpha = 1 and every weight and value 0, so it changes
    // nothing; that keeps the ring loop free of exits in its body (an exit
    // there lets the compiler sink the prefetches down to their use).
    auto step = [&](const MTile<D>& t, int j) {
      const int info = j < scnt ? __builtin_amdgcn_readfirstlane(s_info[sg + j]) : 0;
      const int member = info & 0xff;
      const int valid = info >> 8;
      const bool qok = qc < n && (member == kInfoShared || qc == member - 1);
      mfma_update<D>(t, qb, a.scale_log2, [&](int tok) { return qok && tok < valid; }, m, l,
                     acc, sv, svh, lane);
    };

    // (a do-while: a segment is never empty, and a ring entered only when
    // it has work keeps the compiled loop in the shape the load counters
    // need)
    MTile<D> t[kGroupTiles];
#pragma unroll
    for (int k = 0; k + 1 < kGroupTiles; ++k) fetch(t[k], k);
    int j = 0;
    do {
#pragma unroll
      for (int k = 0; k < kGroupTiles; ++k) {
        fetch(t[(k + kGroupTiles - 1) % kGroupTiles], j + k + kGroupTiles - 1);
        step(t[k], j + k);
      }
      j += kGroupTiles;
    } while (j < scnt);

    // the group's output rows if the segment is the whole group, else one
    // partial (m, l, acc for dims 16s + 4*tg + r) per member: piece 0 if
    // the group began before this range, 1 if it goes on after it
    l = cross_row_sum(l);
    if (qc < n) {
      if (seg_lo == gstart && seg_hi == gend) {
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        _Float16* orow = a.out + ((size_t)(lo + qc) * a.H + h) * D + 4 * tg;
#pragma unroll
        for (int s = 0; s < kS; ++s) {
          h4v o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (_Float16)(acc[s][e] * inv);
          *reinterpret_cast<h4v*>(orow + 16 * s) = o;
        }
      } else {
        // (m, l) for every member; the weighted sums only for a member that
        // met a live token here (m > -inf): the merge skips the others'
        const size_t piece =
            (((size_t)h * a.nr + r) * 2 + (seg_lo > gstart ? 0 : 1)) * a.group_size + qc;
        if (tg == 0) {
          a.ws_ml[piece * 2] = m;
          a.ws_ml[piece * 2 + 1] = l;
        }
        if (m != kNegInf) {
          f4v* dst = reinterpret_cast<f4v*>(a.ws_acc + piece * D);
#pragma unroll
          for (int s = 0; s < kS; ++s) dst[4 * s + tg] = acc[s];
        }
      }
    }
    sg += scnt;
  }
}

// Sum over the wave (every lane ends with the total, the same in every
// lane).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) x += __shfl_xor(x, d, kWave);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) x = fmaxf(x, __shfl_xor(x, d, kWave));
  return x;
}

// One wave per (sequence, head): zero row for a sequence that is in no
// group or has nothing to attend to; for a member of a group cut across
// ranges, combine its partials (weights exp2(m_r - M)); otherwise nothing
// (the decode kernel wrote the row).  A group can span many ranges, so the
// pieces' (m, l) are read one per lane, at once; a piece whose m is -inf (no
// live token of the member in that range) has no weighted sums and is left
// out, and the weighted sums of the others are loaded eight at a time before
// they are added.
template <int D>
__global__ __launch_bounds__(256) void pa_decode_grouped_merge_kernel(GroupArgs a) {
  constexpr int kPer = D / kWave;
  constexpr int kUnroll = 8;
  const int lane = threadIdx.x % kWave;
  const int bh = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (bh >= a.B * a.H) return;
  const int b = bh / a.H;
  const int h = bh % a.H;
  _Float16* orow = a.out + (size_t)bh * D;
  auto zero_row = [&]() {
#pragma unroll
    for (int e = 0; e < kPer; ++e) orow[lane * kPer + e] = (_Float16)0.0f;
  };
  const int map = a.ws_map[b];
  if (map < 0) return zero_row();
  const int g = map / kGroupMaxMembers;
  const int k = map % kGroupMaxMembers;
  const int T = a.ws_gpos[a.G];
  const int S = a.ws_gpos[g];
  const int E = a.ws_gpos[g + 1];
  if (E <= S) return zero_row();
  const int chunk = (T + a.nr - 1) / a.nr;
  const int r0 = S / chunk;
  const int r1 = (E - 1) / chunk;
  if (r0 == r1) return;                // written whole by the decode kernel
  auto piece = [&](int rr) {
    return (((size_t)h * a.nr + rr) * 2 + (rr * chunk > S ? 0 : 1)) * a.group_size + k;
  };
  // the largest reference over all pieces, 64 pieces a round
  float mx = kNegInf;
  for (int base = r0; base <= r1; base += kWave) {
    const int rr = base + lane;
    if (rr <= r1) mx = fmaxf(mx, a.ws_ml[piece(rr) * 2]);
  }
  mx = wave_max(mx);
  if (mx == kNegInf) return zero_row();   // a member with no tokens
  float den = 0.0f;
  float num[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) num[e] = 0.0f;
  for (int base = r0; base <= r1; base += kWave) {
    const int rr = base + lane;
    float w = 0.0f;                    // this lane's piece's weight, 0 if empty
    if (rr <= r1) {
      const size_t pc = piece(rr);
      const float mr = a.ws_ml[pc * 2];
      if (mr != kNegInf) {
        w = exp2f(mr - mx);
        den = fmaf(w, a.ws_ml[pc * 2 + 1], den);
      }
    }
    // the pieces of this round that have weighted sums, in range order:
    // lane j of the round is piece base + j; taken kUnroll at a time, their
    // loads issued before they are added (a slot past the last one repeats
    // it with weight 0)
    uint64_t live = __builtin_amdgcn_ballot_w64(w != 0.0f);
    while (live) {                     // uniform
      float acc_j[kUnroll][kPer];
      float w_j[kUnroll];
      int last = 0;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const bool any = live != 0;
        const int j = any ? __builtin_ctzll(live) : last;
        live = any ? live & (live - 1) : live;
        last = j;
        w_j[u] = any ? __shfl(w, j, kWave) : 0.0f;
        const float* src = a.ws_acc + piece(base + j) * D + lane * kPer;
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc_j[u][e] = src[e];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int e = 0; e < kPer; ++e)
          num[e] = w_j[u] != 0.0f ? fmaf(w_j[u], acc_j[u][e], num[e]) : num[e];
    }
  }
  den = wave_sum(den);
  const float inv = 1.0f / den;
#pragma unroll
  for (int e = 0; e < kPer; ++e) orow[lane * kPer + e] = (_Float16)(num[e] * inv);
}

}  // namespace

size_t grouped_lds_bytes(int B, int G, int max_chunk) {
  return ((size_t)B + G + 1 + 4 * (size_t)max_chunk) * sizeof(int);
}

hipError_t launch_pa_decode_grouped(const GroupArgs& a, int D, hipStream_t stream) {
  const size_t lds = grouped_lds_bytes(a.B, a.G, a.max_chunk);
  const int threads = kWave * kGroupWaves;
  const int grid = a.head_groups * a.nr;
  if (D == 128 && !a.keep_cached)
    hipLaunchKernelGGL((pa_decode_grouped_kernel<128, kStreamPolicy>), dim3(grid), dim3(threads), lds, stream, a);
  else if (D == 128)
    hipLaunchKernelGGL((pa_decode_grouped_kernel<128, kCachedPolicy>), dim3(grid), dim3(threads), lds, stream, a);
  else if (!a.keep_cached)
    hipLaunchKernelGGL((pa_decode_grouped_kernel<64, kStreamPolicy>), dim3(grid), dim3(threads), lds, stream, a);
  else
    hipLaunchKernelGGL((pa_decode_grouped_kernel<64, kCachedPolicy>), dim3(grid), dim3(threads), lds, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int merge_grid = (a.B * a.H + 3) / 4;
  if (D == 128)
    hipLaunchKernelGGL(pa_decode_grouped_merge_kernel<128>, dim3(merge_grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(pa_decode_grouped_merge_kernel<64>, dim3(merge_grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
