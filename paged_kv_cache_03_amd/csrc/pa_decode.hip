// PagedAttention decode for gfx950 (MI355X): the partitioned strategy.
//
// What it computes ("PagedAttention", e-fortepiano.pl, sections
// "Formulació matemàtica" and "Descripció"): for one query token per
// sequence, softmax-weighted values over the sequence's cached keys, read
// block by block through the sequence's block table.  The blockwise form is
// evaluated as an online softmax (running maximum m, running sum l, running
// weighted sum acc, all fp32) so each K/V block is read exactly once; long
// contexts are cut into fixed-length partitions whose (m, l, acc) are merged
// by a second kernel in ascending partition order.
//
// Work mapping.  One wavefront owns one (sequence, head, partition).  A
// workgroup holds up to four wavefronts for four consecutive heads of the
// same (sequence, partition), so the partition's block ids are staged once in
// LDS for all of them and the four heads' tiles of a physical block are
// neighbours in memory.  Workgroup i serves head group i % G, so with
// G == 8 every workgroup of one head group lands on the same XCD (workgroups
// are handed to the 8 XCDs round robin) and blocks shared between sequences
// are found in that XCD's L2.  The flat strategy (pa_decode_flat.hip) is the
// default; this one serves explicit partition lengths.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "pa_common.h"

namespace pkv {
namespace {

using namespace dev;

template <int D, int kPolicy>
__global__ __launch_bounds__(256) void pa_decode_part_kernel(PartArgs a) {
  constexpr int L = Geometry<D>::kLoads;
  constexpr int kAcc = Geometry<D>::kAcc;
  constexpr int kTile = Geometry<D>::kTileBytes;
  __shared__ int s_ids[kMaxPartitionBlocks];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int token = lane % kBlockTokens;
  const int row = lane / kBlockTokens;

  const int group = blockIdx.x % a.head_groups;
  const int rest = blockIdx.x / a.head_groups;
  const int b = rest % a.B;
  const int p = rest / a.B;
  const int h = group * a.waves_per_group + wave;

  int ctx = a.context_lens[b];
  ctx = min(max(ctx, 0), a.ctx_limit);
  const int nblk = (ctx + kBlockTokens - 1) / kBlockTokens;
  const int blk0 = p * a.part_blocks;
  const size_t row_out = ((size_t)b * a.H + h) * D;

  if (nblk == 0) {                     // empty context: zero row
    if (p == 0) {
      for (int d = lane; d < D; d += kWave) a.out[row_out + d] = (_Float16)0.0f;
    }
    return;
  }
  if (blk0 >= nblk) return;            // uniform for the workgroup
  const int nb = min(nblk - blk0, a.part_blocks);
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;

  // Stage this partition's block ids in LDS, clamped into the pool.
  const int* table = a.block_tables + (size_t)b * a.max_blocks + blk0;
  for (int j = threadIdx.x; j < nb; j += blockDim.x) {
    const int id = table[j];
    s_ids[j] = min(max(id, 0), a.num_blocks - 1);
  }
  __syncthreads();

  // This lane's query groups: 4*i + row for i < L.
  u4v q[L];
  {
    const char* qrow = reinterpret_cast<const char*>(a.q) + row_out * 2;
#pragma unroll
    for (int i = 0; i < L; ++i)
      q[i] = *reinterpret_cast<const u4v*>(qrow + (4 * i + row) * 16);
  }

  // Wave-uniform tile addresses: pool + (id * H + h) * tile bytes.
  const char* kpool = reinterpret_cast<const char*>(a.k_pool) + (size_t)h * kTile;
  const char* vpool = reinterpret_cast<const char*>(a.v_pool) + (size_t)h * kTile;
  const size_t block_stride = (size_t)a.H * kTile;
  const uint32_t lane_off = lane * 16u;
  auto block_off = [&](int j) -> size_t {
    return (size_t)__builtin_amdgcn_readfirstlane(s_ids[j]) * block_stride;
  };

  float m = kNegInf, l = 0.0f;
  float acc[kAcc];
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = 0.0f;

  // Blocks before `nfull` are full; a partially filled block can only be
  // the sequence's last one, with `tail` tokens.
  const int tail = ctx - (blk0 + nb - 1) * kBlockTokens;
  const int nfull = tail < kBlockTokens ? nb - 1 : nb;

  // Two tiles alternate: while one is consumed the next one is in flight.
  // The prefetch is unconditional (past the end it re-reads the partition's
  // last tile, an L1/L2 hit) and the loop body has no divergent branch, so
  // the load counters stay exact across iterations.
  Tile<D> ta, tb;
  auto fetch = [&](Tile<D>& t, int j) {
    const size_t o = block_off(min(j, nb - 1));
    load_tile<D, kPolicy>(t, make_rsrc(kpool + o, kTile), make_rsrc(vpool + o, kTile), lane_off);
  };
  fetch(ta, 0);
  int j = 0;
  for (; j + 2 <= nfull; j += 2) {      // ta holds block j on entry
    fetch(tb, j + 1);
    consume<D, false>(ta, q, a.scale_log2, token, kBlockTokens, m, l, acc);
    fetch(ta, j + 2);
    consume<D, false>(tb, q, a.scale_log2, token, kBlockTokens, m, l, acc);
  }
  if (j < nfull) {                      // one full block left, maybe a partial one after it
    fetch(tb, j + 1);
    consume<D, false>(ta, q, a.scale_log2, token, kBlockTokens, m, l, acc);
    if (j + 1 < nb) consume<D, true>(tb, q, a.scale_log2, token, tail, m, l, acc);
  } else if (j < nb) {
    consume<D, true>(ta, q, a.scale_log2, token, tail, m, l, acc);
  }

  float val[Geometry<D>::kOutPerLane];
  const int d0 = reduce_rows<D>(l, acc, token, row, val);

  if (nparts == 1) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int k = 0; k < Geometry<D>::kOutPerLane; ++k)
      a.out[row_out + d0 + k] = (_Float16)(val[k] * inv);
  } else {
    const size_t slot = ((size_t)b * a.H + h) * a.max_parts + p;
    float* wacc = a.ws_acc + slot * D;
#pragma unroll
    for (int k = 0; k < Geometry<D>::kOutPerLane; ++k) wacc[d0 + k] = val[k];
    if (lane == 0) {
      a.ws_ml[slot * 2 + 0] = m;
      a.ws_ml[slot * 2 + 1] = l;
    }
  }
}

// Merge of the partitions of one (sequence, head): weights exp2(m_p - M),
// summed in ascending partition order.
template <int D>
__global__ __launch_bounds__(256) void pa_decode_merge_kernel(MergeArgs a) {
  constexpr int kPer = D / kWave;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int bh = blockIdx.x * (blockDim.x / kWave) + wave;
  if (bh >= a.B * a.H) return;
  const int b = bh / a.H;
  int ctx = a.context_lens[b];
  ctx = min(max(ctx, 0), a.ctx_limit);
  const int nblk = (ctx + kBlockTokens - 1) / kBlockTokens;
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;
  if (nparts <= 1) return;              // written directly by the partition kernel
  const size_t base = (size_t)bh * a.max_parts;
  float mx = kNegInf;
  for (int p = 0; p < nparts; ++p) mx = fmaxf(mx, a.ws_ml[(base + p) * 2]);
  float den = 0.0f;
  float num[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) num[k] = 0.0f;
  for (int p = 0; p < nparts; ++p) {
    const float w = exp2f(a.ws_ml[(base + p) * 2] - mx);
    den = fmaf(w, a.ws_ml[(base + p) * 2 + 1], den);
    const float* acc = a.ws_acc + (base + p) * D;
#pragma unroll
    for (int k = 0; k < kPer; ++k) num[k] = fmaf(w, acc[lane * kPer + k], num[k]);
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int k = 0; k < kPer; ++k) a.out[(size_t)bh * D + lane * kPer + k] = (_Float16)(num[k] * inv);
}

}  // namespace

hipError_t launch_pa_decode(const PartArgs& part, int D, int grid_part, int threads,
                            hipStream_t stream) {
  if (D == 128 && !part.keep_cached)
    hipLaunchKernelGGL((pa_decode_part_kernel<128, kStreamPolicy>), dim3(grid_part), dim3(threads), 0, stream, part);
  else if (D == 128)
    hipLaunchKernelGGL((pa_decode_part_kernel<128, kCachedPolicy>), dim3(grid_part), dim3(threads), 0, stream, part);
  else if (!part.keep_cached)
    hipLaunchKernelGGL((pa_decode_part_kernel<64, kStreamPolicy>), dim3(grid_part), dim3(threads), 0, stream, part);
  else
    hipLaunchKernelGGL((pa_decode_part_kernel<64, kCachedPolicy>), dim3(grid_part), dim3(threads), 0, stream, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || part.max_parts <= 1) return e;
  MergeArgs mg;
  mg.ws_ml = part.ws_ml;
  mg.ws_acc = part.ws_acc;
  mg.context_lens = part.context_lens;
  mg.out = part.out;
  mg.B = part.B;
  mg.H = part.H;
  mg.ctx_limit = part.ctx_limit;
  mg.part_blocks = part.part_blocks;
  mg.max_parts = part.max_parts;
  const int per_wg = 4;
  const int grid = (part.B * part.H + per_wg - 1) / per_wg;
  if (D == 128)
    hipLaunchKernelGGL(pa_decode_merge_kernel<128>, dim3(grid), dim3(per_wg * kWave), 0, stream, mg);
  else
    hipLaunchKernelGGL(pa_decode_merge_kernel<64>, dim3(grid), dim3(per_wg * kWave), 0, stream, mg);
  return hipGetLastError();
}

}  // namespace pkv
