// PagedAttention decode for gfx950 (MI355X).
//
// What it computes ("PagedAttention", e-fortepiano.pl, sections
// "Formulació matemàtica" and "Descripció"): for one query token per
// sequence, softmax-weighted values over the sequence's cached keys, read
// block by block through the sequence's block table.  The blockwise form is
// evaluated here as an online softmax (running maximum m, running sum l,
// running weighted sum acc, all fp32) so each K/V block is read exactly
// once; long contexts are cut into partitions whose (m, l, acc) are merged
// by a second kernel.
//
// Work mapping.  One wavefront owns one (sequence, head, partition).  A
// workgroup holds up to four wavefronts for four consecutive heads of the
// same (sequence, partition), so the partition's block ids are staged once in
// LDS for all of them and the four heads' tiles of a physical block are
// neighbours in memory.  Workgroup i serves head group i % G, so with
// G == 8 every workgroup of one head group lands on the same XCD (workgroups
// are handed to the 8 XCDs round robin) and blocks shared between sequences
// are found in that XCD's L2.
//
// Lane mapping inside one (block, head) tile.  A tile is D/8 groups x 16
// tokens x 8 values (fp16).  Load i of lane l reads the 16 bytes at
// i*1024 + l*16, i.e. token l%16 and dimension group 4*i + l/16: every load
// instruction covers 1 KiB of contiguous memory.  Each lane therefore owns
// one token and D/32 groups of 8 dimensions:
//   * q.k: each lane dots its own groups (v_dot2 fp16 pairs, fp32 sum); the
//     four lanes of a token (one per row of 16) are summed with the gfx950
//     permlane16/32 swaps, after which every row holds the 16 scores;
//   * softmax: block maximum by a 4-step DPP reduction inside a row;
//   * P.V: each lane adds p_t * v_t into its own D/4 fp32 accumulators; the
//     sum over the 16 tokens of a row is done once per partition.
// Masked positions (past the context in the last block) get score -inf and
// never touch the accumulators, so whatever those slots hold is never used.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pkv {
namespace {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) char* gptr;
typedef const __attribute__((address_space(1))) u4v* gu4v_ptr;

constexpr int kBlockTokens = 16;
constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_inff();

// Bit casts go through a by-value scalar: applied directly to a vector
// element (v.x, v[1]) __builtin_bit_cast reads element 0 with this clang.
__device__ __forceinline__ h2v as_h2(uint32_t u) { return __builtin_bit_cast(h2v, u); }
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

__device__ __forceinline__ float dot8(u4v a, u4v b, float c) {
  c = __builtin_amdgcn_fdot2(as_h2(a.x), as_h2(b.x), c, false);
  c = __builtin_amdgcn_fdot2(as_h2(a.y), as_h2(b.y), c, false);
  c = __builtin_amdgcn_fdot2(as_h2(a.z), as_h2(b.z), c, false);
  c = __builtin_amdgcn_fdot2(as_h2(a.w), as_h2(b.w), c, false);
  return c;
}

// DPP move inside a row of 16 lanes; every source lane is valid for the
// patterns used here.
template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, kCtrl, 0xF, 0xF, false);
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kMirror = 0x140;      // lane i <-> 15-i within 16

// Every lane of a row of 16 ends with the row's maximum / sum.  Each step
// combines two disjoint groups that already agree internally.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<kQuadXor1>(x));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  x = fmaxf(x, dpp<kHalfMirror>(x));
  x = fmaxf(x, dpp<kMirror>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kHalfMirror>(x);
  x += dpp<kMirror>(x);
  return x;
}

// Sum over the four rows: row pairs (0,1),(2,3) first, then halves.  The
// order is the same in every lane, so all rows end bit-identical.
__device__ __forceinline__ float cross_row_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  x = as_f32(a[0]) + as_f32(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return as_f32(b[0]) + as_f32(b[1]);
}

// A wave-uniform address kept in SGPRs, so that loads take the form
// "SGPR base + per-lane 32-bit offset".
// The result is a global (address space 1) pointer: a pointer rebuilt from
// integers would otherwise be generic and turn the loads into flat loads.
__device__ __forceinline__ gptr uniform_ptr(const char* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (gptr)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float wave_uniform(float x) {
  return as_f32(__builtin_amdgcn_readfirstlane(as_u32(x)));
}

template <int D>
struct Geometry {
  static constexpr int kLoads = D / 32;                      // 16-byte loads per lane per tile
  static constexpr int kTileBytes = D * kBlockTokens * 2;    // one (block, head) tile
  static constexpr int kAcc = kLoads * 8;                    // fp32 accumulators per lane
  static constexpr int kOutPerLane = kAcc / 16;              // outputs per lane after the row sum
};

template <int D>
struct Tile {
  u4v k[Geometry<D>::kLoads];
  u4v v[Geometry<D>::kLoads];
};

// One (block, head) tile of K and of V; `kbase`/`vbase` are wave-uniform
// tile addresses, `lane_off` = lane * 16.
template <int D>
__device__ __forceinline__ void load_tile(Tile<D>& t, gptr kbase, gptr vbase, uint32_t lane_off) {
#pragma unroll
  for (int i = 0; i < Geometry<D>::kLoads; ++i)
    t.k[i] = *reinterpret_cast<gu4v_ptr>(kbase + i * 1024 + lane_off);
#pragma unroll
  for (int i = 0; i < Geometry<D>::kLoads; ++i)
    t.v[i] = *reinterpret_cast<gu4v_ptr>(vbase + i * 1024 + lane_off);
}

__device__ __forceinline__ h8v as_h8(u4v x) { return __builtin_bit_cast(h8v, x); }

// Online-softmax update with one 16-token block.  With kMasked only the
// first `valid` tokens belong to the context (the sequence's partially
// filled last block); the others get score -inf and never reach the sums.
template <int D, bool kMasked>
__device__ __forceinline__ void consume(const Tile<D>& t, const u4v (&q)[Geometry<D>::kLoads],
                                        float scale_log2, int token, int valid, float& m,
                                        float& l, float (&acc)[Geometry<D>::kAcc]) {
  constexpr int L = Geometry<D>::kLoads;
  float part[L];
#pragma unroll
  for (int i = 0; i < L; ++i) part[i] = dot8(q[i], t.k[i], 0.0f);
  float s = part[0];
#pragma unroll
  for (int i = 1; i < L; ++i) s += part[i];
  s = cross_row_sum(s) * scale_log2;
  const bool live = !kMasked || token < valid;
  if (kMasked) s = live ? s : kNegInf;
  const float bmax = wave_uniform(row_max16(s));
  if (bmax > m) {                       // wave-uniform: the running maximum grows
    const float alpha = exp2f(m - bmax);
    l *= alpha;
#pragma unroll
    for (int j = 0; j < Geometry<D>::kAcc; ++j) acc[j] *= alpha;
    m = bmax;
  }
  if (live) {
    const float p = exp2f(s - m);
    l += p;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const h8v v = as_h8(t.v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i * 8 + e] = fmaf(p, (float)v[e], acc[i * 8 + e]);
    }
  }
}

template <int D>
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
    load_tile<D>(t, uniform_ptr(kpool + o), uniform_ptr(vpool + o), lane_off);
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

  // Sum over the 16 tokens of each row; every lane of a row then holds the
  // totals for its groups 4*i + row.
  l = row_sum16(l);
#pragma unroll
  for (int jj = 0; jj < kAcc; ++jj) acc[jj] = row_sum16(acc[jj]);

  // Lane `token` of row `row` writes values v = token*kOutPerLane + k of the
  // row's kAcc values: group 4*(v/8) + row, element v%8.
  float val[Geometry<D>::kOutPerLane];
#pragma unroll
  for (int k = 0; k < Geometry<D>::kOutPerLane; ++k) {
    const int v = token * Geometry<D>::kOutPerLane + k;
    float x = 0.0f;
#pragma unroll
    for (int jj = 0; jj < kAcc; ++jj) x = (jj == v) ? acc[jj] : x;
    val[k] = x;
  }
  const int v0 = token * Geometry<D>::kOutPerLane;
  const int d0 = (4 * (v0 / 8) + row) * 8 + v0 % 8;

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
  if (D == 128)
    hipLaunchKernelGGL(pa_decode_part_kernel<128>, dim3(grid_part), dim3(threads), 0, stream, part);
  else
    hipLaunchKernelGGL(pa_decode_part_kernel<64>, dim3(grid_part), dim3(threads), 0, stream, part);
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
