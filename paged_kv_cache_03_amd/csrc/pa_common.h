// Device-side building blocks shared by the decode kernels (internal).
//
// Lane mapping inside one (block, head) tile.  A tile is D/8 groups x 16
// tokens x 8 values (fp16).  Load i of lane l reads the 16 bytes at
// i*1024 + l*16, i.e. token l%16 and dimension group 4*i + l/16: every load
// instruction covers 1 KiB of contiguous memory.  Each lane therefore owns
// one token and D/32 groups of 8 dimensions:
//   * q.k: each lane dots its own groups (v_dot2 fp16 pairs, fp32 sum); the
//     four lanes of a token (one per row of 16) are summed with the gfx950
//     permlane16/32 swaps, after which every row holds the 16 scores;
//   * softmax: block maximum by a 4-step DPP reduction inside a row, kept
//     in log2 units (the scale is pre-multiplied by log2(e), exp2 is used);
//   * P.V: each lane adds p_t * v_t into its own D/4 fp32 accumulators; the
//     sum over the 16 tokens of a row is done once per run of blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pkv {
namespace dev {


typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) char* gptr;
typedef const __attribute__((address_space(1))) u4v* gu4v_ptr;
typedef __attribute__((address_space(1))) char* gptr_mut;

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

__device__ __forceinline__ gptr_mut uniform_ptr_mut(void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (gptr_mut)(((uint64_t)hi << 32) | lo);
}

// Buffer resources: a wave-uniform base and byte size in SGPRs, addressed
// with a per-lane VGPR offset.  Accesses past the size read 0 / are dropped.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferFlags = 0x00020000;   // 32-bit data format; untyped access

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(static_cast<const char*>(base)),
                                          (short)0, (int)bytes, kBufferFlags);
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

// One (block, head) tile of K and of V through buffer resources covering
// the two tiles; load i of a lane reads at lane_off + i * kLoadStride.  In
// the paged layout lane_off = lane * 16 and the stride is 1024; in a
// contiguous [token][H][D] layout lane_off = (lane % 16) * row bytes +
// (lane / 16) * 16 and the stride is 64.  Either way load i of lane l holds
// token l % 16, dims 8 * (4i + l/16) .. +7.
// kPolicy: cache-policy bits of the loads (kStreamPolicy or 0).
template <int D, int kPolicy, int kLoadStride = 1024>
__device__ __forceinline__ void load_tile(Tile<D>& t, rsrc_t kr, rsrc_t vr, uint32_t lane_off) {
#pragma unroll
  for (int i = 0; i < Geometry<D>::kLoads; ++i)
    t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, lane_off + i * kLoadStride, 0, kPolicy);
#pragma unroll
  for (int i = 0; i < Geometry<D>::kLoads; ++i)
    t.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, lane_off + i * kLoadStride, 0, kPolicy);
}

__device__ __forceinline__ h8v as_h8(u4v x) { return __builtin_bit_cast(h8v, x); }

// Online-softmax update with one 16-token block.  With kMasked only the
// first `valid` tokens belong to the context (the sequence's partially
// filled last block): the others get score -inf, weight 0 and their values
// are replaced by 0 before use, so whatever those slots hold (NaN included)
// never reaches the sums.  No divergent branch: the load counters stay exact
// across the caller's loop.
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
  float p = exp2f(s - m);
  if (kMasked) p = live ? p : 0.0f;
  l += p;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    u4v w = t.v[i];
    if (kMasked) {
      w.x = live ? w.x : 0u;
      w.y = live ? w.y : 0u;
      w.z = live ? w.z : 0u;
      w.w = live ? w.w : 0u;
    }
    const h8v v = as_h8(w);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i * 8 + e] = fmaf(p, (float)v[e], acc[i * 8 + e]);
  }
}

// End of a run of blocks: sum (l, acc) over the 16 tokens of each row, then
// pick the values this lane stores.  Lane `token` of row `row` ends up with
// values v = token*kOutPerLane + k (k < kOutPerLane) of its row's kAcc sums,
// which are dims d0 + k with d0 = (4*(v0/8) + row)*8 + v0%8.
template <int D>
__device__ __forceinline__ int reduce_rows(float& l, float (&acc)[Geometry<D>::kAcc], int token,
                                           int row, float (&val)[Geometry<D>::kOutPerLane]) {
  constexpr int kAcc = Geometry<D>::kAcc;
  constexpr int kOut = Geometry<D>::kOutPerLane;
  l = row_sum16(l);
#pragma unroll
  for (int j = 0; j < kAcc; ++j) acc[j] = row_sum16(acc[j]);
#pragma unroll
  for (int k = 0; k < kOut; ++k) {
    const int v = token * kOut + k;
    float x = 0.0f;
#pragma unroll
    for (int j = 0; j < kAcc; ++j) x = (j == v) ? acc[j] : x;
    val[k] = x;
  }
  const int v0 = token * kOut;
  return (4 * (v0 / 8) + row) * 8 + v0 % 8;
}
}  // namespace dev
}  // namespace pkv
