// Multi-query attention over one 16-token (block, head) tile on the gfx950
// matrix cores (internal), used by the grouped decode.
//
// A wave serves up to 16 query rows at once, one per MFMA column: lane l
// belongs to query column l%16 and to quarter tg = l/16.
//  * scores S^T (16 tokens x 16 queries) = K (16 x D) . Q^T (D x 16), one
//    v_mfma_f32_16x16x32_f16 per 32 dims.  The K tile as loaded (lane l:
//    token l%16, dims 32i + 8*tg .. +7) is exactly the A operand of the i-th
//    MFMA; the queries are the B operand (lane l: query l%16, same dims).
//    The result's lane l holds tokens 4*tg + r (r < 4) of query l%16.
//  * online softmax per query column: the four lanes l%16 + 16*tg hold one
//    query's 16 scores and are combined with permlane swaps; the reference
//    maximum lags (raised only past a slack), the weights are rounded to
//    fp16 once and the running sum uses the rounded weights.
//  * O^T (D x 16 queries) += V^T (D x 16 tokens) . P^T (16 tokens x 16
//    queries), one v_mfma_f32_16x16x16_f16 per 16 output dims.  P^T is the
//    score result's own layout; V^T is read back transposed from the wave's
//    LDS copy of the V tile with the gfx950 transpose read.  acc[s] lane l:
//    dims 16s + 4*tg + r of query l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_common.h"

namespace pkv {
namespace dev {

typedef _Float16 h4v __attribute__((ext_vector_type(4)));
typedef float f4v __attribute__((ext_vector_type(4)));

// Maximum over the four rows of 16 lanes (same pattern as cross_row_sum).
__device__ __forceinline__ float cross_row_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(as_u32(x), as_u32(x), false, false);
  x = fmaxf(as_f32(a[0]), as_f32(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(as_u32(x), as_u32(x), false, false);
  return fmaxf(as_f32(b[0]), as_f32(b[1]));
}

template <int D>
struct MTile {
  u4v k[D / 32];
  u4v v[D / 32];
};

// Loads one tile: load i of lane l takes token l%16, dims 32i + 8*(l/16)
// .. +7 of K and of V.  v_off is this lane's V offset: lane_off for a token
// inside the context, an offset past the buffer range (the load returns
// zeros) for one at or past it.
template <int D, int kPolicy>
__device__ __forceinline__ void mfma_fetch(MTile<D>& t, rsrc_t kr, rsrc_t vr, uint32_t lane_off,
                                           uint32_t v_off) {
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
    t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, lane_off + i * 1024, 0, kPolicy);
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
    t.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, v_off + i * 1024, 0, kPolicy);
}

// Slack of the reference maximum, in log2 units: the reference m is raised
// only when a tile's maximum exceeds it by more than this, so the weights
// exp2(s - m) stay below 2^8 (exact in fp16's range) and the accumulators
// are rescaled rarely; any reference gives the same result up to rounding
// (softmax is invariant to the shift), and the merge of partial results
// takes each piece's own reference.
constexpr float kGroupRescaleSlack = 8.0f;

// Scores and online-softmax step of one tile: k[i] are the K tile's A
// operands (lane l: token l%16, dims 32i + 8*tg ..).  live(tok) says whether
// token tok (0..15 of the tile) is attended by this lane's query column.
// pb receives the fp16 weights of this lane's tokens 4*tg + r (the P^T
// operand); when some query column's reference maximum moves, every lane's
// accumulators and sum are rescaled (by exactly 1 for the columns whose
// reference stays), behind one wave-uniform branch.
template <int D, typename Live>
__device__ __forceinline__ void mfma_scores(const u4v (&k)[D / 32], const h8v (&qb)[D / 32],
                                            float scale_log2, Live live, float& m, float& l,
                                            f4v (&acc)[D / 16], h4v& pb, int lane) {
  constexpr int kK = D / 32;
  const int tg = lane / 16;
  // two independent chains of score products, added at the end
  f4v s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kK; i += 2) {
    s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(k[i]), qb[i], s0, 0, 0, 0);
    if (i + 1 < kK)
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(k[i + 1]), qb[i + 1], s1, 0, 0, 0);
  }
  f4v sc;
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sc[r] = live(4 * tg + r) ? (s0[r] + s1[r]) * scale_log2 : kNegInf;
    mx = fmaxf(mx, sc[r]);
  }
  mx = cross_row_max(mx);
  const bool raise = mx > m + kGroupRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(raise)) {            // uniform: some column moves
    const float alpha = raise ? __builtin_amdgcn_exp2f(m - mx) : 1.0f;   // m = -inf: 0
    const float mnew = raise ? mx : m;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) acc[s] = acc[s] * alpha;
    l *= alpha;
    m = mnew;
  }
  const float mref = m == kNegInf ? 0.0f : m;
  float psum = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pb[r] = (_Float16)__builtin_amdgcn_exp2f(sc[r] - mref);   // masked: exp2(-inf) = 0
    psum += (float)pb[r];
  }
  l += psum;
}

// P.V step of one tile: vt points at the tile's V in LDS, in the tile's own
// [D/8][16][8] layout, with the slots past the context zero.  V^T for slice
// s comes from ds_read_b64_tr_b16: within each group of 16 lanes it returns
// to lane j, element e, element j%4 of the 8 bytes addressed by lane j/4 +
// 4e.  Lane i (= l%16) of group tg therefore addresses dims 16s + 4*(i%4) ..
// +3 of token 4*tg + i/4 (8 aligned bytes), and receives V[4*tg + e][16s +
// i], e < 4: the A operand (row = dim, k = token).
template <int D>
__device__ __forceinline__ void mfma_pv(f4v (&acc)[D / 16], h4v pb, const _Float16* vt,
                                        int lane) {
  typedef short s4v __attribute__((ext_vector_type(4)));
  const int qc = lane % 16;
  const int tg = lane / 16;
  const int tr_base = (((qc & 3) >> 1) * kBlockTokens + 4 * tg + (qc >> 2)) * 8 + 4 * (qc & 1);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const s4v raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4v*)(vt + tr_base + s * 2 * kBlockTokens * 8));
    acc[s] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4v, raw), pb, acc[s], 0,
                                                   0, 0);
  }
}

// One tile held in the wave's registers.  Tokens at or past the tile's
// valid count are not live, and their V values were loaded as zeros (a
// load past its buffer range returns 0), so that weight 0 never meets
// stale data (0 * NaN would be NaN).  sv / svh: the wave's own LDS area of
// D * 16 fp16 (the wave's LDS operations run in order, so no barrier is
// needed; the wavefront-scope fences, which emit no instruction, keep the
// compiler from moving the transpose reads, which take other lanes' data,
// across the writes).
template <int D, typename Live>
__device__ __forceinline__ void mfma_update(const MTile<D>& t, const h8v (&qb)[D / 32],
                                            float scale_log2, Live live, float& m, float& l,
                                            f4v (&acc)[D / 16], u4v* sv, const _Float16* svh,
                                            int lane) {
  h4v pb;
  mfma_scores<D>(t.k, qb, scale_log2, live, m, l, acc, pb, lane);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
  for (int i = 0; i < D / 32; ++i) sv[i * kWave + lane] = t.v[i];
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  mfma_pv<D>(acc, pb, svh, lane);
}

}  // namespace dev
}  // namespace pkv
