// Multi-query attention over one 16-token (block, head) tile on the gfx950
// matrix cores (internal), shared by the grouped decode and the prefill.
//
// A wave serves up to 16 query rows at once, one per MFMA column: lane l
// belongs to query column l%16 and to quarter tg = l/16.
//  * scores S^T (16 tokens x 16 queries) = K (16 x D) . Q^T (D x 16), one
//    v_mfma_f32_16x16x32_f16 per 32 dims.  The K tile as loaded (lane l:
//    token l%16, dims 32i + 8*tg .. +7) is exactly the A operand of the i-th
//    MFMA; the queries are the B operand (lane l: query l%16, same dims).
//    The result's lane l holds tokens 4*tg + r (r < 4) of query l%16.
//  * online softmax per query column: the four lanes l%16 + 16*tg hold one
//    query's 16 scores and are combined with permlane swaps; the weights are
//    rounded to fp16 once and the running sum uses the rounded weights.
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

template <int D, int kPolicy>
__device__ __forceinline__ void mfma_fetch(MTile<D>& t, rsrc_t kr, rsrc_t vr, uint32_t lane_off) {
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
    t.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, lane_off + i * 1024, 0, kPolicy);
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
    t.v[i] = __builtin_amdgcn_raw_buffer_load_b128(vr, lane_off + i * 1024, 0, kPolicy);
}

// Scores and online-softmax step of one tile: k[i] are the K tile's A
// operands (lane l: token l%16, dims 32i + 8*tg ..).  live(tok) says whether
// token tok (0..15 of the tile) is attended by this lane's query column.
// Returns the rescale factor of the running sums; pb receives the fp16
// weights of this lane's tokens 4*tg + r (the P^T operand).
template <int D, typename Live>
__device__ __forceinline__ float mfma_scores(const u4v (&k)[D / 32], const h8v (&qb)[D / 32],
                                             float scale_log2, Live live, float& m, float& l,
                                             h4v& pb, int lane) {
  constexpr int kK = D / 32;
  const int tg = lane / 16;
  f4v sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kK; ++i)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(k[i]), qb[i], sc, 0, 0, 0);
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sc[r] = live(4 * tg + r) ? sc[r] * scale_log2 : kNegInf;
    mx = fmaxf(mx, sc[r]);
  }
  const float mnew = fmaxf(m, cross_row_max(mx));
  const float mref = mnew == kNegInf ? 0.0f : mnew;
  const float alpha = exp2f(m - mref);
  float psum = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pb[r] = (_Float16)exp2f(sc[r] - mref);
    psum += (float)pb[r];
  }
  l = fmaf(l, alpha, psum);
  m = mnew;
  return alpha;
}

// P.V step of one tile: vt points at the tile's V in LDS, in the tile's own
// [D/8][16][8] layout, with the slots past the context already zeroed.
// V^T for slice s comes from ds_read_b64_tr_b16: within each group of 16
// lanes it returns to lane j, element e, element j%4 of the 8 bytes
// addressed by lane j/4 + 4e.  Lane i (= l%16) of group tg therefore
// addresses dims 16s + 4*(i%4) .. +3 of token 4*tg + i/4 (8 aligned bytes),
// and receives V[4*tg + e][16s + i], e < 4: the A operand (row = dim, k =
// token).
template <int D>
__device__ __forceinline__ void mfma_pv(f4v (&acc)[D / 16], float alpha, h4v pb,
                                        const _Float16* vt, int lane) {
  typedef short s4v __attribute__((ext_vector_type(4)));
  const int qc = lane % 16;
  const int tg = lane / 16;
  const int tr_base = (((qc & 3) >> 1) * kBlockTokens + 4 * tg + (qc >> 2)) * 8 + 4 * (qc & 1);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const s4v raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4v*)(vt + tr_base + s * 2 * kBlockTokens * 8));
    const h4v va = __builtin_bit_cast(h4v, raw);
    acc[s] = acc[s] * alpha;
    acc[s] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pb, acc[s], 0, 0, 0);
  }
}

// Two tiles a, b (32 tokens) at once, for the P.V product on the full-rate
// v_mfma_f32_16x16x32_f16: its 32 k slots are ordered so that lane quarter
// tg's 8 slots are tokens 4*tg .. 4*tg+3 of tile a, then the same tokens of
// tile b.  The P^T operand is then the two score results side by side, and
// V^T is two transpose reads (one per tile) side by side; the order is the
// same for both operands, so the product is the plain sum over the 32
// tokens.  live_a / live_b: as `live` of mfma_scores for each tile.
template <int D, typename LiveA, typename LiveB>
__device__ __forceinline__ void mfma_update_pair(const u4v (&ka)[D / 32], const u4v (&kb)[D / 32],
                                                 const h8v (&qb)[D / 32], float scale_log2,
                                                 LiveA live_a, LiveB live_b, float& m, float& l,
                                                 f4v (&acc)[D / 16], const _Float16* vta,
                                                 const _Float16* vtb, int lane) {
  typedef short s4v __attribute__((ext_vector_type(4)));
  typedef short s8v __attribute__((ext_vector_type(8)));
  constexpr int kK = D / 32;
  const int qc = lane % 16;
  const int tg = lane / 16;
  f4v sa = {0.0f, 0.0f, 0.0f, 0.0f};
  f4v sb = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kK; ++i) {
    sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(ka[i]), qb[i], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(kb[i]), qb[i], sb, 0, 0, 0);
  }
  float mx = kNegInf;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sa[r] = live_a(4 * tg + r) ? sa[r] * scale_log2 : kNegInf;
    sb[r] = live_b(4 * tg + r) ? sb[r] * scale_log2 : kNegInf;
    mx = fmaxf(mx, fmaxf(sa[r], sb[r]));
  }
  const float mnew = fmaxf(m, cross_row_max(mx));
  const float mref = mnew == kNegInf ? 0.0f : mnew;
  const float alpha = exp2f(m - mref);
  h8v pb;
  float psum = 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pb[r] = (_Float16)exp2f(sa[r] - mref);
    pb[4 + r] = (_Float16)exp2f(sb[r] - mref);
    psum += (float)pb[r] + (float)pb[4 + r];
  }
  l = fmaf(l, alpha, psum);
  m = mnew;
  const int tr_base = (((qc & 3) >> 1) * kBlockTokens + 4 * tg + (qc >> 2)) * 8 + 4 * (qc & 1);
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const int off = tr_base + s * 2 * kBlockTokens * 8;
    const s4v ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4v*)(vta + off));
    const s4v rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4v*)(vtb + off));
    const s8v both = {ra[0], ra[1], ra[2], ra[3], rb[0], rb[1], rb[2], rb[3]};
    acc[s] = acc[s] * alpha;
    acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8v, both), pb, acc[s],
                                                    0, 0, 0);
  }
}

// One tile held in the wave's registers.  Tokens at or past `valid` hold no
// data and must not be live; their V rows are zeroed before use (they may
// hold anything, NaN included, and weight 0 * NaN would still be NaN).
// sv / svh: the wave's own LDS area of D * 16 fp16 (the wave's LDS
// operations run in order, so no barrier is needed; the wavefront-scope
// fences, which emit no instruction, keep the compiler from moving the
// transpose reads, which take other lanes' data, across the writes).
template <int D, typename Live>
__device__ __forceinline__ void mfma_update(const MTile<D>& t, const h8v (&qb)[D / 32],
                                            float scale_log2, int valid, Live live, float& m,
                                            float& l, f4v (&acc)[D / 16], u4v* sv,
                                            const _Float16* svh, int lane) {
  h4v pb;
  const float alpha = mfma_scores<D>(t.k, qb, scale_log2, live, m, l, pb, lane);
  const bool tok_ok = lane % 16 < valid;     // this lane's loaded token is l % 16
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    u4v w = t.v[i];
    w.x = tok_ok ? w.x : 0u;
    w.y = tok_ok ? w.y : 0u;
    w.z = tok_ok ? w.z : 0u;
    w.w = tok_ok ? w.w : 0u;
    sv[i * kWave + lane] = w;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  mfma_pv<D>(acc, alpha, pb, svh, lane);
}

}  // namespace dev
}  // namespace pkv
