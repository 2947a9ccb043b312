// HBM bandwidth probes for gfx950: the rates that plain reads (and a plain
// copy) reach on this GPU, the references the kernels' traffic is compared
// with (the 8 TB/s figure is the published peak, which no kernel reaches).
//
//  * linear: a resident grid of workgroups walks the buffer in 16-byte
//    non-temporal loads, four independent loads in flight per thread per
//    step;
//  * gather: the buffer is cut into equal chunks that are read in a given
//    order (a random permutation stands for scattered pages), each wave
//    keeping 16 KiB in flight, the depth the decode's three-tile ring keeps;
//  * copy: every 16 bytes read are written to a second buffer (as many bytes
//    written as read, the mix of a step that reads its inputs once and writes
//    as much), each workgroup over a contiguous slice, non-temporal loads.
//
// The loaded words are folded into one value that is stored only if it
// equals a constant no real data produces, so the loads cannot be removed
// and nothing is written in practice.
//
// An LDS probe beside them: the rate at which one CU reads its LDS with the
// two read forms of the prefill's pair loop (16-byte reads of K rows, and
// the 8-byte transpose reads of V), conflict-free, so that the loop's LDS
// bytes per step can be set against what the CU can deliver.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "pagedkv.h"

namespace pkv {
namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));
constexpr uint32_t kNever = 0x9e3779b9u;
constexpr int kGatherPieces = 16;      // 1 KiB pieces (one load per lane) in flight per wave

__global__ __launch_bounds__(256) void hbm_read_probe_kernel(const u4v* __restrict__ p,
                                                             long long n16, uint32_t* sink) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u4v a = __builtin_nontemporal_load(p + i);
    const u4v b = __builtin_nontemporal_load(p + i + stride);
    const u4v c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u4v d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= (a.x ^ b.y) + (c.z ^ d.w) + (a.w ^ b.x) + (c.y ^ d.z);
  }
  for (; i < n16; i += stride) {
    const u4v a = __builtin_nontemporal_load(p + i);
    acc ^= a.x + a.w;
  }
  if (acc == kNever) *sink = acc;
}

// The buffer as n_chunks chunks of 2^log_kib KiB, read in the order of
// `order` (entries clamped to [0, n_chunks), so any order stays in bounds).
// The chunks' 1 KiB pieces, in that order, are numbered P = i * kib + j
// (chunk order[i], piece j); each wave takes kGatherPieces consecutive P at
// a time, one 16-byte load per lane each, all issued before any is used.
__global__ __launch_bounds__(256) void hbm_gather_probe_kernel(const u4v* __restrict__ p,
                                                               const int32_t* __restrict__ order,
                                                               long long n_pieces, int log_kib,
                                                               uint32_t* sink) {
  const int lane = threadIdx.x % 64;
  const long long wave = (long long)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  const long long waves = (long long)gridDim.x * (blockDim.x / 64);
  const long long kib_mask = (1ll << log_kib) - 1;
  const long long last_chunk = (n_pieces >> log_kib) - 1;
  uint32_t acc = 0;
  for (long long base = wave * kGatherPieces; base < n_pieces; base += waves * kGatherPieces) {
    u4v v[kGatherPieces];
#pragma unroll
    for (int k = 0; k < kGatherPieces; ++k) {
      const long long P = min(base + k, n_pieces - 1);
      const long long chunk = min(max((long long)order[P >> log_kib], 0ll), last_chunk);
      v[k] = __builtin_nontemporal_load(p + ((chunk << log_kib) + (P & kib_mask)) * 64 + lane);
    }
#pragma unroll
    for (int k = 0; k < kGatherPieces; ++k) acc ^= v[k].x + v[k].w;
  }
  if (acc == kNever) *sink = acc;
}

// Each workgroup copies its own contiguous slice of `per` units, 4 units per
// thread in flight (faster than a grid-stride walk of the whole buffer on
// this GPU: 5.3-5.4 against 4.4-5.1 TB/s read + write for 1 GiB).
__global__ __launch_bounds__(256) void hbm_copy_probe_kernel(const u4v* __restrict__ src,
                                                             u4v* __restrict__ dst,
                                                             long long n16, long long per) {
  const long long b0 = (long long)blockIdx.x * per;
  const long long b1 = b0 + per < n16 ? b0 + per : n16;
  for (long long i = b0 + threadIdx.x; i < b1; i += 4 * 256) {
    u4v v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const long long j = i + 256 * k;
      v[k] = j < b1 ? __builtin_nontemporal_load(src + j) : u4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const long long j = i + 256 * k;
      if (j < b1) dst[j] = v[k];
    }
  }
}

// 64 KiB of LDS per workgroup (within a larger dynamic allocation, so that
// one workgroup fits a CU), filled with a pattern, then read `rounds` times
// by every wave: form 0, 16-byte reads of whole 1 KiB rows (lane l reads
// bytes 16 l ..); form 1, the transpose reads of the prefill's value
// products (per 4 KiB V tile of 16 tokens x 128 dims: for each 32-dim
// slice, two reads of 8 bytes per lane at the loop's swizzled offsets).
// Each wave times its reads with the shader clock and stores the cycles
// and a fold of the data read.
__device__ __forceinline__ int lds_v_slot(int u) { return u ^ (4 * ((u >> 4) & 3)); }

__global__ __launch_bounds__(1024) void lds_read_probe_kernel(unsigned long long* cycles,
                                                              uint32_t* sink, int rounds,
                                                              int form) {
  typedef short s4v __attribute__((ext_vector_type(4)));
  extern __shared__ __attribute__((aligned(16))) u4v lds[];
  constexpr int kUnits = 64 * 1024 / 16;
  for (int i = threadIdx.x; i < kUnits; i += blockDim.x)
    lds[i] = u4v{(uint32_t)i, (uint32_t)i * 3u, (uint32_t)i ^ 0x5555u, (uint32_t)i + 7u};
  __syncthreads();
  const int lane = threadIdx.x % 64;
  const int wave = threadIdx.x / 64;
  const int qi = lane % 16, col = lane % 32, hf = lane / 32;
  const int g0 = 2 * (col / 16) + (qi & 3) / 2;
  // offsets in halves inside a V tile, as in the prefill's value products
  const int tr_lo = lds_v_slot(g0 * 16 + 4 * hf + (qi >> 2)) * 8 + 4 * (qi & 1);
  const int tr_hi = lds_v_slot(g0 * 16 + 8 + 4 * hf + (qi >> 2)) * 8 + 4 * (qi & 1);
  uint32_t acc = 0;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  if (form == 0) {
    for (int r = 0; r < rounds; ++r) {
      u4v v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = lds[((r * 16 + k + wave) & 63) * 64 + lane];
#pragma unroll
      for (int k = 0; k < 16; ++k) acc += v[k].x ^ v[k].w;
    }
  } else {
    const _Float16* h = reinterpret_cast<const _Float16*>(lds);
    for (int r = 0; r < rounds; ++r) {
      s4v v[16];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        // tile (r + k + wave) % 16 of the 16 tiles of 4 KiB, slice k % 4
        const _Float16* vt = h + ((r + k + wave) & 15) * 2048 + (k & 3) * 512;
        v[2 * k] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4v*)(vt + tr_lo));
        v[2 * k + 1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s4v*)(vt + tr_hi));
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) acc += (uint32_t)(uint16_t)v[k][0] ^ (uint32_t)(uint16_t)v[k][3];
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) {
    const int w = blockIdx.x * (blockDim.x / 64) + wave;
    cycles[w] = t1 - t0;
  }
  // one fold per wave, from lane 0's value (every lane's reads stay live)
  acc += __shfl_xor(acc, 1, 64);
  if (lane == 0) sink[blockIdx.x * (blockDim.x / 64) + wave] = acc;
}

}  // namespace

hipError_t launch_hbm_copy_probe(const void* src, void* dst, long long n16, int grid,
                                 hipStream_t stream) {
  const long long per = (n16 + grid - 1) / grid;
  hipLaunchKernelGGL(hbm_copy_probe_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<const u4v*>(src), static_cast<u4v*>(dst), n16, per);
  return hipGetLastError();
}

hipError_t launch_hbm_read_probe(const void* buf, long long n16, uint32_t* sink, int grid,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<const u4v*>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_hbm_gather_probe(const void* buf, const int32_t* order, long long n_chunks,
                                   int log_kib, uint32_t* sink, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(hbm_gather_probe_kernel, dim3(grid), dim3(256), 0, stream,
                     static_cast<const u4v*>(buf), order, n_chunks << log_kib, log_kib, sink);
  return hipGetLastError();
}

}  // namespace pkv

// The LDS probe's C entry lives here, beside its kernel (it is a measurement
// aid, not part of the attention path).
extern "C" int pkv_lds_read_probe(uint64_t* cycles, uint32_t* sink, int32_t workgroups,
                                  int32_t waves, int32_t rounds, int32_t form, void* stream) {
  if (workgroups <= 0 || waves < 1 || waves > 16 || rounds <= 0 || (form != 0 && form != 1))
    return PKV_ERR_BAD_SHAPE;
  if (!cycles || !sink) return PKV_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(cycles) % 8 || reinterpret_cast<uintptr_t>(sink) % 4)
    return PKV_ERR_MISALIGNED;
  // 96 KiB: one workgroup per CU (the probe reads the first 64 KiB)
  const int lds = 96 * 1024;
  if (hipFuncSetAttribute((const void*)pkv::lds_read_probe_kernel,
                          hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return PKV_ERR_HIP;
  hipLaunchKernelGGL(pkv::lds_read_probe_kernel, dim3(workgroups), dim3(64 * waves), lds,
                     static_cast<hipStream_t>(stream),
                     reinterpret_cast<unsigned long long*>(cycles), sink, rounds, form);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
