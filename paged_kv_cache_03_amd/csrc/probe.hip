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

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

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
