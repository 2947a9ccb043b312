// The two paging helpers for gfx950: slot-mapped append of new tokens and
// block-granular copy-on-write.  Both move bits only.
//
// Append ("Atención paginada en modelos de lenguaje grandes (LLM)",
// 7minutos.es, PagePool / PagedRequest part): a generated token is stored in
// the page its block table names.  One thread moves one 16-byte group (8
// dims of one head of one token) of K and the same group of V, with one of
// two lane mappings (layout [block][H][D/8][16][8]):
//  * a few tokens, each in its own block (a decode step): consecutive
//    lanes take consecutive groups of one token, so the source rows are
//    read fully coalesced (the destinations sit 256 bytes apart);
//  * many tokens (a prompt, a chunk): within a (head, group), 16 consecutive
//    tokens go to 16 consecutive lanes, so tokens at consecutive positions
//    of one block fill a whole 256-byte row of the tile per 16 lanes, and a
//    wave still reads 64 contiguous bytes of each source row.
//
// Copy-on-write (same page, prefix-sharing part; "PagedAttention",
// e-fortepiano.pl, "Descripció"): a shared page that must change is first
// duplicated whole.  One workgroup copies one block of one pool of one layer
// with 16-byte loads and stores, four in flight per thread.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pkv {
namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));
constexpr int kBlockTokens = 16;
// From this many tokens on, an append is taken to be runs of consecutive
// positions (a prompt or chunk) and uses the token-per-lane mapping.
constexpr int kAppendRunsFrom = 1024;

template <bool kRuns>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
  const int groups = a.D / 8;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  int t, h, c;
  if (kRuns) {
    const long long runs = (a.T + kBlockTokens - 1) / kBlockTokens;
    if (idx >= runs * kBlockTokens * a.H * groups) return;
    const int tin = (int)(idx % kBlockTokens);
    const long long rest = idx / kBlockTokens;
    c = (int)(rest % groups);
    h = (int)((rest / groups) % a.H);
    const long long t64 = (rest / ((long long)groups * a.H)) * kBlockTokens + tin;
    if (t64 >= a.T) return;
    t = (int)t64;
  } else {
    if (idx >= (long long)a.T * a.H * groups) return;
    c = (int)(idx % groups);
    h = (int)((idx / groups) % a.H);
    t = (int)(idx / ((long long)groups * a.H));
  }
  const int slot = a.slots[t];
  if (slot < 0) return;
  const int blk = slot / kBlockTokens;
  const int pos = slot % kBlockTokens;
  if (blk >= a.num_blocks) return;
  const size_t src = ((size_t)t * a.H + h) * a.D * 2 + (size_t)c * 16;
  const size_t dst = ((((size_t)blk * a.H + h) * groups + c) * kBlockTokens + pos) * 16;
  const u4v kv = *reinterpret_cast<const u4v*>(static_cast<const char*>(a.k) + src);
  const u4v vv = *reinterpret_cast<const u4v*>(static_cast<const char*>(a.v) + src);
  *reinterpret_cast<u4v*>(static_cast<char*>(a.k_pool) + dst) = kv;
  *reinterpret_cast<u4v*>(static_cast<char*>(a.v_pool) + dst) = vv;
}

__global__ __launch_bounds__(256) void cow_copy_kernel(CowArgs a) {
  const int which = blockIdx.x % 2;                 // 0: K pool, 1: V pool
  const int layer = (blockIdx.x / 2) % a.layers;
  const int pair = blockIdx.x / (2 * a.layers);
  const int src = a.pairs[2 * pair];
  const int dst = a.pairs[2 * pair + 1];
  if (src < 0 || dst < 0 || src >= a.num_blocks || dst >= a.num_blocks || src == dst) return;
  char* pool = static_cast<char*>(which ? a.v[layer] : a.k[layer]);
  const u4v* s = reinterpret_cast<const u4v*>(pool + (size_t)src * a.block_bytes);
  u4v* d = reinterpret_cast<u4v*>(pool + (size_t)dst * a.block_bytes);
  const long long n = a.block_bytes / 16;
  constexpr int kUnroll = 4;
  const long long stride = (long long)blockDim.x * kUnroll;
  long long i = threadIdx.x;
  for (; i + (kUnroll - 1) * (long long)blockDim.x < n; i += stride) {
    u4v r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) r[u] = s[i + u * blockDim.x];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) d[i + u * blockDim.x] = r[u];
  }
  for (; i < n; i += blockDim.x) d[i] = s[i];
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  const bool runs = a.T >= kAppendRunsFrom;
  const long long tokens = runs ? (a.T + kBlockTokens - 1) / kBlockTokens * kBlockTokens : a.T;
  const long long total = tokens * a.H * (a.D / 8);
  const int threads = 256;
  const long long grid = (total + threads - 1) / threads;
  if (runs)
    hipLaunchKernelGGL(kv_append_kernel<true>, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<false>, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_cow_copy(const CowArgs& a, hipStream_t stream) {
  const long long grid = (long long)a.n_pairs * a.layers * 2;
  hipLaunchKernelGGL(cow_copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
