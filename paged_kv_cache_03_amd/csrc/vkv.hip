// Contiguous KV cache in virtual memory with physical memory mapped on
// demand: the vAttention alternative to paging ("PagedAttention",
// e-fortepiano.pl, "Limitacions i alternatives" and "Atenció").  The K and
// V cache of every layer stays one contiguous virtual buffer of
// [max_batch][max_context][H][D] fp16, so an attention kernel for the plain
// contiguous layout reads it unchanged; physical memory is mapped into a
// request's part of each buffer, chunk by chunk, as its context grows.
//
// Built on the HIP virtual memory API (hipMemAddressReserve, hipMemCreate,
// hipMemMap, hipMemSetAccess).  Chunks of a released request are unmapped
// and kept in a pool for the next growth, so physical memory is created
// once.  A device array holds each request's readable tokens (its mapped
// rows, a multiple of 16); kernels clamp to it, so nothing ever reads an
// unmapped page.
//
// Host-side calls are synchronous and not thread-safe; release and destroy
// wait for the device first (a running kernel may still read the chunks).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <chrono>
#include <new>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr int kBlockTokens = PKV_BLOCK_TOKENS;

__global__ __launch_bounds__(256) void vkv_append_kernel(char* kbuf, char* vbuf, const char* k,
                                                         const char* v, const int32_t* seq_ids,
                                                         const int32_t* positions, int T,
                                                         const int32_t* capacity, int B,
                                                         long long seq_bytes, int row_bytes) {
  typedef uint32_t u4v __attribute__((ext_vector_type(4)));
  const int per_row = row_bytes / 16;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)T * per_row) return;
  const int t = (int)(idx / per_row);
  const int c = (int)(idx % per_row);
  const int seq = seq_ids[t];
  const int pos = positions[t];
  if (seq < 0 || seq >= B || pos < 0 || pos >= capacity[seq]) return;
  const size_t dst = (size_t)seq * seq_bytes + (size_t)pos * row_bytes + (size_t)c * 16;
  const size_t src = (size_t)t * row_bytes + (size_t)c * 16;
  *reinterpret_cast<u4v*>(kbuf + dst) = *reinterpret_cast<const u4v*>(k + src);
  *reinterpret_cast<u4v*>(vbuf + dst) = *reinterpret_cast<const u4v*>(v + src);
}

}  // namespace

struct pkv_vkv {
  int device = 0;
  int B = 0, L = 0, layers = 0, H = 0, D = 0;
  size_t row_bytes = 0;      // one token of one layer's K (or V): H * D * 2
  size_t seq_bytes = 0;      // one request's part of a buffer: L * row_bytes
  size_t chunk = 0;          // physical mapping unit
  size_t granularity = 0;
  std::vector<char*> base;   // 2 * layers buffers: K of layer l at 2l, V at 2l + 1
  // chunks[buffer][seq] = handles mapped, in order, from the request's start
  std::vector<std::vector<std::vector<hipMemGenericAllocationHandle_t>>> chunks;
  std::vector<int> mapped;   // chunks mapped per request (same in every buffer)
  std::vector<hipMemGenericAllocationHandle_t> pool;
  int32_t* d_capacity = nullptr;
  std::vector<int32_t> capacity;
  uint64_t map_calls = 0, created = 0;
  double map_seconds = 0.0;
};

namespace {

hipMemAllocationProp device_prop(int device) {
  hipMemAllocationProp prop = {};
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

// Tokens readable with `n` chunks mapped: whole rows, in groups of 16 (the
// decode reads 16-token tiles), at most L.
int32_t readable_tokens(const pkv_vkv* v, int n) {
  const size_t rows = (size_t)n * v->chunk / v->row_bytes;
  const size_t t = rows / kBlockTokens * kBlockTokens;
  return (int32_t)(t < (size_t)v->L ? t : (size_t)v->L);
}

int set_capacity(pkv_vkv* v, int seq, int32_t tokens) {
  v->capacity[seq] = tokens;
  return hipMemcpy(v->d_capacity + seq, &tokens, sizeof(int32_t), hipMemcpyHostToDevice) ==
                 hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

// Map chunk c of request seq in every buffer, or nothing.
int map_chunk(pkv_vkv* v, int seq, int c) {
  const hipMemAllocationProp prop = device_prop(v->device);
  hipMemAccessDesc access = {};
  access.location = prop.location;
  access.flags = hipMemAccessFlagsProtReadWrite;
  const auto t0 = std::chrono::steady_clock::now();
  size_t done = 0;
  int status = PKV_OK;
  for (; done < v->base.size(); ++done) {
    hipMemGenericAllocationHandle_t h;
    bool fresh = false;
    if (!v->pool.empty()) {
      h = v->pool.back();
      v->pool.pop_back();
    } else {
      if (hipMemCreate(&h, v->chunk, &prop, 0) != hipSuccess) { status = PKV_ERR_HIP; break; }
      fresh = true;
      ++v->created;
    }
    char* at = v->base[done] + (size_t)seq * v->seq_bytes + (size_t)c * v->chunk;
    if (hipMemMap(at, v->chunk, 0, h, 0) != hipSuccess) {
      if (fresh) (void)hipMemRelease(h); else v->pool.push_back(h);
      status = PKV_ERR_HIP;
      break;
    }
    if (hipMemSetAccess(at, v->chunk, &access, 1) != hipSuccess) {
      (void)hipMemUnmap(at, v->chunk);
      v->pool.push_back(h);
      status = PKV_ERR_HIP;
      break;
    }
    v->chunks[done][seq].push_back(h);
    ++v->map_calls;
  }
  if (status != PKV_OK) {              // undo the buffers already mapped for this chunk
    for (size_t b = 0; b < done; ++b) {
      char* at = v->base[b] + (size_t)seq * v->seq_bytes + (size_t)c * v->chunk;
      (void)hipMemUnmap(at, v->chunk);
      v->pool.push_back(v->chunks[b][seq].back());
      v->chunks[b][seq].pop_back();
    }
  }
  v->map_seconds += std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
  return status;
}

void unmap_all(pkv_vkv* v, int seq) {
  for (size_t b = 0; b < v->base.size(); ++b) {
    auto& hs = v->chunks[b][seq];
    for (size_t c = 0; c < hs.size(); ++c) {
      (void)hipMemUnmap(v->base[b] + (size_t)seq * v->seq_bytes + c * v->chunk, v->chunk);
      v->pool.push_back(hs[c]);
    }
    hs.clear();
  }
  v->mapped[seq] = 0;
}

}  // namespace

extern "C" {

int pkv_vkv_create(int32_t max_batch, int32_t max_context, int32_t num_layers, int32_t H,
                   int32_t D, size_t chunk_bytes, pkv_vkv** out) {
  if (!out) return PKV_ERR_NULL_PTR;
  *out = nullptr;
  if (max_batch <= 0 || max_context <= 0 || max_context % kBlockTokens || num_layers <= 0 ||
      H <= 0 || (D != 64 && D != 128) || chunk_bytes == 0 || (long long)H * D * 2 * 16 >= (1LL << 31))
    return PKV_ERR_BAD_SHAPE;
  const size_t row = (size_t)H * D * 2;
  const size_t seq_bytes = row * (size_t)max_context;
  if (seq_bytes % chunk_bytes) return PKV_ERR_BAD_SHAPE;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return PKV_ERR_HIP;
  const hipMemAllocationProp prop = device_prop(device);
  size_t gran = 0;
  if (hipMemGetAllocationGranularity(&gran, &prop, hipMemAllocationGranularityMinimum) !=
          hipSuccess || gran == 0)
    return PKV_ERR_HIP;
  if (chunk_bytes % gran) return PKV_ERR_BAD_SHAPE;
  pkv_vkv* v = new (std::nothrow) pkv_vkv;
  if (!v) return PKV_ERR_HIP;
  v->device = device;
  v->B = max_batch;
  v->L = max_context;
  v->layers = num_layers;
  v->H = H;
  v->D = D;
  v->row_bytes = row;
  v->seq_bytes = seq_bytes;
  v->chunk = chunk_bytes;
  v->granularity = gran;
  const size_t reserve = seq_bytes * (size_t)max_batch;
  for (int b = 0; b < 2 * num_layers; ++b) {
    void* p = nullptr;
    if (hipMemAddressReserve(&p, reserve, 0, nullptr, 0) != hipSuccess || !p ||
        reinterpret_cast<uintptr_t>(p) % gran) {
      if (p) (void)hipMemAddressFree(p, reserve);
      pkv_vkv_destroy(v);
      return PKV_ERR_HIP;
    }
    v->base.push_back(static_cast<char*>(p));
  }
  v->chunks.assign(v->base.size(),
                   std::vector<std::vector<hipMemGenericAllocationHandle_t>>(max_batch));
  v->mapped.assign(max_batch, 0);
  v->capacity.assign(max_batch, 0);
  if (hipMalloc(&v->d_capacity, sizeof(int32_t) * max_batch) != hipSuccess ||
      hipMemset(v->d_capacity, 0, sizeof(int32_t) * max_batch) != hipSuccess) {
    pkv_vkv_destroy(v);
    return PKV_ERR_HIP;
  }
  *out = v;
  return PKV_OK;
}

int pkv_vkv_destroy(pkv_vkv* v) {
  if (!v) return PKV_OK;
  (void)hipDeviceSynchronize();
  for (int s = 0; s < (int)v->mapped.size(); ++s) unmap_all(v, s);
  for (auto h : v->pool) (void)hipMemRelease(h);
  v->pool.clear();
  const size_t reserve = v->seq_bytes * (size_t)v->B;
  for (char* p : v->base) (void)hipMemAddressFree(p, reserve);
  if (v->d_capacity) (void)hipFree(v->d_capacity);
  delete v;
  return PKV_OK;
}

int pkv_vkv_grow(pkv_vkv* v, int32_t seq, int32_t tokens) {
  if (!v) return PKV_ERR_NULL_PTR;
  if (seq < 0 || seq >= v->B || tokens < 0 || tokens > v->L) return PKV_ERR_BAD_SHAPE;
  const size_t t16 = ((size_t)tokens + kBlockTokens - 1) / kBlockTokens * kBlockTokens;
  const int need = (int)((t16 * v->row_bytes + v->chunk - 1) / v->chunk);
  int status = PKV_OK;
  while (v->mapped[seq] < need) {
    status = map_chunk(v, seq, v->mapped[seq]);
    if (status != PKV_OK) break;
    ++v->mapped[seq];
  }
  // chunks are mapped before the readable count grows, so no reader can
  // run ahead of the mapping
  const int c = set_capacity(v, seq, readable_tokens(v, v->mapped[seq]));
  return status != PKV_OK ? status : c;
}

int pkv_vkv_release(pkv_vkv* v, int32_t seq) {
  if (!v) return PKV_ERR_NULL_PTR;
  if (seq < 0 || seq >= v->B) return PKV_ERR_BAD_SHAPE;
  if (hipDeviceSynchronize() != hipSuccess) return PKV_ERR_HIP;
  const int c = set_capacity(v, seq, 0);
  if (c != PKV_OK) return c;
  unmap_all(v, seq);
  return PKV_OK;
}

int pkv_vkv_buffers(const pkv_vkv* v, int32_t layer, void** k_buf, void** v_buf) {
  if (!v || !k_buf || !v_buf) return PKV_ERR_NULL_PTR;
  if (layer < 0 || layer >= v->layers) return PKV_ERR_BAD_SHAPE;
  *k_buf = v->base[2 * layer];
  *v_buf = v->base[2 * layer + 1];
  return PKV_OK;
}

const int32_t* pkv_vkv_capacity(const pkv_vkv* v) { return v ? v->d_capacity : nullptr; }

int pkv_vkv_stats(const pkv_vkv* v, pkv_vkv_info* info) {
  if (!v || !info) return PKV_ERR_NULL_PTR;
  uint64_t mapped = 0;
  for (int m : v->mapped) mapped += (uint64_t)m;
  info->mapped_bytes = mapped * v->chunk * v->base.size();
  info->pooled_bytes = (uint64_t)v->pool.size() * v->chunk;
  info->reserved_bytes = (uint64_t)v->seq_bytes * v->B * v->base.size();
  info->chunk_bytes = v->chunk;
  info->granularity = v->granularity;
  info->map_calls = v->map_calls;
  info->chunks_created = v->created;
  info->map_seconds = v->map_seconds;
  return PKV_OK;
}

int pkv_vkv_append(const pkv_vkv* v, int32_t layer, const void* k, const void* vv,
                   const int32_t* seq_ids, const int32_t* positions, int32_t T, void* stream) {
  if (!v) return PKV_ERR_NULL_PTR;
  if (layer < 0 || layer >= v->layers || T < 0) return PKV_ERR_BAD_SHAPE;
  if (T == 0) return PKV_OK;
  if (!k || !vv || !seq_ids || !positions) return PKV_ERR_NULL_PTR;
  if (reinterpret_cast<uintptr_t>(k) % 16 || reinterpret_cast<uintptr_t>(vv) % 16 ||
      reinterpret_cast<uintptr_t>(seq_ids) % 4 || reinterpret_cast<uintptr_t>(positions) % 4)
    return PKV_ERR_MISALIGNED;
  const long long threads = (long long)T * (long long)(v->row_bytes / 16);
  const long long grid = (threads + 255) / 256;
  if (grid >= (1LL << 31)) return PKV_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(vkv_append_kernel, dim3((unsigned)grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), v->base[2 * layer],
                     v->base[2 * layer + 1], static_cast<const char*>(k),
                     static_cast<const char*>(vv), seq_ids, positions, T, v->d_capacity, v->B,
                     (long long)v->seq_bytes, (int)v->row_bytes);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // extern "C"
