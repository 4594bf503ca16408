// store_kvcache: scatter new K/V rows into the block pools by slot.
//
// The mini-vllm page ("mini-vllm：基于 NanoGPT 的 PagedAttention 风格 KV 缓存
// 管理实现", architecture item 2 "KVCache") writes each new token's K/V at
// the pool location its block table names. With the pool laid out as
// [num_blocks][block_size][Hkv][D], slot s = block*block_size + row is simply
// row s of the pool viewed as [num_blocks*block_size] rows, so the kernel is a
// row copy. One thread moves one 16-byte chunk of a row for both K and V;
// consecutive threads cover consecutive chunks of a row, so every wave reads
// and writes whole rows with 16-byte accesses.
//
// Bound: HBM bytes (read 2 rows, write 2 rows per token).

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

__global__ __launch_bounds__(256) void store_kvcache_kernel(
    const char* __restrict__ key, const char* __restrict__ value, int64_t key_stride,
    int64_t value_stride, char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, int64_t total_chunks, int32_t chunks_per_row,
    int64_t num_slots) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_chunks) return;
  const int64_t t = idx / chunks_per_row;
  const int32_t c = (int32_t)(idx - t * chunks_per_row);
  const int32_t s = slot_mapping[t];
  if (s < 0 || (int64_t)s >= num_slots) return;  // padding, or outside the pool
  const int64_t row_bytes = (int64_t)chunks_per_row * 16;
  const uint4 kv = *reinterpret_cast<const uint4*>(key + t * key_stride + (int64_t)c * 16);
  const uint4 vv = *reinterpret_cast<const uint4*>(value + t * value_stride + (int64_t)c * 16);
  *reinterpret_cast<uint4*>(k_cache + (int64_t)s * row_bytes + (int64_t)c * 16) = kv;
  *reinterpret_cast<uint4*>(v_cache + (int64_t)s * row_bytes + (int64_t)c * 16) = vv;
}

hipError_t launch_store(const StoreArgs& a, hipStream_t stream) {
  const int32_t cpr = a.row_bytes / 16;
  const int64_t total = (int64_t)a.num_tokens * cpr;
  const int64_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(store_kvcache_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const char*>(a.key), static_cast<const char*>(a.value),
                     a.key_stride_bytes, a.value_stride_bytes, static_cast<char*>(a.k_cache),
                     static_cast<char*>(a.v_cache), a.slot_mapping, total, cpr, a.num_slots);
  return hipGetLastError();
}

}  // namespace pa
