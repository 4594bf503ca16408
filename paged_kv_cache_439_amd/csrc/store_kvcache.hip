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

// ---------------------------------------------------------------------------
// E4M3 store: quantise on the way into the pool
// ---------------------------------------------------------------------------
//
// Element x of KV head h is stored as the E4M3 code nearest to x / scale[h]
// (one IEEE fp32 division, ties to the even code), magnitudes saturated at
// 448, the largest finite E4M3 value; NaN becomes the NaN code 0x7F with the
// input's sign. One thread converts 16 consecutive elements of one head into
// one 16-byte piece of the pool row.
//
// Bound: HBM bytes (read 2 rows of the input type, write 2 rows of codes).

template <typename T>
__global__ __launch_bounds__(256) void store_kvcache_e4m3_kernel(
    const char* __restrict__ key, const char* __restrict__ value, int64_t key_stride,
    int64_t value_stride, char* __restrict__ k_cache, char* __restrict__ v_cache,
    const int32_t* __restrict__ slot_mapping, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, int64_t total_pieces, int32_t pieces_per_row,
    int32_t pieces_per_head, int64_t num_slots) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_pieces) return;
  const int64_t t = idx / pieces_per_row;
  const int32_t c = (int32_t)(idx - t * pieces_per_row);
  const int32_t s = slot_mapping[t];
  if (s < 0 || (int64_t)s >= num_slots) return;  // padding, or outside the pool
  const int32_t h = c / pieces_per_head;
  const int64_t src = (int64_t)c * 16 * (int64_t)sizeof(T);
  const uint4 kq = quantize16<T>(key + t * key_stride + src, k_scale[h]);
  const uint4 vq = quantize16<T>(value + t * value_stride + src, v_scale[h]);
  const int64_t dst = (int64_t)s * pieces_per_row * 16 + (int64_t)c * 16;
  *reinterpret_cast<uint4*>(k_cache + dst) = kq;
  *reinterpret_cast<uint4*>(v_cache + dst) = vq;
}

hipError_t launch_store_e4m3(const StoreE4M3Args& a, hipStream_t stream) {
  const int32_t ppr = a.num_kv_heads * a.head_dim / 16;
  const int64_t total = (int64_t)a.num_tokens * ppr;
  const int64_t blocks = (total + 255) / 256;
  const char* key = static_cast<const char*>(a.key);
  const char* value = static_cast<const char*>(a.value);
  char* kc = static_cast<char*>(a.k_cache);
  char* vc = static_cast<char*>(a.v_cache);
  if (a.bf16)
    hipLaunchKernelGGL(store_kvcache_e4m3_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       key, value, a.key_stride_bytes, a.value_stride_bytes, kc, vc, a.slot_mapping,
                       a.k_scale, a.v_scale, total, ppr, a.head_dim / 16, a.num_slots);
  else
    hipLaunchKernelGGL(store_kvcache_e4m3_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       key, value, a.key_stride_bytes, a.value_stride_bytes, kc, vc, a.slot_mapping,
                       a.k_scale, a.v_scale, total, ppr, a.head_dim / 16, a.num_slots);
  return hipGetLastError();
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
