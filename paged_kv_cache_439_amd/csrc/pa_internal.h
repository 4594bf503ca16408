// Launch interface between the C-ABI layer (pa_api.cpp) and the kernels.
// Every argument here has already been validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct StoreArgs {
  const void* key;
  const void* value;
  int64_t key_stride_bytes;
  int64_t value_stride_bytes;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  int32_t num_tokens;
  int32_t row_bytes;       // num_kv_heads * head_dim * element size
  int64_t num_slots;       // num_blocks * block_size
};

struct StoreE4M3Args {
  const void* key;
  const void* value;
  int64_t key_stride_bytes;
  int64_t value_stride_bytes;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  const float* k_scale;
  const float* v_scale;
  int32_t num_tokens, num_kv_heads, head_dim;
  int64_t num_slots;       // num_blocks * block_size
  bool bf16;               // input type: bf16 (else fp32)
};

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* shared_lens;  // null: no sequence shares blocks (a load-policy hint)
  int32_t num_seqs, num_heads, num_kv_heads, head_dim;
  int32_t block_size, num_blocks, max_blocks_per_seq, max_context_len;
  float scale;
  int32_t partition_size;  // 0: no split
  void* workspace;
  bool bf16;
  // fused store (pa_store_decode); key == nullptr otherwise
  const void* key;
  const void* value;
  int64_t key_stride_bytes, value_stride_bytes;
  const int32_t* slot_mapping;
  // E4M3 pools (pa_decode_fp8): per-KV-head scales; kv_e4m3 false otherwise
  bool kv_e4m3;
  const float* k_scale;
  const float* v_scale;
};

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* query_start_loc;
  const int32_t* context_lens;
  int32_t num_seqs, num_heads, num_kv_heads, head_dim;
  int32_t block_size, num_blocks, max_blocks_per_seq, max_query_len, max_context_len;
  float scale;
  bool kv_e4m3 = false;             // pools hold E4M3 codes (pa_prefill_chunk_fp8)
  const float* k_scale = nullptr;   // E4M3: per-KV-head scales
  const float* v_scale = nullptr;
};

// partition_size value that selects the balanced split (pagedattn.h).
constexpr int32_t PA_PARTITION_BALANCED_VALUE = -1;

// Decode work split, shared by the workspace-size query and the launcher.
struct DecodePlan {
  int32_t group;           // query heads per KV head
  int32_t heads_per_unit;  // query heads one wave handles (divides group)
  int32_t units;           // waves per (sequence, partition) = Hkv * group / heads_per_unit
  int32_t partition;       // tokens per partition (> 0)
  int32_t max_parts;       // partitions of the longest context
  bool balanced;           // balanced split: equal chunk ranges per worker
  bool pair;               // balanced split over E4M3 pools, head_dim 64, one query head per KV
                           // head: a unit is a pair of adjacent KV heads (units = Hkv / 2)
  int32_t workers;         // balanced split: workers (waves) per unit
  size_t acc_bytes, ml_bytes, pfx_bytes, total_bytes;  // workspace regions (0 if unsplit)
};

DecodePlan plan_decode(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                       bool kv_e4m3 = false);

hipError_t launch_store(const StoreArgs& a, hipStream_t stream);
hipError_t launch_store_e4m3(const StoreE4M3Args& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& plan, hipStream_t stream);

// pa_decode_noalloc: the bytes of the static per-GPU scratch array
// (decode.hip), the devices it serves, and its address on the current
// device (looked up once per device with hipGetSymbolAddress, then kept).
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(16) << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

// pa_stream_read (stream_probe.hip): waves it launches on the current
// device, the smallest buffer it takes, and the launch (bytes_read: the
// bytes one launch reads, a whole number of per-wave slices).
int64_t stream_read_waves();
int64_t stream_read_min_bytes();
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, size_t* bytes_read,
                              hipStream_t stream);
// a describes the whole batch; its first num_decode sequences are decode
// tokens (workspace: the balanced decode workspace for num_decode sequences).
hipError_t launch_mixed(const PrefillArgs& a, int32_t num_decode, const int32_t* shared_lens,
                        void* workspace, hipStream_t stream);

}  // namespace pa
