// C-ABI entry points of libpagedattn: argument validation on the host, then
// the kernel launchers. No exception crosses the interface; every failure is
// a pa_status plus a per-thread message (pa_last_error).

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/pagedattn.h"
#include "pa_internal.h"

static_assert(PA_PARTITION_BALANCED == pa::PA_PARTITION_BALANCED_VALUE, "balanced split constant");

namespace {

thread_local char g_last_error[512] = "";

pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

pa_status ok() {
  g_last_error[0] = '\0';
  return PA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

int elem_size(pa_dtype d) { return d == PA_BF16 ? 2 : 4; }

pa_status check_dtype(pa_dtype d) {
  if (d != PA_F32 && d != PA_BF16) return fail(PA_ERR_INVALID_ARG, "unknown dtype %d", (int)d);
  return PA_OK;
}

// Shape checks shared by decode and prefill.
pa_status check_attention_shapes(int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks,
                                 int32_t max_blocks_per_seq, int32_t max_context_len) {
  if (num_heads <= 0 || num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "num_heads=%d num_kv_heads=%d must be positive", num_heads,
                num_kv_heads);
  if (num_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_heads=%d is not a multiple of num_kv_heads=%d",
                num_heads, num_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim=%d (supported: 64, 128)", head_dim);
  if (!pow2(block_size) || block_size < 8 || block_size > 1024)
    return fail(PA_ERR_UNSUPPORTED, "block_size=%d (supported: powers of two in [8, 1024])",
                block_size);
  if (num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks=%d must be positive", num_blocks);
  if (max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq=%d must be positive", max_blocks_per_seq);
  if (max_context_len <= 0)
    return fail(PA_ERR_INVALID_ARG, "max_context_len=%d must be positive", max_context_len);
  if ((int64_t)block_size * num_kv_heads * head_dim * 4 > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "a block of %lld elements per pool is too large",
                (long long)block_size * num_kv_heads * head_dim);
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PA_ERR_INVALID_ARG, "max_context_len=%d exceeds max_blocks_per_seq*block_size=%lld",
                max_context_len, (long long)max_blocks_per_seq * block_size);
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
  }
  return "PA_UNKNOWN_STATUS";
}

const char* pa_last_error(void) { return g_last_error; }

pa_status pa_store_kvcache(const void* key, const void* value, int64_t key_tok_stride,
                           int64_t value_tok_stride, void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           pa_dtype dtype, void* stream) {
  try {
    if (pa_status st = check_dtype(dtype)) return st;
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens=%d is negative", num_tokens);
    if (num_tokens == 0) return ok();
    if (!key || !value || !k_cache || !v_cache || !slot_mapping)
      return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
      return fail(PA_ERR_INVALID_ARG, "num_kv_heads, head_dim, block_size, num_blocks must be positive");
    const int e = elem_size(dtype);
    const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
    const int64_t row_bytes = row_elems * e;
    if (row_bytes % 16 != 0 || row_bytes > (1 << 20))
      return fail(PA_ERR_UNSUPPORTED, "row of %lld bytes (needs a multiple of 16, at most 1 MiB)",
                  (long long)row_bytes);
    if (key_tok_stride < row_elems || value_tok_stride < row_elems)
      return fail(PA_ERR_INVALID_ARG, "token strides (%lld, %lld) below a row of %lld elements",
                  (long long)key_tok_stride, (long long)value_tok_stride, (long long)row_elems);
    if ((key_tok_stride * e) % 16 || (value_tok_stride * e) % 16)
      return fail(PA_ERR_UNSUPPORTED, "token strides must be multiples of 16 bytes");
    if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(slot_mapping, 4))
      return fail(PA_ERR_UNSUPPORTED, "pointers must be 16-byte aligned (slot_mapping 4-byte)");
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    if (num_slots > INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, "num_blocks*block_size=%lld exceeds int32 slots",
                  (long long)num_slots);
    if ((int64_t)num_tokens * (row_bytes / 16) > (int64_t)INT32_MAX)
      return fail(PA_ERR_UNSUPPORTED, "too many tokens in one call");
    pa::StoreArgs a{key, value, key_tok_stride * e, value_tok_stride * e, k_cache, v_cache,
                    slot_mapping, num_tokens, (int32_t)row_bytes, num_slots};
    const hipError_t err = pa::launch_store(a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(PA_ERR_HIP, "store launch: %s", hipGetErrorString(err));
    return ok();
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

size_t pa_decode_workspace_size_kv(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t max_context_len,
                                   int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || num_kv_heads <= 0 || num_heads % num_kv_heads ||
      head_dim <= 0 || max_context_len <= 0 ||
      (partition_size < 0 && partition_size != PA_PARTITION_BALANCED))
    return 0;
  // the larger of the two plans: over E4M3 pools the balanced split may pair
  // KV heads, which doubles its workers (the same call serves pa_decode_fp8)
  return std::max(pa::plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                                  partition_size, false)
                      .total_bytes,
                  pa::plan_decode(num_seqs, num_heads, num_kv_heads, head_dim, max_context_len,
                                  partition_size, true)
                      .total_bytes);
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t partition_size) {
  // every grouping a call may use: the largest plan over the KV head counts
  // that divide num_heads
  size_t most = 0;
  for (int32_t hkv = 1; hkv > 0 && hkv <= num_heads; ++hkv)
    if (num_heads % hkv == 0)
      most = std::max(most, pa_decode_workspace_size_kv(num_seqs, num_heads, hkv, head_dim,
                                                        max_context_len, partition_size));
  return most;
}

}  // extern "C"

namespace {

// Shared by pa_decode and pa_store_decode: validation, planning, launch.
// fused == nullptr for a plain decode.
struct Fusion {
  const void* key;
  const void* value;
  int64_t key_tok_stride, value_tok_stride;  // elements
  const int32_t* slot_mapping;
};

// E4M3 pools (pa_decode_fp8): per-KV-head scales.
struct E4M3Scales {
  const float* k_scale;
  const float* v_scale;
};

pa_status decode_impl(const char* fn, void* out, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* shared_lens, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                      int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                      size_t workspace_bytes, pa_dtype dtype, void* stream, const Fusion* fused,
                      const E4M3Scales* e4m3, bool noalloc = false) {
  if (pa_status st = check_dtype(dtype)) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_seqs=%d is negative", fn, num_seqs);
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (pa_status st = check_attention_shapes(num_heads, num_kv_heads, head_dim, block_size,
                                            num_blocks, max_blocks_per_seq, max_context_len))
    return st;
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "%s: num_seqs=%d above 65535", fn, num_seqs);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (partition_size != PA_PARTITION_BALANCED && (partition_size < 0 || partition_size % 16 != 0))
    return fail(PA_ERR_INVALID_ARG,
                "%s: partition_size=%d must be 0, a positive multiple of 16 or PA_PARTITION_BALANCED",
                fn, partition_size);
  if (partition_size == PA_PARTITION_BALANCED && num_seqs > 4096)
    return fail(PA_ERR_UNSUPPORTED, "%s: the balanced split supports at most 4096 sequences (got %d)",
                fn, num_seqs);
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(shared_lens, 4))
    return fail(PA_ERR_UNSUPPORTED, "%s: pointers must be 16-byte aligned (int arrays 4-byte)", fn);
  const int e = elem_size(dtype);
  if (fused) {
    const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
    if (!fused->key || !fused->value || !fused->slot_mapping)
      return fail(PA_ERR_INVALID_ARG, "%s: null key, value or slot_mapping", fn);
    if (fused->key_tok_stride < row_elems || fused->value_tok_stride < row_elems)
      return fail(PA_ERR_INVALID_ARG, "%s: token strides (%lld, %lld) below a row of %lld elements", fn,
                  (long long)fused->key_tok_stride, (long long)fused->value_tok_stride,
                  (long long)row_elems);
    if ((fused->key_tok_stride * e) % 16 || (fused->value_tok_stride * e) % 16)
      return fail(PA_ERR_UNSUPPORTED, "%s: token strides must be multiples of 16 bytes", fn);
    if (!aligned(fused->key, 16) || !aligned(fused->value, 16) || !aligned(fused->slot_mapping, 4))
      return fail(PA_ERR_UNSUPPORTED, "%s: key/value must be 16-byte aligned, slot_mapping 4-byte", fn);
    if ((int64_t)num_blocks * block_size > INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, "%s: num_blocks*block_size=%lld exceeds int32 slots", fn,
                  (long long)num_blocks * block_size);
  }
  if (e4m3) {
    if (fused && dtype != PA_BF16)
      return fail(PA_ERR_UNSUPPORTED, "%s: the fused E4M3 store takes bf16 queries only", fn);
    if (!e4m3->k_scale || !e4m3->v_scale)
      return fail(PA_ERR_INVALID_ARG, "%s: null k_scale or v_scale", fn);
    if (!aligned(e4m3->k_scale, 4) || !aligned(e4m3->v_scale, 4))
      return fail(PA_ERR_UNSUPPORTED, "%s: k_scale/v_scale must be 4-byte aligned", fn);
  }
  const pa::DecodePlan plan = pa::plan_decode(num_seqs, num_heads, num_kv_heads, head_dim,
                                              max_context_len, partition_size, e4m3 != nullptr);
  if ((plan.units + 3) / 4 > 65535) return fail(PA_ERR_UNSUPPORTED, "%s: too many heads", fn);
  if (plan.max_parts > 65535)  // a grid dimension of the fixed split
    return fail(PA_ERR_UNSUPPORTED, "%s: %d partitions of %d tokens (at most 65535)", fn, plan.max_parts,
                partition_size);
  if (noalloc) {
    // pa_decode_noalloc: the library's static scratch is the workspace
    if (plan.total_bytes > pa::NOALLOC_SCRATCH_BYTES)
      return fail(PA_ERR_WORKSPACE,
                  "%s: this split needs %zu bytes of scratch; the static scratch holds %zu (use "
                  "pa_decode with a workspace, or a larger partition_size)",
                  fn, plan.total_bytes, pa::NOALLOC_SCRATCH_BYTES);
    workspace = nullptr;
    workspace_bytes = 0;
    if (plan.total_bytes) {
      const hipError_t err = pa::noalloc_scratch(&workspace);
      if (err != hipSuccess) return fail(PA_ERR_HIP, "%s: scratch lookup: %s", fn, hipGetErrorString(err));
      workspace_bytes = pa::NOALLOC_SCRATCH_BYTES;
    }
  }
  if (plan.total_bytes) {
    if (!workspace)
      return fail(PA_ERR_WORKSPACE, "%s: this split needs a workspace of %zu bytes", fn,
                  plan.total_bytes);
    if (workspace_bytes < plan.total_bytes)
      return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                  plan.total_bytes);
    if (!aligned(workspace, 256))
      return fail(PA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  }
  pa::DecodeArgs a{out, q, k_cache, v_cache, block_tables, context_lens, shared_lens, num_seqs, num_heads,
                   num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                   max_context_len, scale, partition_size, workspace, dtype == PA_BF16,
                   nullptr, nullptr, 0, 0, nullptr, e4m3 != nullptr,
                   e4m3 ? e4m3->k_scale : nullptr, e4m3 ? e4m3->v_scale : nullptr};
  if (fused) {
    a.key = fused->key;
    a.value = fused->value;
    a.key_stride_bytes = fused->key_tok_stride * e;
    a.value_stride_bytes = fused->value_tok_stride * e;
    a.slot_mapping = fused->slot_mapping;
  }
  const hipError_t err = pa::launch_decode(a, plan, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(PA_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(err));
  return ok();
}

}  // namespace

extern "C" {

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                    float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                    pa_dtype dtype, void* stream) {
  try {
    return decode_impl("pa_decode", out, q, k_cache, v_cache, block_tables, context_lens, nullptr,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                       workspace_bytes, dtype, stream, nullptr, nullptr);
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

pa_status pa_decode_hinted(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           const int32_t* shared_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                           float scale, int32_t partition_size, void* workspace,
                           size_t workspace_bytes, pa_dtype dtype, void* stream) {
  try {
    return decode_impl("pa_decode_hinted", out, q, k_cache, v_cache, block_tables, context_lens,
                       shared_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, partition_size,
                       workspace, workspace_bytes, dtype, stream, nullptr, nullptr);
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                            int32_t partition_size, pa_dtype dtype, void* stream) {
  static_assert(PA_NOALLOC_SCRATCH_BYTES == pa::NOALLOC_SCRATCH_BYTES, "scratch size");
  try {
    return decode_impl("pa_decode_noalloc", out, q, k_cache, v_cache, block_tables, context_lens,
                       nullptr, num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len, scale, partition_size, nullptr, 0, dtype,
                       stream, nullptr, nullptr, /*noalloc=*/true);
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

pa_status pa_store_decode(void* out, const void* q, const void* key, const void* value,
                          int64_t key_tok_stride, int64_t value_tok_stride, void* k_cache,
                          void* v_cache, const int32_t* slot_mapping, const int32_t* block_tables,
                          const int32_t* context_lens, const int32_t* shared_lens, int32_t num_seqs,
                          int32_t num_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                          float scale, int32_t partition_size, void* workspace,
                          size_t workspace_bytes, pa_dtype dtype, void* stream) {
  try {
    const Fusion f{key, value, key_tok_stride, value_tok_stride, slot_mapping};
    return decode_impl("pa_store_decode", out, q, k_cache, v_cache, block_tables, context_lens, shared_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                       workspace_bytes, dtype, stream, &f, nullptr);
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

pa_status pa_store_decode_fp8(void* out, const void* q, const void* key, const void* value,
                              int64_t key_tok_stride, int64_t value_tok_stride, void* k_cache,
                              void* v_cache, const float* k_scale, const float* v_scale,
                              const int32_t* slot_mapping, const int32_t* block_tables,
                              const int32_t* context_lens, const int32_t* shared_lens, int32_t num_seqs,
                              int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks_per_seq,
                              int32_t max_context_len, float scale, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, pa_dtype dtype,
                              void* stream) {
  try {
    const Fusion f{key, value, key_tok_stride, value_tok_stride, slot_mapping};
    const E4M3Scales sc{k_scale, v_scale};
    return decode_impl("pa_store_decode_fp8", out, q, k_cache, v_cache, block_tables,
                       context_lens, shared_lens, num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                       num_blocks, max_blocks_per_seq, max_context_len, scale, partition_size,
                       workspace, workspace_bytes, dtype, stream, &f, &sc);
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

pa_status pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale, const int32_t* block_tables,
                        const int32_t* context_lens, const int32_t* shared_lens, int32_t num_seqs,
                        int32_t num_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                        float scale, int32_t partition_size, void* workspace,
                        size_t workspace_bytes, pa_dtype dtype, void* stream) {
  try {
    const E4M3Scales sc{k_scale, v_scale};
    return decode_impl("pa_decode_fp8", out, q, k_cache, v_cache, block_tables, context_lens, shared_lens,
                       num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                       max_blocks_per_seq, max_context_len, scale, partition_size, workspace,
                       workspace_bytes, dtype, stream, nullptr, &sc);
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

pa_status pa_store_kvcache_fp8(const void* key, const void* value, int64_t key_tok_stride,
                               int64_t value_tok_stride, void* k_cache, void* v_cache,
                               const int32_t* slot_mapping, const float* k_scale,
                               const float* v_scale, int32_t num_tokens, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks,
                               pa_dtype dtype, void* stream) {
  try {
    if (pa_status st = check_dtype(dtype)) return st;
    if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens=%d is negative", num_tokens);
    if (num_tokens == 0) return ok();
    if (!key || !value || !k_cache || !v_cache || !slot_mapping || !k_scale || !v_scale)
      return fail(PA_ERR_INVALID_ARG, "null pointer argument");
    if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
      return fail(PA_ERR_INVALID_ARG, "num_kv_heads, head_dim, block_size, num_blocks must be positive");
    if (head_dim % 16 != 0)
      return fail(PA_ERR_UNSUPPORTED, "head_dim=%d must be a multiple of 16", head_dim);
    const int e = elem_size(dtype);
    const int64_t row_elems = (int64_t)num_kv_heads * head_dim;
    if (row_elems > (1 << 20))
      return fail(PA_ERR_UNSUPPORTED, "row of %lld elements (at most 1 Mi)", (long long)row_elems);
    if (key_tok_stride < row_elems || value_tok_stride < row_elems)
      return fail(PA_ERR_INVALID_ARG, "token strides (%lld, %lld) below a row of %lld elements",
                  (long long)key_tok_stride, (long long)value_tok_stride, (long long)row_elems);
    if ((key_tok_stride * e) % 16 || (value_tok_stride * e) % 16)
      return fail(PA_ERR_UNSUPPORTED, "token strides must be multiples of 16 bytes");
    if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(slot_mapping, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
      return fail(PA_ERR_UNSUPPORTED,
                  "pointers must be 16-byte aligned (slot_mapping and scales 4-byte)");
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    if (num_slots > INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, "num_blocks*block_size=%lld exceeds int32 slots",
                  (long long)num_slots);
    if ((int64_t)num_tokens * (row_elems / 16) > (int64_t)INT32_MAX)
      return fail(PA_ERR_UNSUPPORTED, "too many tokens in one call");
    pa::StoreE4M3Args a{key, value, key_tok_stride * e, value_tok_stride * e, k_cache, v_cache,
                        slot_mapping, k_scale, v_scale, num_tokens, num_kv_heads, head_dim,
                        num_slots, dtype == PA_BF16};
    const hipError_t err = pa::launch_store_e4m3(a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(PA_ERR_HIP, "store launch: %s", hipGetErrorString(err));
    return ok();
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

namespace {

// Validation shared by pa_prefill_chunk and pa_mixed_batch.
pa_status check_varlen(const char* fn, void* out, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables,
                       const int32_t* query_start_loc, const int32_t* context_lens,
                       int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                       int32_t max_query_len, int32_t max_context_len, float scale, pa_dtype dtype) {
  if (pa_status st = check_dtype(dtype)) return st;
  if (dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "%s: implemented for bf16 only", fn);
  if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start_loc || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: null pointer argument", fn);
  if (pa_status st = check_attention_shapes(num_heads, num_kv_heads, head_dim, block_size,
                                            num_blocks, max_blocks_per_seq, max_context_len))
    return st;
  if (max_query_len <= 0 || max_query_len > max_context_len)
    return fail(PA_ERR_INVALID_ARG, "%s: max_query_len=%d must be in [1, max_context_len=%d]", fn,
                max_query_len, max_context_len);
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "%s: num_seqs=%d above 65535", fn, num_seqs);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "%s: scale is not finite", fn);
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(query_start_loc, 4) || !aligned(context_lens, 4))
    return fail(PA_ERR_UNSUPPORTED, "%s: pointers must be 16-byte aligned (int arrays 4-byte)", fn);
  if ((int64_t)num_heads > 65535) return fail(PA_ERR_UNSUPPORTED, "%s: too many heads", fn);
  return PA_OK;
}

}  // namespace

pa_status pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* query_start_loc,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_query_len,
                           int32_t max_context_len, float scale, pa_dtype dtype, void* stream) {
  try {
    if (pa_status st = check_dtype(dtype)) return st;
    if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs=%d is negative", num_seqs);
    if (num_seqs == 0) return ok();
    if (pa_status st = check_varlen("pa_prefill_chunk", out, q, k_cache, v_cache, block_tables,
                                    query_start_loc, context_lens, num_seqs, num_heads,
                                    num_kv_heads, head_dim, block_size, num_blocks,
                                    max_blocks_per_seq, max_query_len, max_context_len, scale, dtype))
      return st;
    pa::PrefillArgs a{out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                      num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, max_query_len, max_context_len, scale};
    const hipError_t err = pa::launch_prefill(a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(PA_ERR_HIP, "prefill launch: %s", hipGetErrorString(err));
    return ok();
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

pa_status pa_prefill_chunk_fp8(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const float* k_scale, const float* v_scale,
                               const int32_t* block_tables, const int32_t* query_start_loc,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_query_len, int32_t max_context_len, float scale,
                               pa_dtype dtype, void* stream) {
  try {
    if (pa_status st = check_dtype(dtype)) return st;
    if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs=%d is negative", num_seqs);
    if (num_seqs == 0) return ok();
    if (pa_status st = check_varlen("pa_prefill_chunk_fp8", out, q, k_cache, v_cache, block_tables,
                                    query_start_loc, context_lens, num_seqs, num_heads,
                                    num_kv_heads, head_dim, block_size, num_blocks,
                                    max_blocks_per_seq, max_query_len, max_context_len, scale, dtype))
      return st;
    if (!k_scale || !v_scale)
      return fail(PA_ERR_INVALID_ARG, "pa_prefill_chunk_fp8: null k_scale or v_scale");
    if (!aligned(k_scale, 4) || !aligned(v_scale, 4))
      return fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk_fp8: k_scale/v_scale must be 4-byte aligned");
    pa::PrefillArgs a{out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                      num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                      max_blocks_per_seq, max_query_len, max_context_len, scale};
    a.kv_e4m3 = true;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    const hipError_t err = pa::launch_prefill(a, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(PA_ERR_HIP, "prefill launch: %s", hipGetErrorString(err));
    return ok();
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

namespace {

pa_status mixed_impl(const char* fn, void* out, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* block_tables,
                     const int32_t* query_start_loc, const int32_t* context_lens,
                     const int32_t* shared_lens, int32_t num_seqs,
                     int32_t num_decode_seqs, int32_t num_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                     int32_t max_blocks_per_seq, int32_t max_query_len, int32_t max_context_len,
                     float scale, void* workspace, size_t workspace_bytes, pa_dtype dtype,
                     void* stream, const E4M3Scales* e4m3) {
  if (pa_status st = check_dtype(dtype)) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "%s: num_seqs=%d is negative", fn, num_seqs);
  if (num_seqs == 0) return ok();
  if (num_decode_seqs < 0 || num_decode_seqs > num_seqs)
    return fail(PA_ERR_INVALID_ARG, "%s: num_decode_seqs=%d not in [0, num_seqs=%d]", fn,
                num_decode_seqs, num_seqs);
  if (num_decode_seqs > 2048)
    return fail(PA_ERR_UNSUPPORTED, "%s: at most 2048 decode sequences (got %d)", fn,
                num_decode_seqs);
  if (pa_status st = check_varlen(fn, out, q, k_cache, v_cache, block_tables, query_start_loc,
                                  context_lens, num_seqs, num_heads, num_kv_heads, head_dim,
                                  block_size, num_blocks, max_blocks_per_seq, max_query_len,
                                  max_context_len, scale, dtype))
    return st;
  if (e4m3) {
    if (!e4m3->k_scale || !e4m3->v_scale)
      return fail(PA_ERR_INVALID_ARG, "%s: null k_scale or v_scale", fn);
    if (!aligned(e4m3->k_scale, 4) || !aligned(e4m3->v_scale, 4))
      return fail(PA_ERR_UNSUPPORTED, "%s: k_scale/v_scale must be 4-byte aligned", fn);
  }
  if (num_decode_seqs > 0) {
    const size_t need = pa::plan_decode(num_decode_seqs, num_heads, num_kv_heads, head_dim,
                                        max_context_len, PA_PARTITION_BALANCED)
                            .total_bytes;
    if (!workspace) return fail(PA_ERR_WORKSPACE, "%s: a workspace of %zu bytes is needed", fn, need);
    if (workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                  need);
    if (!aligned(workspace, 256))
      return fail(PA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
  }
  pa::PrefillArgs a{out, q, k_cache, v_cache, block_tables, query_start_loc, context_lens,
                    num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                    max_blocks_per_seq, max_query_len, max_context_len, scale};
  if (e4m3) {
    a.kv_e4m3 = true;
    a.k_scale = e4m3->k_scale;
    a.v_scale = e4m3->v_scale;
  }
  if (!aligned(shared_lens, 4))
    return fail(PA_ERR_UNSUPPORTED, "%s: shared_lens must be 4-byte aligned", fn);
  const hipError_t err = pa::launch_mixed(a, num_decode_seqs, shared_lens, workspace,
                                          static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail(PA_ERR_HIP, "%s launch: %s", fn, hipGetErrorString(err));
  return ok();
}

}  // namespace

pa_status pa_mixed_batch(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* query_start_loc,
                         const int32_t* context_lens, const int32_t* shared_lens,
                         int32_t num_seqs, int32_t num_decode_seqs,
                         int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_query_len, int32_t max_context_len, float scale,
                         void* workspace, size_t workspace_bytes, pa_dtype dtype, void* stream) {
  try {
    return mixed_impl("pa_mixed_batch", out, q, k_cache, v_cache, block_tables, query_start_loc,
                      context_lens, shared_lens, num_seqs, num_decode_seqs, num_heads, num_kv_heads,
                      head_dim, block_size, num_blocks, max_blocks_per_seq, max_query_len, max_context_len,
                      scale, workspace, workspace_bytes, dtype, stream, nullptr);
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

pa_status pa_mixed_batch_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_tables, const int32_t* query_start_loc,
                             const int32_t* context_lens,
                             const int32_t* shared_lens, int32_t num_seqs,
                             int32_t num_decode_seqs, int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks,
                             int32_t max_blocks_per_seq, int32_t max_query_len,
                             int32_t max_context_len, float scale, void* workspace,
                             size_t workspace_bytes, pa_dtype dtype, void* stream) {
  try {
    const E4M3Scales sc{k_scale, v_scale};
    return mixed_impl("pa_mixed_batch_fp8", out, q, k_cache, v_cache, block_tables,
                      query_start_loc, context_lens, shared_lens, num_seqs, num_decode_seqs,
                      num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                      max_query_len, max_context_len, scale, workspace, workspace_bytes, dtype,
                      stream, &sc);
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

pa_status pa_stream_read(const void* buf, size_t bytes, uint32_t* out, size_t* bytes_read,
                         void* stream) {
  try {
    if (!buf || !out || !bytes_read)
      return fail(PA_ERR_INVALID_ARG, "pa_stream_read: null pointer argument");
    if (!aligned(buf, 16) || !aligned(out, 4))
      return fail(PA_ERR_UNSUPPORTED, "pa_stream_read: buf must be 16-byte aligned, out 4-byte");
    const int64_t need = pa::stream_read_min_bytes();
    if ((int64_t)bytes < need)
      return fail(PA_ERR_INVALID_ARG, "pa_stream_read: %zu bytes, at least %lld needed", bytes,
                  (long long)need);
    const hipError_t err = pa::launch_stream_read(buf, bytes, out, bytes_read,
                                                  static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(PA_ERR_HIP, "stream read launch: %s", hipGetErrorString(err));
    return ok();
  } catch (...) {
    return fail(PA_ERR_HIP, "unexpected C++ exception");
  }
}

}  // extern "C"
