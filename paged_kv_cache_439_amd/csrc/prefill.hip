// Prefill launch (pa_prefill_chunk); the kernel is in prefill_device.h.

#include "prefill_device.h"

namespace pa {

template <int D, int HW, typename CT>
static void launch_prefill_t(PrefillParams prm, int32_t max_query_len, int32_t num_seqs,
                             int32_t num_kv_heads, hipStream_t stream) {
  constexpr int ROWS = 32 * (4 / HW);
  prm.row_blocks = (max_query_len + ROWS - 1) / ROWS;
  prm.num_seqs = num_seqs;
  // x: head group, y: sequence, z: row block (from the end of the chunk).
  const dim3 grid((unsigned)(num_kv_heads * prm.n_sub), (unsigned)num_seqs, (unsigned)prm.row_blocks);
  hipLaunchKernelGGL((prefill_chunk_kernel<D, HW, CT>), grid, dim3(256), 0, stream, prm);
}

PrefillParams make_prefill_params(const PrefillArgs& a) {
  PrefillParams prm{};
  prm.out = static_cast<uint16_t*>(a.out);
  prm.q = static_cast<const uint16_t*>(a.q);
  prm.k_cache = static_cast<const char*>(a.k_cache);
  prm.v_cache = static_cast<const char*>(a.v_cache);
  prm.block_tables = a.block_tables;
  prm.query_start_loc = a.query_start_loc;
  prm.context_lens = a.context_lens;
  prm.num_heads = a.num_heads;
  prm.num_kv_heads = a.num_kv_heads;
  prm.group = a.num_heads / a.num_kv_heads;
  prm.n_sub = prm.group / prefill_heads_per_wg(prm.group);
  prm.bs_log2 = __builtin_ctz((unsigned)a.block_size);
  prm.num_blocks = a.num_blocks;
  prm.max_blocks_per_seq = a.max_blocks_per_seq;
  prm.max_query_len = a.max_query_len;
  prm.max_context_len = a.max_context_len;
  prm.scale_log2 = a.scale * 1.4426950408889634f;
  prm.k_scale = a.kv_e4m3 ? a.k_scale : nullptr;
  prm.v_scale = a.kv_e4m3 ? a.v_scale : nullptr;
  return prm;
}

template <typename CT>
static void launch_prefill_ct(const PrefillParams& prm, const PrefillArgs& a, hipStream_t stream) {
  const int32_t hw = prefill_heads_per_wg(prm.group);
  const int32_t mq = a.max_query_len, B = a.num_seqs, H = a.num_kv_heads;
  if (a.head_dim == 64) {
    if (hw == 4) launch_prefill_t<64, 4, CT>(prm, mq, B, H, stream);
    else if (hw == 2) launch_prefill_t<64, 2, CT>(prm, mq, B, H, stream);
    else launch_prefill_t<64, 1, CT>(prm, mq, B, H, stream);
  } else {
    if (hw == 4) launch_prefill_t<128, 4, CT>(prm, mq, B, H, stream);
    else if (hw == 2) launch_prefill_t<128, 2, CT>(prm, mq, B, H, stream);
    else launch_prefill_t<128, 1, CT>(prm, mq, B, H, stream);
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const PrefillParams prm = make_prefill_params(a);
  if (a.kv_e4m3) launch_prefill_ct<uint8_t>(prm, a, stream);
  else launch_prefill_ct<uint16_t>(prm, a, stream);
  return hipGetLastError();
}

}  // namespace pa
