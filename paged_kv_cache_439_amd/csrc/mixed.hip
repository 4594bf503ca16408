// mixed_batch: one launch for a continuous batch that carries decode tokens
// and prefill chunks together.
//
// The nano-vllm page's scheduler (§3.3) keeps forming batches from waiting
// and running sequences, so that one forward step holds new prompts (prefill
// chunks) beside sequences that generate one token (decode). Attention of
// such a batch is exactly pa_prefill_chunk's varlen definition: sequence i
// has n_i query rows at positions c_i .. c_i + n_i - 1 and row t sees keys
// 0 .. c_i + t; a decode sequence is the case n_i = 1.
//
// The two kinds bound on different units: a prefill chunk on bf16 MFMA, a
// decode token on HBM bandwidth (its whole context is read for one row). One
// kernel therefore runs both bodies side by side: balanced-split decode
// workers (balanced_body), planned for one wave per SIMD, are dispatched
// first and take one of the two workgroup slots of every CU for the whole
// launch; prefill work items (prefill_body: one head group, one sequence,
// one row block) stream through the other slot, so every CU holds matrix
// work and streaming work at once. The decode sequences cut by a worker's
// range are merged by the balanced merge kernel afterwards.
//
// Batch layout (a convention of the call): the first num_decode sequences
// are the decode tokens, one query row each (query_start_loc[i] = i for
// i <= num_decode), and the prefill chunks follow.

#include "decode_device.h"
#include "prefill_device.h"

#include <algorithm>

namespace pa {

// Order of the two kinds of workgroup in the grid: 0 alternates them while
// both remain, 1 puts the decode workers first, 2 the prefill items first.
// Measured on MI355X with 128-512 decode tokens beside 4-8 chunks of 512:
// decode first with one decode wave per SIMD is 1-5% faster than the two
// separate calls; alternating, or two decode waves per SIMD (which leave
// prefill waiting for free slots), are slower than the separate calls.
#ifndef MIXED_ORDER
#define MIXED_ORDER 1
#endif
// Resident decode waves per SIMD the mixed launch plans its decode workers
// for (at most the balanced split's own count, whose workspace it uses).
#ifndef MIXED_DECODE_WAVES
#define MIXED_DECODE_WAVES 1
#endif

// Decode sequences one mixed launch supports (their chunk prefix sums sit in
// LDS next to the prefill stages: 8 KB plus 66 KB keeps two workgroups per
// CU).
constexpr int MIXED_MAX_DECODE_SEQS = 2048;

struct MixedParams {
  DecodeParams d;   // decode sub-batch: sequences 0 .. num_decode-1
  PrefillParams f;  // prefill sub-batch: the sequences after them
  int32_t np, nd;   // prefill work items, decode workgroups
  int32_t fx, fy;   // prefill grid extents: head groups, sequences
};

// Loads in flight per lane of the decode workers for pools of element type
// KT (bf16, or E4M3 codes).
template <typename KT>
constexpr int mixed_decode_u() {
  return sizeof(KT) == 1 ? DECODE_U_BALANCED_E4M3 : DECODE_U_BALANCED;
}

// Workgroup k of the grid, in the order MIXED_ORDER selects. KT: the pools'
// element type (uint16_t bf16, uint8_t E4M3 codes).
template <int D, int G, bool UNIFORM_BLOCK, typename KT>
__global__ __launch_bounds__(256, 2) void mixed_batch_kernel(MixedParams p) {
  const int k = blockIdx.x;
  bool prefill;
  int idx;
  if constexpr (MIXED_ORDER == 1) {
    prefill = k >= p.nd;
    idx = prefill ? k - p.nd : k;
  } else if constexpr (MIXED_ORDER == 2) {
    prefill = k < p.np;
    idx = prefill ? k : k - p.np;
  } else {
    const int m = min(p.np, p.nd);
    if (k < 2 * m) {
      prefill = (k & 1) == 0;
      idx = k >> 1;
    } else {
      prefill = p.np > p.nd;
      idx = m + (k - 2 * m);
    }
  }
  if (prefill) {
    const int r = idx / p.fx;
    prefill_body<D, G, KT>(p.f, idx - r * p.fx, r % p.fy, r / p.fy);
  } else {
    balanced_body<uint16_t, KT, D, G, mixed_decode_u<KT>(), UNIFORM_BLOCK, MIXED_MAX_DECODE_SEQS,
                  /*PAIR=*/false, /*MFMA_OK=*/false>(
        p.d, idx, p.nd);
  }
}

template <int D, int G, typename KT>
static void launch_mixed_t(const MixedParams& prm, int32_t bs, hipStream_t stream) {
  constexpr int TPW = 64 / (D * (int)sizeof(KT) / 16);
  constexpr int CT = mixed_decode_u<KT>() * TPW;
  const dim3 grid((unsigned)(prm.np + prm.nd));
  if (bs >= CT)
    hipLaunchKernelGGL((mixed_batch_kernel<D, G, true, KT>), grid, dim3(256), 0, stream, prm);
  else
    hipLaunchKernelGGL((mixed_batch_kernel<D, G, false, KT>), grid, dim3(256), 0, stream, prm);
  hipLaunchKernelGGL((paged_decode_balanced_merge_kernel<uint16_t, D, G>),
                     dim3((unsigned)prm.d.num_seqs, (unsigned)((prm.d.units + 3) / 4)), dim3(256), 0,
                     stream, prm.d);
}

template <typename KT>
static void launch_mixed_kt(const MixedParams& prm, const PrefillArgs& a, int32_t G,
                            hipStream_t stream) {
  if (a.head_dim == 64) {
    if (G == 4) launch_mixed_t<64, 4, KT>(prm, a.block_size, stream);
    else if (G == 2) launch_mixed_t<64, 2, KT>(prm, a.block_size, stream);
    else launch_mixed_t<64, 1, KT>(prm, a.block_size, stream);
  } else {
    if (G == 4) launch_mixed_t<128, 4, KT>(prm, a.block_size, stream);
    else if (G == 2) launch_mixed_t<128, 2, KT>(prm, a.block_size, stream);
    else launch_mixed_t<128, 1, KT>(prm, a.block_size, stream);
  }
}

hipError_t launch_mixed(const PrefillArgs& a, int32_t num_decode, const int32_t* shared_lens,
                        void* workspace, hipStream_t stream) {
  const int32_t Bd = num_decode, Bp = a.num_seqs - num_decode;
  if (Bd == 0) return launch_prefill(a, stream);
  DecodeArgs da{};
  da.out = a.out;
  da.q = a.q;
  da.k_cache = a.k_cache;
  da.v_cache = a.v_cache;
  da.block_tables = a.block_tables;
  da.context_lens = a.context_lens;
  da.shared_lens = shared_lens;  // the decode rows are sequences 0 .. Bd-1
  da.num_seqs = Bd;
  da.num_heads = a.num_heads;
  da.num_kv_heads = a.num_kv_heads;
  da.head_dim = a.head_dim;
  da.block_size = a.block_size;
  da.num_blocks = a.num_blocks;
  da.max_blocks_per_seq = a.max_blocks_per_seq;
  da.max_context_len = a.max_context_len;
  da.scale = a.scale;
  da.partition_size = PA_PARTITION_BALANCED_VALUE;
  da.workspace = workspace;
  da.bf16 = true;
  da.kv_e4m3 = a.kv_e4m3;
  da.k_scale = a.k_scale;
  da.v_scale = a.v_scale;
  DecodePlan plan = plan_decode(Bd, a.num_heads, a.num_kv_heads, a.head_dim, a.max_context_len,
                                PA_PARTITION_BALANCED_VALUE);
  if (Bp == 0) return launch_decode(da, plan, stream);
  static_assert(MIXED_DECODE_WAVES >= 1 && MIXED_DECODE_WAVES <= DECODE_BAL_WAVES_PER_SIMD,
                "the workspace holds the balanced split's workers");
  plan.workers = std::max(1, plan.workers * MIXED_DECODE_WAVES / DECODE_BAL_WAVES_PER_SIMD);

  PrefillArgs fa = a;
  fa.block_tables = a.block_tables + (int64_t)Bd * a.max_blocks_per_seq;
  fa.query_start_loc = a.query_start_loc + Bd;
  fa.context_lens = a.context_lens + Bd;
  fa.num_seqs = Bp;

  MixedParams prm{};
  prm.d = make_decode_params(da, plan);
  prm.f = make_prefill_params(fa);
  const int32_t G = prefill_heads_per_wg(prm.f.group);
  if (G != plan.heads_per_unit) return hipErrorInvalidValue;  // both bodies serve G heads
  const int32_t rows = 32 * (4 / G);
  prm.f.row_blocks = (fa.max_query_len + rows - 1) / rows;
  prm.f.num_seqs = Bp;
  prm.fx = a.num_kv_heads * prm.f.n_sub;
  prm.fy = Bp;
  prm.np = prm.fx * Bp * prm.f.row_blocks;
  prm.nd = (int32_t)(((int64_t)plan.workers * plan.units + 3) / 4);
  if (a.kv_e4m3) launch_mixed_kt<uint8_t>(prm, a, G, stream);
  else launch_mixed_kt<uint16_t>(prm, a, G, stream);
  return hipGetLastError();
}

}  // namespace pa
