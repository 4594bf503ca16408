// Decode planning and launch (pa_decode, pa_store_decode, pa_decode_fp8);
// the kernels are in decode_device.h.

#include "decode_device.h"

#include <algorithm>
#include <mutex>

namespace pa {

// ---------------------------------------------------------------------------
// planning and launch
// ---------------------------------------------------------------------------

// Query heads one wave handles: at most 4 (a group of 8 becomes two waves
// of the same workgroup, which read the same K/V rows through the caches).
static int32_t heads_per_unit(int32_t group) {
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Compute units of the current device (256 on MI355X when none is visible,
// so that workspace sizes can be computed without a GPU).
static int32_t device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return n;
}

DecodePlan plan_decode(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t max_context_len, int32_t partition_size,
                       bool kv_e4m3) {
  DecodePlan pl{};
  pl.group = num_heads / num_kv_heads;
  pl.heads_per_unit = heads_per_unit(pl.group);
  pl.units = num_kv_heads * (pl.group / pl.heads_per_unit);
  if (partition_size == PA_PARTITION_BALANCED_VALUE) {
    pl.balanced = true;
    // A head row of E4M3 codes at head_dim 64 is half a 128-byte line; a
    // wave that reads two adjacent KV heads streams whole lines (one head
    // per wave measured 5.0-5.1 TB/s in this access pattern, a pair
    // 6.35-6.45 TB/s).
    pl.pair = kv_e4m3 && head_dim == 64 && pl.group == 1 && num_kv_heads % 2 == 0;
    if (pl.pair) pl.units = num_kv_heads / 2;
    pl.partition = max_context_len > 0 ? max_context_len : 1;
    pl.max_parts = 1;
    const int64_t waves = (int64_t)DECODE_BAL_WAVES_PER_SIMD * 4 * device_cus();
    pl.workers = (int32_t)std::max<int64_t>(1, waves / pl.units);
    const size_t slots = (size_t)pl.workers * 2 * num_heads;
    pl.acc_bytes = align256(slots * head_dim * sizeof(float));
    pl.ml_bytes = align256(slots * 2 * sizeof(float));
    pl.pfx_bytes = align256(((size_t)num_seqs + 1) * sizeof(int32_t));
    pl.total_bytes = pl.acc_bytes + pl.ml_bytes + pl.pfx_bytes;
    return pl;
  }
  const bool split = partition_size > 0 && partition_size < max_context_len;
  pl.partition = split ? partition_size : (max_context_len > 0 ? max_context_len : 1);
  pl.max_parts = split ? (max_context_len + partition_size - 1) / partition_size : 1;
  if (split) {
    const size_t rows = (size_t)num_seqs * num_heads * pl.max_parts;
    pl.acc_bytes = align256(rows * head_dim * sizeof(float));
    pl.ml_bytes = align256(rows * 2 * sizeof(float));
    pl.total_bytes = pl.acc_bytes + pl.ml_bytes;
  }
  return pl;
}

template <typename T, typename KT, int D, int GT, int U, bool PAIR>
static void launch_balanced_main(const DecodeParams& prm, const DecodePlan& pl, hipStream_t stream) {
  constexpr int TPW = 64 / ((PAIR ? 2 : 1) * D * (int)sizeof(KT) / 16);
  constexpr int CT = U * TPW;
  const bool big_blocks = (1 << prm.bs_log2) >= CT;
  const int64_t waves = (int64_t)pl.workers * pl.units;
  const dim3 bgrid((unsigned)((waves + 3) / 4));
  if (big_blocks)
    hipLaunchKernelGGL((paged_decode_balanced_kernel<T, KT, D, GT, U, true, PAIR>), bgrid, dim3(256), 0,
                       stream, prm);
  else
    hipLaunchKernelGGL((paged_decode_balanced_kernel<T, KT, D, GT, U, false, PAIR>), bgrid, dim3(256),
                       0, stream, prm);
}

template <typename T, typename KT, int D, int GT, int U>
static void launch_balanced(const DecodeParams& prm, const DecodePlan& pl, int32_t num_seqs, hipStream_t stream) {
  if constexpr (sizeof(KT) == 1 && D == 64 && GT == 1) {
    if (pl.pair) launch_balanced_main<T, KT, D, GT, U, true>(prm, pl, stream);
    else launch_balanced_main<T, KT, D, GT, U, false>(prm, pl, stream);
  } else {
    launch_balanced_main<T, KT, D, GT, U, false>(prm, pl, stream);
  }
  // the merge takes one KV head per unit (a pair's two heads separately)
  const unsigned merge_units = (unsigned)(pl.pair ? 2 * pl.units : pl.units);
  hipLaunchKernelGGL((paged_decode_balanced_merge_kernel<T, D, GT>), dim3(num_seqs, (merge_units + 3) / 4),
                     dim3(256), 0, stream, prm);
}

// Fixed slices: grid (unit groups, sequences, partitions), one position per
// (sequence, partition) pair in dispatch order. Within fixed_item's bounds a
// position takes the item that order gives it (whole partitions first, then
// partial ones longest-first); beyond them, sequence y's partition z, so
// that every sequence's first partition is dispatched before any second one
// (on the b512 lognormal workload with 512-token slices that order took
// 730 us against 820 us sequence by sequence).
template <typename T, typename KT, int D, int GT, int U>
static void launch_fixed(const DecodeParams& prm, const DecodePlan& pl, int32_t num_seqs, hipStream_t stream) {
  const dim3 grid((unsigned)((pl.units + 3) / 4), (unsigned)num_seqs, (unsigned)pl.max_parts);
  constexpr int TPW = 64 / (D * (int)sizeof(KT) / 16);
  constexpr int CT = U * TPW;
  const bool big_blocks = (1 << prm.bs_log2) >= CT;
  const bool uniform = big_blocks && (prm.max_parts == 1 || prm.partition % CT == 0);
  if (uniform)
    hipLaunchKernelGGL((paged_decode_kernel<T, KT, D, GT, U, true>), grid, dim3(256), 0, stream, prm);
  else
    hipLaunchKernelGGL((paged_decode_kernel<T, KT, D, GT, U, false>), grid, dim3(256), 0, stream, prm);
  if (pl.max_parts > 1)
    hipLaunchKernelGGL((paged_decode_merge_kernel<T, D, GT>), dim3(num_seqs, grid.x), dim3(256), 0,
                       stream, prm);
}

// Loads in flight per lane (U): DECODE_U for pools in the query type; for
// E4M3 pools DECODE_U_E4M3 in the balanced split and half of it in the fixed
// split, whose four-heads-per-wave kernel would otherwise spill registers.
template <typename T, typename KT, int D, int GT>
static void launch_split(const DecodeParams& prm, const DecodePlan& pl, int32_t num_seqs, hipStream_t stream) {
  constexpr bool E8 = sizeof(KT) == 1;
  constexpr int UB = E8 ? DECODE_U_E4M3 : DECODE_U;
  constexpr int UF = E8 ? (DECODE_U_E4M3 > 2 ? DECODE_U_E4M3 / 2 : DECODE_U_E4M3) : DECODE_U;
  if (pl.balanced) launch_balanced<T, KT, D, GT, UB>(prm, pl, num_seqs, stream);
  else launch_fixed<T, KT, D, GT, UF>(prm, pl, num_seqs, stream);
}

template <typename T, typename KT, int D>
static void launch_gt(const DecodeParams& prm, const DecodePlan& pl, int32_t num_seqs, hipStream_t stream) {
  switch (pl.heads_per_unit) {
    case 1: launch_split<T, KT, D, 1>(prm, pl, num_seqs, stream); break;
    case 2: launch_split<T, KT, D, 2>(prm, pl, num_seqs, stream); break;
    default: launch_split<T, KT, D, 4>(prm, pl, num_seqs, stream); break;
  }
}

template <typename T, typename KT>
static void launch_d(const DecodeParams& prm, const DecodePlan& pl, int head_dim, int32_t num_seqs,
                     hipStream_t stream) {
  if (head_dim == 64) launch_gt<T, KT, 64>(prm, pl, num_seqs, stream);
  else launch_gt<T, KT, 128>(prm, pl, num_seqs, stream);
}

DecodeParams make_decode_params(const DecodeArgs& a, const DecodePlan& pl) {
  DecodeParams prm{};
  prm.out = a.out;
  prm.q = a.q;
  prm.k_cache = static_cast<const char*>(a.k_cache);
  prm.v_cache = static_cast<const char*>(a.v_cache);
  prm.block_tables = a.block_tables;
  prm.context_lens = a.context_lens;
  prm.shared_lens = a.shared_lens;
  if (pl.total_bytes) {
    char* ws = static_cast<char*>(a.workspace);
    if (pl.balanced) {
      prm.part_acc = reinterpret_cast<float*>(ws);
      prm.part_ml = reinterpret_cast<float*>(ws + pl.acc_bytes);
      prm.ws_pfx = reinterpret_cast<int32_t*>(ws + pl.acc_bytes + pl.ml_bytes);
    } else {
      prm.ws_acc = reinterpret_cast<float*>(ws);
      prm.ws_ml = reinterpret_cast<float*>(ws + pl.acc_bytes);
    }
  }
  prm.num_seqs = a.num_seqs;
  prm.workers = pl.workers;
  prm.num_heads = a.num_heads;
  prm.num_kv_heads = a.num_kv_heads;
  prm.group = pl.group;
  prm.n_sub = pl.group / pl.heads_per_unit;
  prm.units = pl.units;
  prm.pair = pl.pair ? 1 : 0;
  prm.bs_log2 = __builtin_ctz((unsigned)a.block_size);
  prm.num_blocks = a.num_blocks;
  prm.max_blocks_per_seq = a.max_blocks_per_seq;
  prm.max_context_len = a.max_context_len;
  prm.partition = pl.partition;
  prm.max_parts = pl.max_parts;
  prm.fixed_order = (!pl.balanced && pl.max_parts > 1 && a.num_seqs <= FIXED_ORDER_MAX_SEQS &&
                     pl.max_parts <= FIXED_ORDER_MAX_PARTS) ? 1 : 0;
  prm.scale_log2 = a.scale * 1.4426950408889634f;
  prm.row_bytes = a.num_kv_heads * a.head_dim * (a.kv_e4m3 ? 1 : a.bf16 ? 2 : 4);
  prm.k_scale = a.k_scale;
  prm.v_scale = a.v_scale;
  prm.block_bytes = (int64_t)a.block_size * prm.row_bytes;
  if (a.key != nullptr) {
    prm.new_k = static_cast<const char*>(a.key);
    prm.new_v = static_cast<const char*>(a.value);
    prm.new_k_stride = a.key_stride_bytes;
    prm.new_v_stride = a.value_stride_bytes;
    prm.slot_mapping = a.slot_mapping;
    prm.num_slots = (int64_t)a.num_blocks * a.block_size;
  }
  return prm;
}

// ---------------------------------------------------------------------------
// static scratch of pa_decode_noalloc
// ---------------------------------------------------------------------------
//
// The split workspace of callers that cannot allocate device memory: one
// array per GPU, in the library's code object, held until the process ends.
// Its address on a device comes from hipGetSymbolAddress with that device
// current (each GPU holds its own copy at its own address); in host code
// the array's name is not a device address, so only the looked-up pointer
// is ever passed on.
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
  const DecodeParams prm = make_decode_params(a, pl);
  if (a.kv_e4m3) {
    if (a.bf16) launch_d<uint16_t, uint8_t>(prm, pl, a.head_dim, a.num_seqs, stream);
    else launch_d<float, uint8_t>(prm, pl, a.head_dim, a.num_seqs, stream);
  } else {
    if (a.bf16) launch_d<uint16_t, uint16_t>(prm, pl, a.head_dim, a.num_seqs, stream);
    else launch_d<float, float>(prm, pl, a.head_dim, a.num_seqs, stream);
  }
  return hipGetLastError();
}

}  // namespace pa
