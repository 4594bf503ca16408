// paged_decode: one query token per sequence, attending over the sequence's
// context through its block table, with an optional split of the context
// into partitions whose softmax states are merged in the same launch.
//
// What is computed (the plain reading of the nano-vllm page's §1 and §3.1 and
// the mini-vllm page's "KVCache" item and its cached-decode benchmark):
//   out[i][h] = softmax(scale * K_i[g] q[i][h]) V_i[g],  g = h / (Hq/Hkv),
// over the context_lens[i] rows of sequence i; logical row j is row
// j % block_size of physical block block_tables[i][j / block_size].
//
// Work decomposition (one wave64 = one unit of work):
//   unit = (sequence, KV head, group of GT query heads, partition of P tokens)
//   grid = (max partitions, sequences, ceil(units per (seq, partition) / 4)),
//   256 threads = 4 independent waves, no LDS and no barriers.
// Lane mapping: a K or V row of one head is D*e bytes = LPT lanes x 16 bytes,
// so a wave-wide 16-byte load covers TPW = 64/LPT token rows; U loads per lane
// give a chunk of CT = U*TPW tokens whose K and V loads are all issued before
// any of them is used.
//   QK:  lane (dc, tr) forms partial dot products over its 16-byte slice
//        (v_dot2_f32_bf16 for bf16), then a DPP butterfly over the LPT lanes
//        of the row completes them.
//   softmax: each token-row group tr keeps its own online state (running max
//        m, sum l, weighted value sum acc) per head, in log2 units, so the
//        main loop needs no cross-row communication; the TPW states are
//        merged once at the end with the exact max-rescaling merge.
//   PV:  acc[h][slice] += p * V-slice, all in registers.
// Split: each partition writes (m, l, acc) in fp32 to the workspace and a
//   second, small kernel (paged_decode_merge_kernel) combines them with the
//   exact max-rescaling merge. The kernel boundary makes the states visible
//   across the chip's separate L2 caches once, instead of a cache writeback
//   per wave.
//
// Bound: HBM. Algorithmic bytes = context rows x 2 (K and V) x Hkv x D x e.

#include "pa_device.h"
#include "pa_internal.h"

#ifndef DECODE_U
#define DECODE_U 8
#endif

namespace pa {

struct DecodeParams {
  void* out;
  const void* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;     // [B][Hq][max_parts][D]
  float* ws_ml;      // [B][Hq][max_parts][2]
  int32_t num_heads, num_kv_heads, group, n_sub, units;
  int32_t bs_log2, num_blocks, max_blocks_per_seq, max_context_len;
  int32_t partition, max_parts;
  int32_t row_bytes;    // Hkv * D * e: bytes between consecutive tokens of a block
  int64_t block_bytes;  // block_size * row_bytes
  float scale_log2;     // scale * log2(e): logits are kept in log2 units
};

// 16-byte streaming load of pool data: every K/V byte is read once per call,
// so the loads carry the nontemporal hint and do not displace reusable lines.
__device__ __forceinline__ uint4 stream_load(const char* ptr) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<float> {
  static constexpr int E = 4;
};
template <>
struct ElemTraits<uint16_t> {  // bf16 storage
  static constexpr int E = 2;
};

// Partial dot product of this lane's 16-byte slice of q (pre-loaded) and k.
template <typename T>
__device__ __forceinline__ float slice_dot(const uint4& qv, const uint4& kv);
template <>
__device__ __forceinline__ float slice_dot<uint16_t>(const uint4& qv, const uint4& kv) {
  float s = dot2_bf16(qv.x, kv.x, 0.0f);
  s = dot2_bf16(qv.y, kv.y, s);
  s = dot2_bf16(qv.z, kv.z, s);
  return dot2_bf16(qv.w, kv.w, s);
}
template <>
__device__ __forceinline__ float slice_dot<float>(const uint4& qv, const uint4& kv) {
  float s = __builtin_bit_cast(float, qv.x) * __builtin_bit_cast(float, kv.x);
  s = fmaf(__builtin_bit_cast(float, qv.y), __builtin_bit_cast(float, kv.y), s);
  s = fmaf(__builtin_bit_cast(float, qv.z), __builtin_bit_cast(float, kv.z), s);
  return fmaf(__builtin_bit_cast(float, qv.w), __builtin_bit_cast(float, kv.w), s);
}

// Widen a 16-byte slice to EPL floats.
template <typename T, int EPL>
__device__ __forceinline__ void widen_slice(const uint4& v, float (&f)[EPL]) {
  if constexpr (sizeof(T) == 2) {
    f[0] = bf16lo(v.x); f[1] = bf16hi(v.x);
    f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
    f[4] = bf16lo(v.z); f[5] = bf16hi(v.z);
    f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
  } else {
    f[0] = __builtin_bit_cast(float, v.x); f[1] = __builtin_bit_cast(float, v.y);
    f[2] = __builtin_bit_cast(float, v.z); f[3] = __builtin_bit_cast(float, v.w);
  }
}

// Store EPL floats as one 16-byte slice of the output type.
template <typename T, int EPL>
__device__ __forceinline__ void store_slice(void* dst, const float (&f)[EPL]) {
  uint4 w;
  if constexpr (sizeof(T) == 2) {
    w.x = pack_bf16x2(f[0], f[1]); w.y = pack_bf16x2(f[2], f[3]);
    w.z = pack_bf16x2(f[4], f[5]); w.w = pack_bf16x2(f[6], f[7]);
  } else {
    w.x = __builtin_bit_cast(uint32_t, f[0]); w.y = __builtin_bit_cast(uint32_t, f[1]);
    w.z = __builtin_bit_cast(uint32_t, f[2]); w.w = __builtin_bit_cast(uint32_t, f[3]);
  }
  *reinterpret_cast<uint4*>(dst) = w;
}

// Merge the online states of the token-row groups that share a d-slice
// (lanes that differ only in the bits at and above log2(LPT)).
template <int LPT, int GT, int EPL>
__device__ __forceinline__ void merge_row_groups(float (&m)[GT], float (&l)[GT],
                                                 float (&acc)[GT][EPL]) {
#pragma unroll
  for (int mask = LPT; mask < 64; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const float mo = __shfl_xor(m[h], mask);
      const float lo = __shfl_xor(l[h], mask);
      const float mn = fmaxf(m[h], mo);
      const float a = fast_exp2(m[h] - mn);
      const float b = fast_exp2(mo - mn);
      l[h] = l[h] * a + lo * b;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * a + __shfl_xor(acc[h][e], mask) * b;
      m[h] = mn;
    }
  }
}

// UNIFORM_BLOCK: every chunk lies inside one block (block_size >= CT and
// partitions start at multiples of CT), so one scalar table lookup serves the
// whole chunk; otherwise each lane looks up its own token's block.
template <typename T, int D, int GT, int U, bool UNIFORM_BLOCK>
__global__ __launch_bounds__(256) void paged_decode_kernel(DecodeParams p) {
  constexpr int E = ElemTraits<T>::E;
  constexpr int EPL = 16 / E;     // elements per 16-byte lane slice
  constexpr int LPT = D / EPL;    // lanes per token row of one head
  constexpr int TPW = 64 / LPT;   // token rows per wave-wide load
  constexpr int CT = U * TPW;     // tokens per chunk
  static_assert(LPT >= 1 && LPT <= 32 && (64 % LPT) == 0, "unsupported head_dim");

  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= p.units) return;
  const int seq = blockIdx.z;
  const int part = blockIdx.y;
  const int L = min(p.context_lens[seq], p.max_context_len);
  const int P = p.partition;
  const int nparts = L > 0 ? (L + P - 1) / P : 0;

  const int kvh = unit / p.n_sub;
  const int h0 = kvh * p.group + (unit - kvh * p.n_sub) * GT;
  const int dc = lane % LPT;
  const int tr = lane / LPT;
  const int64_t head_stride = D;
  char* const out_base = static_cast<char*>(p.out);

  if (nparts == 0) {  // empty context: defined output of zeros
    if (part == 0 && tr == 0) {
      float z[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) z[e] = 0.0f;
#pragma unroll
      for (int h = 0; h < GT; ++h)
        store_slice<T, EPL>(out_base + (((int64_t)seq * p.num_heads + h0 + h) * head_stride + dc * EPL) * E, z);
    }
    return;
  }
  if (part >= nparts) return;

  const int tok_begin = part * P;
  const int tok_end = min(L, tok_begin + P);
  const int bs_log2 = p.bs_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int row_bytes = p.row_bytes;
  const int lane_off = kvh * D * E + dc * 16;
  const int32_t* bt = p.block_tables + (int64_t)seq * p.max_blocks_per_seq;

  // q slices of the GT heads, as stored (bf16 pairs feed v_dot2 directly).
  uint4 qv[GT];
  {
    const char* qb = static_cast<const char*>(p.q);
#pragma unroll
    for (int h = 0; h < GT; ++h)
      qv[h] = *reinterpret_cast<const uint4*>(
          qb + (((int64_t)seq * p.num_heads + h0 + h) * head_stride) * E + dc * 16);
  }

  // Block-table window: lane i holds the physical id of block wbase + i.
  const int last_blk = (tok_end - 1) >> bs_log2;
  int wbase = tok_begin >> bs_log2;
  int tbl = (wbase + lane <= last_blk) ? clamp_block(bt[wbase + lane], p.num_blocks) : 0;

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = NEG_BIG;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
  }

  for (int j0 = tok_begin; j0 < tok_end; j0 += CT) {
    const int chunk_last = (min(j0 + CT, tok_end) - 1) >> bs_log2;
    if (chunk_last >= wbase + 64) {  // uniform: slide the table window
      wbase = j0 >> bs_log2;
      tbl = (wbase + lane <= last_blk) ? clamp_block(bt[wbase + lane], p.num_blocks) : 0;
    }
    // Addresses first, then every K and V load of the chunk, then compute:
    // the whole chunk's bytes are in flight before any of them is waited on.
    bool valid[U];
    int64_t off[U];
    if constexpr (UNIFORM_BLOCK) {
      const int phys = __builtin_amdgcn_readlane(tbl, (j0 >> bs_log2) - wbase);
      const int64_t base = (int64_t)phys * p.block_bytes;
      const int row0 = (j0 & bs_mask) + tr;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * TPW + tr;
        valid[u] = j < tok_end;
        const int row = valid[u] ? row0 + u * TPW : (j0 & bs_mask);
        off[u] = base + (row * row_bytes + lane_off);
      }
    } else {
      int phys[U], row[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = j0 + u * TPW + tr;
        valid[u] = j < tok_end;
        const int jj = valid[u] ? j : j0;  // in-bounds stand-in for tail lanes
        phys[u] = __shfl(tbl, (jj >> bs_log2) - wbase);
        row[u] = jj & bs_mask;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) off[u] = (int64_t)phys[u] * p.block_bytes + (row[u] * row_bytes + lane_off);
    }
    uint4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) kr[u] = stream_load(p.k_cache + off[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) vr[u] = stream_load(p.v_cache + off[u]);
    __builtin_amdgcn_sched_barrier(0);

    float s[U][GT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int h = 0; h < GT; ++h) s[u][h] = group_sum<LPT>(slice_dot<T>(qv[h], kr[u]));

#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float cm = NEG_BIG;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[u][h] = valid[u] ? s[u][h] * p.scale_log2 : -INFINITY;
        cm = fmaxf(cm, s[u][h]);
      }
      const float mn = fmaxf(m[h], cm);
      const float alpha = fast_exp2(m[h] - mn);
      m[h] = mn;
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[u][h] = fast_exp2(s[u][h] - mn);
        l[h] += s[u][h];
      }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
      widen_slice<T, EPL>(vr[u], vf);
#pragma unroll
      for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(s[u][h], vf[e], acc[h][e]);
    }
  }

  merge_row_groups<LPT, GT, EPL>(m, l, acc);

  if (nparts == 1) {
    if (tr == 0) {
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float o[EPL];
        const float inv = 1.0f / l[h];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = acc[h][e] * inv;
        store_slice<T, EPL>(out_base + (((int64_t)seq * p.num_heads + h0 + h) * head_stride + dc * EPL) * E, o);
      }
    }
    return;
  }

  // ---- split: publish this partition's state for the merge kernel ----
  if (tr == 0) {
    const int64_t mp = p.max_parts;
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const int64_t sh = (int64_t)seq * p.num_heads + h0 + h;
      float* dst = p.ws_acc + (sh * mp + part) * D + dc * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
      if (dc == 0) *reinterpret_cast<float2*>(p.ws_ml + (sh * mp + part) * 2) = make_float2(m[h], l[h]);
    }
  }
}

// Merge the partition states of every (sequence, unit) whose context was
// split: with M the largest partition maximum and w_p = 2^(m_p - M),
//   out = sum_p w_p acc_p / sum_p w_p l_p.
// One wave per unit; token-row group tr takes partitions tr, tr+TPW, ...,
// then the groups merge as in the main kernel. Contexts that fit one
// partition were written by the main kernel and are skipped here.
template <typename T, int D, int GT>
__global__ __launch_bounds__(256) void paged_decode_merge_kernel(DecodeParams p) {
  constexpr int E = ElemTraits<T>::E;
  constexpr int EPL = 16 / E;
  constexpr int LPT = D / EPL;
  constexpr int TPW = 64 / LPT;
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (unit >= p.units) return;
  const int seq = blockIdx.x;
  const int L = min(p.context_lens[seq], p.max_context_len);
  const int nparts = L > 0 ? (L + p.partition - 1) / p.partition : 0;
  if (nparts <= 1) return;
  const int kvh = unit / p.n_sub;
  const int h0 = kvh * p.group + (unit - kvh * p.n_sub) * GT;
  const int dc = lane % LPT;
  const int tr = lane / LPT;
  const int64_t mp = p.max_parts;

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    m[h] = NEG_BIG;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
  }
  for (int pp = tr; pp < nparts; pp += TPW) {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const int64_t sh = (int64_t)seq * p.num_heads + h0 + h;
      const float2 ml = *reinterpret_cast<const float2*>(p.ws_ml + (sh * mp + pp) * 2);
      const float* src = p.ws_acc + (sh * mp + pp) * D + dc * EPL;
      const float mn = fmaxf(m[h], ml.x);
      const float a = fast_exp2(m[h] - mn);
      const float b = fast_exp2(ml.x - mn);
      l[h] = l[h] * a + ml.y * b;
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + e);
        acc[h][e] = acc[h][e] * a + v.x * b;
        acc[h][e + 1] = acc[h][e + 1] * a + v.y * b;
        acc[h][e + 2] = acc[h][e + 2] * a + v.z * b;
        acc[h][e + 3] = acc[h][e + 3] * a + v.w * b;
      }
      m[h] = mn;
    }
  }
  merge_row_groups<LPT, GT, EPL>(m, l, acc);
  if (tr == 0) {
    char* const out_base = static_cast<char*>(p.out);
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      float o[EPL];
      const float inv = 1.0f / l[h];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = acc[h][e] * inv;
      store_slice<T, EPL>(out_base + (((int64_t)seq * p.num_heads + h0 + h) * D + dc * EPL) * E, o);
    }
  }
}

// ---------------------------------------------------------------------------
// planning and launch
// ---------------------------------------------------------------------------

static int32_t heads_per_unit(int32_t group) {
  for (int32_t g : {8, 4, 2}) {
    if (group % g == 0) return g;
  }
  return 1;
}

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

DecodePlan plan_decode(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t max_context_len, int32_t partition_size) {
  DecodePlan pl{};
  pl.group = num_heads / num_kv_heads;
  pl.heads_per_unit = heads_per_unit(pl.group);
  pl.units = num_kv_heads * (pl.group / pl.heads_per_unit);
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

template <typename T, int D, int GT, int U>
static void launch_u(const DecodeParams& prm, dim3 grid, bool split, hipStream_t stream) {
  constexpr int TPW = 64 / (D * (int)sizeof(T) / 16);
  constexpr int CT = U * TPW;
  const bool uniform = (1 << prm.bs_log2) >= CT && (prm.max_parts == 1 || prm.partition % CT == 0);
  if (uniform)
    hipLaunchKernelGGL((paged_decode_kernel<T, D, GT, U, true>), grid, dim3(256), 0, stream, prm);
  else
    hipLaunchKernelGGL((paged_decode_kernel<T, D, GT, U, false>), grid, dim3(256), 0, stream, prm);
  if (split)
    hipLaunchKernelGGL((paged_decode_merge_kernel<T, D, GT>), dim3(grid.z, (grid.x)), dim3(256), 0,
                       stream, prm);
}

template <typename T, int D, int GT>
static void launch_one(const DecodeParams& prm, dim3 grid, bool split, hipStream_t stream) {
  launch_u<T, D, GT, DECODE_U>(prm, grid, split, stream);
}

template <typename T, int D>
static void launch_gt(int gt, const DecodeParams& prm, dim3 grid, bool split, hipStream_t stream) {
  switch (gt) {
    case 1: launch_one<T, D, 1>(prm, grid, split, stream); break;
    case 2: launch_one<T, D, 2>(prm, grid, split, stream); break;
    case 4: launch_one<T, D, 4>(prm, grid, split, stream); break;
    default: launch_one<T, D, 8>(prm, grid, split, stream); break;
  }
}

hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& pl, hipStream_t stream) {
  DecodeParams prm{};
  prm.out = a.out;
  prm.q = a.q;
  prm.k_cache = static_cast<const char*>(a.k_cache);
  prm.v_cache = static_cast<const char*>(a.v_cache);
  prm.block_tables = a.block_tables;
  prm.context_lens = a.context_lens;
  if (pl.total_bytes) {
    char* ws = static_cast<char*>(a.workspace);
    prm.ws_acc = reinterpret_cast<float*>(ws);
    prm.ws_ml = reinterpret_cast<float*>(ws + pl.acc_bytes);
  }
  prm.num_heads = a.num_heads;
  prm.num_kv_heads = a.num_kv_heads;
  prm.group = pl.group;
  prm.n_sub = pl.group / pl.heads_per_unit;
  prm.units = pl.units;
  prm.bs_log2 = __builtin_ctz((unsigned)a.block_size);
  prm.num_blocks = a.num_blocks;
  prm.max_blocks_per_seq = a.max_blocks_per_seq;
  prm.max_context_len = a.max_context_len;
  prm.partition = pl.partition;
  prm.max_parts = pl.max_parts;
  prm.scale_log2 = a.scale * 1.4426950408889634f;
  prm.row_bytes = a.num_kv_heads * a.head_dim * (a.bf16 ? 2 : 4);
  prm.block_bytes = (int64_t)a.block_size * prm.row_bytes;
  // x: head group (fastest, so one token's rows of all heads are read by
  // neighbouring workgroups), y: partition, z: sequence.
  const dim3 grid((unsigned)((pl.units + 3) / 4), (unsigned)pl.max_parts, (unsigned)a.num_seqs);
  const bool split = pl.max_parts > 1;
  if (a.bf16) {
    if (a.head_dim == 64) launch_gt<uint16_t, 64>(pl.heads_per_unit, prm, grid, split, stream);
    else launch_gt<uint16_t, 128>(pl.heads_per_unit, prm, grid, split, stream);
  } else {
    if (a.head_dim == 64) launch_gt<float, 64>(pl.heads_per_unit, prm, grid, split, stream);
    else launch_gt<float, 128>(pl.heads_per_unit, prm, grid, split, stream);
  }
  return hipGetLastError();
}

}  // namespace pa
