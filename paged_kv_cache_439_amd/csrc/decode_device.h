// Decode kernels (device code) of libpagedattn; planning and launch are in
// decode.hip, the mixed prefill+decode launch in mixed.hip.
//
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
//   grid = (ceil(units per (seq, partition) / 4), sequences, max partitions),
//   256 threads = 4 independent waves, no barriers (LDS only for the
//   balanced split's chunk prefix sums and attend_range_mfma's per-wave K
//   tiles).
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
//        merged once at the end with the exact max-rescaling merge. With
//        GT >= 2 heads per wave the softmax is spread over lanes (lane dc
//        owns head dc % GT: one exp per token and lane instead of GT; the
//        probabilities reach the other lanes of the quad by DPP) and the
//        running maximum is raised lazily (only past a 2^16 margin).
//   PV:  acc[h][slice] += p * V-slice, all in registers; with GT >= 2 and
//        bf16 outputs, two tokens at a time on v_dot2_f32_bf16 (the
//        probabilities rounded to bf16, the values widened exactly).
//   bf16 queries at head_dim 128 with GT = 2 or 4 take the logits on the
//        matrix cores instead (attend_range_mfma): K is transposed through
//        a wave-private LDS tile into the B operand of
//        v_mfma_f32_16x16x32_bf16, one logit per lane and 16-token tile.
// Split: each partition writes (m, l, acc) in fp32 to the workspace and a
//   second, small kernel (paged_decode_merge_kernel) combines them with the
//   exact max-rescaling merge. The kernel boundary makes the states visible
//   across the chip's separate L2 caches once, instead of a cache writeback
//   per wave.
//
// Bound: HBM. Algorithmic bytes = context rows x 2 (K and V) x Hkv x D x e.

#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

#ifndef DECODE_U
#define DECODE_U 8
#endif
// Loads in flight per lane for E4M3 pools (16 elements per load), balanced
// split.
#ifndef DECODE_U_E4M3
#define DECODE_U_E4M3 8
#endif
// Resident waves per SIMD the balanced split plans for.
#ifndef DECODE_BAL_WAVES_PER_SIMD
#define DECODE_BAL_WAVES_PER_SIMD 2
#endif

namespace pa {

struct DecodeParams {
  void* out;
  const void* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* shared_lens;  // [B] leading tokens in blocks other sequences read, or null
  float* ws_acc;     // fixed split: [B][Hq][max_parts][D]
  float* ws_ml;      // fixed split: [B][Hq][max_parts][2]
  float* part_acc;   // balanced split: [workers][2 slots][Hq][D]
  float* part_ml;    // balanced split: [workers][2 slots][Hq][2]
  int32_t* ws_pfx;   // balanced split: chunk prefix sums [B + 1]
  int32_t num_seqs, workers;  // balanced split: workers per unit
  int32_t num_heads, num_kv_heads, group, n_sub, units;
  int32_t pair;         // balanced split: 1 when a unit is a pair of KV heads (units = Hkv / 2)
  int32_t bs_log2, num_blocks, max_blocks_per_seq, max_context_len;
  int32_t partition, max_parts;
  int32_t row_bytes;    // Hkv * D * e: bytes between consecutive tokens of a block
  int64_t block_bytes;  // block_size * row_bytes
  float scale_log2;     // scale * log2(e): logits are kept in log2 units
  // Fused store (pa_store_decode), else null: sequence i's newest K/V row
  // [Hkv][D] at new_k + i*new_k_stride, to be written at slot_mapping[i].
  const char* new_k;
  const char* new_v;
  int64_t new_k_stride, new_v_stride;  // bytes
  const int32_t* slot_mapping;
  int64_t num_slots;  // num_blocks * block_size
  // E4M3 pools: per-KV-head scales (element = value(code) * scale[head]), else null.
  const float* k_scale;
  const float* v_scale;
  int32_t fixed_order;  // fixed split: dispatch positions take items longest-first (fixed_item)
};

// Fused store + decode is built for pools in the query type and for E4M3
// pools with bf16 queries (with fp32 queries the four-head E4M3 kernel
// would spill registers inside its streaming loop).
template <typename T, typename KT>
constexpr bool fused_store_supported() {
  return sizeof(KT) == sizeof(T) || sizeof(T) == 2;
}

// Fused store: does this call write sequence seq's newest row into the pool
// (the same test pa_store_kvcache applies to a slot)?
__device__ __forceinline__ bool stores_new_row(const DecodeParams& p, int seq) {
  if (p.new_k == nullptr) return false;
  const int32_t s = p.slot_mapping[seq];
  return s >= 0 && (int64_t)s < p.num_slots;
}

// Fused store: write the newest rows of sequences into the pools, 16 pool
// bytes per thread: (sequence, granule) pairs first, first + stride, ...
// below end (pairs numbered sequence-major, row_bytes / 16 granules per
// sequence). Pools in the input type T take a copy; E4M3 pools (KT =
// uint8_t) take the codes of 16 input elements of one head, quantised as
// pa_store_kvcache_fp8 quantises them.
template <typename T, typename KT>
__device__ __forceinline__ void store_new_rows(const DecodeParams& p, int64_t first, int64_t stride,
                                               int64_t end) {
  const int32_t cpr = p.row_bytes / 16;
  end = min(end, (int64_t)p.num_seqs * cpr);
  for (int64_t idx = first; idx < end; idx += stride) {
    const int64_t t = idx / cpr;
    const int32_t c = (int32_t)(idx - t * cpr);
    if (!stores_new_row(p, (int)t)) continue;
    const int64_t dst = (int64_t)p.slot_mapping[t] * p.row_bytes + (int64_t)c * 16;
    uint4 kv, vv;
    if constexpr (sizeof(KT) == 1) {
      const int32_t h = c / (cpr / p.num_kv_heads);
      const int64_t src = (int64_t)c * 16 * (int64_t)sizeof(T);
      kv = quantize16<T>(p.new_k + t * p.new_k_stride + src, p.k_scale[h]);
      vv = quantize16<T>(p.new_v + t * p.new_v_stride + src, p.v_scale[h]);
    } else {
      kv = *reinterpret_cast<const uint4*>(p.new_k + t * p.new_k_stride + (int64_t)c * 16);
      vv = *reinterpret_cast<const uint4*>(p.new_v + t * p.new_v_stride + (int64_t)c * 16);
    }
    *reinterpret_cast<uint4*>(const_cast<char*>(p.k_cache) + dst) = kv;
    *reinterpret_cast<uint4*>(const_cast<char*>(p.v_cache) + dst) = vv;
  }
}

// 16-byte load of pool data. Every K/V byte is read once per call, so the
// loads carry the nontemporal hint and do not displace reusable lines --
// except when a head's row is shorter than a 128-byte line (E4M3, head_dim
// 64): the other half of each line belongs to the neighbouring KV head,
// which a sibling wave of the same workgroup reads moments later, and a
// plain load keeps it in L2 for that read (measured: 7% faster there, 1-8%
// slower everywhere else).
template <bool NT>
__device__ __forceinline__ uint4 stream_load(const char* ptr) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 v;
  if constexpr (NT) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ptr));
  else v = *reinterpret_cast<const u32x4*>(ptr);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte load of pool data that other sequences also read (a shared
// prefix block): the default policy keeps the lines in L2 for them. The
// compiler must not take these loads for the nontemporal ones of the other
// branch and hoist the pair out of the branches, which drops the hint from
// both: the caller issues them in another order (V before K), and they are
// typed with 8-byte alignment (still one global_load_dwordx4 each).
__device__ __forceinline__ uint4 shared_load(const char* ptr) {
  typedef unsigned int u32x4a8 __attribute__((ext_vector_type(4), aligned(8)));
  const u32x4a8 v = *reinterpret_cast<const u32x4a8*>(ptr);
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
template <>
struct ElemTraits<uint8_t> {  // E4M3 storage (KV pools only)
  static constexpr int E = 1;
};

// E4M3 -> two bf16 (exact: every E4M3 value is a bf16 value) from byte
// pair HI (0: bytes 0-1, 1: bytes 2-3) of w.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
// E4M3 -> two fp32 from byte pair HI of w.
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

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
  if constexpr (sizeof(T) == 1) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x2 a = e4m3x2_to_f32x2<false>(w[i]);
      const f32x2 b = e4m3x2_to_f32x2<true>(w[i]);
      f[4 * i] = a.x; f[4 * i + 1] = a.y; f[4 * i + 2] = b.x; f[4 * i + 3] = b.y;
    }
  } else if constexpr (sizeof(T) == 2) {
    f[0] = bf16lo(v.x); f[1] = bf16hi(v.x);
    f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
    f[4] = bf16lo(v.z); f[5] = bf16hi(v.z);
    f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
  } else {
    f[0] = __builtin_bit_cast(float, v.x); f[1] = __builtin_bit_cast(float, v.y);
    f[2] = __builtin_bit_cast(float, v.z); f[3] = __builtin_bit_cast(float, v.w);
  }
}

// Store EPL floats as EPL consecutive elements of the output type T, in
// 16-byte pieces.
template <typename T, int EPL>
__device__ __forceinline__ void store_slice(void* dst, const float (&f)[EPL]) {
  constexpr int PER = 16 / (int)sizeof(T);  // elements per 16-byte piece
  static_assert(EPL % PER == 0, "slice must be whole 16-byte pieces");
#pragma unroll
  for (int c = 0; c < EPL / PER; ++c) {
    const float* g = f + c * PER;
    uint4 w;
    if constexpr (sizeof(T) == 2) {
      w.x = pack_bf16x2(g[0], g[1]); w.y = pack_bf16x2(g[2], g[3]);
      w.z = pack_bf16x2(g[4], g[5]); w.w = pack_bf16x2(g[6], g[7]);
    } else {
      w.x = __builtin_bit_cast(uint32_t, g[0]); w.y = __builtin_bit_cast(uint32_t, g[1]);
      w.z = __builtin_bit_cast(uint32_t, g[2]); w.w = __builtin_bit_cast(uint32_t, g[3]);
    }
    reinterpret_cast<uint4*>(dst)[c] = w;
  }
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

// The online-softmax state of one wave: per head of its group, the running
// maximum m (log2 units), the running sum l and the weighted value sum acc
// over this lane's d-slice, kept separately per token-row group tr.
template <int GT, int EPL>
struct WaveState {
  float m[GT], l[GT], acc[GT][EPL];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      m[h] = NEG_BIG;
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
    }
  }
};

// This lane's slice of one query head, in the form that its partial dot
// product with a 16-byte K slice of storage type KT needs.
template <typename T, typename KT>
struct QSlice {  // K in the query's own type: the raw 16 bytes
  static_assert(sizeof(T) == sizeof(KT), "K must be stored in the query type or as E4M3");
  uint4 v;
  __device__ __forceinline__ void load(const char* src) { v = *reinterpret_cast<const uint4*>(src); }
  __device__ __forceinline__ float dot(const uint4& k) const { return slice_dot<T>(v, k); }
};
template <>
struct QSlice<uint16_t, uint8_t> {  // bf16 query, E4M3 keys: 16 elements, bf16 dot2
  uint4 v[2];
  __device__ __forceinline__ void load(const char* src) {
    v[0] = reinterpret_cast<const uint4*>(src)[0];
    v[1] = reinterpret_cast<const uint4*>(src)[1];
  }
  __device__ __forceinline__ float dot(const uint4& k) const {
    float s = dot2_bf16(v[0].x, e4m3x2_to_bf16x2<false>(k.x), 0.0f);
    s = dot2_bf16(v[0].y, e4m3x2_to_bf16x2<true>(k.x), s);
    s = dot2_bf16(v[0].z, e4m3x2_to_bf16x2<false>(k.y), s);
    s = dot2_bf16(v[0].w, e4m3x2_to_bf16x2<true>(k.y), s);
    s = dot2_bf16(v[1].x, e4m3x2_to_bf16x2<false>(k.z), s);
    s = dot2_bf16(v[1].y, e4m3x2_to_bf16x2<true>(k.z), s);
    s = dot2_bf16(v[1].z, e4m3x2_to_bf16x2<false>(k.w), s);
    return dot2_bf16(v[1].w, e4m3x2_to_bf16x2<true>(k.w), s);
  }
};
template <>
struct QSlice<float, uint8_t> {  // fp32 query, E4M3 keys: 16 elements, fp32 FMA
  float f[16];
  __device__ __forceinline__ void load(const char* src) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 x = reinterpret_cast<const float4*>(src)[c];
      f[4 * c] = x.x; f[4 * c + 1] = x.y; f[4 * c + 2] = x.z; f[4 * c + 3] = x.w;
    }
  }
  __device__ __forceinline__ float dot(const uint4& k) const {
    float kf[16];
    widen_slice<uint8_t, 16>(k, kf);
    float s = f[0] * kf[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) s = fmaf(f[e], kf[e], s);
    return s;
  }
};

// Load this lane's q slices (EPL elements from element dc*EPL) of heads
// h0 .. h0+GT-1 of sequence seq.
template <typename T, typename KT, int D, int GT>
__device__ __forceinline__ void load_q(const DecodeParams& p, int seq, int h0, int dc,
                                       QSlice<T, KT> (&qv)[GT]) {
  constexpr int E = ElemTraits<T>::E;
  constexpr int EPL = 16 / ElemTraits<KT>::E;
  const char* qb = static_cast<const char*>(p.q);
#pragma unroll
  for (int h = 0; h < GT; ++h)
    qv[h].load(qb + (((int64_t)seq * p.num_heads + h0 + h) * D + dc * EPL) * E);
}

// Logit multiplier of a KV head, log2 units: scale * log2(e), times the
// head's K scale for an E4M3 pool.
template <typename KT>
__device__ __forceinline__ float logit_scale(const DecodeParams& p, int kvh) {
  if constexpr (sizeof(KT) == 1) return p.scale_log2 * p.k_scale[kvh];
  return p.scale_log2;
}

// E4M3 pool: the weighted sums were taken over V codes' values; multiply by
// the head's V scale (every token of a KV head shares it).
template <typename KT, int GT, int EPL>
__device__ __forceinline__ void apply_v_scale(const DecodeParams& p, int kvh, float (&acc)[GT][EPL]) {
  if constexpr (sizeof(KT) == 1) {
    const float vs = p.v_scale[kvh];
#pragma unroll
    for (int h = 0; h < GT; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= vs;
  }
}

// Waves serving GT >= 2 query heads spread the softmax over lanes: lane
// (dc, tr) owns head dc % GT of its token rows, so each logit's exp is taken
// once per GT lanes instead of in every lane, and the probabilities reach
// the other lanes of the quad by DPP.
//
// The value v of the lane owning head H, among the GT consecutive lanes
// that share this lane's rows (quad_perm broadcast within each quad).
template <int GT, int H>
__device__ __forceinline__ uint32_t from_head_owner(uint32_t v) {
  static_assert(GT == 2 || GT == 4, "heads per wave");
  constexpr int CTRL = GT == 4 ? H * 0x55 : (H | (H << 2) | ((2 + H) << 4) | ((2 + H) << 6));
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int GT, int H>
__device__ __forceinline__ float from_head_owner(float v) {
  return __builtin_bit_cast(float, from_head_owner<GT, H>(__builtin_bit_cast(uint32_t, v)));
}
// This lane's own entry of t[GT] (head myh = dc % GT), chosen with bitwise
// selects on lane masks: written as a conditional, the choice becomes a
// dynamically indexed private array, whose scratch reads wait on every
// outstanding global load.
__device__ __forceinline__ float bit_select(uint32_t mask, float if_set, float if_clear) {
  const uint32_t a = __builtin_bit_cast(uint32_t, if_set), b = __builtin_bit_cast(uint32_t, if_clear);
  return __builtin_bit_cast(float, (a & mask) | (b & ~mask));
}
template <int GT>
__device__ __forceinline__ float own_head(const float (&t)[GT], int myh) {
  const uint32_t m0 = 0u - (uint32_t)(myh & 1);
  if constexpr (GT == 2) {
    return bit_select(m0, t[1], t[0]);
  } else {
    const uint32_t m1 = 0u - (uint32_t)((myh >> 1) & 1);
    return bit_select(m1, bit_select(m0, t[3], t[2]), bit_select(m0, t[1], t[0]));
  }
}
template <int GT, typename F>
__device__ __forceinline__ void for_heads(F&& f) {
  f(std::integral_constant<int, 0>{});
  f(std::integral_constant<int, 1>{});
  if constexpr (GT == 4) {
    f(std::integral_constant<int, 2>{});
    f(std::integral_constant<int, 3>{});
  }
}

// Lazy rescale of the spread softmax (log2 units): the running maximum is
// raised, and the accumulators rescaled, only when a logit exceeds it by
// more than this, so probabilities stay below 2^16 (exact range for bf16 and
// fp32, and a row sum of up to 2^16 per key cannot overflow fp32).
constexpr float DECODE_RESCALE_SLACK = 16.0f;

// acc[h][*] += p_u[h] v_u + p_u1[h] v_u1 for the EPL elements of two tokens'
// 16-byte V slices, with the probabilities of both tokens packed as bf16
// pairs (pp[h]: low half token u) and the values widened exactly to bf16,
// paired across the two tokens by v_perm, one v_dot2_f32_bf16 per element.
template <typename KT, int GT, int EPL>
__device__ __forceinline__ void pv_token_pair(const uint4& vu, const uint4& vu1, const uint32_t (&pp)[GT],
                                              float (&acc)[GT][EPL]) {
  const uint32_t a[4] = {vu.x, vu.y, vu.z, vu.w};
  const uint32_t b[4] = {vu1.x, vu1.y, vu1.z, vu1.w};
  constexpr uint32_t LO = 0x05040100u, HI = 0x07060302u;  // (a.lo16, b.lo16), (a.hi16, b.hi16)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (sizeof(KT) == 1) {  // 4 E4M3 codes per dword
      const uint32_t a01 = e4m3x2_to_bf16x2<false>(a[i]), a23 = e4m3x2_to_bf16x2<true>(a[i]);
      const uint32_t b01 = e4m3x2_to_bf16x2<false>(b[i]), b23 = e4m3x2_to_bf16x2<true>(b[i]);
      const uint32_t e[4] = {__builtin_amdgcn_perm(b01, a01, LO), __builtin_amdgcn_perm(b01, a01, HI),
                             __builtin_amdgcn_perm(b23, a23, LO), __builtin_amdgcn_perm(b23, a23, HI)};
#pragma unroll
      for (int h = 0; h < GT; ++h)
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[h][4 * i + k] = dot2_bf16(pp[h], e[k], acc[h][4 * i + k]);
    } else {  // 2 bf16 per dword
      const uint32_t lo = __builtin_amdgcn_perm(b[i], a[i], LO), hi = __builtin_amdgcn_perm(b[i], a[i], HI);
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        acc[h][2 * i] = dot2_bf16(pp[h], lo, acc[h][2 * i]);
        acc[h][2 * i + 1] = dot2_bf16(pp[h], hi, acc[h][2 * i + 1]);
      }
    }
  }
}

// Fused store: the newest token of sequence seq (KV head kvh), taken from
// the new row itself (over E4M3 pools, as the codes the store writes), into
// the state st with the exact max-rescaling update. Token-row group 0 holds
// it (every lane loads the same row so that the butterfly over the row's
// lanes stays uniform); lane dc holds the row's slice dc.
template <typename T, typename KT, int D, int GT>
__device__ __forceinline__ void attend_new_row(const DecodeParams& p, int seq, int kvh, int dc, int tr,
                                               const QSlice<T, KT> (&qv)[GT], float sm,
                                               WaveState<GT, 16 / ElemTraits<KT>::E>& st) {
  constexpr int E = ElemTraits<KT>::E;
  constexpr int EPL = 16 / E;
  constexpr int LPT = D / EPL;
  uint4 kr, vr;
  if constexpr (E == 1) {  // E4M3 pools: this lane's 16 elements, quantised
    const int64_t src = ((int64_t)kvh * D + dc * 16) * (int64_t)sizeof(T);
    kr = quantize16<T>(p.new_k + seq * p.new_k_stride + src, p.k_scale[kvh]);
    vr = quantize16<T>(p.new_v + seq * p.new_v_stride + src, p.v_scale[kvh]);
  } else {
    const int64_t off = (int64_t)kvh * D * E + dc * 16;
    kr = *reinterpret_cast<const uint4*>(p.new_k + seq * p.new_k_stride + off);
    vr = *reinterpret_cast<const uint4*>(p.new_v + seq * p.new_v_stride + off);
  }
  float vf[EPL];
  widen_slice<KT, EPL>(vr, vf);
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    float sc = group_sum<LPT>(qv[h].dot(kr)) * sm;
    sc = (tr == 0) ? sc : -INFINITY;
    const float mn = fmaxf(st.m[h], sc);
    const float alpha = fast_exp2(st.m[h] - mn);
    const float pr = fast_exp2(sc - mn);
    st.m[h] = mn;
    st.l[h] = st.l[h] * alpha + pr;
#pragma unroll
    for (int e = 0; e < EPL; ++e) st.acc[h][e] = fmaf(pr, vf[e], st.acc[h][e] * alpha);
  }
}

// The pool offsets of a streaming loop's chunks: lane (dc, tr) reads the
// 16-byte slice at lane_off of token rows tr, tr + TPW, ..., tr + (U-1)*TPW
// of the chunk. The block-table window (lane i holds the physical id of
// block wbase + i) slides with the chunks. UNIFORM_BLOCK: every chunk lies
// inside one block (block_size >= U*TPW and the range starts at a multiple
// of it), so one table lookup serves all lanes; otherwise each lane looks up
// its own token's block. Rows past tok_end (valid false) re-read the chunk's
// first row, so that they hold finite pool data.
//
// The loads themselves stay in each loop (issue_chunk_loads): behind a
// function boundary, LLVM sinks the last loads of the two cache-policy
// branches into one store through a selected pointer, and the chunk's
// arrays go to scratch memory.
template <int U, int TPW, bool NT, bool UNIFORM_BLOCK>
struct ChunkAddresses {
  static constexpr int CT = U * TPW;
  const char* k_cache;
  const char* v_cache;
  const int32_t* bt;
  int64_t block_bytes;
  int num_blocks, bs_log2, bs_mask, row_bytes, lane_off, lane, tr, tok_end, last_blk, wbase, tbl;
  // Tokens [0, shared_len) lie in blocks that other sequences read too
  // (prefix sharing shares leading blocks only): they are loaded with the
  // cache-retaining policy, so that the other readers find them in L2,
  // while the rest of the context streams past. Only the hint differs.
  int shared_len;

  __device__ __forceinline__ ChunkAddresses(const DecodeParams& p, int seq, int lane_, int tr_, int lane_off_,
                                         int tok_begin, int tok_end_)
      : k_cache(p.k_cache), v_cache(p.v_cache), bt(p.block_tables + (int64_t)seq * p.max_blocks_per_seq),
        block_bytes(p.block_bytes), num_blocks(p.num_blocks), bs_log2(p.bs_log2),
        bs_mask((1 << p.bs_log2) - 1), row_bytes(p.row_bytes), lane_off(lane_off_), lane(lane_), tr(tr_),
        tok_end(tok_end_) {
    shared_len = (NT && p.shared_lens != nullptr) ? p.shared_lens[seq] : 0;
    last_blk = (tok_end - 1) >> bs_log2;
    wbase = tok_begin >> bs_log2;
    tbl = (wbase + lane <= last_blk) ? clamp_block(bt[wbase + lane], num_blocks) : 0;
  }

  __device__ __forceinline__ void chunk(int j0, int64_t (&off)[U], bool (&valid)[U]) {
    const int chunk_last = (min(j0 + CT, tok_end) - 1) >> bs_log2;
    if (chunk_last >= wbase + 64) {  // uniform: slide the table window
      wbase = j0 >> bs_log2;
      tbl = (wbase + lane <= last_blk) ? clamp_block(bt[wbase + lane], num_blocks) : 0;
    }
    if constexpr (UNIFORM_BLOCK) {
      const int phys = __builtin_amdgcn_readlane(tbl, (j0 >> bs_log2) - wbase);
      const int64_t base = (int64_t)phys * block_bytes;
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
      for (int u = 0; u < U; ++u) off[u] = (int64_t)phys[u] * block_bytes + (row[u] * row_bytes + lane_off);
    }
  }
};

// Every K and V load of a chunk at the offsets ca.chunk gave, issued before
// any of them is used (a macro so that the branches stay in the loop body).
#define PA_ISSUE_CHUNK_LOADS(ca, j0, off, kr, vr, U, NT)                                \
  do {                                                                                   \
    if ((j0) < (ca).shared_len) { /* V first: see shared_load */                         \
      _Pragma("unroll") for (int u_ = 0; u_ < (U); ++u_) (vr)[u_] = shared_load((ca).v_cache + (off)[u_]); \
      _Pragma("unroll") for (int u_ = 0; u_ < (U); ++u_) (kr)[u_] = shared_load((ca).k_cache + (off)[u_]); \
    } else {                                                                             \
      _Pragma("unroll") for (int u_ = 0; u_ < (U); ++u_) (kr)[u_] = stream_load<NT>((ca).k_cache + (off)[u_]); \
      _Pragma("unroll") for (int u_ = 0; u_ < (U); ++u_) (vr)[u_] = stream_load<NT>((ca).v_cache + (off)[u_]); \
    }                                                                                    \
  } while (0)

// Issue priority of a balanced-split wave from the share of its own range
// still to do (rest of total tokens: above 1/2, 1/4, 1/8, or less): a wave
// that has fallen behind the other wave of its SIMD wins the issue slots
// until it has caught up. Waves with equal chunk counts otherwise end far
// apart: the older workgroup of a CU wins the arbitration, and some XCDs
// stream more slowly than others.
__device__ __forceinline__ void set_progress_prio(int rest, int total) {
  const int r = __builtin_amdgcn_readfirstlane(rest), t = __builtin_amdgcn_readfirstlane(total);
  const int lvl = 2 * r > t ? 3 : 4 * r > t ? 2 : 8 * r > t ? 1 : 0;
  if (lvl >= 3) __builtin_amdgcn_s_setprio(3);
  else if (lvl == 2) __builtin_amdgcn_s_setprio(2);
  else if (lvl == 1) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Stream tokens [tok_begin, tok_end) of sequence seq (KV head kvh) through
// the online softmax of st. UNIFORM_BLOCK: every chunk lies inside one block
// (block_size >= CT and tok_begin a multiple of CT), so one table lookup per
// chunk serves all lanes; otherwise each lane looks up its own token's block.
// KT is the pools' storage type: T itself, or uint8_t for E4M3 codes, whose
// logits are multiplied by sm (the logit scale times the head's K scale)
// and whose weighted value sums still lack the head's V scale.
//
// PAIR (E4M3 pools, head_dim 64, one query head per wave): the wave reads two
// adjacent KV heads, so that each token row it reads is one whole 128-byte
// line; lanes 0-3 of every 8 hold the first head's slices and lanes 4-7 the
// second's, kvh is this lane's own head, and each head keeps its own
// online-softmax state (the dot products reduce over 4 lanes).
template <typename T, typename KT, int D, int GT, int U, bool UNIFORM_BLOCK, bool PAIR = false>
__device__ __forceinline__ void attend_range(const DecodeParams& p, int seq, int kvh, int lane,
                                             int tok_begin, int tok_end,
                                             const QSlice<T, KT> (&qv)[GT], float sm,
                                             WaveState<GT, 16 / ElemTraits<KT>::E>& st,
                                             int prio_rest = 0, int prio_total = 0) {
  // With a fused store, the newest token (position L-1, L = the context
  // length) comes from the new row itself, not from the pool slot this same
  // launch is writing (over E4M3 pools, as the codes the store writes).
  constexpr bool FUSABLE = fused_store_supported<T, KT>();
  const bool new_row = FUSABLE && tok_end > tok_begin && stores_new_row(p, seq) &&
                       tok_end == min(p.context_lens[seq], p.max_context_len);
  if (new_row) --tok_end;
  constexpr int E = ElemTraits<KT>::E;
  constexpr int EPL = 16 / E;     // elements per 16-byte lane slice
  constexpr int LPT = D / EPL;    // lanes per token row of one head
  constexpr int LPR = PAIR ? 2 * LPT : LPT;  // lanes per token row the wave reads
  constexpr int TPW = 64 / LPR;   // token rows per wave-wide load
  constexpr int CT = U * TPW;     // tokens per chunk
  constexpr bool NT = LPR * 16 >= 128;  // whole lines per row read: streaming hint
  static_assert(!PAIR || (GT == 1 && LPR * 16 == 128), "pairs: one head per lane group, whole lines");
  const int dc = lane % LPT;
  const int tr = lane / LPR;

  // Spread softmax (GT >= 2): this lane's head, its running maximum and sum.
  // bf16 outputs take the V product on v_dot2 with the probabilities rounded
  // to bf16 (the row sum adds the same rounded values); fp32 outputs keep
  // fp32 probabilities and FMAs.
  constexpr bool SPREAD = GT >= 2;
  constexpr bool PV_BF16 = SPREAD && sizeof(T) == 2;
  const int myh = dc % GT;
  float mm = 0.0f, ll = 0.0f;
  if constexpr (SPREAD) {
    mm = own_head<GT>(st.m, myh);
    ll = own_head<GT>(st.l, myh);
  }

  ChunkAddresses<U, TPW, NT, UNIFORM_BLOCK> ca(p, seq, lane, tr, kvh * D * E + dc * 16, tok_begin, tok_end);
  for (int j0 = tok_begin; j0 < tok_end; j0 += CT) {
    // priority from the work left (prio_total > 0: a balanced-split wave, every 4 chunks)
    if (prio_total > 0 && ((j0 - tok_begin) & (4 * CT - 1)) == 0)
      set_progress_prio(prio_rest + tok_end - j0, prio_total);
    // the whole chunk's bytes are in flight before any of them is waited on
    bool valid[U];
    int64_t off[U];
    ca.chunk(j0, off, valid);
    uint4 kr[U], vr[U];
    PA_ISSUE_CHUNK_LOADS(ca, j0, off, kr, vr, U, NT);
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (SPREAD) {
      float sc[U];
      float cm = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float t[GT];
#pragma unroll
        for (int h = 0; h < GT; ++h) t[h] = group_sum<LPT>(qv[h].dot(kr[u]));
        // branch-free (a conditional here becomes a branch per token)
        sc[u] = bit_select(0u - (uint32_t)valid[u], own_head<GT>(t, myh) * sm, -INFINITY);
        cm = fmaxf(cm, sc[u]);
      }
      if (__any(cm > mm + DECODE_RESCALE_SLACK)) {  // raise the maximum (wave-uniform)
        const float mn = fmaxf(mm, cm);
        const float alpha = fast_exp2(mm - mn);
        mm = mn;
        ll *= alpha;
        for_heads<GT>([&](auto H) {
          const float a = from_head_owner<GT, H.value>(alpha);
#pragma unroll
          for (int e = 0; e < EPL; ++e) st.acc[H.value][e] *= a;
        });
      }
      if constexpr (PV_BF16) {
        static_assert(U % 2 == 0, "token pairs");
#pragma unroll
        for (int u = 0; u < U; u += 2) {
          const uint32_t mine = pack2_bf16(fast_exp2(sc[u] - mm), fast_exp2(sc[u + 1] - mm));
          ll = dot2_bf16(mine, 0x3F803F80u, ll);  // + both rounded probabilities
          uint32_t pp[GT];
          for_heads<GT>([&](auto H) { pp[H.value] = from_head_owner<GT, H.value>(mine); });
          pv_token_pair<KT, GT, EPL>(vr[u], vr[u + 1], pp, st.acc);
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float pu = fast_exp2(sc[u] - mm);
          ll += pu;
          float ph[GT];
          for_heads<GT>([&](auto H) { ph[H.value] = from_head_owner<GT, H.value>(pu); });
          float vf[EPL];
          widen_slice<KT, EPL>(vr[u], vf);
#pragma unroll
          for (int h = 0; h < GT; ++h)
#pragma unroll
            for (int e = 0; e < EPL; ++e) st.acc[h][e] = fmaf(ph[h], vf[e], st.acc[h][e]);
        }
      }
    } else {
      float s[U][GT];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < GT; ++h) s[u][h] = group_sum<LPT>(qv[h].dot(kr[u]));

#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float cm = NEG_BIG;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          s[u][h] = valid[u] ? s[u][h] * sm : -INFINITY;
          cm = fmaxf(cm, s[u][h]);
        }
        const float mn = fmaxf(st.m[h], cm);
        const float alpha = fast_exp2(st.m[h] - mn);
        st.m[h] = mn;
        st.l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.acc[h][e] *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          s[u][h] = fast_exp2(s[u][h] - mn);
          st.l[h] += s[u][h];
        }
      }

#pragma unroll
      for (int u = 0; u < U; ++u) {
        float vf[EPL];
        widen_slice<KT, EPL>(vr[u], vf);
#pragma unroll
        for (int h = 0; h < GT; ++h)
#pragma unroll
          for (int e = 0; e < EPL; ++e) st.acc[h][e] = fmaf(s[u][h], vf[e], st.acc[h][e]);
      }
    }
  }

  if constexpr (SPREAD) {  // every lane gets every head's (m, l) back
    for_heads<GT>([&](auto H) {
      st.m[H.value] = from_head_owner<GT, H.value>(mm);
      st.l[H.value] = from_head_owner<GT, H.value>(ll);
    });
  }

  if constexpr (FUSABLE) {
    if (new_row) attend_new_row<T, KT, D, GT>(p, seq, kvh, dc, tr, qv, sm, st);
  }
}

// attend_range with the logits on the matrix cores, for bf16 queries over
// bf16 or E4M3 pools (head_dim 128, GT = 2 or 4 query heads of one KV head
// per wave). Loads and the PV product are attend_range's: lane (dc, tr)
// holds the 16-byte slices dc of token rows tr, tr + TPW, ... (TPW = 4 rows
// of bf16 or 8 of E4M3 per load), and PV pairs the rows of loads u and
// u + 1 on v_dot2. The rest differs:
//   * tokens go in 16-token tiles (16 / TPW loads). Load v of a tile, row
//     tr, is tile column c = tr + 8 (v & 1) + 4 (v >> 1), so that the two
//     rows every PV pair combines sit in columns c and c ^ 8;
//   * the K slices go through a wave-private LDS tile and come back
//     transposed: lane 16g + c holds dims 32g .. 32g+31 of column c's
//     token, in bf16 (E4M3 codes widened exactly): the B operand (K^T, 32
//     dims x 16 tokens per step) of v_mfma_f32_16x16x32_bf16. Granule j of
//     a row is stored at j ^ swz(c) (swz: 3 bits for the 8-granule E4M3
//     rows, 4 for the 16-granule bf16 rows), so that the row writes and the
//     transposed reads touch distinct banks (for 32 and for 64 banks);
//   * the A operand holds the GT query rows, each repeated 16 / GT times, so
//     S = Q K^T leaves lane 16g + c with the logit of head g * GT / 4 and
//     column c in all four of its result registers: one logit, one
//     exponential per lane and tile, instead of GT dot products reduced
//     over the lanes of a token row;
//   * the running maximum is kept per head, equal in all lanes of the head,
//     and raised lazily past the same margin as the spread softmax, so that
//     the probabilities of all tokens of a head share it;
//   * each lane packs its probability with that of column c ^ 8 (DPP) and
//     the PV lanes fetch the pairs of their row tr from lanes 16g + tr + 4q
//     (pair q of the tile; ds_bpermute).
// st is reset here; on return each lane holds, per head, the shared
// maximum, the probability sum of its row group's tokens and the weighted V
// sums of its slice, as attend_range leaves them.
template <typename T, typename KT, int D, int GT, int U, bool UNIFORM_BLOCK>
__device__ __forceinline__ void attend_range_mfma(const DecodeParams& p, int seq, int kvh, int h0, int lane,
                                                  int tok_begin, int tok_end, float sm,
                                                  WaveState<GT, 16 / ElemTraits<KT>::E>& st,
                                                  int prio_rest = 0, int prio_total = 0) {
  constexpr int E = ElemTraits<KT>::E;
  constexpr int EPL = 16 / E;       // elements per 16-byte slice
  constexpr int LPT = D / EPL;      // lanes per token row = granules per row
  constexpr int TPW = 64 / LPT;     // token rows per load
  constexpr int CT = U * TPW;       // tokens per chunk
  constexpr int LPU = 16 / TPW;     // loads per 16-token tile
  constexpr int TILES = U / LPU;
  constexpr int GL = 32 * E / 16;   // granules of a lane's 32 dims
  constexpr int REP = 16 / GT;      // rows of the A operand per head
  static_assert(sizeof(T) == 2 && (E == 1 || E == 2) && D == 128 && (GT == 2 || GT == 4) && U % LPU == 0,
                "bf16 queries, bf16 or E4M3 pools, head_dim 128, 2 or 4 heads, whole tiles");
  auto column = [](int v, int r) { return r + 8 * (v & 1) + 4 * (v >> 1); };
  auto swz = [](int c) { return TPW == 8 ? ((c & 7) ^ (c >> 3)) : c; };
  // K tile: per wave, U loads x 64 lanes x 16 bytes
  __shared__ uint4 ktile[4][U * 64];
  uint4* const kt = ktile[threadIdx.x >> 6];

  const bool new_row = tok_end > tok_begin && stores_new_row(p, seq) &&
                       tok_end == min(p.context_lens[seq], p.max_context_len);
  if (new_row) --tok_end;
  const int dc = lane % LPT, tr = lane / LPT;  // load and PV layout
  const int g = lane >> 4, c = lane & 15;      // MFMA layout
  // this lane's column as a (load of the tile, row) pair, and its token
  const int cr = c & (TPW - 1);
  const int cv = TPW == 8 ? (c >> 3) : (((c >> 3) & 1) | (((c >> 2) & 1) << 1));
  const int ctok = cv * TPW + cr;
  const int cswz = swz(c);

  // A operand of step k: Q[h0 + c / REP][32g + 8k .. 32g + 8k + 7]
  bf16x8 qa[4];
  {
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(p.q) +
                                                      (((int64_t)seq * p.num_heads + h0 + c / REP) * D + 32 * g) * 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) qa[k] = __builtin_bit_cast(bf16x8, src[k]);
  }
  // head h's logits are in lanes 16 * (h * 4 / GT) + c; a PV lane takes the
  // pair of columns tr + 4q and tr + 4q + 8 from lane 16 * (h * 4 / GT) + tr + 4q
  int src_addr[GT];
#pragma unroll
  for (int h = 0; h < GT; ++h) src_addr[h] = (16 * (h * 4 / GT) + tr) * 4;

  st.reset();
  float mm = NEG_BIG, ll = 0.0f;
  ChunkAddresses<U, TPW, true, UNIFORM_BLOCK> ca(p, seq, lane, tr, kvh * D * E + dc * 16, tok_begin, tok_end);
  for (int j0 = tok_begin; j0 < tok_end; j0 += CT) {
    // priority from the work left (prio_total > 0: a balanced-split wave, every 4 chunks)
    if (prio_total > 0 && ((j0 - tok_begin) & (4 * CT - 1)) == 0)
      set_progress_prio(prio_rest + tok_end - j0, prio_total);
    bool valid[U];  // the PV products need no mask: masked logits give zero probabilities
    int64_t off[U];
    ca.chunk(j0, off, valid);
    uint4 kr[U], vr[U];
    PA_ISSUE_CHUNK_LOADS(ca, j0, off, kr, vr, U, true);
    __builtin_amdgcn_sched_barrier(0);

#pragma unroll
    for (int u = 0; u < U; ++u) kt[u * 64 + tr * LPT + (dc ^ swz(column(u % LPU, tr)))] = kr[u];

    float s[TILES];
    float cm = -INFINITY;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const uint4* row = kt + (LPU * t + cv) * 64 + cr * LPT;
      uint32_t kw[4 * GL];
#pragma unroll
      for (int j = 0; j < GL; ++j) {
        const uint4 w = row[(GL * g + j) ^ cswz];
        kw[4 * j] = w.x; kw[4 * j + 1] = w.y; kw[4 * j + 2] = w.z; kw[4 * j + 3] = w.w;
      }
      f32x4 acc4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint4 bw;
        if constexpr (E == 1) {  // 8 codes -> 8 bf16
          bw = make_uint4(e4m3x2_to_bf16x2<false>(kw[2 * k]), e4m3x2_to_bf16x2<true>(kw[2 * k]),
                          e4m3x2_to_bf16x2<false>(kw[2 * k + 1]), e4m3x2_to_bf16x2<true>(kw[2 * k + 1]));
        } else {
          bw = make_uint4(kw[4 * k], kw[4 * k + 1], kw[4 * k + 2], kw[4 * k + 3]);
        }
        acc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[k], __builtin_bit_cast(bf16x8, bw), acc4, 0, 0, 0);
      }
      const bool ok = j0 + 16 * t + ctok < tok_end;
      s[t] = bit_select(0u - (uint32_t)ok, acc4[0] * sm, -INFINITY);
      cm = fmaxf(cm, s[t]);
    }
    if (__any(cm > mm + DECODE_RESCALE_SLACK)) {  // raise the heads' maxima (wave-uniform branch)
      float rmax = cm;
      rmax = fmaxf(rmax, dpp_f32<DPP_ROW_ROR8>(rmax));
      rmax = fmaxf(rmax, dpp_f32<DPP_ROW_ROR4>(rmax));
      rmax = fmaxf(rmax, dpp_f32<DPP_ROW_ROR2>(rmax));
      rmax = fmaxf(rmax, dpp_f32<DPP_ROW_ROR1>(rmax));
      const float mn = fmaxf(mm, rmax);
      const float alpha = fast_exp2(mm - mn);
      mm = mn;
      ll *= alpha;
      for_heads<GT>([&](auto H) {
        const float a = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), 16 * (H.value * 4 / GT)));
#pragma unroll
        for (int e = 0; e < EPL; ++e) st.acc[H.value][e] *= a;
      });
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const float pr = fast_exp2(s[t] - mm);
      const uint32_t pk = pack2_bf16(pr, dpp_f32<DPP_ROW_ROR8>(pr));  // (column c, column c ^ 8)
      ll = dot2_bf16(pk, 0x3F80u, ll);                                 // + this column's rounded probability
#pragma unroll
      for (int q = 0; q < LPU / 2; ++q) {
        uint32_t pp[GT];
#pragma unroll
        for (int h = 0; h < GT; ++h) pp[h] = (uint32_t)__builtin_amdgcn_ds_bpermute(src_addr[h] + 16 * q, (int)pk);
        pv_token_pair<KT, GT, EPL>(vr[LPU * t + 2 * q], vr[LPU * t + 2 * q + 1], pp, st.acc);
      }
    }
  }

  // every lane gets each head's maximum and its row group's probability sum
  // (columns tr + 4q and tr + 4q + 8 for every pair q)
  float lsum = ll + dpp_f32<DPP_ROW_ROR8>(ll);
  if constexpr (LPU == 4) lsum += dpp_f32<DPP_ROW_ROR4>(lsum);  // either direction: lsum(c ^ 8) = lsum(c)
  for_heads<GT>([&](auto H) {
    st.m[H.value] = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mm), 16 * (H.value * 4 / GT)));
    st.l[H.value] = __builtin_bit_cast(
        float, __builtin_amdgcn_ds_bpermute(src_addr[H.value], __builtin_bit_cast(int, lsum)));
  });

  if (new_row) {
    QSlice<T, KT> qv[GT];
    load_q<T, KT, D, GT>(p, seq, h0, dc, qv);
    attend_new_row<T, KT, D, GT>(p, seq, kvh, dc, tr, qv, sm, st);
  }
}

// Does a wave of this kernel take its logits on the matrix cores? MFMA_OK:
// the kernel can spare what attend_range_mfma needs beyond attend_range:
// 16 * U KiB of LDS for the K tiles per workgroup (the mixed prefill +
// decode kernel cannot: its prefill stages hold that LDS) and about 20 more
// registers (the fixed split over bf16 pools, built for 3 workgroups per
// CU, would spill).
template <typename T, typename KT, int D, int GT, int U, bool PAIR, bool MFMA_OK>
constexpr bool decode_mfma_logits() {
  constexpr int rows_per_load = 64 / (D * (int)sizeof(KT) / 16);  // token rows per wave-wide load
  constexpr int loads_per_tile = 16 / rows_per_load;              // loads per 16-token tile
  return MFMA_OK && !PAIR && sizeof(T) == 2 && (sizeof(KT) == 1 || sizeof(KT) == 2) && D == 128 &&
         (GT == 2 || GT == 4) && U % loads_per_tile == 0;
}

// One wave's pass over tokens [tok_begin, tok_end) of sequence seq into a
// fresh state st: attend_range_mfma where it applies, else attend_range
// with the lane's q slices (dc: the lane's slice).
template <typename T, typename KT, int D, int GT, int U, bool UNIFORM_BLOCK, bool PAIR = false, bool MFMA_OK = true>
__device__ __forceinline__ void attend(const DecodeParams& p, int seq, int kvh, int h0, int lane, int dc,
                                       int tok_begin, int tok_end, float sm,
                                       WaveState<GT, 16 / ElemTraits<KT>::E>& st,
                                       int prio_rest = 0, int prio_total = 0) {
  if constexpr (decode_mfma_logits<T, KT, D, GT, U, PAIR, MFMA_OK>()) {
    attend_range_mfma<T, KT, D, GT, U, UNIFORM_BLOCK>(p, seq, kvh, h0, lane, tok_begin, tok_end, sm, st,
                                                      prio_rest, prio_total);
  } else {
    QSlice<T, KT> qv[GT];
    load_q<T, KT, D, GT>(p, seq, h0, dc, qv);
    st.reset();
    attend_range<T, KT, D, GT, U, UNIFORM_BLOCK, PAIR>(p, seq, kvh, lane, tok_begin, tok_end, qv, sm, st,
                                                       prio_rest, prio_total);
  }
}

// Write the (merged) state of heads h0.. of sequence seq as the final
// output: this lane's EPL elements from element dc*EPL.
template <typename T, int D, int GT, int EPL>
__device__ __forceinline__ void store_output(const DecodeParams& p, int seq, int h0, int dc,
                                             const WaveState<GT, EPL>& st) {
  constexpr int E = ElemTraits<T>::E;
  char* const out_base = static_cast<char*>(p.out);
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    float o[EPL];
    const float inv = 1.0f / st.l[h];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = st.acc[h][e] * inv;
    store_slice<T, EPL>(out_base + (((int64_t)seq * p.num_heads + h0 + h) * D + dc * EPL) * E, o);
  }
}

// Zeros for heads h0.. of sequence seq (the defined output of an empty
// context): this lane's EPL elements from element dc*EPL.
template <typename T, int D, int GT, int EPL>
__device__ __forceinline__ void store_zeros(const DecodeParams& p, int seq, int h0, int dc) {
  constexpr int E = ElemTraits<T>::E;
  char* const out_base = static_cast<char*>(p.out);
  float z[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) z[e] = 0.0f;
#pragma unroll
  for (int h = 0; h < GT; ++h)
    store_slice<T, EPL>(out_base + (((int64_t)seq * p.num_heads + h0 + h) * D + dc * EPL) * E, z);
}

// Fixed split, dispatched longest-first. Workgroups start in the order of
// their grid position, so the order of the (sequence, partition) items
// decides the tail: whole partitions all take the same time, a context's
// last partition anything up to that. Position k (over grid y and z) takes
// the k-th item of: every whole partition, partition index by partition
// index (sequences in order within one); then the partial last partitions,
// in 16 buckets of decreasing length (sequences in order within a bucket);
// then one item per empty context (its zeros and its fused store); the
// positions past the last item come last and do nothing. A list schedule of
// the b512 lognormal workload's 2149 items over 768 workgroup slots puts
// this order 3% above a perfect balance and the partition-major grid order
// 12% above; measured on that workload with 512-token slices, 720 us against
// 743 us (b64 with 256-token slices: 79 against 86 us). Each workgroup
// derives the order from the context lengths: two passes over them and four
// barriers. Used for at most FIXED_ORDER_MAX_SEQS sequences and
// FIXED_ORDER_MAX_PARTS partitions.
constexpr int FIXED_ORDER_MAX_SEQS = 4096;
constexpr int FIXED_ORDER_MAX_PARTS = 64;
constexpr int FIXED_ORDER_BUCKETS = 16;

// The item at position k: false past the last item. Called by every thread
// of the workgroup.
__device__ __forceinline__ bool fixed_item(const DecodeParams& p, int k, int& seq, int& part) {
  constexpr int NB = FIXED_ORDER_BUCKETS;
  // [0, MAXP): contexts with q + 1 whole partitions; then partials by bucket; then empty contexts
  __shared__ int cnt[FIXED_ORDER_MAX_PARTS + NB + 1];
  __shared__ int wave_total[4];
  __shared__ int pick[3];  // class (0 whole, 1 partial, 2 empty, 3 none), partition or bucket, index in class
  const int B = p.num_seqs, P = p.partition;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < FIXED_ORDER_MAX_PARTS + NB + 1; i += 256) cnt[i] = 0;
  const int per = (B + 255) / 256;
  const int s0 = min(B, tid * per), s1 = min(B, s0 + per);
  auto len = [&](int s) { return min(max(p.context_lens[s], 0), p.max_context_len); };
  __syncthreads();
  for (int s = s0; s < s1; ++s) {
    const int L = len(s), whole = L / P, rem = L - whole * P;
    if (whole > 0) atomicAdd(&cnt[whole - 1], 1);
    if (rem > 0) atomicAdd(&cnt[FIXED_ORDER_MAX_PARTS + (int)((int64_t)rem * NB / P)], 1);
    if (L == 0) atomicAdd(&cnt[FIXED_ORDER_MAX_PARTS + NB], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int kk = k, cls = 3, sel = 0;
    int in_part = 0;  // whole partitions with index q: contexts with more than q whole partitions
    for (int q = 0; q < p.max_parts; ++q) in_part += cnt[q];
    for (int q = 0; q < p.max_parts && cls == 3; ++q) {
      if (kk < in_part) { cls = 0; sel = q; } else { kk -= in_part; in_part -= cnt[q]; }
    }
    for (int b = NB - 1; b >= 0 && cls == 3; --b) {
      const int n = cnt[FIXED_ORDER_MAX_PARTS + b];
      if (kk < n) { cls = 1; sel = b; } else kk -= n;
    }
    if (cls == 3 && kk < cnt[FIXED_ORDER_MAX_PARTS + NB]) cls = 2;
    pick[0] = cls; pick[1] = sel; pick[2] = kk;
  }
  __syncthreads();
  const int cls = pick[0], sel = pick[1], idx = pick[2];
  if (cls == 3) return false;  // uniform: every thread read the same pick
  auto member = [&](int s) {
    const int L = len(s), whole = L / P, rem = L - whole * P;
    if (cls == 0) return whole > sel;
    if (cls == 1) return rem > 0 && (int)((int64_t)rem * NB / P) == sel;
    return L == 0;
  };
  int local = 0;
  for (int s = s0; s < s1; ++s) local += member(s) ? 1 : 0;
  int x = local;  // inclusive scan over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_total[wv] = x;
  __syncthreads();
  int before = x - local;
  for (int w = 0; w < wv; ++w) before += wave_total[w];
  if (idx >= before && idx < before + local) {
    int r = idx - before;
    for (int s = s0; s < s1; ++s) {
      if (member(s)) {
        if (r == 0) {
          pick[0] = s;
          pick[1] = cls == 0 ? sel : cls == 1 ? len(s) / P : 0;
        }
        --r;
      }
    }
  }
  __syncthreads();
  seq = pick[0];
  part = pick[1];
  return true;
}

// Workgroups per CU the decode kernels are compiled for: 3 (12 waves) keeps
// enough loads in flight; four heads of fp32 queries over E4M3 keys (16
// query elements per lane and head) need the registers of 2.
template <typename T, typename KT, int GT>
constexpr int decode_min_wgs() { return (GT >= 4 && sizeof(T) == 4 && sizeof(KT) == 1) ? 2 : 3; }

// One wave = (sequence, KV head, group of GT query heads, partition).
template <typename T, typename KT, int D, int GT, int U, bool UNIFORM_BLOCK>
__global__ __launch_bounds__(256, (decode_min_wgs<T, KT, GT>())) void paged_decode_kernel(DecodeParams p) {
  constexpr int EPL = 16 / ElemTraits<KT>::E;  // elements per 16-byte lane slice
  constexpr int LPT = D / EPL;                 // lanes per token row of one head
  static_assert(LPT >= 1 && LPT <= 32 && (64 % LPT) == 0, "unsupported head_dim");

  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.x * 4 + (threadIdx.x >> 6);
  int seq = blockIdx.y, part = blockIdx.z;
  if (p.fixed_order) {
    if (!fixed_item(p, blockIdx.z * p.num_seqs + blockIdx.y, seq, part)) return;
    seq = __builtin_amdgcn_readfirstlane(seq);  // uniform over the workgroup: keep it scalar
    part = __builtin_amdgcn_readfirstlane(part);
  }
  // Fused store of seq's row, by the workgroup of its first partition once
  // its own work is done (the attention reads a sequence's newest row from
  // the new rows themselves, so the pool copy may land at any time).
  auto fused_store = [&]() {
    if constexpr (fused_store_supported<T, KT>()) {
      if (p.new_k != nullptr && blockIdx.x == 0 && part == 0) {
        const int64_t cpr = p.row_bytes / 16;
        store_new_rows<T, KT>(p, (int64_t)seq * cpr + threadIdx.x, 256, (int64_t)(seq + 1) * cpr);
      }
    }
  };
  if (unit >= p.units) {
    fused_store();
    return;
  }
  const int L = min(p.context_lens[seq], p.max_context_len);
  const int P = p.partition;
  const int nparts = L > 0 ? (L + P - 1) / P : 0;

  const int kvh = unit / p.n_sub;
  const int h0 = kvh * p.group + (unit - kvh * p.n_sub) * GT;
  const int dc = lane % LPT;
  const int tr = lane / LPT;

  if (nparts == 0) {  // empty context: defined output of zeros
    if (part == 0 && tr == 0) store_zeros<T, D, GT, EPL>(p, seq, h0, dc);
    fused_store();
    return;
  }
  if (part >= nparts) {
    fused_store();
    return;
  }

  const int tok_begin = part * P;
  const int tok_end = min(L, tok_begin + P);
  // MFMA logits over E4M3 pools only: over bf16 pools this kernel would
  // spill at 3 workgroups per CU (see decode_mfma_logits)
  WaveState<GT, EPL> st;
  attend<T, KT, D, GT, U, UNIFORM_BLOCK, false, (sizeof(KT) == 1)>(p, seq, kvh, h0, lane, dc, tok_begin, tok_end,
                                                                   logit_scale<KT>(p, kvh), st);
  apply_v_scale<KT, GT, EPL>(p, kvh, st.acc);
  merge_row_groups<LPT, GT, EPL>(st.m, st.l, st.acc);

  if (nparts == 1) {
    if (tr == 0) store_output<T, D, GT, EPL>(p, seq, h0, dc, st);
    fused_store();
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
        *reinterpret_cast<float4*>(dst + e) =
            make_float4(st.acc[h][e], st.acc[h][e + 1], st.acc[h][e + 2], st.acc[h][e + 3]);
      if (dc == 0) *reinterpret_cast<float2*>(p.ws_ml + (sh * mp + part) * 2) = make_float2(st.m[h], st.l[h]);
    }
  }
  fused_store();
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
// balanced split
// ---------------------------------------------------------------------------
//
// The contexts of all sequences, cut into chunks of CT tokens, are laid end
// to end; the W workers of each unit (one wave each, all resident at once)
// take equal contiguous ranges of that chunk sequence. A worker streams its
// range without a break, crossing from one sequence into another: a
// sequence wholly inside one range is written out directly, and a sequence
// cut by a range boundary leaves a partial (m, l, acc) state in one of the
// worker's two slots (slot 0: the piece the range starts in, slot 1: the
// piece it ends in), which paged_decode_balanced_merge_kernel combines.
// Every worker does the same amount of work whatever the length mix, and
// each wave pays its start-up (prefix sums, q, table window) once.

// Sequences the balanced split supports (their chunk prefix sums live in LDS).
constexpr int BAL_MAX_SEQS = 4096;

// pfx[0] = 0, pfx[k+1] = pfx[k] + ceil(L_k / CT): chunk prefix sums of the
// clamped context lengths, computed by the whole workgroup.
template <int CT>
__device__ __forceinline__ void chunk_prefix(const DecodeParams& p, int32_t* pfx) {
  __shared__ int32_t wave_total[4];
  const int B = p.num_seqs;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int per = (B + 255) / 256;
  const int k0 = min(B, tid * per);
  const int k1 = min(B, k0 + per);
  auto chunks = [&](int k) {
    const int L = min(p.context_lens[k], p.max_context_len);
    return L > 0 ? (L + CT - 1) / CT : 0;
  };
  int local = 0;
  for (int k = k0; k < k1; ++k) local += chunks(k);
  int x = local;  // inclusive scan over the wave
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_total[wv] = x;
  __syncthreads();
  int run = x - local;
  for (int w = 0; w < wv; ++w) run += wave_total[w];
  if (tid == 0) pfx[0] = 0;
  for (int k = k0; k < k1; ++k) {
    run += chunks(k);
    pfx[k + 1] = run;
  }
  __syncthreads();
}

// The worker whose range holds chunk ch, and the first chunk of worker wk's
// range, when C chunks are cut into W equal ranges.
__device__ __forceinline__ int bal_worker_of(int ch, int C, int W) {
  return (int)((((int64_t)ch + 1) * W - 1) / C);
}
__device__ __forceinline__ int bal_start_of(int wk, int C, int W) { return (int)((int64_t)wk * C / W); }

// Combine the partial states the workers left for a sequence whose chunks
// cb .. ce-1 their ranges cut, and write heads h0.. of its output. Lane
// mapping (dc, tr) as in the caller: token-row group tr takes the pieces of
// workers wf+tr, wf+tr+TPW, ...; the groups merge at the end.
template <typename T, int D, int GT, int EPL, int LPT>
__device__ __forceinline__ void merge_pieces(const DecodeParams& p, int seq, int h0, int dc, int tr,
                                             int cb, int ce, int C) {
  constexpr int TPW = 64 / LPT;
  const int W = p.workers;
  const int wf = bal_worker_of(cb, C, W), wl = bal_worker_of(ce - 1, C, W);
  WaveState<GT, EPL> st;
  st.reset();
  for (int wk = wf + tr; wk <= wl; wk += TPW) {
    const int s0 = bal_start_of(wk, C, W);
    if (s0 == bal_start_of(wk + 1, C, W)) continue;  // an empty range left nothing
    const int64_t slot = (int64_t)wk * 2 + ((wk == wf && s0 != cb) ? 1 : 0);
#pragma unroll
    for (int h = 0; h < GT; ++h) {
      const int64_t sh = slot * p.num_heads + h0 + h;
      const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + sh * 2);
      const float* src = p.part_acc + sh * D + dc * EPL;
      const float mn = fmaxf(st.m[h], ml.x);
      const float a = fast_exp2(st.m[h] - mn);
      const float b = fast_exp2(ml.x - mn);
      st.l[h] = st.l[h] * a + ml.y * b;
#pragma unroll
      for (int e = 0; e < EPL; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + e);
        st.acc[h][e] = st.acc[h][e] * a + v.x * b;
        st.acc[h][e + 1] = st.acc[h][e + 1] * a + v.y * b;
        st.acc[h][e + 2] = st.acc[h][e + 2] * a + v.z * b;
        st.acc[h][e + 3] = st.acc[h][e + 3] * a + v.w * b;
      }
      st.m[h] = mn;
    }
  }
  merge_row_groups<LPT, GT, EPL>(st.m, st.l, st.acc);
  if (tr == 0) store_output<T, D, GT, EPL>(p, seq, h0, dc, st);
}

// The balanced split's workers, as workgroup wg of num_wgs (each workgroup
// holds 4 waves, i.e. 4 (unit, worker) pairs). MAXS bounds num_seqs (the
// chunk prefix sums live in LDS). MFMA_OK: see decode_mfma_logits.
// PRIO: waves set their issue priority from the work they have left
// (set_progress_prio); off where they share CUs with other work.
template <typename T, typename KT, int D, int GT, int U, bool UNIFORM_BLOCK, int MAXS,
          bool PAIR = false, bool MFMA_OK = true, bool PRIO = false>
__device__ __forceinline__ void balanced_body(const DecodeParams& p, int wg, int num_wgs) {
  constexpr int EPL = 16 / ElemTraits<KT>::E;
  constexpr int LPT = D / EPL;
  constexpr int LPR = PAIR ? 2 * LPT : LPT;  // lanes per token row the wave reads
  constexpr int TPW = 64 / LPR;
  constexpr int CT = U * TPW;
  __shared__ int32_t pfx[MAXS + 1];
  // Fused store: every thread of the grid writes a share of the rows, once
  // its own work is done (the attention reads a sequence's newest row from
  // the new rows themselves, so the pool copy may land at any time).
  auto fused_store = [&]() {
    if constexpr (fused_store_supported<T, KT>()) {
      if (p.new_k != nullptr)
        store_new_rows<T, KT>(p, (int64_t)wg * 256 + threadIdx.x, (int64_t)num_wgs * 256, INT64_MAX);
    }
  };
  chunk_prefix<CT>(p, pfx);
  const int B = p.num_seqs;
  if (wg == 0)
    for (int k = threadIdx.x; k <= B; k += 256) p.ws_pfx[k] = pfx[k];
  const int C = __builtin_amdgcn_readfirstlane(pfx[B]);

  const int lane = threadIdx.x & 63;
  // uniform over the wave: kept in scalar registers
  const int g = __builtin_amdgcn_readfirstlane(wg * 4 + (threadIdx.x >> 6));
  const int unit = g % p.units;  // the waves of a workgroup share a range
  const int w = g / p.units;
  if (w >= p.workers) {
    fused_store();
    return;
  }
  const int c0 = (int)((int64_t)w * C / p.workers);
  const int c1 = (int)((int64_t)(w + 1) * C / p.workers);
  if (c0 >= c1) {
    fused_store();
    return;
  }
  // this lane's KV head (a pair's first or second) and first query head
  const int kvh = PAIR ? 2 * unit + (lane % LPR) / LPT : unit / p.n_sub;
  const int h0 = PAIR ? kvh : kvh * p.group + (unit - kvh * p.n_sub) * GT;
  const int dc = lane % LPT;
  const int tr = lane / LPR;
  const float sm = logit_scale<KT>(p, kvh);

  // Pieces are taken from the end of the range backwards. The last piece
  // begins at a context's first token (unless the range lies inside one
  // context), so the first blocks of contexts, which prefix sharing makes
  // common to many sequences, are read by all workers near the start of the
  // kernel, while the shared lines are still cached.
  // The sequence holding chunk c1 - 1: the last i with pfx[i] <= c1 - 1.
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pfx[mid] <= c1 - 1) lo = mid;
    else hi = mid - 1;
  }
  int i = lo;
  for (;;) {
    const int cb = pfx[i], ce = pfx[i + 1];
    const int ps = max(c0, cb), pe = min(c1, ce);
    const int L = min(p.context_lens[i], p.max_context_len);
    WaveState<GT, EPL> st;
    attend<T, KT, D, GT, U, UNIFORM_BLOCK, PAIR, MFMA_OK>(p, i, kvh, h0, lane, dc, (ps - cb) * CT,
                                                         min((pe - cb) * CT, L), sm, st,
                                                         PRIO ? (ps - c0) * CT : 0, PRIO ? (c1 - c0) * CT : 0);
    apply_v_scale<KT, GT, EPL>(p, kvh, st.acc);
    merge_row_groups<LPR, GT, EPL>(st.m, st.l, st.acc);
    if (tr == 0) {
      if (ps == cb && pe == ce) {
        store_output<T, D, GT, EPL>(p, i, h0, dc, st);
      } else {
        // slot 0: the piece holding c0; slot 1: the piece holding c1 - 1
        const int64_t slot = (int64_t)w * 2 + (ps == c0 ? 0 : 1);
#pragma unroll
        for (int h = 0; h < GT; ++h) {
          const int64_t sh = slot * p.num_heads + h0 + h;
          float* dst = p.part_acc + sh * D + dc * EPL;
#pragma unroll
          for (int e = 0; e < EPL; e += 4)
            *reinterpret_cast<float4*>(dst + e) =
                make_float4(st.acc[h][e], st.acc[h][e + 1], st.acc[h][e + 2], st.acc[h][e + 3]);
          if (dc == 0) *reinterpret_cast<float2*>(p.part_ml + sh * 2) = make_float2(st.m[h], st.l[h]);
        }
      }
    }
    if (ps <= c0) break;
    do {
      --i;
    } while (pfx[i] == pfx[i + 1]);  // skip empty contexts
  }
  fused_store();
}

template <typename T, typename KT, int D, int GT, int U, bool UNIFORM_BLOCK, bool PAIR = false>
__global__ __launch_bounds__(256, DECODE_BAL_WAVES_PER_SIMD) void paged_decode_balanced_kernel(DecodeParams p) {
  balanced_body<T, KT, D, GT, U, UNIFORM_BLOCK, BAL_MAX_SEQS, PAIR, true, true>(p, blockIdx.x, gridDim.x);
}

// One wave per (sequence, unit): combine the partial states the workers
// left for a sequence their ranges cut, and write zeros for an empty
// context. Sequences inside one range were written by the main kernel.
template <typename T, int D, int GT>
__global__ __launch_bounds__(256) void paged_decode_balanced_merge_kernel(DecodeParams p) {
  constexpr int E = ElemTraits<T>::E;
  constexpr int EPL = 16 / E;
  constexpr int LPT = D / EPL;
  const int lane = threadIdx.x & 63;
  const int unit = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (unit >= (p.units << p.pair)) return;  // one KV head per unit (a pair's heads separately)
  const int seq = blockIdx.x;
  const int kvh = unit / p.n_sub;
  const int h0 = kvh * p.group + (unit - kvh * p.n_sub) * GT;
  const int dc = lane % LPT;
  const int tr = lane / LPT;
  // one round of loads: the chunk prefix sums (an empty context has none)
  const int cb = p.ws_pfx[seq], ce = p.ws_pfx[seq + 1], C = p.ws_pfx[p.num_seqs];
  if (cb == ce) {
    if (tr == 0) store_zeros<T, D, GT, EPL>(p, seq, h0, dc);
    return;
  }
  const int W = p.workers;
  if (bal_worker_of(cb, C, W) == bal_worker_of(ce - 1, C, W)) return;  // written by one worker
  merge_pieces<T, D, GT, EPL, LPT>(p, seq, h0, dc, tr, cb, ce, C);
}

// DecodeParams of a validated call and its plan (decode.hip).
DecodeParams make_decode_params(const DecodeArgs& a, const DecodePlan& pl);

// Loads in flight per lane of the balanced split for pools in the query
// type / as E4M3 codes.
constexpr int DECODE_U_BALANCED = DECODE_U;
constexpr int DECODE_U_BALANCED_E4M3 = DECODE_U_E4M3;

}  // namespace pa
