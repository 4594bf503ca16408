// prefill_chunk: causal attention of a chunk of new tokens over the cached
// plus new context of each sequence, read through the block table, on bf16
// MFMA with fp32 accumulation.
//
// What is computed (the prefill pass of the mini-vllm page's inference
// engine, run chunk by chunk): sequence i has n_i new rows at positions
// c_i .. c_i + n_i - 1 (c_i = context_lens[i] - n_i tokens cached); row t
// attends to keys 0 .. c_i + t (causal, aligned to the end of the context).
//
// Work decomposition: a workgroup of 4 waves handles one KV head and 32*RG
// query rows of one sequence; HW = 4/RG query heads of that KV head's group
// share the workgroup, so every K/V tile staged in LDS serves HW heads x 32*RG
// rows. Wave w takes head (w % HW) and rows 32*(w / HW) .. +32 (two 16-row
// MFMA tiles).
//
// Per 64-key tile:
//   * stage K as [key][d] and V transposed as [d][key] in LDS (rows padded by
//     16 bytes), reading 16-byte slices of paged rows through the table;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16 keys x 32 d from LDS,
//     B = Q^T slice held in registers for the whole kernel). The C layout puts
//     one query row in each lane (column = lane % 16) and 4 keys per register
//     group, so the softmax max/sum of a row needs only the 4 lanes
//     l, l^16, l^32, l^48;
//   * keys inside each 32-key step are assigned to tile rows so that lane
//     group q ends up holding keys 8q .. 8q+7 contiguously: the probabilities
//     then ARE the B operand (P^T) of the next product without a register
//     transpose;
//   * O^T += V^T P^T with the same MFMA (A = 16 d x 32 keys from the
//     transposed V tile); O^T's column is again the lane's query row, so the
//     online-softmax rescale is a per-lane multiply.
//
// Bound: MFMA (bf16 dense). Algorithmic flops = 4 * D * Hq * (visible
// query-key pairs).

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

struct PrefillParams {
  uint16_t* out;
  const uint16_t* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_tables;
  const int32_t* query_start_loc;
  const int32_t* context_lens;
  int32_t num_heads, num_kv_heads, group, n_sub;
  int32_t bs_log2, num_blocks, max_blocks_per_seq, max_query_len, max_context_len;
  float scale_log2;
};

__device__ __forceinline__ uint32_t bf16_elem(const uint4& v, int d) {
  const uint32_t w = (d < 2) ? v.x : (d < 4) ? v.y : (d < 6) ? v.z : v.w;
  return (d & 1) ? (w >> 16) : (w & 0xFFFFu);
}

template <int D, int HW>
__global__ __launch_bounds__(256) void prefill_chunk_kernel(PrefillParams p) {
  constexpr int RG = 4 / HW;      // row groups of 32 rows
  constexpr int ROWS = 32 * RG;   // query rows per workgroup
  constexpr int KT = 64;          // keys per tile
  constexpr int KS = D / 32;      // MFMA k-steps over head_dim for S
  constexpr int DT = D / 16;      // 16-wide d tiles of O^T
  constexpr int DCH = D / 8;      // 16-byte slices per row
  constexpr int KROW = D + 8;     // LDS row pitch of the K tile (elements)
  constexpr int VROW = KT + 8;    // LDS row pitch of the V^T tile (elements)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qgrp = lane >> 4;     // 0..3
  const int lrow = lane & 15;
  const int seq = blockIdx.y;
  const int qs = p.query_start_loc[seq];
  const int n = min(p.query_start_loc[seq + 1] - qs, p.max_query_len);
  const int t0 = blockIdx.x * ROWS;
  if (t0 >= n) return;  // whole workgroup
  const int L = min(p.context_lens[seq], p.max_context_len);
  const int c = L - n;
  const int kvh = blockIdx.z / p.n_sub;
  const int head = kvh * p.group + (blockIdx.z - kvh * p.n_sub) * HW + (wave % HW);
  const int wrow0 = t0 + (wave / HW) * 32;
  const int kv_end = min(L, c + min(t0 + ROWS, n));  // keys this workgroup needs
  const int bs_log2 = p.bs_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int64_t row_bytes = (int64_t)p.num_kv_heads * D * 2;
  const int64_t head_off = (int64_t)kvh * D * 2;
  const int32_t* bt = p.block_tables + (int64_t)seq * p.max_blocks_per_seq;

  // Q^T B operands: lane holds Q[row lrow][32*ks + 8*qgrp .. +8] per tile.
  bf16x8 qreg[2][KS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int t = wrow0 + rt * 16 + lrow;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < n)
        v = *reinterpret_cast<const uint4*>(
            p.q + ((int64_t)(qs + t) * p.num_heads + head) * D + 32 * ks + 8 * qgrp);
      qreg[rt][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m[2], lsum[2];
  f32x4 o[DT][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    m[rt] = NEG_BIG;
    lsum[rt] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int kt0 = 0; kt0 < kv_end; kt0 += KT) {
    __syncthreads();  // the previous tile's LDS reads are done
    // ---- stage K [key][d] ----
#pragma unroll
    for (int it = tid; it < KT * DCH; it += 256) {
      const int key = it / DCH, dch = it % DCH;
      const int j = kt0 + key;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j < kv_end) {
        const int phys = clamp_block(bt[j >> bs_log2], p.num_blocks);
        v = *reinterpret_cast<const uint4*>(
            p.k_cache + (((int64_t)phys << bs_log2) + (j & bs_mask)) * row_bytes + head_off + dch * 16);
      }
      *reinterpret_cast<uint4*>(&Ks[key * KROW + dch * 8]) = v;
    }
    // ---- stage V transposed [d][key]: a thread moves 4 keys x 8 d ----
    for (int it = tid; it < (KT / 4) * DCH; it += 256) {
      const int kq = it / DCH, dch = it % DCH;
      uint4 v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = kt0 + 4 * kq + e;
        v[e] = make_uint4(0, 0, 0, 0);
        if (j < kv_end) {
          const int phys = clamp_block(bt[j >> bs_log2], p.num_blocks);
          v[e] = *reinterpret_cast<const uint4*>(
              p.v_cache + (((int64_t)phys << bs_log2) + (j & bs_mask)) * row_bytes + head_off + dch * 16);
        }
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        uint2 w;
        w.x = bf16_elem(v[0], d) | (bf16_elem(v[1], d) << 16);
        w.y = bf16_elem(v[2], d) | (bf16_elem(v[3], d) << 16);
        *reinterpret_cast<uint2*>(&Vt[(dch * 8 + d) * VROW + 4 * kq]) = w;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: tiles [step c2][half hf][row tile rt] ----
    f32x4 s[2][2][2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int key = 32 * c2 + 8 * (lrow >> 2) + 4 * hf + (lrow & 3);
        s[c2][hf][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        s[c2][hf][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[key * KROW + 32 * ks + 8 * qgrp]);
          s[c2][hf][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[0][ks], s[c2][hf][0], 0, 0, 0);
          s[c2][hf][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[1][ks], s[c2][hf][1], 0, 0, 0);
        }
      }

    // ---- online softmax per query row (lane row lrow of tile rt) ----
    bf16x8 pb[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int tpos = c + wrow0 + rt * 16 + lrow;  // absolute position of the row
      float mt = NEG_BIG;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kt0 + 32 * c2 + 8 * qgrp + 4 * hf + i;
            float v = s[c2][hf][rt][i] * p.scale_log2;
            v = (key <= tpos && key < kv_end) ? v : -INFINITY;
            s[c2][hf][rt][i] = v;
            mt = fmaxf(mt, v);
          }
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m[rt], mt);
      const float alpha = fast_exp2(m[rt] - mn);
      m[rt] = mn;
      float ps = 0.0f;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        uint32_t w[4];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const float p0 = fast_exp2(s[c2][hf][rt][0] - mn);
          const float p1 = fast_exp2(s[c2][hf][rt][1] - mn);
          const float p2 = fast_exp2(s[c2][hf][rt][2] - mn);
          const float p3 = fast_exp2(s[c2][hf][rt][3] - mn);
          w[2 * hf] = pack_bf16x2(p0, p1);
          w[2 * hf + 1] = pack_bf16x2(p2, p3);
          // sum the rounded weights, the ones the PV product uses
          ps += bf16lo(w[2 * hf]) + bf16hi(w[2 * hf]) + bf16lo(w[2 * hf + 1]) + bf16hi(w[2 * hf + 1]);
        }
        pb[rt][c2] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
      }
      lsum[rt] = lsum[rt] * alpha + ps;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Vt[(16 * dt + lrow) * VROW + 32 * c2 + 8 * qgrp]);
        o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[0][c2], o[dt][0], 0, 0, 0);
        o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[1][c2], o[dt][1], 0, 0, 0);
      }
  }

  // ---- normalise and write: lane holds O[row][16*dt + 4*qgrp + 0..3] ----
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float lt = lsum[rt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = 1.0f / lt;
    const int t = wrow0 + rt * 16 + lrow;
    if (t < n) {
      uint16_t* dst = p.out + ((int64_t)(qs + t) * p.num_heads + head) * D + 4 * qgrp;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint2 w;
        w.x = pack_bf16x2(o[dt][rt][0] * inv, o[dt][rt][1] * inv);
        w.y = pack_bf16x2(o[dt][rt][2] * inv, o[dt][rt][3] * inv);
        *reinterpret_cast<uint2*>(dst + 16 * dt) = w;
      }
    }
  }
}

static int32_t prefill_heads_per_wg(int32_t group) {
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

template <int D, int HW>
static void launch_prefill_t(const PrefillParams& prm, int32_t max_query_len, int32_t num_seqs,
                             int32_t num_kv_heads, hipStream_t stream) {
  constexpr int ROWS = 32 * (4 / HW);
  const dim3 grid((unsigned)((max_query_len + ROWS - 1) / ROWS), (unsigned)num_seqs,
                  (unsigned)(num_kv_heads * prm.n_sub));
  hipLaunchKernelGGL((prefill_chunk_kernel<D, HW>), grid, dim3(256), 0, stream, prm);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
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
  const int32_t hw = prefill_heads_per_wg(prm.group);
  prm.n_sub = prm.group / hw;
  prm.bs_log2 = __builtin_ctz((unsigned)a.block_size);
  prm.num_blocks = a.num_blocks;
  prm.max_blocks_per_seq = a.max_blocks_per_seq;
  prm.max_query_len = a.max_query_len;
  prm.max_context_len = a.max_context_len;
  prm.scale_log2 = a.scale * 1.4426950408889634f;
  const int32_t mq = a.max_query_len, B = a.num_seqs, H = a.num_kv_heads;
  if (a.head_dim == 64) {
    if (hw == 4) launch_prefill_t<64, 4>(prm, mq, B, H, stream);
    else if (hw == 2) launch_prefill_t<64, 2>(prm, mq, B, H, stream);
    else launch_prefill_t<64, 1>(prm, mq, B, H, stream);
  } else {
    if (hw == 4) launch_prefill_t<128, 4>(prm, mq, B, H, stream);
    else if (hw == 2) launch_prefill_t<128, 2>(prm, mq, B, H, stream);
    else launch_prefill_t<128, 1>(prm, mq, B, H, stream);
  }
  return hipGetLastError();
}

}  // namespace pa
