// Prefill kernel (device code) of libpagedattn; the launch is in
// prefill.hip, the mixed prefill+decode launch in mixed.hip.
//
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
// query positions of one sequence; HW = 4/RG query heads of that KV head's
// group share the workgroup, so every K/V tile staged in LDS serves
// HW heads x 32*RG rows. Wave w takes head (w % HW) and positions
// 32*(w / HW) .. +32 (two 16-row MFMA tiles). The grid's slowest dimension
// walks the row blocks from the end of the chunk, so the workgroups with the
// longest key ranges are dispatched first.
//
// Per 64-key tile (software-pipelined: the K/V rows of tile i+1 move from
// global memory straight into the other of two LDS stages while tile i is
// computed):
//   * the physical block ids come from a window of the block table held in
//     LDS, loaded once (and again only if a context outgrows the window);
//   * K and V are staged as [key][d]; 16-byte granules are XOR-swizzled
//     within a row (the swizzle is applied to the global addresses of the
//     loads) so that the MFMA operand reads spread over the LDS banks;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (A = 16 keys x 32 d from LDS,
//     B = Q^T slice held in registers for the whole kernel). The C layout puts
//     one query row in each lane (column = lane % 16) and 4 keys per register
//     group, so the softmax max/sum of a row needs only the 4 lanes
//     l, l^16, l^32, l^48;
//   * keys inside each 32-key step are assigned to tile rows so that lane
//     group q ends up holding keys 8q .. 8q+7 contiguously: the probabilities
//     then ARE the B operand (P^T) of the next product without a register
//     transpose;
//   * O^T += V^T P^T with the same MFMA; its A operand (16 d x 32 keys) is
//     read from the untransposed V tile with ds_read_b64_tr_b16; O^T's column
//     is again the lane's query row, so the online-softmax rescale is a
//     per-lane multiply;
//   * the running maximum is only raised (and O rescaled) when a tile's
//     maximum exceeds it by more than 2^32 in probability, so almost every
//     tile after the first skips the rescale; the result is the same
//     softmax, with probabilities below 2^32 relative to the kept maximum;
//   * only tiles that straddle a wave's causal diagonal are masked.
//
// Bound: MFMA (bf16 dense). Algorithmic flops = 4 * D * Hq * (visible
// query-key pairs).

#pragma once

#include <type_traits>

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
  int32_t num_seqs;
  int32_t row_blocks;  // gridDim.z: ceil(max_query_len / ROWS)
  float scale_log2;
  const float* k_scale;  // E4M3 pools: per-KV-head scales (else null)
  const float* v_scale;
};

// Work items (sequence, row block) are ranked by their number of key tiles
// with a counting sort over this many bins (two per thread).
constexpr int RANK_BINS = 512;

// Maximum over lanes l, l^16, l^32, l^48 (the four lanes that hold one row
// of an MFMA C tile): the cross-half and cross-row swaps of gfx950, with
// copies of x in both operands, leave x of lane l and of its partner lane
// in the two results.
__device__ __forceinline__ float max_over_row_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t v = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Lazy-rescale threshold in log2 units: probabilities stay below 2^32. bf16
// and fp32 keep their relative precision at that size, and a row sum of at
// most 2^32 per key cannot overflow fp32, so after the first tile a rescale
// of the accumulators is needed only when a row's maximum jumps by 2^32.
constexpr float RESCALE_SLACK = 32.0f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16 bytes from global memory straight into LDS: lane l of the wave writes
// lds_base + 16*l (lds_base must be the same for every lane).
__device__ __forceinline__ void load_lds16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)gptr,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// A buffer resource over the bytes from base on (record limit 2^31 - 1, raw
// 32-bit data format for untyped loads), and a 16-byte load from it straight
// into LDS: lane l reads at its own offset voff and writes lds_base + 16*l
// (lds_base the same for every lane).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const char* base) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, 0x7FFFFFFF, 0x00020000);
}
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, 0, 0, 0);
}

// Two E4M3 codes (byte pair HI of w: 0 = bytes 0-1, 1 = bytes 2-3) as two
// bf16 (exact: every E4M3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t widen_e4m3x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// Transposing LDS read of 4 bf16. Within each group of 16 lanes, lane i
// receives element i % 4 of the 8 bytes addressed by lanes 4j + i/4,
// j = 0..3: when lane s of the group points at row r0 + s/4, columns
// c0 + 4*(s%4) .. +3 of a row-major tile, lane i gets column c0 + i of rows
// r0 .. r0+3.
__device__ __forceinline__ uint2 lds_read_tr4(const uint16_t* ptr) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)ptr);
  return __builtin_bit_cast(uint2, v);
}

// One workgroup's work: head group bx, sequence by, row block bz of the
// grid (head groups x sequences x row blocks) that prefill_chunk_kernel
// launches. CT is the pools' element type: uint16_t (bf16) or uint8_t (E4M3
// codes, read back as value(code) * scale of the KV head).
template <int D, int HW, typename CT = uint16_t>
__device__ __forceinline__ void prefill_body(const PrefillParams& p, int bx, int by, int bz) {
  constexpr bool E4 = sizeof(CT) == 1;
  constexpr int RG = 4 / HW;      // row groups of 32 rows
  constexpr int ROWS = 32 * RG;   // query positions per workgroup
  constexpr int KT = 64;          // keys per tile
  constexpr int KS = D / 32;      // MFMA k-steps over head_dim for S
  constexpr int DT = D / 16;      // 16-wide d tiles of O^T
  constexpr int GPR = D / 8;      // 16-byte granules per K/V row of one head
  constexpr int KPI = 64 / GPR;   // keys one wave-wide 16-byte load covers
  constexpr int NIW = KT / KPI / 4;  // such loads per wave per tile, per tensor
  constexpr int TE = KT * D;      // elements of one staged tile
  constexpr int TBL = 512;        // block-table window (entries)
  static_assert(NIW >= 1, "tile shape");

  // Two stages, each [0 = K, 1 = V][key][granule] of bf16 with granules
  // XOR-swizzled per key. Separate arrays, so the compiler can tell that a
  // load into one stage does not feed the reads of the other. bf16 pools:
  // the rows are copied from global memory straight into a stage; E4M3
  // pools: each thread loads its share of a tile's codes into registers one
  // tile ahead and widens them into the stage at the start of that tile.
  __shared__ __attribute__((aligned(16))) uint16_t kv0[2][TE];
  __shared__ __attribute__((aligned(16))) uint16_t kv1[2][TE];
  __shared__ int32_t tbl[TBL];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qgrp = lane >> 4;     // 0..3
  const int lrow = lane & 15;

  // ---- which (sequence, row block) this workgroup takes ----
  // Workgroups are dispatched in order of (blockIdx.z, blockIdx.y); the k-th
  // one takes the work item with the k-th most key tiles, so the longest
  // items start first and short ones fill in at the end.
  auto item_tiles = [&](int s, int rb) {
    const int q0 = p.query_start_loc[s];
    const int nn = min(p.query_start_loc[s + 1] - q0, p.max_query_len);
    const int tt = rb * ROWS;
    if (tt >= nn) return 0;
    const int LL = min(p.context_lens[s], p.max_context_len);
    const int ke = min(LL, LL - nn + min(tt + ROWS, nn));
    return ke > 0 ? (ke + KT - 1) / KT : 0;
  };
  const int R = p.row_blocks;
  const int n_items = p.num_seqs * R;
  const int k_rank = bz * p.num_seqs + by;
  int seq, rb;
  {
    // Counting sort of the items by key tiles (descending; equal counts in
    // item order): a histogram of the counts, the bin holding rank k_rank
    // from a scan over the bins, then the item of that bin from a scan over
    // the items. Counts of RANK_BINS - 1 tiles or more share the last bin.
    int* hist = reinterpret_cast<int*>(&kv0[0][0]);  // LDS, free until the main loop
    int* wtot = hist + RANK_BINS;                    // per-wave totals
    int* pick = wtot + 4;                            // bin, index in the bin, item
    const int per = (n_items + 255) / 256;
    const int x0 = min(n_items, tid * per), x1 = min(n_items, x0 + per);
    auto bin_of = [&](int x) { return min(item_tiles(x / R, x % R), RANK_BINS - 1); };
    auto block_exclusive = [&](int v) {  // exclusive prefix of v over the workgroup's threads
      int incl = v;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
      }
      if (lane == 63) wtot[wave] = incl;
      __syncthreads();
      int before = incl - v;
      for (int w = 0; w < wave; ++w) before += wtot[w];
      return before;
    };
    for (int i = tid; i < RANK_BINS; i += 256) hist[i] = 0;
    __syncthreads();
    for (int x = x0; x < x1; ++x) atomicAdd(&hist[bin_of(x)], 1);
    __syncthreads();
    {
      const int b0 = RANK_BINS - 1 - 2 * tid, b1 = b0 - 1;  // thread t: bins from the top
      const int h0 = hist[b0], h1 = hist[b1];
      const int before = block_exclusive(h0 + h1);  // items in higher bins
      if (k_rank >= before && k_rank < before + h0) {
        pick[0] = b0;
        pick[1] = k_rank - before;
      } else if (k_rank >= before + h0 && k_rank < before + h0 + h1) {
        pick[0] = b1;
        pick[1] = k_rank - before - h0;
      }
      __syncthreads();
    }
    const int bin = pick[0], idx = pick[1];
    int local = 0;
    for (int x = x0; x < x1; ++x) local += bin_of(x) == bin;
    __syncthreads();  // wtot is reused
    const int before = block_exclusive(local);
    if (idx >= before && idx < before + local) {
      int r = idx - before;
      for (int x = x0; x < x1; ++x)
        if (bin_of(x) == bin) {
          if (r == 0) pick[2] = x;
          --r;
        }
    }
    __syncthreads();
    const int x = pick[2];
    __syncthreads();  // the stage is reused for K/V below
    seq = x / R;
    rb = x % R;
  }
  const int qs = p.query_start_loc[seq];
  const int n = min(p.query_start_loc[seq + 1] - qs, p.max_query_len);
  const int t0 = rb * ROWS;
  if (t0 >= n) return;  // whole workgroup
  const int L = min(p.context_lens[seq], p.max_context_len);
  const int c = L - n;
  const int kvh = bx / p.n_sub;
  const int head = kvh * p.group + (bx - kvh * p.n_sub) * HW + (wave % HW);
  const int wrow0 = t0 + (wave / HW) * 32;
  const int kv_end = min(L, c + min(t0 + ROWS, n));  // keys this workgroup needs
  if (kv_end <= 0) return;  // only when a precondition is violated (n > L)
  const int wave_last_key = c + wrow0 + 31;          // last key any row of this wave sees
  const int bs_log2 = p.bs_log2;
  const int bs_mask = (1 << bs_log2) - 1;
  const int64_t row_bytes = (int64_t)p.num_kv_heads * D * (int)sizeof(CT);
  const int64_t head_off = (int64_t)kvh * D * (int)sizeof(CT);
  const int32_t* bt = p.block_tables + (int64_t)seq * p.max_blocks_per_seq;
  const int nblk = (kv_end + bs_mask) >> bs_log2;

  // Granule swizzles (key = index within the tile). K rows are read 16 keys
  // at a time at one granule: key bits 0,1,3,4 pick distinct granules. V rows
  // are read by the transposing load, 8 keys x 2 granules at a time: even
  // swizzles from key bits 0,1,3.
  auto swz_k = [](int key) { return ((key & 3) | ((key >> 1) & 12)) & (GPR - 1); };
  auto swz_v = [](int key) { return (2 * ((key & 3) | ((key >> 1) & 4))) & (GPR - 1); };

  // ---- block-table window ----
  int wb = 0;
  auto load_window = [&](int base) {
    for (int i = tid; i < TBL; i += 256)
      tbl[i] = (base + i < nblk) ? clamp_block(bt[base + i], p.num_blocks) : 0;
  };
  load_window(0);

  // Issue the global->LDS loads of tile kt0 into a stage. Keys past the
  // workgroup's range read the last needed row instead (finite data whose
  // probability is zero), so no NaN from outside the context reaches V.
  // A whole tile inside one block is copied through buffer loads: the tile's
  // first row is the base of a buffer resource in scalar registers, and each
  // lane's offsets from it (NIW K and NIW V copies) are fixed for the kernel.
  uint32_t koff[NIW], voff[NIW];
#pragma unroll
  for (int i = 0; i < NIW; ++i) {
    const int key = (wave * NIW + i) * KPI + lane / GPR;
    const int gl = lane % GPR;
    koff[i] = (uint32_t)(key * row_bytes + head_off + (gl ^ swz_k(key)) * 16);
    voff[i] = (uint32_t)(key * row_bytes + head_off + (gl ^ swz_v(key)) * 16);
  }
  auto issue = [&](int kt0, uint16_t (&stage)[2][TE]) {
    // When the tile lies inside one block (block_size >= KT) one table entry
    // serves every lane.
    const bool one_block = KT <= (1 << bs_log2);
    const int phys0 = __builtin_amdgcn_readfirstlane(tbl[(kt0 >> bs_log2) - wb]);
    if (__builtin_amdgcn_readfirstlane((int)(one_block && kt0 + KT <= kv_end))) {  // a whole tile of one block
      const int64_t t64 = (((int64_t)phys0 << bs_log2) + (kt0 & bs_mask)) * row_bytes;
      const int64_t tile = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(t64 >> 32)) << 32) |
                                     (uint32_t)__builtin_amdgcn_readfirstlane((int)t64));
      const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.k_cache + tile);
      const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(p.v_cache + tile);
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const int ins = wave * NIW + i;
        buffer_load_lds16(rk, koff[i], &stage[0][ins * KPI * D]);
        buffer_load_lds16(rv, voff[i], &stage[1][ins * KPI * D]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int ins = wave * NIW + i;
      const int key = ins * KPI + lane / GPR;
      const int j = min(kt0 + key, kv_end - 1);
      const int phys = one_block ? phys0 : tbl[(j >> bs_log2) - wb];
      const int64_t row = (((int64_t)phys << bs_log2) + (j & bs_mask)) * row_bytes + head_off;
      const int gl = lane % GPR;
      load_lds16(p.k_cache + row + ((gl ^ swz_k(key)) * 16), &stage[0][ins * KPI * D]);
      load_lds16(p.v_cache + row + ((gl ^ swz_v(key)) * 16), &stage[1][ins * KPI * D]);
    }
  };

  // E4M3: the codes of tile kt0 into registers, each thread 16 codes of a
  // key row per tensor and chunk (CPR chunks per row of one head), clamped
  // to the last needed key like the bf16 loads; widen_store later widens
  // them exactly to bf16 into a stage, in the swizzled layout above.
  constexpr int CPR = D / 16;
  constexpr int PER = E4 ? KT * CPR / 256 : 1;
  uint4 kcode[PER], vcode[PER];
  auto load_codes = [&](int kt0) {
    const bool one_block = KT <= (1 << bs_log2);
    const int phys0 = one_block ? __builtin_amdgcn_readfirstlane(tbl[(kt0 >> bs_log2) - wb]) : 0;
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int ci = tid + 256 * x;
      const int key = ci / CPR, part = ci % CPR;
      const int j = min(kt0 + key, kv_end - 1);
      const int phys = one_block ? phys0 : tbl[(j >> bs_log2) - wb];
      const int64_t row = (((int64_t)phys << bs_log2) + (j & bs_mask)) * row_bytes + head_off + part * 16;
      kcode[x] = *reinterpret_cast<const uint4*>(p.k_cache + row);
      vcode[x] = *reinterpret_cast<const uint4*>(p.v_cache + row);
    }
  };
  auto widen_store = [&](uint16_t (&stage)[2][TE]) {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int ci = tid + 256 * x;
      const int key = ci / CPR, part = ci % CPR;
#pragma unroll
      for (int tsr = 0; tsr < 2; ++tsr) {
        const uint4 w = tsr == 0 ? kcode[x] : vcode[x];
        const uint4 lo = make_uint4(widen_e4m3x2<false>(w.x), widen_e4m3x2<true>(w.x),
                                    widen_e4m3x2<false>(w.y), widen_e4m3x2<true>(w.y));
        const uint4 hi = make_uint4(widen_e4m3x2<false>(w.z), widen_e4m3x2<true>(w.z),
                                    widen_e4m3x2<false>(w.w), widen_e4m3x2<true>(w.w));
        const int sw = tsr == 0 ? swz_k(key) : swz_v(key);
        *reinterpret_cast<uint4*>(&stage[tsr][key * D + (((2 * part) ^ sw) * 8)]) = lo;
        *reinterpret_cast<uint4*>(&stage[tsr][key * D + (((2 * part + 1) ^ sw) * 8)]) = hi;
      }
    }
  };

  // Q^T B operands: lane holds Q[row lrow][32*ks + 8*qgrp .. +8] per tile.
  // A negative scale is applied as an (exact) sign flip of Q, so that the
  // logit scale sl2 below is never negative. E4M3: the KV head's K scale
  // multiplies the logit scale, its V scale the output.
  float eff_scale = p.scale_log2;
  float out_scale = 1.0f;
  if constexpr (E4) {
    eff_scale *= p.k_scale[kvh];
    out_scale = p.v_scale[kvh];
  }
  const uint32_t qsign = eff_scale < 0.0f ? 0x80008000u : 0u;
  const float sl2 = fabsf(eff_scale);
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
      v.x ^= qsign; v.y ^= qsign; v.z ^= qsign; v.w ^= qsign;
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

  __syncthreads();  // table window visible
  if constexpr (E4) load_codes(0);
  else issue(0, kv0);

  // One 64-key tile: wait for its loads, start the next tile's loads into
  // the other stage, then compute from this stage.
  // One 64-key tile: wait for its loads, start the next tile's loads into
  // the other stage, then compute from this stage. E4M3 pools: the loads are
  // the codes (code stage st, the next tile's into st ^ 1), widened into kv0
  // (cur) before the products.
  auto step = [&](int kt0, uint16_t (&cur)[2][TE], uint16_t (&nxt_stage)[2][TE], int st) {
    // E4M3: widen tile kt0's codes (loaded during the previous tile) into
    // this stage, which every wave finished reading before the previous
    // tile's barrier
    if constexpr (E4) widen_store(cur);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's part of tile kt0 landed
    __syncthreads();  // the whole tile is in LDS; every wave is done with the other stage
    const int nxt = kt0 + KT;
    if (nxt < kv_end) {
      const int last_blk = (min(nxt + KT, kv_end) - 1) >> bs_log2;
      if (last_blk >= wb + TBL) {  // uniform and rare: slide the window
        wb = nxt >> bs_log2;
        load_window(wb);
        __syncthreads();
      }
      if constexpr (E4) load_codes(nxt);  // in registers while this tile is computed
      else issue(nxt, nxt_stage);  // in flight while this tile is computed
    }
    if (kt0 > wave_last_key) return;  // every key of this tile is masked for this wave
    const uint16_t* Kt = cur[0];
    const uint16_t* Vt = cur[1];

    // ---- S^T = K Q^T: tiles [step c2][half hf][row tile rt] ----
    f32x4 s[2][2][2];
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int key = 32 * c2 + 8 * (lrow >> 2) + 4 * hf + (lrow & 3);
        const int sk = swz_k(key);
        bf16x8 a[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          a[ks] = *reinterpret_cast<const bf16x8*>(&Kt[key * D + (((4 * ks + qgrp) ^ sk) * 8)]);
        s[c2][hf][0] = f32x4{0.f, 0.f, 0.f, 0.f};
        s[c2][hf][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s[c2][hf][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], qreg[0][ks], s[c2][hf][0], 0, 0, 0);
          s[c2][hf][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], qreg[1][ks], s[c2][hf][1], 0, 0, 0);
        }
      }
    // Schedule: the K operands of two (c2, hf) groups, then each group's
    // MFMAs followed by the next group's operand reads, so that the reads
    // run one group ahead and at most two groups' operands are live.
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KS, 0);  // LDS reads
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS, 0);  // MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4 * KS, 0);

    // ---- online softmax per query row (lane row lrow of tile rt) ----
    // Logits are s * sl2 with sl2 >= 0 (a negative scale was moved into the
    // sign of Q), so a row's largest logit comes from its largest raw score.
    // Only tiles that cross this wave's causal diagonal take the masked path.
    bf16x8 pb[2][2];
    auto softmax = [&](auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
      // Each lane's maximum over its own logits of a row; the maximum over
      // the row's four lanes is only needed when some lane's exceeds the
      // row's running maximum by more than the slack.
      float lm[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int tpos = c + wrow0 + rt * 16 + lrow;  // absolute position of the row
        float mx = -INFINITY;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float v = s[c2][hf][rt][i];
              if constexpr (MASKED) {
                const int key = kt0 + 32 * c2 + 8 * qgrp + 4 * hf + i;
                v = (key <= tpos) ? v : -INFINITY;
                s[c2][hf][rt][i] = v;
              }
              mx = __builtin_elementwise_maximum(mx, v);
            }
        lm[rt] = mx;
      }
      // Raise a row's running maximum only when the tile's maximum exceeds it
      // by more than the slack. The wave takes the branch when any of its
      // rows needs it; rows that keep their maximum scale by exp2(0) = 1
      // exactly.
      if (__builtin_amdgcn_ballot_w64(lm[0] * sl2 > m[0] + RESCALE_SLACK ||
                                      lm[1] * sl2 > m[1] + RESCALE_SLACK) != 0) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          const float mx = max_over_row_groups(lm[rt]);
          const float mt = (MASKED && mx == -INFINITY) ? -INFINITY : mx * sl2;
          const float nm = mt > m[rt] + RESCALE_SLACK ? mt : m[rt];
          const float alpha = fast_exp2(m[rt] - nm);
          m[rt] = nm;
          lsum[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt][rt] *= alpha;
        }
      }
      const uint32_t ones = 0x3F803F80u;  // two bf16 1.0
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const float nm = -m[rt];
        float ps = lsum[rt];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          uint32_t w[4];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int i2 = 0; i2 < 2; ++i2) {
              float p0 = fast_exp2(fmaf(s[c2][hf][rt][2 * i2], sl2, nm));
              float p1 = fast_exp2(fmaf(s[c2][hf][rt][2 * i2 + 1], sl2, nm));
              if constexpr (MASKED) {
                p0 = (s[c2][hf][rt][2 * i2] == -INFINITY) ? 0.0f : p0;
                p1 = (s[c2][hf][rt][2 * i2 + 1] == -INFINITY) ? 0.0f : p1;
              }
              const uint32_t pk = pack2_bf16(p0, p1);
              w[2 * hf + i2] = pk;
              ps = dot2_bf16(pk, ones, ps);  // the rounded weights the PV product uses
            }
          pb[rt][c2] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        }
        lsum[rt] = ps;
      }
    };
    if (kt0 + KT - 1 > c + wrow0) softmax(std::true_type{});
    else softmax(std::false_type{});

    // ---- O^T += V^T P^T; V^T fragments come from the transposing read ----
    const int src_key = 8 * qgrp + (lrow >> 2);  // + 32*c2 + 4*h
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int gran = 2 * dt + ((lrow & 3) >> 1);
      const int half = (lrow & 1) * 4;
      bf16x8 a[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        uint2 r[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int key = 32 * c2 + 4 * h + src_key;
          r[h] = lds_read_tr4(&Vt[key * D + ((gran ^ swz_v(key)) * 8) + half]);
        }
        a[c2] = __builtin_bit_cast(bf16x8, make_uint4(r[0].x, r[0].y, r[1].x, r[1].y));
      }
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        o[dt][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c2], pb[0][c2], o[dt][0], 0, 0, 0);
        o[dt][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c2], pb[1][c2], o[dt][1], 0, 0, 0);
      }
    }
    // Schedule: the V^T operands of two d tiles, then each d tile's MFMAs
    // followed by the reads of the d tile two ahead.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int g = 0; g < DT - 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  for (int kt0 = 0; kt0 < kv_end; kt0 += 2 * KT) {
    step(kt0, kv0, kv1, 0);
    if (kt0 + KT < kv_end) step(kt0 + KT, kv1, kv0, 1);
  }

  // ---- normalise and write: lane holds O[row][16*dt + 4*qgrp + 0..3] ----
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    float lt = lsum[rt];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = out_scale / lt;
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

template <int D, int HW, typename CT>
__global__ __launch_bounds__(256, 2) void prefill_chunk_kernel(PrefillParams p) {
  prefill_body<D, HW, CT>(p, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Query heads one prefill workgroup serves (4 waves: HW heads x 4/HW row
// groups); it divides the group size.
inline int32_t prefill_heads_per_wg(int32_t group) {
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

// PrefillParams of a validated call (prefill.hip); row_blocks and num_seqs
// are set by the launcher.
PrefillParams make_prefill_params(const PrefillArgs& a);

}  // namespace pa
