"""8-bit float (E4M3) KV cache: quantise on store, dequantise in decode and
chunked prefill (CPU oracle).

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the library.

The nano-vllm page lists quantisation among its extension suggestions
(section 5.3) and the Nano-vLLM tutorial page names the effect of quantised
compression on inference speed as a direction for further study (its closing
list). The pages give no format; this oracle takes the OCP 8-bit floating-point
format E4M3 (the FP8 type gfx950 converts to and from in hardware), defined by its fields:

  * 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
  * exponent field 0: subnormal, (-1)^s * 2^-6 * m/8;
  * exponent field 1..15: (-1)^s * 2^(e-7) * (1 + m/8), except that
    exponent 15 with mantissa 7 is NaN; there is no infinity;
  * the largest finite magnitude is 2^8 * 1.75 = 448.

Readings where the pages are silent:
  * a K or V element x of KV head h is stored as the E4M3 code nearest to
    x / scale_h (ties to the even code, i.e. the even mantissa), where the
    division is one IEEE float32 division and |x / scale_h| is first
    saturated at 448; the per-head scales are caller inputs;
  * decode reads element x back as value(code) * scale_h and attends in the
    usual way (oracle.attention.attend) over those values; chunked prefill
    does the same for each row of a chunk over its causal prefix.
"""

from __future__ import annotations

import functools
import math

import numpy as np

from oracle import attention as oa

E4M3_MAX = 448.0


def e4m3_value(code):
    """The value of one E4M3 code (NaN for the two NaN codes)."""
    c = int(code) & 0xFF
    sign = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 0xF
    m = c & 0x7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table():
    """fp64 value of every code 0..255 (index = code)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def quantize_e4m3(x, scale):
    """uint8 codes of x / scale (one float32 division), nearest E4M3 value
    with ties to the even code, magnitude saturated at 448 (infinities
    included). NaN gives the NaN code 0x7F with the sign of the input."""
    table = e4m3_table()
    pos = table[:0x7F]                    # codes 0x00..0x7E: the non-negative finite values, ascending
    y = (np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float32)
    a = np.abs(y.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    hi = np.minimum(np.searchsorted(pos, a, side="left"), len(pos) - 1)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    dlo = a - pos[lo]
    dhi = pos[hi] - a
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | np.where(np.signbit(y), np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def dequantize_rows(codes, scales):
    """fp64 values of codes [..][Hkv][D]: head h's codes times scales[h]."""
    vals = e4m3_table()[np.asarray(codes, dtype=np.uint8)]
    return vals * np.asarray(scales, dtype=np.float64)[:, None]


def store_kvcache_fp8(k_codes, v_codes, key, value, slot_mapping, block_size, k_scale, v_scale,
                      dtype):
    """Quantise each new token's K/V row (KV head h with k_scale[h],
    v_scale[h]) into the code pools at its slot: block s // block_size, row
    s % block_size, as for the unquantised store; negative slots are
    skipped. key/value are [T][Hkv][D] of storage type dtype ("bf16" bit
    patterns or "f32"); the code pools are uint8 [NB][bs][Hkv][D]; new
    arrays are returned."""
    k_out = np.array(k_codes, copy=True)
    v_out = np.array(v_codes, copy=True)
    kf = oa.widen(key, dtype).astype(np.float32)      # exact: both storage types fit float32
    vf = oa.widen(value, dtype).astype(np.float32)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = np.flatnonzero(slots >= 0)
    block, row = slots[keep] // block_size, slots[keep] % block_size
    for h in range(k_out.shape[2]):
        k_out[block, row, h] = quantize_e4m3(kf[keep, h], k_scale[h])
        v_out[block, row, h] = quantize_e4m3(vf[keep, h], v_scale[h])
    return k_out, v_out


def decode_fp8(q, k_codes, v_codes, k_scale, v_scale, block_tables, context_lens, scale,
               block_size, q_dtype):
    """Decode attention over an E4M3 cache: walk the block table for the
    sequence's codes (oracle.attention.gather_context), read them back as
    value(code) * scale_h, and apply softmax(scale * K q) V
    (oracle.attention.attend) in fp64. q is [B][Hq][D] of q_dtype."""
    B, Hq, D = q.shape
    Hkv = k_codes.shape[2]
    group = Hq // Hkv
    qf = oa.widen(q, q_dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for i in range(B):
        L = int(context_lens[i])
        kc = dequantize_rows(oa.gather_context(k_codes, block_tables[i], L, block_size), k_scale)
        vc = dequantize_rows(oa.gather_context(v_codes, block_tables[i], L, block_size), v_scale)
        for h in range(Hq):
            g = h // group
            out[i, h] = oa.attend(qf[i, h], kc[:, g, :], vc[:, g, :], scale)
    return out


def prefill_fp8(q, k_codes, v_codes, k_scale, v_scale, block_tables, query_start_loc,
                context_lens, scale, block_size, q_dtype, rows=None):
    """Chunked causal prefill over an E4M3 cache: the chunked-prefill
    definition (sequence i owns query rows query_start_loc[i] ..
    query_start_loc[i+1]-1; row t of its chunk sits at position c_i + t with
    c_i = context_lens[i] - n_i and attends to keys 0 .. c_i + t) over the
    context read back as value(code) * scale_h for K and V.

    q is [sum n_i][Hq][D] of q_dtype. Without rows: fp64 [sum n_i][Hq][D].
    With rows, a list of (query row, head) pairs: fp64 [len(rows)][D] for
    just those (sampled checks at sizes the full chunk is too slow for)."""
    T, Hq, D = q.shape
    Hkv = k_codes.shape[2]
    group = Hq // Hkv
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    qf = oa.widen(q, q_dtype)
    wanted = {}
    if rows is None:
        for r in range(T):
            for h in range(Hq):
                wanted.setdefault(r, []).append(h)
    else:
        for r, h in rows:
            wanted.setdefault(int(r), []).append(int(h))
    result = {}
    for i in range(len(context_lens)):
        start, stop = int(qsl[i]), int(qsl[i + 1])
        mine = [r for r in wanted if start <= r < stop]
        if not mine:
            continue
        L = int(context_lens[i])
        c = L - (stop - start)
        kc = dequantize_rows(oa.gather_context(k_codes, block_tables[i], L, block_size), k_scale)
        vc = dequantize_rows(oa.gather_context(v_codes, block_tables[i], L, block_size), v_scale)
        for r in mine:
            visible = c + (r - start) + 1
            for h in wanted[r]:
                g = h // group
                result[(r, h)] = oa.attend(qf[r, h], kc[:visible, g, :], vc[:visible, g, :], scale)
    if rows is None:
        out = np.zeros((T, Hq, D), dtype=np.float64)
        for (r, h), v in result.items():
            out[r, h] = v
        return out
    return np.stack([result[(int(r), int(h))] for r, h in rows]) if rows else np.zeros((0, D))
