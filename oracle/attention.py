"""Plain fp64 attention over a block-paged KV cache (CPU oracle).

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the library.

What the method computes. The mini-vllm page (section "mini-vllm 的架构设计",
item 2 "KVCache") keeps K/V rows in a preallocated tensor split into
fixed-size physical blocks and finds the rows of a sequence through its block
table; the nano-vllm page (section 3.1, the Sequence fields) gives each
sequence a list of physical block ids. Paging only changes WHERE a row lives:
attention over the paged cache equals ordinary scaled dot-product attention
over the sequence's rows taken in logical order (the mini-vllm page's
benchmark section compares exactly this cached path against full recompute).
So every function here first walks the block table literally to rebuild the
contiguous rows, then applies the plain definition

    o = softmax(scale * K q) V

in fp64. Neither page prints the attention formula; this plain reading, the
head grouping g = h // (Hq/Hkv) for grouped-query attention, and the
bottom-right causal alignment of a prefill chunk are readings, not quotes.

Array conventions (all numpy):
  * dtype "f32": float32 arrays.  dtype "bf16": uint16 arrays holding the
    bfloat16 bit patterns; they are widened to fp64 exactly.
  * pools: [num_blocks][block_size][num_kv_heads][head_dim]
  * q / out: [tokens][num_heads][head_dim]
  * block_tables: int [num_seqs][max_blocks_per_seq]
  * context_lens[i] counts every token of sequence i, the newest included.
"""

from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# element widening
# ---------------------------------------------------------------------------

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact conversion of stored elements to fp64.

    bf16 is the upper half of an IEEE float32, so shifting the 16 stored bits
    into the high half of a 32-bit word gives the same value as a float32,
    which fp64 holds exactly.
    """
    if dtype == "bf16":
        a = np.ascontiguousarray(a, dtype=np.uint16)
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# O-store: scatter new rows into the pools by slot
# ---------------------------------------------------------------------------

def store_kvcache(k_pool, v_pool, key, value, slot_mapping, block_size):
    """Write each new token's K/V row into the pool slot named for it.

    Slot s lives in physical block s // block_size at row s % block_size
    (the block table locates writes as well as reads: mini-vllm page, item 2
    "KVCache"). A negative slot marks padding and is skipped (a reading: the
    pages say nothing about padding). Rows are copied bit for bit; the pools
    passed in are not modified, new arrays are returned.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    for t, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        block, row = divmod(int(s), block_size)
        k_out[block, row] = key[t]
        v_out[block, row] = value[t]
    return k_out, v_out


# ---------------------------------------------------------------------------
# O-gather: the literal block-table walk
# ---------------------------------------------------------------------------

def gather_context(pool, table_row, length, block_size):
    """Rows 0..length-1 of one sequence, in logical order.

    Logical token j sits in physical block table_row[j // block_size] at row
    j % block_size (nano-vllm page §3.1: block_table maps a sequence onto
    physical blocks; mini-vllm page item 2: reads go through the table).
    Returns [length][num_kv_heads][head_dim] in the pool's storage type.
    """
    j = np.arange(int(length))
    blocks = np.asarray(table_row)[j // block_size]
    rows = j % block_size
    return pool[blocks, rows]


# ---------------------------------------------------------------------------
# plain attention of one query row
# ---------------------------------------------------------------------------

def attend(q_row, keys, values, scale):
    """softmax(scale * keys @ q_row) @ values, fp64, max-shifted for range.

    q_row [D], keys [L][D], values [L][D] (fp64). Subtracting the maximum
    logit leaves the softmax unchanged and keeps exp() finite.
    """
    s = scale * (keys @ q_row)
    p = np.exp(s - s.max())
    return (p @ values) / p.sum()


# ---------------------------------------------------------------------------
# O-decode: one query token per sequence
# ---------------------------------------------------------------------------

def decode(q, k_pool, v_pool, block_tables, context_lens, scale, block_size, dtype):
    """Decode attention: sequence i's single query attends to its
    context_lens[i] cached tokens (the newest included).

    q [B][Hq][D]; returns fp64 [B][Hq][D]. Query head h reads KV head
    h // (Hq // Hkv).
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    group = Hq // Hkv
    qf = widen(q, dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for i in range(B):
        L = int(context_lens[i])
        kc = widen(gather_context(k_pool, block_tables[i], L, block_size), dtype)
        vc = widen(gather_context(v_pool, block_tables[i], L, block_size), dtype)
        for h in range(Hq):
            g = h // group
            out[i, h] = attend(qf[i, h], kc[:, g, :], vc[:, g, :], scale)
    return out


# ---------------------------------------------------------------------------
# O-split: split-context partitions, then the exact merge
# ---------------------------------------------------------------------------

def partition_state(q_row, keys, values, scale):
    """Unnormalised softmax state of one slice of the context.

    Returns (m, l, acc): the slice's largest logit, the sum of exp(s - m),
    and the exp(s - m)-weighted sum of value rows.
    """
    s = scale * (keys @ q_row)
    m = s.max()
    p = np.exp(s - m)
    return m, p.sum(), p @ values


def merge_states(states):
    """Combine slice states into the softmax over their union.

    With M the largest slice maximum and w_p = exp(m_p - M), the union's
    normaliser is sum_p w_p l_p and its weighted value sum is sum_p w_p acc_p;
    their ratio is the attention output. In exact arithmetic this equals
    attention over the whole context for any slicing.
    """
    M = max(m for m, _, _ in states)
    num = sum(np.exp(m - M) * acc for m, _, acc in states)
    den = sum(np.exp(m - M) * l for m, l, _ in states)
    return num / den


def decode_partitioned(q, k_pool, v_pool, block_tables, context_lens, scale,
                       block_size, dtype, partition_size):
    """Decode with the context of each sequence cut into slices of
    partition_size tokens ([p*P, min((p+1)*P, L))), one state per slice,
    merged by merge_states."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    group = Hq // Hkv
    qf = widen(q, dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for i in range(B):
        L = int(context_lens[i])
        kc = widen(gather_context(k_pool, block_tables[i], L, block_size), dtype)
        vc = widen(gather_context(v_pool, block_tables[i], L, block_size), dtype)
        for h in range(Hq):
            g = h // group
            states = []
            for start in range(0, L, partition_size):
                stop = min(start + partition_size, L)
                states.append(partition_state(qf[i, h], kc[start:stop, g, :],
                                              vc[start:stop, g, :], scale))
            out[i, h] = merge_states(states)
    return out


# ---------------------------------------------------------------------------
# O-prefill: a chunk of new tokens, causal over cached + new context
# ---------------------------------------------------------------------------

def prefill(q, k_pool, v_pool, block_tables, query_start_loc, context_lens,
            scale, block_size, dtype):
    """Chunked causal prefill.

    Sequence i owns query rows query_start_loc[i] .. query_start_loc[i+1]-1
    (n_i rows). Its context holds context_lens[i] = c_i + n_i tokens, the
    first c_i already cached and the last n_i the chunk's own (already
    stored). Row t of the chunk sits at absolute position c_i + t and attends
    to keys 0 .. c_i + t (causal, aligned to the end of the context).
    Returns fp64 [sum n_i][Hq][D].
    """
    T, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    group = Hq // Hkv
    qf = widen(q, dtype)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    B = len(context_lens)
    for i in range(B):
        start, stop = int(query_start_loc[i]), int(query_start_loc[i + 1])
        n = stop - start
        L = int(context_lens[i])
        c = L - n
        kc = widen(gather_context(k_pool, block_tables[i], L, block_size), dtype)
        vc = widen(gather_context(v_pool, block_tables[i], L, block_size), dtype)
        for t in range(n):
            visible = c + t + 1
            for h in range(Hq):
                g = h // group
                out[start + t, h] = attend(qf[start + t, h], kc[:visible, g, :],
                                           vc[:visible, g, :], scale)
    return out


def prefill_rows(q, k_pool, v_pool, block_tables, query_start_loc, context_lens,
                 scale, block_size, dtype, rows):
    """The same as prefill() but only for the listed (token, head) pairs;
    for sampled checks at sizes where the full chunk is too slow on a CPU.
    Returns fp64 [len(rows)][D]."""
    Hq = q.shape[1]
    Hkv = k_pool.shape[2]
    group = Hq // Hkv
    qsl = np.asarray(query_start_loc)
    out = np.zeros((len(rows), q.shape[2]), dtype=np.float64)
    cache = {}
    for r, (tok, h) in enumerate(rows):
        i = int(np.searchsorted(qsl, tok, side="right") - 1)
        n = int(qsl[i + 1] - qsl[i])
        L = int(context_lens[i])
        t = tok - int(qsl[i])
        if i not in cache:
            cache[i] = (widen(gather_context(k_pool, block_tables[i], L, block_size), dtype),
                        widen(gather_context(v_pool, block_tables[i], L, block_size), dtype))
        kc, vc = cache[i]
        visible = L - n + t + 1
        g = h // group
        out[r] = attend(widen(q[tok, h], dtype), kc[:visible, g, :], vc[:visible, g, :], scale)
    return out


def decode_rows(q, k_pool, v_pool, block_tables, context_lens, scale, block_size,
                dtype, rows):
    """decode() for the listed (sequence, head) pairs only; fp64 [len(rows)][D]."""
    Hq = q.shape[1]
    Hkv = k_pool.shape[2]
    group = Hq // Hkv
    out = np.zeros((len(rows), q.shape[2]), dtype=np.float64)
    cache = {}
    for r, (i, h) in enumerate(rows):
        L = int(context_lens[i])
        if i not in cache:
            cache[i] = (widen(gather_context(k_pool, block_tables[i], L, block_size), dtype),
                        widen(gather_context(v_pool, block_tables[i], L, block_size), dtype))
        kc, vc = cache[i]
        g = h // group
        out[r] = attend(widen(q[i, h], dtype), kc[:, g, :], vc[:, g, :], scale)
    return out
