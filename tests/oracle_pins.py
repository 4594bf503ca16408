"""Checks that tie the CPU oracle to facts outside itself.

Each pin_* function raises AssertionError when the oracle disagrees with what
the pages or the mathematics fix: closed forms, a library attention routine,
invariances of paging (block renumbering, sharing vs duplication), the
grouped-query/multi-head equivalence, slicing invariance of the split merge,
the prefill/decode identity, and the rolling hash's closed-form vectors.

The functions look the oracle up through its modules at call time, so a test
can plant a mistake in the oracle (monkeypatch) and see which pins catch it.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle.attention as oa
import oracle.fp8 as of8
import oracle.prefix_cache as opc


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _paged_from_contiguous(rows_per_seq, block_size, num_blocks, rng, fill=np.nan):
    """Lay contiguous per-sequence rows into a block pool, block by block
    (slice copies; no slot arithmetic), with a random block order."""
    shape = rows_per_seq[0].shape[1:]
    pool = np.full((num_blocks, block_size) + shape, fill, dtype=rows_per_seq[0].dtype)
    perm = rng.permutation(num_blocks)
    nmax = max(math.ceil(len(r) / block_size) for r in rows_per_seq)
    tables = np.full((len(rows_per_seq), nmax), -1, dtype=np.int64)
    nxt = 0
    for i, rows in enumerate(rows_per_seq):
        for k in range(math.ceil(len(rows) / block_size)):
            b = int(perm[nxt])
            nxt += 1
            part = rows[k * block_size:(k + 1) * block_size]
            pool[b, :len(part)] = part
            tables[i, k] = b
    return pool, tables


def _sdpa(q, k, v, scale, causal=False):
    """torch's attention routine on CPU in fp64. q [H][Lq][D], k/v [H][L][D]."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=scale, is_causal=causal)
    return out[0].numpy()


def _decode_case(seed=1, lens=(1, 5, 13, 32), Hq=6, Hkv=2, D=16, bs=4, dtype="f32"):
    rng = _rng(seed)
    kc = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    vc = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    nb = sum(math.ceil(L / bs) for L in lens) + 3
    r2 = _rng(seed + 100)
    kp, tables = _paged_from_contiguous(kc, bs, nb, r2)
    vp, tables_v = _paged_from_contiguous(vc, bs, nb, _rng(seed + 100))
    assert np.array_equal(tables, tables_v)
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
    return dict(q=q, kp=kp, vp=vp, tables=tables, lens=np.array(lens), kc=kc, vc=vc,
                bs=bs, scale=1.0 / math.sqrt(D), Hq=Hq, Hkv=Hkv, D=D)


# ---------------------------------------------------------------------------
# store / gather
# ---------------------------------------------------------------------------

def pin_store_bytes():
    """Stored rows land at slot = flat row index of the [NB*bs] row view;
    every other byte is untouched; negative slots write nothing."""
    rng = _rng(2)
    NB, bs, Hkv, D = 6, 8, 2, 4
    for dt in (np.uint16, np.float32):
        if dt is np.uint16:
            kp = rng.integers(0, 1 << 16, size=(NB, bs, Hkv, D), dtype=np.uint16)
            vp = rng.integers(0, 1 << 16, size=(NB, bs, Hkv, D), dtype=np.uint16)
            key = rng.integers(0, 1 << 16, size=(5, Hkv, D), dtype=np.uint16)
            val = rng.integers(0, 1 << 16, size=(5, Hkv, D), dtype=np.uint16)
        else:
            kp = rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32)
            vp = rng.standard_normal((NB, bs, Hkv, D)).astype(np.float32)
            key = rng.standard_normal((5, Hkv, D)).astype(np.float32)
            val = rng.standard_normal((5, Hkv, D)).astype(np.float32)
        slots = np.array([7, -1, 40, 0, 47], dtype=np.int32)
        k2, v2 = oa.store_kvcache(kp, vp, key, val, slots, bs)
        ek = kp.reshape(NB * bs, Hkv, D).copy()
        ev = vp.reshape(NB * bs, Hkv, D).copy()
        for t, s in enumerate(slots):
            if s >= 0:
                ek[s] = key[t]
                ev[s] = val[t]
        assert k2.tobytes() == ek.reshape(kp.shape).tobytes()
        assert v2.tobytes() == ev.reshape(vp.shape).tobytes()
        assert kp.tobytes() != k2.tobytes()


def pin_gather_inverts_layout():
    """Gathering through the table returns the contiguous rows that were laid
    out block by block."""
    c = _decode_case(seed=3, lens=(1, 4, 9, 17), bs=4)
    for i, L in enumerate(c["lens"]):
        got = oa.gather_context(c["kp"], c["tables"][i], L, c["bs"])
        assert np.array_equal(got, c["kc"][i])


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def pin_decode_vs_sdpa():
    """Paged decode equals torch's attention over the contiguous rows."""
    c = _decode_case(seed=4)
    out = oa.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], c["scale"], c["bs"], "f32")
    G = c["Hq"] // c["Hkv"]
    for i, L in enumerate(c["lens"]):
        k = np.repeat(c["kc"][i].astype(np.float64), G, axis=1).transpose(1, 0, 2)
        v = np.repeat(c["vc"][i].astype(np.float64), G, axis=1).transpose(1, 0, 2)
        q = c["q"][i].astype(np.float64)[:, None, :]
        ref = _sdpa(q, np.ascontiguousarray(k), np.ascontiguousarray(v), c["scale"])[:, 0, :]
        assert np.max(np.abs(out[i] - ref)) < 1e-12


def pin_decode_closed_forms():
    """L=1 returns v_0 exactly; q=0 or equal keys give the mean value row;
    a logit raised by 1e3 over the rest returns that row's value."""
    rng = _rng(5)
    D, bs = 8, 4
    # L = 1
    kp = rng.standard_normal((3, bs, 1, D)).astype(np.float32)
    vp = rng.standard_normal((3, bs, 1, D)).astype(np.float32)
    q = rng.standard_normal((1, 1, D)).astype(np.float32)
    out = oa.decode(q, kp, vp, np.array([[2]]), np.array([1]), 0.3, bs, "f32")
    assert np.array_equal(out[0, 0], vp[2, 0, 0].astype(np.float64))
    # q = 0 -> uniform weights over the L rows
    L = 11
    rows_k = rng.standard_normal((L, 1, D)).astype(np.float32)
    rows_v = rng.standard_normal((L, 1, D)).astype(np.float32)
    kp, tb = _paged_from_contiguous([rows_k], bs, 5, _rng(6))
    vp, _ = _paged_from_contiguous([rows_v], bs, 5, _rng(6))
    out = oa.decode(np.zeros((1, 1, D), np.float32), kp, vp, tb, np.array([L]), 0.5, bs, "f32")
    assert np.max(np.abs(out[0, 0] - rows_v[:, 0].astype(np.float64).mean(0))) < 1e-14
    # equal keys -> uniform weights as well
    same = np.repeat(rows_k[:1], L, axis=0)
    kp2, _ = _paged_from_contiguous([same], bs, 5, _rng(6))
    qn = rng.standard_normal((1, 1, D)).astype(np.float32)
    out = oa.decode(qn, kp2, vp, tb, np.array([L]), 0.5, bs, "f32")
    assert np.max(np.abs(out[0, 0] - rows_v[:, 0].astype(np.float64).mean(0))) < 1e-14
    # one dominant logit: key 7 = q * c with scale*c*|q|^2 = 1e3 + others
    qd = np.zeros((1, 1, D), np.float32)
    qd[0, 0, 0] = 1.0
    ks = np.zeros((L, 1, D), np.float32)
    ks[:, 0, 0] = rng.standard_normal(L).astype(np.float32)
    ks[7, 0, 0] = 2000.0
    kp3, _ = _paged_from_contiguous([ks], bs, 5, _rng(6))
    out = oa.decode(qd, kp3, vp, tb, np.array([L]), 1.0, bs, "f32")
    assert np.max(np.abs(out[0, 0] - rows_v[7, 0].astype(np.float64))) < 1e-12


def pin_decode_block_permutation():
    """Renumbering physical blocks (and rewriting the tables) changes nothing,
    bit for bit."""
    c = _decode_case(seed=7)
    out = oa.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], c["scale"], c["bs"], "f32")
    nb = c["kp"].shape[0]
    perm = _rng(8).permutation(nb)           # new id of old block b is perm[b]
    kp2 = np.empty_like(c["kp"])
    vp2 = np.empty_like(c["vp"])
    kp2[perm] = c["kp"]
    vp2[perm] = c["vp"]
    t2 = np.where(c["tables"] >= 0, perm[np.maximum(c["tables"], 0)], -1)
    out2 = oa.decode(c["q"], kp2, vp2, t2, c["lens"], c["scale"], c["bs"], "f32")
    assert out.tobytes() == out2.tobytes()


def pin_decode_sharing_equals_duplication():
    """Two sequences reading one shared prefix block give the same result as
    when each owns a copy of it."""
    rng = _rng(9)
    bs, Hkv, D = 4, 2, 8
    prefix_k = rng.standard_normal((bs, Hkv, D)).astype(np.float32)
    prefix_v = rng.standard_normal((bs, Hkv, D)).astype(np.float32)
    tails_k = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in (3, 6)]
    tails_v = [rng.standard_normal((n, Hkv, D)).astype(np.float32) for n in (3, 6)]
    nb = 8
    kp = np.full((nb, bs, Hkv, D), np.nan, np.float32)
    vp = np.full((nb, bs, Hkv, D), np.nan, np.float32)
    kp[5], vp[5] = prefix_k, prefix_v
    kp[1, :3], vp[1, :3] = tails_k[0], tails_v[0]
    kp[6], vp[6] = tails_k[1][:4], tails_v[1][:4]
    kp[2, :2], vp[2, :2] = tails_k[1][4:], tails_v[1][4:]
    shared = np.array([[5, 1, -1], [5, 6, 2]])
    kd, vd = kp.copy(), vp.copy()
    kd[0], vd[0] = prefix_k, prefix_v       # private copy for sequence 1
    dup = np.array([[5, 1, -1], [0, 6, 2]])
    lens = np.array([bs + 3, bs + 6])
    q = rng.standard_normal((2, 4, D)).astype(np.float32)
    a = oa.decode(q, kp, vp, shared, lens, 0.35, bs, "f32")
    b = oa.decode(q, kd, vd, dup, lens, 0.35, bs, "f32")
    assert a.tobytes() == b.tobytes()
    assert np.isfinite(a).all()


def pin_gqa_equals_expanded_mha():
    """Grouped-query decode equals multi-head decode with each KV head
    repeated for the query heads of its group (heads h*G .. h*G+G-1)."""
    c = _decode_case(seed=10, Hq=6, Hkv=2)
    G = 3
    out = oa.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], c["scale"], c["bs"], "f32")
    kp = np.repeat(c["kp"], G, axis=2)
    vp = np.repeat(c["vp"], G, axis=2)
    out2 = oa.decode(c["q"], kp, vp, c["tables"], c["lens"], c["scale"], c["bs"], "f32")
    assert out.tobytes() == out2.tobytes()
    # and the groups really differ (a mapping h % Hkv would read other heads)
    assert np.max(np.abs(out[:, 1] - out[:, 3])) > 1e-3


def pin_partition_invariance():
    """Slicing the context and merging slice states gives the unsliced
    result to fp64 rounding, for any slice length."""
    c = _decode_case(seed=11, lens=(1, 7, 16, 33))
    ref = oa.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], c["scale"], c["bs"], "f32")
    for P in (1, 3, 4, 7, 16, 1000):
        got = oa.decode_partitioned(c["q"], c["kp"], c["vp"], c["tables"], c["lens"],
                                    c["scale"], c["bs"], "f32", P)
        assert np.max(np.abs(got - ref)) < 1e-12, P


def pin_merge_of_disjoint_states():
    """merge_states of two slices equals attention over their union (also
    when one slice's maximum is far below the other's)."""
    rng = _rng(12)
    D = 6
    q = rng.standard_normal(D)
    k1, k2 = rng.standard_normal((5, D)), rng.standard_normal((4, D)) + 3 * q
    v1, v2 = rng.standard_normal((5, D)), rng.standard_normal((4, D))
    s1 = oa.partition_state(q, k1, v1, 0.9)
    s2 = oa.partition_state(q, k2, v2, 0.9)
    got = oa.merge_states([s1, s2])
    ref = _sdpa(q[None, None], np.concatenate([k1, k2])[None], np.concatenate([v1, v2])[None], 0.9)[0, 0]
    assert np.max(np.abs(got - ref)) < 1e-12


def pin_bf16_widening():
    """bf16 bit patterns widen to the float32 values with the same top 16
    bits (0x3F80 is 1.0, 0xC000 is -2.0, 0x0001 the smallest subnormal)."""
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x0000, 0x8000], dtype=np.uint16)
    got = oa.widen(bits, "bf16")
    ref = np.array([1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0])
    assert np.array_equal(got, ref)
    assert np.signbit(got[5])
    t = torch.tensor([0.1, -3.7, 1e-3, 65504.0], dtype=torch.float32).to(torch.bfloat16)
    via_torch = t.to(torch.float64).numpy()
    assert np.array_equal(oa.widen(t.view(torch.int16).numpy().view(np.uint16), "bf16"), via_torch)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def _prefill_case(seed, cached, chunk, Hq=4, Hkv=2, D=8, bs=4):
    rng = _rng(seed)
    lens = [c + n for c, n in zip(cached, chunk)]
    kc = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    vc = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    nb = sum(math.ceil(L / bs) for L in lens) + 2
    kp, tables = _paged_from_contiguous(kc, bs, nb, _rng(seed + 1))
    vp, _ = _paged_from_contiguous(vc, bs, nb, _rng(seed + 1))
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int64)
    q = rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32)
    return dict(q=q, kp=kp, vp=vp, tables=tables, lens=np.array(lens), qsl=qsl, kc=kc, vc=vc,
                bs=bs, scale=1.0 / math.sqrt(D), Hq=Hq, Hkv=Hkv, D=D, cached=cached, chunk=chunk)


def pin_prefill_row_is_decode():
    """Prefill row t of a sequence equals decode of that row's query over
    the first c + t + 1 tokens, bit for bit."""
    c = _prefill_case(13, cached=[0, 5, 9], chunk=[3, 4, 6])
    out = oa.prefill(c["q"], c["kp"], c["vp"], c["tables"], c["qsl"], c["lens"], c["scale"], c["bs"], "f32")
    for i in range(3):
        for t in range(c["chunk"][i]):
            r = int(c["qsl"][i]) + t
            one = oa.decode(c["q"][r:r + 1], c["kp"], c["vp"], c["tables"][i:i + 1],
                            np.array([c["cached"][i] + t + 1]), c["scale"], c["bs"], "f32")
            assert out[r].tobytes() == one[0].tobytes()


def pin_prefill_c0_is_causal_sdpa():
    """With nothing cached, prefill is ordinary causal attention."""
    c = _prefill_case(14, cached=[0, 0], chunk=[7, 12])
    out = oa.prefill(c["q"], c["kp"], c["vp"], c["tables"], c["qsl"], c["lens"], c["scale"], c["bs"], "f32")
    G = c["Hq"] // c["Hkv"]
    for i in range(2):
        rows = slice(int(c["qsl"][i]), int(c["qsl"][i + 1]))
        q = c["q"][rows].astype(np.float64).transpose(1, 0, 2)
        k = np.repeat(c["kc"][i].astype(np.float64), G, axis=1).transpose(1, 0, 2)
        v = np.repeat(c["vc"][i].astype(np.float64), G, axis=1).transpose(1, 0, 2)
        ref = _sdpa(np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v),
                    c["scale"], causal=True).transpose(1, 0, 2)
        assert np.max(np.abs(out[rows] - ref)) < 1e-12


def pin_prefill_chunk_split():
    """Running a chunk as two smaller chunks (the second with the first one
    counted as cached) gives the same rows, bit for bit."""
    c = _prefill_case(15, cached=[6], chunk=[9])
    full = oa.prefill(c["q"], c["kp"], c["vp"], c["tables"], c["qsl"], c["lens"], c["scale"], c["bs"], "f32")
    n1 = 4
    first = oa.prefill(c["q"][:n1], c["kp"], c["vp"], c["tables"], np.array([0, n1]),
                       np.array([6 + n1]), c["scale"], c["bs"], "f32")
    second = oa.prefill(c["q"][n1:], c["kp"], c["vp"], c["tables"], np.array([0, 9 - n1]),
                        np.array([15]), c["scale"], c["bs"], "f32")
    assert np.concatenate([first, second]).tobytes() == full.tobytes()


def pin_prefill_rows_subset():
    """The sampled-row form returns the same values as the full chunk."""
    c = _prefill_case(16, cached=[2, 7], chunk=[5, 3])
    full = oa.prefill(c["q"], c["kp"], c["vp"], c["tables"], c["qsl"], c["lens"], c["scale"], c["bs"], "f32")
    rows = [(0, 0), (4, 3), (5, 1), (7, 2)]
    got = oa.prefill_rows(c["q"], c["kp"], c["vp"], c["tables"], c["qsl"], c["lens"], c["scale"],
                          c["bs"], "f32", rows)
    for r, (tok, h) in enumerate(rows):
        assert got[r].tobytes() == full[tok, h].tobytes()
    d = _decode_case(seed=17)
    fulld = oa.decode(d["q"], d["kp"], d["vp"], d["tables"], d["lens"], d["scale"], d["bs"], "f32")
    rows = [(0, 0), (3, 5), (2, 2)]
    got = oa.decode_rows(d["q"], d["kp"], d["vp"], d["tables"], d["lens"], d["scale"], d["bs"], "f32", rows)
    for r, (i, h) in enumerate(rows):
        assert got[r].tobytes() == fulld[i, h].tobytes()


# ---------------------------------------------------------------------------
# rolling hash and allocation
# ---------------------------------------------------------------------------

def pin_hash_vectors():
    """Closed-form values of h <- (31*h + t) mod 2**32."""
    for h in (0, 1, 12345, 0xFFFFFFFF):
        assert opc.compute_hash([], h) == h
    assert opc.compute_hash([1, 2, 3], 0) == 1 * 31 ** 2 + 2 * 31 + 3 == 1026
    assert opc.compute_hash([0], 0xFFFFFFFF) == (2 ** 32 - 31) == 4294967265
    ref = sum(t * pow(31, 255 - t, 2 ** 32) for t in range(256)) % 2 ** 32
    assert opc.compute_hash(range(256), 0) == ref == 452919424


def pin_hash_polynomial_and_chaining():
    """The fold equals the polynomial h*31^n + sum_k t_k 31^(n-1-k) mod 2^32,
    and hashing a+b equals hashing b from the hash of a."""
    rng = _rng(18)
    for n in (1, 2, 17, 256):
        toks = rng.integers(0, 50257, size=n).tolist()
        h0 = int(rng.integers(0, 2 ** 32))
        poly = (h0 * pow(31, n, 2 ** 32) + sum(t * pow(31, n - 1 - k, 2 ** 32)
                                               for k, t in enumerate(toks))) % 2 ** 32
        assert opc.compute_hash(toks, h0) == poly
        cut = n // 2
        assert opc.compute_hash(toks[cut:], opc.compute_hash(toks[:cut], h0)) == opc.compute_hash(toks, h0)


def pin_allocator_sharing_small():
    """Three sequences, two with a common two-block prefix: the prefix blocks
    are shared with two references; partial blocks are never shared; freeing
    returns every block and forgets every hash."""
    bs = 4
    common = [5, 6, 7, 8, 9, 10, 11, 12]
    seqs = [common + [1, 2], [40, 41, 42, 43, 44], common + [1, 2]]
    alloc = opc.PrefixBlockAllocator(list(range(10)), bs)
    tables = [alloc.allocate(s) for s in seqs]
    assert tables[0] == [0, 1, 2]
    assert tables[1] == [3, 4]
    assert tables[2] == [0, 1, 5]            # same partial tail, still private
    rc = alloc.ref_counts()
    assert rc[0] == 2 and rc[1] == 2 and rc[2] == 1 and rc[5] == 1
    assert sum(rc.values()) == sum(len(t) for t in tables)
    # a block of equal tokens after a different prefix is not shared
    t4 = alloc.allocate([50, 51, 52, 53] + common[4:8])
    assert t4[1] != 1
    for t in tables + [t4]:
        alloc.free_table(t)
    assert alloc.ref_counts() == {} and not alloc.hash_to_block_id
    assert sorted(alloc.free) == list(range(10))


def pin_cached_tokens():
    """num_cached_tokens counts the leading blocks that were hits: all of a
    repeated full-block prompt, none of a fresh one, and never a hit after a
    miss."""
    bs = 4
    alloc = opc.PrefixBlockAllocator(list(range(12)), bs)
    a = list(range(100, 110))                       # 2 full blocks + 2 tokens
    assert alloc.allocate_cached(a) == ([0, 1, 2], 0)
    assert alloc.allocate_cached(a) == ([0, 1, 3], 8)
    assert alloc.allocate_cached(a[:8]) == ([0, 1], 8)
    b = [1, 2, 3, 4] + a[4:8]                        # second block equal, first not
    t, c = alloc.allocate_cached(b)
    assert c == 0 and t[1] != 1
    # hits are always leading blocks: a hit needs the block before it in the
    # table to be its recorded parent, which a block just taken never is
    rng = _rng(31)
    alloc = opc.PrefixBlockAllocator(list(range(400)), bs)
    base = rng.integers(0, 6, size=40).tolist()
    for _ in range(30):
        cut = int(rng.integers(0, 41))
        toks = base[:cut] + rng.integers(0, 6, size=int(rng.integers(0, 12))).tolist()
        before = alloc.ref_counts()
        t, c = alloc.allocate_cached(toks)
        hit = [before.get(x, 0) > 0 for x in t]
        assert c == bs * sum(hit) and all(hit[:sum(hit)])


def pin_append_equals_allocate():
    """Appending a sequence token by token to an empty table builds the same
    table, slots and block hashes as allocating it whole, on allocators with
    the same free list."""
    rng = _rng(23)
    for bs, n in ((4, 1), (4, 4), (4, 13), (16, 50), (8, 64)):
        free = rng.permutation(64).tolist()
        toks = rng.integers(0, 50257, size=n).tolist()
        a1 = opc.PrefixBlockAllocator(free, bs)
        whole = a1.allocate(toks)
        a2 = opc.PrefixBlockAllocator(free, bs)
        table = []
        slots = [a2.append_token(table, j, t) for j, t in enumerate(toks)]
        assert table == whole
        assert slots == [whole[j // bs] * bs + j % bs for j in range(n)]
        assert a2.hash_to_block_id == a1.hash_to_block_id
        assert a2.ref_counts() == a1.ref_counts()


def pin_append_fills_are_shareable():
    """Blocks that decode appends fill are hashed like prompt blocks, so a
    later prompt with the same prefix shares them."""
    bs = 4
    alloc = opc.PrefixBlockAllocator(list(range(16)), bs)
    gen = [7, 7, 8, 9, 1, 2, 3, 4, 5]
    table = []
    for j, t in enumerate(gen):
        alloc.append_token(table, j, t)
    t2, c2 = alloc.allocate_cached(gen[:8] + [99])
    assert t2[:2] == table[:2] and c2 == 8 and t2[2] != table[2]
    assert alloc.ref_counts()[table[0]] == 2 and alloc.ref_counts()[table[2]] == 1
    alloc.free_table(table)
    alloc.free_table(t2)
    assert alloc.ref_counts() == {} and not alloc.hash_to_block_id


def pin_allocator_matches_structure(structure, block_size, num_sharers, prefix_tokens):
    """The hash-sharing allocator, fed the drawn token ids and free list,
    reproduces the drawn block tables; reference counts add up."""
    alloc = opc.PrefixBlockAllocator(structure["free_list"].tolist(), block_size)
    lens = structure["context_lens"]
    logical = 0
    for i, ids in enumerate(structure["token_ids"]):
        t = alloc.allocate(ids.tolist())
        nb = math.ceil(int(lens[i]) / block_size)
        assert t == structure["block_tables"][i, :nb].tolist(), i
        logical += nb
    rc = alloc.ref_counts()
    assert sum(rc.values()) == logical
    pb = prefix_tokens // block_size
    shared = [b for b, n in rc.items() if n > 1]
    if num_sharers > 1:
        assert sorted(shared) == sorted(structure["shared_blocks"])
        assert all(rc[b] == num_sharers for b in shared) and len(shared) == pb
    else:
        assert not shared
    assert len(rc) == logical - max(0, num_sharers - 1) * pb


# ---------------------------------------------------------------------------
# E4M3 KV cache
# ---------------------------------------------------------------------------

def pin_e4m3_closed_forms():
    """Codes whose values the format's field definition fixes by hand: one,
    two, the largest finite value, the smallest normal and subnormal, the
    sign bit, the NaN codes."""
    t = of8.e4m3_table()
    want = {0x00: 0.0, 0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x30: 0.5, 0x7E: 448.0, 0x78: 256.0,
            0x77: 240.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x04: 2.0 ** -7,
            0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9)}
    for code, v in want.items():
        assert t[code] == v, (hex(code), t[code], v)
    assert t[0x80] == 0.0 and math.copysign(1.0, t[0x80]) < 0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    assert np.array_equal(t[0x80:], -t[:0x80], equal_nan=True)


def pin_e4m3_table_vs_torch():
    """The value table equals torch's float8_e4m3fn reading of every byte."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    t = of8.e4m3_table()
    assert np.array_equal(np.isnan(ref), np.isnan(t))
    fin = ~np.isnan(t)
    assert np.array_equal(ref[fin], t[fin])


def pin_e4m3_quantize_vs_torch():
    """Inside the finite range, quantisation with scale 1 equals torch's
    float32 -> float8_e4m3fn conversion (nearest, ties to even), on random
    values over every binade, on every midpoint between neighbouring codes,
    and one float32 ulp either side of each midpoint."""
    rng = _rng(40)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 9, 20000))).astype(np.float32)
    t = of8.e4m3_table()
    pos = t[:0x7F]
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    x = np.concatenate([x, mid, -mid, up, dn, -up, -dn])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = of8.quantize_e4m3(x, 1.0)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:5]


def pin_e4m3_round_trip_and_ties():
    """Every finite code survives value -> quantise; a midpoint goes to the
    code with even mantissa; the rounding error is at most half the gap
    between neighbouring values."""
    t = of8.e4m3_table()
    codes = np.array([c for c in range(256) if not np.isnan(t[c])], dtype=np.uint8)
    assert np.array_equal(of8.quantize_e4m3(t[codes].astype(np.float32), 1.0), codes)
    pos = t[:0x7F]
    for c in range(0x7E):
        m = np.float32((pos[c] + pos[c + 1]) / 2)
        even = c if c % 2 == 0 else c + 1
        assert of8.quantize_e4m3(m, 1.0) == even, hex(c)
        assert of8.quantize_e4m3(-m, 1.0) == (even | 0x80)
    x = np.linspace(-448, 448, 40001).astype(np.float32)
    y = t[of8.quantize_e4m3(x, 1.0)]
    gap = np.where(np.abs(x) < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -6))) - 3))
    assert np.all(np.abs(y - x.astype(np.float64)) <= gap / 2)


def pin_e4m3_saturation_and_specials():
    """Magnitudes past 448, infinities included, saturate to +-448; NaN maps
    to a NaN code; signed zeros keep their sign."""
    q = of8.quantize_e4m3(np.array([448.0, 464.0, 480.0, 1e6, np.inf, -500.0, -np.inf],
                                   dtype=np.float32), 1.0)
    assert q.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert np.isnan(of8.e4m3_table()[of8.quantize_e4m3(np.float32(np.nan), 1.0)])
    assert of8.quantize_e4m3(np.float32(0.0), 1.0) == 0x00
    assert of8.quantize_e4m3(np.float32(-0.0), 1.0) == 0x80
    assert of8.quantize_e4m3(np.float32(2.0 ** -11), 1.0) == 0x00   # below half the smallest subnormal


def pin_e4m3_scale_divides():
    """The stored code is that of x / scale (not x * scale): scaling x and
    the scale by one power of two leaves every code unchanged."""
    rng = _rng(41)
    x = (rng.standard_normal(4000) * 8).astype(np.float32)
    base = of8.quantize_e4m3(x, 1.0)
    for k in (-3, 1, 5):
        assert np.array_equal(of8.quantize_e4m3(x * np.float32(2.0 ** k), 2.0 ** k), base)
    assert of8.quantize_e4m3(np.float32(3.0), 2.0) == of8.quantize_e4m3(np.float32(1.5), 1.0)
    assert of8.quantize_e4m3(np.float32(3.0), 0.5) == 0x4C           # 6.0 = 1.5 * 2^2: e=9, m=4


def pin_fp8_store_layout():
    """The E4M3 store puts, at slot s, the per-head quantised row (head h with
    its own k/v scale) and leaves every other byte alone; negative slots
    write nothing; bf16 and f32 inputs of equal value give equal codes."""
    rng = _rng(42)
    NB, bs, Hkv, D = 5, 4, 3, 8
    kp = rng.integers(0, 256, size=(NB, bs, Hkv, D), dtype=np.uint8)
    vp = rng.integers(0, 256, size=(NB, bs, Hkv, D), dtype=np.uint8)
    key = (rng.standard_normal((6, Hkv, D)) * 4).astype(np.float32)
    val = (rng.standard_normal((6, Hkv, D)) * 4).astype(np.float32)
    ks = np.array([0.5, 1.0, 0.03125])
    vs = np.array([2.0, 0.25, 1.0])
    slots = np.array([3, -1, 19, 0, 8, 13], dtype=np.int64)
    k2, v2 = of8.store_kvcache_fp8(kp, vp, key, val, slots, bs, ks, vs, "f32")
    ek = kp.reshape(NB * bs, Hkv, D).copy()
    ev = vp.reshape(NB * bs, Hkv, D).copy()
    t = of8.e4m3_table()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        for h in range(Hkv):
            for d in range(D):
                ek[s, h, d] = int(np.argmin(np.abs(np.nan_to_num(t[:0x7F], nan=1e9) - abs(key[i, h, d] / ks[h])))) | (0x80 if key[i, h, d] < 0 else 0)
                ev[s, h, d] = int(np.argmin(np.abs(np.nan_to_num(t[:0x7F], nan=1e9) - abs(val[i, h, d] / vs[h])))) | (0x80 if val[i, h, d] < 0 else 0)
    assert k2.tobytes() == ek.reshape(kp.shape).tobytes()
    assert v2.tobytes() == ev.reshape(vp.shape).tobytes()
    kb = (key.view(np.uint32) >> 16).astype(np.uint16)       # bf16 truncations are exact bf16 values
    key_b = (kb.astype(np.uint32) << 16).view(np.float32)
    k3, _ = of8.store_kvcache_fp8(kp, vp, kb, (val.view(np.uint32) >> 16).astype(np.uint16), slots,
                                  bs, ks, vs, "bf16")
    k4, _ = of8.store_kvcache_fp8(kp, vp, key_b, val, slots, bs, ks, vs, "f32")
    assert np.array_equal(k3, k4)


def _e4m3_by_fields(c):
    """E4M3 code values by hand from the format's fields (no NaN codes)."""
    c = c.astype(np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.exp2(e - 7.0))
    return np.where(c & 0x80, -mag, mag)


def _fp8_codes(rng, shape, moderate=False):
    c = rng.integers(0, 0x7F, size=shape).astype(np.uint8) | rng.choice(
        np.array([0, 0x80], dtype=np.uint8), size=shape)
    if moderate:  # keep logits moderate
        c = np.where((c & 0x7F) > 0x50, c & 0x87, c).astype(np.uint8)
    return c


def pin_fp8_decode_vs_sdpa():
    """E4M3 decode equals torch's attention over the contiguous rows read
    back as value(code) * scale (per KV head), the pool laid out block by
    block; scaling k_scale by c equals scaling the softmax scale by c, and
    scaling v_scale by c scales the output by c."""
    rng = _rng(43)
    lens, Hq, Hkv, D, bs = (1, 6, 13, 20), 6, 2, 16, 4
    kcodes = [rng.integers(0, 0x7F, size=(L, Hkv, D)).astype(np.uint8) | rng.choice(np.array([0, 0x80], dtype=np.uint8), size=(L, Hkv, D)) for L in lens]
    vcodes = [rng.integers(0, 0x7F, size=(L, Hkv, D)).astype(np.uint8) | rng.choice(np.array([0, 0x80], dtype=np.uint8), size=(L, Hkv, D)) for L in lens]
    kcodes = [np.where((c & 0x7F) > 0x50, c & 0x87, c).astype(np.uint8) for c in kcodes]   # keep logits moderate
    nb = sum(math.ceil(L / bs) for L in lens) + 2
    kp, tables = _paged_from_contiguous(kcodes, bs, nb, _rng(44), fill=0x7F)
    vp, tables_v = _paged_from_contiguous(vcodes, bs, nb, _rng(44), fill=0x7F)
    assert np.array_equal(tables, tables_v)
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
    ks, vs = np.array([0.5, 0.125]), np.array([2.0, 0.75])
    scale = 1.0 / math.sqrt(D)
    out = of8.decode_fp8(q, kp, vp, ks, vs, tables, np.array(lens), scale, bs, "f32")
    val = _e4m3_by_fields
    G = Hq // Hkv
    for i, L in enumerate(lens):
        k = np.repeat(val(kcodes[i]) * ks[None, :, None], G, axis=1).transpose(1, 0, 2)
        v = np.repeat(val(vcodes[i]) * vs[None, :, None], G, axis=1).transpose(1, 0, 2)
        ref = _sdpa(q[i].astype(np.float64)[:, None, :], np.ascontiguousarray(k),
                    np.ascontiguousarray(v), scale)[:, 0, :]
        assert np.max(np.abs(out[i] - ref)) < 1e-12
    out_k = of8.decode_fp8(q, kp, vp, ks * 3, vs, tables, np.array(lens), scale, bs, "f32")
    out_s = of8.decode_fp8(q, kp, vp, ks, vs, tables, np.array(lens), scale * 3, bs, "f32")
    assert np.max(np.abs(out_k - out_s)) < 1e-12
    out_v = of8.decode_fp8(q, kp, vp, ks, vs * np.array([3.0, 1.0]), tables, np.array(lens), scale, bs, "f32")
    assert np.max(np.abs(out_v[:, :G] - 3 * out[:, :G])) < 1e-12
    assert np.max(np.abs(out_v[:, G:] - out[:, G:])) < 1e-12


def _fp8_prefill_case(seed, cached, chunk, Hq=6, Hkv=2, D=16, bs=4):
    rng = _rng(seed)
    lens = [c + n for c, n in zip(cached, chunk)]
    kcodes = [_fp8_codes(rng, (L, Hkv, D), moderate=True) for L in lens]
    vcodes = [_fp8_codes(rng, (L, Hkv, D)) for L in lens]
    nb = sum(math.ceil(L / bs) for L in lens) + 2
    kp, tables = _paged_from_contiguous(kcodes, bs, nb, _rng(seed + 1), fill=0x7F)
    vp, tables_v = _paged_from_contiguous(vcodes, bs, nb, _rng(seed + 1), fill=0x7F)
    assert np.array_equal(tables, tables_v)
    qsl = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int64)
    q = rng.standard_normal((int(qsl[-1]), Hq, D)).astype(np.float32)
    ks, vs = rng.uniform(0.1, 2.0, Hkv), rng.uniform(0.1, 2.0, Hkv)
    return dict(q=q, kp=kp, vp=vp, tables=tables, lens=np.array(lens), qsl=qsl, kcodes=kcodes,
                vcodes=vcodes, ks=ks, vs=vs, bs=bs, scale=1.0 / math.sqrt(D), Hq=Hq, Hkv=Hkv,
                cached=cached, chunk=chunk)


def _prefill_fp8_of(c, **kw):
    return of8.prefill_fp8(c["q"], c["kp"], c["vp"], c["ks"], c["vs"], c["tables"], c["qsl"],
                           c["lens"], c["scale"], c["bs"], "f32", **kw)


def pin_fp8_prefill_vs_sdpa():
    """E4M3 chunked prefill equals torch's attention over the contiguous
    rows read back (by hand, from the format's fields) as value(code) *
    scale, with the causal mask aligned to the end of the context (row t
    sees keys 0 .. c + t); with nothing cached it is torch's ordinary causal
    attention."""
    c = _fp8_prefill_case(45, cached=[0, 7, 10], chunk=[9, 5, 1])
    out = _prefill_fp8_of(c)
    G = c["Hq"] // c["Hkv"]
    for i in range(3):
        rows = slice(int(c["qsl"][i]), int(c["qsl"][i + 1]))
        n, L = c["chunk"][i], int(c["lens"][i])
        k = np.repeat(_e4m3_by_fields(c["kcodes"][i]) * c["ks"][None, :, None], G, axis=1)
        v = np.repeat(_e4m3_by_fields(c["vcodes"][i]) * c["vs"][None, :, None], G, axis=1)
        q = c["q"][rows].astype(np.float64).transpose(1, 0, 2)
        mask = np.arange(L)[None, :] <= (L - n + np.arange(n))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(np.ascontiguousarray(q))[None],
            torch.from_numpy(np.ascontiguousarray(k.transpose(1, 0, 2)))[None],
            torch.from_numpy(np.ascontiguousarray(v.transpose(1, 0, 2)))[None],
            attn_mask=torch.from_numpy(mask), scale=c["scale"])[0].numpy().transpose(1, 0, 2)
        assert np.max(np.abs(out[rows] - ref)) < 1e-12
        if c["cached"][i] == 0:
            causal = _sdpa(np.ascontiguousarray(q), np.ascontiguousarray(k.transpose(1, 0, 2)),
                           np.ascontiguousarray(v.transpose(1, 0, 2)), c["scale"], causal=True)
            assert np.max(np.abs(out[rows] - causal.transpose(1, 0, 2))) < 1e-12


def pin_fp8_prefill_row_is_decode():
    """E4M3 prefill row t of a sequence equals E4M3 decode of that row's
    query over the first c + t + 1 tokens, bit for bit."""
    c = _fp8_prefill_case(46, cached=[0, 6, 3], chunk=[4, 3, 7])
    out = _prefill_fp8_of(c)
    for i in range(3):
        for t in range(c["chunk"][i]):
            r = int(c["qsl"][i]) + t
            one = of8.decode_fp8(c["q"][r:r + 1], c["kp"], c["vp"], c["ks"], c["vs"],
                                 c["tables"][i:i + 1], np.array([c["cached"][i] + t + 1]),
                                 c["scale"], c["bs"], "f32")
            assert out[r].tobytes() == one[0].tobytes()


def pin_fp8_prefill_rows_subset():
    """The sampled-row form of E4M3 prefill returns the full form's values."""
    c = _fp8_prefill_case(47, cached=[5, 2], chunk=[3, 6])
    full = _prefill_fp8_of(c)
    rng = _rng(48)
    picks = [(int(r), int(h)) for r, h in zip(rng.integers(0, 9, 12), rng.integers(0, c["Hq"], 12))]
    sub = _prefill_fp8_of(c, rows=picks)
    assert np.stack([full[r, h] for r, h in picks]).tobytes() == sub.tobytes()


ALL_PINS = [
    pin_store_bytes, pin_gather_inverts_layout, pin_decode_vs_sdpa, pin_decode_closed_forms,
    pin_decode_block_permutation, pin_decode_sharing_equals_duplication,
    pin_gqa_equals_expanded_mha, pin_partition_invariance, pin_merge_of_disjoint_states,
    pin_bf16_widening, pin_prefill_row_is_decode, pin_prefill_c0_is_causal_sdpa,
    pin_prefill_chunk_split, pin_prefill_rows_subset, pin_hash_vectors,
    pin_hash_polynomial_and_chaining, pin_allocator_sharing_small, pin_cached_tokens,
    pin_append_equals_allocate, pin_append_fills_are_shareable,
    pin_e4m3_closed_forms, pin_e4m3_table_vs_torch, pin_e4m3_quantize_vs_torch,
    pin_e4m3_round_trip_and_ties, pin_e4m3_saturation_and_specials, pin_e4m3_scale_divides,
    pin_fp8_store_layout, pin_fp8_decode_vs_sdpa, pin_fp8_prefill_vs_sdpa,
    pin_fp8_prefill_row_is_decode, pin_fp8_prefill_rows_subset,
]
