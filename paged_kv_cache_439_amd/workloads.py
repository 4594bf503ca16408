"""Seeded synthetic inputs for paged-KV attention.

This module only draws inputs; it holds none of the attention arithmetic and
none of the prefix-hash arithmetic, and it serves both the library's tests and
benchmark and the CPU oracle's checks.

Structure (context lengths, token ids, block tables, slot mapping) is drawn
with numpy's PCG64 from seed ``439000 + workload id`` in this order:

  1. for prefix-sharing workloads, the subset of sequences that share;
  2. context lengths (decode) or cached lengths (prefill);
  3. token ids, uniform in [0, 50257) (the GPT-2 vocabulary the NanoGPT model
     of the mini-vllm page uses), with one common prefix for sharers;
  4. a random permutation of the pool's block ids, used as the free list;
     sequences take blocks from its front in order, and a sharing sequence
     reuses the blocks of the common prefix that the first sharer took.

Dense values (pool K/V, the new K/V rows, Q) are N(0, 1) float32 from a
seeded torch generator on the target device, rounded to nearest-even when the
workload is bf16. Drawing them on the device keeps multi-GB pools fast to
build; the oracle receives host copies of exactly these values.

Block-table entries past a sequence's last block are -1.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

VOCAB = 50257
SEED_BASE = 439000

# The workloads, by name; each integer is the workload's seed id (structure is
# drawn from PCG64(SEED_BASE + id)). Lengths include the newest token.
# partition_size is the decode split the benchmark times (-1: the library's
# balanced split); fixed_partition_size is the fixed-slice split measured
# beside it (0: whole contexts), the 512-token slices the b512 workload names
# among them.
TINY_FP32_DECODE = 1           # 4 sequences, fp32 MHA 8 heads, D 64, block 16
B64_MHA_DECODE = 2             # 64 sequences, bf16 MHA 12 heads, D 64, block 256, lengths U[512, 4096]
B256_SHARED_PREFIX_DECODE = 3  # 256 sequences, bf16 GQA 16/8, D 128, block 256; 128 share a 1024-token prefix
CHUNKED_PREFILL = 4            # 8 chunks of 512 over cached U[0, 3584], bf16 GQA 32/8, D 128, block 256
B512_LOGNORMAL_DECODE = 5      # 512 sequences, bf16 GQA 32/8, D 128, block 64, lognormal lengths (median 1500)
MIXED_BATCH = 6                # 256 decode tokens and 4 chunks of 512, bf16 GQA 32/8, D 128, block 256
DECODE_WORKLOADS = (B64_MHA_DECODE, B256_SHARED_PREFIX_DECODE, B512_LOGNORMAL_DECODE)

WORKLOADS = {
    1: dict(name="tiny_fp32_mha_decode", kind="decode", dtype="f32", num_seqs=4,
            num_heads=8, num_kv_heads=8, head_dim=64, block_size=16,
            lens=("fixed", [17, 33, 64, 100]), pool=("blocks", 64),
            max_context=100, partition_size=0),
    2: dict(name="bf16_mha_decode_b64", kind="decode", dtype="bf16", num_seqs=64,
            num_heads=12, num_kv_heads=12, head_dim=64, block_size=256,
            lens=("uniform", 512, 4096), pool=("factor", 1.25),
            max_context=4096, partition_size=-1, fixed_partition_size=256),
    3: dict(name="bf16_gqa_decode_b256_shared_prefix", kind="decode", dtype="bf16",
            num_seqs=256, num_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
            lens=("uniform", 1024, 4096), pool=("factor", 1.25),
            share=dict(num_sharers=128, prefix_tokens=1024),
            max_context=4096, partition_size=-1, fixed_partition_size=0),
    4: dict(name="bf16_gqa_chunked_prefill", kind="prefill", dtype="bf16", num_seqs=8,
            num_heads=32, num_kv_heads=8, head_dim=128, block_size=256,
            cached=("uniform", 0, 3584), chunk=512, pool=("factor", 1.25),
            max_context=4096),
    5: dict(name="bf16_gqa_decode_b512_lognormal", kind="decode", dtype="bf16",
            num_seqs=512, num_heads=32, num_kv_heads=8, head_dim=128, block_size=64,
            lens=("lognormal", 1500.0, 1.0, 64, 4096), pool=("factor", 1.25),
            max_context=4096, partition_size=-1, fixed_partition_size=512),
    # A continuous batch (pa_mixed_batch): 256 decode tokens (contexts uniform
    # in [512, 4096]) followed by 4 prefill chunks of 512 new tokens over
    # cached contexts uniform in [0, 3584], on the GQA 32/8 model of the
    # prefill workload.
    6: dict(name="bf16_gqa_mixed_decode256_prefill4x512", kind="mixed", dtype="bf16", num_seqs=260,
            num_decode=256, num_heads=32, num_kv_heads=8, head_dim=128, block_size=256,
            decode_lens=("uniform", 512, 4096), cached=("uniform", 0, 3584), chunk=512,
            pool=("factor", 1.25), max_context=4096),
}


def torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def elem_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


@dataclass
class Batch:
    """One batch of paged-attention inputs."""
    spec: dict
    kind: str                      # "decode" | "prefill" | "mixed" (decode rows, then chunks)
    dtype: str                     # "f32" | "bf16"
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    context_lens: np.ndarray       # int32 [B]
    block_tables: np.ndarray       # int32 [B][max_blocks_per_seq]
    slot_mapping: np.ndarray       # int32 [T]
    token_ids: list
    query_start_loc: np.ndarray | None = None   # prefill: int32 [B+1]
    shared_blocks: list = field(default_factory=list)
    k_cache: torch.Tensor | None = None   # [NB][bs][Hkv][D]
    v_cache: torch.Tensor | None = None
    key: torch.Tensor | None = None       # new rows [T][Hkv][D]
    value: torch.Tensor | None = None
    q: torch.Tensor | None = None         # [T_q][Hq][D]
    device: str = "cpu"
    k_scale: torch.Tensor | None = None   # E4M3 pools: float32 [Hkv] per-head scales
    v_scale: torch.Tensor | None = None

    @property
    def kv_e4m3(self) -> bool:
        return self.k_scale is not None

    @property
    def num_decode(self) -> int:
        """Leading sequences that are decode tokens, one row each (mixed batches)."""
        return int(self.spec.get("num_decode", 0)) if self.kind == "mixed" else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0

    @property
    def shared_lens(self) -> np.ndarray:
        """int32 [B]: leading context tokens of each sequence that lie in the
        shared prefix blocks (the decode calls' load-policy hint); 0 for a
        sequence that shares nothing."""
        shared = set(int(b) for b in self.shared_blocks)
        out = np.zeros(self.num_seqs, dtype=np.int32)
        bs = self.block_size
        for i, L in enumerate(self.context_lens.tolist()):
            k = 0
            while k * bs < L and int(self.block_tables[i, k]) in shared:
                k += 1
            out[i] = min(k * bs, L)
        return out

    @property
    def max_query_len(self) -> int:
        if self.query_start_loc is None:
            return 1
        return int(np.diff(self.query_start_loc).max())

    @property
    def logical_blocks(self) -> int:
        return int(sum(math.ceil(int(L) / self.block_size) for L in self.context_lens))

    @property
    def unique_blocks(self) -> int:
        used = set()
        for i, L in enumerate(self.context_lens):
            used.update(self.block_tables[i, :math.ceil(int(L) / self.block_size)].tolist())
        return len(used)

    def kv_bytes(self, unique: bool = True) -> int:
        """K+V bytes a decode pass must read: one row per distinct
        (physical block, row) that some context covers when unique (a block
        shared by several sequences counts once), else one per
        (sequence, token)."""
        row = self.num_kv_heads * self.head_dim * (1 if self.kv_e4m3 else elem_bytes(self.dtype)) * 2
        if not unique:
            return int(self.context_lens.astype(np.int64).sum()) * row
        return int(covered_rows(self).sum()) * row


# ---------------------------------------------------------------------------
# structure
# ---------------------------------------------------------------------------

def _draw_lengths(rng, spec, n, lo_override=None):
    kind = spec[0]
    if kind == "fixed":
        return np.asarray(spec[1], dtype=np.int64)
    if kind == "uniform":
        lo, hi = spec[1], spec[2]
        if lo_override is not None:
            lo = np.maximum(lo, lo_override)
        return rng.integers(lo, hi + 1, size=n, dtype=np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = spec[1:5]
        z = rng.standard_normal(n)
        return np.clip(np.rint(median * np.exp(sigma * z)), lo, hi).astype(np.int64)
    raise ValueError(spec)


def _allocate(rng, lens, bs, pool_spec, sharers, prefix_blocks, max_blocks):
    """Tables from a shuffled free list; sharers reuse the prefix blocks."""
    need_logical = [math.ceil(int(L) / bs) for L in lens]
    n_shared_users = sum(1 for i in range(len(lens)) if sharers[i])
    need_unique = sum(need_logical) - max(0, n_shared_users - 1) * prefix_blocks
    if pool_spec[0] == "blocks":
        num_blocks = int(pool_spec[1])
    else:
        num_blocks = int(math.ceil(pool_spec[1] * need_unique))
    if num_blocks < need_unique:
        raise ValueError("pool too small for the drawn lengths")
    free = rng.permutation(num_blocks).astype(np.int64)
    free_list = free.copy()
    pos = 0
    tables = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    shared_ids = [None] * prefix_blocks
    for i, nb in enumerate(need_logical):
        for k in range(nb):
            if sharers[i] and k < prefix_blocks:
                if shared_ids[k] is None:
                    shared_ids[k] = int(free[pos])
                    pos += 1
                tables[i, k] = shared_ids[k]
            else:
                tables[i, k] = int(free[pos])
                pos += 1
    return num_blocks, tables, [b for b in shared_ids if b is not None], free_list


def draw_structure(spec, seed=None):
    """Structure only (no dense values): a dict with context_lens, chunks
    (prefill), token_ids, num_blocks, block_tables, shared_blocks and the
    free list the tables were taken from."""
    if seed is None:
        seed = SEED_BASE + int(spec.get("id", 0))
    lens, chunks, token_ids, num_blocks, tables, shared, free = _structure(spec, seed)
    return dict(context_lens=lens, chunks=chunks, token_ids=token_ids, num_blocks=num_blocks,
                block_tables=tables, shared_blocks=shared, free_list=free)


def _structure(spec, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    B = spec["num_seqs"]
    bs = spec["block_size"]
    share = spec.get("share")
    sharers = np.zeros(B, dtype=bool)
    prefix_tokens = 0
    if share:
        sharers[rng.choice(B, size=share["num_sharers"], replace=False)] = True
        prefix_tokens = share["prefix_tokens"]
        if prefix_tokens % bs:
            raise ValueError("shared prefix must be whole blocks")
    if spec["kind"] == "decode":
        lens = _draw_lengths(rng, spec["lens"], B)
        if share:
            # a sharer's newest token must land past the shared blocks, so
            # that storing it never writes into a block other tables use
            lo = prefix_tokens + 1
            redo = sharers & (lens < lo)
            while redo.any():
                lens[redo] = _draw_lengths(rng, spec["lens"], int(redo.sum()), lo_override=lo)
                redo = sharers & (lens < lo)
        chunks = None
    elif spec["kind"] == "mixed":
        # decode tokens first (one new row each), then the prefill chunks
        Bd = spec["num_decode"]
        lens_d = _draw_lengths(rng, spec["decode_lens"], Bd)
        cached = _draw_lengths(rng, spec["cached"], B - Bd)
        chunk = spec["chunk"]
        tail = (np.full(B - Bd, chunk, dtype=np.int64) if np.isscalar(chunk)
                else np.asarray(chunk, np.int64))
        chunks = np.concatenate([np.ones(Bd, dtype=np.int64), tail])
        lens = np.concatenate([lens_d, cached + tail])
    else:
        cached = _draw_lengths(rng, spec["cached"], B)
        chunk = spec["chunk"]
        chunks = np.full(B, chunk, dtype=np.int64) if np.isscalar(chunk) else np.asarray(chunk, np.int64)
        lens = cached + chunks
    common = rng.integers(0, VOCAB, size=prefix_tokens, dtype=np.int64)
    token_ids = []
    for i in range(B):
        ids = rng.integers(0, VOCAB, size=int(lens[i]), dtype=np.int64)
        if sharers[i]:
            ids[:prefix_tokens] = common
        token_ids.append(ids)
    max_blocks = math.ceil(spec["max_context"] / bs)
    if int(lens.max()) > spec["max_context"]:
        raise ValueError("a drawn length exceeds max_context")
    num_blocks, tables, shared, free = _allocate(rng, lens, bs, spec["pool"], sharers,
                                                 prefix_tokens // bs, max_blocks)
    return lens.astype(np.int32), chunks, token_ids, num_blocks, tables, shared, free


def _slot(tables, i, pos, bs):
    return int(tables[i, pos // bs]) * bs + pos % bs


# ---------------------------------------------------------------------------
# dense values
# ---------------------------------------------------------------------------

def _randn(shape, dtype, device, seed, chunk_rows=None):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    td = torch_dtype(dtype)
    out = torch.empty(shape, dtype=td, device=device)
    rows = shape[0]
    step = chunk_rows or rows or 1
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                                 device=device, dtype=torch.float32).to(td)
    return out


# E4M3 pools (spec["kv"] == "e4m3"): pool entries are drawn as values
# N(0, 1) * E4M3_AMP, clamped to the format's +-448 and converted by torch's
# own float8_e4m3fn cast; they are read with per-KV-head scales
# E4M3_SCALE_BASE * u, u ~ U[0.75, 1.25) (seeded), so that the dequantised
# pools follow about the same N(0, 1) as the bf16 workloads.
E4M3_AMP = 112.0
E4M3_SCALE_BASE = 1.0 / 112.0


def _randn_e4m3(shape, device, seed, chunk_rows=None):
    """uint8 E4M3 codes of seeded N(0, 1) * E4M3_AMP values."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    rows = shape[0]
    step = chunk_rows or rows or 1
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                        dtype=torch.float32) * E4M3_AMP
        out[r0:r1] = x.clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def e4m3_scales(num_kv_heads, seed, device):
    """Seeded per-KV-head (k_scale, v_scale) float32 tensors."""
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    k = (E4M3_SCALE_BASE * rng.uniform(0.75, 1.25, num_kv_heads)).astype(np.float32)
    v = (E4M3_SCALE_BASE * rng.uniform(0.75, 1.25, num_kv_heads)).astype(np.float32)
    return torch.from_numpy(k).to(device), torch.from_numpy(v).to(device)


def make_batch(spec, device="cpu", seed=None, poison=False):
    """Draw a full batch for ``spec`` (an entry of WORKLOADS or a variant).

    poison=True fills every pool row that no context covers, and the rows the
    new tokens are about to be stored into, with NaN; a kernel that reads
    outside the context then shows NaN in its output.
    """
    if seed is None:
        seed = SEED_BASE + int(spec.get("id", 0))
    lens, chunks, token_ids, num_blocks, tables, shared, _ = _structure(spec, seed)
    B = spec["num_seqs"]
    Hq, Hkv, D, bs = spec["num_heads"], spec["num_kv_heads"], spec["head_dim"], spec["block_size"]
    if spec["kind"] == "decode":
        slots = np.array([_slot(tables, i, int(lens[i]) - 1, bs) for i in range(B)], dtype=np.int32)
        qsl = None
        n_new = B
        n_q = B
    else:
        slots = []
        for i in range(B):
            c = int(lens[i] - chunks[i])
            slots.extend(_slot(tables, i, p, bs) for p in range(c, int(lens[i])))
        slots = np.asarray(slots, dtype=np.int32)
        qsl = np.zeros(B + 1, dtype=np.int32)
        qsl[1:] = np.cumsum(chunks)
        n_new = int(qsl[-1])
        n_q = n_new
    dtype = spec["dtype"]
    base = int(seed) * 16
    row_elems = bs * Hkv * D
    chunk_rows = max(1, (1 << 26) // row_elems)    # ~64M elements per draw
    e4m3 = spec.get("kv") == "e4m3"
    if e4m3:
        k_cache = _randn_e4m3((num_blocks, bs, Hkv, D), device, base + 1, chunk_rows)
        v_cache = _randn_e4m3((num_blocks, bs, Hkv, D), device, base + 2, chunk_rows)
        k_scale, v_scale = e4m3_scales(Hkv, base + 6, device)
    else:
        k_cache = _randn((num_blocks, bs, Hkv, D), dtype, device, base + 1, chunk_rows)
        v_cache = _randn((num_blocks, bs, Hkv, D), dtype, device, base + 2, chunk_rows)
        k_scale = v_scale = None
    key = _randn((n_new, Hkv, D), dtype, device, base + 3)
    value = _randn((n_new, Hkv, D), dtype, device, base + 4)
    q = _randn((n_q, Hq, D), dtype, device, base + 5)
    batch = Batch(spec=spec, kind=spec["kind"], dtype=dtype, num_seqs=B, num_heads=Hq,
                  num_kv_heads=Hkv, head_dim=D, block_size=bs, num_blocks=num_blocks,
                  scale=float(spec.get("scale", 1.0 / math.sqrt(D))), context_lens=lens, block_tables=tables,
                  slot_mapping=slots, token_ids=token_ids, query_start_loc=qsl,
                  shared_blocks=shared, k_cache=k_cache, v_cache=v_cache, key=key,
                  value=value, q=q, device=str(device), k_scale=k_scale, v_scale=v_scale)
    if poison:
        poison_unused_rows(batch)
    return batch


def covered_rows(batch):
    """Boolean [num_blocks][block_size]: rows some context covers."""
    bs = batch.block_size
    mask = np.zeros((batch.num_blocks, bs), dtype=bool)
    for i, L in enumerate(batch.context_lens):
        j = np.arange(int(L))
        mask[batch.block_tables[i, j // bs], j % bs] = True
    return mask


def poison_unused_rows(batch):
    mask = covered_rows(batch)
    bs = batch.block_size
    for s in batch.slot_mapping.tolist():
        if s >= 0:
            mask[s // bs, s % bs] = False
    dead = torch.from_numpy(~mask).to(batch.k_cache.device)
    fill = 0x7F if batch.kv_e4m3 else float("nan")   # 0x7F: the E4M3 NaN code
    batch.k_cache[dead] = fill
    batch.v_cache[dead] = fill


# ---------------------------------------------------------------------------
# host copies for the oracle
# ---------------------------------------------------------------------------

def to_numpy(t: torch.Tensor):
    """Host copy; bf16 tensors come back as uint16 bit patterns."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


@dataclass
class HostBatch:
    """Host (numpy) copy of the inputs of a subset of sequences."""
    dtype: str
    block_size: int
    scale: float
    seqs: list
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    slot_mapping: np.ndarray
    key: np.ndarray
    value: np.ndarray
    q: np.ndarray
    query_start_loc: np.ndarray | None
    new_rows: list            # index of each sequence's new rows in the full batch


def host_subset(batch: Batch, seqs=None):
    """Copy the inputs the given sequences depend on to the host.

    Only the blocks those sequences reference are copied; they are renumbered
    0..n-1 in order of first use, and the tables and slots are rewritten to
    match. A renumbering of physical blocks does not change any result.
    """
    if seqs is None:
        seqs = list(range(batch.num_seqs))
    seqs = [int(s) for s in seqs]
    bs = batch.block_size
    remap = {}
    for i in seqs:
        nb = math.ceil(int(batch.context_lens[i]) / bs)
        for b in batch.block_tables[i, :nb].tolist():
            if b not in remap:
                remap[b] = len(remap)
    order = torch.tensor(list(remap.keys()), dtype=torch.long, device=batch.k_cache.device)
    k = to_numpy(batch.k_cache.index_select(0, order)) if len(remap) else None
    v = to_numpy(batch.v_cache.index_select(0, order)) if len(remap) else None
    tables = np.full((len(seqs), batch.max_blocks_per_seq), -1, dtype=np.int32)
    for r, i in enumerate(seqs):
        nb = math.ceil(int(batch.context_lens[i]) / bs)
        tables[r, :nb] = [remap[b] for b in batch.block_tables[i, :nb].tolist()]
    lens = batch.context_lens[seqs].copy()
    key_all, value_all, q_all = to_numpy(batch.key), to_numpy(batch.value), to_numpy(batch.q)
    if batch.kind == "decode":
        rows = [[i] for i in seqs]
        qsl = None
        q_rows = seqs
    else:
        qsl_full = batch.query_start_loc
        rows = [list(range(int(qsl_full[i]), int(qsl_full[i + 1]))) for i in seqs]
        qsl = np.zeros(len(seqs) + 1, dtype=np.int32)
        qsl[1:] = np.cumsum([len(r) for r in rows])
        q_rows = [t for r in rows for t in r]
    flat = [t for r in rows for t in r]
    slots = []
    for r, i in enumerate(seqs):
        for t in rows[r]:
            s = int(batch.slot_mapping[t])
            slots.append(remap[s // bs] * bs + s % bs if s >= 0 else -1)
    return HostBatch(dtype=batch.dtype, block_size=bs, scale=batch.scale, seqs=seqs,
                     k_cache=k, v_cache=v, block_tables=tables, context_lens=lens,
                     slot_mapping=np.asarray(slots, dtype=np.int32),
                     key=key_all[flat], value=value_all[flat], q=q_all[q_rows],
                     query_start_loc=qsl, new_rows=rows)


def spec(workload, **overrides):
    """A copy of WORKLOADS[workload] with overrides, tagged with its id."""
    s = dict(WORKLOADS[workload])
    s["id"] = workload
    s.update(overrides)
    return s
