"""Rolling prefix hash and hash-sharing block allocation (CPU oracle).

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the
benchmark's CPU-baseline leg; never by the library.

Follows the nano-vllm page ("nano vllm：轻量级大模型推理框架的KV Cache优化实践"):
  * §4.2 (前缀共享实现): the hash folds each token id t into the running
    value as h <- (31*h + t) mod 2**32, starting from the prefix's hash.
  * §3.2.1 (Block设计): a block carries its physical id, a reference count
    starting at 0, a hash whose "none" value is -1, and its token ids; a
    match adds one reference, a finished request drops one, and a block
    whose count reaches zero is reclaimed.
  * §3.2.2 (BlockManager核心逻辑): for each block of a request, hash it; on a
    hit reuse the block and add a reference, otherwise take a new block with
    one reference and record its hash.

Readings where the page is silent:
  * the first block of a sequence chains from prefix hash 0;
  * only full blocks are hashed and shared; a partial last block keeps
    hash -1 and is always private;
  * a hash hit is accepted only if the stored token ids and the parent
    block (the block before it in the table) also match; otherwise it is
    treated as a miss and the hash is re-pointed to the new block;
  * new blocks are taken from the front of the free list given to the
    allocator, and reclaimed blocks go to its back;
  * the number of cached tokens of a new sequence (the Sequence field
    num_cached_tokens, §3.1) is block_size times the number of leading
    blocks that were hits;
  * decode (the mini-vllm page's BlockAllocator serves the prefill and the
    decode phase, architecture item 1) appends one token at a time: a new
    block is taken when the last one is full, and a block that the append
    fills is hashed, chained from the block before it, and its hash is
    recorded as for a miss, so that later requests can share it.
"""

from __future__ import annotations

from collections import deque

MASK32 = 0xFFFFFFFF
NO_HASH = -1


def compute_hash(token_ids, prefix_hash):
    """Fold token ids into prefix_hash with h <- (h*31 + t) & 0xFFFFFFFF."""
    h = int(prefix_hash)
    for t in token_ids:
        h = (h * 31 + int(t)) & MASK32
    return h


class Block:
    """One physical KV block (nano-vllm page §3.2.1)."""

    def __init__(self, block_id):
        self.block_id = block_id
        self.ref_count = 0
        self.hash = NO_HASH
        self.token_ids = []
        self.parent = -1          # block before this one in the owning table

    def reset(self):
        self.ref_count = 0
        self.hash = NO_HASH
        self.token_ids = []
        self.parent = -1


class PrefixBlockAllocator:
    """Hash-sharing allocator over a fixed pool of physical blocks."""

    def __init__(self, free_ids, block_size):
        self.block_size = int(block_size)
        self.blocks = {int(b): Block(int(b)) for b in free_ids}
        self.free = deque(int(b) for b in free_ids)
        self.hash_to_block_id = {}

    def _take_free(self):
        if not self.free:
            raise MemoryError("no free KV block")
        return self.blocks[self.free.popleft()]

    def allocate(self, token_ids):
        """Block table (list of physical ids) for a sequence's tokens."""
        return self.allocate_cached(token_ids)[0]

    def allocate_cached(self, token_ids):
        """(block table, number of leading tokens whose blocks were hits)."""
        bs = self.block_size
        table = []
        h = 0
        parent = -1
        cached = 0
        for start in range(0, len(token_ids), bs):
            chunk = [int(t) for t in token_ids[start:start + bs]]
            if len(chunk) == bs:
                h = compute_hash(chunk, h)
                hit = self.hash_to_block_id.get(h)
                if hit is not None:
                    blk = self.blocks[hit]
                    if blk.token_ids == chunk and blk.parent == parent:
                        blk.ref_count += 1
                        table.append(blk.block_id)
                        parent = blk.block_id
                        if cached == start:
                            cached += bs
                        continue
                blk = self._take_free()
                blk.ref_count = 1
                blk.hash = h
                blk.token_ids = chunk
                blk.parent = parent
                self.hash_to_block_id[h] = blk.block_id
            else:
                blk = self._take_free()
                blk.ref_count = 1
                blk.hash = NO_HASH
                blk.token_ids = chunk
                blk.parent = parent
            table.append(blk.block_id)
            parent = blk.block_id
        return table, cached

    def append_token(self, table, num_tokens, token_id):
        """Append token_id at position num_tokens of the sequence owning
        table (a list, extended in place when a new block is needed); returns
        the token's slot, block * block_size + row."""
        bs = self.block_size
        row = num_tokens % bs
        if row == 0:
            blk = self._take_free()
            blk.ref_count = 1
            blk.hash = NO_HASH
            blk.token_ids = []
            blk.parent = table[-1] if table else -1
            table.append(blk.block_id)
        blk = self.blocks[table[num_tokens // bs]]
        blk.token_ids.append(int(token_id))
        if len(blk.token_ids) == bs:
            prev = self.blocks[blk.parent].hash if blk.parent >= 0 else 0
            blk.hash = compute_hash(blk.token_ids, prev)
            self.hash_to_block_id[blk.hash] = blk.block_id
        return blk.block_id * bs + row

    def free_table(self, table):
        """Drop one reference from every block of a finished sequence;
        blocks left with none are reclaimed."""
        for bid in reversed(list(table)):
            blk = self.blocks[int(bid)]
            if blk.ref_count <= 0:
                raise ValueError(f"block {bid} freed more often than referenced")
            blk.ref_count -= 1
            if blk.ref_count == 0:
                if blk.hash != NO_HASH and self.hash_to_block_id.get(blk.hash) == blk.block_id:
                    del self.hash_to_block_id[blk.hash]
                blk.reset()
                self.free.append(blk.block_id)

    def ref_counts(self):
        return {b: blk.ref_count for b, blk in self.blocks.items() if blk.ref_count}
