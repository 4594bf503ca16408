// Host-side KV block manager: physical blocks of a fixed pool, handed out to
// sequences through block tables, shared between sequences whose prompts
// start with the same full blocks.
//
// What it implements:
//   * the Block of the nano-vllm page ("nano vllm：轻量级大模型推理框架的KV
//     Cache优化实践", §3.2.1): a physical id, a reference count, a content
//     hash whose "none" value is -1, and the block's token ids. A prompt
//     block that matches an existing block takes one more reference, a
//     finished sequence drops one, and a block left with none is reclaimed;
//   * the allocation loop of §3.2.2: for every block of a prompt, hash it;
//     on a hit reuse the block, otherwise take a free block with one
//     reference and record its hash;
//   * the rolling hash of §4.2: h <- (31 h + t) mod 2^32 over the block's
//     tokens, starting from the hash of the block before it (0 for a
//     sequence's first block);
//   * the BlockAllocator of the mini-vllm page ("mini-vllm：基于 NanoGPT 的
//     PagedAttention 风格 KV 缓存管理实现", architecture item 1), which serves
//     the prefill and the decode phase and frees a request's blocks when it
//     completes, here as a C++ allocator (the page's planned rewrite).
// Where the pages are silent: only full blocks are hashed and shared (a
// partial block stays private); a hit counts only if the block's stored
// tokens and its parent (the block before it in the owning table) match,
// otherwise the hash is re-pointed to the new block; new blocks come from
// the front of the free list and reclaimed ones go to its back; a block
// that a decode append fills is hashed and recorded like a prompt block.
//
// Not thread-safe: one manager per scheduling thread.

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pagedattn.h"

namespace {

constexpr int64_t NO_HASH = -1;

uint32_t fold_hash(const int32_t* tokens, int32_t n, uint32_t h) {
  for (int32_t i = 0; i < n; ++i) h = h * 31u + static_cast<uint32_t>(tokens[i]);
  return h;
}

struct Block {
  int32_t ref = 0;
  int32_t parent = -1;   // block before this one in the owning table, -1 for none
  int32_t ntok = 0;      // tokens stored (block_size when full)
  int64_t hash = NO_HASH;
};

}  // namespace

struct pa_block_manager {
  int32_t block_size;
  std::vector<Block> blocks;
  std::vector<int32_t> tokens;        // block b's tokens at [b*block_size, b*block_size + ntok)
  std::deque<int32_t> free_list;
  std::unordered_map<uint32_t, int32_t> by_hash;

  const int32_t* toks(int32_t b) const { return tokens.data() + (int64_t)b * block_size; }
  int32_t* toks(int32_t b) { return tokens.data() + (int64_t)b * block_size; }

  void reset_block(int32_t b) {
    blocks[b] = Block{};
  }
};

namespace {

thread_local char g_bm_error[256] = "";

pa_status bm_fail(pa_status st, const char* msg) {
  std::strncpy(g_bm_error, msg, sizeof(g_bm_error) - 1);
  g_bm_error[sizeof(g_bm_error) - 1] = '\0';
  return st;
}

}  // namespace

extern "C" {

const char* pa_bm_last_error(void) { return g_bm_error; }

pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_block_manager** out) {
  try {
    if (!out) return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_create: out is null");
    *out = nullptr;
    if (num_blocks <= 0 || block_size <= 0)
      return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_create: num_blocks and block_size must be positive");
    if ((int64_t)num_blocks * block_size > INT32_MAX)
      return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_create: num_blocks*block_size exceeds int32 slots");
    std::vector<char> seen(num_blocks, 0);
    if (free_order) {
      for (int32_t i = 0; i < num_blocks; ++i) {
        const int32_t b = free_order[i];
        if (b < 0 || b >= num_blocks || seen[b])
          return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_create: free_order is not a permutation of the blocks");
        seen[b] = 1;
      }
    }
    auto* bm = new pa_block_manager();
    bm->block_size = block_size;
    bm->blocks.assign(num_blocks, Block{});
    bm->tokens.assign((size_t)num_blocks * block_size, 0);
    for (int32_t i = 0; i < num_blocks; ++i) bm->free_list.push_back(free_order ? free_order[i] : i);
    bm->by_hash.reserve((size_t)num_blocks * 2);
    *out = bm;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_create: out of host memory");
  } catch (...) {
    return bm_fail(PA_ERR_HIP, "pa_bm_create: unexpected C++ exception");
  }
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_num_free(const pa_block_manager* bm) { return bm ? (int32_t)bm->free_list.size() : -1; }

int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block_id) {
  if (!bm || block_id < 0 || block_id >= (int32_t)bm->blocks.size()) return -1;
  return bm->blocks[block_id].ref;
}

int32_t pa_bm_shared_tokens(const pa_block_manager* bm, const int32_t* table, int32_t num_table_blocks,
                            int32_t num_tokens) {
  if (!bm || num_table_blocks < 0 || num_tokens < 0 || (num_table_blocks > 0 && !table)) return -1;
  const int64_t bs = bm->block_size;
  int64_t k = 0;
  while (k < num_table_blocks && k * bs < num_tokens) {
    const int32_t b = table[k];
    if (b < 0 || b >= (int32_t)bm->blocks.size()) return -1;
    if (bm->blocks[b].ref <= 1) break;
    ++k;
  }
  return (int32_t)std::min<int64_t>(k * bs, num_tokens);
}

pa_status pa_bm_allocate(pa_block_manager* bm, const int32_t* token_ids, int32_t num_tokens,
                         int32_t* table, int32_t table_capacity, int32_t* num_table_blocks,
                         int32_t* num_cached_tokens, int32_t* slots) {
  try {
    if (!bm || !table || !num_table_blocks || !num_cached_tokens || (num_tokens > 0 && !token_ids))
      return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_allocate: null argument");
    if (num_tokens < 0) return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_allocate: negative num_tokens");
    const int32_t bs = bm->block_size;
    const int32_t nb = (int32_t)(((int64_t)num_tokens + bs - 1) / bs);
    if (nb > table_capacity)
      return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_allocate: table_capacity below the blocks needed");

    // undo log, so that running out of free blocks leaves no trace
    struct MapUndo {
      uint32_t h;
      bool had;
      int32_t prev;
    };
    std::vector<int32_t> hits, taken;
    std::vector<MapUndo> map_undo;
    auto rollback = [&]() {
      for (auto it = map_undo.rbegin(); it != map_undo.rend(); ++it) {
        if (it->had) bm->by_hash[it->h] = it->prev;
        else bm->by_hash.erase(it->h);
      }
      for (int32_t b : hits) --bm->blocks[b].ref;
      for (auto it = taken.rbegin(); it != taken.rend(); ++it) {
        bm->reset_block(*it);
        bm->free_list.push_front(*it);
      }
    };

    uint32_t h = 0;
    int32_t parent = -1;
    int32_t cached = 0;
    for (int32_t k = 0; k < nb; ++k) {
      const int32_t start = k * bs;
      const int32_t n = std::min(bs, num_tokens - start);
      const int32_t* chunk = token_ids + start;
      int32_t b = -1;
      if (n == bs) {
        h = fold_hash(chunk, n, h);
        auto it = bm->by_hash.find(h);
        if (it != bm->by_hash.end()) {
          const int32_t c = it->second;
          const Block& blk = bm->blocks[c];
          if (blk.ntok == bs && blk.parent == parent &&
              std::memcmp(bm->toks(c), chunk, sizeof(int32_t) * bs) == 0) {
            ++bm->blocks[c].ref;
            hits.push_back(c);
            if (cached == start) cached += bs;
            table[k] = c;
            parent = c;
            continue;
          }
        }
      }
      if (bm->free_list.empty()) {
        rollback();
        return bm_fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_allocate: not enough free blocks");
      }
      b = bm->free_list.front();
      bm->free_list.pop_front();
      taken.push_back(b);
      Block& blk = bm->blocks[b];
      blk.ref = 1;
      blk.parent = parent;
      blk.ntok = n;
      std::memcpy(bm->toks(b), chunk, sizeof(int32_t) * n);
      if (n == bs) {
        blk.hash = h;
        auto it = bm->by_hash.find(h);
        map_undo.push_back(MapUndo{h, it != bm->by_hash.end(), it != bm->by_hash.end() ? it->second : -1});
        bm->by_hash[h] = b;
      } else {
        blk.hash = NO_HASH;
      }
      table[k] = b;
      parent = b;
    }
    *num_table_blocks = nb;
    *num_cached_tokens = cached;
    if (slots)
      for (int32_t j = 0; j < num_tokens; ++j) slots[j] = table[j / bs] * bs + j % bs;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_allocate: out of host memory");
  } catch (...) {
    return bm_fail(PA_ERR_HIP, "pa_bm_allocate: unexpected C++ exception");
  }
}

pa_status pa_bm_append(pa_block_manager* bm, int32_t* table, int32_t* num_table_blocks,
                       int32_t table_capacity, int32_t num_tokens, int32_t token_id, int32_t* slot) {
  try {
    if (!bm || !table || !num_table_blocks || !slot)
      return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_append: null argument");
    const int32_t bs = bm->block_size;
    const int32_t nb = *num_table_blocks;
    if (num_tokens < 0 || nb != (int32_t)(((int64_t)num_tokens + bs - 1) / bs))
      return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_append: num_tokens does not match the table");
    const int32_t row = num_tokens % bs;
    if (row != 0) {
      const int32_t last = table[nb - 1];
      if (last < 0 || last >= (int32_t)bm->blocks.size() || bm->blocks[last].ntok != row ||
          bm->blocks[last].ref != 1)
        return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_append: the last block is not this sequence's partial block");
    } else {
      if (nb + 1 > table_capacity) return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_append: table is full");
      if (bm->free_list.empty()) return bm_fail(PA_ERR_OUT_OF_BLOCKS, "pa_bm_append: no free block");
      const int32_t b = bm->free_list.front();
      bm->free_list.pop_front();
      Block& blk = bm->blocks[b];
      blk.ref = 1;
      blk.hash = NO_HASH;
      blk.ntok = 0;
      blk.parent = nb > 0 ? table[nb - 1] : -1;
      table[nb] = b;
      *num_table_blocks = nb + 1;
    }
    const int32_t b = table[num_tokens / bs];
    Block& blk = bm->blocks[b];
    bm->toks(b)[blk.ntok++] = token_id;
    if (blk.ntok == bs) {
      const uint32_t prev = blk.parent >= 0 ? (uint32_t)bm->blocks[blk.parent].hash : 0u;
      const uint32_t h = fold_hash(bm->toks(b), bs, prev);
      blk.hash = h;
      bm->by_hash[h] = b;
    }
    *slot = b * bs + row;
    return PA_OK;
  } catch (const std::bad_alloc&) {
    return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_append: out of host memory");
  } catch (...) {
    return bm_fail(PA_ERR_HIP, "pa_bm_append: unexpected C++ exception");
  }
}

pa_status pa_bm_free(pa_block_manager* bm, const int32_t* table, int32_t num_table_blocks) {
  try {
    if (!bm || (num_table_blocks > 0 && !table)) return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_free: null argument");
    if (num_table_blocks < 0) return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_free: negative num_table_blocks");
    // check first, so that a bad table changes nothing
    std::unordered_map<int32_t, int32_t> uses;
    for (int32_t k = 0; k < num_table_blocks; ++k) {
      const int32_t b = table[k];
      if (b < 0 || b >= (int32_t)bm->blocks.size())
        return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_free: block id outside the pool");
      if (++uses[b] > bm->blocks[b].ref)
        return bm_fail(PA_ERR_INVALID_ARG, "pa_bm_free: a block freed more often than referenced");
    }
    for (int32_t k = num_table_blocks - 1; k >= 0; --k) {
      const int32_t b = table[k];
      Block& blk = bm->blocks[b];
      if (--blk.ref == 0) {
        if (blk.hash != NO_HASH) {
          auto it = bm->by_hash.find((uint32_t)blk.hash);
          if (it != bm->by_hash.end() && it->second == b) bm->by_hash.erase(it);
        }
        bm->reset_block(b);
        bm->free_list.push_back(b);
      }
    }
    return PA_OK;
  } catch (...) {
    return bm_fail(PA_ERR_HIP, "pa_bm_free: unexpected C++ exception");
  }
}

}  // extern "C"
