/*
 * pagedattn.h -- C ABI of libpagedattn.so: attention over a block-paged KV
 * cache on AMD Instinct MI355X (gfx950).
 *
 * The operation. The mini-vllm page ("mini-vllm：基于 NanoGPT 的
 * PagedAttention 风格 KV 缓存管理实现", section "mini-vllm 的架构设计",
 * item 2 "KVCache") keeps every sequence's K/V rows in fixed-size physical
 * blocks of one preallocated device tensor and finds them, for reads and
 * writes alike, through a per-sequence block table; the nano-vllm page
 * ("nano vllm：轻量级大模型推理框架的KV Cache优化实践", §3.1 and §3.2) gives a
 * sequence its list of physical block ids and lets blocks be shared between
 * sequences through prefix hashing and reference counts. Attention through
 * the table equals ordinary scaled dot-product attention over the sequence's
 * rows in logical order:
 *
 *     out[h] = softmax(scale * K[g(h)] q[h]) V[g(h)],   g(h) = h / (Hq / Hkv)
 *
 * Layouts (all row-major, contiguous unless a stride is given):
 *   k_cache, v_cache   [num_blocks][block_size][num_kv_heads][head_dim]
 *   q, out             [tokens][num_heads][head_dim]
 *   key, value         [num_tokens][num_kv_heads][head_dim], token stride given
 *   block_tables       int32 [num_seqs][max_blocks_per_seq]; logical token j
 *                      of sequence i is row j % block_size of physical block
 *                      block_tables[i][j / block_size]
 *   context_lens       int32 [num_seqs]; number of context tokens, INCLUDING
 *                      the newest one (store it first, then attend)
 *   slot_mapping       int32 [num_tokens]; slot s = block * block_size + row
 *   query_start_loc    int32 [num_seqs + 1]; prefill rows of sequence i are
 *                      query_start_loc[i] .. query_start_loc[i+1]-1
 *
 * Element type: PA_F32 or PA_BF16 for every floating-point buffer of one
 * call; out has the type of q. Accumulation is always fp32.
 *
 * Ownership and streams. The caller owns every buffer (device pointers; the
 * library allocates no device memory in these calls). Each call enqueues its
 * kernels on the given hipStream_t (passed as void*, NULL = default stream)
 * and returns without synchronising; it never reads device memory on the
 * host, which is why the maxima (max_context_len, max_query_len) are
 * arguments.
 *
 * Errors. Arguments are checked on the host before anything is enqueued; a
 * bad argument returns a code and enqueues nothing. A failed launch returns
 * PA_ERR_HIP. No C++ exception crosses this interface. pa_last_error()
 * returns a description of the calling thread's last failure. A call with
 * num_seqs == 0 or num_tokens == 0 is a no-op returning PA_OK.
 *
 * Supported shapes: head_dim 64 or 128; block_size a power of two in
 * [8, 1024]; num_heads a multiple of num_kv_heads; pointers 16-byte aligned.
 *
 * Device-content preconditions (documented, not checked on the host; the
 * kernels clamp indices so a violation gives wrong numbers, not a fault):
 *   - 1 <= context_lens[i] <= max_context_len <= max_blocks_per_seq*block_size
 *   - block table entries used by a context lie in [0, num_blocks)
 *   - slots >= 0 are unique; a slot never lies in a block that another
 *     sequence's table also references (no store into a shared block)
 *   - prefill: 1 <= n_i <= max_query_len and n_i <= context_lens[i]
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, inconsistent sizes */
  PA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head_dim, block_size, alignment) */
  PA_ERR_WORKSPACE = 3,    /* split decode without a large enough workspace */
  PA_ERR_HIP = 4,          /* a HIP runtime call or launch failed */
  PA_ERR_OUT_OF_BLOCKS = 5 /* block manager: too few free blocks; nothing was changed */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* partition_size value of pa_decode that selects the balanced split. */
#define PA_PARTITION_BALANCED (-1)

/*
 * pa_store_kvcache -- scatter new K/V rows into the pools.
 *
 * For each token t with s = slot_mapping[t] in [0, num_blocks*block_size):
 *   k_cache[s / block_size][s % block_size][:][:] = key[t][:][:]
 *   v_cache[s / block_size][s % block_size][:][:] = value[t][:][:]
 * (mini-vllm page, item 2 "KVCache": the block table locates writes).
 * A negative slot is padding and writes nothing; a slot past the pool is
 * skipped too. The copy is bit-exact.
 *
 * key_tok_stride / value_tok_stride: elements between consecutive tokens of
 * key / value (>= num_kv_heads*head_dim, a multiple of 16 bytes), so that
 * slices of a fused QKV tensor can be passed directly.
 */
pa_status pa_store_kvcache(const void* key, const void* value,
                           int64_t key_tok_stride, int64_t value_tok_stride,
                           void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks,
                           pa_dtype dtype, void* stream);

/*
 * pa_decode_workspace_size -- bytes of workspace pa_decode needs for the
 * given split, whatever num_kv_heads the call passes (any divisor of
 * num_heads): partitions of partition_size tokens (0 when no sequence can
 * need more than one partition, i.e. partition_size == 0 or partition_size
 * >= max_context_len), or the balanced split (PA_PARTITION_BALANCED; the
 * size depends on the current device's compute-unit count, 256 assumed when
 * no device is visible). The size also serves pa_decode_hinted and the
 * E4M3 calls. Returns 0 for invalid arguments too.
 *
 * pa_decode_workspace_size_kv -- the same for a known num_kv_heads: the
 * exact size of that call's plan (the balanced split's workers depend on
 * how many query heads a wave serves). Over E4M3 pools at head_dim 64 with
 * one query head per KV head (and an even KV head count) the balanced split
 * reads pairs of KV heads and plans twice the workers; the size returned is
 * the larger of the paired and unpaired plans, so it serves pa_decode,
 * pa_decode_hinted, pa_decode_fp8 and the fused calls alike.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t max_context_len, int32_t partition_size);
size_t pa_decode_workspace_size_kv(int32_t num_seqs, int32_t num_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode -- one query token per sequence.
 *
 * For every sequence i and query head h:
 *   out[i][h] = softmax(scale * K_i[g] q[i][h]) V_i[g]
 * over the context_lens[i] tokens of sequence i gathered through
 * block_tables[i], g = h / (num_heads / num_kv_heads).
 *
 * partition_size selects how contexts are split across waves:
 *   0                      whole contexts, one kernel;
 *   > 0 (multiple of 16)   slices of that many tokens; every slice yields an
 *                          fp32 (max, sum, weighted values) state in the
 *                          workspace, and a second kernel on the same stream
 *                          merges the states of each (sequence, head);
 *   PA_PARTITION_BALANCED  the contexts laid end to end are cut into equal
 *                          ranges, one per resident wave, so that every wave
 *                          streams the same number of K/V bytes whatever the
 *                          length mix; sequences cut by a range boundary are
 *                          merged by a second kernel. At most 4096 sequences.
 * The result does not depend on the split beyond fp32 rounding.
 *
 * workspace: device memory of at least pa_decode_workspace_size(...) bytes
 * (or pa_decode_workspace_size_kv(...) with this call's num_kv_heads),
 * 256-byte aligned; its contents on entry do not matter and are scratch
 * afterwards. Calls sharing a workspace must not overlap in time (same
 * stream, or synchronised). May be NULL when the size is 0.
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq, int32_t max_context_len,
                    float scale, int32_t partition_size,
                    void* workspace, size_t workspace_bytes, pa_dtype dtype, void* stream);

/*
 * pa_decode_hinted -- pa_decode with a load-policy hint for shared prefix
 * blocks; every other argument is pa_decode's, in the same order.
 *
 * shared_lens: NULL, or int32 [num_seqs] on the device (4-byte aligned):
 * the number of leading context tokens of sequence i that lie in blocks
 * other sequences of the batch also read. Prefix sharing (the nano-vllm
 * page, sections 3.2 and 4.2: full blocks found by their rolling hash, with
 * reference counts) only ever shares a sequence's leading blocks, so one
 * count per sequence describes it; the Sequence's num_cached_tokens
 * (pa_bm_allocate) and pa_bm_shared_tokens give such a count. Those tokens
 * are read with a cache-retaining load policy, so that the sequences
 * sharing them find them in L2, while every other K/V byte is streamed past
 * the caches. It is a hint only: the result is bit-identical to pa_decode's
 * for any values (NULL streams everything, exactly as pa_decode does).
 */
pa_status pa_decode_hinted(void* out, const void* q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           const int32_t* shared_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_context_len,
                           float scale, int32_t partition_size,
                           void* workspace, size_t workspace_bytes,
                           pa_dtype dtype, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and result. A split's partial states go to a static scratch
 * array of PA_NOALLOC_SCRATCH_BYTES in the library, one per GPU, held
 * until the process ends; the call allocates and frees nothing. Its address
 * on a GPU is looked up the first time the call runs there (PA_ERR_HIP if
 * that fails).
 *
 * Limit: a split whose workspace (pa_decode_workspace_size_kv with the same
 * arguments) exceeds PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_WORKSPACE and
 * enqueues nothing. The balanced split (PA_PARTITION_BALANCED) needs at
 * most about 8.5 MB on a 256-CU device for any batch the call accepts;
 * whole contexts (0) need none; fixed slices need num_seqs * num_heads *
 * partitions * (head_dim + 2) * 4 bytes.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents (nothing in it needs clearing: every call writes what it
 * reads). Calls that overlap in time on one GPU (different streams, or
 * different host threads without ordering) race on it.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                            int32_t partition_size, pa_dtype dtype, void* stream);

/*
 * pa_store_decode -- pa_store_kvcache of each sequence's newest token fused
 * with pa_decode_hinted, in one launch (plus the merge kernel of a split).
 *
 * Row i of key/value ([num_seqs][num_kv_heads][head_dim], token strides in
 * elements as for pa_store_kvcache) is sequence i's newest token, at
 * position context_lens[i] - 1, and slot_mapping[i] is that position's slot
 * (block_tables[i][(L-1)/block_size] * block_size + (L-1) % block_size) or
 * negative. The result equals pa_store_kvcache(key, value, slot_mapping)
 * followed by pa_decode with the same arguments, up to fp32 rounding: the
 * rows are written into the pools, and the attention takes the newest token
 * from key/value directly instead of reading back the slot it writes (the
 * mini-vllm page's engine, whose decode step appends one token's K/V through
 * the block table and attends over the whole cached context). A sequence
 * with a negative slot is not stored and attends over the pool as it is.
 * All other arguments, errors and the workspace are those of
 * pa_decode_hinted (shared_lens may be NULL).
 */
pa_status pa_store_decode(void* out, const void* q,
                          const void* key, const void* value,
                          int64_t key_tok_stride, int64_t value_tok_stride,
                          void* k_cache, void* v_cache,
                          const int32_t* slot_mapping,
                          const int32_t* block_tables, const int32_t* context_lens,
                          const int32_t* shared_lens,
                          int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks,
                          int32_t max_blocks_per_seq, int32_t max_context_len,
                          float scale, int32_t partition_size,
                          void* workspace, size_t workspace_bytes,
                          pa_dtype dtype, void* stream);

/*
 * pa_prefill_chunk -- causal attention of a chunk of new tokens over the
 * cached-plus-new paged context (the prefill pass of the mini-vllm page's
 * inference engine, run chunk by chunk).
 *
 * Sequence i has n_i = query_start_loc[i+1] - query_start_loc[i] new rows
 * and c_i = context_lens[i] - n_i cached tokens; the new tokens' K/V must
 * already be stored (pa_store_kvcache). Row t (0 <= t < n_i) sits at
 * position c_i + t and attends to keys 0 .. c_i + t:
 *   out[r][h] = softmax(scale * K_i[g][0..c_i+t] q[r][h]) V_i[g][0..c_i+t],
 *   r = query_start_loc[i] + t.
 * Only PA_BF16 is implemented (bf16 MFMA, fp32 accumulation; the
 * probabilities are rounded to bf16 before the PV product).
 */
pa_status pa_prefill_chunk(void* out, const void* q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_tables,
                           const int32_t* query_start_loc,
                           const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads,
                           int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks_per_seq, int32_t max_query_len,
                           int32_t max_context_len, float scale,
                           pa_dtype dtype, void* stream);

/*
 * pa_mixed_batch -- one call for a continuous batch holding decode tokens
 * and prefill chunks together (the nano-vllm page's scheduler, §3.3, forms
 * such batches step after step).
 *
 * The result is pa_prefill_chunk's over the whole batch: sequence i has
 * n_i = query_start_loc[i+1] - query_start_loc[i] query rows, row t seeing
 * keys 0 .. context_lens[i] - n_i + t. The batch is ordered: its first
 * num_decode_seqs sequences are decode tokens, one row each
 * (query_start_loc[i] = i for i <= num_decode_seqs), and the prefill chunks
 * follow (n_i >= 1). Decode rows are computed as pa_decode computes them
 * (balanced split), prefill chunks on bf16 MFMA as pa_prefill_chunk does;
 * the two run in one kernel launch, side by side on the CUs, plus the small
 * merge kernel of the decode split.
 *
 * max_query_len: the largest n_i. workspace: at least
 * pa_decode_workspace_size_kv(num_decode_seqs, num_heads, num_kv_heads,
 * head_dim, max_context_len, PA_PARTITION_BALANCED) bytes, 256-byte aligned
 * (may be NULL when num_decode_seqs is 0). At most 2048 decode sequences.
 * shared_lens: NULL or int32 [num_seqs], the decode rows' load-policy hint
 * as for pa_decode_hinted (entries of prefill sequences are not read); the result
 * does not depend on it.
 * PA_BF16 only. Other arguments, shapes and errors as for pa_prefill_chunk.
 */
pa_status pa_mixed_batch(void* out, const void* q,
                         const void* k_cache, const void* v_cache,
                         const int32_t* block_tables,
                         const int32_t* query_start_loc,
                         const int32_t* context_lens,
                         const int32_t* shared_lens,
                         int32_t num_seqs, int32_t num_decode_seqs,
                         int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, int32_t max_blocks_per_seq,
                         int32_t max_query_len, int32_t max_context_len,
                         float scale, void* workspace, size_t workspace_bytes,
                         pa_dtype dtype, void* stream);

/*
 * 8-bit float (E4M3) pools.
 *
 * Quantisation of the cache is among the extensions both the nano-vllm page
 * (§5.3, extension suggestions) and the Nano-vLLM tutorial page (its closing
 * list of directions) leave for later; the pages fix no format. These calls
 * store each K/V element as one byte in the OCP E4M3 format (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; no infinity; 0x7F/0xFF are
 * NaN; largest finite value 448), with one fp32 scale per KV head for K and
 * one for V:
 *   stored value of element x of KV head h = value(code) * scale[h],
 *   code = the E4M3 code nearest to fp32(x / scale[h]) (ties to the even
 *          code), |x / scale[h]| saturated at 448; NaN -> 0x7F with x's sign.
 * The pools are uint8 [num_blocks][block_size][num_kv_heads][head_dim],
 * half the bytes of bf16. k_scale and v_scale are device fp32 arrays of
 * num_kv_heads entries (4-byte aligned) owned by the caller; choosing them
 * (e.g. max |x| / 448 per head) is the caller's business.
 *
 * pa_store_kvcache_fp8 -- pa_store_kvcache with quantisation: key/value are
 * dtype (PA_BF16 or PA_F32) rows with token strides in elements (multiples
 * of 16 bytes); head_dim a multiple of 16. The codes are bit-exact.
 */
pa_status pa_store_kvcache_fp8(const void* key, const void* value,
                               int64_t key_tok_stride, int64_t value_tok_stride,
                               void* k_cache, void* v_cache,
                               const int32_t* slot_mapping,
                               const float* k_scale, const float* v_scale,
                               int32_t num_tokens, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, pa_dtype dtype, void* stream);

/*
 * pa_decode_fp8 -- pa_decode over E4M3 pools: the same operation with
 * K[g] = value(codes) * k_scale[g] and V[g] = value(codes) * v_scale[g].
 * q and out are dtype (PA_BF16: q . K by bf16 dot products of q with the
 * exactly widened codes; PA_F32: fp32), accumulation fp32. Splits,
 * workspace (pa_decode_workspace_size or pa_decode_workspace_size_kv with
 * the same arguments), shapes and errors as for pa_decode, and shared_lens
 * as for pa_decode_hinted (pa_store_decode_fp8 below is the fused-store
 * form).
 */
pa_status pa_decode_fp8(void* out, const void* q,
                        const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_tables, const int32_t* context_lens,
                        const int32_t* shared_lens,
                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                        int32_t max_blocks_per_seq, int32_t max_context_len,
                        float scale, int32_t partition_size,
                        void* workspace, size_t workspace_bytes,
                        pa_dtype dtype, void* stream);

/*
 * pa_store_decode_fp8 -- pa_store_decode over E4M3 pools: in one launch,
 * sequence i's new K/V row (key/value rows i, dtype elements, token strides
 * in elements as for pa_store_kvcache_fp8) is quantised into slot
 * slot_mapping[i] exactly as pa_store_kvcache_fp8 quantises it, and the
 * sequence attends as pa_decode_fp8 does, its newest token taken as those
 * same codes. A negative slot stores nothing and that sequence reads its
 * newest token from the pool. Equal to pa_store_kvcache_fp8 followed by
 * pa_decode_fp8 up to the rounding order of the newest token; arguments,
 * workspace and errors as for those two calls, except that only PA_BF16 is
 * implemented here (PA_F32 returns PA_ERR_UNSUPPORTED).
 */
pa_status pa_store_decode_fp8(void* out, const void* q, const void* key,
                              const void* value, int64_t key_tok_stride,
                              int64_t value_tok_stride, void* k_cache, void* v_cache,
                              const float* k_scale, const float* v_scale,
                              const int32_t* slot_mapping,
                              const int32_t* block_tables, const int32_t* context_lens,
                              const int32_t* shared_lens,
                              int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t max_blocks_per_seq, int32_t max_context_len,
                              float scale, int32_t partition_size,
                              void* workspace, size_t workspace_bytes,
                              pa_dtype dtype, void* stream);

/*
 * pa_prefill_chunk_fp8 -- pa_prefill_chunk over E4M3 pools: the same
 * chunked causal attention with K[g] = value(codes) * k_scale[g] and
 * V[g] = value(codes) * v_scale[g]. The codes are widened exactly to bf16
 * and the products run on bf16 MFMA with fp32 accumulation; the K scale
 * multiplies the logit scale, the V scale the output. q and out are
 * PA_BF16 [sum n_i][num_heads][head_dim]; scales as for pa_decode_fp8.
 * Shapes, preconditions and errors as for pa_prefill_chunk, plus
 * PA_ERR_INVALID_ARG for a null scale array and PA_ERR_UNSUPPORTED for one
 * not 4-byte aligned.
 */
pa_status pa_prefill_chunk_fp8(void* out, const void* q,
                               const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const int32_t* block_tables,
                               const int32_t* query_start_loc,
                               const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_heads,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks_per_seq, int32_t max_query_len,
                               int32_t max_context_len, float scale,
                               pa_dtype dtype, void* stream);

/*
 * pa_mixed_batch_fp8 -- pa_mixed_batch over E4M3 pools: the same batch
 * layout and launch, its decode rows computed as pa_decode_fp8 computes them
 * (balanced split) and its prefill chunks as pa_prefill_chunk_fp8 does.
 * Scales as for pa_decode_fp8; workspace, shared_lens, shapes and errors
 * as for pa_mixed_batch, plus PA_ERR_INVALID_ARG for a null scale array and
 * PA_ERR_UNSUPPORTED for one not 4-byte aligned. PA_BF16 q/out only.
 */
pa_status pa_mixed_batch_fp8(void* out, const void* q,
                             const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale,
                             const int32_t* block_tables,
                             const int32_t* query_start_loc,
                             const int32_t* context_lens,
                             const int32_t* shared_lens,
                             int32_t num_seqs, int32_t num_decode_seqs,
                             int32_t num_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, int32_t max_blocks_per_seq,
                             int32_t max_query_len, int32_t max_context_len,
                             float scale, void* workspace, size_t workspace_bytes,
                             pa_dtype dtype, void* stream);

/*
 * Block manager (host only; no device memory, no HIP calls).
 *
 * Hands out the physical blocks of a pool of num_blocks blocks of block_size
 * tokens to sequences and shares full prompt blocks between sequences with
 * the same prefix (the nano-vllm page: Block with reference count, hash and
 * token ids, §3.2.1; the allocation loop, §3.2.2; the rolling hash
 * h <- (31 h + t) mod 2^32 chained from the block before, §4.2; and the
 * mini-vllm page's BlockAllocator, architecture item 1, which serves prefill
 * and decode and frees a finished request's blocks). Only full blocks are
 * hashed and shared; a hash hit counts only when the block's tokens and the
 * block before it match. The tables and slots it produces are the
 * block_tables rows and slot_mapping entries of the calls above.
 *
 * The manager owns its host memory; it is not thread-safe. Every call
 * validates its arguments and, on failure, changes nothing.
 */
typedef struct pa_block_manager pa_block_manager;

/* A manager over blocks 0 .. num_blocks-1. free_order (may be NULL: 0, 1,
 * 2, ...) is a permutation of the block ids giving the free list, front
 * first; new blocks come from its front, reclaimed blocks go to its back. */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                       pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* Blocks for a new sequence's num_tokens prompt tokens: for each block,
 * reuse a matching shared block (one more reference) or take a free one.
 * Writes ceil(num_tokens/block_size) ids to table (table_capacity entries
 * available) and their count to *num_table_blocks; *num_cached_tokens is
 * block_size times the number of leading blocks that were reused (tokens
 * whose K/V are already in the pool); slots (may be NULL) receives every
 * token's slot, block * block_size + row. PA_ERR_OUT_OF_BLOCKS if the free
 * list runs out. */
pa_status pa_bm_allocate(pa_block_manager* bm, const int32_t* token_ids, int32_t num_tokens,
                         int32_t* table, int32_t table_capacity, int32_t* num_table_blocks,
                         int32_t* num_cached_tokens, int32_t* slots);

/* Decode: append token_id at position num_tokens of the sequence holding
 * table (*num_table_blocks entries). A new block is taken when the last one
 * is full (the table grows by one entry); a block the token fills is hashed
 * and becomes shareable. *slot receives the token's slot. */
pa_status pa_bm_append(pa_block_manager* bm, int32_t* table, int32_t* num_table_blocks,
                       int32_t table_capacity, int32_t num_tokens, int32_t token_id,
                       int32_t* slot);

/* A finished sequence: one reference less on each block of its table (last
 * block first); blocks left with none return to the free list. */
pa_status pa_bm_free(pa_block_manager* bm, const int32_t* table, int32_t num_table_blocks);

/* Free blocks, and a block's reference count (-1 for an invalid id). */
int32_t pa_bm_num_free(const pa_block_manager* bm);
int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block_id);

/* The leading tokens of a sequence (num_tokens long, its table of
 * num_table_blocks entries) that lie in blocks with more than one reference,
 * i.e. that other sequences read too: the decode calls' shared_lens entry
 * for it. Prefix sharing shares leading blocks only (the nano-vllm page,
 * sections 3.2 and 4.2), so the count stops at the first private block. -1
 * for a null manager, negative sizes or an invalid block id. */
int32_t pa_bm_shared_tokens(const pa_block_manager* bm, const int32_t* table,
                            int32_t num_table_blocks, int32_t num_tokens);

/* Description of the calling thread's last failed block-manager call. */
const char* pa_bm_last_error(void);

/*
 * pa_stream_read -- a measurement aid, not an operation of the pages: the
 * rate at which this device sustains plain streaming reads, the reference
 * the decode calls' K/V read rate is compared with. Reads the first
 * *bytes_read bytes of buf (a whole number of equal per-wave slices, at most
 * bytes) once, each wave one contiguous slice with 16-byte nontemporal
 * loads at two waves per SIMD, and combines them into a value that decides
 * whether *out (device, 4-byte aligned) is written; in practice it is not.
 * buf: device memory, 16-byte aligned, at least 16 KB per resident wave
 * (16 MB on a 256-CU device), contents irrelevant. *bytes_read (host) is
 * set before the launch, which is asynchronous on stream. Errors:
 * PA_ERR_INVALID_ARG for null pointers or a buffer below the minimum,
 * PA_ERR_UNSUPPORTED for misaligned pointers, PA_ERR_HIP for a failed launch.
 */
pa_status pa_stream_read(const void* buf, size_t bytes, uint32_t* out, size_t* bytes_read,
                         void* stream);

/* Static description of a status code. */
const char* pa_status_string(pa_status s);

/* Description of the calling thread's last failed call ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
