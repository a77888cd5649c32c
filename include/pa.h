/*
 * pa.h — C ABI of the paged KV-cache attention library (libpa.so, gfx950).
 *
 * Each sequence's keys and values live in fixed-size physical blocks of one
 * shared pool per tensor; a per-sequence block table maps the sequence's
 * logical blocks to physical ones.  The calls below write new tokens into
 * the pool, copy blocks for copy-on-write, and compute attention for decode
 * tokens and for causal prefill chunks by resolving every block through the
 * table.
 *
 * Pages this interface follows (by title):
 *   [bogosort]  "五十三：vLLM-PagedAttention" (book.bogosort.top, lesson 53)
 *   [datawhale] "17. vLLM PagedAttention | 经典推理框架: 模拟 Continuous
 *               Batching 与 PagedAttention" (datawhalechina llm-algo-leetcode)
 *   [ybb]       "vLLM 与 LLM 推理部署实战：从 PagedAttention 到生产级服务架构"
 *   [intelli]   "vLLM与PagedAttention：大模型推理内存优化技术解析"
 *   [aieng]     "推理引擎内部机制——PagedAttention、连续批处理、分块预填充"
 *
 * Conventions shared by every call
 * --------------------------------
 * Pools.  k_pool and v_pool are separate dense arrays laid out
 *   [num_blocks][num_kv_heads][block_size][head_dim]   (row-major)
 *   so one (block, KV head) tile of block_size x head_dim elements is
 *   contiguous.  A token's slot is physical_block * block_size + offset.
 * Element types (pa_dtype): f32, f16, bf16, OCP fp8 E4M3FN and int8 (cache
 *   only).  Supported (q, cache) pairs: (f32,f32) (f16,f16) (bf16,bf16)
 *   (bf16,fp8) (f16,fp8); with separate K/V types also an fp8 K pool beside a
 *   V pool of the query type (pa_*_kv); int8 K and V pools with per-block
 *   scales and bf16/f16 queries (pa_*_int8).  Outputs have the query's type.
 *   For an fp8 cache the stored code times the per-tensor k_scale / v_scale
 *   is the value; the scales are applied the same way for other cache types
 *   (pass 1.0f).
 * Shapes.  head_dim is 64 or 128; block_size is 8, 16, 32 or 64; num_q_heads is a
 *   multiple of num_kv_heads with at most 16 query heads per KV head.  Query
 *   head h uses KV head h / (num_q_heads / num_kv_heads).
 * Memory.  Every pointer is device memory owned by the caller, dense, and
 *   16-byte aligned (block tables, lengths and slot arrays: 4-byte aligned).
 *   The library allocates nothing, keeps no per-call state and never
 *   synchronises: each call only enqueues work on `stream` (a hipStream_t;
 *   NULL = the null stream) and returns.  Results are stream-ordered.
 * Errors.  Arguments are checked on the host before anything is enqueued; a
 *   failed check returns a non-zero pa_status and enqueues nothing.  Launch
 *   failures return PA_ERR_HIP.  pa_last_error() gives a message for the
 *   last failure on the calling thread.  Device-resident contents (block
 *   ids, slots, lengths, chunk offsets) are trusted: the kernels clamp
 *   lengths to the table width, but a block id outside the pool is
 *   undefined behaviour.  pa_check_block_tables / pa_check_slots (end of
 *   this file) check them on the device and report through an error word.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_DTYPE_F32 = 0,
  PA_DTYPE_F16 = 1,
  PA_DTYPE_BF16 = 2,
  PA_DTYPE_FP8_E4M3 = 3,
  PA_DTYPE_INT8 = 4      /* symmetric int8 codes with per-(block, KV head) scales */
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, ... */
  PA_ERR_UNSUPPORTED = 2, /* valid but not implemented: dtype pair, shape */
  PA_ERR_WORKSPACE = 3,   /* split decode needs a larger workspace */
  PA_ERR_HIP = 4,         /* the HIP runtime reported an error */
  PA_ERR_OUT_OF_BLOCKS = 5 /* host block manager: not enough free blocks (nothing changed) */
} pa_status;

/*
 * pa_reshape_and_cache — write new tokens' K/V into their pool slots.
 *
 * [datawhale] Step 3 item 3 and Step 4: physical blocks are handed out on
 * demand as tokens are generated and each token's K/V is stored in its
 * block; [bogosort] §8: the block table maps logical to physical blocks.
 * For token t with slot_mapping[t] >= 0, for every KV head h:
 *   k_pool[slot / block_size][h][slot % block_size][:] = key[t][h][:]
 * and the same for value / v_pool.  A negative slot skips the token.
 * If cache_dtype == src_dtype the bits are copied unchanged.  For an fp8
 * cache ([ybb] §6.2, KV cache in FP8) each element is stored as
 * e4m3(float32(x) / k_scale) (v_scale for V): one correctly rounded float32
 * division, round-to-nearest-even, magnitudes above 448 (and infinities)
 * saturate to 448, NaN stays NaN.
 *
 *   key, value    [num_tokens][num_kv_heads][head_dim], src_dtype; row t
 *                 starts at key + t * key_token_stride elements
 *                 (0 = dense, num_kv_heads * head_dim); same for value.
 *   k_pool,v_pool [num_blocks][num_kv_heads][block_size][head_dim], cache_dtype
 *   slot_mapping  int64 [num_tokens]; slots must be distinct and
 *                 < num_blocks * block_size.
 * src_dtype must equal cache_dtype, or cache_dtype is fp8 and src_dtype is
 * bf16/f16/f32.  num_tokens == 0 is a no-op.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                               const int64_t* slot_mapping, int32_t num_tokens,
                               int64_t key_token_stride, int64_t value_token_stride,
                               int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, pa_dtype src_dtype, pa_dtype cache_dtype,
                               float k_scale, float v_scale, void* stream);

/*
 * pa_reshape_and_cache_kv — pa_reshape_and_cache with separate K and V pool
 * element types, for the mixed-precision cache of [intelli] §6.1 (an fp8 K
 * cache beside a bf16 V cache: 3 bytes per K/V element pair instead of 4).
 * K follows the pa_reshape_and_cache rules with cache_dtype = k_cache_dtype;
 * v_cache_dtype equals k_cache_dtype (then the call equals
 * pa_reshape_and_cache), or k_cache_dtype is fp8 and v_cache_dtype equals
 * src_dtype (V bits copied unchanged; v_scale unused for V).  Any other pair
 * returns PA_ERR_UNSUPPORTED.
 */
pa_status pa_reshape_and_cache_kv(const void* key, const void* value, void* k_pool, void* v_pool,
                                  const int64_t* slot_mapping, int32_t num_tokens,
                                  int64_t key_token_stride, int64_t value_token_stride,
                                  int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, pa_dtype src_dtype, pa_dtype k_cache_dtype,
                                  pa_dtype v_cache_dtype, float k_scale, float v_scale, void* stream);

/*
 * pa_reshape_and_cache_int8 — the scatter into an INT8 cache ([ybb] §6.2:
 * an INT8 or FP8 KV cache halves the bytes per token; the page fixes no scale
 * granularity or rounding).  Each (block, KV head) of the K pool has one
 * float32 scale k_scales[block][head], likewise v_scales for V, set by the
 * caller (for instance from the amax of the block's tokens) before tokens
 * are written into the block.  Element x of token t (slot s, block
 * b = s / block_size) of head h is stored as
 *   code = clamp(round_half_even(float32(x) / k_scales[b][h]), -127, 127)
 * with one correctly rounded float32 division; NaN stores 0.  Scales must be
 * finite and positive (device data, not checked).  The other arguments and
 * rules are those of pa_reshape_and_cache with src_dtype f32/f16/bf16; pools
 * hold int8 codes.
 *   k_scales, v_scales  float32 [num_blocks][num_kv_heads], device memory
 */
pa_status pa_reshape_and_cache_int8(const void* key, const void* value, void* k_pool, void* v_pool,
                                    const float* k_scales, const float* v_scales,
                                    const int64_t* slot_mapping, int32_t num_tokens,
                                    int64_t key_token_stride, int64_t value_token_stride,
                                    int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, pa_dtype src_dtype, void* stream);

/*
 * pa_copy_blocks — copy whole blocks for copy-on-write.
 *
 * [ybb] §2.2 Copy-on-Write: when several sequences reference one block, a
 * write to it first duplicates the whole block.  For each pair p,
 *   block block_pairs[2p+1] of k_pool and of v_pool becomes a copy of block
 *   block_pairs[2p].
 * block_bytes is the size of one block of one pool
 * (num_kv_heads * block_size * head_dim * element bytes); it must be a
 * multiple of 16.  block_pairs is int64 [num_pairs][2] (src, dst) in device
 * memory.  Destinations must be distinct and never a source in the same
 * call.  num_pairs == 0 is a no-op.
 */
pa_status pa_copy_blocks(void* k_pool, void* v_pool, const int64_t* block_pairs, int32_t num_pairs,
                         int64_t block_bytes, void* stream);

/*
 * pa_copy_blocks_partial — copy-on-write of partly filled blocks.
 *
 * [bogosort] §17 Parallel Sampling: sequences forked from one prompt share
 * its blocks and write what follows the fork into blocks of their own; when
 * the fork falls inside a block, the new block needs only the tokens that
 * precede the fork.  For each triple p of block_triples (int64
 * [num_pairs][3] = src, dst, n in device memory), rows [0, n) of every KV
 * head of block dst of k_pool and of v_pool become those of block src; the
 * other rows of dst are left as they are.  n is clamped to
 * [0, block_size].  Pools are [blocks][num_kv_heads][block_size][row] with
 * row_bytes = head_dim * element bytes (a multiple of 16).  Destinations
 * must be distinct and never a source in the same call.  num_pairs == 0 is
 * a no-op.
 */
pa_status pa_copy_blocks_partial(void* k_pool, void* v_pool, const int64_t* block_triples, int32_t num_pairs,
                                 int32_t num_kv_heads, int32_t block_size, int64_t row_bytes, void* stream);

/*
 * pa_copy_blocks_layers — the same whole-block copies in every layer.
 *
 * [ybb] §2.2 Copy-on-Write: a fork duplicates a shared block in each
 * layer's cache.  k_pools and v_pools are device arrays of num_layers
 * device pointers (one K and one V pool per layer, all with the same block
 * size block_bytes, a multiple of 16); for each (src, dst) pair of
 * block_pairs (int64 [num_pairs][2], device memory) and each layer, block
 * dst becomes a copy of block src.  One launch covers all layers.
 */
pa_status pa_copy_blocks_layers(void* const* k_pools, void* const* v_pools, int32_t num_layers,
                                const int64_t* block_pairs, int32_t num_pairs, int64_t block_bytes,
                                void* stream);

/*
 * pa_swap_blocks — move blocks between two pools, e.g. to and from CPU
 * memory.
 *
 * [ybb] §三 Continuous Batching, the preemption bullet: when memory runs
 * short, the block manager swaps blocks out to CPU memory (and back in
 * later).  For each (src, dst) pair of block_pairs (int64 [num_pairs][2]),
 * block dst of dst_pool becomes a copy of block src of src_pool
 * (block_bytes each, a multiple of 16).  Each of dst_pool, src_pool and
 * block_pairs is device memory or pinned host memory (hipHostMalloc, or a
 * pinned torch tensor), reached by the kernel through its device mapping;
 * pageable host memory is rejected with PA_ERR_INVALID_ARG.  Call it once
 * for the K pools and once for the V pools.  The pools must not overlap.
 */
pa_status pa_swap_blocks(void* dst_pool, const void* src_pool, const int64_t* block_pairs, int32_t num_pairs,
                         int64_t block_bytes, void* stream);

/*
 * Split-KV planning for decode.  The decode kernel is persistent: each of
 * its waves processes one or more segments, a segment being a run of
 * 32-token steps of one (sequence, KV head) pair.  A pair whose context is
 * cut into several segments gets partial results (unnormalised output,
 * running max, running sum), merged by log-sum-exp: in LDS by the attention
 * kernel itself when all of the pair's segments fall in one workgroup's
 * share of the work, else through the workspace by the reduce kernel (both
 * merges sum in the same order and give the same bits).  partition_size
 * chooses the cut:
 *   0   : balanced (the default) — the (sequence, KV head, 32-token step)
 *         units of the whole batch are cut into equal contiguous ranges, one
 *         per wave, from the lengths on the device; a pair is cut into at
 *         most 17 segments;
 *   > 0 : fixed partitions of partition_size tokens from each sequence's
 *         start (a multiple of 32 and of block_size);
 *   -1  : never split: every pair is processed whole by one wave.
 *
 * pa_decode_partition_size validates a request and returns it resolved: the
 * partition length for > 0, 0 for the balanced cut, a value >= max_seq_len
 * for -1, or a negative value for an invalid request.
 *
 * pa_decode_workspace_bytes returns the workspace pa_decode needs (0 for -1):
 * fp32 partial outputs [S][Hq][max_parts][D], maxima and sums
 * [S][Hq][max_parts] and int32 segment counts [S][Hkv], each 256-byte
 * aligned.  max_seq_len is an upper bound on every seq_lens[s]
 * (0 = max_blocks_per_seq * block_size).
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                 int32_t max_seq_len, int32_t partition_size);
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t max_seq_len,
                                 int32_t partition_size);

/*
 * pa_decode — attention of one query token per sequence over its paged
 * context.
 *
 * [bogosort] §8: the attention kernel finds a sequence's past K/V through
 * the block table; [ybb] §2.3: attention walks every K/V pair, jumping to
 * each block through the table; [datawhale] Step 2: the blocks named by the
 * table, in table order and cut to seq_len tokens, form the sequence's
 * cache.  For sequence s with n = seq_lens[s] (the new token included; its
 * K/V must already be in the pool) and query head h, kv = h / group:
 *   logit_j = scale * k_scale * (q[s][h] . Kcode[j])   for j < n
 *   out[s][h] = v_scale * sum_j softmax(logit)_j * Vcode[j]
 * Accumulation is float32; probabilities enter the value product in the
 * query's 16-bit type (f32 queries stay f32).  n <= 0 gives a zero output.
 *
 *   out            [num_seqs][num_q_heads][head_dim], q_dtype (written)
 *   q              [num_seqs][num_q_heads][head_dim], q_dtype
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]; entries at or past
 *                  ceil(n / block_size) are never read
 *   seq_lens       int32 [num_seqs]; each <= max_seq_len and
 *                  <= max_blocks_per_seq * block_size (clamped otherwise)
 *   max_seq_len    upper bound used to size the split grid (0 = table width)
 *   partition_size see pa_decode_partition_size
 *   workspace      >= pa_decode_workspace_bytes(...) bytes of device memory,
 *                  256-byte aligned (may be NULL when that is 0); its
 *                  contents need no initialisation
 * Limits: num_seqs <= 8000 (the per-call plan lives in LDS) and
 * num_seqs * ceil(max_seq_len / 32) * num_kv_heads <= 2^30; beyond them the
 * call returns PA_ERR_UNSUPPORTED.
 */
pa_status pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                    const int32_t* block_tables, const int32_t* seq_lens, float scale,
                    int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                    int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype, float k_scale,
                    float v_scale, int32_t partition_size, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc — pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): it takes no workspace argument and calls no allocating
 * routine.  The split-KV partials go to a device array inside the library,
 * pa_decode_noalloc_max_workspace_bytes() (64 MiB) long; each GPU the
 * library runs on holds its own copy from the first call on that device
 * until the process ends.  The caller still owns out, q, the pools, tables
 * and lengths.  Arguments, results and limits are those of pa_decode (same
 * kernels, same bits); a call whose pa_decode_workspace_bytes(...) exceeds
 * the array returns PA_ERR_WORKSPACE and enqueues nothing.  The array keeps
 * the last call's contents; nothing in it has to start at zero.  Every call
 * on one GPU shares that GPU's array, so calls that can overlap on one GPU
 * (concurrent streams, several host threads) race and must be ordered by
 * the caller.
 */
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* seq_lens, float scale,
                            int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                            int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype,
                            float k_scale, float v_scale, int32_t partition_size, void* stream);
size_t pa_decode_noalloc_max_workspace_bytes(void);

/*
 * The two stages of pa_decode, for callers that time or schedule them
 * separately.  pa_decode_attention runs the attention kernel: pairs
 * processed as one segment, pairs whose partials it merged on the CU, and
 * empty sequences (which get zeros) have their final output in `out`; the
 * others leave partial results and their segment count in `workspace`.
 * pa_decode_reduce then merges those
 * partials into `out` (nothing to do for partition_size -1).  Both take
 * exactly the arguments of pa_decode; calling them in order on one stream
 * equals one pa_decode call.
 */
pa_status pa_decode_attention(void* out, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens, float scale,
                              int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype,
                              float k_scale, float v_scale, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, void* stream);
pa_status pa_decode_reduce(void* out, const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens, float scale,
                           int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                           int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype,
                           float k_scale, float v_scale, int32_t partition_size, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * pa_decode_kv — pa_decode with separate K and V pool element types
 * ([intelli] §6.1: fp8 K cache, bf16 V cache, bf16 activations).  The
 * result is the pa_decode formula with K read as k_cache_dtype and V as
 * v_cache_dtype (fp8 codes decoded exactly, then scaled by k_scale /
 * v_scale; 16-bit pools use the scales the same way).  Supported: the pairs
 * of pa_decode with v_cache_dtype == k_cache_dtype, and k_cache_dtype fp8
 * with v_cache_dtype == q_dtype (bf16 or f16).  Other pairs return
 * PA_ERR_UNSUPPORTED.  Workspace and partition rules are those of
 * pa_decode (pa_decode_workspace_bytes does not depend on the pool types).
 */
pa_status pa_decode_kv(void* out, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* seq_lens, float scale,
                       int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                       int32_t max_seq_len, pa_dtype q_dtype, pa_dtype k_cache_dtype,
                       pa_dtype v_cache_dtype, float k_scale, float v_scale,
                       int32_t partition_size, void* workspace, size_t workspace_bytes,
                       void* stream);
/* The two stages of pa_decode_kv (as pa_decode_attention / pa_decode_reduce
 * are for pa_decode), taking exactly its arguments. */
pa_status pa_decode_attention_kv(void* out, const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* seq_lens, float scale,
                                 int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                                 int32_t max_seq_len, pa_dtype q_dtype, pa_dtype k_cache_dtype,
                                 pa_dtype v_cache_dtype, float k_scale, float v_scale,
                                 int32_t partition_size, void* workspace, size_t workspace_bytes,
                                 void* stream);
pa_status pa_decode_reduce_kv(void* out, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens, float scale,
                              int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                              int32_t max_seq_len, pa_dtype q_dtype, pa_dtype k_cache_dtype,
                              pa_dtype v_cache_dtype, float k_scale, float v_scale,
                              int32_t partition_size, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * pa_decode_int8 — pa_decode over an INT8 cache with per-block scales (see
 * pa_reshape_and_cache_int8): for token j in block b,
 *   logit_j = scale * k_scales[b][kv] * (q . Kcode[j])
 *   out = sum_j softmax(logit)_j * v_scales[b][kv] * Vcode[j]
 * q_dtype bf16 or f16 (codes enter the matrix products exactly as that
 * type; p * v_scales is rounded once to it for the value product, the sums
 * of p stay float32).  Other arguments, limits, workspace and partition
 * rules are those of pa_decode; the attention / reduce stages are split as for pa_decode.
 */
pa_status pa_decode_int8(void* out, const void* q, const void* k_pool, const void* v_pool,
                         const float* k_scales, const float* v_scales, const int32_t* block_tables,
                         const int32_t* seq_lens, float scale, int32_t block_size, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t max_blocks_per_seq, int32_t max_seq_len, pa_dtype q_dtype,
                         int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);
pa_status pa_decode_attention_int8(void* out, const void* q, const void* k_pool, const void* v_pool,
                                   const float* k_scales, const float* v_scales,
                                   const int32_t* block_tables, const int32_t* seq_lens, float scale,
                                   int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                                   int32_t max_seq_len, pa_dtype q_dtype, int32_t partition_size,
                                   void* workspace, size_t workspace_bytes, void* stream);
pa_status pa_decode_reduce_int8(void* out, const void* q, const void* k_pool, const void* v_pool,
                                const float* k_scales, const float* v_scales,
                                const int32_t* block_tables, const int32_t* seq_lens, float scale,
                                int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                                int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                                int32_t max_seq_len, pa_dtype q_dtype, int32_t partition_size,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_append — pa_reshape_and_cache of each sequence's newest token
 * followed by pa_decode, in one kernel ([datawhale] Step 4: a decode step
 * stores the new token's K/V in its block, then attends over the table).
 * Sequence s with n = seq_lens[s] > 0 has its newest token at position
 * n - 1; its slot is block_tables[s][(n - 1) / block_size] * block_size +
 * (n - 1) % block_size.  The call's result equals
 *   pa_reshape_and_cache(new_k, new_v, ..., slot_mapping = those slots)
 *   pa_decode(...)
 * on one stream, bit for bit: the attention reads the newest rows from
 * new_k / new_v, and the wave that covers them writes them into the pool.
 *   new_k, new_v  [num_seqs][num_kv_heads][head_dim] in the cache type; row
 *                 s starts at s * new_*_stride elements (0 = dense)
 * Requirements: q_dtype == cache_dtype, bf16 or f16; seq_lens[s] <=
 * max_seq_len (when max_seq_len > 0) so that no length is clamped; n <= 0
 * appends nothing.  pa_decode_attention_append is the first stage
 * (pa_decode_reduce with the same pools, tables and workspace completes it).
 */
pa_status pa_decode_append(void* out, const void* q, const void* new_k, const void* new_v,
                           int64_t new_k_stride, int64_t new_v_stride, void* k_pool, void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens, float scale,
                           int32_t block_size, int32_t num_seqs, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t max_blocks_per_seq,
                           int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype, float k_scale,
                           float v_scale, int32_t partition_size, void* workspace,
                           size_t workspace_bytes, void* stream);
pa_status pa_decode_attention_append(void* out, const void* q, const void* new_k, const void* new_v,
                                     int64_t new_k_stride, int64_t new_v_stride, void* k_pool,
                                     void* v_pool, const int32_t* block_tables,
                                     const int32_t* seq_lens, float scale, int32_t block_size,
                                     int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t max_blocks_per_seq,
                                     int32_t max_seq_len, pa_dtype q_dtype, pa_dtype cache_dtype,
                                     float k_scale, float v_scale, int32_t partition_size,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_prefill_chunk — causal attention of one prefill chunk per sequence
 * over its paged context.
 *
 * [bogosort] §15 Chunked Prefill and [aieng] "分块预填充保护 TTFT 尾部": a long
 * prompt is prefilled in consecutive chunks (about 512 tokens) interleaved
 * with decode.  Sequence s has seq_lens[s] = n context tokens, whose last
 * L = query_start_loc[s+1] - query_start_loc[s] tokens are this chunk; the
 * chunk's own K/V must already be in the pool (pa_reshape_and_cache).
 * Chunk query i sits at position n - L + i and attends keys 0 .. n - L + i
 * (causal, aligned to the end of the context).  Requires n >= L.
 *
 *   out, q          [total_q_tokens][num_q_heads][head_dim], q_dtype; the
 *                   chunk of sequence s is rows query_start_loc[s] ..
 *                   query_start_loc[s+1] - 1
 *   query_start_loc int32 [num_seqs + 1], non-decreasing, last = total
 *   max_q_len       >= every chunk length (sizes the grid)
 * Supported (q, cache) pairs: (bf16, bf16), (f16, f16), (f32, f32), and an
 * fp8 E4M3 cache beside bf16 or f16 queries ([ybb] §6.2, KV cache in FP8):
 * codes are decoded exactly to the query type and the per-tensor k_scale /
 * v_scale apply as in pa_decode (logit = scale * k_scale * q . Kcode,
 * out = v_scale * sum softmax * Vcode).  For 16-bit and fp8 caches
 * num_q_heads / num_kv_heads is a power of two <= 16 (any group <= 16 for
 * f32).  Accumulation is float32; 16-bit and fp8 paths feed probabilities
 * to the matrix cores in the query's type.
 */
pa_status pa_prefill_chunk(void* out, const void* q, const int32_t* query_start_loc,
                           const void* k_pool, const void* v_pool, const int32_t* block_tables,
                           const int32_t* seq_lens, float scale, int32_t block_size,
                           int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t max_blocks_per_seq, pa_dtype q_dtype, pa_dtype cache_dtype,
                           float k_scale, float v_scale, void* stream);

/*
 * pa_prefill_chunk_int8 — pa_prefill_chunk over an INT8 cache with
 * per-block scales (see pa_reshape_and_cache_int8): for key j in block b,
 *   logit = scale * k_scales[b][kv] * (q . Kcode[j])
 *   out = sum_j softmax(logit)_j * v_scales[b][kv] * Vcode[j]
 * the formula of pa_decode_int8 applied to each chunk query over its causal
 * context.  q_dtype bf16 or f16 (codes enter the matrix products exactly as
 * that type; each probability of the value product carries its key's V
 * scale and is rounded once to the query type, the row sums add the float32
 * probabilities without it).  Other arguments, layouts and limits are
 * those of pa_prefill_chunk; an int8 cache given to pa_prefill_chunk without
 * scales returns PA_ERR_INVALID_ARG.
 */
pa_status pa_prefill_chunk_int8(void* out, const void* q, const int32_t* query_start_loc,
                                const void* k_pool, const void* v_pool, const float* k_scales,
                                const float* v_scales, const int32_t* block_tables,
                                const int32_t* seq_lens, float scale, int32_t block_size,
                                int32_t num_seqs, int32_t total_q_tokens, int32_t max_q_len,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t max_blocks_per_seq, pa_dtype q_dtype, void* stream);

/*
 * pa_mixed_attention — the attention of one mixed serving step in one
 * launch: the prefill chunks of some sequences and the one-token decodes of
 * others, over the same K/V pools.
 *
 * [aieng] "推理引擎内部机制", section "调度器长什么样": each engine step
 * batches prefill chunks with decodes and runs them as one fused GPU call;
 * [bogosort] §15 Chunked Prefill for the chunks.  The prefill part computes
 * pa_prefill_chunk over (prefill_out, prefill_q, query_start_loc,
 * prefill_block_tables, prefill_seq_lens, num_chunks, total_q_tokens,
 * max_q_len, prefill_max_blocks_per_seq) and the decode part pa_decode over
 * (decode_out, decode_q, decode_block_tables, decode_seq_lens, num_decodes,
 * decode_max_blocks_per_seq, max_seq_len, partition_size, workspace); the
 * remaining arguments are common to both, with the meaning, layouts, limits
 * and errors of those two calls.  Either part may be empty (num_chunks or
 * total_q_tokens 0; num_decodes 0).
 *
 * Supported: bf16 or f16 queries over a cache of the same type, or over an
 * fp8 E4M3 cache with per-tensor k_scale / v_scale as in pa_decode and
 * pa_prefill_chunk ([ybb] §6.2); an int8 cache goes through
 * pa_mixed_attention_int8 (here it returns PA_ERR_INVALID_ARG); other pairs
 * return PA_ERR_UNSUPPORTED.  The
 * prefill outputs equal pa_prefill_chunk's bit for bit; the decode outputs
 * may differ from a pa_decode call by rounding, since the work is cut for
 * this launch's waves.  The workspace is pa_decode_workspace_bytes(num_decodes, ...) long
 * (contents need no initialisation).  Two kernels are enqueued on `stream`:
 * the mixed one and the log-sum-exp reduce of the decode partials.
 */
pa_status pa_mixed_attention(void* prefill_out, const void* prefill_q,
                             const int32_t* query_start_loc, const int32_t* prefill_block_tables,
                             const int32_t* prefill_seq_lens, int32_t num_chunks,
                             int32_t total_q_tokens, int32_t max_q_len,
                             int32_t prefill_max_blocks_per_seq, void* decode_out,
                             const void* decode_q, const int32_t* decode_block_tables,
                             const int32_t* decode_seq_lens, int32_t num_decodes,
                             int32_t decode_max_blocks_per_seq, int32_t max_seq_len,
                             const void* k_pool, const void* v_pool, float scale,
                             int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, pa_dtype q_dtype, pa_dtype cache_dtype,
                             float k_scale, float v_scale, int32_t partition_size,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_mixed_attention_int8 — pa_mixed_attention over an INT8 cache with
 * per-(block, KV head) scales (layout and meaning of pa_reshape_and_cache_int8;
 * [ybb] §6.2, KV cache quantisation): the prefill part computes
 * pa_prefill_chunk_int8, the decode part pa_decode_int8, in one launch.
 * k_scales / v_scales: float32 [num_blocks, num_kv_heads] device arrays,
 * caller-owned, read only (null returns PA_ERR_INVALID_ARG).  q_dtype bf16 or
 * f16.  Other arguments, limits, outputs and errors are pa_mixed_attention's;
 * the prefill outputs equal pa_prefill_chunk_int8's bit for bit.
 */
pa_status pa_mixed_attention_int8(void* prefill_out, const void* prefill_q,
                                  const int32_t* query_start_loc, const int32_t* prefill_block_tables,
                                  const int32_t* prefill_seq_lens, int32_t num_chunks,
                                  int32_t total_q_tokens, int32_t max_q_len,
                                  int32_t prefill_max_blocks_per_seq, void* decode_out,
                                  const void* decode_q, const int32_t* decode_block_tables,
                                  const int32_t* decode_seq_lens, int32_t num_decodes,
                                  int32_t decode_max_blocks_per_seq, int32_t max_seq_len,
                                  const void* k_pool, const void* v_pool, const float* k_scales,
                                  const float* v_scales, float scale, int32_t block_size,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  pa_dtype q_dtype, int32_t partition_size, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Index checks.  The calls above trust device-resident indices (a block id
 * outside the pool is undefined behaviour there, as checking would need a
 * synchronisation).  A caller that wants them checked enqueues these calls
 * on the same stream first: each writes a device error record of three
 * int32 (caller-owned device memory, reset by the call itself before it
 * checks): error[0] = OR of the pa_check_flag values found, error[1] =
 * number of offending sequences (tables) or tokens (slots), error[2] = the
 * smallest offending sequence / token index (INT32_MAX when none).  Nothing
 * the indices name is read, so the checks are safe on any input.
 *
 * pa_check_block_tables ([datawhale] TODO 5 and [bogosort] §8: a sequence's
 * blocks are the first ceil(seq_len / block_size) entries of its table row):
 * for each sequence s, seq_lens[s] must lie in [0, max_blocks_per_seq *
 * block_size] and, when max_seq_len > 0, not exceed max_seq_len (else
 * PA_CHECK_LENGTH); each of those entries must lie in [0, num_blocks) (else
 * PA_CHECK_BLOCK_ID).  With query_start_loc (may be NULL; [num_seqs + 1],
 * as pa_prefill_chunk takes it): offsets must be non-decreasing from >= 0,
 * each chunk no longer than its context, and the last offset equal to
 * total_q_tokens (else PA_CHECK_CHUNK).
 *
 * pa_check_slots ([datawhale] Step 4, slot = block * block_size + row):
 * every non-negative slot must be < num_blocks * block_size (else
 * PA_CHECK_SLOT); negative slots are the documented skip.  Uniqueness is not
 * checked.
 */
typedef enum {
  PA_CHECK_BLOCK_ID = 1,
  PA_CHECK_LENGTH = 2,
  PA_CHECK_SLOT = 4,
  PA_CHECK_CHUNK = 8
} pa_check_flag;

pa_status pa_check_block_tables(const int32_t* block_tables, const int32_t* seq_lens,
                                const int32_t* query_start_loc, int32_t num_seqs,
                                int32_t total_q_tokens, int32_t max_blocks_per_seq,
                                int32_t block_size, int32_t num_blocks, int32_t max_seq_len,
                                int32_t* error, void* stream);
pa_status pa_check_slots(const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                         int32_t block_size, int32_t* error, void* stream);

/* Human-readable name of a status code (static storage). */
const char* pa_status_string(pa_status status);

/* Detail message of the last failed call on this thread ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
