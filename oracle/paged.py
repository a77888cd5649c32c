"""The paged KV-cache method, written out plainly in float64 — TEST INFRASTRUCTURE.

Nothing in the HIP library imports or mirrors this file.

Layout of a pool (the reading taken where the pages are silent about heads):
``pool[num_blocks][num_kv_heads][block_size][head_dim]``, one pool for K and
one for V.  The datawhalechina page ("17. vLLM PagedAttention", Step 3 item 1)
gives a single-head pool of shape [num_blocks, block_size, hidden_dim]; the
intelliparadigm page (§2.2 "分页式内存管理设计", the ``Block`` sketch) keeps K
and V as separate per-block arrays of shape [block_size, head_dim].  Adding the
KV-head axis between the block and the token axes keeps each (block, head) tile
contiguous.

Pools are passed as raw element bits plus an element-type name (see
``elements``).  All arithmetic is float64.
"""

from __future__ import annotations

import numpy as np

from .elements import decode_elements, e4m3_encode, int8_encode


def num_blocks(seq_len: int, block_size: int) -> int:
    """Blocks a sequence of ``seq_len`` tokens occupies: ceil(seq_len / block_size).

    datawhalechina page, "参考代码与解析", TODO 2: the block count of a prompt is
    the token count divided by the block size, rounded up, computed in integers.
    """
    if block_size <= 0:
        raise ValueError("block_size must be positive")
    if seq_len <= 0:
        return 0
    return (seq_len + block_size - 1) // block_size


def locate_token(block_table_row, position: int, block_size: int):
    """Physical location of logical token ``position`` of a sequence.

    bogosort page, §7 "PagedAttention 的核心思想" and §8 "Logical Block 与
    Physical Block": tokens form logical blocks, and the block table maps
    logical block i to a physical block.  The token's logical block is
    position // block_size and its offset inside the block is
    position % block_size.  The flat slot index (physical * block_size +
    offset) is the linearisation the scatter's slot mapping uses.

    Returns (physical_block, offset, slot).
    """
    logical = position // block_size
    offset = position % block_size
    physical = int(block_table_row[logical])
    return physical, offset, physical * block_size + offset


def gather_sequence(pool_bits, dtype: str, block_table_row, seq_len: int,
                    block_size: int, block_scales=None) -> np.ndarray:
    """Gather one sequence's cache from the pool into a contiguous array.

    datawhalechina page, Step 2 and "参考代码与解析" TODO 5: take the physical
    blocks the block table names, in table order, join them along the token
    axis into one logically contiguous cache, and keep only the first
    seq_len tokens because the last block may be only partly filled.

    With ``block_scales`` ([num_blocks][num_kv_heads], the int8 cache's
    per-block scales) each block's values are its codes times its scale.

    Returns float64 [num_kv_heads][seq_len][head_dim].
    """
    nb = num_blocks(seq_len, block_size)
    ids = np.asarray(block_table_row[:nb], dtype=np.int64)
    blocks = decode_elements(pool_bits[ids], dtype)        # [nb][H][bs][D]
    if block_scales is not None:
        sc = np.asarray(block_scales, dtype=np.float32).astype(np.float64)[ids]
        blocks = blocks * sc[:, :, None, None]
    heads = blocks.shape[1]
    dim = blocks.shape[3]
    joined = blocks.transpose(1, 0, 2, 3).reshape(heads, nb * block_size, dim)
    return joined[:, :seq_len, :]


def softmax_attention(q_rows: np.ndarray, keys: np.ndarray, values: np.ndarray,
                      scale: float, last_key=None) -> np.ndarray:
    """Textbook scaled-dot-product attention with a two-pass softmax.

    out[r] = sum_j p[r, j] * V[j] / sum_j p[r, j], where
    p[r, j] = exp(s[r, j] - max_j s[r, j]) and s[r, j] = scale * q[r] . K[j].
    With ``last_key`` given, row r may only use keys j <= last_key[r] (the
    causal limit); the others get probability zero.

    q_rows [R][D], keys/values [N][D], all float64; returns [R][D].
    """
    logits = scale * (q_rows @ keys.T)                       # [R][N]
    if last_key is not None:
        j = np.arange(keys.shape[0])[None, :]
        allowed = j <= np.asarray(last_key)[:, None]
        logits = np.where(allowed, logits, -np.inf)
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    return (p @ values) / p.sum(axis=1, keepdims=True)


def decode_attention(q_bits, q_dtype: str, k_pool, v_pool, cache_dtype: str,
                     block_tables, seq_lens, scale: float, block_size: int,
                     num_kv_heads: int, k_scale: float = 1.0,
                     v_scale: float = 1.0, v_cache_dtype: str | None = None,
                     k_block_scales=None, v_block_scales=None) -> np.ndarray:
    """Paged decode attention: one query token per sequence.

    bogosort page §8 (the attention kernel finds each sequence's past K/V
    through the block table) and ybb.press page §2.3 "非连续存储的计算兼容性"
    (attention walks every K/V pair of the sequence, resolving each block
    through the table).  The query of sequence s sits at its last position
    seq_lens[s] - 1 and attends every token 0..seq_lens[s]-1, itself included
    (its own K/V were written to the cache first).  Query head h reads KV head
    h // (Hq / Hkv).  Stored fp8 codes are multiplied by the per-tensor
    k_scale / v_scale; for other element types the scales are applied the
    same way (1.0 leaves them unchanged).  A sequence of length <= 0 yields a
    zero output.  v_cache_dtype names the V pool's element type when it
    differs from the K pool's (the intelliparadigm page §6.1 pairs an fp8 K
    cache with a bf16 V cache); by default both pools hold cache_dtype.
    k_block_scales / v_block_scales ([num_blocks][num_kv_heads]) give the int8
    cache's per-block scales (ybb.press §6.2, INT8 KV cache), applied before
    k_scale / v_scale.

    q_bits [S][Hq][D]; pools [NB][Hkv][bs][D]; block_tables [S][MB];
    seq_lens [S].  Returns float64 [S][Hq][D].
    """
    q = decode_elements(q_bits, q_dtype)
    num_seqs, num_q_heads, head_dim = q.shape
    if num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        n = int(seq_lens[s])
        if n <= 0:
            continue
        keys = gather_sequence(k_pool, cache_dtype, block_tables[s], n, block_size,
                               k_block_scales) * float(k_scale)
        vals = gather_sequence(v_pool, v_cache_dtype or cache_dtype, block_tables[s], n,
                               block_size, v_block_scales) * float(v_scale)
        for h in range(num_q_heads):
            kv = h // group
            out[s, h] = softmax_attention(q[s, h][None, :], keys[kv], vals[kv], scale)[0]
    return out


def prefill_chunk_attention(q_bits, q_dtype: str, query_start_loc, k_pool, v_pool,
                            cache_dtype: str, block_tables, seq_lens, scale: float,
                            block_size: int, num_kv_heads: int,
                            k_scale: float = 1.0, v_scale: float = 1.0,
                            rows=None, k_block_scales=None, v_block_scales=None) -> np.ndarray:
    """Causal attention of one prefill chunk per sequence over its paged context.

    bogosort page §15 "Chunked Prefill" and ai-engineering page "分块预填充保护
    TTFT 尾部": a long prompt's prefill runs as consecutive chunks (about 512
    tokens).  Sequence s has a context of seq_lens[s] tokens whose last
    L = query_start_loc[s+1] - query_start_loc[s] tokens are this chunk (their
    K/V already written to the cache).  Chunk query i therefore sits at
    position seq_lens[s] - L + i and attends keys 0..that position.

    q_bits is [total_q_tokens][Hq][D] with sequence s's chunk in rows
    query_start_loc[s] .. query_start_loc[s+1]-1.  With ``rows`` (a list of
    (token_row, head) pairs) only those outputs are evaluated and the result
    is [len(rows)][D]; otherwise it is float64 [total_q_tokens][Hq][D].
    Scales apply as in decode_attention: per-tensor k_scale / v_scale, and for
    an int8 cache the per-(block, KV head) k_block_scales / v_block_scales
    before them.
    """
    q = decode_elements(q_bits, q_dtype)
    total, num_q_heads, head_dim = q.shape
    group = num_q_heads // num_kv_heads
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    num_seqs = len(qsl) - 1
    gathered = {}

    def context(s):
        if s not in gathered:
            n = int(seq_lens[s])
            gathered[s] = (
                gather_sequence(k_pool, cache_dtype, block_tables[s], n, block_size,
                                k_block_scales) * float(k_scale),
                gather_sequence(v_pool, cache_dtype, block_tables[s], n, block_size,
                                v_block_scales) * float(v_scale),
            )
        return gathered[s]

    def one_head(s, h, token_rows):
        keys, vals = context(s)
        kv = h // group
        chunk = int(qsl[s + 1] - qsl[s])
        last = int(seq_lens[s]) - chunk + (token_rows - qsl[s])
        return softmax_attention(q[token_rows, h, :], keys[kv], vals[kv], scale, last_key=last)

    if rows is not None:
        out = np.zeros((len(rows), head_dim), dtype=np.float64)
        for idx, (t, h) in enumerate(rows):
            s = int(np.searchsorted(qsl, t, side="right") - 1)
            out[idx] = one_head(s, int(h), np.array([t], dtype=np.int64))[0]
        return out

    out = np.zeros((total, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        if qsl[s + 1] <= qsl[s] or int(seq_lens[s]) <= 0:
            continue
        token_rows = np.arange(qsl[s], qsl[s + 1])
        for h in range(num_q_heads):
            out[token_rows, h, :] = one_head(s, h, token_rows)
    return out


def reshape_and_cache(k_pool, v_pool, cache_dtype: str, key_bits, value_bits,
                      src_dtype: str, slot_mapping, block_size: int,
                      k_scale: float = 1.0, v_scale: float = 1.0,
                      v_cache_dtype: str | None = None, k_block_scales=None,
                      v_block_scales=None):
    """Write new tokens' K/V into their pool slots; returns new (k_pool, v_pool).

    datawhalechina page, Step 3 item 3 and Step 4: physical block indices are
    assigned on demand as tokens are generated, and each token's K/V is
    stored in its block.  Token t goes to slot = physical * block_size +
    offset, i.e. block slot // block_size, row slot % block_size, for every KV
    head.  A negative slot means "no slot" and the token is skipped.  When the
    cache holds the same element type as the source, the bits are copied
    unchanged.  An fp8 cache stores e4m3(float32(x) / float32(scale)) — the
    division done once in float32, as the ybb.press page's §6.2 (FP8 KV cache)
    leaves the arithmetic open.  Slots are assumed distinct.  v_cache_dtype
    names the V pool's element type when it differs from the K pool's
    (intelliparadigm page §6.1: fp8 K cache, bf16 V cache).  An int8 cache
    stores int8_encode(x, scale[block][head]) with the per-block scales
    k_block_scales / v_block_scales ([num_blocks][num_kv_heads] float32).

    key_bits/value_bits [T][Hkv][D]; slot_mapping [T] int64.
    """
    k_new = np.array(k_pool, copy=True)
    v_new = np.array(v_pool, copy=True)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    for src, dst, scale, pool_dtype, bsc in ((key_bits, k_new, k_scale, cache_dtype, k_block_scales),
                                             (value_bits, v_new, v_scale, v_cache_dtype or cache_dtype,
                                              v_block_scales)):
        src = np.asarray(src)
        for t, slot in enumerate(slots):
            if slot < 0:
                continue
            blk, row = int(slot // block_size), int(slot % block_size)
            if pool_dtype == src_dtype:
                dst[blk, :, row, :] = src[t]
            elif pool_dtype == "int8":
                x32 = decode_elements(src[t], src_dtype).astype(np.float32)   # [H][D]
                sc = np.asarray(bsc, dtype=np.float32)[blk]                  # [H]
                dst[blk, :, row, :] = int8_encode(x32, sc[:, None])
            elif pool_dtype == "fp8_e4m3":
                x32 = decode_elements(src[t], src_dtype).astype(np.float32)
                q32 = x32 / np.float32(scale)
                dst[blk, :, row, :] = e4m3_encode(q32)
            else:
                raise ValueError(f"unsupported conversion {src_dtype} -> {pool_dtype}")
    return k_new, v_new


def copy_blocks(k_pool, v_pool, pairs):
    """Copy whole blocks (copy-on-write); returns new (k_pool, v_pool).

    ybb.press page §2.2 "Copy-on-Write 与共享前缀": when several sequences
    reference one block, a write to it first duplicates the whole block.  For
    each (src, dst) pair block dst of both pools becomes a copy of block src.
    Destinations are distinct and never a source in the same call.
    """
    k_new = np.array(k_pool, copy=True)
    v_new = np.array(v_pool, copy=True)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_new[dst] = k_pool[src]
        v_new[dst] = v_pool[src]
    return k_new, v_new


def copy_block_rows(k_pool, v_pool, triples):
    """Copy-on-write of partly filled blocks; returns new (k_pool, v_pool).

    bogosort page "五十三：vLLM-PagedAttention" §17 Parallel Sampling: forked
    sequences share the prompt's blocks and write what follows the fork into
    blocks of their own.  When the fork falls inside a block, only the tokens
    before it are carried over: for each (src, dst, n) triple, rows [0, n)
    of every KV head of block dst become those of block src, with n clamped
    to [0, block_size]; every other row keeps its contents.
    """
    k_new = np.array(k_pool, copy=True)
    v_new = np.array(v_pool, copy=True)
    block_size = k_pool.shape[2]
    for src, dst, n in np.asarray(triples, dtype=np.int64).reshape(-1, 3):
        n = min(max(int(n), 0), block_size)
        k_new[dst, :, :n, :] = k_pool[src, :, :n, :]
        v_new[dst, :, :n, :] = v_pool[src, :, :n, :]
    return k_new, v_new


def copy_blocks_layers(k_pools, v_pools, pairs):
    """The same copy-on-write block copies applied in every layer's pools.

    ybb.press page §2.2 "Copy-on-Write 与共享前缀": a fork duplicates each
    shared block, and a model keeps one K and one V cache per layer, so the
    copy is repeated layer by layer.  Returns lists of new pools.
    """
    out_k, out_v = [], []
    for kp, vp in zip(k_pools, v_pools):
        nk, nv = copy_blocks(kp, vp, pairs)
        out_k.append(nk)
        out_v.append(nv)
    return out_k, out_v


def swap_blocks(dst_pool, src_pool, pairs):
    """Block moves between two pools (swap out to CPU memory and back in).

    ybb.press page §三 (Continuous Batching), the preemption bullet: under
    memory pressure the block manager moves blocks to CPU memory and later
    back.  For each (src, dst) pair block dst of a copy of dst_pool becomes
    block src of src_pool.
    """
    out = np.array(dst_pool, copy=True)
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        out[dst] = src_pool[src]
    return out
