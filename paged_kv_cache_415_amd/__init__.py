"""Python binding of libpa.so — paged KV-cache attention on gfx950.

The functions here carry the C entry points' names and only marshal
arguments: torch tensors become device pointers, the current torch stream
becomes the hipStream_t, and a non-zero status becomes an exception.  Every
step of the computation runs in the library's HIP kernels; there is no other
code path.  Importing this module loads the shared library and fails loudly
if it has not been built (``python paged_kv_cache_415_amd/build.py``).

Tensor layouts (all contiguous, on the GPU):
  q, out            [num_seqs or tokens][num_q_heads][head_dim]
  k_pool, v_pool    [num_blocks][num_kv_heads][block_size][head_dim]
  block_tables      int32 [num_seqs][max_blocks_per_seq]
  seq_lens          int32 [num_seqs]
  slot_mapping      int64 [num_tokens]
  block_pairs       int64 [num_pairs][2]
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_DTYPE = {
    torch.float32: 0,
    torch.float16: 1,
    torch.bfloat16: 2,
    torch.float8_e4m3fn: 3,
    torch.int8: 4,
}
STATUS = {0: "PA_OK", 1: "PA_ERR_INVALID_ARG", 2: "PA_ERR_UNSUPPORTED", 3: "PA_ERR_WORKSPACE",
          4: "PA_ERR_HIP", 5: "PA_ERR_OUT_OF_BLOCKS"}


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python paged_kv_cache_415_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, f32, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    lib.pa_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i32, i32,
                                         i32, f32, f32, vp]
    lib.pa_reshape_and_cache_kv.argtypes = [vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, i32,
                                            i32, i32, i32, f32, f32, vp]
    lib.pa_copy_blocks.argtypes = [vp, vp, vp, i32, i64, vp]
    lib.pa_copy_blocks_partial.argtypes = [vp, vp, vp, i32, i32, i32, i64, vp]
    lib.pa_copy_blocks_layers.argtypes = [vp, vp, i32, vp, i32, i64, vp]
    lib.pa_swap_blocks.argtypes = [vp, vp, vp, i32, i64, vp]
    lib.pa_decode_partition_size.argtypes = [i32, i32, i32, i32, i32]
    lib.pa_decode_partition_size.restype = i32
    lib.pa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.pa_decode_workspace_bytes.restype = sz
    dec = [vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, f32, i32,
           vp, sz, vp]
    for name in ("pa_decode", "pa_decode_attention", "pa_decode_reduce"):
        getattr(lib, name).argtypes = dec
        getattr(lib, name).restype = i32
    lib.pa_decode_noalloc.argtypes = dec[:19] + [vp]
    lib.pa_decode_noalloc.restype = i32
    lib.pa_decode_noalloc_max_workspace_bytes.argtypes = []
    lib.pa_decode_noalloc_max_workspace_bytes.restype = sz
    for name in ("pa_decode_kv", "pa_decode_attention_kv", "pa_decode_reduce_kv"):
        getattr(lib, name).argtypes = dec[:16] + [i32] + dec[16:]
        getattr(lib, name).restype = i32
    dec8 = [vp, vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    for name in ("pa_decode_int8", "pa_decode_attention_int8", "pa_decode_reduce_int8"):
        getattr(lib, name).argtypes = dec8
        getattr(lib, name).restype = i32
    lib.pa_reshape_and_cache_int8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32,
                                              i32, i32, vp]
    lib.pa_reshape_and_cache_int8.restype = i32
    app = [vp, vp, vp, vp, i64, i64, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
           f32, f32, i32, vp, sz, vp]
    for name in ("pa_decode_append", "pa_decode_attention_append"):
        getattr(lib, name).argtypes = app
        getattr(lib, name).restype = i32
    lib.pa_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32,
                                     i32, i32, i32, i32, f32, f32, vp]
    lib.pa_prefill_chunk_int8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32,
                                          i32, i32, i32, vp]
    lib.pa_mixed_attention.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32,
                                       i32, vp, vp, f32, i32, i32, i32, i32, i32, i32, f32, f32, i32,
                                       vp, sz, vp]
    lib.pa_mixed_attention_int8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, i32, i32,
                                            i32, vp, vp, vp, vp, f32, i32, i32, i32, i32, i32, i32, vp, sz,
                                            vp]
    lib.pa_check_block_tables.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.pa_check_block_tables.restype = i32
    lib.pa_check_slots.argtypes = [vp, i32, i32, i32, vp, vp]
    lib.pa_check_slots.restype = i32
    lib.pa_status_string.argtypes = [i32]
    lib.pa_status_string.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_probe_read.argtypes = [vp, sz, vp, vp]
    lib.pa_probe_copy.argtypes = [vp, vp, sz, vp]
    for name in ("pa_reshape_and_cache", "pa_reshape_and_cache_kv", "pa_copy_blocks", "pa_copy_blocks_partial",
                 "pa_copy_blocks_layers", "pa_swap_blocks", "pa_prefill_chunk", "pa_prefill_chunk_int8",
                 "pa_mixed_attention", "pa_mixed_attention_int8",
                 "pa_probe_read",
                 "pa_probe_copy"):
        getattr(lib, name).restype = i32
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise PagedAttentionError(status, _lib.pa_last_error().decode())


def _ptr(t, contiguous: bool = True, host_ok: bool = False):
    """Data pointer of a GPU tensor (or, with host_ok, of a CPU tensor: the
    library itself accepts only pinned host memory there)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    if t.device.type != "cuda" and not (host_ok and t.device.type == "cpu"):
        raise ValueError("tensors must be on the GPU")
    return t.data_ptr()


def _dtype(t: torch.Tensor) -> int:
    if t.dtype in (torch.uint8,):          # raw fp8 codes
        return 3
    try:
        return PA_DTYPE[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def pa_reshape_and_cache(key, value, k_pool, v_pool, slot_mapping, k_scale: float = 1.0,
                         v_scale: float = 1.0, stream=None) -> None:
    """Scatter key/value [T][Hkv][D] into pool slots (see pa.h)."""
    _scatter(_lib.pa_reshape_and_cache, key, value, k_pool, v_pool, slot_mapping, k_scale, v_scale,
             stream, mixed=False)


def pa_reshape_and_cache_kv(key, value, k_pool, v_pool, slot_mapping, k_scale: float = 1.0,
                            v_scale: float = 1.0, stream=None) -> None:
    """pa_reshape_and_cache with the K and V pool types taken apart (fp8 K
    cache beside a V cache of the source type; see pa.h)."""
    _scatter(_lib.pa_reshape_and_cache_kv, key, value, k_pool, v_pool, slot_mapping, k_scale,
             v_scale, stream, mixed=True)


def _scatter(fn, key, value, k_pool, v_pool, slot_mapping, k_scale, v_scale, stream, mixed):
    if not mixed and _dtype(k_pool) != _dtype(v_pool):
        raise ValueError("K and V pools of different types need pa_reshape_and_cache_kv")
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    nb, hkv, bs, d = k_pool.shape
    t = slot_mapping.shape[0]
    for x in (key, value):      # token rows may be strided (e.g. views into a fused QKV buffer)
        if x.dim() != 3 or x.shape[1:] != (hkv, d) or x.stride(2) != 1 or x.stride(1) != d:
            raise ValueError("key/value must be [T][num_kv_heads][head_dim] with dense rows")
    key_stride = key.stride(0) if t > 0 else 0
    value_stride = value.stride(0) if t > 0 else 0
    if v_pool.shape[1:] != k_pool.shape[1:] or v_pool.shape[0] < nb:
        raise ValueError("V pool shape does not match the K pool")
    types = [_dtype(k_pool), _dtype(v_pool)] if mixed else [_dtype(k_pool)]
    _check(fn(_ptr(key, False), _ptr(value, False), _ptr(k_pool), _ptr(v_pool), _ptr(slot_mapping),
              t, key_stride, value_stride, nb, hkv, d, bs, _dtype(key), *types, k_scale, v_scale,
              _stream(stream)))


def _scales(t, k_pool):
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    if t.dtype != torch.float32 or tuple(t.shape) != (nb, hkv):
        raise ValueError("per-block scales must be float32 [num_blocks][num_kv_heads]")
    return _ptr(t)


def pa_reshape_and_cache_int8(key, value, k_pool, v_pool, k_scales, v_scales, slot_mapping,
                              stream=None) -> None:
    """Scatter key/value into an int8 cache with per-(block, KV head) scales (see pa.h)."""
    if slot_mapping.dtype != torch.int64:
        raise TypeError("slot_mapping must be int64")
    if k_pool.dtype != torch.int8 or v_pool.dtype != torch.int8:
        raise TypeError("int8 pools expected")
    nb, hkv, bs, d = k_pool.shape
    if v_pool.shape != k_pool.shape:
        raise ValueError("V pool shape does not match the K pool")
    t = slot_mapping.shape[0]
    for x in (key, value):
        if x.dim() != 3 or x.shape[1:] != (hkv, d) or x.stride(2) != 1 or x.stride(1) != d:
            raise ValueError("key/value must be [T][num_kv_heads][head_dim] with dense rows")
    _check(_lib.pa_reshape_and_cache_int8(
        _ptr(key, False), _ptr(value, False), _ptr(k_pool), _ptr(v_pool), _scales(k_scales, k_pool),
        _scales(v_scales, k_pool), _ptr(slot_mapping), t, key.stride(0) if t > 0 else 0,
        value.stride(0) if t > 0 else 0, nb, hkv, d, bs, _dtype(key), _stream(stream)))


def _decode_int8_call(fn, out, q, k_pool, v_pool, k_scales, v_scales, block_tables, seq_lens, scale,
                      max_seq_len, partition_size, workspace, stream):
    s, hq, d = q.shape
    _, hkv, bs, _ = k_pool.shape
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if k_pool.dtype != torch.int8 or v_pool.dtype != torch.int8 or v_pool.shape != k_pool.shape:
        raise TypeError("int8 pools of one shape expected")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(_ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _scales(k_scales, k_pool),
              _scales(v_scales, k_pool), _ptr(block_tables), _ptr(seq_lens), float(scale), bs, s,
              hq, hkv, d, block_tables.shape[1], int(max_seq_len), _dtype(q), int(partition_size),
              _ptr(workspace), wbytes, _stream(stream)))


def pa_decode_int8(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, seq_lens,
                   scale: float, max_seq_len: int = 0, partition_size: int = 0, workspace=None,
                   stream=None) -> None:
    """Decode attention over an int8 cache with per-(block, KV head) scales (see pa.h)."""
    _decode_int8_call(_lib.pa_decode_int8, out, q, k_pool, v_pool, k_scales, v_scales, block_tables,
                      seq_lens, scale, max_seq_len, partition_size, workspace, stream)


def pa_decode_attention_int8(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, seq_lens,
                             scale: float, max_seq_len: int = 0, partition_size: int = 0,
                             workspace=None, stream=None) -> None:
    """First stage of pa_decode_int8."""
    _decode_int8_call(_lib.pa_decode_attention_int8, out, q, k_pool, v_pool, k_scales, v_scales,
                      block_tables, seq_lens, scale, max_seq_len, partition_size, workspace, stream)


def pa_decode_reduce_int8(out, q, k_pool, v_pool, k_scales, v_scales, block_tables, seq_lens,
                          scale: float, max_seq_len: int = 0, partition_size: int = 0,
                          workspace=None, stream=None) -> None:
    """Second stage of pa_decode_int8."""
    _decode_int8_call(_lib.pa_decode_reduce_int8, out, q, k_pool, v_pool, k_scales, v_scales,
                      block_tables, seq_lens, scale, max_seq_len, partition_size, workspace, stream)


def pa_copy_blocks(k_pool, v_pool, block_pairs, stream=None) -> None:
    """Copy whole blocks (src, dst) pairs in both pools (see pa.h)."""
    if block_pairs.dtype != torch.int64:
        raise TypeError("block_pairs must be int64")
    block_bytes = k_pool[0].numel() * k_pool.element_size()
    _check(_lib.pa_copy_blocks(_ptr(k_pool), _ptr(v_pool), _ptr(block_pairs),
                               block_pairs.shape[0], block_bytes, _stream(stream)))


def pa_copy_blocks_partial(k_pool, v_pool, block_triples, stream=None) -> None:
    """Copy rows [0, n) of every KV head of block src into block dst, for each
    (src, dst, n) triple, in both pools (see pa.h)."""
    if block_triples.dtype != torch.int64:
        raise TypeError("block_triples must be int64")
    _, hkv, bs, d = k_pool.shape
    _check(_lib.pa_copy_blocks_partial(_ptr(k_pool), _ptr(v_pool), _ptr(block_triples),
                                       block_triples.shape[0], hkv, bs, d * k_pool.element_size(),
                                       _stream(stream)))


def layer_pool_pointers(pools, device) -> torch.Tensor:
    """Device array of the pools' addresses, as pa_copy_blocks_layers takes them
    (build it once for a fixed set of layer caches)."""
    shape, dtype = pools[0].shape, pools[0].dtype
    for t in pools:
        if t.shape != shape or t.dtype != dtype or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("every pool must be a contiguous GPU tensor of one shape and dtype")
    return torch.tensor([t.data_ptr() for t in pools], dtype=torch.int64, device=device)


def pa_copy_blocks_layers(k_pools, v_pools, block_pairs, stream=None, block_bytes=None) -> None:
    """Apply the same whole-block (src, dst) copies to the K and V pools of
    every layer in one launch (see pa.h).  k_pools, v_pools: lists of pools of
    one shape and dtype, or address arrays from layer_pool_pointers (then
    block_bytes, the bytes of one block of one pool, is required)."""
    if block_pairs.dtype != torch.int64:
        raise TypeError("block_pairs must be int64")
    if isinstance(k_pools, torch.Tensor):
        if not isinstance(v_pools, torch.Tensor) or k_pools.dtype != torch.int64 or block_bytes is None:
            raise ValueError("address arrays need int64 tensors for both pools and block_bytes")
        kp, vp = k_pools, v_pools
    else:
        if len(k_pools) != len(v_pools):
            raise ValueError("k_pools and v_pools differ in length")
        if not k_pools:
            return
        kp = layer_pool_pointers(k_pools, block_pairs.device)
        vp = layer_pool_pointers(v_pools, block_pairs.device)
        if k_pools[0].shape != v_pools[0].shape or k_pools[0].dtype != v_pools[0].dtype:
            raise ValueError("K and V pools differ in shape or dtype")
        block_bytes = k_pools[0][0].numel() * k_pools[0].element_size()
    if kp.numel() != vp.numel():
        raise ValueError("k_pools and v_pools differ in length")
    _check(_lib.pa_copy_blocks_layers(_ptr(kp), _ptr(vp), kp.numel(), _ptr(block_pairs),
                                      block_pairs.shape[0], block_bytes, _stream(stream)))
    if stream is not None:
        # the address arrays may be freed when this call returns: keep them
        # alive for the launch on a stream other than the allocator's
        kp.record_stream(stream)
        vp.record_stream(stream)


def pa_swap_blocks(dst_pool, src_pool, block_pairs, stream=None) -> None:
    """Block dst of dst_pool = block src of src_pool for each (src, dst) pair;
    either pool may be a pinned CPU tensor (see pa.h)."""
    if block_pairs.dtype != torch.int64:
        raise TypeError("block_pairs must be int64")
    if dst_pool.dtype != src_pool.dtype or dst_pool.shape[1:] != src_pool.shape[1:]:
        raise ValueError("pools must have the same dtype and block shape")
    block_bytes = dst_pool[0].numel() * dst_pool.element_size()
    _check(_lib.pa_swap_blocks(_ptr(dst_pool, host_ok=True), _ptr(src_pool, host_ok=True), _ptr(block_pairs),
                               block_pairs.shape[0], block_bytes, _stream(stream)))


def pa_decode_partition_size(num_seqs: int, num_kv_heads: int, block_size: int, max_seq_len: int,
                             partition_size: int = 0) -> int:
    return _lib.pa_decode_partition_size(num_seqs, num_kv_heads, block_size, max_seq_len,
                                         partition_size)


def pa_decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                              block_size: int, max_seq_len: int, partition_size: int = 0) -> int:
    return _lib.pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                          max_seq_len, partition_size)


def decode_workspace(q, k_pool, max_seq_len: int, partition_size: int = 0):
    """Allocate a workspace tensor for pa_decode (torch caching allocator)."""
    s, hq, d = q.shape
    _, hkv, bs, _ = k_pool.shape
    n = pa_decode_workspace_bytes(s, hq, hkv, d, bs, max_seq_len, partition_size)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=q.device)


def _decode_call(fn, out, q, k_pool, v_pool, block_tables, seq_lens, scale, max_seq_len,
                 k_scale, v_scale, partition_size, workspace, stream, mixed=False):
    s, hq, d = q.shape
    _, hkv, bs, _ = k_pool.shape
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if v_pool.shape[1:] != k_pool.shape[1:]:
        raise ValueError("V pool shape does not match the K pool")
    if not mixed and _dtype(k_pool) != _dtype(v_pool):
        raise ValueError("K and V pools of different types need pa_decode_kv")
    types = [_dtype(k_pool), _dtype(v_pool)] if mixed else [_dtype(k_pool)]
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(_ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables), _ptr(seq_lens),
              float(scale), bs, s, hq, hkv, d, block_tables.shape[1], int(max_seq_len),
              _dtype(q), *types, float(k_scale), float(v_scale), int(partition_size),
              _ptr(workspace), wbytes, _stream(stream)))


def pa_decode(out, q, k_pool, v_pool, block_tables, seq_lens, scale: float, max_seq_len: int = 0,
              k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 0,
              workspace=None, stream=None) -> None:
    """Decode attention of one query per sequence over its paged context (see pa.h)."""
    _decode_call(_lib.pa_decode, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                 max_seq_len, k_scale, v_scale, partition_size, workspace, stream)


def pa_decode_noalloc(out, q, k_pool, v_pool, block_tables, seq_lens, scale: float,
                      max_seq_len: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
                      partition_size: int = 0, stream=None) -> None:
    """pa_decode without a workspace argument: the split partials go to the
    library's own device array (for callers that cannot allocate; see pa.h)."""
    s, hq, d = q.shape
    _, hkv, bs, _ = k_pool.shape
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    if v_pool.shape[1:] != k_pool.shape[1:] or _dtype(k_pool) != _dtype(v_pool):
        raise ValueError("K and V pools must match in block shape and type")
    _check(_lib.pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
                                  _ptr(seq_lens), float(scale), bs, s, hq, hkv, d,
                                  block_tables.shape[1], int(max_seq_len), _dtype(q), _dtype(k_pool),
                                  float(k_scale), float(v_scale), int(partition_size),
                                  _stream(stream)))


def pa_decode_noalloc_max_workspace_bytes() -> int:
    return _lib.pa_decode_noalloc_max_workspace_bytes()


def pa_decode_kv(out, q, k_pool, v_pool, block_tables, seq_lens, scale: float, max_seq_len: int = 0,
                 k_scale: float = 1.0, v_scale: float = 1.0, partition_size: int = 0,
                 workspace=None, stream=None) -> None:
    """pa_decode with the K and V pool types taken apart (fp8 K cache beside
    a V cache of the query type; see pa.h)."""
    _decode_call(_lib.pa_decode_kv, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                 max_seq_len, k_scale, v_scale, partition_size, workspace, stream, mixed=True)


def pa_decode_attention_kv(out, q, k_pool, v_pool, block_tables, seq_lens, scale: float,
                           max_seq_len: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
                           partition_size: int = 0, workspace=None, stream=None) -> None:
    """First stage of pa_decode_kv (attention kernel only)."""
    _decode_call(_lib.pa_decode_attention_kv, out, q, k_pool, v_pool, block_tables, seq_lens,
                 scale, max_seq_len, k_scale, v_scale, partition_size, workspace, stream, mixed=True)


def pa_decode_reduce_kv(out, q, k_pool, v_pool, block_tables, seq_lens, scale: float,
                        max_seq_len: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
                        partition_size: int = 0, workspace=None, stream=None) -> None:
    """Second stage of pa_decode_kv."""
    _decode_call(_lib.pa_decode_reduce_kv, out, q, k_pool, v_pool, block_tables, seq_lens,
                 scale, max_seq_len, k_scale, v_scale, partition_size, workspace, stream, mixed=True)


def _append_call(fn, out, q, new_k, new_v, k_pool, v_pool, block_tables, seq_lens, scale,
                 max_seq_len, k_scale, v_scale, partition_size, workspace, stream):
    s, hq, d = q.shape
    _, hkv, bs, _ = k_pool.shape
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_tables and seq_lens must be int32")
    for x in (new_k, new_v):
        if x.dim() != 3 or tuple(x.shape) != (s, hkv, d) or x.stride(2) != 1 or x.stride(1) != d:
            raise ValueError("new_k/new_v must be [num_seqs][num_kv_heads][head_dim] with dense rows")
    if _dtype(v_pool) != _dtype(k_pool):
        raise ValueError("K and V pools must have one type")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(_ptr(out), _ptr(q), _ptr(new_k, False), _ptr(new_v, False),
              new_k.stride(0) if s > 0 else 0, new_v.stride(0) if s > 0 else 0, _ptr(k_pool),
              _ptr(v_pool), _ptr(block_tables), _ptr(seq_lens), float(scale), bs, s, hq, hkv, d,
              block_tables.shape[1], int(max_seq_len), _dtype(q), _dtype(k_pool), float(k_scale),
              float(v_scale), int(partition_size), _ptr(workspace), wbytes, _stream(stream)))


def pa_decode_append(out, q, new_k, new_v, k_pool, v_pool, block_tables, seq_lens, scale: float,
                     max_seq_len: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
                     partition_size: int = 0, workspace=None, stream=None) -> None:
    """Scatter of each sequence's newest token plus decode, in one kernel (see pa.h)."""
    _append_call(_lib.pa_decode_append, out, q, new_k, new_v, k_pool, v_pool, block_tables,
                 seq_lens, scale, max_seq_len, k_scale, v_scale, partition_size, workspace, stream)


def pa_decode_attention_append(out, q, new_k, new_v, k_pool, v_pool, block_tables, seq_lens,
                               scale: float, max_seq_len: int = 0, k_scale: float = 1.0,
                               v_scale: float = 1.0, partition_size: int = 0, workspace=None,
                               stream=None) -> None:
    """First stage of pa_decode_append (pa_decode_reduce completes it)."""
    _append_call(_lib.pa_decode_attention_append, out, q, new_k, new_v, k_pool, v_pool,
                 block_tables, seq_lens, scale, max_seq_len, k_scale, v_scale, partition_size,
                 workspace, stream)


def pa_decode_attention(out, q, k_pool, v_pool, block_tables, seq_lens, scale: float,
                        max_seq_len: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
                        partition_size: int = 0, workspace=None, stream=None) -> None:
    """First stage of pa_decode (attention kernel only)."""
    _decode_call(_lib.pa_decode_attention, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                 max_seq_len, k_scale, v_scale, partition_size, workspace, stream)


def pa_decode_reduce(out, q, k_pool, v_pool, block_tables, seq_lens, scale: float,
                     max_seq_len: int = 0, k_scale: float = 1.0, v_scale: float = 1.0,
                     partition_size: int = 0, workspace=None, stream=None) -> None:
    """Second stage of pa_decode (log-sum-exp merge of split partials)."""
    _decode_call(_lib.pa_decode_reduce, out, q, k_pool, v_pool, block_tables, seq_lens, scale,
                 max_seq_len, k_scale, v_scale, partition_size, workspace, stream)


def pa_prefill_chunk(out, q, query_start_loc, k_pool, v_pool, block_tables, seq_lens,
                     scale: float, max_q_len: int, k_scale: float = 1.0, v_scale: float = 1.0,
                     stream=None) -> None:
    """Causal attention of one chunk per sequence over its paged context (see pa.h)."""
    t, hq, d = q.shape
    _, hkv, bs, _ = k_pool.shape
    if _dtype(v_pool) != _dtype(k_pool) or v_pool.shape[1:] != k_pool.shape[1:]:
        raise ValueError("K and V pools must have one type and block shape")
    num_seqs = query_start_loc.shape[0] - 1
    _check(_lib.pa_prefill_chunk(_ptr(out), _ptr(q), _ptr(query_start_loc), _ptr(k_pool),
                                 _ptr(v_pool), _ptr(block_tables), _ptr(seq_lens), float(scale),
                                 bs, num_seqs, t, int(max_q_len), hq, hkv, d,
                                 block_tables.shape[1], _dtype(q), _dtype(k_pool),
                                 float(k_scale), float(v_scale), _stream(stream)))


def pa_prefill_chunk_int8(out, q, query_start_loc, k_pool, v_pool, k_scales, v_scales, block_tables,
                          seq_lens, scale: float, max_q_len: int, stream=None) -> None:
    """pa_prefill_chunk over an INT8 cache with per-(block, KV head) scales (see pa.h)."""
    t, hq, d = q.shape
    _, hkv, bs, _ = k_pool.shape
    if k_pool.dtype != torch.int8 or v_pool.dtype != torch.int8 or v_pool.shape[1:] != k_pool.shape[1:]:
        raise ValueError("K and V pools must be int8 with one block shape")
    _scales(k_scales, k_pool)
    _scales(v_scales, k_pool)
    _check(_lib.pa_prefill_chunk_int8(_ptr(out), _ptr(q), _ptr(query_start_loc), _ptr(k_pool), _ptr(v_pool),
                                      _ptr(k_scales), _ptr(v_scales), _ptr(block_tables), _ptr(seq_lens),
                                      float(scale), bs, query_start_loc.shape[0] - 1, t, int(max_q_len), hq,
                                      hkv, d, block_tables.shape[1], _dtype(q), _stream(stream)))


def pa_mixed_attention(prefill_out, prefill_q, query_start_loc, prefill_block_tables, prefill_seq_lens,
                       max_q_len: int, decode_out, decode_q, decode_block_tables, decode_seq_lens,
                       max_seq_len: int, k_pool, v_pool, scale: float, k_scale: float = 1.0,
                       v_scale: float = 1.0, partition_size: int = 0, workspace=None,
                       stream=None) -> None:
    """The prefill chunks and the decodes of one step in one launch (see pa.h);
    the workspace is decode_workspace(decode_q, k_pool, max_seq_len, partition_size)."""
    t, hq, d = prefill_q.shape
    s, hq_d, d_d = decode_q.shape
    _, hkv, bs, _ = k_pool.shape
    if (hq_d, d_d) != (hq, d) or _dtype(decode_q) != _dtype(prefill_q):
        raise ValueError("prefill and decode queries differ in heads, head size or type")
    if _dtype(v_pool) != _dtype(k_pool) or v_pool.shape[1:] != k_pool.shape[1:]:
        raise ValueError("K and V pools must have one type and block shape")
    for a in (query_start_loc, prefill_block_tables, prefill_seq_lens, decode_block_tables, decode_seq_lens):
        if a.dtype != torch.int32:
            raise TypeError("offsets, block tables and lengths must be int32")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pa_mixed_attention(
        _ptr(prefill_out), _ptr(prefill_q), _ptr(query_start_loc), _ptr(prefill_block_tables),
        _ptr(prefill_seq_lens), query_start_loc.shape[0] - 1, t, int(max_q_len),
        prefill_block_tables.shape[1], _ptr(decode_out), _ptr(decode_q), _ptr(decode_block_tables),
        _ptr(decode_seq_lens), s, decode_block_tables.shape[1], int(max_seq_len), _ptr(k_pool),
        _ptr(v_pool), float(scale), bs, hq, hkv, d, _dtype(prefill_q), _dtype(k_pool), float(k_scale),
        float(v_scale), int(partition_size), _ptr(workspace), wbytes, _stream(stream)))


def pa_mixed_attention_int8(prefill_out, prefill_q, query_start_loc, prefill_block_tables, prefill_seq_lens,
                            max_q_len: int, decode_out, decode_q, decode_block_tables, decode_seq_lens,
                            max_seq_len: int, k_pool, v_pool, k_scales, v_scales, scale: float,
                            partition_size: int = 0, workspace=None, stream=None) -> None:
    """pa_mixed_attention over an INT8 cache with per-(block, KV head) scales (see pa.h)."""
    t, hq, d = prefill_q.shape
    s, hq_d, d_d = decode_q.shape
    _, hkv, bs, _ = k_pool.shape
    if (hq_d, d_d) != (hq, d) or _dtype(decode_q) != _dtype(prefill_q):
        raise ValueError("prefill and decode queries differ in heads, head size or type")
    if k_pool.dtype != torch.int8 or v_pool.dtype != torch.int8 or v_pool.shape[1:] != k_pool.shape[1:]:
        raise ValueError("K and V pools must be int8 with one block shape")
    _scales(k_scales, k_pool)
    _scales(v_scales, k_pool)
    for a in (query_start_loc, prefill_block_tables, prefill_seq_lens, decode_block_tables, decode_seq_lens):
        if a.dtype != torch.int32:
            raise TypeError("offsets, block tables and lengths must be int32")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.pa_mixed_attention_int8(
        _ptr(prefill_out), _ptr(prefill_q), _ptr(query_start_loc), _ptr(prefill_block_tables),
        _ptr(prefill_seq_lens), query_start_loc.shape[0] - 1, t, int(max_q_len),
        prefill_block_tables.shape[1], _ptr(decode_out), _ptr(decode_q), _ptr(decode_block_tables),
        _ptr(decode_seq_lens), s, decode_block_tables.shape[1], int(max_seq_len), _ptr(k_pool),
        _ptr(v_pool), _ptr(k_scales), _ptr(v_scales), float(scale), bs, hq, hkv, d, _dtype(prefill_q),
        int(partition_size), _ptr(workspace), wbytes, _stream(stream)))


CHECK_FLAGS = {"block_id": 1, "length": 2, "slot": 4, "chunk": 8}


def pa_check_block_tables(block_tables, seq_lens, num_blocks: int, block_size: int, error,
                          max_seq_len: int = 0, query_start_loc=None, stream=None) -> None:
    """Check block ids, lengths (and chunk offsets) on the device; the result
    lands in ``error`` (int32 [3] on the GPU: flags, count, first index)."""
    if block_tables.dtype != torch.int32 or seq_lens.dtype != torch.int32 or error.dtype != torch.int32:
        raise TypeError("block_tables, seq_lens and error must be int32")
    if error.numel() < 3:
        raise ValueError("error needs three int32")
    s = seq_lens.shape[0]
    total = 0
    if query_start_loc is not None:
        if query_start_loc.dtype != torch.int32 or query_start_loc.shape[0] != s + 1:
            raise ValueError("query_start_loc must be int32 [num_seqs + 1]")
        total = int(query_start_loc[-1].item()) if s > 0 else 0
    _check(_lib.pa_check_block_tables(_ptr(block_tables), _ptr(seq_lens), _ptr(query_start_loc), s,
                                      total, block_tables.shape[1], int(block_size), int(num_blocks),
                                      int(max_seq_len), _ptr(error), _stream(stream)))


def pa_check_slots(slot_mapping, num_blocks: int, block_size: int, error, stream=None) -> None:
    """Check that every non-negative slot lies inside the pool; the result
    lands in ``error`` (int32 [3] on the GPU)."""
    if slot_mapping.dtype != torch.int64 or error.dtype != torch.int32:
        raise TypeError("slot_mapping must be int64 and error int32")
    _check(_lib.pa_check_slots(_ptr(slot_mapping), slot_mapping.shape[0], int(num_blocks),
                               int(block_size), _ptr(error), _stream(stream)))


def pa_probe_read(src, sink, stream=None) -> None:
    _check(_lib.pa_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                              _stream(stream)))


def pa_probe_copy(dst, src, stream=None) -> None:
    _check(_lib.pa_probe_copy(_ptr(dst), _ptr(src), src.numel() * src.element_size(),
                              _stream(stream)))


__all__ = [
    "pa_reshape_and_cache", "pa_reshape_and_cache_kv", "pa_decode_kv", "pa_decode_attention_kv",
    "pa_decode_reduce_kv", "pa_reshape_and_cache_int8", "pa_decode_int8", "pa_decode_attention_int8",
    "pa_decode_reduce_int8", "pa_decode_append", "pa_decode_attention_append", "pa_copy_blocks", "pa_copy_blocks_partial", "pa_copy_blocks_layers",
    "layer_pool_pointers",
    "pa_swap_blocks", "pa_decode", "pa_decode_noalloc", "pa_decode_noalloc_max_workspace_bytes",
    "pa_decode_attention",
    "pa_decode_reduce", "pa_prefill_chunk", "pa_prefill_chunk_int8", "pa_mixed_attention",
    "pa_mixed_attention_int8", "pa_decode_partition_size",
    "pa_decode_workspace_bytes", "decode_workspace", "pa_probe_read", "pa_probe_copy",
    "pa_check_block_tables", "pa_check_slots", "CHECK_FLAGS",
    "PagedAttentionError", "library", "LIB_PATH",
]

from .blocks import BlockManager, OutOfBlocks  # noqa: E402  (needs the names above)

__all__ += ["BlockManager", "OutOfBlocks"]
