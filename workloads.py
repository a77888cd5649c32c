"""Seeded synthetic inputs for the paged KV-cache attention path.

This module draws random numbers and lays them out in the shapes the library
consumes.  It holds none of the attention arithmetic: no softmax, no dot
products, no fp8 encoder of its own (fp8 pool contents come from torch's CPU
cast to ``float8_e4m3fn``).  Both the HIP path and the CPU oracle read the
arrays produced here; nothing here reads either of them.

Host-side block management (free list, reference counts, fork, copy-on-write
plan, OOM) also lives here, because the workloads need it to build block
tables.  It follows the datawhalechina page "17. vLLM PagedAttention"
(Step 4 and "参考代码与解析": allocate ceil(len / block_size) blocks for a prompt,
one more block when a decode step crosses a block boundary, raise "OOM" when
the free list runs short) and the ybb.press page "vLLM 与 LLM 推理部署实战"
(§2.1 block table + free list; §2.2 reference counts and copy-on-write).

Element storage: every tensor is a numpy array of the element's raw bits
(f32 -> uint32, f16/bf16 -> uint16, fp8_e4m3 -> uint8).  Pools are
[num_blocks][num_kv_heads][block_size][head_dim].  Slots that hold no token
are NaN-poisoned so that a kernel reading them shows up as NaN.
"""

from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np
import torch

BITS_DTYPE = {"f32": np.uint32, "f16": np.uint16, "bf16": np.uint16, "fp8_e4m3": np.uint8,
              "int8": np.uint8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8_e4m3": 1, "int8": 1}
# int8 has no NaN: unwritten slots hold -128, a code the quantiser never writes
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "fp8_e4m3": 0x7F, "int8": 0x80}
TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "fp8_e4m3": torch.float8_e4m3fn, "int8": torch.int8}
TORCH_BITS = {"f32": torch.int32, "f16": torch.int16, "bf16": torch.int16, "fp8_e4m3": torch.uint8,
              "int8": torch.int8}
INT8_MAX = 127.0
FP8_MAX = 448.0


def to_bits(x_f32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type (torch CPU cast, RNE) -> raw bits."""
    x = np.ascontiguousarray(x_f32, dtype=np.float32)
    if dtype == "f32":
        return x.view(np.uint32).copy()
    t = torch.from_numpy(x)
    if dtype == "fp8_e4m3":
        t = t.clamp(-FP8_MAX, FP8_MAX)
    return t.to(TORCH_DTYPE[dtype]).view(TORCH_BITS[dtype]).numpy().view(BITS_DTYPE[dtype]).copy()


def bits_to_torch(bits: np.ndarray, dtype: str) -> torch.Tensor:
    """View raw bits as a torch CPU tensor of the element type (no copy of values)."""
    arr = np.ascontiguousarray(bits)
    signed = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16,
              np.dtype(np.uint8): np.uint8}[arr.dtype]
    return torch.from_numpy(arr.view(signed)).view(TORCH_DTYPE[dtype])


def bits_to_device(bits: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Upload raw bits and view them on the device as the element type."""
    arr = np.ascontiguousarray(bits)
    signed = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16,
              np.dtype(np.uint8): np.uint8}[arr.dtype]
    return torch.from_numpy(arr.view(signed)).to(device).view(TORCH_DTYPE[dtype])


def torch_to_bits(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Raw bits of a (CPU or device) torch tensor of the element type."""
    return t.detach().cpu().contiguous().view(TORCH_BITS[dtype]).numpy().view(BITS_DTYPE[dtype]).copy()


def blocks_for(num_tokens: int, block_size: int) -> int:
    """Blocks needed to hold num_tokens tokens (integer ceiling)."""
    return -(-num_tokens // block_size) if num_tokens > 0 else 0


class BlockManager:
    """Free list + reference counts for a pool of physical KV blocks.

    ``order`` is the order in which free blocks are handed out (the pages'
    exercise pops the lowest index first; the workloads pass a seeded
    permutation so that physical IDs are scattered).
    """

    def __init__(self, num_blocks: int, block_size: int, order=None):
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(range(num_blocks)) if order is None else [int(b) for b in order]
        self.ref = np.zeros(num_blocks, dtype=np.int64)

    def _take(self) -> int:
        if not self.free:
            raise RuntimeError("OOM")
        b = self.free.pop(0)
        self.ref[b] = 1
        return b

    def allocate(self, num_tokens: int) -> list:
        """Blocks for a new prompt of num_tokens tokens (all or nothing)."""
        need = blocks_for(num_tokens, self.block_size)
        if len(self.free) < need:
            raise RuntimeError("OOM")
        return [self._take() for _ in range(need)]

    def grow(self, table: list, new_len: int) -> None:
        """Append blocks so that the table covers new_len tokens."""
        while blocks_for(new_len, self.block_size) > len(table):
            table.append(self._take())

    def fork(self, table: list) -> list:
        """A new sequence sharing every block of ``table`` (reference counts +1)."""
        for b in table:
            self.ref[b] += 1
        return list(table)

    def copy_on_write(self, table: list, logical: int):
        """Give ``table`` a private copy of logical block ``logical`` if it is shared.

        Returns the (src, dst) pair the device copy must perform, or None.
        """
        b = table[logical]
        if self.ref[b] <= 1:
            return None
        dst = self._take()
        self.ref[b] -= 1
        table[logical] = dst
        return (b, dst)

    def release(self, table: list) -> None:
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        table.clear()


# ---------------------------------------------------------------------------
# Workload specifications
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class DecodeSpec:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q_dtype: str
    cache_dtype: str
    lens: tuple            # ("fixed", values) | ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
    pool: tuple            # ("fixed", num_blocks) | ("factor", f)
    value_std: float
    max_len: int           # largest length the distribution allows (sizes the block table)
    partition_size: int = 0   # 0 = library's choice
    per_tensor_fp8_scale: bool = False
    description: str = ""
    v_cache_dtype: str | None = None   # V pool type when it differs from the K pool's
    seed_name: str | None = None       # draw lengths and block order from another workload's stream

    @property
    def v_dtype(self) -> str:
        return self.v_cache_dtype or self.cache_dtype

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def max_blocks_per_seq(self) -> int:
        return blocks_for(self.max_len, self.block_size)


DECODE_SPECS = {
    "tiny_f32": DecodeSpec(
        "tiny_f32", 4, 2, 2, 64, 16, "f32", "f32", ("fixed", (1, 17, 33, 64)),
        ("fixed", 64), 1.0, 64,
        description="4 sequences of lengths 1/17/33/64, 2 q / 2 KV heads, head_dim 64, "
                    "block 16, 64-block pool, fp32"),
    "llama2_7b_mha_f16": DecodeSpec(
        "llama2_7b_mha_f16", 64, 32, 32, 128, 16, "f16", "f16", ("uniform", 128, 2048),
        ("fixed", 8192), 0.5, 2048,
        description="Llama-2-7B-shaped layer: batch 64, 32/32 heads, head_dim 128, block 16, "
                    "lens U[128,2048], 8192-block pool, fp16, values N(0,1)*0.5"),
    "llama3_8b_gqa_bf16": DecodeSpec(
        "llama3_8b_gqa_bf16", 256, 32, 8, 128, 16, "bf16", "bf16",
        ("lognormal", 1200.0, 0.8, 16, 8192), ("factor", 1.1), 1.0, 8192,
        description="Llama-3-8B-shaped GQA layer: batch 256, 32/8 heads, head_dim 128, block 16, "
                    "lens lognormal(median 1200, sigma 0.8) in [16,8192], pool 1.1x, bf16"),
    "llama3_70b_fp8kv": DecodeSpec(
        "llama3_70b_fp8kv", 128, 64, 8, 128, 16, "bf16", "fp8_e4m3",
        ("lognormal", 1500.0, 0.8, 16, 8192), ("factor", 1.1), 1.0, 8192,
        partition_size=512, per_tensor_fp8_scale=True,
        description="70B-shaped layer on one GPU: 128 sequences, 64/8 heads, head_dim 128, block 16, "
                    "lens lognormal(median 1500, sigma 0.8) in [16,8192], fp8 e4m3 KV with "
                    "per-tensor scales, bf16 q, 512-token split-KV partitions"),
    # One GPU's share of the 70B-shaped layer under 8-way tensor parallelism (KV
    # heads split across GPUs): the same sequences, lengths and block order, one
    # KV head and its 8 query heads.
    "llama3_70b_fp8kv_tp8": DecodeSpec(
        "llama3_70b_fp8kv_tp8", 128, 8, 1, 128, 16, "bf16", "fp8_e4m3",
        ("lognormal", 1500.0, 0.8, 16, 8192), ("factor", 1.1), 1.0, 8192,
        partition_size=512, per_tensor_fp8_scale=True, seed_name="llama3_70b_fp8kv",
        description="one GPU's share of the 70B-shaped layer under 8-way tensor parallelism: "
                    "the same 128 sequences and lengths, 1 KV head and its 8 query heads, "
                    "head_dim 128, block 16, fp8 e4m3 KV with per-tensor scales, bf16 q, "
                    "512-token split-KV partitions"),
    "llama3_8b_int8kv": DecodeSpec(
        "llama3_8b_int8kv", 256, 32, 8, 128, 16, "bf16", "int8",
        ("lognormal", 1200.0, 0.8, 16, 8192), ("factor", 1.1), 1.0, 8192,
        description="Llama-3-8B-shaped GQA layer with an INT8 KV cache (one float32 scale per "
                    "block and KV head for K and for V, amax/127), bf16 q: batch 256, 32/8 heads, "
                    "head_dim 128, block 16, lens lognormal(median 1200, sigma 0.8) in [16,8192], "
                    "pool 1.1x"),
    "llama3_8b_kfp8_vbf16": DecodeSpec(
        "llama3_8b_kfp8_vbf16", 256, 32, 8, 128, 16, "bf16", "fp8_e4m3",
        ("lognormal", 1200.0, 0.8, 16, 8192), ("factor", 1.1), 1.0, 8192,
        per_tensor_fp8_scale=True, v_cache_dtype="bf16",
        description="Llama-3-8B-shaped GQA layer with the mixed-precision cache (fp8 e4m3 K with "
                    "a per-tensor scale, bf16 V, bf16 q): batch 256, 32/8 heads, head_dim 128, "
                    "block 16, lens lognormal(median 1200, sigma 0.8) in [16,8192], pool 1.1x"),
}


def draw_lengths(spec_lens: tuple, count: int, rng: np.random.Generator) -> np.ndarray:
    kind = spec_lens[0]
    if kind == "fixed":
        vals = np.asarray(spec_lens[1], dtype=np.int64)
        assert len(vals) == count
        return vals
    if kind == "uniform":
        return rng.integers(spec_lens[1], spec_lens[2] + 1, size=count).astype(np.int64)
    if kind == "lognormal":
        median, sigma, lo, hi = spec_lens[1:]
        raw = np.rint(np.exp(rng.normal(math.log(median), sigma, size=count)))
        return np.clip(raw, lo, hi).astype(np.int64)
    raise ValueError(kind)


def _rng(name: str, rep: int) -> np.random.Generator:
    salt = sum((i + 1) * ord(c) for i, c in enumerate(name))
    return np.random.default_rng(np.random.SeedSequence((415, salt, rep)))


@dataclass
class DecodeCase:
    """One decode step's inputs: a pool holding every token but the newest,
    the newest token's K/V and slot, and the queries."""
    spec: DecodeSpec
    q: np.ndarray              # bits [S][Hq][D]
    k_pool: np.ndarray         # bits [NB][Hkv][bs][D]
    v_pool: np.ndarray
    block_tables: np.ndarray   # int32 [S][MB]; padding -> poison_block
    seq_lens: np.ndarray       # int32 [S], includes the new token
    new_k: np.ndarray          # bits [S][Hkv][D] in the source dtype
    new_v: np.ndarray
    src_dtype: str
    slot_mapping: np.ndarray   # int64 [S]
    k_scale: float
    v_scale: float
    poison_block: int
    k_block_scales: np.ndarray | None = None   # int8 cache: float32 [NB][Hkv]
    v_block_scales: np.ndarray | None = None
    extra: dict = field(default_factory=dict)

    @property
    def num_blocks(self) -> int:
        return self.k_pool.shape[0]


@dataclass
class DecodeLayout:
    """The integer part of a decode step: lengths, block tables and slots.

    ``rng`` is the case's generator, positioned just after the draws that
    built the layout, so value draws continue the same stream."""
    spec: DecodeSpec
    seq_lens: np.ndarray       # int64 [S], includes the new token
    tables: list               # per sequence, its physical block ids
    block_tables: np.ndarray   # int32 [S][MB]; padding -> poison_block
    slot_mapping: np.ndarray   # int64 [S], slot of each sequence's newest token
    num_blocks: int
    poison_block: int
    rng: np.random.Generator


def make_decode_layout(spec: DecodeSpec | str, rep: int = 0, num_seqs: int | None = None,
                       lens=None) -> DecodeLayout:
    """Seeded lengths, shuffled physical block ids, padded block tables and the
    newest token's slot for every sequence (no element values)."""
    if isinstance(spec, str):
        spec = DECODE_SPECS[spec]
    rng = _rng(spec.seed_name or spec.name, rep)
    S = spec.num_seqs if num_seqs is None else num_seqs
    bs = spec.block_size
    if lens is None:
        seq_lens = draw_lengths(spec.lens, spec.num_seqs, rng)[:S]
    else:
        seq_lens = np.asarray(lens, dtype=np.int64)
        S = len(seq_lens)
    need = [blocks_for(int(n), bs) for n in seq_lens]
    total_blocks = sum(need)
    if spec.pool[0] == "fixed":
        nb = max(spec.pool[1], total_blocks + 1)
    else:
        nb = int(math.ceil(spec.pool[1] * total_blocks)) + 1
    mb = max(spec.max_blocks_per_seq, max(need) if need else 1)

    mgr = BlockManager(nb, bs, order=rng.permutation(nb))
    tables = [mgr.allocate(int(n)) for n in seq_lens]
    poison_block = mgr._take()

    block_tables = np.full((S, mb), poison_block, dtype=np.int32)
    slot_mapping = np.zeros(S, dtype=np.int64)
    for s, n in enumerate(seq_lens):
        block_tables[s, : len(tables[s])] = tables[s]
        pos = int(n) - 1
        slot_mapping[s] = tables[s][pos // bs] * bs + pos % bs
    return DecodeLayout(spec=spec, seq_lens=seq_lens, tables=tables, block_tables=block_tables,
                        slot_mapping=slot_mapping, num_blocks=nb, poison_block=poison_block,
                        rng=rng)


def make_decode_case(spec: DecodeSpec | str, rep: int = 0, num_seqs: int | None = None,
                     lens=None) -> DecodeCase:
    """Build a seeded decode step for ``spec`` (optionally with fewer sequences or
    explicit lengths, for small parity cases)."""
    lay = make_decode_layout(spec, rep, num_seqs, lens)
    spec, rng, seq_lens, tables = lay.spec, lay.rng, lay.seq_lens, lay.tables
    S = len(seq_lens)
    H, Hq, D, bs = spec.num_kv_heads, spec.num_q_heads, spec.head_dim, spec.block_size
    nb, poison_block = lay.num_blocks, lay.poison_block

    cache_dt, v_dt, q_dt = spec.cache_dtype, spec.v_dtype, spec.q_dtype
    src_dt = q_dt                                  # new K/V arrive in the activation dtype
    std = np.float32(spec.value_std)

    # Values for every token of every sequence, newest included (float32).
    k_vals = [rng.standard_normal((blocks_for(int(n), bs), H, bs, D), dtype=np.float32) * std
              for n in seq_lens]
    v_vals = [rng.standard_normal((blocks_for(int(n), bs), H, bs, D), dtype=np.float32) * std
              for n in seq_lens]
    q_vals = rng.standard_normal((S, Hq, D), dtype=np.float32) * std

    # The newest token's K/V, rounded to the source dtype.
    new_k_f = np.stack([k_vals[s][(int(n) - 1) // bs, :, (int(n) - 1) % bs, :]
                        for s, n in enumerate(seq_lens)]) if S else np.zeros((0, H, D), np.float32)
    new_v_f = np.stack([v_vals[s][(int(n) - 1) // bs, :, (int(n) - 1) % bs, :]
                        for s, n in enumerate(seq_lens)]) if S else np.zeros((0, H, D), np.float32)
    new_k = to_bits(new_k_f, src_dt)
    new_v = to_bits(new_v_f, src_dt)

    k_scale = v_scale = 1.0
    if spec.per_tensor_fp8_scale:
        # Per-tensor scale: largest magnitude of the valid cache contents / 448.
        def amax(vals, new_bits):
            m = 0.0
            for s, n in enumerate(seq_lens):
                flat = vals[s].transpose(1, 0, 2, 3).reshape(H, -1, D)[:, : int(n) - 1, :]
                if flat.size:
                    m = max(m, float(np.abs(flat).max()))
            from_new = np.abs(bits_to_torch(new_bits, src_dt).float().numpy()).max() if S else 0.0
            return max(m, float(from_new))
        if cache_dt == "fp8_e4m3":
            k_scale = float(np.float32(amax(k_vals, new_k) / FP8_MAX))
        if v_dt == "fp8_e4m3":
            v_scale = float(np.float32(amax(v_vals, new_v) / FP8_MAX))

    k_bsc = v_bsc = None
    if cache_dt == "int8":
        # one scale per (block, KV head): the amax of the block's tokens, the
        # newest (as its source-type value) included, over 127
        def block_scales(vals, new_bits):
            sc = np.ones((nb, H), np.float32)
            newf = bits_to_torch(new_bits, src_dt).float().numpy()
            for q, n in enumerate(seq_lens):
                n = int(n)
                v = vals[q].copy()
                v[(n - 1) // bs, :, (n - 1) % bs, :] = newf[q]
                flat = v.transpose(1, 0, 2, 3).reshape(H, -1, D)
                flat[:, n:, :] = 0
                per = np.abs(flat.reshape(H, -1, bs, D)).max(axis=(2, 3)).T        # [nblk][H]
                sc[np.asarray(tables[q])] = np.where(per > 0, per / np.float32(INT8_MAX), 1.0)
            return sc.astype(np.float32)
        k_bsc, v_bsc = block_scales(k_vals, new_k), block_scales(v_vals, new_v)

    k_pool = np.full((nb, H, bs, D), NAN_BITS[cache_dt], dtype=BITS_DTYPE[cache_dt])
    v_pool = np.full((nb, H, bs, D), NAN_BITS[v_dt], dtype=BITS_DTYPE[v_dt])
    for s, n in enumerate(seq_lens):
        n = int(n)
        ids = np.asarray(tables[s], dtype=np.int64)
        for vals, pool, sc, dt, bsc in ((k_vals[s], k_pool, k_scale, cache_dt, k_bsc),
                                        (v_vals[s], v_pool, v_scale, v_dt, v_bsc)):
            nan = NAN_BITS[dt]
            if dt == "int8":      # torch.round: half to even
                q8 = torch.from_numpy(vals / bsc[ids][:, :, None, None]).round().clamp(-127, 127)
                stored = q8.to(torch.int8).numpy().view(np.uint8).copy()
            else:
                stored = to_bits(vals / np.float32(sc) if dt == "fp8_e4m3" else vals, dt)
            # poison every slot from the newest token on (the newest is written by the scatter)
            flat = stored.transpose(1, 0, 2, 3).reshape(H, -1, D)
            flat[:, n - 1:, :] = nan
            pool[ids] = flat.reshape(H, len(ids), bs, D).transpose(1, 0, 2, 3)

    block_tables, slot_mapping = lay.block_tables, lay.slot_mapping
    return DecodeCase(spec=spec, q=to_bits(q_vals, q_dt), k_pool=k_pool, v_pool=v_pool,
                      block_tables=block_tables, seq_lens=seq_lens.astype(np.int32),
                      new_k=new_k, new_v=new_v, src_dtype=src_dt, slot_mapping=slot_mapping,
                      k_scale=k_scale, v_scale=v_scale, poison_block=poison_block,
                      k_block_scales=k_bsc, v_block_scales=v_bsc)


# ---------------------------------------------------------------------------
# Mixed chunked-prefill + decode step with a shared, copy-on-write prefix
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class MixedSpec:
    name: str = "mixed_prefix_bf16"
    num_forks: int = 16
    prefix_len: int = 1024
    chunk_len: int = 512
    num_decode: int = 112
    decode_lens: tuple = (256, 4096)
    num_q_heads: int = 32
    num_kv_heads: int = 8
    head_dim: int = 128
    block_size: int = 32
    dtype: str = "bf16"              # queries and new K/V rows
    pool_factor: float = 1.1
    description: str = ("16 sequences share a 1024-token prefix (ref-counted blocks) and each "
                        "appends a 512-token causal chunk; 112 others decode one token at lens "
                        "U[256,4096]; 32/8 heads, head_dim 128, block 32, bf16; copy-on-write "
                        "of the first divergent block")
    cache_dtype: str | None = None   # K/V pools: the same as dtype, "fp8_e4m3" with per-tensor
                                     # scales (amax of the values / 448), or "int8" with one
                                     # scale per (block, KV head) (the block's amax / 127)

    @property
    def pool_dtype(self) -> str:
        return self.cache_dtype or self.dtype

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


MIXED_SPEC = MixedSpec()

# A 70B-shaped serving step over an fp8 cache ([ybb] 6.2, KV cache in FP8; the
# pages' throughput figure is for Llama 3.3 70B FP8): four sequences share a
# 1,024-token prefix and each prefills a 512-token chunk while 128 others
# decode one token; 64 query / 8 KV heads, head_dim 128, block 16, bf16
# activations, fp8 E4M3 K/V with per-tensor scales.
MIXED_70B_FP8 = MixedSpec(
    name="mixed_70b_fp8kv", num_forks=4, num_decode=128, num_q_heads=64, num_kv_heads=8,
    block_size=16, cache_dtype="fp8_e4m3",
    description=("70B-shaped serving step over an fp8 cache: 4 sequences share a 1024-token "
                 "prefix and each appends a 512-token causal chunk; 128 others decode one "
                 "token at lens U[256,4096]; 64/8 heads, head_dim 128, block 16, bf16 "
                 "activations, fp8 e4m3 K/V with per-tensor scales; copy-on-write of the "
                 "first divergent block"))

# The same step over an INT8 cache with one scale per (block, KV head) for K
# and for V ([ybb] 6.2 names INT8 beside FP8 for the KV cache); copy-on-write
# copies the source block's scales with its codes.
MIXED_70B_INT8 = MixedSpec(
    name="mixed_70b_int8kv", num_forks=4, num_decode=128, num_q_heads=64, num_kv_heads=8,
    block_size=16, cache_dtype="int8",
    description=("70B-shaped serving step over an INT8 cache: 4 sequences share a 1024-token "
                 "prefix and each appends a 512-token causal chunk; 128 others decode one "
                 "token at lens U[256,4096]; 64/8 heads, head_dim 128, block 16, bf16 "
                 "activations, int8 K/V with one float32 scale per block and KV head (amax/127); "
                 "copy-on-write of the first divergent block with its scales"))


@dataclass
class MixedCase:
    spec: MixedSpec
    k_pool: np.ndarray
    v_pool: np.ndarray
    cow_pairs: np.ndarray            # int64 [P][2] (src, dst)
    # scatter of every new token (chunk tokens first, then decode tokens)
    new_k: np.ndarray                # bits [T][Hkv][D]
    new_v: np.ndarray
    slot_mapping: np.ndarray         # int64 [T]
    # prefill chunk
    q_chunk: np.ndarray              # bits [Tq][Hq][D]
    query_start_loc: np.ndarray      # int32 [F+1]
    prefill_tables: np.ndarray       # int32 [F][MBp] (after copy-on-write)
    prefill_tables_shared: np.ndarray  # same tables before copy-on-write (all share the prefix)
    prefill_lens: np.ndarray         # int32 [F]  (prefix + chunk)
    # decode
    q_decode: np.ndarray             # bits [Sd][Hq][D]
    decode_tables: np.ndarray        # int32 [Sd][MBd]
    decode_lens: np.ndarray          # int32 [Sd]
    poison_block: int
    k_scale: float = 1.0             # per-tensor scales of an fp8 pool (1.0 otherwise)
    v_scale: float = 1.0
    k_block_scales: np.ndarray | None = None   # int8 pool: float32 [NB][Hkv] (before copy-on-write)
    v_block_scales: np.ndarray | None = None


def make_mixed_case(spec: MixedSpec = MIXED_SPEC, rep: int = 0, num_forks: int | None = None,
                    prefix_len: int | None = None, chunk_len: int | None = None,
                    num_decode: int | None = None, decode_lens=None) -> MixedCase:
    """Build the mixed step; the optional overrides shrink it for small parity cases."""
    rng = _rng(spec.name, rep)
    F = spec.num_forks if num_forks is None else num_forks
    P = spec.prefix_len if prefix_len is None else prefix_len
    C = spec.chunk_len if chunk_len is None else chunk_len
    Sd = spec.num_decode if num_decode is None else num_decode
    H, Hq, D, bs, dt = spec.num_kv_heads, spec.num_q_heads, spec.head_dim, spec.block_size, spec.dtype
    if decode_lens is None:
        dlens = rng.integers(spec.decode_lens[0], spec.decode_lens[1] + 1, size=Sd).astype(np.int64)
    else:
        dlens = np.asarray(decode_lens, dtype=np.int64)
        Sd = len(dlens)

    prefix_blocks = blocks_for(P, bs)
    chunk_blocks = blocks_for(P + C, bs) - prefix_blocks
    decode_blocks = sum(blocks_for(int(n), bs) for n in dlens)
    demand = prefix_blocks + F * chunk_blocks + max(F - 1, 0) + decode_blocks
    nb = int(math.ceil(spec.pool_factor * demand)) + 1
    mgr = BlockManager(nb, bs, order=rng.permutation(nb))

    # Shared prefix: one sequence allocates it, the others fork it.
    base = mgr.allocate(P)
    prefix_ids = list(base[:prefix_blocks])          # before any fork remaps its table
    forks = [base] + [mgr.fork(base) for _ in range(F - 1)]
    # Each fork appends its chunk.
    for t in forks:
        mgr.grow(t, P + C)
    shared_tables = [list(t) for t in forks]
    # Copy-on-write of the first divergent block.  The prefix is block-aligned
    # here, so no chunk token lands in a shared block; the last prefix block is
    # taken as the first divergent one so that the copy happens.
    cow_pairs = []
    if prefix_blocks > 0:
        for t in forks:
            pair = mgr.copy_on_write(t, prefix_blocks - 1)
            if pair is not None:
                cow_pairs.append(pair)
    dec_tables = [mgr.allocate(int(n)) for n in dlens]
    poison_block = mgr._take()

    cdt = spec.pool_dtype
    nan = NAN_BITS[cdt]
    k_pool = np.full((nb, H, bs, D), nan, dtype=BITS_DTYPE[cdt])
    v_pool = np.full((nb, H, bs, D), nan, dtype=BITS_DTYPE[cdt])

    # Values are drawn first and stored once the scales are known (an fp8
    # pool's per-tensor scale is the amax of everything it will hold).
    drawn = {"k": [], "v": []}

    def fill(which, ids, ntok):
        vals = rng.standard_normal((len(ids), H, bs, D), dtype=np.float32)
        drawn[which].append((ids, ntok, vals))

    # prefix contents (the chunk's own K/V come through the scatter)
    fill("k", prefix_ids, P)
    fill("v", prefix_ids, P)
    # decode sequences: everything but the newest token
    for t, n in zip(dec_tables, dlens):
        fill("k", t, int(n) - 1)
        fill("v", t, int(n) - 1)

    # New tokens: F*C chunk tokens then Sd decode tokens.
    T = F * C + Sd
    new_k = to_bits(rng.standard_normal((T, H, D), dtype=np.float32), dt)
    new_v = to_bits(rng.standard_normal((T, H, D), dtype=np.float32), dt)

    slot_mapping = np.zeros(T, dtype=np.int64)
    for f, t in enumerate(forks):
        for i in range(C):
            pos = P + i
            slot_mapping[f * C + i] = t[pos // bs] * bs + pos % bs
    for d, (t, n) in enumerate(zip(dec_tables, dlens)):
        pos = int(n) - 1
        slot_mapping[F * C + d] = t[pos // bs] * bs + pos % bs

    scales = {"k": 1.0, "v": 1.0}
    bscales = {"k": None, "v": None}
    if cdt == "int8":
        # one scale per (block, KV head): the amax of everything the block will
        # hold (its drawn tokens and the new tokens the scatter writes into it)
        # over 127; copy-on-write destinations take their source's scales when
        # the step copies them
        for which, new in (("k", new_k), ("v", new_v)):
            amax = np.zeros((nb, H), np.float32)
            for ids, ntok, vals in drawn[which]:
                flat = np.abs(vals).transpose(1, 0, 2, 3).reshape(H, -1, D)
                flat[:, ntok:, :] = 0
                idx = np.asarray(ids, dtype=np.int64)
                amax[idx] = np.maximum(amax[idx], flat.reshape(H, len(ids), bs, D).max(axis=(2, 3)).T)
            if T:
                newa = np.abs(bits_to_torch(new, dt).float().numpy()).max(axis=2)       # [T][H]
                np.maximum.at(amax, slot_mapping // bs, newa)
            bscales[which] = np.where(amax > 0, amax / np.float32(INT8_MAX), 1.0).astype(np.float32)
    if cdt == "fp8_e4m3":
        for which, new in (("k", new_k), ("v", new_v)):
            m = float(np.abs(bits_to_torch(new, dt).float().numpy()).max()) if T else 0.0
            for ids, ntok, vals in drawn[which]:
                flat = vals.transpose(1, 0, 2, 3).reshape(H, -1, D)[:, :ntok, :]
                if flat.size:
                    m = max(m, float(np.abs(flat).max()))
            scales[which] = float(np.float32(m / FP8_MAX)) if m > 0 else 1.0
    for which, pool in (("k", k_pool), ("v", v_pool)):
        for ids, ntok, vals in drawn[which]:
            idx = np.asarray(ids, dtype=np.int64)
            if cdt == "int8":      # torch.round: half to even
                q8 = torch.from_numpy(vals / bscales[which][idx][:, :, None, None]).round().clamp(-127, 127)
                bits = q8.to(torch.int8).numpy().view(np.uint8).copy()
            else:
                bits = to_bits(vals / np.float32(scales[which]) if cdt == "fp8_e4m3" else vals, cdt)
            flat = bits.transpose(1, 0, 2, 3).reshape(H, -1, D)
            flat[:, ntok:, :] = nan
            pool[idx] = flat.reshape(H, len(ids), bs, D).transpose(1, 0, 2, 3)

    mbp = blocks_for(P + C, bs)
    prefill_tables = np.full((F, max(mbp, 1)), poison_block, dtype=np.int32)
    prefill_shared = np.full((F, max(mbp, 1)), poison_block, dtype=np.int32)
    for f in range(F):
        prefill_tables[f, : len(forks[f])] = forks[f]
        prefill_shared[f, : len(shared_tables[f])] = shared_tables[f]
    mbd = max(blocks_for(spec.decode_lens[1], bs), max((len(t) for t in dec_tables), default=1))
    decode_tables = np.full((Sd, mbd), poison_block, dtype=np.int32)
    for d, t in enumerate(dec_tables):
        decode_tables[d, : len(t)] = t

    q_chunk = to_bits(rng.standard_normal((F * C, Hq, D), dtype=np.float32), dt)
    q_decode = to_bits(rng.standard_normal((Sd, Hq, D), dtype=np.float32), dt)
    qsl = (np.arange(F + 1, dtype=np.int64) * C).astype(np.int32)
    return MixedCase(spec=spec, k_pool=k_pool, v_pool=v_pool,
                     cow_pairs=np.asarray(cow_pairs, dtype=np.int64).reshape(-1, 2),
                     new_k=new_k, new_v=new_v, slot_mapping=slot_mapping,
                     q_chunk=q_chunk, query_start_loc=qsl, prefill_tables=prefill_tables,
                     prefill_tables_shared=prefill_shared,
                     prefill_lens=np.full(F, P + C, dtype=np.int32),
                     q_decode=q_decode, decode_tables=decode_tables,
                     decode_lens=dlens.astype(np.int32), poison_block=poison_block,
                     k_scale=scales["k"], v_scale=scales["v"],
                     k_block_scales=bscales["k"], v_block_scales=bscales["v"])


# ---------------------------------------------------------------------------
# Byte accounting used by the benchmark
# ---------------------------------------------------------------------------

def block_scale_bytes(seq_lens, num_kv_heads: int, block_size: int) -> int:
    """Bytes of the per-block K and V scales an int8 decode step reads (float32 each)."""
    nblk = sum(blocks_for(int(n), block_size) for n in np.asarray(seq_lens).ravel())
    return nblk * num_kv_heads * 2 * 4


def effective_kv_bytes(seq_lens, num_kv_heads: int, head_dim: int, cache_dtype: str,
                       v_cache_dtype: str | None = None) -> int:
    """K and V bytes a decode step must read: sum_s len_s * Hkv * D * (eb_K + eb_V).

    For a Llama-2-7B-shaped fp16 layer (32 KV heads, head_dim 128) this is
    16 KiB per token, the per-layer figure the ybb.press page gives in §一.
    """
    eb = ELEM_BYTES[cache_dtype] + ELEM_BYTES[v_cache_dtype or cache_dtype]
    return int(np.asarray(seq_lens, dtype=np.int64).sum()) * num_kv_heads * head_dim * eb
