"""Helpers shared by the GPU parity tests: run a workload through the HIP
library (via the binding) and through the oracle, on the same seeded inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

# Max-abs tolerances on attention outputs (fp32 queries / 16-bit or fp8 paths).
TOL = {"f32": 5e-3, "f16": 2e-2, "bf16": 2e-2}


def lib():
    import paged_kv_cache_415_amd as pa   # fails loudly if the library is missing
    return pa


def dev():
    return torch.device("cuda:0")


def up(bits, dtype):
    return W.bits_to_device(bits, dtype, dev())


def up_int(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def max_abs(gpu: torch.Tensor, ref: np.ndarray) -> float:
    got = as_f64(gpu)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert not np.isnan(got).any(), "NaN in GPU output"
    return float(np.abs(got - ref).max()) if got.size else 0.0


class DecodeRun:
    """Device copies of a DecodeCase plus the scatter and decode calls."""

    def __init__(self, case: W.DecodeCase):
        self.case = case
        s = case.spec
        self.q = up(case.q, s.q_dtype)
        self.k_pool = up(case.k_pool, s.cache_dtype)
        self.v_pool = up(case.v_pool, s.v_dtype)
        self.mixed = s.v_dtype != s.cache_dtype
        self.int8 = s.cache_dtype == "int8"
        if self.int8:
            self.k_scales = torch.from_numpy(case.k_block_scales).to(dev())
            self.v_scales = torch.from_numpy(case.v_block_scales).to(dev())
        self.new_k = up(case.new_k, case.src_dtype)
        self.new_v = up(case.new_v, case.src_dtype)
        self.tables = up_int(case.block_tables)
        self.lens = up_int(case.seq_lens)
        self.slots = up_int(case.slot_mapping)
        self.max_len = int(case.seq_lens.max()) if len(case.seq_lens) else 1

    def scatter(self):
        pa = lib()
        if self.int8:
            pa.pa_reshape_and_cache_int8(self.new_k, self.new_v, self.k_pool, self.v_pool,
                                         self.k_scales, self.v_scales, self.slots)
            return
        fn = pa.pa_reshape_and_cache_kv if self.mixed else pa.pa_reshape_and_cache
        fn(self.new_k, self.new_v, self.k_pool, self.v_pool, self.slots, self.case.k_scale,
           self.case.v_scale)

    def decode(self, partition_size=None, stages=False, max_seq_len=None):
        pa = lib()
        s = self.case.spec
        ps = s.partition_size if partition_size is None else partition_size
        msl = self.max_len if max_seq_len is None else max_seq_len
        ws = pa.decode_workspace(self.q, self.k_pool, msl, ps)
        out = torch.empty_like(self.q)
        args = (out, self.q, self.k_pool, self.v_pool, self.tables, self.lens, s.scale, msl,
                self.case.k_scale, self.case.v_scale, ps, ws)
        if self.int8:
            a8 = (out, self.q, self.k_pool, self.v_pool, self.k_scales, self.v_scales, self.tables,
                  self.lens, s.scale, msl, ps, ws)
            if stages:
                pa.pa_decode_attention_int8(*a8)
                pa.pa_decode_reduce_int8(*a8)
            else:
                pa.pa_decode_int8(*a8)
        elif self.mixed:
            if stages:
                pa.pa_decode_attention_kv(*args)
                pa.pa_decode_reduce_kv(*args)
            else:
                pa.pa_decode_kv(*args)
        elif stages:
            pa.pa_decode_attention(*args)
            pa.pa_decode_reduce(*args)
        else:
            pa.pa_decode(*args)
        torch.cuda.synchronize()
        return out


def oracle_step(case: W.DecodeCase):
    """Oracle scatter of the newest tokens then decode; returns (out, k_pool, v_pool)."""
    s = case.spec
    kp, vp = oracle.reshape_and_cache(case.k_pool, case.v_pool, s.cache_dtype, case.new_k,
                                      case.new_v, case.src_dtype, case.slot_mapping, s.block_size,
                                      case.k_scale, case.v_scale, v_cache_dtype=s.v_dtype,
                                      k_block_scales=case.k_block_scales,
                                      v_block_scales=case.v_block_scales)
    out = oracle.decode_attention(case.q, s.q_dtype, kp, vp, s.cache_dtype, case.block_tables,
                                  case.seq_lens, s.scale, s.block_size, s.num_kv_heads,
                                  case.k_scale, case.v_scale, v_cache_dtype=s.v_dtype,
                                  k_block_scales=case.k_block_scales,
                                  v_block_scales=case.v_block_scales)
    return out, kp, vp


def custom_spec(name, hq, hkv, d, bs, q_dtype, cache_dtype, v_cache_dtype=None):
    return W.DecodeSpec(name, 1, hq, hkv, d, bs, q_dtype, cache_dtype, ("fixed", (1,)),
                        ("factor", 1.3), 1.0, 8192, 0,
                        per_tensor_fp8_scale=(cache_dtype == "fp8_e4m3"),
                        v_cache_dtype=v_cache_dtype)


def random_chunks(rng, chunks, ctxs, hq, hkv, d, bs, dtype, q_dtype=None):
    """Pool holding each sequence's whole context (chunk included) + packed queries.
    An fp8 pool holds the values / a per-tensor scale (amax / 448); the scales
    are returned as the last two items."""
    need = [-(-n // bs) for n in ctxs]
    nb = sum(need) + 2
    ids = rng.permutation(nb)
    poison = int(ids[-1])
    nan = W.NAN_BITS[dtype]
    kp = np.full((nb, hkv, bs, d), nan, W.BITS_DTYPE[dtype])
    vp = np.full((nb, hkv, bs, d), nan, W.BITS_DTYPE[dtype])
    tables = np.full((len(ctxs), max(need)), poison, np.int32)
    cur = 0
    vals = {0: [], 1: []}
    for s, n in enumerate(ctxs):
        for b in range(need[s]):
            tables[s, b] = ids[cur]
            cur += 1
        for i in (0, 1):
            vals[i].append(rng.standard_normal((need[s], hkv, bs, d)).astype(np.float32))
    scales = [1.0, 1.0]
    if dtype == "fp8_e4m3":
        for i in (0, 1):
            amax = max(float(np.abs(v.transpose(1, 0, 2, 3).reshape(hkv, -1, d)[:, :n]).max())
                       for v, n in zip(vals[i], ctxs))
            scales[i] = float(np.float32(amax / W.FP8_MAX))
    for s, n in enumerate(ctxs):
        for i, pool in ((0, kp), (1, vp)):
            x = vals[i][s] / np.float32(scales[i]) if dtype == "fp8_e4m3" else vals[i][s]
            bits = W.to_bits(x, dtype)
            flat = bits.transpose(1, 0, 2, 3).reshape(hkv, -1, d)
            flat[:, n:, :] = nan
            pool[tables[s, :need[s]]] = flat.reshape(hkv, need[s], bs, d).transpose(1, 0, 2, 3)
    qsl = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = W.to_bits(rng.standard_normal((int(qsl[-1]), hq, d)).astype(np.float32), q_dtype or dtype)
    if dtype == "fp8_e4m3":
        return q, qsl, kp, vp, tables, np.asarray(ctxs, np.int32), scales[0], scales[1]
    return q, qsl, kp, vp, tables, np.asarray(ctxs, np.int32)


def random_chunks_int8(rng, chunks, ctxs, hq, hkv, d, bs, q_dtype, v_scale_mul=1.0):
    """As random_chunks, over an int8 cache: codes uniform in [-127, 127], one
    float32 scale per (block, KV head) per pool (V scales times v_scale_mul);
    rows past each context hold code 127.  Returns q, qsl, kp, vp, tables,
    lens, k_scales, v_scales (pools as raw bytes)."""
    need = [-(-n // bs) for n in ctxs]
    nb = sum(need) + 2
    ids = rng.permutation(nb)
    poison = int(ids[-1])
    kp = rng.integers(-127, 128, (nb, hkv, bs, d)).astype(np.int8)
    vp = rng.integers(-127, 128, (nb, hkv, bs, d)).astype(np.int8)
    ks = (rng.uniform(0.5, 2.0, (nb, hkv)) / 32).astype(np.float32)
    vs = (rng.uniform(0.5, 2.0, (nb, hkv)) / 64 * v_scale_mul).astype(np.float32)
    tables = np.full((len(ctxs), max(need)), poison, np.int32)
    cur = 0
    for s_, n in enumerate(ctxs):
        tables[s_, :need[s_]] = ids[cur:cur + need[s_]]
        cur += need[s_]
        for pool in (kp, vp):
            flat = pool[tables[s_, :need[s_]]].transpose(1, 0, 2, 3).reshape(hkv, -1, d)
            flat[:, n:, :] = 127
            pool[tables[s_, :need[s_]]] = flat.reshape(hkv, need[s_], bs, d).transpose(1, 0, 2, 3)
    qsl = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = W.to_bits(rng.standard_normal((int(qsl[-1]), hq, d)).astype(np.float32), q_dtype)
    return q, qsl, kp.view(np.uint8), vp.view(np.uint8), tables, np.asarray(ctxs, np.int32), ks, vs

