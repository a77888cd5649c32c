"""GPU parity of pa_mixed_attention (16-bit and fp8 E4M3 caches) and
pa_mixed_attention_int8 (INT8 cache with per-block scales), the mixed step's
prefill chunks and decodes in one launch: every output against the oracle
(max-abs 2e-2), the prefill outputs bit for bit against the standalone
prefill call, and HIP-graph replays bit for bit against the eager call."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_cases import TOL, lib, max_abs, random_chunks, random_chunks_int8, up, up_int

pytestmark = pytest.mark.gpu


class MixedRun:
    """Device copies of a MixedCase after its copy-on-write and scatter."""

    def __init__(self, case, decode_lens=None):
        pa = lib()
        self.case = case
        s = case.spec
        dt, cdt = s.dtype, s.pool_dtype
        self.sc = dict(k_scale=case.k_scale, v_scale=case.v_scale)
        self.kp, self.vp = up(case.k_pool, cdt), up(case.v_pool, cdt)
        self.i8 = cdt == "int8"
        pa.pa_copy_blocks(self.kp, self.vp, up_int(case.cow_pairs))
        if self.i8:
            # copy-on-write takes the source block's scales with its codes
            self.ks = torch.from_numpy(case.k_block_scales).to(self.kp.device)
            self.vs = torch.from_numpy(case.v_block_scales).to(self.kp.device)
            pa.pa_copy_blocks(self.ks, self.vs, up_int(case.cow_pairs))
            pa.pa_reshape_and_cache_int8(up(case.new_k, dt), up(case.new_v, dt), self.kp, self.vp, self.ks,
                                         self.vs, up_int(case.slot_mapping))
        else:
            pa.pa_reshape_and_cache(up(case.new_k, dt), up(case.new_v, dt), self.kp, self.vp,
                                    up_int(case.slot_mapping), case.k_scale, case.v_scale)
        self.qc, self.qd = up(case.q_chunk, dt), up(case.q_decode, dt)
        self.qsl = up_int(case.query_start_loc)
        self.ptab, self.plen = up_int(case.prefill_tables), up_int(case.prefill_lens)
        self.dlens = case.decode_lens if decode_lens is None else np.asarray(decode_lens, np.int32)
        self.dtab, self.dlen = up_int(case.decode_tables), up_int(self.dlens)
        self.max_q = int(np.diff(case.query_start_loc).max()) if len(case.query_start_loc) > 1 else 0
        self.max_len = max(int(self.dlens.max()), 1) if len(self.dlens) else 1

    def fused(self, partition_size=0, out=None):
        pa = lib()
        s = self.case.spec
        out_c, out_d = out if out is not None else (torch.empty_like(self.qc), torch.empty_like(self.qd))
        ws = pa.decode_workspace(self.qd, self.kp, self.max_len, partition_size)
        common = (out_c, self.qc, self.qsl, self.ptab, self.plen, self.max_q, out_d, self.qd, self.dtab,
                  self.dlen, self.max_len, self.kp, self.vp)
        if self.i8:
            pa.pa_mixed_attention_int8(*common, self.ks, self.vs, s.scale, partition_size=partition_size,
                                       workspace=ws)
        else:
            pa.pa_mixed_attention(*common, s.scale, partition_size=partition_size, workspace=ws, **self.sc)
        return out_c, out_d

    def separate(self):
        pa = lib()
        s = self.case.spec
        out_c, out_d = torch.empty_like(self.qc), torch.empty_like(self.qd)
        ws = pa.decode_workspace(self.qd, self.kp, self.max_len)
        if self.i8:
            if self.max_q > 0:
                pa.pa_prefill_chunk_int8(out_c, self.qc, self.qsl, self.kp, self.vp, self.ks, self.vs, self.ptab,
                                         self.plen, s.scale, self.max_q)
            pa.pa_decode_int8(out_d, self.qd, self.kp, self.vp, self.ks, self.vs, self.dtab, self.dlen, s.scale,
                              max_seq_len=self.max_len, workspace=ws)
            return out_c, out_d
        if self.max_q > 0:
            pa.pa_prefill_chunk(out_c, self.qc, self.qsl, self.kp, self.vp, self.ptab, self.plen, s.scale,
                                self.max_q, **self.sc)
        pa.pa_decode(out_d, self.qd, self.kp, self.vp, self.dtab, self.dlen, s.scale,
                     max_seq_len=self.max_len, workspace=ws, **self.sc)
        return out_c, out_d

    def oracle_scales(self):
        """The int8 pool's block scales after copy-on-write (None otherwise)."""
        c = self.case
        if not self.i8:
            return None, None
        return oracle.copy_blocks(c.k_block_scales, c.v_block_scales, c.cow_pairs)

    def oracle_pools(self):
        c, s = self.case, self.case.spec
        okp, ovp = oracle.copy_blocks(c.k_pool, c.v_pool, c.cow_pairs)
        oks, ovs = self.oracle_scales()
        return oracle.reshape_and_cache(okp, ovp, s.pool_dtype, c.new_k, c.new_v, s.dtype, c.slot_mapping,
                                        s.block_size, c.k_scale, c.v_scale, k_block_scales=oks,
                                        v_block_scales=ovs)

    def oracle(self):
        c, s = self.case, self.case.spec
        okp, ovp = self.oracle_pools()
        oks, ovs = self.oracle_scales()
        bsc = dict(k_block_scales=oks, v_block_scales=ovs)
        ref_c = oracle.prefill_chunk_attention(c.q_chunk, s.dtype, c.query_start_loc, okp, ovp, s.pool_dtype,
                                               c.prefill_tables, c.prefill_lens, s.scale, s.block_size,
                                               s.num_kv_heads, k_scale=c.k_scale, v_scale=c.v_scale, **bsc)
        ref_d = oracle.decode_attention(c.q_decode, s.dtype, okp, ovp, s.pool_dtype, c.decode_tables,
                                        self.dlens, s.scale, s.block_size, s.num_kv_heads,
                                        k_scale=c.k_scale, v_scale=c.v_scale, **bsc)
        return ref_c, ref_d


def _bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


SMALL = [
    # (spec overrides, forks, prefix, chunk, decode lengths)
    ({}, 4, 96, 40, [33, 64, 65, 300, 1000]),
    ({}, 3, 64, 70, [1, 2, 31, 32, 4096, 777, 129, 64, 5]),        # ragged chunk tiles, 1-token decodes
    ({"dtype": "f16"}, 2, 128, 33, [100, 2000, 31]),
    ({"head_dim": 64, "num_q_heads": 8, "num_kv_heads": 2}, 3, 40, 55, [7, 500, 1500, 64]),
    ({"block_size": 16, "num_q_heads": 16, "num_kv_heads": 1}, 2, 48, 90, [300, 17, 1024]),
    ({"block_size": 8, "num_q_heads": 8, "num_kv_heads": 8}, 2, 24, 20, [9, 250, 64]),
    ({"block_size": 64, "num_q_heads": 32, "num_kv_heads": 2}, 2, 128, 64, [65, 1, 1200]),
]


@pytest.mark.parametrize("over,forks,prefix,chunk,dlens", SMALL)
@pytest.mark.parametrize("partition", [0, 64, -1])
def test_fused_step_matches_oracle(over, forks, prefix, chunk, dlens, partition):
    spec = dataclasses.replace(W.MIXED_SPEC, **over)
    case = W.make_mixed_case(spec, num_forks=forks, prefix_len=prefix, chunk_len=chunk, decode_lens=dlens)
    run = MixedRun(case)
    out_c, out_d = run.fused(partition)
    sep_c, _ = run.separate()
    torch.cuda.synchronize()
    ref_c, ref_d = run.oracle()
    assert max_abs(out_c, ref_c) <= TOL[spec.dtype]
    assert max_abs(out_d, ref_d) <= TOL[spec.dtype]
    assert _bits_equal(out_c, sep_c), "prefill part differs from pa_prefill_chunk"


def test_fused_step_empty_decode_sequences():
    """Decode sequences of length 0 get zero outputs, beside live ones."""
    case = W.make_mixed_case(num_forks=2, prefix_len=64, chunk_len=50, decode_lens=[40, 300, 90, 1000, 5])
    run = MixedRun(case, decode_lens=[40, 0, 90, 0, 5])
    out_c, out_d = run.fused()
    torch.cuda.synchronize()
    ref_c, ref_d = run.oracle()
    assert not ref_d[1].any() and not ref_d[3].any()
    assert max_abs(out_c, ref_c) <= TOL["bf16"]
    assert max_abs(out_d, ref_d) <= TOL["bf16"]


@pytest.mark.parametrize("cache", ["bf16", "int8"])
def test_fused_step_without_prefill_or_decode(cache):
    """One part empty: the launch holds only the other kind of workgroup
    (16-bit cache, and an int8 cache through pa_mixed_attention_int8)."""
    spec = W.MIXED_SPEC if cache == "bf16" else W.MIXED_70B_INT8
    case = W.make_mixed_case(spec, num_forks=2, prefix_len=64, chunk_len=48, decode_lens=[100, 2000, 33])
    run = MixedRun(case)
    ref_c, ref_d = run.oracle()
    pa = lib()
    s = case.spec

    def call(*args, workspace=None):
        if run.i8:
            pa.pa_mixed_attention_int8(*args, run.kp, run.vp, run.ks, run.vs, s.scale, workspace=workspace)
        else:
            pa.pa_mixed_attention(*args, run.kp, run.vp, s.scale, workspace=workspace)

    # decodes only: no query tokens
    out_d = torch.empty_like(run.qd)
    empty_q = run.qc[:0]
    ws = pa.decode_workspace(run.qd, run.kp, run.max_len)
    call(torch.empty_like(empty_q), empty_q, up_int(np.zeros(1, np.int32)), run.ptab[:0], run.plen[:0], 0, out_d,
         run.qd, run.dtab, run.dlen, run.max_len, workspace=ws)
    # prefill chunks only: no decode sequences
    out_c = torch.empty_like(run.qc)
    call(out_c, run.qc, run.qsl, run.ptab, run.plen, run.max_q, run.qd[:0], run.qd[:0], run.dtab[:0],
         run.dlen[:0], 1)
    torch.cuda.synchronize()
    assert max_abs(out_d, ref_d) <= TOL["bf16"]
    assert max_abs(out_c, ref_c) <= TOL["bf16"]


def test_fused_full_size_step():
    """The full mixed workload (16 chunks of 512 tokens over a 1,536-token
    context, 112 decodes): every decode output against the oracle, every
    prefill output bit for bit against pa_prefill_chunk (which the prefill
    tests compare with the oracle at this size), and against the oracle on
    the first and last chunk."""
    case = W.make_mixed_case()
    print(f"[fused] forks={len(case.prefill_lens)} decode={len(case.decode_lens)}", flush=True)
    run = MixedRun(case)
    out_c, out_d = run.fused()
    sep_c, sep_d = run.separate()
    torch.cuda.synchronize()
    assert _bits_equal(out_c, sep_c), "prefill part differs from pa_prefill_chunk"
    s = case.spec
    okp, ovp = oracle.copy_blocks(case.k_pool, case.v_pool, case.cow_pairs)
    okp, ovp = oracle.reshape_and_cache(okp, ovp, s.dtype, case.new_k, case.new_v, s.dtype,
                                        case.slot_mapping, s.block_size)
    ref_d = oracle.decode_attention(case.q_decode, s.dtype, okp, ovp, s.dtype, case.decode_tables,
                                    case.decode_lens, s.scale, s.block_size, s.num_kv_heads)
    err_d = max_abs(out_d, ref_d)
    print(f"[fused] decode max-abs {err_d:.3e}", flush=True)
    assert err_d <= TOL["bf16"]
    qsl = case.query_start_loc
    for f in (0, len(qsl) - 2):
        sub_qsl = np.array([0, qsl[f + 1] - qsl[f]], np.int32)
        ref = oracle.prefill_chunk_attention(case.q_chunk[qsl[f]:qsl[f + 1]], s.dtype, sub_qsl, okp, ovp,
                                             s.dtype, case.prefill_tables[f:f + 1], case.prefill_lens[f:f + 1],
                                             s.scale, s.block_size, s.num_kv_heads)
        assert max_abs(out_c[qsl[f]:qsl[f + 1]], ref) <= TOL["bf16"]


def test_fused_step_graph_replays_equal_eager():
    """The call captured in a HIP graph: each replay (with eager work and a
    synchronisation between replays) gives the eager call's bits."""
    case = W.make_mixed_case(num_forks=3, prefix_len=96, chunk_len=70, decode_lens=[40, 300, 2000, 65, 1])
    run = MixedRun(case)
    eager_c, eager_d = run.fused()
    torch.cuda.synchronize()
    out_c, out_d = torch.empty_like(run.qc), torch.empty_like(run.qd)
    pa = lib()
    s = case.spec
    ws = pa.decode_workspace(run.qd, run.kp, run.max_len)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pa.pa_mixed_attention(out_c, run.qc, run.qsl, run.ptab, run.plen, run.max_q, out_d, run.qd,
                                  run.dtab, run.dlen, run.max_len, run.kp, run.vp, s.scale, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        out_c.fill_(0)
        out_d.fill_(0)
        ws.fill_(0xFF)          # stale workspace contents must not matter
        g.replay()
        torch.cuda.synchronize()
        assert _bits_equal(out_c, eager_c), f"prefill, replay {rep}"
        assert _bits_equal(out_d, eager_d), f"decode, replay {rep}"


def _fp8_step(rng, pchunks, pctx, dctx, hq, hkv, d, bs, q_dt, partition):
    """Prefill chunks and decodes over one fp8 pool with per-tensor scales: a
    decode is a one-token chunk at the end of its context, so one pool from
    random_chunks holds both; the sequences are then split into the two parts."""
    q, qsl, kp, vp, tables, lens, ks, vs = random_chunks(rng, list(pchunks) + [1] * len(dctx),
                                                          list(pctx) + list(dctx), hq, hkv, d, bs, "fp8_e4m3",
                                                          q_dtype=q_dt)
    P = len(pchunks)
    qsl_p, q_p, tab_p, len_p = qsl[:P + 1], q[:qsl[P]], tables[:P], lens[:P]
    q_d, tab_d, len_d = q[qsl[P]:], tables[P:], lens[P:]
    scale = 1.0 / np.sqrt(d)
    pa = lib()
    gk, gv = up(kp, "fp8_e4m3"), up(vp, "fp8_e4m3")
    gq_p, gq_d = up(q_p, q_dt), up(q_d, q_dt)
    out_p, out_d = torch.empty_like(gq_p), torch.empty_like(gq_d)
    max_len = int(len_d.max())
    ws = pa.decode_workspace(gq_d, gk, max_len, partition)
    pa.pa_mixed_attention(out_p, gq_p, up_int(qsl_p), up_int(tab_p), up_int(len_p), int(max(pchunks)), out_d,
                          gq_d, up_int(tab_d), up_int(len_d), max_len, gk, gv, scale, k_scale=ks, v_scale=vs,
                          partition_size=partition, workspace=ws)
    sep_p = torch.empty_like(gq_p)
    pa.pa_prefill_chunk(sep_p, gq_p, up_int(qsl_p), gk, gv, up_int(tab_p), up_int(len_p), scale,
                        int(max(pchunks)), k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    ref_p = oracle.prefill_chunk_attention(q_p, q_dt, qsl_p, kp, vp, "fp8_e4m3", tab_p, len_p, scale, bs, hkv,
                                           k_scale=ks, v_scale=vs)
    ref_d = oracle.decode_attention(q_d, q_dt, kp, vp, "fp8_e4m3", tab_d, len_d, scale, bs, hkv,
                                    k_scale=ks, v_scale=vs)
    return out_p, out_d, sep_p, ref_p, ref_d


FP8_SHAPES = [
    # (Hq, Hkv, D, bs, query type)
    (64, 8, 128, 16, "bf16"),
    (32, 8, 128, 32, "bf16"),
    (8, 2, 64, 16, "f16"),
    (16, 1, 128, 64, "bf16"),
    (4, 4, 64, 8, "f16"),
]


@pytest.mark.parametrize("hq,hkv,d,bs,q_dt", FP8_SHAPES)
@pytest.mark.parametrize("partition", [0, 512, -1])
def test_fused_fp8_step_matches_oracle(hq, hkv, d, bs, q_dt, partition):
    """fp8 E4M3 K/V with per-tensor scales ([ybb] 6.2): ragged chunks and decodes
    of 1 to 2,049 tokens in one launch."""
    rng = np.random.default_rng(hq * 7 + d + bs + (partition % 97))
    out_p, out_d, sep_p, ref_p, ref_d = _fp8_step(rng, [40, 70, 17], [300, 170, 17],
                                                  [1, 33, 500, 1200, 64, 2049, 16, 17], hq, hkv, d, bs, q_dt,
                                                  partition)
    assert max_abs(out_p, ref_p) <= TOL[q_dt]
    assert max_abs(out_d, ref_d) <= TOL[q_dt]
    assert _bits_equal(out_p, sep_p), "prefill part differs from pa_prefill_chunk"


def test_fused_fp8_70b_shaped_step():
    """A 70B-shaped layer with an fp8 cache (64 query / 8 KV heads, head_dim 128,
    block 16, bf16 activations): four 512-token chunks over 1,536-token contexts
    beside 128 decodes of lognormal lengths (median 1,500, clipped to
    [16, 8,192]), 512-token decode partitions; every output against the oracle."""
    rng = np.random.default_rng(415)
    dctx = np.clip(np.round(rng.lognormal(np.log(1500.0), 0.8, 128)), 16, 8192).astype(int)
    print(f"[fused fp8] decode tokens {int(dctx.sum())}", flush=True)
    out_p, out_d, sep_p, ref_p, ref_d = _fp8_step(rng, [512] * 4, [1536] * 4, dctx, 64, 8, 128, 16, "bf16", 512)
    err_p, err_d = max_abs(out_p, ref_p), max_abs(out_d, ref_d)
    print(f"[fused fp8] prefill max-abs {err_p:.3e}, decode max-abs {err_d:.3e}", flush=True)
    assert err_p <= TOL["bf16"] and err_d <= TOL["bf16"]
    assert _bits_equal(out_p, sep_p)


def _int8_step(rng, pchunks, pctx, dctx, hq, hkv, d, bs, q_dt, partition, v_scale_mul=1.0, q_mul=1.0):
    """As _fp8_step over an INT8 pool with per-(block, KV head) scales (V
    scales times v_scale_mul, queries times q_mul)."""
    q, qsl, kp, vp, tables, lens, ks, vs = random_chunks_int8(rng, list(pchunks) + [1] * len(dctx),
                                                              list(pctx) + list(dctx), hq, hkv, d, bs, q_dt,
                                                              v_scale_mul=v_scale_mul)
    if q_mul != 1.0:
        q = W.to_bits(W.bits_to_torch(q, q_dt).float().numpy() * q_mul, q_dt)
    P = len(pchunks)
    qsl_p, q_p, tab_p, len_p = qsl[:P + 1], q[:qsl[P]], tables[:P], lens[:P]
    q_d, tab_d, len_d = q[qsl[P]:], tables[P:], lens[P:]
    scale = 1.0 / np.sqrt(d)
    pa = lib()
    gk, gv = up(kp, "int8"), up(vp, "int8")
    gq_p, gq_d = up(q_p, q_dt), up(q_d, q_dt)
    gks, gvs = torch.from_numpy(ks).to(gq_p.device), torch.from_numpy(vs).to(gq_p.device)
    out_p, out_d = torch.empty_like(gq_p), torch.empty_like(gq_d)
    max_len = int(len_d.max())
    ws = pa.decode_workspace(gq_d, gk, max_len, partition)
    pa.pa_mixed_attention_int8(out_p, gq_p, up_int(qsl_p), up_int(tab_p), up_int(len_p), int(max(pchunks)), out_d,
                               gq_d, up_int(tab_d), up_int(len_d), max_len, gk, gv, gks, gvs, scale,
                               partition_size=partition, workspace=ws)
    sep_p = torch.empty_like(gq_p)
    pa.pa_prefill_chunk_int8(sep_p, gq_p, up_int(qsl_p), gk, gv, gks, gvs, up_int(tab_p), up_int(len_p), scale,
                             int(max(pchunks)))
    torch.cuda.synchronize()
    ref_p = oracle.prefill_chunk_attention(q_p, q_dt, qsl_p, kp, vp, "int8", tab_p, len_p, scale, bs, hkv,
                                           k_block_scales=ks, v_block_scales=vs)
    ref_d = oracle.decode_attention(q_d, q_dt, kp, vp, "int8", tab_d, len_d, scale, bs, hkv,
                                    k_block_scales=ks, v_block_scales=vs)
    return out_p, out_d, sep_p, ref_p, ref_d


INT8_SHAPES = [
    # (Hq, Hkv, D, bs, query type)
    (64, 8, 128, 16, "bf16"),
    (8, 2, 128, 32, "bf16"),
    (32, 8, 128, 16, "f16"),
    (4, 1, 64, 8, "f16"),
    (4, 4, 64, 64, "bf16"),
]


@pytest.mark.parametrize("hq,hkv,d,bs,q_dt", INT8_SHAPES)
@pytest.mark.parametrize("partition", [0, 512, -1])
def test_fused_int8_step_matches_oracle(hq, hkv, d, bs, q_dt, partition):
    """INT8 K/V with per-(block, KV head) scales ([ybb] 6.2): ragged chunks and
    decodes of 1 to 2,049 tokens in one launch."""
    rng = np.random.default_rng(hq * 11 + d + bs + (partition % 89))
    out_p, out_d, sep_p, ref_p, ref_d = _int8_step(rng, [40, 70, 17], [300, 170, 17],
                                                   [1, 33, 500, 1200, 64, 2049, 16, 17], hq, hkv, d, bs, q_dt,
                                                   partition)
    assert max_abs(out_p, ref_p) <= TOL[q_dt]
    assert max_abs(out_d, ref_d) <= TOL[q_dt]
    assert _bits_equal(out_p, sep_p), "prefill part differs from pa_prefill_chunk_int8"


def test_fused_int8_f16_queries_large_value_scales():
    """f16 queries over an int8 cache whose V values reach about 4e4 (block V
    scales near 300) with widely spread logits, in one launch: the value
    operand p x scale stays inside f16's range in both programs (the
    reference max moves with every larger logit).  Compared relative to the
    values' size."""
    rng = np.random.default_rng(919)
    out_p, out_d, sep_p, ref_p, ref_d = _int8_step(rng, [64, 33], [300, 700], [1, 90, 1500, 17], 8, 2, 128, 16,
                                                   "f16", 0, v_scale_mul=1.5e4, q_mul=6.0)
    vmax = float(max(np.abs(ref_p).max(), np.abs(ref_d).max()))
    assert vmax > 1e3
    assert torch.isfinite(out_p).all() and torch.isfinite(out_d).all()
    assert max_abs(out_p, ref_p) <= TOL["f16"] * vmax / 4
    assert max_abs(out_d, ref_d) <= TOL["f16"] * vmax / 4
    assert _bits_equal(out_p, sep_p)


def test_fused_int8_70b_shaped_step():
    """The 70B-shaped layer of the fp8 case over an INT8 cache: four 512-token
    chunks over 1,536-token contexts beside 128 lognormal decodes; every output
    against the oracle."""
    rng = np.random.default_rng(416)
    dctx = np.clip(np.round(rng.lognormal(np.log(1500.0), 0.8, 128)), 16, 8192).astype(int)
    out_p, out_d, sep_p, ref_p, ref_d = _int8_step(rng, [512] * 4, [1536] * 4, dctx, 64, 8, 128, 16, "bf16",
                                                   512)
    err_p, err_d = max_abs(out_p, ref_p), max_abs(out_d, ref_d)
    print(f"[fused int8] prefill max-abs {err_p:.3e}, decode max-abs {err_d:.3e}", flush=True)
    assert err_p <= TOL["bf16"] and err_d <= TOL["bf16"]
    assert _bits_equal(out_p, sep_p)


@pytest.mark.parametrize("cache", ["bf16", "fp8_e4m3", "int8"])
def test_fused_step_at_the_plan_limit(cache):
    """8,000 decodes of 1-64 tokens (the most a call plans: the lengths and
    their prefix sums fill 64 KB of LDS, with the fp8 K staging on top) beside
    two prefill chunks; every output against the oracle."""
    rng = np.random.default_rng(8000)
    dctx = rng.integers(1, 65, 8000)
    hq, hkv, d, bs = 8, 2, 128, 16
    pchunks, pctx = [33, 64], [100, 64]
    chunks, ctxs = pchunks + [1] * len(dctx), pctx + list(dctx)
    bscales = {}
    if cache == "fp8_e4m3":
        q, qsl, kp, vp, tables, lens, ks, vs = random_chunks(rng, chunks, ctxs, hq, hkv, d, bs, cache,
                                                              q_dtype="bf16")
    elif cache == "int8":
        q, qsl, kp, vp, tables, lens, bks, bvs = random_chunks_int8(rng, chunks, ctxs, hq, hkv, d, bs, "bf16")
        ks = vs = 1.0
        bscales = dict(k_block_scales=bks, v_block_scales=bvs)
    else:
        q, qsl, kp, vp, tables, lens = random_chunks(rng, chunks, ctxs, hq, hkv, d, bs, cache)
        ks = vs = 1.0
    P = len(pchunks)
    scale = 1.0 / np.sqrt(d)
    pa = lib()
    gk, gv = up(kp, cache), up(vp, cache)
    gq_p, gq_d = up(q[:qsl[P]], "bf16"), up(q[qsl[P]:], "bf16")
    out_p, out_d = torch.empty_like(gq_p), torch.empty_like(gq_d)
    for partition in (0, 512, -1):
        ws = pa.decode_workspace(gq_d, gk, 64, partition)
        common = (out_p, gq_p, up_int(qsl[:P + 1]), up_int(tables[:P]), up_int(lens[:P]), 64, out_d, gq_d,
                  up_int(tables[P:]), up_int(lens[P:]), 64, gk, gv)
        if cache == "int8":
            dev = gq_p.device
            pa.pa_mixed_attention_int8(*common, torch.from_numpy(bks).to(dev), torch.from_numpy(bvs).to(dev),
                                       scale, partition_size=partition, workspace=ws)
        else:
            pa.pa_mixed_attention(*common, scale, k_scale=ks, v_scale=vs, partition_size=partition, workspace=ws)
        torch.cuda.synchronize()
        ref_p = oracle.prefill_chunk_attention(q[:qsl[P]], "bf16", qsl[:P + 1], kp, vp, cache, tables[:P],
                                               lens[:P], scale, bs, hkv, k_scale=ks, v_scale=vs, **bscales)
        ref_d = oracle.decode_attention(q[qsl[P]:], "bf16", kp, vp, cache, tables[P:], lens[P:], scale, bs, hkv,
                                        k_scale=ks, v_scale=vs, **bscales)
        assert max_abs(out_p, ref_p) <= TOL["bf16"], partition
        assert max_abs(out_d, ref_d) <= TOL["bf16"], partition


@pytest.mark.parametrize("cache", ["fp8_e4m3", "int8"])
def test_fused_quantised_step_graph_replays_equal_eager(cache):
    """The one-launch step over an fp8 or int8 cache captured in a HIP graph:
    each of four replays (eager fills and a stale workspace between them)
    gives the eager bits."""
    rng = np.random.default_rng(88)
    hq, hkv, d, bs = 32, 8, 128, 16
    chunks, ctxs = [70, 33] + [1] * 6, [300, 33, 1, 64, 500, 1200, 17, 2049]
    if cache == "int8":
        q, qsl, kp, vp, tables, lens, ks, vs = random_chunks_int8(rng, chunks, ctxs, hq, hkv, d, bs, "bf16")
    else:
        q, qsl, kp, vp, tables, lens, ks, vs = random_chunks(rng, chunks, ctxs, hq, hkv, d, bs, cache,
                                                              q_dtype="bf16")
    P = 2
    scale = 1.0 / np.sqrt(d)
    pa = lib()
    gk, gv = up(kp, cache), up(vp, cache)
    gq_p, gq_d = up(q[:qsl[P]], "bf16"), up(q[qsl[P]:], "bf16")
    args = (up_int(qsl[:P + 1]), up_int(tables[:P]), up_int(lens[:P]), 70)
    dargs = (up_int(tables[P:]), up_int(lens[P:]), 2049)
    ws = pa.decode_workspace(gq_d, gk, 2049)
    if cache == "int8":
        gks, gvs = torch.from_numpy(ks).to(gq_p.device), torch.from_numpy(vs).to(gq_p.device)

    def call(out_p, out_d):
        if cache == "int8":
            pa.pa_mixed_attention_int8(out_p, gq_p, *args, out_d, gq_d, *dargs, gk, gv, gks, gvs, scale,
                                       workspace=ws)
        else:
            pa.pa_mixed_attention(out_p, gq_p, *args, out_d, gq_d, *dargs, gk, gv, scale, k_scale=ks,
                                  v_scale=vs, workspace=ws)

    eager_p, eager_d = torch.empty_like(gq_p), torch.empty_like(gq_d)
    call(eager_p, eager_d)
    torch.cuda.synchronize()
    out_p, out_d = torch.empty_like(gq_p), torch.empty_like(gq_d)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            call(out_p, out_d)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        out_p.fill_(0)
        out_d.fill_(0)
        ws.fill_(0xFF)
        g.replay()
        torch.cuda.synchronize()
        assert _bits_equal(out_p, eager_p), f"prefill, replay {rep}"
        assert _bits_equal(out_d, eager_d), f"decode, replay {rep}"


def test_fused_70b_fp8_serving_step_full_size():
    """The 70B-shaped serving step over an fp8 cache (4 chunks of 512 tokens
    after a shared 1,024-token prefix, 128 decodes of 256-4,096 tokens, 64/8
    heads, block 16, per-tensor scales): copy-on-write and the quantising
    scatter byte-exact against the oracle, every decode output and every
    prefill output against the oracle, prefill bits equal to pa_prefill_chunk's."""
    case = W.make_mixed_case(W.MIXED_70B_FP8)
    print(f"[fused fp8 70b] decode tokens {int(case.decode_lens.sum())}, pool {case.k_pool.shape[0]} blocks",
          flush=True)
    run = MixedRun(case)
    out_c, out_d = run.fused()
    sep_c, _ = run.separate()
    torch.cuda.synchronize()
    assert _bits_equal(out_c, sep_c), "prefill part differs from pa_prefill_chunk"
    okp, ovp = run.oracle_pools()
    cdt = case.spec.pool_dtype
    assert np.array_equal(W.torch_to_bits(run.kp, cdt), okp)
    assert np.array_equal(W.torch_to_bits(run.vp, cdt), ovp)
    ref_c, ref_d = run.oracle()
    err_c, err_d = max_abs(out_c, ref_c), max_abs(out_d, ref_d)
    print(f"[fused fp8 70b] prefill max-abs {err_c:.3e}, decode max-abs {err_d:.3e}", flush=True)
    assert err_c <= TOL["bf16"] and err_d <= TOL["bf16"]


def test_fused_70b_int8_serving_step_full_size():
    """The 70B-shaped serving step over an INT8 cache with per-(block, KV head)
    scales: copy-on-write of the codes and of their scales, then the int8
    scatter, byte-exact against the oracle; every decode and prefill output of
    pa_mixed_attention_int8 against the oracle; prefill bits equal to
    pa_prefill_chunk_int8's."""
    case = W.make_mixed_case(W.MIXED_70B_INT8)
    print(f"[fused int8 70b] decode tokens {int(case.decode_lens.sum())}, pool {case.k_pool.shape[0]} blocks",
          flush=True)
    run = MixedRun(case)
    out_c, out_d = run.fused()
    sep_c, _ = run.separate()
    torch.cuda.synchronize()
    assert _bits_equal(out_c, sep_c), "prefill part differs from pa_prefill_chunk_int8"
    oks, ovs = run.oracle_scales()
    assert np.array_equal(run.ks.cpu().numpy(), oks) and np.array_equal(run.vs.cpu().numpy(), ovs)
    okp, ovp = run.oracle_pools()
    assert np.array_equal(W.torch_to_bits(run.kp, "int8"), okp)
    assert np.array_equal(W.torch_to_bits(run.vp, "int8"), ovp)
    ref_c, ref_d = run.oracle()
    err_c, err_d = max_abs(out_c, ref_c), max_abs(out_d, ref_d)
    print(f"[fused int8 70b] prefill max-abs {err_c:.3e}, decode max-abs {err_d:.3e}", flush=True)
    assert err_c <= TOL["bf16"] and err_d <= TOL["bf16"]
