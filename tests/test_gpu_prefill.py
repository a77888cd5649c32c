"""GPU parity of pa_prefill_chunk and of the mixed chunked-prefill + decode
step with a shared, copy-on-write prefix (tolerance 2e-2 max-abs)."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_cases import TOL, as_f64, lib, max_abs, random_chunks as _random_chunks, random_chunks_int8, up, up_int

pytestmark = pytest.mark.gpu


CASES = [
    # (chunks, contexts, Hq, Hkv, D, bs, dtype)
    ([5, 16, 1], [5, 40, 70], 4, 1, 128, 16, "bf16"),
    ([33, 100], [33, 300], 8, 2, 128, 32, "bf16"),
    ([64, 7], [200, 7], 32, 8, 128, 32, "bf16"),
    ([130], [131], 16, 1, 128, 16, "f16"),
    ([17, 50], [60, 99], 2, 2, 64, 16, "f16"),
    ([40], [555], 8, 1, 64, 32, "bf16"),
    # 8- and 64-token blocks
    ([20, 9], [85, 9], 8, 2, 128, 8, "bf16"),
    ([70], [300], 4, 4, 64, 64, "f16"),
    ([33], [77], 16, 1, 128, 64, "bf16"),
    ([100], [130], 4, 1, 64, 8, "bf16"),
]


@pytest.mark.parametrize("chunks,ctxs,hq,hkv,d,bs,dtype", CASES)
def test_prefill_matches_oracle(chunks, ctxs, hq, hkv, d, bs, dtype):
    rng = np.random.default_rng(sum(chunks) + hq + d)
    q, qsl, kp, vp, tables, lens = _random_chunks(rng, chunks, ctxs, hq, hkv, d, bs, dtype)
    scale = 1.0 / np.sqrt(d)
    ref = oracle.prefill_chunk_attention(q, dtype, qsl, kp, vp, dtype, tables, lens, scale, bs, hkv)
    gq = up(q, dtype)
    out = torch.empty_like(gq)
    lib().pa_prefill_chunk(out, gq, up_int(qsl), up(kp, dtype), up(vp, dtype), up_int(tables),
                           up_int(lens), scale, max(chunks))
    torch.cuda.synchronize()
    assert max_abs(out, ref) <= TOL[dtype]


def test_prefill_last_row_matches_decode():
    rng = np.random.default_rng(5)
    chunks, ctxs = [9, 30], [100, 64]
    q, qsl, kp, vp, tables, lens = _random_chunks(rng, chunks, ctxs, 8, 2, 128, 16, "bf16")
    pa = lib()
    gq = up(q, "bf16")
    gk, gv, gt, gl = up(kp, "bf16"), up(vp, "bf16"), up_int(tables), up_int(lens)
    out = torch.empty_like(gq)
    pa.pa_prefill_chunk(out, gq, up_int(qsl), gk, gv, gt, gl, 0.1, 30)
    last = gq[torch.tensor([8, 38], device=gq.device)].contiguous()
    dec = torch.empty_like(last)
    pa.pa_decode(dec, last, gk, gv, gt, gl, 0.1, max_seq_len=100, partition_size=-1)
    torch.cuda.synchronize()
    diff = np.abs(as_f64(out[[8, 38]]) - as_f64(dec)).max()
    assert diff <= TOL["bf16"]


def _mixed_step(case):
    """Device: copy-on-write -> scatter -> prefill chunk + decode (one stream)."""
    pa = lib()
    s = case.spec
    dt = s.dtype
    kp, vp = up(case.k_pool, dt), up(case.v_pool, dt)
    pa.pa_copy_blocks(kp, vp, up_int(case.cow_pairs))
    pa.pa_reshape_and_cache(up(case.new_k, dt), up(case.new_v, dt), kp, vp, up_int(case.slot_mapping))
    qc, qd = up(case.q_chunk, dt), up(case.q_decode, dt)
    out_c, out_d = torch.empty_like(qc), torch.empty_like(qd)
    pa.pa_prefill_chunk(out_c, qc, up_int(case.query_start_loc), kp, vp, up_int(case.prefill_tables),
                        up_int(case.prefill_lens), s.scale, int(np.diff(case.query_start_loc).max()))
    max_len = int(case.decode_lens.max())
    ws = pa.decode_workspace(qd, kp, max_len)
    pa.pa_decode(out_d, qd, kp, vp, up_int(case.decode_tables), up_int(case.decode_lens), s.scale,
                 max_seq_len=max_len, workspace=ws)
    torch.cuda.synchronize()
    return out_c, out_d, kp, vp


def _oracle_pools(case):
    s = case.spec
    kp, vp = oracle.copy_blocks(case.k_pool, case.v_pool, case.cow_pairs)
    return oracle.reshape_and_cache(kp, vp, s.dtype, case.new_k, case.new_v, s.dtype,
                                    case.slot_mapping, s.block_size)


def test_mixed_step_small_full_compare():
    case = W.make_mixed_case(num_forks=4, prefix_len=96, chunk_len=40, num_decode=5,
                             decode_lens=[33, 64, 65, 300, 1000])
    s = case.spec
    out_c, out_d, kp, vp = _mixed_step(case)
    okp, ovp = _oracle_pools(case)
    assert np.array_equal(W.torch_to_bits(kp, s.dtype), okp)
    assert np.array_equal(W.torch_to_bits(vp, s.dtype), ovp)
    ref_c = oracle.prefill_chunk_attention(case.q_chunk, s.dtype, case.query_start_loc, okp, ovp,
                                           s.dtype, case.prefill_tables, case.prefill_lens,
                                           s.scale, s.block_size, s.num_kv_heads)
    ref_d = oracle.decode_attention(case.q_decode, s.dtype, okp, ovp, s.dtype, case.decode_tables,
                                    case.decode_lens, s.scale, s.block_size, s.num_kv_heads)
    assert max_abs(out_c, ref_c) <= TOL["bf16"]
    assert max_abs(out_d, ref_d) <= TOL["bf16"]


def test_mixed_step_full_size():
    """The full mixed workload: pools byte-exact, every decode output and every
    prefill output (16 chunks x 512 rows x 32 heads x 128 dims) against the oracle."""
    case = W.make_mixed_case()
    s = case.spec
    print(f"[mixed] forks={len(case.prefill_lens)} decode={len(case.decode_lens)} "
          f"pool={case.k_pool.shape[0]}", flush=True)
    out_c, out_d, kp, vp = _mixed_step(case)
    okp, ovp = _oracle_pools(case)
    assert np.array_equal(W.torch_to_bits(kp, s.dtype), okp)
    assert np.array_equal(W.torch_to_bits(vp, s.dtype), ovp)
    ref_d = oracle.decode_attention(case.q_decode, s.dtype, okp, ovp, s.dtype, case.decode_tables,
                                    case.decode_lens, s.scale, s.block_size, s.num_kv_heads)
    assert max_abs(out_d, ref_d) <= TOL["bf16"]
    print("[mixed] decode outputs match; oracle prefill over every chunk, head and row", flush=True)
    ref_c = oracle.prefill_chunk_attention(case.q_chunk, s.dtype, case.query_start_loc, okp, ovp,
                                           s.dtype, case.prefill_tables, case.prefill_lens,
                                           s.scale, s.block_size, s.num_kv_heads)
    err = max_abs(out_c, ref_c)
    print(f"[mixed] prefill max-abs over all {ref_c.size} outputs {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_rising_logits_move_the_running_max(dtype):
    """Each row's logits rise along the keys, so every 64-key tile raises
    every row's max (the kernel defers rescaling until the max has grown by
    2^8): many small and some large moves per row."""
    rng = np.random.default_rng(11)
    chunks, ctxs = [200, 37], [700, 300]
    hq, hkv, d, bs = 8, 2, 128, 16
    q, qsl, kp, vp, tables, lens = _random_chunks(rng, chunks, ctxs, hq, hkv, d, bs, dtype)
    kf = W.bits_to_torch(kp, dtype).float().numpy()
    for s, n in enumerate(ctxs):
        for j in range(n):
            kf[tables[s, j // bs], :, j % bs, 0] = 0.12 * j * (1 if s == 0 else -1) + (j % 7)
    kp = W.to_bits(kf, dtype)
    qf = np.zeros((int(qsl[-1]), hq, d), np.float32)
    qf[:, :, 0] = np.linspace(0.5, 4.0, hq)
    q = W.to_bits(qf, dtype)
    scale = 1.0 / np.sqrt(d)
    ref = oracle.prefill_chunk_attention(q, dtype, qsl, kp, vp, dtype, tables, lens, scale, bs, hkv)
    gq = up(q, dtype)
    out = torch.empty_like(gq)
    lib().pa_prefill_chunk(out, gq, up_int(qsl), up(kp, dtype), up(vp, dtype), up_int(tables),
                           up_int(lens), scale, max(chunks))
    torch.cuda.synchronize()
    assert max_abs(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("scale", [0.0, -0.09, 1e-3, 0.4])
def test_prefill_any_scale(scale):
    """Zero scale (every visible key equally weighted) and a negative scale
    (the kernel folds the sign into the query) against the oracle."""
    rng = np.random.default_rng(21)
    chunks, ctxs = [70, 9], [150, 9]
    q, qsl, kp, vp, tables, lens = _random_chunks(rng, chunks, ctxs, 8, 2, 128, 32, "bf16")
    ref = oracle.prefill_chunk_attention(q, "bf16", qsl, kp, vp, "bf16", tables, lens, scale, 32, 2)
    gq = up(q, "bf16")
    out = torch.empty_like(gq)
    lib().pa_prefill_chunk(out, gq, up_int(qsl), up(kp, "bf16"), up(vp, "bf16"), up_int(tables),
                           up_int(lens), scale, max(chunks))
    torch.cuda.synchronize()
    assert max_abs(out, ref) <= TOL["bf16"]


FP8_CASES = [
    # (chunks, contexts, Hq, Hkv, D, bs, q dtype)
    ([5, 16, 1], [5, 40, 70], 4, 1, 128, 16, "bf16"),
    ([33, 100], [33, 300], 8, 2, 128, 32, "bf16"),
    ([64, 7], [200, 7], 32, 8, 128, 32, "f16"),
    ([17, 50], [60, 99], 2, 2, 64, 16, "f16"),
    ([40], [555], 8, 1, 64, 32, "bf16"),
    ([20, 9], [85, 9], 8, 2, 128, 8, "bf16"),
    ([70], [300], 4, 4, 64, 64, "f16"),
    ([33], [77], 16, 1, 128, 64, "bf16"),
    ([100], [130], 4, 1, 64, 8, "bf16"),
]


@pytest.mark.parametrize("chunks,ctxs,hq,hkv,d,bs,q_dt", FP8_CASES)
def test_prefill_fp8_cache_matches_oracle(chunks, ctxs, hq, hkv, d, bs, q_dt):
    """Prefill over an fp8 E4M3 cache with per-tensor scales: codes decoded
    exactly to the query type, the scales folded into the logit scale and
    the output."""
    rng = np.random.default_rng(sum(chunks) + 3 * hq + d + bs)
    q, qsl, kp, vp, tables, lens, ks, vs = _random_chunks(rng, chunks, ctxs, hq, hkv, d, bs,
                                                          "fp8_e4m3", q_dtype=q_dt)
    scale = 1.0 / np.sqrt(d)
    ref = oracle.prefill_chunk_attention(q, q_dt, qsl, kp, vp, "fp8_e4m3", tables, lens, scale, bs,
                                         hkv, k_scale=ks, v_scale=vs)
    gq = up(q, q_dt)
    out = torch.empty_like(gq)
    lib().pa_prefill_chunk(out, gq, up_int(qsl), up(kp, "fp8_e4m3"), up(vp, "fp8_e4m3"),
                           up_int(tables), up_int(lens), scale, max(chunks), k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert max_abs(out, ref) <= TOL[q_dt]


def test_prefill_fp8_70b_shaped_serving_step():
    """A 70B-shaped layer (64 query / 8 KV heads, head_dim 128, block 16, fp8
    cache with per-tensor scales, bf16 activations): four sequences each
    prefill a 512-token chunk after a 1,024-token prefix.  The chunk's bf16
    K/V is quantised into the pool by pa_reshape_and_cache, then
    pa_prefill_chunk reads the whole 1,536-token context through the table;
    the pools must equal the oracle's byte for byte and every output must
    match."""
    rng = np.random.default_rng(70)
    hq, hkv, d, bs, prefix, chunk, nseq = 64, 8, 128, 16, 1024, 512, 4
    ctx = prefix + chunk
    q, qsl, kp, vp, tables, lens, ks, vs = _random_chunks(rng, [chunk] * nseq, [ctx] * nseq, hq, hkv,
                                                          d, bs, "fp8_e4m3", q_dtype="bf16")
    # the chunk's rows are not in the pool yet: they arrive through the scatter
    nan = W.NAN_BITS["fp8_e4m3"]
    slots = np.zeros(nseq * chunk, np.int64)
    for s in range(nseq):
        for i in range(chunk):
            pos = prefix + i
            blk = int(tables[s, pos // bs])
            kp[blk, :, pos % bs, :] = nan
            vp[blk, :, pos % bs, :] = nan
            slots[s * chunk + i] = blk * bs + pos % bs
    new_k = W.to_bits(rng.standard_normal((nseq * chunk, hkv, d)).astype(np.float32), "bf16")
    new_v = W.to_bits(rng.standard_normal((nseq * chunk, hkv, d)).astype(np.float32), "bf16")
    okp, ovp = oracle.reshape_and_cache(kp, vp, "fp8_e4m3", new_k, new_v, "bf16", slots, bs, ks, vs)
    scale = 1.0 / np.sqrt(d)
    pa = lib()
    gk, gv = up(kp, "fp8_e4m3"), up(vp, "fp8_e4m3")
    pa.pa_reshape_and_cache(up(new_k, "bf16"), up(new_v, "bf16"), gk, gv, up_int(slots), ks, vs)
    gq = up(q, "bf16")
    out = torch.empty_like(gq)
    pa.pa_prefill_chunk(out, gq, up_int(qsl), gk, gv, up_int(tables), up_int(lens), scale, chunk,
                        k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(gk, "fp8_e4m3"), okp)
    assert np.array_equal(W.torch_to_bits(gv, "fp8_e4m3"), ovp)
    ref = oracle.prefill_chunk_attention(q, "bf16", qsl, okp, ovp, "fp8_e4m3", tables, lens, scale, bs,
                                         hkv, k_scale=ks, v_scale=vs)
    err = max_abs(out, ref)
    print(f"[prefill fp8] 70B-shaped step max-abs {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


def test_prefill_fp8_last_row_matches_fp8_decode():
    """The last row of a chunk over an fp8 cache equals the fp8 decode of the
    same context (two kernels, one result up to rounding)."""
    rng = np.random.default_rng(9)
    chunks, ctxs = [9, 30], [100, 64]
    q, qsl, kp, vp, tables, lens, ks, vs = _random_chunks(rng, chunks, ctxs, 8, 2, 128, 16, "fp8_e4m3",
                                                          q_dtype="bf16")
    pa = lib()
    gq = up(q, "bf16")
    gk, gv, gt, gl = up(kp, "fp8_e4m3"), up(vp, "fp8_e4m3"), up_int(tables), up_int(lens)
    out = torch.empty_like(gq)
    pa.pa_prefill_chunk(out, gq, up_int(qsl), gk, gv, gt, gl, 0.1, 30, k_scale=ks, v_scale=vs)
    last = gq[torch.tensor([8, 38], device=gq.device)].contiguous()
    dec = torch.empty_like(last)
    pa.pa_decode(dec, last, gk, gv, gt, gl, 0.1, max_seq_len=100, k_scale=ks, v_scale=vs,
                 partition_size=-1)
    torch.cuda.synchronize()
    assert np.abs(as_f64(out[[8, 38]]) - as_f64(dec)).max() <= TOL["bf16"]


F32_CASES = [
    # (chunks, contexts, Hq, Hkv, D, bs)
    ([1, 17, 33, 64], [1, 17, 33, 64], 2, 2, 64, 16),     # the tiny workload's lengths, whole prompts
    ([5, 16, 1], [5, 40, 70], 4, 1, 128, 16),
    ([33, 100], [33, 300], 12, 4, 64, 32),                 # group 3
    ([9], [77], 16, 1, 128, 8),
    ([70], [300], 4, 4, 64, 64),
]


@pytest.mark.parametrize("chunks,ctxs,hq,hkv,d,bs", F32_CASES)
def test_prefill_f32_matches_oracle(chunks, ctxs, hq, hkv, d, bs):
    rng = np.random.default_rng(sum(ctxs) + hq + bs)
    q, qsl, kp, vp, tables, lens = _random_chunks(rng, chunks, ctxs, hq, hkv, d, bs, "f32")
    scale = 1.0 / np.sqrt(d)
    ref = oracle.prefill_chunk_attention(q, "f32", qsl, kp, vp, "f32", tables, lens, scale, bs, hkv)
    gq = up(q, "f32")
    out = torch.empty_like(gq)
    lib().pa_prefill_chunk(out, gq, up_int(qsl), up(kp, "f32"), up(vp, "f32"), up_int(tables),
                           up_int(lens), scale, max(chunks))
    torch.cuda.synchronize()
    assert max_abs(out, ref) <= TOL["f32"]


INT8_CASES = [
    # (chunks, contexts, Hq, Hkv, D, bs, query type)
    ([5, 16, 1], [5, 40, 70], 4, 1, 128, 16, "bf16"),
    ([33, 100], [33, 300], 8, 2, 128, 32, "bf16"),
    ([64, 7], [200, 7], 32, 8, 128, 16, "f16"),
    ([20, 9], [85, 9], 8, 2, 128, 8, "bf16"),
    ([70], [300], 4, 4, 64, 64, "f16"),
    ([17, 50], [60, 99], 16, 1, 64, 16, "bf16"),
    ([100], [130], 4, 1, 64, 8, "f16"),
    ([40, 130], [555, 131], 64, 8, 128, 16, "bf16"),
]


def _prefill_int8(q, qsl, kp, vp, tables, lens, ks, vs, hkv, d, bs, q_dt, scale, max_q):
    gq = up(q, q_dt)
    out = torch.empty_like(gq)
    lib().pa_prefill_chunk_int8(out, gq, up_int(qsl), up(kp, "int8"), up(vp, "int8"),
                                torch.from_numpy(ks).to(gq.device), torch.from_numpy(vs).to(gq.device),
                                up_int(tables), up_int(lens), scale, max_q)
    torch.cuda.synchronize()
    ref = oracle.prefill_chunk_attention(q, q_dt, qsl, kp, vp, "int8", tables, lens, scale, bs, hkv,
                                         k_block_scales=ks, v_block_scales=vs)
    return out, ref


@pytest.mark.parametrize("chunks,ctxs,hq,hkv,d,bs,q_dt", INT8_CASES)
def test_prefill_int8_cache_matches_oracle(chunks, ctxs, hq, hkv, d, bs, q_dt):
    """Prefill over an INT8 cache with per-(block, KV head) scales ([ybb] 6.2):
    codes exact in the 16-bit operands, each key's block K scale on its score
    and V scale on its probability."""
    rng = np.random.default_rng(sum(chunks) + 5 * hq + d + bs)
    q, qsl, kp, vp, tables, lens, ks, vs = random_chunks_int8(rng, chunks, ctxs, hq, hkv, d, bs, q_dt)
    out, ref = _prefill_int8(q, qsl, kp, vp, tables, lens, ks, vs, hkv, d, bs, q_dt, 1.0 / np.sqrt(d),
                             max(chunks))
    assert max_abs(out, ref) <= TOL[q_dt]


def test_prefill_int8_last_row_matches_int8_decode():
    """The last row of each chunk over an int8 cache equals the int8 decode of
    its sequence (two kernels, one formula)."""
    rng = np.random.default_rng(808)
    chunks, ctxs, hq, hkv, d, bs = [9, 30], [100, 64], 8, 2, 128, 16
    q, qsl, kp, vp, tables, lens, ks, vs = random_chunks_int8(rng, chunks, ctxs, hq, hkv, d, bs, "bf16")
    out, _ = _prefill_int8(q, qsl, kp, vp, tables, lens, ks, vs, hkv, d, bs, "bf16", 0.1, 30)
    pa = lib()
    gq = up(q, "bf16")
    last = gq[torch.tensor([8, 38], device=gq.device)].contiguous()
    dec = torch.empty_like(last)
    pa.pa_decode_int8(dec, last, up(kp, "int8"), up(vp, "int8"), torch.from_numpy(ks).to(gq.device),
                      torch.from_numpy(vs).to(gq.device), up_int(tables), up_int(lens), 0.1, max_seq_len=100,
                      partition_size=-1)
    torch.cuda.synchronize()
    assert np.abs(as_f64(out[[8, 38]]) - as_f64(dec)).max() <= TOL["bf16"]


def test_prefill_int8_f16_queries_large_value_scales():
    """f16 queries over an int8 cache whose V values reach about 4e4 (block V
    scales near 300): the value operand p x scale must stay inside f16's
    range while the running max moves (queries x 6, logits spread widely)."""
    rng = np.random.default_rng(909)
    chunks, ctxs, hq, hkv, d, bs = [64, 33], [300, 700], 8, 2, 128, 16
    q, qsl, kp, vp, tables, lens, ks, vs = random_chunks_int8(rng, chunks, ctxs, hq, hkv, d, bs, "f16",
                                                              v_scale_mul=1.5e4)
    q = W.to_bits(W.bits_to_torch(q, "f16").float().numpy() * 6, "f16")
    assert float(vs.max()) > 300
    out, ref = _prefill_int8(q, qsl, kp, vp, tables, lens, ks, vs, hkv, d, bs, "f16", 1.0 / np.sqrt(d), 64)
    err = max_abs(out, ref)
    assert err <= TOL["f16"] * float(np.abs(ref).max()) / 4, err

