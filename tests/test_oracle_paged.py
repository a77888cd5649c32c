"""Pins for the oracle's paged-attention definitions (CPU only).

Each test checks the oracle against something other than itself: values the
pages print, closed forms, invariants, a library routine (torch's float64
scaled_dot_product_attention) or brute force with math.fsum.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W


def _f32_bits(x):
    return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)


def _random_paged(rng, lens, hkv, d, bs, nb=None, permute=True):
    """Random fp32 pool with the given lengths; returns (pool_k, pool_v, tables, K, V)
    where K/V are the contiguous per-sequence caches (float32 values)."""
    need = [-(-n // bs) for n in lens]
    nb = nb or (sum(need) + 3)
    ids = rng.permutation(nb) if permute else np.arange(nb)
    pk = np.full((nb, hkv, bs, d), np.nan, np.float32)
    pv = np.full((nb, hkv, bs, d), np.nan, np.float32)
    tables = np.full((len(lens), max(need)), nb - 1, np.int32)
    ks, vs = [], []
    cur = 0
    for s, n in enumerate(lens):
        k = rng.standard_normal((hkv, n, d)).astype(np.float32)
        v = rng.standard_normal((hkv, n, d)).astype(np.float32)
        ks.append(k)
        vs.append(v)
        for b in range(need[s]):
            phys = ids[cur]
            cur += 1
            tables[s, b] = phys
            lo, hi = b * bs, min(n, (b + 1) * bs)
            pk[phys, :, : hi - lo, :] = k[:, lo:hi, :]
            pv[phys, :, : hi - lo, :] = v[:, lo:hi, :]
    return _f32_bits(pk), _f32_bits(pv), tables, ks, vs


def _sdpa(q, k, v, scale, mask=None):
    """torch float64 SDPA; q [Hq][R][D], k/v [Hkv][N][D] -> [Hq][R][D]."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None]
    kt = torch.from_numpy(np.asarray(k, np.float64))[None]
    vt = torch.from_numpy(np.asarray(v, np.float64))[None]
    mt = None if mask is None else torch.from_numpy(mask)
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale, enable_gqa=True)
    return out[0].numpy()


# ---------------------------------------------------------------- index work

def test_block_count_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "datawhale_kv_cache_manager_example.json")))
    mgr = W.BlockManager(g["num_blocks"], g["block_size"])
    table = []
    for step in g["steps"]:
        if step["op"] == "prefill":
            table = mgr.allocate(step["seq_len"])
        else:
            mgr.grow(table, step["seq_len"])
        assert oracle.num_blocks(step["seq_len"], g["block_size"]) == len(table)
        if "table_len" in step:
            assert len(table) == step["table_len"]
        if "free_blocks" in step:
            assert len(mgr.free) == step["free_blocks"]


def test_block_count_brute_force():
    for bs in range(1, 34):
        for n in range(0, 200):
            k = 0
            while k * bs < n:
                k += 1
            assert oracle.num_blocks(n, bs) == k
            assert W.blocks_for(n, bs) == k


def test_block_counts_tiny_config():
    assert [oracle.num_blocks(n, 16) for n in (1, 17, 33, 64)] == [1, 2, 3, 4]


def test_mapping_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "bogosort_block_table_example.json")))
    for tok in g["tokens"]:
        got = oracle.locate_token(g["block_table"], tok["position"], g["block_size"])
        assert got == (tok["physical"], tok["offset"], tok["slot"])


def test_sentinel_gather(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "datawhale_kv_cache_manager_example.json")))
    mgr = W.BlockManager(g["num_blocks"], g["block_size"])
    table = mgr.allocate(g["steps"][0]["seq_len"])
    for step in g["steps"][1:]:
        mgr.grow(table, step["seq_len"])
    seq_len = g["steps"][-1]["seq_len"]
    pool = np.zeros((g["num_blocks"], 1, g["block_size"], g["head_dim"]), np.float32)
    sen = g["sentinel"]
    pool[table[sen["table_index"]], 0, sen["row"], sen["col"]] = sen["value"]
    cache = oracle.gather_sequence(_f32_bits(pool), "f32", table, seq_len, g["block_size"])[0]
    assert list(cache.shape) == sen["gathered_shape"]
    assert cache[sen["gathered_row"], sen["gathered_col"]] == sen["value"]


def test_gather_never_reads_past_length():
    rng = np.random.default_rng(1)
    pk, _, tables, ks, _ = _random_paged(rng, [5, 16, 17, 31], 2, 8, 16)
    for s, n in enumerate([5, 16, 17, 31]):
        got = oracle.gather_sequence(pk, "f32", tables[s], n, 16)
        assert not np.isnan(got).any()
        np.testing.assert_array_equal(got, ks[s].astype(np.float64))


# ------------------------------------------------------------- decode attention

@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1), (8, 2), (6, 3)])
@pytest.mark.parametrize("permute", [False, True])
def test_decode_matches_sdpa(hq, hkv, permute):
    rng = np.random.default_rng(hq * 10 + hkv + permute)
    lens = [1, 3, 16, 17, 40]
    d, bs = 16, 8
    pk, pv, tables, ks, vs = _random_paged(rng, lens, hkv, d, bs, permute=permute)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    scale = 0.37
    got = oracle.decode_attention(_f32_bits(q), "f32", pk, pv, "f32", tables, lens, scale, bs, hkv)
    for s in range(len(lens)):
        ref = _sdpa(q[s][:, None, :], ks[s], vs[s], scale)[:, 0, :]
        np.testing.assert_allclose(got[s], ref, rtol=0, atol=1e-12)


def test_decode_permutation_invariance_bitwise():
    rng = np.random.default_rng(7)
    lens = [9, 33, 64]
    pk, pv, tables, _, _ = _random_paged(rng, lens, 2, 16, 16, permute=False)
    q = _f32_bits(rng.standard_normal((3, 4, 16)))
    base = oracle.decode_attention(q, "f32", pk, pv, "f32", tables, lens, 0.25, 16, 2)
    nb = pk.shape[0]
    perm = rng.permutation(nb)            # new id of old block b is perm[b]
    pk2 = np.empty_like(pk)
    pv2 = np.empty_like(pv)
    pk2[perm] = pk
    pv2[perm] = pv
    tables2 = perm[tables].astype(np.int32)
    moved = oracle.decode_attention(q, "f32", pk2, pv2, "f32", tables2, lens, 0.25, 16, 2)
    assert np.array_equal(base, moved)


def test_length_one_returns_its_own_v():
    rng = np.random.default_rng(3)
    pk, pv, tables, _, vs = _random_paged(rng, [1, 1], 2, 32, 16)
    q = _f32_bits(rng.standard_normal((2, 4, 32)) * 10)
    out = oracle.decode_attention(q, "f32", pk, pv, "f32", tables, [1, 1], 0.5, 16, 2)
    for s in range(2):
        for h in range(4):
            assert np.array_equal(out[s, h], vs[s][h // 2, 0].astype(np.float64))


def test_constant_values_give_that_constant():
    rng = np.random.default_rng(4)
    pk, pv, tables, _, _ = _random_paged(rng, [23], 1, 8, 4)
    pv_vals = pv.view(np.float32).copy()
    pv_vals[~np.isnan(pv_vals)] = 0.625
    q = _f32_bits(rng.standard_normal((1, 3, 8)))
    out = oracle.decode_attention(q, "f32", pk, _f32_bits(pv_vals), "f32", tables, [23], 1.3, 4, 1)
    np.testing.assert_allclose(out, 0.625, rtol=0, atol=1e-15)


def test_zero_scale_gives_mean_of_values():
    rng = np.random.default_rng(5)
    pk, pv, tables, _, vs = _random_paged(rng, [37], 2, 8, 16)
    q = _f32_bits(rng.standard_normal((1, 2, 8)))
    out = oracle.decode_attention(q, "f32", pk, pv, "f32", tables, [37], 0.0, 16, 2)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], vs[0][h].astype(np.float64).mean(axis=0),
                                   rtol=0, atol=1e-14)


def test_dominant_logit_selects_its_value():
    rng = np.random.default_rng(6)
    lens = [20]
    pk, pv, tables, ks, vs = _random_paged(rng, lens, 1, 8, 4)
    target = 13
    q = ks[0][0, target][None, None, :] * 1.0
    out = oracle.decode_attention(_f32_bits(q), "f32", pk, pv, "f32", tables, lens, 200.0, 4, 1)
    np.testing.assert_allclose(out[0, 0], vs[0][0, target], rtol=0, atol=1e-9)


def test_decode_brute_force_fsum():
    """Pure-Python loops with exactly-rounded sums on the tiny fp32 workload."""
    case = W.make_decode_case("tiny_f32")
    spec = case.spec
    kp, vp = oracle.reshape_and_cache(case.k_pool, case.v_pool, "f32", case.new_k, case.new_v,
                                      "f32", case.slot_mapping, spec.block_size)
    got = oracle.decode_attention(case.q, "f32", kp, vp, "f32", case.block_tables, case.seq_lens,
                                  spec.scale, spec.block_size, spec.num_kv_heads)
    q = case.q.view(np.float32)
    kf = kp.view(np.float32)
    vf = vp.view(np.float32)
    bs = spec.block_size
    for s, n in enumerate(case.seq_lens):
        for h in range(spec.num_q_heads):
            kv = h // spec.group
            logits = []
            rows = []
            for j in range(int(n)):
                blk = int(case.block_tables[s, j // bs])
                krow = [float(x) for x in kf[blk, kv, j % bs]]
                logits.append(spec.scale * math.fsum(float(a) * b for a, b in zip(q[s, h], krow)))
                rows.append([float(x) for x in vf[blk, kv, j % bs]])
            m = max(logits)
            p = [math.exp(x - m) for x in logits]
            denom = math.fsum(p)
            for d in range(spec.head_dim):
                ref = math.fsum(pi * r[d] for pi, r in zip(p, rows)) / denom
                assert abs(got[s, h, d] - ref) <= 1e-13


def test_decode_ignores_block_table_padding():
    rng = np.random.default_rng(8)
    pk, pv, tables, _, _ = _random_paged(rng, [5, 40], 1, 8, 16)
    q = _f32_bits(rng.standard_normal((2, 1, 8)))
    a = oracle.decode_attention(q, "f32", pk, pv, "f32", tables, [5, 40], 0.3, 16, 1)
    t2 = tables.copy()
    t2[0, 1:] = 10 ** 6        # entries past ceil(len / bs) are never read
    b = oracle.decode_attention(q, "f32", pk, pv, "f32", t2, [5, 40], 0.3, 16, 1)
    assert np.array_equal(a, b)


def test_decode_scales_multiply_stored_values():
    rng = np.random.default_rng(9)
    pk, pv, tables, ks, vs = _random_paged(rng, [12], 1, 8, 4)
    q = rng.standard_normal((1, 2, 8)).astype(np.float32)
    got = oracle.decode_attention(_f32_bits(q), "f32", pk, pv, "f32", tables, [12], 0.5, 4, 1,
                                  k_scale=2.0, v_scale=0.25)
    ref = _sdpa(q[0][:, None, :], ks[0] * 2.0, vs[0] * 0.25, 0.5)[:, 0, :]
    np.testing.assert_allclose(got[0], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------------ prefill chunk

def _bottom_right_mask(rows, n):
    chunk = rows
    i = np.arange(chunk)[:, None]
    j = np.arange(n)[None, :]
    return j <= (n - chunk + i)


@pytest.mark.parametrize("chunk,ctx", [(5, 5), (4, 19), (9, 40), (1, 33)])
def test_prefill_matches_sdpa_bottom_right(chunk, ctx):
    rng = np.random.default_rng(chunk * 100 + ctx)
    hq, hkv, d, bs = 4, 2, 16, 8
    pk, pv, tables, ks, vs = _random_paged(rng, [ctx, ctx + 3], hkv, d, bs)
    lens = [ctx, ctx + 3]
    qsl = [0, chunk, 2 * chunk]
    q = rng.standard_normal((2 * chunk, hq, d)).astype(np.float32)
    got = oracle.prefill_chunk_attention(_f32_bits(q), "f32", qsl, pk, pv, "f32", tables, lens,
                                         0.3, bs, hkv)
    for s in range(2):
        rows = q[qsl[s]:qsl[s + 1]].transpose(1, 0, 2)
        # torch's is_causal aligns top-left when chunk != ctx, so the mask is explicit.
        ref = _sdpa(rows, ks[s], vs[s], 0.3, mask=_bottom_right_mask(chunk, lens[s]))
        np.testing.assert_allclose(got[qsl[s]:qsl[s + 1]], ref.transpose(1, 0, 2), rtol=0,
                                   atol=1e-12)


def test_prefill_last_row_equals_decode():
    rng = np.random.default_rng(11)
    lens = [21, 48]
    pk, pv, tables, _, _ = _random_paged(rng, lens, 2, 16, 8)
    q = rng.standard_normal((2 * 6, 4, 16)).astype(np.float32)
    qsl = [0, 6, 12]
    pre = oracle.prefill_chunk_attention(_f32_bits(q), "f32", qsl, pk, pv, "f32", tables, lens,
                                         0.25, 8, 2)
    last = q[[5, 11]]
    dec = oracle.decode_attention(_f32_bits(last), "f32", pk, pv, "f32", tables, lens, 0.25, 8, 2)
    # same arithmetic up to BLAS summation order
    np.testing.assert_allclose(pre[[5, 11]], dec, rtol=0, atol=1e-14)


def test_prefill_two_chunks_equal_one():
    rng = np.random.default_rng(12)
    ctx = 50
    pk, pv, tables, _, _ = _random_paged(rng, [ctx], 1, 8, 8)
    q = rng.standard_normal((16, 2, 8)).astype(np.float32)
    whole = oracle.prefill_chunk_attention(_f32_bits(q), "f32", [0, 16], pk, pv, "f32", tables,
                                           [ctx], 0.4, 8, 1)
    first = oracle.prefill_chunk_attention(_f32_bits(q[:8]), "f32", [0, 8], pk, pv, "f32", tables,
                                           [ctx - 8], 0.4, 8, 1)
    second = oracle.prefill_chunk_attention(_f32_bits(q[8:]), "f32", [0, 8], pk, pv, "f32",
                                            tables, [ctx], 0.4, 8, 1)
    np.testing.assert_allclose(whole, np.concatenate([first, second]), rtol=0, atol=1e-15)


def test_prefill_sampled_rows_match_full():
    rng = np.random.default_rng(13)
    lens = [30, 19]
    pk, pv, tables, _, _ = _random_paged(rng, lens, 2, 8, 8)
    q = _f32_bits(rng.standard_normal((10, 4, 8)))
    qsl = [0, 7, 10]
    full = oracle.prefill_chunk_attention(q, "f32", qsl, pk, pv, "f32", tables, lens, 0.5, 8, 2)
    rows = [(0, 0), (6, 3), (7, 1), (9, 2)]
    part = oracle.prefill_chunk_attention(q, "f32", qsl, pk, pv, "f32", tables, lens, 0.5, 8, 2,
                                          rows=rows)
    for i, (t, h) in enumerate(rows):
        np.testing.assert_allclose(part[i], full[t, h], rtol=0, atol=1e-14)


# ------------------------------------------------------ scatter and block copy

def test_reshape_and_cache_hand_example():
    nb, hkv, bs, d = 3, 2, 4, 2
    pool = np.full((nb, hkv, bs, d), 0xFFFF, np.uint16)
    key = np.arange(3 * hkv * d, dtype=np.uint16).reshape(3, hkv, d)
    val = key + 100
    slots = np.array([5, -1, 2], np.int64)      # block 1 row 1; skipped; block 0 row 2
    kp, vp = oracle.reshape_and_cache(pool, pool, "f16", key, val, "f16", slots, bs)
    expect_k = pool.copy()
    expect_k[1, :, 1, :] = [[0, 1], [2, 3]]
    expect_k[0, :, 2, :] = [[8, 9], [10, 11]]
    assert np.array_equal(kp, expect_k)
    expect_v = pool.copy()
    expect_v[1, :, 1, :] = [[100, 101], [102, 103]]
    expect_v[0, :, 2, :] = [[108, 109], [110, 111]]
    assert np.array_equal(vp, expect_v)
    assert np.array_equal(pool, np.full_like(pool, 0xFFFF))    # inputs untouched


def test_reshape_and_cache_fp8_hand_values():
    # bf16 bits: 1.0 = 0x3F80, -3.0 = 0xC040, 0.0 = 0, 1000.0 = 0x447A
    key = np.array([[[0x3F80, 0xC040, 0x0000, 0x447A]]], np.uint16)
    pool = np.zeros((1, 1, 2, 4), np.uint8)
    kp, vp = oracle.reshape_and_cache(pool, pool, "fp8_e4m3", key, key, "bf16",
                                      np.array([1], np.int64), 2, k_scale=0.5, v_scale=4.0)
    # k: x / 0.5 -> 2.0 (0x40), -6.0 (0xCC), 0.0 (0x00), 2000 -> saturates to 448 (0x7E)
    assert list(kp[0, 0, 1]) == [0x40, 0xCC, 0x00, 0x7E]
    # v: x / 4 -> 0.25 (0x28), -0.75 (0xB4), 0 (0x00), 250 -> 256 (0x78) under RNE
    assert list(vp[0, 0, 1]) == [0x28, 0xB4, 0x00, 0x78]
    assert list(kp[0, 0, 0]) == [0, 0, 0, 0]


def test_copy_blocks_hand_example():
    kp = np.arange(4 * 2 * 3, dtype=np.uint8).reshape(4, 2, 3, 1)
    vp = kp + 50
    k2, v2 = oracle.copy_blocks(kp, vp, [[0, 3], [2, 1]])
    assert np.array_equal(k2[3], kp[0]) and np.array_equal(k2[1], kp[2])
    assert np.array_equal(k2[0], kp[0]) and np.array_equal(k2[2], kp[2])
    assert np.array_equal(v2[3], vp[0]) and np.array_equal(v2[1], vp[2])


def test_copy_on_write_is_transparent():
    """Reading through the copied blocks gives bit-identical attention."""
    case = W.make_mixed_case(num_forks=3, prefix_len=64, chunk_len=8, num_decode=2,
                             decode_lens=[40, 70])
    spec = case.spec
    assert case.cow_pairs.shape == (2, 2)
    kp, vp = oracle.copy_blocks(case.k_pool, case.v_pool, case.cow_pairs)
    kp, vp = oracle.reshape_and_cache(kp, vp, "bf16", case.new_k, case.new_v, "bf16",
                                      case.slot_mapping, spec.block_size)
    # without the copy: the shared tables still name the original block
    ks, vs = oracle.reshape_and_cache(case.k_pool, case.v_pool, "bf16", case.new_k, case.new_v,
                                      "bf16", case.slot_mapping, spec.block_size)
    a = oracle.prefill_chunk_attention(case.q_chunk, "bf16", case.query_start_loc, kp, vp, "bf16",
                                       case.prefill_tables, case.prefill_lens, spec.scale,
                                       spec.block_size, spec.num_kv_heads)
    b = oracle.prefill_chunk_attention(case.q_chunk, "bf16", case.query_start_loc, ks, vs, "bf16",
                                       case.prefill_tables_shared, case.prefill_lens, spec.scale,
                                       spec.block_size, spec.num_kv_heads)
    assert np.array_equal(a, b)
    assert not np.isnan(a).any()


# ------------------------------------------------------------ byte accounting

def test_effective_bytes_match_llama2_7b_figure(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ybb_llama2_7b_kv_bytes.json")))
    per_tok = W.effective_kv_bytes([1], g["num_kv_heads"], g["head_dim"], g["cache_dtype"])
    assert per_tok == g["bytes_per_token_per_layer"]
    assert per_tok * g["layers"] == g["bytes_per_token_all_layers"]
    assert per_tok * g["layers"] * g["request_tokens"] == g["bytes_per_request_all_layers"]
