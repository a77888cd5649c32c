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



# ------------------------------------------------------------ fp8 K beside a bf16 V pool

def _mixed_pools(rng, lens, hkv, d, bs):
    """An fp8 K pool and a bf16 V pool with the given lengths, plus float32
    pools holding exactly the same values (both formats are exact in float32)."""
    need = [-(-n // bs) for n in lens]
    nb = sum(need) + 2
    ids = rng.permutation(nb)
    k8 = rng.integers(0, 256, (nb, hkv, bs, d)).astype(np.uint8)
    k8[(k8 & 0x7F) == 0x7F] = 0x3C             # no NaN codes
    vb = W.to_bits(rng.standard_normal((nb, hkv, bs, d)).astype(np.float32), "bf16")
    kf = oracle.decode_elements(k8, "fp8_e4m3").astype(np.float32)
    vf = oracle.decode_elements(vb, "bf16").astype(np.float32)
    tables = np.full((len(lens), max(need)), nb - 1, np.int32)
    cur = 0
    for s, n in enumerate(lens):
        tables[s, :need[s]] = ids[cur:cur + need[s]]
        cur += need[s]
    return k8, vb, _f32_bits(kf), _f32_bits(vf), tables


def test_mixed_pools_equal_float32_pools_of_the_same_values():
    # intelliparadigm page §6.1: fp8 K cache, bf16 V cache.  Reading each pool
    # in its own format must give the attention over the decoded values, which
    # float32 pools hold exactly; decoding V as fp8 (or K as bf16) would not.
    rng = np.random.default_rng(21)
    lens = [1, 17, 40]
    k8, vb, kf, vf, tables = _mixed_pools(rng, lens, 2, 16, 8)
    q = W.to_bits(rng.standard_normal((3, 4, 16)).astype(np.float32), "bf16")
    got = oracle.decode_attention(q, "bf16", k8, vb, "fp8_e4m3", tables, lens, 0.3, 8, 2,
                                  k_scale=0.05, v_scale=1.5, v_cache_dtype="bf16")
    ref = oracle.decode_attention(q, "bf16", kf, vf, "f32", tables, lens, 0.3, 8, 2,
                                  k_scale=0.05, v_scale=1.5)
    assert np.array_equal(got, ref)


def test_mixed_length_one_returns_its_scaled_bf16_value():
    rng = np.random.default_rng(22)
    k8, vb, _, _, tables = _mixed_pools(rng, [1], 1, 8, 16)
    q = W.to_bits(rng.standard_normal((1, 2, 8)).astype(np.float32), "bf16")
    out = oracle.decode_attention(q, "bf16", k8, vb, "fp8_e4m3", tables, [1], 0.5, 16, 1,
                                  k_scale=3.0, v_scale=0.5, v_cache_dtype="bf16")
    blk = tables[0, 0]
    v = oracle.decode_elements(vb[blk, 0, 0], "bf16") * 0.5
    for h in range(2):
        assert np.array_equal(out[0, h], v)


def test_mixed_scatter_is_fp8_k_and_copied_v():
    rng = np.random.default_rng(23)
    key = W.to_bits(rng.standard_normal((5, 2, 16)).astype(np.float32) * 30, "bf16")
    val = W.to_bits(rng.standard_normal((5, 2, 16)).astype(np.float32), "bf16")
    slots = np.array([3, -1, 0, 9, 6], np.int64)
    k0 = np.zeros((3, 2, 4, 16), np.uint8)
    v0 = np.zeros((3, 2, 4, 16), np.uint16)
    km, vm = oracle.reshape_and_cache(k0, v0, "fp8_e4m3", key, val, "bf16", slots, 4,
                                      k_scale=0.25, v_scale=7.0, v_cache_dtype="bf16")
    k8, _ = oracle.reshape_and_cache(k0, k0, "fp8_e4m3", key, val, "bf16", slots, 4,
                                     k_scale=0.25, v_scale=7.0)
    _, v16 = oracle.reshape_and_cache(v0, v0, "bf16", key, val, "bf16", slots, 4)
    assert np.array_equal(km, k8) and np.array_equal(vm, v16)
    # the copied V rows are the source bits (slot = block * 4 + row); rows no
    # slot names, like the skipped token's, keep their old contents
    assert np.array_equal(vm[0, :, 3], val[0]) and np.array_equal(vm[2, :, 1], val[3])
    assert np.array_equal(vm[1, :, 2], val[4]) and np.array_equal(vm[0, :, 0], val[2])
    assert not vm[1, :, 0].any() and not vm[2, :, 0].any()



# ------------------------------------------------------------ int8 cache with per-block scales

def test_int8_codec_hand_values():
    x = np.array([2.5, 3.5, -2.5, -3.5, 126.7, 127.5, 1000.0, -1000.0, np.nan, np.inf, 0.49,
                  -0.5, 1.0000001], np.float32)
    got = oracle.int8_encode(x, np.float32(1.0))
    assert list(got) == [2, 4, -2, -4, 127, 127, 127, -127, 0, 127, 0, 0, 1]
    # one float32 division, then round half to even
    assert oracle.int8_encode(np.float32(0.3), np.float32(0.1)) == 3
    assert oracle.int8_encode(np.float32(-7.0), np.float32(2.0)) == -4      # -3.5 -> -4 (even)


def _int8_pools(rng, lens, hkv, d, bs):
    need = [-(-n // bs) for n in lens]
    nb = sum(need) + 2
    ids = rng.permutation(nb)
    kc = rng.integers(-127, 128, (nb, hkv, bs, d)).astype(np.int8)
    vc = rng.integers(-127, 128, (nb, hkv, bs, d)).astype(np.int8)
    ks = (rng.uniform(0.5, 2.0, (nb, hkv)) / 127).astype(np.float32)
    vs = (rng.uniform(0.5, 2.0, (nb, hkv)) / 127).astype(np.float32)
    tables = np.full((len(lens), max(need)), nb - 1, np.int32)
    cur = 0
    for s, n in enumerate(lens):
        tables[s, :need[s]] = ids[cur:cur + need[s]]
        cur += need[s]
    return kc, vc, ks, vs, tables


def test_int8_uniform_scales_equal_the_per_tensor_path():
    # every block with the same scale: the per-block path must equal codes held
    # exactly in float32 pools with that scale applied per tensor
    rng = np.random.default_rng(31)
    lens = [1, 9, 40]
    kc, vc, _, _, tables = _int8_pools(rng, lens, 2, 16, 8)
    nb = kc.shape[0]
    ks = np.full((nb, 2), np.float32(0.013), np.float32)
    vs = np.full((nb, 2), np.float32(0.021), np.float32)
    q = W.to_bits(rng.standard_normal((3, 4, 16)).astype(np.float32), "bf16")
    got = oracle.decode_attention(q, "bf16", kc.view(np.uint8), vc.view(np.uint8), "int8", tables,
                                  lens, 0.25, 8, 2, k_block_scales=ks, v_block_scales=vs)
    ref = oracle.decode_attention(q, "bf16", _f32_bits(kc.astype(np.float32)),
                                  _f32_bits(vc.astype(np.float32)), "f32", tables, lens, 0.25, 8, 2,
                                  k_scale=float(np.float32(0.013)), v_scale=float(np.float32(0.021)))
    assert np.array_equal(got, ref)


def test_int8_per_block_scales_match_sdpa_of_dequantised_cache():
    rng = np.random.default_rng(32)
    lens = [23, 50]
    bs, hkv, d = 8, 2, 16
    kc, vc, ks, vs, tables = _int8_pools(rng, lens, hkv, d, bs)
    qf = rng.standard_normal((2, 4, d)).astype(np.float32)
    got = oracle.decode_attention(_f32_bits(qf), "f32", kc.view(np.uint8), vc.view(np.uint8), "int8",
                                  tables, lens, 0.3, bs, hkv, k_block_scales=ks, v_block_scales=vs)
    for s, n in enumerate(lens):
        keys = np.zeros((hkv, n, d))
        vals = np.zeros((hkv, n, d))
        for p in range(n):                       # token by token, through the block table
            b = tables[s, p // bs]
            for h in range(hkv):
                keys[h, p] = kc[b, h, p % bs].astype(np.float64) * np.float64(ks[b, h])
                vals[h, p] = vc[b, h, p % bs].astype(np.float64) * np.float64(vs[b, h])
        ref = _sdpa(qf[s][:, None, :], keys, vals, 0.3)[:, 0, :]
        np.testing.assert_allclose(got[s], ref, rtol=0, atol=1e-12)


def test_int8_prefill_per_block_scales_match_sdpa_of_dequantised_cache():
    # a chunk over an int8 context: each key and value is its code times its
    # block's scale, looked up token by token here; chunk query i at position
    # n - L + i sees keys 0 .. n - L + i
    rng = np.random.default_rng(33)
    lens, chunks = [23, 50], [5, 17]
    bs, hkv, d, hq = 8, 2, 16, 4
    kc, vc, ks, vs, tables = _int8_pools(rng, lens, hkv, d, bs)
    qsl = np.array([0, 5, 22], np.int32)
    qf = rng.standard_normal((22, hq, d)).astype(np.float32)
    got = oracle.prefill_chunk_attention(_f32_bits(qf), "f32", qsl, kc.view(np.uint8), vc.view(np.uint8),
                                         "int8", tables, lens, 0.3, bs, hkv, k_block_scales=ks,
                                         v_block_scales=vs)
    for s, (n, L) in enumerate(zip(lens, chunks)):
        keys = np.zeros((hkv, n, d))
        vals = np.zeros((hkv, n, d))
        for p in range(n):
            b = tables[s, p // bs]
            for h in range(hkv):
                keys[h, p] = kc[b, h, p % bs].astype(np.float64) * np.float64(ks[b, h])
                vals[h, p] = vc[b, h, p % bs].astype(np.float64) * np.float64(vs[b, h])
        for i in range(L):
            vis = n - L + i + 1
            for h in range(hq):
                ref = _sdpa(qf[qsl[s] + i, h][None, None, :], keys[h // 2:h // 2 + 1, :vis],
                            vals[h // 2:h // 2 + 1, :vis], 0.3)[0, 0]
                np.testing.assert_allclose(got[qsl[s] + i, h], ref, rtol=0, atol=1e-12)


def test_int8_scatter_uses_each_blocks_scale():
    key = np.array([[[1.0, -2.0, 0.3, 100.0]], [[0.5, 0.25, -0.75, 3.0]]], np.float32)
    pool = np.zeros((3, 1, 2, 4), np.uint8)
    ks = np.array([[0.5], [0.25], [1.0]], np.float32)
    vs = np.array([[1.0], [1.0], [0.1]], np.float32)
    slots = np.array([5, 0], np.int64)              # token 0 -> block 2 row 1, token 1 -> block 0 row 0
    kp, vp = oracle.reshape_and_cache(pool, pool, "int8", _f32_bits(key), _f32_bits(key), "f32",
                                      slots, 2, k_block_scales=ks, v_block_scales=vs)
    k = kp.view(np.int8)
    v = vp.view(np.int8)
    assert list(k[2, 0, 1]) == [1, -2, 0, 100]       # scale 1.0
    assert list(k[0, 0, 0]) == [1, 0, -2, 6]         # scale 0.5: 1, 0.5 -> 0, -1.5 -> -2, 6
    assert list(v[2, 0, 1]) == [10, -20, 3, 127]     # scale 0.1 (100 / 0.1 saturates)
    assert list(v[0, 0, 0]) == [0, 0, -1, 3]         # scale 1.0: 0.5 -> 0, 0.25 -> 0, -0.75 -> -1
    assert not k[1].any() and not v[1].any()


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


def _random_pools(rng, nb, hkv, bs, d):
    kp = rng.integers(0, 2 ** 16, size=(nb, hkv, bs, d), dtype=np.uint64).astype(np.uint16)
    vp = rng.integers(0, 2 ** 16, size=(nb, hkv, bs, d), dtype=np.uint64).astype(np.uint16)
    return kp, vp


def test_copy_block_rows_brute_force():
    """Element by element: row r of head h of block b changes only when b is a
    destination and r < the clamped count, and then takes the source's row."""
    rng = np.random.default_rng(11)
    nb, hkv, bs, d = 10, 2, 4, 3
    kp, vp = _random_pools(rng, nb, hkv, bs, d)
    triples = np.array([[0, 5, 2], [1, 6, 0], [2, 7, 4], [3, 8, 9], [4, 9, -3]], dtype=np.int64)
    k2, v2 = oracle.copy_block_rows(kp, vp, triples)
    dst_of = {int(t[1]): (int(t[0]), int(t[2])) for t in triples}
    for b in range(nb):
        for h in range(hkv):
            for r in range(bs):
                for e in range(d):
                    want_k, want_v = kp[b, h, r, e], vp[b, h, r, e]
                    if b in dst_of:
                        src, n = dst_of[b]
                        if r < max(0, min(n, bs)):
                            want_k, want_v = kp[src, h, r, e], vp[src, h, r, e]
                    assert k2[b, h, r, e] == want_k and v2[b, h, r, e] == want_v


def test_copy_block_rows_whole_block_equals_copy_blocks():
    rng = np.random.default_rng(12)
    kp, vp = _random_pools(rng, 6, 3, 8, 4)
    pairs = np.array([[0, 3], [1, 4], [2, 5]], dtype=np.int64)
    full_k, full_v = oracle.copy_blocks(kp, vp, pairs)
    for n in (8, 50):   # the block size and beyond it (clamped)
        triples = np.concatenate([pairs, np.full((3, 1), n, dtype=np.int64)], axis=1)
        k2, v2 = oracle.copy_block_rows(kp, vp, triples)
        assert np.array_equal(k2, full_k) and np.array_equal(v2, full_v)
    k0, v0 = oracle.copy_block_rows(kp, vp, np.concatenate([pairs, np.zeros((3, 1), np.int64)], axis=1))
    assert np.array_equal(k0, kp) and np.array_equal(v0, vp)


def test_partial_fork_is_transparent():
    """A sequence forked inside a block reads the same attention through the
    partial copy of that block as through the shared block."""
    rng = np.random.default_rng(13)
    nb, hkv, hq, bs, d, length = 12, 2, 4, 16, 64, 37     # 37 = 2 blocks + 5 rows
    kp = W.to_bits(rng.standard_normal((nb, hkv, bs, d)).astype(np.float32), "bf16")
    vp = W.to_bits(rng.standard_normal((nb, hkv, bs, d)).astype(np.float32), "bf16")
    q = W.to_bits(rng.standard_normal((1, hq, d)).astype(np.float32), "bf16")
    parent = np.array([[3, 7, 1]], dtype=np.int32)
    child = np.array([[3, 7, 10]], dtype=np.int32)        # tail block 1 copied into 10
    k2, v2 = oracle.copy_block_rows(kp, vp, [[1, 10, length % bs]])
    lens = np.array([length], dtype=np.int32)
    a = oracle.decode_attention(q, "bf16", kp, vp, "bf16", parent, lens, 0.125, bs, hkv)
    b = oracle.decode_attention(q, "bf16", k2, v2, "bf16", child, lens, 0.125, bs, hkv)
    assert np.array_equal(a, b)


def test_copy_blocks_layers_brute_force():
    rng = np.random.default_rng(14)
    layers = [_random_pools(rng, 5, 2, 4, 2) for _ in range(3)]
    pairs = np.array([[0, 2], [4, 1]], dtype=np.int64)
    ks, vs = oracle.copy_blocks_layers([l[0] for l in layers], [l[1] for l in layers], pairs)
    for (kp, vp), k2, v2 in zip(layers, ks, vs):
        for b in range(5):
            src = {2: 0, 1: 4}.get(b, b)
            assert np.array_equal(k2[b], kp[src]) and np.array_equal(v2[b], vp[src])


def test_swap_out_and_back_in_restores_blocks():
    """Swapping blocks out to a (smaller) host pool and back into freed slots
    of the device pool gives back the same bytes at the new places."""
    rng = np.random.default_rng(15)
    dev, _ = _random_pools(rng, 10, 2, 4, 3)
    host = np.zeros((4, 2, 4, 3), dtype=np.uint16)
    out_pairs = np.array([[7, 0], [2, 3], [5, 1]], dtype=np.int64)     # device -> host slot
    host2 = oracle.swap_blocks(host, dev, out_pairs)
    for src, dst in out_pairs:
        assert np.array_equal(host2[dst], dev[src])
    assert not host2[2].any()                                          # untouched slot
    in_pairs = np.array([[0, 9], [3, 8], [1, 0]], dtype=np.int64)      # host slot -> new device block
    dev2 = oracle.swap_blocks(dev, host2, in_pairs)
    assert np.array_equal(dev2[9], dev[7]) and np.array_equal(dev2[8], dev[2])
    assert np.array_equal(dev2[0], dev[5])
    for b in range(1, 8):
        assert np.array_equal(dev2[b], dev[b])


# ------------------------------------------------------------ byte accounting

def test_effective_bytes_match_llama2_7b_figure(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ybb_llama2_7b_kv_bytes.json")))
    per_tok = W.effective_kv_bytes([1], g["num_kv_heads"], g["head_dim"], g["cache_dtype"])
    assert per_tok == g["bytes_per_token_per_layer"]
    assert per_tok * g["layers"] == g["bytes_per_token_all_layers"]
    assert per_tok * g["layers"] * g["request_tokens"] == g["bytes_per_request_all_layers"]
