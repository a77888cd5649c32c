"""Host-side workload construction: determinism, sizing, block manager (CPU only)."""

import numpy as np
import pytest

import workloads as W


def test_decode_case_is_deterministic():
    a = W.make_decode_case("tiny_f32")
    b = W.make_decode_case("tiny_f32")
    for name in ("q", "k_pool", "v_pool", "block_tables", "seq_lens", "new_k", "new_v",
                 "slot_mapping"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    c = W.make_decode_case("tiny_f32", rep=1)
    assert not np.array_equal(a.q, c.q)


def test_decode_case_layout_and_poison():
    case = W.make_decode_case("tiny_f32")
    spec = case.spec
    assert case.k_pool.shape == (64, 2, 16, 64)
    assert list(case.seq_lens) == [1, 17, 33, 64]
    nb_used = [W.blocks_for(int(n), 16) for n in case.seq_lens]
    ids = np.concatenate([case.block_tables[s, :k] for s, k in enumerate(nb_used)])
    assert len(set(ids.tolist())) == len(ids)                    # no block shared
    assert case.poison_block not in set(ids.tolist())
    for s, k in enumerate(nb_used):
        assert np.all(case.block_tables[s, k:] == case.poison_block)
    # the newest token's slot holds NaN until the scatter writes it
    for s, slot in enumerate(case.slot_mapping):
        blk, row = slot // 16, slot % 16
        n = int(case.seq_lens[s])
        assert blk == case.block_tables[s, (n - 1) // 16] and row == (n - 1) % 16
        assert np.all(case.k_pool[blk, :, row, :] == W.NAN_BITS["f32"])
    assert np.all(case.k_pool[case.poison_block] == W.NAN_BITS["f32"])
    assert spec.scale == 1.0 / 8.0


def test_fp8_case_scales_cover_amax():
    case = W.make_decode_case("llama3_70b_fp8kv", num_seqs=6)
    valid = case.k_pool[case.k_pool != 0x7F]
    assert case.k_scale > 0 and case.v_scale > 0
    # some stored code reaches the top binade (the amax maps to ~448)
    assert ((valid & 0x7F) >= 0x78).any()


def test_pool_sizing_rules():
    c2 = W.make_decode_case("llama2_7b_mha_f16", num_seqs=4)
    assert c2.k_pool.shape[0] == 8192
    c3 = W.make_decode_case("llama3_8b_gqa_bf16", num_seqs=5)
    blocks = sum(W.blocks_for(int(n), 16) for n in c3.seq_lens)
    assert c3.k_pool.shape[0] == int(np.ceil(1.1 * blocks)) + 1
    assert c3.block_tables.shape == (5, 512)


def test_lognormal_lengths_are_clipped():
    rng = np.random.default_rng(0)
    lens = W.draw_lengths(("lognormal", 1200.0, 0.8, 16, 8192), 10000, rng)
    assert lens.min() >= 16 and lens.max() <= 8192
    assert 1000 < np.median(lens) < 1400


def test_block_manager_oom_and_refcounts():
    mgr = W.BlockManager(4, 2)
    t = mgr.allocate(3)
    assert len(t) == 2
    with pytest.raises(RuntimeError, match="OOM"):
        mgr.allocate(5)
    f = mgr.fork(t)
    assert all(mgr.ref[b] == 2 for b in t)
    pair = mgr.copy_on_write(f, 1)
    assert pair == (t[1], f[1]) and mgr.ref[t[1]] == 1 and mgr.ref[f[1]] == 1
    assert mgr.copy_on_write(f, 1) is None
    mgr.release(f)
    assert mgr.ref[t[0]] == 1
    mgr.release(t)
    assert sorted(mgr.free) == [0, 1, 2, 3]


def test_block_manager_grow_at_block_size_one():
    mgr = W.BlockManager(8, 1)
    t = mgr.allocate(2)
    mgr.grow(t, 3)
    assert len(t) == 3


def test_mixed_case_structure():
    case = W.make_mixed_case(num_forks=4, prefix_len=64, chunk_len=16, num_decode=3,
                             decode_lens=[33, 64, 65])
    bs = case.spec.block_size
    assert case.cow_pairs.shape == (3, 2)
    last = 64 // bs - 1
    original = case.prefill_tables_shared[0, last]
    assert np.all(case.prefill_tables_shared[:, last] == original)
    assert np.all(case.cow_pairs[:, 0] == original)
    # exactly one fork keeps the original block, the others hold distinct copies
    now = case.prefill_tables[:, last].tolist()
    assert now.count(original) == 1
    assert sorted(b for b in now if b != original) == sorted(case.cow_pairs[:, 1].tolist())
    # blocks before the divergent one stay shared
    assert np.all(case.prefill_tables[:, : last] == case.prefill_tables_shared[:, : last])
    assert case.slot_mapping.shape == (4 * 16 + 3,)
    assert len(set(case.slot_mapping.tolist())) == len(case.slot_mapping)
    assert list(case.query_start_loc) == [0, 16, 32, 48, 64]


def test_mixed_case_over_an_fp8_cache():
    """The fp8 mixed step: pools hold E4M3 codes, its bf16 activations and new
    rows are unchanged, and each per-tensor scale makes the largest magnitude
    the pool will hold (stored values or quantised new rows) code to 448."""
    import dataclasses
    import oracle
    spec = dataclasses.replace(W.MIXED_70B_FP8, num_q_heads=8, num_kv_heads=2, head_dim=64)
    case = W.make_mixed_case(spec, num_forks=2, prefix_len=32, chunk_len=16, decode_lens=[20, 50, 1])
    assert case.k_pool.dtype == np.uint8 and case.q_chunk.dtype == np.uint16
    assert 0 < case.k_scale and 0 < case.v_scale and case.k_scale != case.v_scale
    kp, vp = oracle.copy_blocks(case.k_pool, case.v_pool, case.cow_pairs)
    kp, vp = oracle.reshape_and_cache(kp, vp, "fp8_e4m3", case.new_k, case.new_v, "bf16", case.slot_mapping,
                                      spec.block_size, case.k_scale, case.v_scale)
    for pool in (kp, vp):
        vals = oracle.decode_elements(pool, "fp8_e4m3")
        finite = vals[np.isfinite(vals)]
        assert np.abs(finite).max() == 448.0



def test_mixed_case_over_an_int8_cache():
    """The int8 mixed step: one float32 scale per (block, KV head); after
    copy-on-write (codes and scales) and the int8 scatter, every block that
    holds tokens has, in each KV head, a code of magnitude 127 (its scale is
    the amax of what it holds over 127), and rows past each context keep the
    unwritten code -128."""
    import dataclasses
    import oracle
    spec = dataclasses.replace(W.MIXED_70B_INT8, num_q_heads=8, num_kv_heads=4, head_dim=64)
    case = W.make_mixed_case(spec, num_forks=2, prefix_len=32, chunk_len=16, decode_lens=[20, 50, 1])
    nb, h = case.k_pool.shape[:2]
    assert case.k_block_scales.shape == (nb, h) and case.k_block_scales.dtype == np.float32
    assert np.all(case.k_block_scales > 0) and np.all(case.v_block_scales > 0)
    kp, vp = oracle.copy_blocks(case.k_pool, case.v_pool, case.cow_pairs)
    ks, vs = oracle.copy_blocks(case.k_block_scales, case.v_block_scales, case.cow_pairs)
    kp, vp = oracle.reshape_and_cache(kp, vp, "int8", case.new_k, case.new_v, "bf16", case.slot_mapping,
                                      spec.block_size, k_block_scales=ks, v_block_scales=vs)
    bs = spec.block_size
    tables = [(t, int(n)) for t, n in zip(case.prefill_tables, case.prefill_lens)] + \
             [(t, int(n)) for t, n in zip(case.decode_tables, case.decode_lens)]
    for pool in (kp, vp):
        codes = pool.view(np.int8).astype(np.int32)
        for t, n in tables:
            flat = codes[t[: W.blocks_for(n, bs)]].transpose(1, 0, 2, 3).reshape(h, -1, spec.head_dim)
            assert np.all(np.abs(flat[:, :n]) <= 127)
            assert np.all(flat[:, n:] == -128)
            for b in range(W.blocks_for(n, bs)):
                assert np.all(np.abs(flat[:, b * bs: min(n, (b + 1) * bs)]).max(axis=(1, 2)) == 127)
