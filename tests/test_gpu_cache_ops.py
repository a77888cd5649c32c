"""GPU byte-exact parity of pa_reshape_and_cache and pa_copy_blocks."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_cases import lib, up, up_int

pytestmark = pytest.mark.gpu


def _pools(nb, hkv, bs, d, dtype, rng):
    bits = rng.integers(0, 2 ** (8 * W.ELEM_BYTES[dtype]), size=(nb, hkv, bs, d),
                        dtype=np.uint64).astype(W.BITS_DTYPE[dtype])
    return bits, bits.copy()


@pytest.mark.parametrize("dtype,hkv,d,bs", [("f32", 2, 64, 16), ("f16", 32, 128, 16),
                                            ("bf16", 8, 128, 32), ("bf16", 3, 64, 32)])
def test_scatter_same_type_bytes(dtype, hkv, d, bs):
    rng = np.random.default_rng(1)
    nb, t = 40, 97
    kp, vp = _pools(nb, hkv, bs, d, dtype, rng)
    key = rng.integers(0, 2 ** 16, size=(t, hkv, d), dtype=np.uint64).astype(W.BITS_DTYPE[dtype])
    val = rng.integers(0, 2 ** 16, size=(t, hkv, d), dtype=np.uint64).astype(W.BITS_DTYPE[dtype])
    slots = rng.choice(nb * bs, size=t, replace=False).astype(np.int64)
    slots[::7] = -1
    okp, ovp = oracle.reshape_and_cache(kp, vp, dtype, key, val, dtype, slots, bs)
    gk, gv = up(kp, dtype), up(vp, dtype)
    lib().pa_reshape_and_cache(up(key, dtype), up(val, dtype), gk, gv, up_int(slots))
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(gk, dtype), okp)
    assert np.array_equal(W.torch_to_bits(gv, dtype), ovp)


def test_scatter_strided_rows():
    """K/V rows taken as views of a wider per-token buffer (e.g. a fused QKV output)."""
    rng = np.random.default_rng(2)
    nb, hkv, bs, d, t = 8, 2, 16, 128, 10
    kp, vp = _pools(nb, hkv, bs, d, "bf16", rng)
    fused = rng.integers(0, 2 ** 16, size=(t, 3 * hkv, d), dtype=np.uint64).astype(np.uint16)
    slots = rng.choice(nb * bs, size=t, replace=False).astype(np.int64)
    g = up(fused, "bf16")
    key, val = g[:, hkv:2 * hkv, :], g[:, 2 * hkv:, :]
    okp, ovp = oracle.reshape_and_cache(kp, vp, "bf16", fused[:, hkv:2 * hkv], fused[:, 2 * hkv:],
                                        "bf16", slots, bs)
    gk, gv = up(kp, "bf16"), up(vp, "bf16")
    lib().pa_reshape_and_cache(key, val, gk, gv, up_int(slots))
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(gk, "bf16"), okp)
    assert np.array_equal(W.torch_to_bits(gv, "bf16"), ovp)


@pytest.mark.parametrize("scale", [1.0, 0.013489825651049614, 3.75, 2.0 ** -10, 1e-30])
def test_scatter_fp8_every_bf16_input(scale):
    """All 65,536 bf16 bit patterns (NaN, inf, subnormals, ties) through the quantiser."""
    hkv, d, bs = 4, 128, 16
    t = 65536 // (hkv * d)
    key = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(t, hkv, d)
    val = key[::-1].copy()
    nb = t
    kp = np.zeros((nb, hkv, bs, d), np.uint8)
    vp = np.zeros((nb, hkv, bs, d), np.uint8)
    slots = (np.arange(t, dtype=np.int64) * bs + 3)
    sc = float(np.float32(scale))
    okp, ovp = oracle.reshape_and_cache(kp, vp, "fp8_e4m3", key, val, "bf16", slots, bs,
                                        k_scale=sc, v_scale=sc * 2)
    gk, gv = up(kp, "fp8_e4m3"), up(vp, "fp8_e4m3")
    lib().pa_reshape_and_cache(up(key, "bf16"), up(val, "bf16"), gk, gv, up_int(slots),
                               k_scale=sc, v_scale=sc * 2)
    torch.cuda.synchronize()
    got_k, got_v = W.torch_to_bits(gk, "fp8_e4m3"), W.torch_to_bits(gv, "fp8_e4m3")
    bad = np.nonzero(got_k != okp)
    assert bad[0].size == 0, f"{bad[0].size} K codes differ, e.g. got {got_k[bad][:5]} want {okp[bad][:5]}"
    assert np.array_equal(got_v, ovp)


def test_scatter_fp8_from_f32_edge_values():
    hkv, d, bs = 1, 64, 16
    rng = np.random.default_rng(3)
    t4 = oracle.e4m3_value_table()[:0x7E]
    mids = ((t4[:-1] + t4[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(-np.inf)), -mids,
                           rng.standard_normal(2000).astype(np.float32) * 100,
                           np.array([0.0, -0.0, 448.0, 464.0, 1e9, -np.inf, np.inf, np.nan,
                                     2 ** -10, 2 ** -126, 1e-45], np.float32)])
    n = -(-len(vals) // d) * d
    vals = np.concatenate([vals, np.zeros(n - len(vals), np.float32)]).reshape(-1, hkv, d)
    t = vals.shape[0]
    key = vals.view(np.uint32)
    kp = np.zeros((t, hkv, bs, d), np.uint8)
    slots = np.arange(t, dtype=np.int64) * bs
    okp, _ = oracle.reshape_and_cache(kp, kp, "fp8_e4m3", key, key, "f32", slots, bs)
    gk, gv = up(kp, "fp8_e4m3"), up(kp, "fp8_e4m3")
    lib().pa_reshape_and_cache(up(key, "f32"), up(key, "f32"), gk, gv, up_int(slots))
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(gk, "fp8_e4m3"), okp)


@pytest.mark.parametrize("dtype,hkv,bs,d", [("bf16", 8, 32, 128), ("fp8_e4m3", 8, 16, 128),
                                            ("f32", 2, 16, 64)])
def test_copy_blocks_bytes(dtype, hkv, bs, d):
    rng = np.random.default_rng(4)
    nb = 64
    kp, _ = _pools(nb, hkv, bs, d, dtype, rng)
    vp, _ = _pools(nb, hkv, bs, d, dtype, rng)
    ids = rng.permutation(nb)
    pairs = np.stack([ids[:15], ids[15:30]], axis=1).astype(np.int64)
    okp, ovp = oracle.copy_blocks(kp, vp, pairs)
    gk, gv = up(kp, dtype), up(vp, dtype)
    lib().pa_copy_blocks(gk, gv, up_int(pairs))
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(gk, dtype), okp)
    assert np.array_equal(W.torch_to_bits(gv, dtype), ovp)


def test_empty_calls_are_noops():
    pa = lib()
    gk = up(np.zeros((2, 1, 16, 64), np.uint16), "bf16")
    before = gk.clone()
    empty = torch.empty((0, 1, 64), dtype=torch.bfloat16, device=gk.device)
    pa.pa_reshape_and_cache(empty, empty, gk, gk, up_int(np.zeros(0, np.int64)))
    pa.pa_copy_blocks(gk, gk, up_int(np.zeros((0, 2), np.int64)))
    torch.cuda.synchronize()
    assert torch.equal(gk, before)


@pytest.mark.parametrize("dtype,hkv,bs,d", [("bf16", 8, 32, 128), ("fp8_e4m3", 8, 16, 128),
                                            ("f32", 2, 16, 64), ("f16", 3, 32, 64)])
def test_copy_blocks_partial_bytes(dtype, hkv, bs, d):
    """Token-granular copy-on-write: counts 0, 1, mid, whole block, beyond the
    block and negative (clamped), whole pools compared byte for byte."""
    rng = np.random.default_rng(5)
    nb = 48
    kp, _ = _pools(nb, hkv, bs, d, dtype, rng)
    vp, _ = _pools(nb, hkv, bs, d, dtype, rng)
    ids = rng.permutation(nb)
    counts = np.array([0, 1, bs // 2, bs - 1, bs, bs + 7, -4, 3, bs // 3, 2, 5, bs], dtype=np.int64)
    triples = np.stack([ids[:12], ids[12:24], counts], axis=1).astype(np.int64)
    okp, ovp = oracle.copy_block_rows(kp, vp, triples)
    gk, gv = up(kp, dtype), up(vp, dtype)
    lib().pa_copy_blocks_partial(gk, gv, up_int(triples))
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(gk, dtype), okp)
    assert np.array_equal(W.torch_to_bits(gv, dtype), ovp)


@pytest.mark.parametrize("form", ["lists", "addresses"])
def test_copy_blocks_layers_bytes(form):
    """One launch applies the block copies to the K and V pools of 5 layers."""
    rng = np.random.default_rng(6)
    nb, hkv, bs, d, layers = 40, 8, 32, 128, 5
    kps = [_pools(nb, hkv, bs, d, "bf16", rng)[0] for _ in range(layers)]
    vps = [_pools(nb, hkv, bs, d, "bf16", rng)[0] for _ in range(layers)]
    ids = rng.permutation(nb)
    pairs = np.stack([ids[:9], ids[9:18]], axis=1).astype(np.int64)
    oks, ovs = oracle.copy_blocks_layers(kps, vps, pairs)
    gks, gvs = [up(k, "bf16") for k in kps], [up(v, "bf16") for v in vps]
    pa = lib()
    if form == "lists":
        pa.pa_copy_blocks_layers(gks, gvs, up_int(pairs))
    else:
        kp = pa.layer_pool_pointers(gks, gks[0].device)
        vp = pa.layer_pool_pointers(gvs, gvs[0].device)
        pa.pa_copy_blocks_layers(kp, vp, up_int(pairs), block_bytes=hkv * bs * d * 2)
    torch.cuda.synchronize()
    for gk, gv, ok, ov in zip(gks, gvs, oks, ovs):
        assert np.array_equal(W.torch_to_bits(gk, "bf16"), ok)
        assert np.array_equal(W.torch_to_bits(gv, "bf16"), ov)


@pytest.mark.parametrize("dtype", ["bf16", "fp8_e4m3"])
def test_swap_blocks_out_to_pinned_host_and_back(dtype):
    """Swap-out from the device pool into a pinned host pool, then swap-in into
    other device blocks; both steps match the oracle byte for byte."""
    rng = np.random.default_rng(7)
    nb, nh, hkv, bs, d = 64, 24, 8, 16, 128
    dev_bits, _ = _pools(nb, hkv, bs, d, dtype, rng)
    host_bits, _ = _pools(nh, hkv, bs, d, dtype, rng)
    ids = rng.permutation(nb)
    out_pairs = np.stack([ids[:20], rng.permutation(nh)[:20]], axis=1).astype(np.int64)
    want_host = oracle.swap_blocks(host_bits, dev_bits, out_pairs)
    g = up(dev_bits, dtype)
    h = W.bits_to_torch(host_bits, dtype).pin_memory()
    pa = lib()
    pa.pa_swap_blocks(h, g, up_int(out_pairs))
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(h, dtype), want_host)
    in_pairs = np.stack([out_pairs[:, 1], ids[20:40]], axis=1).astype(np.int64)
    want_dev = oracle.swap_blocks(dev_bits, want_host, in_pairs)
    pa.pa_swap_blocks(g, h, up_int(in_pairs))
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(g, dtype), want_dev)


def test_swap_blocks_device_to_device():
    rng = np.random.default_rng(8)
    a_bits, _ = _pools(30, 4, 32, 64, "f16", rng)
    b_bits, _ = _pools(20, 4, 32, 64, "f16", rng)
    pairs = np.stack([rng.permutation(30)[:11], rng.permutation(20)[:11]], axis=1).astype(np.int64)
    want = oracle.swap_blocks(b_bits, a_bits, pairs)
    ga, gb = up(a_bits, "f16"), up(b_bits, "f16")
    lib().pa_swap_blocks(gb, ga, up_int(pairs))
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(gb, "f16"), want)
    assert np.array_equal(W.torch_to_bits(ga, "f16"), a_bits)


def test_swap_blocks_rejects_pageable_host_memory():
    """A pageable host pool is refused before any launch."""
    pa = lib()
    g = up(np.zeros((4, 1, 16, 64), np.uint16), "bf16")
    pageable = torch.zeros((4, 1, 16, 64), dtype=torch.bfloat16)
    with pytest.raises(pa.PagedAttentionError):
        pa.pa_swap_blocks(pageable, g, up_int(np.array([[0, 1]], np.int64)))
