"""GPU: the native block manager's prefix cache feeding the kernels.

Two prompts share a system prompt.  The first is prefilled whole; the
second, allocated through the prefix cache, finds the system prompt's full
blocks cached and prefills only its own tokens as a chunk whose context is
the cached blocks plus the chunk.  Its outputs must equal the oracle's
attention over the second prompt's whole context (held in a separate,
contiguous pool), within the bf16 tolerance: the cached blocks hold the right
K/V and the chunk reads them through its block table.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_cases import TOL, lib, max_abs, up, up_int

pytestmark = pytest.mark.gpu


def _kv_of(tokens, base_k, base_v, pos_k, pos_v):
    """Synthetic K/V of a token sequence: a per-token part plus a per-position
    part, so that equal prefixes have equal K/V (as a model's would)."""
    t = np.asarray(tokens)
    p = np.arange(len(t))
    return base_k[t] + pos_k[p], base_v[t] + pos_v[p]


@pytest.mark.parametrize("bs,hq,hkv,d", [(16, 8, 2, 128), (8, 4, 4, 64), (32, 16, 1, 128)])
def test_cached_prefix_plus_chunk_equals_whole_prompt(bs, hq, hkv, d):
    pa = lib()
    dt = "bf16"
    rng = np.random.default_rng(bs * 10 + d)
    vocab, max_pos = 50, 512
    base_k = rng.standard_normal((vocab, hkv, d)).astype(np.float32)
    base_v = rng.standard_normal((vocab, hkv, d)).astype(np.float32)
    pos_k = 0.5 * rng.standard_normal((max_pos, hkv, d)).astype(np.float32)
    pos_v = 0.5 * rng.standard_normal((max_pos, hkv, d)).astype(np.float32)

    system = list(map(int, rng.integers(0, vocab, 3 * bs + 5)))       # 3 full blocks + 5
    prompt_a = system + list(map(int, rng.integers(0, vocab, 21)))
    prompt_b = system + list(map(int, rng.integers(0, vocab, 37)))
    nb = 64
    mgr = pa.BlockManager(nb, bs, order=rng.permutation(nb))
    kp = up(np.full((nb, hkv, bs, d), W.NAN_BITS[dt], np.uint16), dt)
    vp = up(np.full((nb, hkv, bs, d), W.NAN_BITS[dt], np.uint16), dt)
    scale = 1.0 / np.sqrt(d)

    def prefill(prompt, table, start):
        """Scatter the prompt's tokens [start, n) and prefill them as one chunk."""
        n = len(prompt)
        k, v = _kv_of(prompt, base_k, base_v, pos_k, pos_v)
        slots = np.array([table[p // bs] * bs + p % bs for p in range(start, n)], np.int64)
        pa.pa_reshape_and_cache(up(W.to_bits(k[start:], dt), dt), up(W.to_bits(v[start:], dt), dt),
                                kp, vp, up_int(slots))
        q = W.to_bits(rng.standard_normal((n - start, hq, d)).astype(np.float32), dt)
        out = torch.empty((n - start, hq, d), dtype=torch.bfloat16, device="cuda:0")
        pa.pa_prefill_chunk(out, up(q, dt), up_int(np.array([0, n - start], np.int32)), kp, vp,
                            up_int(np.array([table], np.int32)), up_int(np.array([n], np.int32)),
                            scale, n - start)
        return out, q

    table_a, hits_a = mgr.allocate_prompt(7, prompt_a)
    assert hits_a == 0
    prefill(prompt_a, table_a, 0)
    table_b, hits_b = mgr.allocate_prompt(7, prompt_b)
    assert hits_b == 3 and table_b[:3] == table_a[:3]                 # the system prompt's full blocks
    assert set(table_b[3:]).isdisjoint(table_a)
    out_b, q_b = prefill(prompt_b, table_b, hits_b * bs)
    torch.cuda.synchronize()

    # oracle: prompt B's whole context in its own contiguous pool
    n = len(prompt_b)
    k, v = _kv_of(prompt_b, base_k, base_v, pos_k, pos_v)
    nblk = -(-n // bs)
    ck = np.zeros((nblk * bs, hkv, d), np.float32)
    cv = np.zeros((nblk * bs, hkv, d), np.float32)
    ck[:n], cv[:n] = k, v
    okp = W.to_bits(ck.reshape(nblk, bs, hkv, d).transpose(0, 2, 1, 3), dt)
    ovp = W.to_bits(cv.reshape(nblk, bs, hkv, d).transpose(0, 2, 1, 3), dt)
    chunk = n - hits_b * bs
    ref = oracle.prefill_chunk_attention(q_b, dt, np.array([0, chunk]), okp, ovp, dt,
                                         np.arange(nblk, dtype=np.int32)[None, :], [n], scale, bs,
                                         hkv)
    assert max_abs(out_b, ref) <= TOL[dt]
    # another namespace shares nothing
    _, hits_c = mgr.allocate_prompt(8, prompt_b)
    assert hits_c == 0
