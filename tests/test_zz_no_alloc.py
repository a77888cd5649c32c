"""pa_decode_noalloc (the decode entry point that allocates nothing: its
split-KV partials live in the library's own device array) against pa_decode
with a caller workspace, and both against the fp64 oracle.

Two calls in a row on the same GPU, the second with a smaller batch, so the
second reuses the array the first left behind."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_cases import TOL, DecodeRun, lib, max_abs, oracle_step

pytestmark = pytest.mark.gpu


def _both(run: DecodeRun, partition_size: int):
    """Outputs of pa_decode (caller workspace) and of pa_decode_noalloc."""
    pa = lib()
    s = run.case.spec
    ref_out = run.decode(partition_size=partition_size)
    out = torch.empty_like(run.q)
    out.fill_(float("nan"))
    pa.pa_decode_noalloc(out, run.q, run.k_pool, run.v_pool, run.tables, run.lens, s.scale,
                         run.max_len, run.case.k_scale, run.case.v_scale, partition_size)
    torch.cuda.synchronize()
    return ref_out, out


def _check(case, partition_size):
    s = case.spec
    print(f"[noalloc] {s.name} S={len(case.seq_lens)} partition={partition_size} "
          f"max_len={int(case.seq_lens.max())}", flush=True)
    run = DecodeRun(case)
    run.scatter()
    torch.cuda.synchronize()
    need = lib().pa_decode_workspace_bytes(len(case.seq_lens), s.num_q_heads, s.num_kv_heads,
                                           s.head_dim, s.block_size, run.max_len, partition_size)
    assert need <= lib().pa_decode_noalloc_max_workspace_bytes()
    ref_out, out = _both(run, partition_size)
    # same kernels, same plan: the same bits as the call with a caller workspace
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    want, _, _ = oracle_step(case)
    assert max_abs(out, want) <= TOL[s.q_dtype]
    return need


def test_noalloc_two_calls_second_smaller():
    big = W.make_decode_case("llama3_8b_gqa_bf16", rep=3, num_seqs=48)
    small = W.make_decode_case("llama3_8b_gqa_bf16", rep=4, num_seqs=7)
    # fixed 64-token partitions: every pair longer than 64 tokens leaves partials
    n1 = _check(big, 64)
    n2 = _check(small, 64)
    assert n1 > n2 > 0


def test_noalloc_balanced_cut_then_smaller_mha():
    first = W.make_decode_case("llama2_7b_mha_f16", rep=5, num_seqs=40)
    second = W.make_decode_case("llama2_7b_mha_f16", rep=6, num_seqs=3)
    _check(first, 0)
    _check(second, 0)


def test_noalloc_after_larger_call_poisoned_scratch():
    """A call that writes partials for many pairs, then a small call whose
    pairs are few: stale partials left in the array must not leak into it."""
    pa = lib()
    big = W.make_decode_case("llama3_70b_fp8kv", rep=2, num_seqs=32)
    _check(big, 512)
    small = W.make_decode_case("llama3_70b_fp8kv", rep=7, num_seqs=4, lens=[1, 600, 33, 1500])
    _check(small, 512)
    _check(small, 32)


def test_noalloc_rejects_a_batch_beyond_the_array():
    """The full Llama-3-8B-shaped batch needs more split-KV workspace than the
    array holds: the call fails before anything is enqueued."""
    pa = lib()
    case = W.make_decode_case("llama3_8b_gqa_bf16", num_seqs=2, lens=[5, 9])
    run = DecodeRun(case)
    s = case.spec
    out = torch.empty_like(run.q)
    tables = torch.zeros((256, 512), dtype=torch.int32, device=run.q.device)
    lens = torch.zeros(256, dtype=torch.int32, device=run.q.device)
    q = torch.zeros((256, s.num_q_heads, s.head_dim), dtype=run.q.dtype, device=run.q.device)
    out = torch.empty_like(q)
    need = pa.pa_decode_workspace_bytes(256, s.num_q_heads, s.num_kv_heads, s.head_dim,
                                        s.block_size, 8192, 0)
    assert need > pa.pa_decode_noalloc_max_workspace_bytes()
    with pytest.raises(pa.PagedAttentionError) as exc:
        pa.pa_decode_noalloc(out, q, run.k_pool, run.v_pool, tables, lens, s.scale, 8192)
    assert exc.value.status == 3     # PA_ERR_WORKSPACE
    # nothing was launched: the output buffer is untouched and the stream is healthy
    torch.cuda.synchronize()
