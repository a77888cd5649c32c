"""Decode and prefill launched from captured HIP graphs: every replay, with
eager work and synchronisations between replays, must give bit-identical
results to the eager launches (the kernels write no memset nodes)."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_cases import DecodeRun, lib, up, up_int

pytestmark = pytest.mark.gpu


def _decode_launches(pa, run, out, ws, partition):
    s = run.case.spec
    pa.pa_reshape_and_cache(run.new_k, run.new_v, run.k_pool, run.v_pool, run.slots,
                            run.case.k_scale, run.case.v_scale)
    args = (out, run.q, run.k_pool, run.v_pool, run.tables, run.lens, s.scale, run.max_len,
            run.case.k_scale, run.case.v_scale, partition, ws)
    pa.pa_decode_attention(*args)
    pa.pa_decode_reduce(*args)


@pytest.mark.parametrize("name,partition", [("llama3_8b_gqa_bf16", 0), ("llama3_70b_fp8kv", 512),
                                            ("llama2_7b_mha_f16", -1)])
def test_decode_graph_replays_match_eager(name, partition):
    pa = lib()
    case = W.make_decode_case(name, num_seqs=24)
    run = DecodeRun(case)
    ws = pa.decode_workspace(run.q, run.k_pool, run.max_len, partition)
    eager = torch.empty_like(run.q)
    _decode_launches(pa, run, eager, ws, partition)
    torch.cuda.synchronize()
    graphed = torch.empty_like(run.q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _decode_launches(pa, run, graphed, ws, partition)
    bits = torch.int16
    for rep in range(3):
        graphed.fill_(7.0)                        # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(graphed.view(bits), eager.view(bits)), f"replay {rep} differs"
        other = torch.empty_like(run.q)           # an eager call between replays
        _decode_launches(pa, run, other, ws, partition)
        torch.cuda.synchronize()
        assert torch.equal(other.view(bits), eager.view(bits))


def test_prefill_graph_replays_match_eager():
    pa = lib()
    case = W.make_mixed_case(num_forks=4, prefix_len=256, chunk_len=200, num_decode=3,
                             decode_lens=[40, 300, 900])
    s = case.spec
    dt = s.dtype
    kp, vp = up(case.k_pool, dt), up(case.v_pool, dt)
    pa.pa_copy_blocks(kp, vp, up_int(case.cow_pairs))
    pa.pa_reshape_and_cache(up(case.new_k, dt), up(case.new_v, dt), kp, vp, up_int(case.slot_mapping))
    qc = up(case.q_chunk, dt)
    qsl, tab, lens = up_int(case.query_start_loc), up_int(case.prefill_tables), up_int(case.prefill_lens)
    eager, graphed = torch.empty_like(qc), torch.empty_like(qc)
    pa.pa_prefill_chunk(eager, qc, qsl, kp, vp, tab, lens, s.scale, 200)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pa.pa_prefill_chunk(graphed, qc, qsl, kp, vp, tab, lens, s.scale, 200)
    for rep in range(3):
        graphed.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(graphed.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"


def test_mixed_step_graph_with_two_streams_matches_eager():
    """The whole mixed step captured as one graph: copy-on-write and scatter,
    then the prefill chunks on the capturing stream and the decodes (attention
    and reduce) on a forked stream, joined at the end.  Every replay matches
    the eager, single-stream step bit for bit."""
    pa = lib()
    case = W.make_mixed_case(num_forks=4, prefix_len=256, chunk_len=120, num_decode=6,
                             decode_lens=[40, 300, 900, 17, 2000, 64])
    s = case.spec
    dt = s.dtype
    base_k, base_v = up(case.k_pool, dt), up(case.v_pool, dt)
    pairs, slots = up_int(case.cow_pairs), up_int(case.slot_mapping)
    nk, nv = up(case.new_k, dt), up(case.new_v, dt)
    qc, qd = up(case.q_chunk, dt), up(case.q_decode, dt)
    qsl, ptab, plen = up_int(case.query_start_loc), up_int(case.prefill_tables), up_int(case.prefill_lens)
    dtab, dlen = up_int(case.decode_tables), up_int(case.decode_lens)
    max_q = int(np.diff(case.query_start_loc).max())
    max_len = int(case.decode_lens.max())
    ws = pa.decode_workspace(qd, base_k, max_len)

    def step(kp, vp, out_c, out_d, side=None):
        pa.pa_copy_blocks(kp, vp, pairs)
        pa.pa_reshape_and_cache(nk, nv, kp, vp, slots)
        if side is not None:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                pa.pa_decode_attention(out_d, qd, kp, vp, dtab, dlen, s.scale, max_len, workspace=ws)
                pa.pa_decode_reduce(out_d, qd, kp, vp, dtab, dlen, s.scale, max_len, workspace=ws)
            pa.pa_prefill_chunk(out_c, qc, qsl, kp, vp, ptab, plen, s.scale, max_q)
            torch.cuda.current_stream().wait_stream(side)
        else:
            pa.pa_prefill_chunk(out_c, qc, qsl, kp, vp, ptab, plen, s.scale, max_q)
            pa.pa_decode_attention(out_d, qd, kp, vp, dtab, dlen, s.scale, max_len, workspace=ws)
            pa.pa_decode_reduce(out_d, qd, kp, vp, dtab, dlen, s.scale, max_len, workspace=ws)

    ek, ev = base_k.clone(), base_v.clone()
    e_c, e_d = torch.empty_like(qc), torch.empty_like(qd)
    step(ek, ev, e_c, e_d)
    torch.cuda.synchronize()
    gk, gv = base_k.clone(), base_v.clone()
    g_c, g_d = torch.empty_like(qc), torch.empty_like(qd)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(gk, gv, g_c, g_d, side)
    bits = torch.int16
    for rep in range(3):
        gk.copy_(base_k)                      # eager work between replays
        gv.copy_(base_v)
        g_c.zero_()
        g_d.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_c.view(bits), e_c.view(bits)), f"prefill, replay {rep}"
        assert torch.equal(g_d.view(bits), e_d.view(bits)), f"decode, replay {rep}"
        assert torch.equal(gk.view(bits), ek.view(bits)) and torch.equal(gv.view(bits), ev.view(bits))
