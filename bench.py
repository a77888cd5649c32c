"""Benchmark of the paged KV-cache decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME|all] [--rotate R]

One step is one pass of the decode hot path over one batch: scatter of each
sequence's newest K/V into its pool slot (pa_reshape_and_cache), then paged
decode attention (pa_decode_attention) and the log-sum-exp merge of split
partials (pa_decode_reduce), all on torch's current stream; for 16-bit caches
the headline also reports the step with the scatter folded into the decode
kernel (pa_decode_attention_append + pa_decode_reduce).  For the mixed
workload a step is copy-on-write (pa_copy_blocks), the scatter of every new
token, and the attention of the causal prefill chunks and the decodes in one
launch (pa_mixed_attention); the same step with separate pa_prefill_chunk,
pa_decode_attention and pa_decode_reduce launches is timed beside it.

By default (--config all) the headline is the largest single-GPU decode
workload, the Llama-3-8B-shaped GQA layer (256 sequences, 32/8 heads,
head_dim 128, block 16, lognormal lengths, bf16); the same JSON line carries
the Llama-2-7B-shaped MHA layer, the 70B-shaped fp8 layer (512-token
partitions), the mixed prefill + decode step and the tiny fp32 case under
"configs", each with its own step time, rate and roofline.  --config NAME
runs one workload alone.

Throughput is effective KV bytes per second: sum over sequences of len * Hkv
* D * (bytes of K + bytes of V), the K and V the method must read, divided by
the time of the whole step.  Batch layouts (lengths, shuffled physical ids,
tables, slots) come from workloads.py; element values are drawn on the device
with torch's seeded generator (same distributions).  R batches with separate
pools are rotated so that no step finds its KV in the 256 MB last-level
cache.

The CPU baseline runs the fp64 oracle, as it stands, on the same workloads
(generated on the CPU by workloads.py: the whole headline and 70B-shaped
batches, bounded samples of the others), before the GPU is touched: on every
host core this process may use (one oracle process per core, sequences or
heads spread over them) and, for the two smallest workloads, on one thread.

Printed: one JSON line with the step rate, a roofline object for the
dominant kernel (its average duration measured with HIP events on the
launch stream) and the CPU baseline.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16/fp16 MFMA, vendor figure
METRIC = "pa_decode effective KV GB/s (% of HBM peak); decode tokens/s per layer"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="all",
                    help="all (headline llama3_8b_gqa_bf16 plus the other workloads) | "
                         "llama2_7b_mha_f16 | llama3_8b_gqa_bf16 | llama3_70b_fp8kv | llama3_8b_kfp8_vbf16 "
                         "| llama3_8b_int8kv | llama3_70b_fp8kv_tp8 "
                         "| tiny_f32 "
                         "| mixed_prefix_bf16 | mixed_70b_fp8kv | mixed_70b_int8kv")
    ap.add_argument("--rotate", type=int, default=4, help="batches with separate pools")
    ap.add_argument("--partition", type=int, default=None,
                    help="decode partition size override (default: the workload's)")
    ap.add_argument("--block-size", type=int, default=None,
                    help="decode workloads: run with this block size (8, 16, 32, 64) instead; a "
                         "fixed pool keeps its token capacity")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay comparison")
    return ap.parse_args()


HEADLINE = "llama3_8b_gqa_bf16"
SUB_CONFIGS = ["llama2_7b_mha_f16", "llama3_70b_fp8kv", "mixed_prefix_bf16", "tiny_f32"]


# ---------------------------------------------------------------------------
# Device batches
# ---------------------------------------------------------------------------

def _randn(shape, gen, dev, std=1.0):
    import torch
    x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
    return x.mul_(std) if std != 1.0 else x


def _to_cache(x, dtype: str):
    """float32 values -> stored element type; fp8 gets a per-tensor amax/448 scale."""
    import torch
    import workloads as W
    if dtype == "fp8_e4m3":
        scale = float((x.abs().max() / W.FP8_MAX).item())
        return (x / scale).clamp_(-W.FP8_MAX, W.FP8_MAX).to(torch.float8_e4m3fn), scale
    return x.to(W.TORCH_DTYPE[dtype]), 1.0


def _to_int8_blocks(x):
    """float32 pool -> int8 codes with one scale per (block, KV head): amax / 127."""
    import torch
    amax = x.abs().amax(dim=(2, 3))
    scales = torch.where(amax > 0, amax / 127.0, torch.ones_like(amax)).float().contiguous()
    codes = (x / scales[:, :, None, None]).round_().clamp_(-127, 127).to(torch.int8)
    return codes, scales


class DecodeBatch:
    """One decode batch resident in HBM (values drawn on the device)."""

    def __init__(self, lay, seed: int, dev):
        import torch
        import workloads as W
        s = lay.spec
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        shape = (lay.num_blocks, s.num_kv_heads, s.block_size, s.head_dim)
        if s.cache_dtype == "int8":
            self.k_pool, self.k_scales = _to_int8_blocks(_randn(shape, gen, dev, s.value_std))
            self.v_pool, self.v_scales = _to_int8_blocks(_randn(shape, gen, dev, s.value_std))
            self.k_scale = self.v_scale = 1.0
        else:
            self.k_pool, self.k_scale = _to_cache(_randn(shape, gen, dev, s.value_std), s.cache_dtype)
            self.v_pool, self.v_scale = _to_cache(_randn(shape, gen, dev, s.value_std), s.v_dtype)
        S = len(lay.seq_lens)
        qdt = W.TORCH_DTYPE[s.q_dtype]
        self.q = _randn((S, s.num_q_heads, s.head_dim), gen, dev, s.value_std).to(qdt)
        self.new_k = _randn((S, s.num_kv_heads, s.head_dim), gen, dev, s.value_std).to(qdt)
        self.new_v = _randn((S, s.num_kv_heads, s.head_dim), gen, dev, s.value_std).to(qdt)
        self.tables = torch.from_numpy(lay.block_tables).to(dev)
        self.lens = torch.from_numpy(lay.seq_lens.astype("int32")).to(dev)
        self.slots = torch.from_numpy(lay.slot_mapping).to(dev)
        self.out = torch.empty_like(self.q)


def run_decode_bench(args, dev, name: str, extras: bool = True):
    """One decode workload: the timed steps, then (with ``extras``) the same
    steps with the scatter folded into the decode kernel and replayed from
    captured HIP graphs, for comparison."""
    import numpy as np
    import torch
    import paged_kv_cache_415_amd as pa
    import workloads as W

    spec = W.DECODE_SPECS[name]
    if args.block_size is not None and args.block_size != spec.block_size:
        import dataclasses
        pool = spec.pool
        if pool[0] == "fixed":
            pool = ("fixed", max(1, pool[1] * spec.block_size // args.block_size))
        # the same name keeps the same seeded lengths
        spec = dataclasses.replace(spec, block_size=args.block_size, pool=pool,
                                   description=f"{spec.description}; block size {args.block_size}")
    lay = W.make_decode_layout(spec, rep=0)
    max_len = int(lay.seq_lens.max())
    part = spec.partition_size if args.partition is None else args.partition
    batches = [DecodeBatch(lay, seed=4150 + r, dev=dev) for r in range(max(1, args.rotate))]
    torch.cuda.synchronize()
    b0 = batches[0]
    resolved = pa.pa_decode_partition_size(len(lay.seq_lens), spec.num_kv_heads, spec.block_size,
                                           max_len, part)
    ws = pa.decode_workspace(b0.q, b0.k_pool, max_len, part)

    mixed = spec.v_dtype != spec.cache_dtype     # fp8 K beside a 16-bit V pool
    int8 = spec.cache_dtype == "int8"            # per-(block, KV head) scales
    scatter = pa.pa_reshape_and_cache_kv if mixed else pa.pa_reshape_and_cache
    attention = pa.pa_decode_attention_kv if mixed else pa.pa_decode_attention
    reduce = pa.pa_decode_reduce_kv if mixed else pa.pa_decode_reduce

    def step_separate(b, ev=None):
        """Scatter kernel, decode attention, reduce: three launches."""
        if int8:
            pa.pa_reshape_and_cache_int8(b.new_k, b.new_v, b.k_pool, b.v_pool, b.k_scales,
                                         b.v_scales, b.slots)
        else:
            scatter(b.new_k, b.new_v, b.k_pool, b.v_pool, b.slots, b.k_scale, b.v_scale)
        if ev is not None:
            ev[0].record()
        if int8:
            pa.pa_decode_attention_int8(b.out, b.q, b.k_pool, b.v_pool, b.k_scales, b.v_scales,
                                        b.tables, b.lens, spec.scale, max_len, part, ws)
        else:
            attention(b.out, b.q, b.k_pool, b.v_pool, b.tables, b.lens, spec.scale,
                      max_len, b.k_scale, b.v_scale, part, ws)
        if ev is not None:
            ev[1].record()
        if int8:
            pa.pa_decode_reduce_int8(b.out, b.q, b.k_pool, b.v_pool, b.k_scales, b.v_scales,
                                     b.tables, b.lens, spec.scale, max_len, part, ws)
        else:
            reduce(b.out, b.q, b.k_pool, b.v_pool, b.tables, b.lens, spec.scale,
                   max_len, b.k_scale, b.v_scale, part, ws)
        if ev is not None:
            ev[2].record()

    # 16-bit caches: the scatter folded into the decode kernel
    can_append = spec.cache_dtype == spec.q_dtype == spec.v_dtype and spec.q_dtype in ("f16", "bf16")

    def step_append(b, ev=None):
        """Decode kernel with the scatter folded in, then the reduce: two launches."""
        if ev is not None:
            ev[0].record()
        pa.pa_decode_attention_append(b.out, b.q, b.new_k, b.new_v, b.k_pool, b.v_pool, b.tables,
                                      b.lens, spec.scale, max_len, b.k_scale, b.v_scale, part, ws)
        if ev is not None:
            ev[1].record()
        pa.pa_decode_reduce(b.out, b.q, b.k_pool, b.v_pool, b.tables, b.lens, spec.scale,
                            max_len, b.k_scale, b.v_scale, part, ws)
        if ev is not None:
            ev[2].record()

    step = step_separate
    for i in range(args.warmup):
        step(batches[i % len(batches)])
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(batches[i % len(batches)], evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn_ms = [e[0].elapsed_time(e[1]) for e in evs]
    red_ms = [e[1].elapsed_time(e[2]) for e in evs]

    # After the timed region: the same steps with the scatter folded into the
    # decode kernel (append kernel + reduce), for comparison
    def time_steps(fn):
        for i in range(args.warmup):
            fn(batches[i % len(batches)])
        torch.cuda.synchronize()
        cevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        t1 = time.perf_counter()
        for i in range(args.steps):
            fn(batches[i % len(batches)], cevs[i])
        torch.cuda.synchronize()
        return ((time.perf_counter() - t1) * 1e3 / args.steps,
                float(np.mean([e[0].elapsed_time(e[1]) for e in cevs])),
                float(np.mean([e[1].elapsed_time(e[2]) for e in cevs])))

    appended = None
    if extras and can_append:
        appended = time_steps(step_append)

    # After the timed region: the same steps replayed from captured HIP graphs
    # (one graph per batch), as a serving loop replays captured decode steps.
    graph_ms = None
    try:
        if not extras or args.no_graph:
            raise RuntimeError("not requested")
        graphs = []
        for b in batches:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(b)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    except RuntimeError as exc:
        if str(exc) != "not requested":
            print(f"bench.py: hipGraph replay skipped ({exc})", file=sys.stderr)
    assert not torch.isnan(b0.out).any(), "NaN in decode output"

    eff = W.effective_kv_bytes(lay.seq_lens, spec.num_kv_heads, spec.head_dim, spec.cache_dtype,
                               spec.v_dtype)
    if spec.cache_dtype == "int8":
        eff += W.block_scale_bytes(lay.seq_lens, spec.num_kv_heads, spec.block_size)
    ms_step = elapsed * 1e3 / args.steps
    attn_avg = float(np.mean(attn_ms))
    S = len(lay.seq_lens)
    value = eff / (ms_step * 1e-3) / 1e9
    achieved = eff / (attn_avg * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s",
        "ms_per_step": round(ms_step, 5),
        "dtype": spec.cache_dtype if spec.cache_dtype == spec.q_dtype == spec.v_dtype else
        f"{spec.q_dtype}+{spec.cache_dtype}" if spec.v_dtype == spec.cache_dtype else
        f"{spec.q_dtype}+K {spec.cache_dtype}+V {spec.v_dtype}",
        "config": {"workload": spec.description, "name": spec.name, "num_seqs": S,
                   "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
                   "head_dim": spec.head_dim, "block_size": spec.block_size,
                   "total_context_tokens": int(lay.seq_lens.sum()), "max_seq_len": max_len,
                   "partition_size": resolved, "rotated_batches": len(batches)},
        "roofline": {"bound": "hbm", "kernel": "decode_kernel<MfmaDecode>" if spec.cache_dtype != "f32"
                     else "decode_kernel<F32Decode>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": (decode_traffic_bytes(spec.name)
                                 if args.block_size is None and args.partition is None else None),
                     "traffic_unit": "bytes per launch",
                     "algorithmic_bytes_per_launch": eff,
                     "avg_launch_ms": round(attn_avg, 5)},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "decode_tokens_per_s_per_layer": round(S / (ms_step * 1e-3), 1),
        "decode_gbps_attention_plus_reduce": round(
            eff / ((attn_avg + float(np.mean(red_ms))) * 1e-3) / 1e9, 1),
        "reduce_avg_ms": round(float(np.mean(red_ms)), 5),
        "hipgraph_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "hipgraph_gbps": None if graph_ms is None else round(eff / (graph_ms * 1e-3) / 1e9, 1),
        "attention_p10_p50_p90_ms": [round(float(x), 5) for x in
                                      np.percentile(attn_ms, [10, 50, 90])],
        "effective_kv_bytes_per_step": eff,
    }
    res["step"] = "scatter kernel + decode attention + reduce"
    if appended is not None:
        res["append_plus_reduce_ms_per_step"] = round(appended[0], 5)
        res["append_plus_reduce_gbps"] = round(eff / (appended[0] * 1e-3) / 1e9, 1)
        res["append_attention_avg_ms"] = round(appended[1], 5)
    return res


# ---------------------------------------------------------------------------
# Mixed chunked-prefill + decode step (copy-on-write, scatter, prefill, decode)
# ---------------------------------------------------------------------------

def run_mixed_bench(args, dev, spec=None):
    import numpy as np
    import torch
    import paged_kv_cache_415_amd as pa
    import workloads as W

    case = W.make_mixed_case(spec or W.MIXED_SPEC)
    s = case.spec
    dt, cdt = s.dtype, s.pool_dtype
    ks, vs = case.k_scale, case.v_scale
    up = lambda a: W.bits_to_device(a, dt, dev)
    upi = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    kp, vp = W.bits_to_device(case.k_pool, cdt, dev), W.bits_to_device(case.v_pool, cdt, dev)
    pairs = upi(case.cow_pairs)
    nk, nv, slots = up(case.new_k), up(case.new_v), upi(case.slot_mapping)
    qc, qd = up(case.q_chunk), up(case.q_decode)
    qsl, ptab, plen = upi(case.query_start_loc), upi(case.prefill_tables), upi(case.prefill_lens)
    dtab, dlen = upi(case.decode_tables), upi(case.decode_lens)
    out_c, out_d = torch.empty_like(qc), torch.empty_like(qd)
    max_q = int(np.diff(case.query_start_loc).max())
    max_len = int(case.decode_lens.max())
    ws = pa.decode_workspace(qd, kp, max_len)

    sc = dict(k_scale=ks, v_scale=vs)
    i8 = cdt == "int8"
    if i8:
        # per-(block, KV head) scales: copy-on-write copies them with the codes
        gks = torch.from_numpy(case.k_block_scales).to(dev)
        gvs = torch.from_numpy(case.v_block_scales).to(dev)

    def write_step():
        pa.pa_copy_blocks(kp, vp, pairs)
        if i8:
            pa.pa_copy_blocks(gks, gvs, pairs)
            pa.pa_reshape_and_cache_int8(nk, nv, kp, vp, gks, gvs, slots)
        else:
            pa.pa_reshape_and_cache(nk, nv, kp, vp, slots, ks, vs)

    def prefill():
        if i8:
            pa.pa_prefill_chunk_int8(out_c, qc, qsl, kp, vp, gks, gvs, ptab, plen, s.scale, max_q)
        else:
            pa.pa_prefill_chunk(out_c, qc, qsl, kp, vp, ptab, plen, s.scale, max_q, **sc)

    def decode_attention():
        if i8:
            pa.pa_decode_attention_int8(out_d, qd, kp, vp, gks, gvs, dtab, dlen, s.scale, max_len, workspace=ws)
        else:
            pa.pa_decode_attention(out_d, qd, kp, vp, dtab, dlen, s.scale, max_len, workspace=ws, **sc)

    def decode_reduce():
        if i8:
            pa.pa_decode_reduce_int8(out_d, qd, kp, vp, gks, gvs, dtab, dlen, s.scale, max_len, workspace=ws)
        else:
            pa.pa_decode_reduce(out_d, qd, kp, vp, dtab, dlen, s.scale, max_len, workspace=ws, **sc)

    def fused_step(ev=None):
        write_step()
        if ev is not None:
            ev[0].record()
        if i8:
            pa.pa_mixed_attention_int8(out_c, qc, qsl, ptab, plen, max_q, out_d, qd, dtab, dlen, max_len, kp,
                                       vp, gks, gvs, s.scale, workspace=ws)
        else:
            pa.pa_mixed_attention(out_c, qc, qsl, ptab, plen, max_q, out_d, qd, dtab, dlen, max_len, kp, vp,
                                  s.scale, workspace=ws, **sc)
        if ev is not None:
            ev[1].record()

    def step(ev=None, side=None):
        write_step()
        if side is not None:
            # prefill chunks and decodes on two streams (joined at the end)
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                decode_attention()
                decode_reduce()
            prefill()
            torch.cuda.current_stream().wait_stream(side)
            return
        if ev is not None:
            ev[0].record()
        prefill()
        if ev is not None:
            ev[1].record()
        decode_attention()
        if ev is not None:
            ev[2].record()
        decode_reduce()
        if ev is not None:
            ev[3].record()

    for _ in range(args.warmup):
        step()
        fused_step()
    torch.cuda.synchronize()
    # the step with the prefill chunks and the decodes in one launch
    fevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        fused_step(fevs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # the same step as separate prefill, decode and reduce launches
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    sep_elapsed = time.perf_counter() - t0
    # the same step captured as one HIP graph with the prefill and the decode
    # on forked streams (timed after the eager measurement above)
    graph_ms = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(side=side)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    # the one-launch step captured as a HIP graph (one stream)
    fused_graph_ms = None
    if not args.no_graph:
        gf = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gf):
            fused_step()
        for _ in range(3):
            gf.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(args.steps):
            gf.replay()
        torch.cuda.synchronize()
        fused_graph_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    pre_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    fused_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in fevs]))
    sep_ms = float(np.mean([e[0].elapsed_time(e[3]) for e in evs]))
    ms_step = elapsed * 1e3 / args.steps
    sep_ms_step = sep_elapsed * 1e3 / args.steps
    flops = mixed_prefill_flops(case)
    eff = W.effective_kv_bytes(case.decode_lens, s.num_kv_heads, s.head_dim, cdt)
    if i8:
        eff += W.block_scale_bytes(case.decode_lens, s.num_kv_heads, s.block_size)
    tflops = flops / (pre_ms * 1e-3) / 1e12
    dec_gbps = eff / (dec_ms * 1e-3) / 1e9
    return {
        "metric": METRIC, "value": round(eff / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s",
        "ms_per_step": round(ms_step, 5), "dtype": dt if cdt == dt else f"{dt}+{cdt}",
        "config": {"workload": s.description, "name": s.name,
                   "prefill_tokens": int(case.query_start_loc[-1]),
                   "decode_seqs": int(len(case.decode_lens)), "cow_pairs": int(len(case.cow_pairs))},
        "roofline": {"bound": "mfma", "kernel": "prefill_mfma_kernel", "achieved": round(tflops, 2),
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": decode_traffic_bytes(s.name, "prefill"),
                     "traffic_unit": "bytes per launch",
                     "algorithmic_flops_per_launch": flops, "avg_launch_ms": round(pre_ms, 5)},
        "decode_roofline": {"bound": "hbm", "kernel": "decode_kernel<MfmaDecode>",
                            "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                            "traffic": decode_traffic_bytes(s.name, "decode"),
                            "traffic_unit": "bytes per launch",
                            "algorithmic_bytes_per_launch": eff, "avg_launch_ms": round(dec_ms, 5)},
        "fused_attention": {
            "kernels": "mixed_kernel + lse_reduce_kernel ("
                       + ("pa_mixed_attention_int8)" if i8 else "pa_mixed_attention)"),
            "avg_ms": round(fused_ms, 5),
            "prefill_tflops": round(flops / (fused_ms * 1e-3) / 1e12, 2),
            "decode_gbps": round(eff / (fused_ms * 1e-3) / 1e9, 1),
            "mfma_frac": round(flops / (fused_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
            "hbm_frac": round(eff / (fused_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            # time both parts would take at their peaks, one after the other, over the fused time
            "combined_frac": round((flops / (BF16_MFMA_PEAK_TFLOPS * 1e12) + eff / (HBM_PEAK_GBPS * 1e9))
                                   / (fused_ms * 1e-3), 4),
            "separate_launches_ms": round(sep_ms, 5),
            "traffic": decode_traffic_bytes(s.name, "mixed"), "traffic_unit": "bytes per launch of mixed_kernel"},
        "separate_launches_ms_per_step": round(sep_ms_step, 5),
        "prefill_flops": flops, "effective_kv_bytes_per_step": eff,
        "prefill_tflops": round(tflops, 2), "decode_gbps": round(dec_gbps, 1),
        "prefill_tokens_per_s": round(int(case.query_start_loc[-1]) / (pre_ms * 1e-3), 1),
        "hipgraph_two_stream_ms_per_step": None if graph_ms is None else round(graph_ms, 5),
        "hipgraph_fused_ms_per_step": None if fused_graph_ms is None else round(fused_graph_ms, 5),
        "decode_tokens_per_s_per_layer": round(len(case.decode_lens) / (ms_step * 1e-3), 1),
    }


def run_block_ops_bench(dev, iters: int = 20) -> dict:
    """Rates of the block-management copies beside the mixed step: token-
    granular copy-on-write, one block copy applied to 32 layers, and swapping
    blocks out to pinned host memory and back (shapes of the mixed workload:
    8 KV heads x 32 tokens x 128 dims, bf16 = 64 KB per block and pool)."""
    import numpy as np
    import torch
    import paged_kv_cache_415_amd as pa

    gen = torch.Generator(device=dev)
    gen.manual_seed(4151)
    hkv, bs, d = 8, 32, 128
    blk_bytes = hkv * bs * d * 2

    def pool(n, device=dev):
        return torch.randn((n, hkv, bs, d), generator=gen, device=dev, dtype=torch.float32).to(
            torch.bfloat16).to(device)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(iters):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    rng = np.random.default_rng(4152)
    out = {}
    # token-granular CoW: 1,024 forks inside a block, n ~ U[1, 31] rows each
    kp, vp = pool(4096), pool(4096)
    ids = rng.permutation(4096)
    counts = rng.integers(1, bs, size=1024)
    triples = torch.from_numpy(np.stack([ids[:1024], ids[1024:2048], counts], 1).astype(np.int64)).to(dev)
    ms = timed(lambda: pa.pa_copy_blocks_partial(kp, vp, triples))
    moved = int(counts.sum()) * hkv * d * 2 * 2 * 2          # rows x (K, V) x (read, write)
    out["copy_partial"] = {"pairs": 1024, "bytes_moved": moved, "ms": round(ms, 5),
                           "gbps": round(moved / (ms * 1e-3) / 1e9, 1)}
    del kp, vp
    # one fork across 32 layers: 15 block copies per layer, one launch
    layers = 32
    kps, vps = [pool(64) for _ in range(layers)], [pool(64) for _ in range(layers)]
    pairs = torch.from_numpy(np.stack([np.arange(15), np.arange(32, 47)], 1).astype(np.int64)).to(dev)
    kptr, vptr = pa.layer_pool_pointers(kps, dev), pa.layer_pool_pointers(vps, dev)
    ms = timed(lambda: pa.pa_copy_blocks_layers(kptr, vptr, pairs, block_bytes=blk_bytes))
    moved = layers * 15 * blk_bytes * 2 * 2
    out["copy_layers"] = {"layers": layers, "pairs": 15, "bytes_moved": moved, "ms": round(ms, 5),
                          "gbps": round(moved / (ms * 1e-3) / 1e9, 1)}
    del kps, vps
    # swap 512 blocks (32 MB) of one pool out to pinned host memory and back
    dp = pool(2048)
    hp = torch.empty((512, hkv, bs, d), dtype=torch.bfloat16).pin_memory()
    dev_ids = torch.from_numpy(rng.permutation(2048)[:512].astype(np.int64))
    out_pairs = torch.stack([dev_ids, torch.arange(512)], 1).to(dev)
    in_pairs = torch.stack([torch.arange(512), dev_ids], 1).to(dev)
    ms_out = timed(lambda: pa.pa_swap_blocks(hp, dp, out_pairs))
    ms_in = timed(lambda: pa.pa_swap_blocks(dp, hp, in_pairs))
    moved = 512 * blk_bytes
    out["swap"] = {"blocks": 512, "bytes_each_way": moved,
                   "out_ms": round(ms_out, 5), "out_gbps": round(moved / (ms_out * 1e-3) / 1e9, 1),
                   "in_ms": round(ms_in, 5), "in_gbps": round(moved / (ms_in * 1e-3) / 1e9, 1)}
    # host prefix cache (native block manager): the mixed workload's 16 prompts
    # of a shared 1,024-token prefix plus 512 own tokens, block 32, allocated
    # then released, repeated; the first prompt of each round finds the prefix
    # still cached from the round before
    mgr = pa.BlockManager(8192, bs, order=rng.permutation(8192))
    prefix = rng.integers(0, 32000, 1024).astype(np.int32)
    prompts = [np.concatenate([prefix, rng.integers(0, 32000, 512).astype(np.int32)])
               for _ in range(16)]
    rounds, hits = 50, 0
    t0 = time.perf_counter()
    for _ in range(rounds):
        tables = []
        for p in prompts:
            t, h = mgr.allocate_prompt(0, p)
            tables.append(t)
            hits += h
        for t in tables:
            mgr.release(t)
    us = (time.perf_counter() - t0) * 1e6 / (rounds * len(prompts))
    out["prefix_cache"] = {"prompts": rounds * len(prompts), "tokens_per_prompt": 1536,
                           "us_per_prompt_allocate_and_release": round(us, 2),
                           "cached_block_fraction": round(hits / (rounds * len(prompts) * 48), 4)}
    mgr.close()
    return out


# ---------------------------------------------------------------------------
# HBM traffic of the decode kernel from committed rocprofv3 counter runs
# ---------------------------------------------------------------------------

KERNEL_SOURCES = {"decode": ["decode.hip", "decode_dev.h", "pa_device.h", "pa_launch.h", "pa_api.cpp"],
                  "prefill": ["prefill.hip", "prefill_dev.h", "pa_device.h", "pa_launch.h", "pa_api.cpp"],
                  "mixed": ["mixed.hip", "decode_dev.h", "prefill_dev.h", "pa_device.h", "pa_launch.h",
                            "pa_api.cpp"]}


def traffic_profile(name: str) -> str:
    """The committed rocprofv3 summary that records a workload's counters."""
    if name == "mixed_prefix_bf16":
        return os.path.join(ROOT, "profiles", "prefill_mfma_mixed_prefix_bf16.md")
    if name.startswith("mixed_"):
        return os.path.join(ROOT, "profiles", f"mixed_serving_{name}.md")
    return os.path.join(ROOT, "profiles", f"decode_mfma_{name}.md")


def kernel_sources_sha256(kind: str = "decode") -> str:
    """Hash of a kernel's sources with comments and blank lines removed (a
    comment edit does not change the kernel the counters were taken on)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "paged_kv_cache_415_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def decode_traffic_bytes(name: str, kind: str = "decode"):
    """HBM bytes per launch of the workload's decode (or prefill) kernel from
    the FETCH_SIZE / WRITE_SIZE runs recorded in profiles/, each scaled by what
    the same counter reads for a copy of known size; None when no counters are
    recorded or they were taken on other kernel sources."""
    try:
        text = open(traffic_profile(name)).read()
    except OSError:
        return None
    line = next((l for l in text.splitlines() if l.startswith(f"{kind}_traffic:")), None)
    if line is None:
        return None
    kv = dict(item.split("=", 1) for item in line.split()[1:])
    if kv.get("sources_sha256") != kernel_sources_sha256(kind):
        return None
    copy_bytes = float(kv["copy_bytes"])
    fetch = float(kv["fetch_kib"]) * copy_bytes / float(kv["copy_fetch_kib"])
    write = float(kv["write_kib"]) * copy_bytes / float(kv["copy_write_kib"])
    return int(round(fetch + write))


# ---------------------------------------------------------------------------
# Practical HBM read rate of a plain streaming kernel (context for the peak)
# ---------------------------------------------------------------------------

def probe_copy_once(dev, nbytes=1 << 30):
    """One plain copy of a known size: the reference for the HBM byte counters."""
    import torch
    import paged_kv_cache_415_amd as pa
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    pa.pa_probe_copy(dst, src)
    torch.cuda.synchronize()
    del src, dst
    return nbytes


def probe_read_gbps(dev, nbytes=4 << 30, iters=10):
    import torch
    import paged_kv_cache_415_amd as pa
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    sink = torch.empty(16 * 2048, dtype=torch.uint8, device=dev)
    pa.pa_probe_read(src, sink)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        pa.pa_probe_read(src, sink)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / iters
    del src
    return nbytes / (ms * 1e-3) / 1e9


# ---------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands, on bounded samples, on the host's cores
# ---------------------------------------------------------------------------

# Samples (CPU-generated by workloads.py with the bench's seeds): the whole
# seeded batch (None) or the sequences at its front.
CPU_SAMPLES = {"llama3_8b_gqa_bf16": None, "llama2_7b_mha_f16": 16, "llama3_70b_fp8kv": None,
               "tiny_f32": None}
MIXED_SAMPLE = dict(num_forks=4, num_decode=28)
_CPU = {}          # inputs shared with the forked oracle processes


def host_cores() -> int:
    """Cores this process may run on, capped by OMP_NUM_THREADS when it is set."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _one_blas_thread():
    from threadpoolctl import threadpool_limits
    global _LIMIT
    _LIMIT = threadpool_limits(limits=1)


def _oracle_task(task):
    """One oracle call on one forked process: the decode of a set of
    sequences, or the prefill of one chunk over all heads."""
    import oracle
    kind, key, idx = task
    c = _CPU[key]
    if kind == "decode":
        s = c.spec
        oracle.decode_attention(c.q[idx], s.q_dtype, c.k_pool, c.v_pool, s.cache_dtype,
                                c.block_tables[idx], c.seq_lens[idx], s.scale, s.block_size,
                                s.num_kv_heads, c.k_scale, c.v_scale, v_cache_dtype=s.v_dtype,
                                k_block_scales=c.k_block_scales, v_block_scales=c.v_block_scales)
    elif kind == "mixed_decode":
        s = c.spec
        oracle.decode_attention(c.q_decode[idx], s.dtype, c.k_pool, c.v_pool, s.dtype,
                                c.decode_tables[idx], c.decode_lens[idx], s.scale, s.block_size,
                                s.num_kv_heads)
    else:    # one prefill chunk: rows of chunk idx[0], every head
        s = c.spec
        f = int(idx[0])
        qsl = c.query_start_loc
        lo, hi = int(qsl[f]), int(qsl[f + 1])
        oracle.prefill_chunk_attention(c.q_chunk[lo:hi], s.dtype, [0, hi - lo], c.k_pool, c.v_pool,
                                       s.dtype, c.prefill_tables[f:f + 1], c.prefill_lens[f:f + 1],
                                       s.scale, s.block_size, s.num_kv_heads)
    return 0


def cpu_baseline(args) -> dict:
    """The oracle on bounded samples of the workloads, timed on this host
    before the GPU is initialised: every core (one forked oracle process per
    core, one BLAS thread each) and, for the tiny and the Llama-2-7B-shaped
    samples, one thread."""
    import multiprocessing as mp
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W

    cores = host_cores()
    out = {"kind": "oracle", "cores": cores, "cpu_model": cpu_model(),
           "affinity_cores": len(os.sched_getaffinity(0)), "configs": {}}
    t_gen = time.perf_counter()
    tasks = {}
    for name, n in CPU_SAMPLES.items():
        case = W.make_decode_case(name, rep=0, num_seqs=n)
        _CPU[name] = case
        order = np.argsort(-case.seq_lens.astype(np.int64), kind="stable")   # longest first
        tasks[name] = [("decode", name, np.array([int(i)])) for i in order]
    mixed = W.make_mixed_case(**MIXED_SAMPLE)
    kp, vp = oracle.copy_blocks(mixed.k_pool, mixed.v_pool, mixed.cow_pairs)
    mixed.k_pool, mixed.v_pool = oracle.reshape_and_cache(
        kp, vp, mixed.spec.dtype, mixed.new_k, mixed.new_v, mixed.spec.dtype, mixed.slot_mapping,
        mixed.spec.block_size)
    _CPU["mixed"] = mixed
    out["generation_s"] = round(time.perf_counter() - t_gen, 2)

    ctx = mp.get_context("fork")       # the GPU is not initialised yet
    with ctx.Pool(cores, initializer=_one_blas_thread) as pool:
        pool.map(_oracle_task, tasks["tiny_f32"][:1])      # start-up of the workers
        for name in CPU_SAMPLES:
            case = _CPU[name]
            spec = case.spec
            t0 = time.perf_counter()
            pool.map(_oracle_task, tasks[name], chunksize=1)
            dt = time.perf_counter() - t0
            eff = W.effective_kv_bytes(case.seq_lens, spec.num_kv_heads, spec.head_dim,
                                       spec.cache_dtype, spec.v_dtype)
            what = (f"all {len(case.seq_lens)} sequences" if CPU_SAMPLES[name] is None
                    else f"the first {len(case.seq_lens)} sequences")
            out["configs"][name] = {
                "sample": f"{what} of the seeded batch ({int(case.seq_lens.sum())} context tokens, "
                          f"all heads)",
                "oracle_wall_s": round(dt, 4), "sample_effective_bytes": eff,
                "oracle_gbps": round(eff / dt / 1e9, 4)}
        # mixed step: every prefill chunk (one process each) and the decodes
        ms = mixed.spec
        pre = [("prefill", "mixed", np.array([f])) for f in range(len(mixed.prefill_lens))]
        dec = [("mixed_decode", "mixed", np.array([int(i)]))
               for i in np.argsort(-mixed.decode_lens.astype(np.int64), kind="stable")]
        t0 = time.perf_counter()
        pool.map(_oracle_task, pre + dec, chunksize=1)
        dt = time.perf_counter() - t0
    flops = mixed_prefill_flops(mixed)
    dec_eff = W.effective_kv_bytes(mixed.decode_lens, ms.num_kv_heads, ms.head_dim, ms.dtype)
    out["configs"]["mixed_prefix_bf16"] = {
        "sample": f"{len(mixed.prefill_lens)} of the 16 prefill chunks (512 tokens over a "
                  f"1,536-token context, all heads) and {len(mixed.decode_lens)} of the 112 decodes",
        "oracle_wall_s": round(dt, 4), "sample_prefill_flops": flops,
        "sample_decode_effective_bytes": dec_eff,
        "oracle_tflops_prefill_and_decode": round(flops / dt / 1e12, 5)}

    # one thread: the tiny workload (repeated for at least a second) and the
    # Llama-2-7B-shaped sample
    one = {}
    with threadpool_limits(1):
        for name, min_s in (("tiny_f32", 1.0), ("llama2_7b_mha_f16", 0.0)):
            case = _CPU[name]
            spec = case.spec
            idx = np.arange(len(case.seq_lens))
            passes, spent = 0, 0.0
            while passes == 0 or spent < min_s:
                t0 = time.perf_counter()
                _oracle_task(("decode", name, idx))
                spent += time.perf_counter() - t0
                passes += 1
            eff = W.effective_kv_bytes(case.seq_lens, spec.num_kv_heads, spec.head_dim,
                                       spec.cache_dtype, spec.v_dtype)
            one[name] = {"oracle_s_per_pass": round(spent / passes, 6), "passes": passes,
                         "oracle_gbps": round(eff / (spent / passes) / 1e9, 5)}
    out["one_thread"] = one
    _CPU.clear()
    head = out["configs"][HEADLINE]
    out["value"] = head["oracle_gbps"]
    out["unit"] = "GB/s"
    out["sample"] = (f"fp64 oracle decode of {head['sample']} of {HEADLINE} on {cores} cores "
                     f"(one oracle process per core, one BLAS thread each, sequences longest "
                     f"first), {head['oracle_wall_s']} s wall; the other workloads' samples under "
                     f"'configs', one-thread runs under 'one_thread'")
    return out


def mixed_prefill_flops(case) -> int:
    """Causal (query, key) pairs of the chunks x 4 D flops x query heads: query
    i of a chunk of L tokens in a context of n sees n - L + i + 1 keys."""
    import numpy as np
    s = case.spec
    pairs = 0
    for f in range(len(case.prefill_lens)):
        n, L = int(case.prefill_lens[f]), int(np.diff(case.query_start_loc)[f])
        pairs += L * (n - L) + L * (L + 1) // 2
    return pairs * s.num_q_heads * 4 * s.head_dim


def compare_cpu_gpu(cpu: dict, gpu: dict) -> None:
    """Oracle seconds beside GPU microseconds per step for each workload (the
    oracle's seconds scaled from its sample to the full batch by bytes, or
    flops for the mixed step), and their ratio."""
    for name, c in cpu.get("configs", {}).items():
        g = gpu.get(name)
        if g is None:
            continue
        if name == "mixed_prefix_bf16":
            full = g["prefill_flops"] + 0.0
            sample = c["sample_prefill_flops"]
            note = "prefill flops"
        else:
            full = g["effective_kv_bytes_per_step"] + 0.0
            sample = c["sample_effective_bytes"]
            note = "effective KV bytes"
        est = c["oracle_wall_s"] * full / sample
        c["oracle_s_per_step_est"] = round(est, 4)
        c["oracle_scaled_by"] = note
        c["gpu_us_per_step"] = round(g["ms_per_step"] * 1e3, 2)
        c["oracle_over_gpu"] = round(est / (g["ms_per_step"] * 1e-3), 1)


def decode_summary(res: dict) -> dict:
    """The per-workload object of the JSON line."""
    keep = ("ms_per_step", "value", "unit", "dtype", "pct_of_hbm_peak", "decode_tokens_per_s_per_layer",
            "decode_gbps_attention_plus_reduce", "reduce_avg_ms", "effective_kv_bytes_per_step")
    out = {k: res[k] for k in keep if k in res}
    out["config"] = res["config"]
    out["roofline"] = res["roofline"]
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path shards by sequence or KV head with no exchange)", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.config != "all" and args.config not in SUB_CONFIGS + [HEADLINE, "llama3_8b_int8kv",
                                                                   "llama3_8b_kfp8_vbf16",
                                                                   "llama3_70b_fp8kv_tp8",
                                                                   "mixed_70b_fp8kv", "mixed_70b_int8kv"]:
        print(f"unknown --config {args.config}", file=sys.stderr)
        sys.exit(2)
    # the CPU baseline forks oracle processes, so it runs before the GPU is initialised
    cpu = None if (args.no_cpu_baseline or args.config not in ("all", HEADLINE)) else cpu_baseline(args)

    import paged_kv_cache_415_amd  # noqa: F401  (fails loudly if libpa.so is missing)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    name = HEADLINE if args.config == "all" else args.config
    if name == "mixed_prefix_bf16":
        res = run_mixed_bench(args, dev)
        res["block_ops"] = run_block_ops_bench(dev)
    elif name in ("mixed_70b_fp8kv", "mixed_70b_int8kv"):
        import workloads as W
        res = run_mixed_bench(args, dev, W.MIXED_70B_FP8 if name == "mixed_70b_fp8kv" else W.MIXED_70B_INT8)
    else:
        res = run_decode_bench(args, dev, name)
    gpu_by_name = {name: res}
    if args.config == "all":
        subs = {}
        for sub in SUB_CONFIGS:
            torch.cuda.empty_cache()
            r = run_mixed_bench(args, dev) if sub == "mixed_prefix_bf16" else \
                run_decode_bench(args, dev, sub, extras=False)
            gpu_by_name[sub] = r
            subs[sub] = r if sub == "mixed_prefix_bf16" else decode_summary(r)
            subs[sub].pop("metric", None)
        res["configs"] = subs
    torch.cuda.empty_cache()
    res["probe_read_gbps"] = round(probe_read_gbps(dev), 1)
    res["probe_copy_bytes"] = probe_copy_once(dev)
    # the decode kernel's rate against what a plain streaming read gets from HBM
    dec = res["roofline"] if res["roofline"]["unit"] == "GB/s" else res.get("decode_roofline")
    if dec is not None and res["probe_read_gbps"] > 0:
        res["decode_kernel_pct_of_probe"] = round(100 * dec["achieved"] / res["probe_read_gbps"], 1)
    if cpu is not None:
        compare_cpu_gpu(cpu, gpu_by_name)
    line = {"metric": res.pop("metric"), "value": res.pop("value"), "unit": res.pop("unit"),
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": res.pop("ms_per_step"), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": res.pop("dtype"), "data": "synthetic",
            "config": res.pop("config"), "roofline": res.pop("roofline")}
    line["cpu_baseline"] = cpu
    line.update(res)
    line["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
