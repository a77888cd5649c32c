"""GPU parity of pa_reshape_and_cache + pa_decode against the fp64 oracle.

Tolerances (max-abs on outputs): 5e-3 for fp32 queries, 2e-2 for fp16 / bf16
queries (including fp8 caches).  Scatter results must be byte-identical over
the whole pool, NaN-poisoned slots included.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_cases import TOL, DecodeRun, as_f64, custom_spec, lib, max_abs, oracle_step, up, up_int

pytestmark = pytest.mark.gpu

FULL_CONFIGS = ["tiny_f32", "llama2_7b_mha_f16", "llama3_8b_gqa_bf16", "llama3_70b_fp8kv",
                "llama3_8b_kfp8_vbf16", "llama3_8b_int8kv", "llama3_70b_fp8kv_tp8"]


@pytest.fixture(scope="module")
def full_cases():
    cache = {}

    def get(name):
        if name not in cache:
            case = W.make_decode_case(name)
            cache[name] = (case, oracle_step(case))
        return cache[name]
    return get


@pytest.mark.parametrize("name", FULL_CONFIGS)
def test_full_config_scatter_and_decode(name, full_cases):
    """Every output of the full workload, in the launch configuration the bench uses."""
    case, (ref, okp, ovp) = full_cases(name)
    print(f"[decode parity] {name}: S={len(case.seq_lens)} tokens={int(case.seq_lens.sum())}",
          flush=True)
    run = DecodeRun(case)
    run.scatter()
    torch.cuda.synchronize()
    dt, vdt = case.spec.cache_dtype, case.spec.v_dtype
    assert np.array_equal(W.torch_to_bits(run.k_pool, dt), okp), "K pool differs after scatter"
    assert np.array_equal(W.torch_to_bits(run.v_pool, vdt), ovp), "V pool differs after scatter"
    out = run.decode()
    err = max_abs(out, ref)
    print(f"[decode parity] {name}: max-abs {err:.3e}", flush=True)
    assert err <= TOL[case.spec.q_dtype]


@pytest.mark.parametrize("partition", [32, 512])
def test_full_gqa_fixed_partitions(partition, full_cases):
    """Fixed partitions over the full Llama-3-8B-shaped batch: with 512-token partitions every
    workgroup's share fits its LDS merge slots (partials merged on the CU); 32-token partitions
    give shares of hundreds of partitions, which go through the workspace and the reduce."""
    case, (ref, _, _) = full_cases("llama3_8b_gqa_bf16")
    print(f"[decode parity] llama3_8b_gqa_bf16 fixed partitions of {partition}", flush=True)
    run = DecodeRun(case)
    run.scatter()
    out = run.decode(partition_size=partition)
    assert max_abs(out, ref) <= TOL[case.spec.q_dtype]


@pytest.fixture(scope="module")
def max_seqs_case():
    """8000 sequences (the most one call plans in LDS) of 1-64 tokens: the plan takes most of
    the workgroup's LDS, which leaves fewer slots for partials merged on the CU."""
    spec = custom_spec("maxseqs_bf16_8_2_128_16", 8, 2, 128, 16, "bf16", "bf16")
    lens = [int(x) for x in np.random.default_rng(7).integers(1, 65, size=8000)]
    case = W.make_decode_case(spec, lens=lens)
    return case, oracle_step(case)


@pytest.mark.parametrize("partition", [0, 32, -1])
def test_max_sequences(partition, max_seqs_case):
    case, (ref, okp, ovp) = max_seqs_case
    print(f"[decode parity] 8000 sequences, partition {partition}", flush=True)
    run = DecodeRun(case)
    run.scatter()
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(run.k_pool, "bf16"), okp)
    out = run.decode(partition_size=partition)
    assert max_abs(out, ref) <= TOL["bf16"]


@pytest.fixture(scope="module")
def max_seqs_8bit_cases():
    """The 8000-sequence plan with 8-bit caches at head_dim 128, whose waves also
    take 4 KB each of LDS for whole-line K staging, placed after the merge slots."""
    lens = [int(x) for x in np.random.default_rng(8).integers(1, 65, size=8000)]
    out = {}
    for c_dt in ("fp8_e4m3", "int8"):
        spec = custom_spec(f"maxseqs_{c_dt}_8_2_128_16", 8, 2, 128, 16, "bf16", c_dt)
        case = W.make_decode_case(spec, lens=lens)
        out[c_dt] = (case, oracle_step(case))
    return out


@pytest.mark.parametrize("c_dt", ["fp8_e4m3", "int8"])
@pytest.mark.parametrize("partition", [0, 512, -1])
def test_max_sequences_8bit(c_dt, partition, max_seqs_8bit_cases):
    case, (ref, okp, ovp) = max_seqs_8bit_cases[c_dt]
    print(f"[decode parity] 8000 sequences, {c_dt}, partition {partition}", flush=True)
    run = DecodeRun(case)
    run.scatter()
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(run.k_pool, c_dt), okp)
    assert np.array_equal(W.torch_to_bits(run.v_pool, c_dt), ovp)
    out = run.decode(partition_size=partition)
    assert max_abs(out, ref) <= TOL["bf16"]


@pytest.mark.parametrize("partition", [0, 32, -1])
def test_int8_rows_past_the_end_never_count(partition):
    """int8 has no NaN to poison unwritten rows with: they hold the code -128
    (never written by the quantiser).  With every query -1 and every K code of
    a valid row >= 0, a poisoned K row would give by far the largest logit and
    pull the output to -128 x the V scale, so a read past a sequence's end (or
    into table padding) shows as a large error instead of a NaN."""
    spec = custom_spec("int8_past_end", 8, 2, 128, 16, "bf16", "int8")
    case = W.make_decode_case(spec, lens=[1, 15, 17, 31, 33, 100, 257, 1000])
    kp = case.k_pool.view(np.int8).copy()
    kp[kp != -128] = np.abs(kp[kp != -128])         # valid K codes >= 0
    case.k_pool = kp.view(np.uint8)
    case.new_k = W.to_bits(np.abs(W.bits_to_torch(case.new_k, "bf16").float().numpy()), "bf16")
    case.q = W.to_bits(-np.ones(W.bits_to_torch(case.q, "bf16").shape, np.float32), "bf16")
    ref, okp, _ = oracle_step(case)
    assert (kp.view(np.int8) == -128).any()
    run = DecodeRun(case)
    run.scatter()
    out = run.decode(partition_size=partition)
    assert np.array_equal(W.torch_to_bits(run.k_pool, "int8"), okp)
    assert max_abs(out, ref) <= TOL["bf16"]
    # the oracle's output stays within the valid V values; -128 x scale would not
    bound = float(np.max(case.v_block_scales)) * 127
    assert float(np.abs(ref).max()) <= bound


@pytest.mark.parametrize("partition", [32, 64, 160, 512, -1])
def test_split_sizes_agree(partition):
    sub = W.make_decode_case("llama3_8b_gqa_bf16", lens=[1, 31, 32, 33, 200, 511, 512, 513, 2500])
    sref, _, _ = oracle_step(sub)
    run = DecodeRun(sub)
    run.scatter()
    out = run.decode(partition_size=partition)
    assert max_abs(out, sref) <= TOL["bf16"]


def test_stages_equal_single_call():
    case = W.make_decode_case("llama3_70b_fp8kv", lens=[5, 700, 1500, 3000])
    run = DecodeRun(case)
    run.scatter()
    a = run.decode(partition_size=512)
    b = run.decode(partition_size=512, stages=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_bitwise_repeatable():
    case = W.make_decode_case("llama3_8b_gqa_bf16", num_seqs=24)
    run = DecodeRun(case)
    run.scatter()
    a = run.decode()
    for _ in range(3):
        assert torch.equal(run.decode().view(torch.int16), a.view(torch.int16))


@pytest.mark.parametrize("name", ["llama2_7b_mha_f16", "llama3_70b_fp8kv"])
def test_permuting_physical_blocks_is_bitwise_invisible(name):
    case = W.make_decode_case(name, num_seqs=12)
    run = DecodeRun(case)
    run.scatter()
    a = run.decode()
    rng = np.random.default_rng(99)
    perm = rng.permutation(case.num_blocks)          # block b moves to perm[b]
    kp = np.empty_like(case.k_pool)
    vp = np.empty_like(case.v_pool)
    kp[perm] = case.k_pool
    vp[perm] = case.v_pool
    moved = W.DecodeCase(**{**case.__dict__, "k_pool": kp, "v_pool": vp,
                            "block_tables": perm[case.block_tables].astype(np.int32),
                            "slot_mapping": perm[case.slot_mapping // case.spec.block_size]
                            * case.spec.block_size + case.slot_mapping % case.spec.block_size,
                            "poison_block": int(perm[case.poison_block])})
    run2 = DecodeRun(moved)
    run2.scatter()
    b = run2.decode()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("q_dt,c_dt", [("f32", "f32"), ("f16", "f16"), ("bf16", "bf16"),
                                       ("bf16", "fp8_e4m3"), ("f16", "fp8_e4m3")])
def test_length_one_returns_its_value_row(q_dt, c_dt):
    spec = custom_spec(f"len1_{q_dt}_{c_dt}", 8, 2, 128, 16, q_dt, c_dt)
    case = W.make_decode_case(spec, lens=[1, 1, 1])
    if c_dt == "fp8_e4m3":
        case.k_scale = case.v_scale = 1.0
    ref, _, _ = oracle_step(case)
    run = DecodeRun(case)
    run.scatter()
    out = run.decode()
    # p = 1 exactly, so the output is the stored value row rounded once to q's type
    exp = torch.from_numpy(ref).to(out.dtype)
    assert torch.equal(out.cpu().view(torch.int16 if q_dt != "f32" else torch.int32),
                       exp.view(torch.int16 if q_dt != "f32" else torch.int32))


@pytest.mark.parametrize("q_dt", ["bf16", "f16"])
def test_fp8_every_code_decodes_exactly(q_dt):
    """Length-1 sequences whose value rows hold every finite E4M3 code."""
    spec = custom_spec(f"codes_{q_dt}", 1, 1, 128, 16, q_dt, "fp8_e4m3")
    case = W.make_decode_case(spec, lens=[1, 1])
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] + [0, 0], np.uint8)
    for s in range(2):
        blk = case.block_tables[s, 0]
        case.v_pool[blk, 0, 0, :] = codes[s * 128:(s + 1) * 128]
        case.k_pool[blk, 0, 0, :] = 0          # logit 0: the single token gets p = 1
    # scatter of the newest token is skipped so the planted rows stay
    case.slot_mapping[:] = -1
    case.k_scale = case.v_scale = 1.0
    run = DecodeRun(case)
    run.scatter()
    out = as_f64(run.decode())
    want = oracle.e4m3_value_table()[codes].reshape(2, 1, 128)
    bad = np.nonzero(out != want)
    assert bad[0].size == 0, f"codes decoded wrongly: {[(int(codes[s*128+d]), out[s,0,d]) for s,_,d in zip(*bad)][:8]}"


@pytest.mark.parametrize("partition", [0, 32, -1])
def test_lengths_over_max_seq_len_are_clamped(partition):
    """seq_lens above max_seq_len are clamped to it: the output is the attention over the first
    max_seq_len tokens (the newest token of a longer sequence is scattered but not attended)."""
    case = W.make_decode_case("llama3_8b_gqa_bf16", lens=[50, 150, 300, 128])
    print(f"[decode parity] lengths clamped to 128, partition {partition}", flush=True)
    run = DecodeRun(case)
    run.scatter()
    out = run.decode(partition_size=partition, max_seq_len=128)
    _, kp, vp = oracle_step(case)
    s = case.spec
    clamped = np.minimum(case.seq_lens, 128).astype(np.int32)
    ref = oracle.decode_attention(case.q, s.q_dtype, kp, vp, s.cache_dtype, case.block_tables,
                                  clamped, s.scale, s.block_size, s.num_kv_heads, case.k_scale,
                                  case.v_scale, v_cache_dtype=s.v_dtype)
    assert max_abs(out, ref) <= TOL["bf16"]


def test_zero_length_sequence_gives_zeros():
    case = W.make_decode_case("llama3_8b_gqa_bf16", lens=[40, 1, 17])
    run = DecodeRun(case)
    run.scatter()
    run.lens = up_int(np.array([40, 0, 17], np.int32))
    out = run.decode(partition_size=32)
    ref, _, _ = oracle_step(case)
    assert torch.count_nonzero(out[1]) == 0
    assert max_abs(out[[0, 2]], ref[[0, 2]]) <= TOL["bf16"]


@pytest.mark.parametrize("partition", [0, -1])
def test_tp8_share_other_cuts(partition, full_cases):
    """The tensor-parallel share of the 70B-shaped layer (one KV head) with
    the balanced cut and whole pairs: few pairs, so most waves of a launch
    have no work."""
    case, (ref, _, _) = full_cases("llama3_70b_fp8kv_tp8")
    print(f"[decode parity] llama3_70b_fp8kv_tp8, partition {partition}", flush=True)
    run = DecodeRun(case)
    run.scatter()
    out = run.decode(partition_size=partition)
    assert max_abs(out, ref) <= TOL["bf16"]


@pytest.mark.parametrize("name", ["llama3_8b_gqa_bf16", "llama3_70b_fp8kv"])
@pytest.mark.parametrize("partition", [0, 32, 512, -1])
def test_runs_of_empty_sequences(name, partition):
    """Empty sequences first, last and in runs, with every cut: their outputs
    are zero, and the work shares of the others (cut by units, which empty
    sequences do not have) and their merges are unaffected."""
    lens = [1, 700, 1, 1, 45, 1300, 1, 33, 1, 1, 2049, 1]
    empty = [0, 2, 3, 6, 8, 9, 11]
    keep = [i for i in range(len(lens)) if i not in empty]
    case = W.make_decode_case(name, lens=lens)
    print(f"[decode parity] {name}, empty sequences {empty}, partition {partition}", flush=True)
    run = DecodeRun(case)
    run.scatter()
    dl = np.array(lens, np.int32)
    dl[empty] = 0
    run.lens = up_int(dl)
    out = run.decode(partition_size=partition)
    ref, _, _ = oracle_step(case)
    assert torch.count_nonzero(out[empty]) == 0
    assert max_abs(out[keep], ref[keep]) <= TOL[case.spec.q_dtype]


def test_all_sequences_empty():
    """A batch whose sequences are all empty: every output is zero, every cut."""
    case = W.make_decode_case("llama3_8b_gqa_bf16", lens=[1, 1, 1, 1])
    run = DecodeRun(case)
    run.scatter()
    run.lens = up_int(np.zeros(4, np.int32))
    for partition in (0, 32, -1):
        out = run.decode(partition_size=partition)
        assert torch.count_nonzero(out) == 0


SWEEP = [
    # (q, cache, Hq, Hkv, D, bs)
    ("bf16", "bf16", 8, 8, 128, 16),
    ("bf16", "bf16", 16, 1, 128, 32),
    ("bf16", "bf16", 6, 2, 64, 16),
    ("f16", "f16", 32, 4, 64, 32),
    ("f16", "f16", 4, 2, 128, 32),
    ("bf16", "fp8_e4m3", 8, 1, 64, 16),
    ("f16", "fp8_e4m3", 12, 3, 128, 32),
    ("bf16", "fp8_e4m3", 64, 8, 128, 32),
    ("f32", "f32", 4, 1, 128, 32),
    ("f32", "f32", 5, 5, 64, 16),
    # 8- and 64-token blocks
    ("bf16", "bf16", 8, 2, 128, 8),
    ("f16", "f16", 4, 4, 64, 64),
    ("bf16", "fp8_e4m3", 16, 2, 128, 8),
    ("bf16", "fp8_e4m3", 8, 8, 64, 64),
    ("bf16", "fp8_e4m3", 16, 4, 128, 64),
    ("f16", "f16", 32, 32, 128, 64),
    ("f32", "f32", 4, 2, 64, 8),
    ("f32", "f32", 2, 1, 128, 64),
]
LENS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 257, 600, 1031]


@pytest.mark.parametrize("q_dt,c_dt,hq,hkv,d,bs", SWEEP)
@pytest.mark.parametrize("partition", [0, 64, -1])
def test_shape_sweep(q_dt, c_dt, hq, hkv, d, bs, partition):
    if partition > 0 and partition % bs:
        pytest.skip("partition must be a multiple of block_size")
    spec = custom_spec(f"sweep_{q_dt}_{c_dt}_{hq}_{hkv}_{d}_{bs}", hq, hkv, d, bs, q_dt, c_dt)
    case = W.make_decode_case(spec, lens=LENS)
    ref, okp, ovp = oracle_step(case)
    run = DecodeRun(case)
    run.scatter()
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(run.k_pool, c_dt), okp)
    out = run.decode(partition_size=partition)
    assert max_abs(out, ref) <= TOL[q_dt]


MIXED = [
    # fp8 K beside a V pool of the query type: (q, Hq, Hkv, D, bs)
    ("bf16", 8, 8, 128, 16),
    ("bf16", 32, 8, 128, 32),
    ("f16", 12, 3, 128, 16),
    ("bf16", 8, 1, 64, 16),
    ("f16", 4, 4, 64, 32),
    ("bf16", 16, 2, 128, 8),
    ("bf16", 8, 8, 64, 64),
]


@pytest.mark.parametrize("q_dt,hq,hkv,d,bs", MIXED)
@pytest.mark.parametrize("partition", [0, 64, -1])
def test_mixed_k_fp8_v_16bit_sweep(q_dt, hq, hkv, d, bs, partition):
    """intelliparadigm page §6.1: fp8 K cache, 16-bit V cache (scatter byte-exact in both pools)."""
    if partition > 0 and partition % bs:
        pytest.skip("partition must be a multiple of block_size")
    spec = custom_spec(f"mixed_{q_dt}_{hq}_{hkv}_{d}_{bs}", hq, hkv, d, bs, q_dt, "fp8_e4m3",
                       v_cache_dtype=q_dt)
    case = W.make_decode_case(spec, lens=LENS)
    ref, okp, ovp = oracle_step(case)
    run = DecodeRun(case)
    run.scatter()
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(run.k_pool, "fp8_e4m3"), okp)
    assert np.array_equal(W.torch_to_bits(run.v_pool, q_dt), ovp)
    out = run.decode(partition_size=partition)
    assert max_abs(out, ref) <= TOL[q_dt]
    if partition == 64:
        staged = run.decode(partition_size=partition, stages=True)
        assert torch.equal(out.view(torch.int16), staged.view(torch.int16))


def test_mixed_length_one_returns_its_value_row():
    spec = custom_spec("len1_mixed", 8, 2, 128, 16, "bf16", "fp8_e4m3", v_cache_dtype="bf16")
    case = W.make_decode_case(spec, lens=[1, 1, 1])
    ref, _, _ = oracle_step(case)
    run = DecodeRun(case)
    run.scatter()
    out = run.decode()
    exp = torch.from_numpy(ref).to(out.dtype)
    assert torch.equal(out.cpu().view(torch.int16), exp.view(torch.int16))


INT8 = [
    # int8 K and V with per-(block, KV head) scales: (q, Hq, Hkv, D, bs)
    ("bf16", 8, 8, 128, 16),
    ("bf16", 32, 8, 128, 32),
    ("f16", 12, 3, 128, 16),
    ("bf16", 8, 1, 64, 16),
    ("f16", 4, 4, 64, 32),
    ("bf16", 16, 2, 128, 8),
    ("bf16", 8, 8, 64, 64),
    ("f16", 16, 4, 128, 64),
]


@pytest.mark.parametrize("q_dt,hq,hkv,d,bs", INT8)
@pytest.mark.parametrize("partition", [0, 64, -1])
def test_int8_per_block_scales_sweep(q_dt, hq, hkv, d, bs, partition):
    """ybb.press §6.2 (INT8 KV cache), per-(block, KV head) scales: scatter byte-exact, decode
    within the bar, staged == single call bitwise."""
    if partition > 0 and partition % bs:
        pytest.skip("partition must be a multiple of block_size")
    spec = custom_spec(f"int8_{q_dt}_{hq}_{hkv}_{d}_{bs}", hq, hkv, d, bs, q_dt, "int8")
    case = W.make_decode_case(spec, lens=LENS)
    ref, okp, ovp = oracle_step(case)
    run = DecodeRun(case)
    run.scatter()
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(run.k_pool, "int8"), okp)
    assert np.array_equal(W.torch_to_bits(run.v_pool, "int8"), ovp)
    out = run.decode(partition_size=partition)
    assert max_abs(out, ref) <= TOL[q_dt]
    if partition == 64:
        staged = run.decode(partition_size=partition, stages=True)
        assert torch.equal(out.view(torch.int16), staged.view(torch.int16))


def test_int8_every_code_decodes_exactly():
    """Length-1 sequences (p = 1) whose value rows hold every code -127..127, scale 1."""
    spec = custom_spec("int8_codes", 1, 1, 128, 16, "bf16", "int8")
    case = W.make_decode_case(spec, lens=[1, 1])
    codes = np.r_[np.arange(-127, 128), np.zeros(1)].astype(np.int8)        # 256 entries
    for s in range(2):
        blk = case.block_tables[s, 0]
        case.v_pool[blk, 0, 0, :] = codes[s * 128:(s + 1) * 128].view(np.uint8)
        case.k_pool[blk, 0, 0, :] = 0
        case.k_block_scales[blk, 0] = case.v_block_scales[blk, 0] = 1.0
    case.slot_mapping[:] = -1
    run = DecodeRun(case)
    run.scatter()
    out = as_f64(run.decode())
    want = codes.astype(np.float64).reshape(2, 1, 128)
    assert np.array_equal(out, want)


APPEND = [
    # (q = cache, Hq, Hkv, D, bs, lens)
    ("f16", 32, 32, 128, 16, None),            # the Llama-2-7B-shaped workload in full
    ("bf16", 8, 2, 128, 16, LENS),
    ("bf16", 16, 1, 128, 32, LENS),
    ("f16", 6, 2, 64, 16, LENS),
    ("bf16", 8, 2, 128, 8, LENS),
    ("f16", 4, 4, 64, 64, LENS),
]


@pytest.mark.parametrize("q_dt,hq,hkv,d,bs,lens", APPEND)
@pytest.mark.parametrize("partition", [0, 64, -1])
def test_append_equals_scatter_then_decode(q_dt, hq, hkv, d, bs, lens, partition):
    """pa_decode_append == pa_reshape_and_cache + pa_decode, bit for bit (outputs and pools)."""
    if partition > 0 and partition % bs:
        pytest.skip("partition must be a multiple of block_size")
    if lens is None:
        case = W.make_decode_case("llama2_7b_mha_f16")
    else:
        spec = custom_spec(f"append_{q_dt}_{hq}_{hkv}_{d}_{bs}", hq, hkv, d, bs, q_dt, q_dt)
        case = W.make_decode_case(spec, lens=lens)
    pa = lib()
    ref_run = DecodeRun(case)
    ref_run.scatter()
    ref = ref_run.decode(partition_size=partition)
    run = DecodeRun(case)
    # the new rows as a strided view (every other row of a buffer twice as tall)
    wide_k = torch.zeros((2 * run.new_k.shape[0], *run.new_k.shape[1:]), dtype=run.new_k.dtype,
                         device=run.new_k.device)
    wide_k[::2] = run.new_k
    nk = wide_k[::2]
    out = torch.empty_like(run.q)
    ws = pa.decode_workspace(run.q, run.k_pool, run.max_len, partition)
    pa.pa_decode_append(out, run.q, nk, run.new_v, run.k_pool, run.v_pool, run.tables, run.lens,
                        case.spec.scale, max_seq_len=run.max_len, partition_size=partition,
                        workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(run.k_pool.view(torch.int16), ref_run.k_pool.view(torch.int16))
    assert torch.equal(run.v_pool.view(torch.int16), ref_run.v_pool.view(torch.int16))
    # the two stages give the same
    run2 = DecodeRun(case)
    out2 = torch.empty_like(run2.q)
    args = (out2, run2.q, run2.new_k, run2.new_v, run2.k_pool, run2.v_pool, run2.tables, run2.lens,
            case.spec.scale)
    pa.pa_decode_attention_append(*args, max_seq_len=run2.max_len, partition_size=partition,
                                  workspace=ws)
    pa.pa_decode_reduce(out2, run2.q, run2.k_pool, run2.v_pool, run2.tables, run2.lens,
                        case.spec.scale, max_seq_len=run2.max_len, partition_size=partition,
                        workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("name", ["llama2_7b_mha_f16", "llama3_8b_gqa_bf16"])
@pytest.mark.parametrize("partition", [0, 64, -1])
def test_append_full_config_matches_oracle(name, partition, full_cases):
    """pa_decode_append (the scatter folded into the decode kernel) on the full
    workload against the oracle's scatter + decode: every output, both pools
    byte for byte."""
    case, (ref, okp, ovp) = full_cases(name)
    print(f"[append parity] {name} partition {partition}", flush=True)
    pa = lib()
    run = DecodeRun(case)
    out = torch.empty_like(run.q)
    ws = pa.decode_workspace(run.q, run.k_pool, run.max_len, partition)
    pa.pa_decode_append(out, run.q, run.new_k, run.new_v, run.k_pool, run.v_pool, run.tables,
                        run.lens, case.spec.scale, max_seq_len=run.max_len,
                        partition_size=partition, workspace=ws)
    torch.cuda.synchronize()
    dt = case.spec.cache_dtype
    assert np.array_equal(W.torch_to_bits(run.k_pool, dt), okp)
    assert np.array_equal(W.torch_to_bits(run.v_pool, dt), ovp)
    assert max_abs(out, ref) <= TOL[case.spec.q_dtype]


def _rewrite_k_dim0(case, values_per_seq, k_scale=None):
    """Set dimension 0 of every K row of head 0 to the given per-token values
    (the newest token's through the scatter input); other dims keep their
    values.  For an fp8 cache the pool is re-encoded with k_scale."""
    s = case.spec
    bs, dt = s.block_size, s.cache_dtype
    old_scale = case.k_scale
    kf = W.bits_to_torch(case.k_pool, dt).float().numpy() * np.float32(old_scale)
    nk = W.bits_to_torch(case.new_k, case.src_dtype).float().numpy()
    for q, vals in enumerate(values_per_seq):
        n = int(case.seq_lens[q])
        for j in range(n - 1):
            kf[case.block_tables[q, j // bs], 0, j % bs, 0] = vals[j]
        nk[q, 0, 0] = vals[n - 1]
    if k_scale is not None:
        case.k_scale = float(np.float32(k_scale))
    case.k_pool = W.to_bits(kf / np.float32(case.k_scale) if dt == "fp8_e4m3" else kf, dt)
    case.new_k = W.to_bits(nk, case.src_dtype)


@pytest.mark.parametrize("q_dt,c_dt", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "fp8_e4m3"),
                                       ("f32", "f32")])
@pytest.mark.parametrize("partition", [0, -1])
def test_running_max_moves_many_times(q_dt, c_dt, partition):
    """Logits that rise along the context, fall, jump at the last token or
    saw-tooth: the running max must move many times inside one segment, by
    small and by large steps (the decode kernel defers rescaling until the
    max has grown by 2^8)."""
    spec = custom_spec(f"trend_{q_dt}_{c_dt}", 4, 1, 128, 16, q_dt, c_dt)
    lens = [1500, 700, 64, 333]
    case = W.make_decode_case(spec, lens=lens)
    trends = [np.linspace(0.0, 85.0, 1500), np.linspace(85.0, 0.0, 700),
              np.r_[np.zeros(63), 100.0], (np.arange(333) % 50) * 1.5]
    _rewrite_k_dim0(case, trends, k_scale=100.0 / 448.0 if c_dt == "fp8_e4m3" else None)
    qf = np.zeros((len(lens), 4, 128), np.float32)
    qf[:, :, 0] = [8.0, 4.0, -8.0, 1.0]          # logit = scale * q0 * k0
    case.q = W.to_bits(qf, q_dt)
    ref, okp, _ = oracle_step(case)
    run = DecodeRun(case)
    run.scatter()
    torch.cuda.synchronize()
    assert np.array_equal(W.torch_to_bits(run.k_pool, c_dt), okp)
    out = run.decode(partition_size=partition)
    assert max_abs(out, ref) <= TOL[q_dt]


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.4])
def test_decode_any_scale(scale):
    """Zero scale (uniform weights) and a negative scale against the oracle."""
    spec = custom_spec("scale_sweep", 8, 2, 128, 16, "bf16", "bf16")
    case = W.make_decode_case(spec, lens=[1, 40, 333, 1000])
    s = case.spec
    kp, vp = oracle.reshape_and_cache(case.k_pool, case.v_pool, s.cache_dtype, case.new_k,
                                      case.new_v, case.src_dtype, case.slot_mapping, s.block_size)
    ref = oracle.decode_attention(case.q, s.q_dtype, kp, vp, s.cache_dtype, case.block_tables,
                                  case.seq_lens, scale, s.block_size, s.num_kv_heads)
    run = DecodeRun(case)
    run.scatter()
    pa = lib()
    out = torch.empty_like(run.q)
    ws = pa.decode_workspace(run.q, run.k_pool, run.max_len, 0)
    pa.pa_decode(out, run.q, run.k_pool, run.v_pool, run.tables, run.lens, scale,
                 max_seq_len=run.max_len, workspace=ws)
    torch.cuda.synchronize()
    assert max_abs(out, ref) <= TOL["bf16"]


@pytest.mark.parametrize("partition", [0, 64, -1])
def test_int8_f16_queries_large_value_scales(partition):
    """f16 queries over an int8 cache whose V values reach about 6e4 (block V
    scales near 470): the value operand p x scale must stay inside f16's range
    while the running max moves (queries x 6 so that logits spread widely)."""
    spec = custom_spec("int8_f16_big_v", 8, 2, 128, 16, "f16", "int8")
    case = W.make_decode_case(spec, lens=[3, 40, 130, 700, 1500])
    grow = np.float32(1.2e4)
    case.v_block_scales = (case.v_block_scales * grow).astype(np.float32)
    nv = W.bits_to_torch(case.new_v, "f16").float().numpy() * grow
    case.new_v = W.to_bits(np.clip(nv, -6e4, 6e4), "f16")
    case.q = W.to_bits(W.bits_to_torch(case.q, "f16").float().numpy() * 6, "f16")
    ref, _, ovp = oracle_step(case)
    assert float(np.max(case.v_block_scales)) > 300
    run = DecodeRun(case)
    run.scatter()
    out = run.decode(partition_size=partition)
    assert np.array_equal(W.torch_to_bits(run.v_pool, "int8"), ovp)
    # relative to the values' size: f16 keeps 11 significant bits
    err = max_abs(out, ref)
    assert err <= TOL["f16"] * float(np.abs(ref).max()) / 4, err


LONG = [("bf16", "bf16", 32, 8), ("bf16", "fp8_e4m3", 64, 8)]
_LONG_CASES = {}


def _long_case(q_dt, c_dt, hq, hkv):
    """Contexts of 131,072 and 70,001 tokens beside two short ones (D 128,
    block 16); built and checked against the oracle once per format."""
    key = (q_dt, c_dt, hq, hkv)
    if key not in _LONG_CASES:
        spec = custom_spec(f"long_{c_dt}_{hq}_{hkv}", hq, hkv, 128, 16, q_dt, c_dt)
        case = W.make_decode_case(spec, lens=[131072, 70001, 1, 4097])
        ref, _, _ = oracle_step(case)
        _LONG_CASES[key] = (case, ref)
    return _LONG_CASES[key]


@pytest.mark.parametrize("q_dt,c_dt,hq,hkv", LONG)
@pytest.mark.parametrize("partition", [0, 512, -1])
def test_long_contexts(q_dt, c_dt, hq, hkv, partition):
    """The split planning at its largest: the balanced cut's shortest range
    grows with the longest context (256 steps here, 17 partials at most),
    512-token partitions give 256 partials for the longest pair, and a whole
    pair is one wave streaming 131,072 tokens."""
    print(f"[decode parity] long contexts {c_dt} {hq}/{hkv} partition {partition}", flush=True)
    case, ref = _long_case(q_dt, c_dt, hq, hkv)
    run = DecodeRun(case)
    run.scatter()
    torch.cuda.synchronize()
    out = run.decode(partition_size=partition)
    assert max_abs(out, ref) <= TOL[q_dt]
