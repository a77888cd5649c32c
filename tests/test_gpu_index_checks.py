"""GPU tests of the index checks (pa_check_block_tables, pa_check_slots): bad
block ids, lengths, chunk offsets and slots planted on the host are reported
in the device error record; valid inputs report nothing; table entries past
a sequence's last block (padding) are never looked at."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_cases import lib, up_int

pytestmark = pytest.mark.gpu

INT_MAX = 2 ** 31 - 1


def _err():
    return torch.full((3,), -7, dtype=torch.int32, device="cuda")   # the call resets it


def _tables_check(tables, lens, num_blocks, bs, max_len=0, qsl=None):
    pa = lib()
    err = _err()
    pa.pa_check_block_tables(up_int(tables), up_int(lens), num_blocks, bs, err, max_seq_len=max_len,
                             query_start_loc=None if qsl is None else up_int(qsl))
    torch.cuda.synchronize()
    return [int(x) for x in err.cpu()]


def test_valid_workload_tables_report_nothing():
    lay = W.make_decode_layout("llama3_8b_gqa_bf16")
    lens = lay.seq_lens.astype(np.int32)
    # the padding entries hold a poison block id; give them out-of-range values too
    tables = lay.block_tables.copy()
    for s, n in enumerate(lens):
        tables[s, -(-int(n) // 16):] = INT_MAX
    assert _tables_check(tables, lens, lay.num_blocks, 16, max_len=int(lens.max())) == [0, 0, INT_MAX]


def test_planted_block_ids_and_lengths_are_reported():
    lay = W.make_decode_layout("llama2_7b_mha_f16")
    lens = lay.seq_lens.astype(np.int32).copy()
    tables = lay.block_tables.copy()
    nb = lay.num_blocks
    tables[5, 0] = nb                     # one past the pool
    tables[9, int(lens[9] - 1) // 16] = -3  # the last block of sequence 9
    lens[12] = tables.shape[1] * 16 + 1    # beyond the table
    lens[40] = -1
    got = _tables_check(tables, lens, nb, 16)
    assert got[0] == 1 | 2
    assert got[1] == 4 and got[2] == 5
    # max_seq_len: lengths above it are reported as well
    lens2 = lay.seq_lens.astype(np.int32)
    got = _tables_check(lay.block_tables, lens2, nb, 16, max_len=int(lens2.max()) - 1)
    assert got[0] == 2 and got[1] == int((lens2 == lens2.max()).sum())


def test_planted_chunk_offsets_are_reported():
    lens = np.array([40, 70, 9], np.int32)
    tables = np.arange(3 * 8, dtype=np.int32).reshape(3, 8)
    good = np.array([0, 10, 50, 59], np.int32)
    assert _tables_check(tables, lens, 64, 16, qsl=good) == [0, 0, INT_MAX]
    bad = good.copy()
    bad[2] = 5                              # decreasing
    got = _tables_check(tables, lens, 64, 16, qsl=bad)
    assert got[0] == 8 and got[2] == 1
    longer = np.array([0, 41, 50, 59], np.int32)   # a chunk longer than its context
    assert _tables_check(tables, lens, 64, 16, qsl=longer)[0] == 8


def test_slots():
    pa = lib()
    nb, bs = 100, 16
    slots = np.array([0, 5, -1, nb * bs - 1, nb * bs, 77, nb * bs + 9000, -5], np.int64)
    err = _err()
    pa.pa_check_slots(up_int(slots), nb, bs, err)
    torch.cuda.synchronize()
    assert [int(x) for x in err.cpu()] == [4, 2, 4]
    err = _err()
    pa.pa_check_slots(up_int(slots[:4]), nb, bs, err)
    torch.cuda.synchronize()
    assert [int(x) for x in err.cpu()] == [0, 0, INT_MAX]
    # no tokens: only the reset
    err = _err()
    pa.pa_check_slots(torch.zeros(0, dtype=torch.int64, device="cuda"), nb, bs, err)
    torch.cuda.synchronize()
    assert [int(x) for x in err.cpu()] == [0, 0, INT_MAX]


def test_mixed_workload_indices_are_valid():
    case = W.make_mixed_case()
    nb, bs = case.k_pool.shape[0], case.spec.block_size
    lens = case.prefill_lens
    assert _tables_check(case.prefill_tables, lens, nb, bs, qsl=case.query_start_loc) == [0, 0, INT_MAX]
    assert _tables_check(case.decode_tables, case.decode_lens, nb, bs) == [0, 0, INT_MAX]
    pa = lib()
    err = _err()
    pa.pa_check_slots(up_int(case.slot_mapping), nb, bs, err)
    torch.cuda.synchronize()
    assert [int(x) for x in err.cpu()] == [0, 0, INT_MAX]
