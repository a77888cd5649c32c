"""Pins for the oracle's block management with a prefix cache (CPU only).

The rules are checked against the FNV-1a published test vectors, the
datawhalechina page's worked allocation example, hand-worked sharing /
isolation / eviction sequences, and invariants counted by brute force over
random request streams.
"""

import json
import os
from collections import Counter

import numpy as np
import pytest

from oracle.blocks import OutOfBlocks, PrefixBlockManager, block_key, fnv1a64


def test_fnv1a64_published_vectors():
    # test vectors of the Fowler-Noll-Vo reference suite (FNV-1a, 64-bit)
    assert fnv1a64(b"") == 0xCBF29CE484222325
    assert fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert fnv1a64(b"foobar") == 0x85944171F73967E8


def test_block_key_is_fnv_over_little_endian_fields():
    want = fnv1a64(bytes([7, 0, 0, 0, 0, 0, 0, 0]) + bytes([2, 0, 0, 0, 0, 0, 0, 0])
                   + bytes([1, 0, 0, 0, 0xFF, 0xFF, 0xFF, 0xFF]))
    assert block_key(7, 2, [1, -1]) == want


def test_datawhale_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "datawhale_kv_cache_manager_example.json")))
    m = PrefixBlockManager(g["num_blocks"], g["block_size"])
    table = []
    for step in g["steps"]:
        if step["op"] == "prefill":
            table, hits = m.allocate_prompt(0, list(range(100, 100 + step["seq_len"])))
            assert hits == 0
        else:
            m.append(table, step["seq_len"])
        if "table_len" in step:
            assert len(table) == step["table_len"]
        if "free_blocks" in step:
            assert m.num_free() == step["free_blocks"]


def test_shared_prefix_shares_full_blocks_only():
    m = PrefixBlockManager(16, 4)
    sys_prompt = [11, 12, 13, 14, 15, 16, 17, 18]            # two full blocks
    a, ha = m.allocate_prompt(5, sys_prompt + [1, 2, 3])      # 3 blocks, last partial
    b, hb = m.allocate_prompt(5, sys_prompt + [9])            # hits the two prefix blocks
    assert (a, ha) == ([0, 1, 2], 0)
    assert (b, hb) == ([0, 1, 3], 2)
    assert [m.ref[x] for x in range(4)] == [2, 2, 1, 1]
    assert m.num_cached() == 2                                 # partial blocks are not cached
    # a prompt equal to A's: its partial block is fresh again
    c, hc = m.allocate_prompt(5, sys_prompt + [1, 2, 3])
    assert (c, hc) == ([0, 1, 4], 2)


def test_namespaces_are_isolated():
    m = PrefixBlockManager(8, 2)
    a, _ = m.allocate_prompt(1, [5, 6, 7, 8])
    b, hb = m.allocate_prompt(2, [5, 6, 7, 8])
    assert hb == 0 and set(a).isdisjoint(b)
    assert m.num_cached() == 4


def test_chain_breaks_at_the_first_difference():
    m = PrefixBlockManager(8, 2)
    m.allocate_prompt(0, [1, 2, 3, 4, 5, 6])
    t, h = m.allocate_prompt(0, [1, 2, 9, 9, 5, 6])
    # block 2 has the same tokens as before but a different parent
    assert h == 1 and t == [0, 3, 4]


def test_released_prefix_stays_cached_then_is_evicted_lru_tail_first():
    m = PrefixBlockManager(4, 2)
    a, _ = m.allocate_prompt(0, [1, 2, 3, 4, 5, 6])    # blocks 0, 1, 2 cached
    m.release(a)                                      # tail first onto the LRU: 2, 1, 0
    assert m.num_free() == 1 and m.num_evictable() == 3 and m.num_cached() == 3
    b, hb = m.allocate_prompt(0, [1, 2, 3, 4])         # hits 0, 1 without taking a block
    assert (b, hb) == ([0, 1], 2) and m.num_free() == 1 and m.num_evictable() == 1
    c, hc = m.allocate_prompt(0, [7, 7, 8, 8])         # free block 3, then evicts block 2
    assert (c, hc) == ([3, 2], 0)
    assert m.num_evictable() == 0
    with pytest.raises(OutOfBlocks):
        m.allocate_prompt(0, [9])
    # the failed call changed nothing
    assert m.num_free() == 0 and sorted(m.ref) == [1, 1, 1, 1]
    # block 2 now holds [8, 8] (cached); [5, 6] is gone
    m.release(b)
    m.release(c)                                      # LRU: 1, 0, then c's tail first: 2, 3
    assert m.num_evictable() == 4 and m.num_free() == 0
    d, hd = m.allocate_prompt(0, [1, 2, 3, 4, 5, 6])   # hits 0, 1; [5, 6] evicts block 2
    assert (d, hd) == ([0, 1, 2], 2)
    # [7, 7] still hits block 3, but [8, 8] needs a block and none is left
    with pytest.raises(OutOfBlocks):
        m.allocate_prompt(0, [7, 7, 8, 8])
    assert m.num_evictable() == 1 and m.ref[3] == 0


def test_blocks_filled_by_decode_serve_the_next_turn():
    # a dialogue: turn 1's prompt, then its reply generated token by token;
    # turn 2's prompt repeats both and adds the new question
    m = PrefixBlockManager(16, 4)
    p1 = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10]                    # 2 full blocks + 2 tokens
    t1, h1 = m.allocate_prompt(3, p1)
    assert (t1, h1) == ([0, 1, 2], 0) and m.num_cached() == 2
    reply = [11, 12, 13, 14, 15, 16]
    m.append(t1, len(p1) + len(reply))                     # 16 tokens: blocks 2 and 3 full
    assert t1 == [0, 1, 2, 3]
    assert m.register_blocks(3, p1 + reply, t1) == 2       # blocks 2 and 3 join the cache
    assert m.register_blocks(3, p1 + reply, t1) == 0       # idempotent
    t2, h2 = m.allocate_prompt(3, p1 + reply + [20, 21])
    assert h2 == 4 and t2[:4] == t1 and t2[4] == 4
    # another namespace still shares nothing
    _, h3 = m.allocate_prompt(4, p1 + reply)
    assert h3 == 0


def test_copy_on_write_and_fork():
    m = PrefixBlockManager(6, 4)
    a, _ = m.allocate_prompt(0, [1, 2, 3, 4, 5])
    f = m.fork(a)
    assert [m.ref[b] for b in a] == [2, 2]
    pair = m.copy_on_write(f, 1)
    assert pair == (1, 2) and f == [0, 2] and m.ref[1] == 1 and m.ref[2] == 1
    assert m.copy_on_write(f, 1) is None


def _check_invariants(m, live):
    uses = Counter(b for t in live for b in t)
    for b in range(m.num_blocks):
        assert m.ref[b] == uses.get(b, 0)
    free, lru = set(m.free), set(m.lru)
    assert len(free) == len(m.free) and len(lru) == len(m.lru)
    assert not (free & lru) and not (free & set(uses)) and not (lru & set(uses))
    assert lru == {b for b in m.entry if m.ref[b] == 0}
    assert len(free) + len(lru) + len(uses) == m.num_blocks
    assert {m.cache[k] for k in m.cache} == set(m.entry)


def test_random_streams_keep_the_invariants():
    rng = np.random.default_rng(7)
    for trial in range(20):
        nb, bs = int(rng.integers(8, 40)), int(rng.integers(1, 6))
        m = PrefixBlockManager(nb, bs, order=rng.permutation(nb))
        prefixes = [list(rng.integers(0, 5, size=int(rng.integers(0, 3 * bs)))) for _ in range(3)]
        live = []
        for _ in range(200):
            op = rng.integers(0, 5)
            before = (list(m.free), list(m.ref), list(m.lru), dict(m.cache), [list(t) for t in live])
            try:
                if op == 0 or not live:
                    p = prefixes[int(rng.integers(0, 3))] + list(rng.integers(0, 5, int(rng.integers(0, 2 * bs + 1))))
                    t, h = m.allocate_prompt(int(rng.integers(0, 2)), p)
                    assert len(t) == -(-len(p) // bs) and 0 <= h <= len(p) // bs
                    live.append(t)
                elif op == 1:
                    t = live[int(rng.integers(0, len(live)))]
                    m.append(t, len(t) * bs + int(rng.integers(0, 2 * bs)))
                elif op == 2:
                    live.append(m.fork(live[int(rng.integers(0, len(live)))]))
                elif op == 3:
                    t = live[int(rng.integers(0, len(live)))]
                    if t:
                        m.copy_on_write(t, int(rng.integers(0, len(t))))
                else:
                    m.release(live.pop(int(rng.integers(0, len(live)))))
            except OutOfBlocks:
                # a failed call changes nothing
                assert before == (m.free, m.ref, m.lru, m.cache, live)
            _check_invariants(m, live)
