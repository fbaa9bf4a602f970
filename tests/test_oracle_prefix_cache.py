"""Pins for the prefix-cache oracle.

[arch] "Production PyTorch Implementation" Step 3: two prompts with one
16-token system prefix share its block, count 2 (tests/golden/
arch_driver_prefix.json).  [lesson] "Sharing, and the reference counting it
needs": blocks are shared only when every token id of the prefix is equal.
[claims] "Paged Attention": a hit needs an unbroken matching prefix.  Plus
the free-list / count invariants under random traffic with eviction.
"""

import json
import os

import numpy as np
import pytest

from oracle.block_manager import NoFreeBlock, OracleSequence
from oracle.prefix_cache import OraclePrefixPool, admit_prompt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_arch_driver_system_prefix_shares_one_block():
    fx = json.load(open(os.path.join(GOLDEN, "arch_driver_prefix.json")))
    pool = OraclePrefixPool(fx["num_blocks"], fx["block_size"])
    system = [101, 2054, 2003, 1037] * 4
    a, b = OracleSequence(pool), OracleSequence(pool)
    assert admit_prompt(a, system + [1001, 1002, 1003]) == 0
    assert admit_prompt(b, system + [2001, 2002, 2003]) == fx["prefix_tokens"]
    assert a.table[0] == b.table[0] and a.table[1] != b.table[1]
    assert pool.ref[a.table[0]] == fx["shared_prefix_refcount"]


def test_one_differing_token_ends_the_chain():
    pool = OraclePrefixPool(32, 4)
    base = list(range(100, 116))                 # 4 full blocks
    a = OracleSequence(pool)
    admit_prompt(a, base)
    other = base.copy()
    other[5] = 999                               # block 1 differs
    b = OracleSequence(pool)
    assert admit_prompt(b, other) == 4           # only block 0
    assert b.table[0] == a.table[0]
    assert not set(b.table[1:]) & set(a.table)   # blocks 2, 3 match but are not reached


def test_partial_last_block_is_never_shared():
    pool = OraclePrefixPool(16, 4)
    a, b = OracleSequence(pool), OracleSequence(pool)
    admit_prompt(a, list(range(6)))
    assert admit_prompt(b, list(range(6))) == 4
    assert a.table[0] == b.table[0] and a.table[1] != b.table[1]


def test_freed_blocks_stay_cached_until_evicted():
    pool = OraclePrefixPool(4, 2)
    a = OracleSequence(pool)
    admit_prompt(a, [1, 2, 3, 4, 5])             # 3 blocks, 2 full ones cached
    a.free_all()
    assert pool.num_free() == 4 and pool.num_cached() == 2
    b = OracleSequence(pool)
    assert admit_prompt(b, [1, 2, 3, 4]) == 4    # both revived
    assert all(pool.ref[x] == 1 for x in b.table) and pool.lru == []
    b.free_all()
    # Pressure: 4 new uncached blocks evict both cached ones, oldest first.
    c = OracleSequence(pool)
    admit_prompt(c, [9] * 8)
    assert pool.num_cached() == 4 and pool.num_free() == 0
    d = OracleSequence(pool)
    with pytest.raises(NoFreeBlock):
        admit_prompt(d, [1, 2, 3, 4])


def test_eviction_takes_the_least_recently_released_block():
    # LRU eviction ([lesson] "Sharing, and the reference counting it needs"
    # names it): of two cached blocks whose counts fell to 0, an allocation
    # under pressure evicts the one released first; the other stays hittable.
    pool = OraclePrefixPool(3, 2)
    a, b = OracleSequence(pool), OracleSequence(pool)
    admit_prompt(a, [1, 2])
    admit_prompt(b, [3, 4])
    a.free_all()                                  # released first
    b.free_all()
    assert pool.num_cached() == 2 and len(pool.free) == 1
    c = OracleSequence(pool)
    admit_prompt(c, [7, 7, 8, 8])                 # needs 2 blocks: the free one + one eviction
    assert pool.num_cached() == 3                  # [3, 4] stayed, [7, 7] and [7, 7, 8, 8] added
    e = OracleSequence(pool)
    assert admit_prompt(e, [3, 4]) == 2            # [3, 4] still cached: a hit, revived
    d = OracleSequence(pool)
    with pytest.raises(NoFreeBlock):
        admit_prompt(d, [1, 2])                    # [1, 2] was evicted: no hit, no block left


def test_admission_is_all_or_none():
    pool = OraclePrefixPool(3, 2)
    a = OracleSequence(pool)
    admit_prompt(a, [1, 2])
    a.free_all()                                 # block cached, evictable
    b = OracleSequence(pool)
    before = (list(pool.free), list(pool.lru), dict(pool.block_of), list(pool.ref))
    with pytest.raises(NoFreeBlock):
        admit_prompt(b, [1, 2, 3, 4, 5, 6, 7])   # 1 hit + 3 new > 2 allocatable
    assert (list(pool.free), list(pool.lru), dict(pool.block_of), list(pool.ref)) == before


def test_random_traffic_keeps_the_invariants():
    rng = np.random.default_rng(3)
    pool = OraclePrefixPool(20, 4)
    prefixes = [list(rng.integers(0, 50, 12)) for _ in range(3)]
    live = []
    for _ in range(500):
        if live and rng.random() < 0.4:
            live.pop(int(rng.integers(len(live)))).free_all()
        else:
            p = prefixes[int(rng.integers(3))][: int(rng.integers(0, 13))]
            toks = p + list(rng.integers(0, 50, int(rng.integers(1, 9))))
            s = OracleSequence(pool)
            try:
                cached = admit_prompt(s, toks)
                live.append(s)
                # A hit means the cached blocks hold exactly those prefixes.
                for j in range(cached // 4):
                    assert pool.key_of[s.table[j]] == tuple(toks[: 4 * (j + 1)])
            except NoFreeBlock:
                pass
        held = [x for s in live for x in s.table]
        assert sum(pool.ref) == len(held)
        assert all(pool.ref[x] == held.count(x) for x in set(held))
        assert len(pool.free) + len(pool.lru) + len(set(held)) == pool.num_blocks
        assert set(pool.lru) == {x for x in pool.key_of if pool.ref[x] == 0}
