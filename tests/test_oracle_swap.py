"""Pins for the swap oracle: block copies to host and back, and preemption
by swapping in the block manager.

The copies are pinned to the [note] "Map a ten-token sequence into pages"
example (swapping out a sequence's blocks in table order gives its
contiguous history) and to copy_blocks (out then in at new ids is a block
copy); the manager to the free-list / reference-count invariants and the
all-or-none rule of [pofe] "When memory runs out".
"""

import numpy as np
import pytest

from oracle import cache_ops, paging
from oracle.block_manager import NoFreeBlock, OracleBlockPool, OracleSequence


def test_swap_out_of_the_ten_token_sequence_is_its_history():
    N, B, H, D = 16, 4, 2, 3
    rng = np.random.default_rng(0)
    kp = rng.standard_normal((N, B, H, D))
    vp = rng.standard_normal((N, B, H, D))
    hk, hv = cache_ops.swap_out(kp, vp, [7, 2, 11])
    assert hk.shape == (3, B, H, D)
    np.testing.assert_array_equal(hk.reshape(12, H, D)[:10],
                                  paging.gather_contiguous(kp, [7, 2, 11], 10, B))
    np.testing.assert_array_equal(hv.reshape(12, H, D)[:10],
                                  paging.gather_contiguous(vp, [7, 2, 11], 10, B))


def test_out_then_in_at_new_ids_is_a_block_copy():
    rng = np.random.default_rng(1)
    kp = rng.standard_normal((20, 8, 1, 4))
    vp = rng.standard_normal((20, 8, 1, 4))
    src, dst = [3, 9, 0], [12, 5, 17]
    hk, hv = cache_ops.swap_out(kp, vp, src)
    k2, v2 = cache_ops.swap_in(kp, vp, dst, hk, hv)
    k3, v3 = cache_ops.copy_blocks(kp, vp, src, dst)
    assert np.array_equal(k2, k3) and np.array_equal(v2, v3)


def test_swap_in_rejects_duplicate_or_bad_ids():
    kp = np.zeros((4, 2, 1, 2))
    h = np.ones((2, 2, 1, 2))
    with pytest.raises(ValueError):
        cache_ops.swap_in(kp, kp, [1, 1], h, h)
    with pytest.raises(IndexError):
        cache_ops.swap_in(kp, kp, [1, 4], h, h)
    with pytest.raises(IndexError):
        cache_ops.swap_out(kp, kp, [-1])


def test_manager_swap_releases_and_restores():
    pool = OracleBlockPool(10, 4)
    a = OracleSequence(pool)
    a.reserve_prompt(9)                    # 3 blocks
    b = a.fork()                           # shares all 3
    out = a.swap_out()
    assert out == b.table and a.len == 9 and a.table == [] and a.swapped
    assert pool.num_free() == 7            # shared blocks stay with b
    assert all(pool.ref[i] == 1 for i in b.table)
    with pytest.raises(ValueError):
        a.append_slot()
    with pytest.raises(ValueError):
        a.fork()
    new = a.swap_in()
    assert len(new) == 3 and not set(new) & set(b.table)
    assert pool.num_free() == 4 and not a.swapped
    blk, slot, cow = a.append_slot()       # private again: no copy-on-write
    assert (blk, slot, cow) == (new[-1], 1, None)


def test_swap_in_is_all_or_none():
    pool = OracleBlockPool(4, 2)
    a = OracleSequence(pool)
    a.reserve_prompt(5)                    # 3 blocks
    a.swap_out()
    c = OracleSequence(pool)
    c.reserve_prompt(4)                    # 2 of the 4 blocks
    free_before = list(pool.free)
    with pytest.raises(NoFreeBlock):
        a.swap_in()
    assert a.swapped and a.table == [] and pool.free == free_before
    c.free_all()
    assert len(a.swap_in()) == 3


def test_random_preemption_keeps_the_invariants():
    rng = np.random.default_rng(5)
    pool = OracleBlockPool(24, 4)
    seqs = []
    for _ in range(400):
        op = rng.integers(0, 5)
        try:
            if op == 0 or not seqs:
                s = OracleSequence(pool)
                s.reserve_prompt(int(rng.integers(1, 10)))
                seqs.append(s)
            else:
                s = seqs[int(rng.integers(0, len(seqs)))]
                if op == 1 and not s.swapped:
                    s.append_slot()
                elif op == 2 and not s.swapped:
                    seqs.append(s.fork())
                elif op == 3:
                    if s.swapped:
                        s.swap_in()
                    else:
                        s.swap_out()
                elif op == 4:
                    s.free_all()
                    seqs.remove(s)
        except NoFreeBlock:
            pass
        held = [i for s in seqs if not s.swapped for i in s.table]
        assert sum(pool.ref) == len(held)
        assert pool.num_free() + sum(1 for r in pool.ref if r > 0) == pool.num_blocks
        for s in seqs:
            if not s.swapped:
                assert len(s.table) == -(-s.len // 4)
            else:
                assert s.table == []
