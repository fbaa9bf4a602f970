"""Pins for oracle.block_manager and oracle.allocator_toy.

The lesson's allocator toy prints what a paged allocator holds for four
requests; the [arch] driver prints the refcount of a shared prefix block;
the copy-on-write rule of [pofe] fixes which sequence copies.  Random
operation sequences check the allocator invariants of [note].
"""

import json
import os

import numpy as np
import pytest

from oracle import allocator_toy
from oracle.block_manager import NoFreeBlock, OracleBlockPool, OracleSequence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_lesson_toy_contiguous_and_paged():
    g = golden("lesson_allocator_toy.json")
    reqs = {k: tuple(v) for k, v in g["requests"].items()}
    pool_slots = g["pool_blocks"] * g["block_size"]
    c = allocator_toy.contiguous_reservation(reqs, pool_slots, g["max_len"])
    for name, (reserved, used, wasted) in g["contiguous"]["per_request"].items():
        r = c["per_request"][name]
        assert (r["reserved"], r["used"], r["wasted"]) == (reserved, used, wasted)
    assert c["served"] == g["contiguous"]["served"]
    assert c["reserved"] == g["contiguous"]["reserved"]
    assert c["needed"] == g["contiguous"]["needed"]
    assert round(c["waste_pct"]) == g["contiguous"]["waste_pct_rounded"]

    p = allocator_toy.paged_on_demand(reqs, g["pool_blocks"], g["block_size"])
    for name, (blocks, tokens, wasted) in g["paged"]["per_request"].items():
        r = p["per_request"][name]
        assert (r["blocks"], r["tokens"], r["wasted"]) == (blocks, tokens, wasted)
        assert not r["preempted"]
    assert p["served"] == g["paged"]["served"]
    assert p["held"] == g["paged"]["held"]
    assert p["needed"] == g["paged"]["needed"]
    assert round(p["waste_pct"]) == g["paged"]["waste_pct_rounded"]
    assert p["free_blocks"] == g["paged"]["free_blocks"]

    # The reservation rule at other pool sizes: a pool one slot short of
    # four reservations serves three and shows the fourth the slots left; a
    # bigger pool serves all four and wastes the same share of what they
    # reserved (the unreserved slots are free, not wasted).
    short = allocator_toy.contiguous_reservation(reqs, 4 * g["max_len"] - 1, g["max_len"])
    assert short["served"] == 3 and short["reserved"] == 3 * g["max_len"]
    assert short["per_request"]["r4"] == {"rejected": True, "free_slots": g["max_len"] - 1}
    assert short["needed"] == 52 + 20 + 135
    big = allocator_toy.contiguous_reservation(reqs, 10 * g["max_len"], g["max_len"])
    assert big["served"] == 4 and big["reserved"] == 4 * g["max_len"]
    assert round(big["waste_pct"]) == g["contiguous"]["waste_pct_rounded"]

    s = allocator_toy.shared_prompt(g["sharing"]["sys_tokens"], g["sharing"]["users"],
                                    g["block_size"])
    for key in ("copied_blocks", "shared_blocks", "refcount", "saved_slots"):
        assert s[key] == g["sharing"][key], key
    assert s["all_free_after"]


def test_arch_driver_shared_prefix_refcount():
    g = golden("arch_driver_prefix.json")
    pool = OracleBlockPool(g["num_blocks"], g["block_size"])
    r1 = OracleSequence(pool)
    r1.reserve_prompt(g["prefix_tokens"] + g["suffix_tokens"][0])
    r2 = OracleSequence(pool)
    r2.adopt_prefix(r1, g["prefix_tokens"] // g["block_size"])
    r2.extend_prompt(g["suffix_tokens"][1])
    assert r1.table[0] == r2.table[0] and r1.table[1] != r2.table[1]
    assert pool.ref[r1.table[0]] == g["shared_prefix_refcount"]
    assert len(r1.table) == len(r2.table) == 2


def test_adopt_and_extend_count_exactly():
    # Adopting k full blocks adds one reference to each of those k blocks and
    # to no other; extending to a block-aligned length takes exactly the
    # blocks that length needs (ceil(len / B)); freeing every sequence gives
    # every block back ([note] "Useful allocator invariants").
    pool = OracleBlockPool(16, 4)
    src = OracleSequence(pool)
    src.reserve_prompt(14)                       # 4 blocks, the last one half full
    dst = OracleSequence(pool)
    dst.adopt_prefix(src, 2)
    assert [pool.ref[i] for i in src.table] == [2, 2, 1, 1]
    assert dst.table == src.table[:2] and dst.len == 8
    dst.extend_prompt(8)                         # 16 tokens: exactly 4 blocks
    assert len(dst.table) == 4 and dst.len == 16
    assert pool.num_free() == 16 - 4 - 2
    dst.extend_prompt(1)                         # 17 tokens: a fifth block
    assert len(dst.table) == 5
    for seq in (src, dst):
        seq.free_all()
    assert pool.num_free() == 16 and all(r == 0 for r in pool.ref)


def test_copy_on_write_first_appender_copies():
    # A 6-token sequence with B = 4 holds a full block and a half block.
    # After fork both blocks have count 2.  The first sequence to append
    # writes into the shared half block, so it copies it; the second then
    # owns the old block alone and writes in place ([pofe] "Sharing and
    # copy-on-write": at most one block per sample is duplicated).
    pool = OracleBlockPool(8, 4)
    parent = OracleSequence(pool)
    parent.reserve_prompt(6)
    full, half = parent.table
    child = parent.fork()
    assert pool.ref[full] == pool.ref[half] == 2
    blk, slot, cow = parent.append_slot()
    assert cow is not None and cow[0] == half and blk == cow[1] and slot == 2
    assert parent.table == [full, cow[1]]
    assert pool.ref[half] == 1 and pool.ref[cow[1]] == 1 and pool.ref[full] == 2
    blk2, slot2, cow2 = child.append_slot()
    assert cow2 is None and blk2 == half and slot2 == 2
    assert pool.num_free() == 8 - 3
    # A block boundary allocates instead of copying.
    child.append_slot()                     # len 7 -> 8, slot 3 of `half`
    blk3, slot3, cow3 = child.append_slot()  # len 8: new block
    assert cow3 is None and slot3 == 0 and blk3 not in (full, half, cow[1])
    parent.free_all()
    child.free_all()
    assert pool.num_free() == 8 and all(r == 0 for r in pool.ref)


def test_lifo_free_list_order():
    pool = OracleBlockPool(4, 2)
    assert [pool.alloc() for _ in range(2)] == [3, 2]
    pool.release(3)
    assert pool.alloc() == 3


def test_exhaustion_leaves_state_unchanged():
    pool = OracleBlockPool(3, 2)
    a = OracleSequence(pool)
    a.reserve_prompt(3)                 # 2 blocks
    b = a.fork()
    c = OracleSequence(pool)
    c.reserve_prompt(2)                 # last free block
    snapshot = (list(pool.free), list(pool.ref), list(a.table), a.len, list(b.table), b.len)
    with pytest.raises(NoFreeBlock):
        a.append_slot()                 # CoW needs a block
    with pytest.raises(NoFreeBlock):
        c.append_slot()                 # boundary needs a block
    assert snapshot == (list(pool.free), list(pool.ref), list(a.table), a.len,
                        list(b.table), b.len)
    with pytest.raises(NoFreeBlock):
        OracleSequence(pool).reserve_prompt(1)


def test_release_of_free_block_is_an_error():
    pool = OracleBlockPool(2, 2)
    with pytest.raises(ValueError):
        pool.release(0)
    with pytest.raises(ValueError):
        pool.share(1)


def check_invariants(pool, seqs):
    # [note] "Useful allocator invariants": each live logical block refers to
    # allocated storage, counts equal the number of tables holding the block,
    # and free blocks are exactly the ones nobody references.
    counts = np.zeros(pool.num_blocks, dtype=int)
    for s in seqs:
        assert len(s.table) == -(-s.len // pool.block_size)
        for i in s.table:
            counts[i] += 1
    assert list(counts) == pool.ref
    assert sorted(pool.free) == [i for i in range(pool.num_blocks) if counts[i] == 0]
    assert len(set(pool.free)) == len(pool.free)


@pytest.mark.parametrize("seed", range(6))
def test_random_operations_keep_invariants(seed):
    rng = np.random.default_rng(seed)
    pool = OracleBlockPool(40, int(rng.choice([1, 2, 4, 8])))
    seqs = []
    for _ in range(400):
        op = rng.integers(0, 5)
        try:
            if op == 0 or not seqs:
                s = OracleSequence(pool)
                s.reserve_prompt(int(rng.integers(0, 20)))
                seqs.append(s)
            elif op == 1:
                seqs.append(seqs[int(rng.integers(len(seqs)))].fork())
            elif op in (2, 3):
                seqs[int(rng.integers(len(seqs)))].append_slot()
            else:
                seqs.pop(int(rng.integers(len(seqs)))).free_all()
        except NoFreeBlock:
            pass
        check_invariants(pool, seqs)
    for s in seqs:
        s.free_all()
    assert pool.num_free() == pool.num_blocks
