"""Pins for oracle.paging: block-table resolution, gather and slot accounting.

Every expected value is either printed on the pages (tests/golden/*.json,
each with its citation), a closed form, or an independent construction
(numpy's row-major reshape) rather than a retyping of the oracle's formula.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import paging

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_ten_token_example_resolution():
    g = golden("ten_token_example.json")
    table, B = g["table"], g["block_size"]
    for lo, hi, phys in g["position_ranges"]:
        for t in range(lo, hi + 1):
            assert paging.resolve(table, B, t)[0] == phys, t
    p, o = paging.resolve(table, B, 6)
    assert (6 // B, p, o) == (g["token_6"]["logical"], g["token_6"]["physical"],
                              g["token_6"]["offset"])
    assert paging.blocks_needed(g["length"], B) == g["blocks_needed"]
    assert paging.slots_allocated(g["length"], B) == g["slots_allocated"]
    assert paging.wasted_slots(g["length"], B) == g["wasted_slots"]


def test_ten_token_valid_slot_mask():
    g = golden("ten_token_example.json")
    mask = paging.valid_slot_mask(np.array([g["table"]]), [g["length"]], 16, g["block_size"])
    expected = np.zeros((16, 4), dtype=bool)
    for lo, hi, phys in g["position_ranges"]:
        expected[phys, : hi - lo + 1] = True
    assert (mask == expected).all()
    assert mask.sum() == g["length"]


@pytest.mark.parametrize("B", [4, 8, 16, 32])
def test_waste_closed_form(B):
    # Waste lies in [0, B-1] for every length, and averages (B-1)/2 over any
    # whole period of lengths ([pofe] "The memory accounting").
    n = np.arange(1, 100_001)
    waste = np.array([paging.wasted_slots(int(x), B) for x in n[:5000]])
    assert waste.min() == 0 and waste.max() == B - 1
    period = np.array([paging.wasted_slots(int(x), B) for x in range(1, B + 1)])
    assert period.mean() == (B - 1) / 2
    # the big range, vectorised independently: ceil via -(-n // B)
    assert (((-(-n // B)) * B - n) <= B - 1).all()


def test_worked_example_llama3_8b():
    g = golden("worked_example_llama3_8b.json")
    B, lens = g["block_size"], g["lengths"]
    shape = g["kv_shape"]
    bpt = paging.kv_bytes_per_token(shape["layers"], shape["kv_heads"], shape["head_dim"],
                                    shape["dtype_bytes"])
    assert bpt == g["bytes_per_token"]
    blocks = [paging.blocks_needed(n, B) for n in lens]
    assert blocks == g["paged"]["blocks"]
    assert sum(blocks) == g["paged"]["total_blocks"]
    slots = sum(paging.slots_allocated(n, B) for n in lens)
    assert slots == g["paged"]["slots"]
    assert round(slots * bpt / 1e6) == g["paged"]["megabytes"]
    waste = [paging.wasted_slots(n, B) for n in lens]
    assert waste == g["paged"]["waste"] and sum(waste) == g["paged"]["total_waste"]
    assert round(100 * sum(lens) / slots, 1) == g["paged"]["utilisation_pct"]
    res = g["reservation"]
    assert len(lens) * g["max_len"] == res["slots"]
    assert round(res["slots"] * bpt / 1e9, 2) == res["gigabytes"]
    assert sum(lens) == res["real_tokens"]
    assert round(100 * sum(paging.eta_naive(n, g["max_len"]) for n in lens) / len(lens), 1) \
        == res["utilisation_pct"]
    assert math.floor(60e9 / (g["max_len"] * bpt)) == g["capacity_60GB_reservation"]


def test_utilisation_bounds():
    g = golden("utilisation_and_sizes.json")
    a = g["pofe_memory_accounting"]
    up = paging.utilisation_paged_worst(a["mean_len"], a["block_size"])
    ur = paging.utilisation_reserve(a["mean_len"], a["s_max"])
    assert math.floor(1000 * up) / 10 == a["u_paged_at_least_pct"]
    assert round(100 * ur, 1) == a["u_reserve_pct"]
    assert round(up / ur) == a["batch_gain_about"]
    # closed forms of the reservation rule: a reservation filled to S_max is
    # fully used, one filled to half is half used, and the batch figure is
    # the mean of the per-request utilisations
    assert paging.utilisation_reserve(4096, 4096) == 1.0
    assert paging.utilisation_reserve(2048, 4096) == 0.5
    lens = [37, 1203, 450]
    assert math.isclose(paging.utilisation_reserve(sum(lens) / 3, 4096),
                        sum(paging.eta_naive(n, 4096) for n in lens) / 3, rel_tol=1e-15)
    e = g["arch_eta_bound"]
    assert round(100 * paging.eta_paged_lower_bound(e["s"], e["block_size"]), 2) \
        == e["eta_lower_bound_pct"]
    # exact utilisation is never below the bound (brute force over lengths)
    for B in (8, 16, 32):
        for s in range(1, 3000):
            assert paging.eta_paged(s, B) >= paging.eta_paged_lower_bound(s, B) - 1e-15
    assert paging.eta_paged(2048, 16) == 1.0


def test_kv_bytes_per_token_pages():
    g = golden("utilisation_and_sizes.json")
    a = g["arch_70b_kv"]
    bpt = paging.kv_bytes_per_token(a["layers"], a["kv_heads"], a["head_dim"], a["dtype_bytes"])
    assert bpt == a["per_token_about_kb"] * 1024
    assert bpt * a["tokens"] == 2.5 * 2**30
    assert round(a["per_token_about_kb"] * 1000 * a["tokens"] / 1e9, 2) == a["total_about_gb"]
    o = g["pofe_opt13b_kv"]
    s = o["kv_shape"]
    bpt = paging.kv_bytes_per_token(s["layers"], s["kv_heads"], s["head_dim"], s["dtype_bytes"])
    assert bpt == o["per_token_about_kb"] * 1024
    assert round(bpt * o["reservation_tokens"] / 2**30, 1) == o["reservation_about_gb"]


def test_element_offset_matches_row_major_layout():
    rng = np.random.default_rng(0)
    N, B, H, D = 5, 4, 3, 8
    pool = rng.standard_normal((N, B, H, D))
    flat = pool.reshape(-1)
    for _ in range(200):
        p, o, h, d = (int(rng.integers(0, x)) for x in (N, B, H, D))
        assert flat[paging.element_offset(p, o, h, d, B, H, D)] == pool[p, o, h, d]


@pytest.mark.parametrize("B", [1, 4, 8, 16])
def test_gather_matches_reshape_construction(B):
    # Build the pool the other way round: pad the contiguous history to whole
    # blocks, reshape row-major to [nb, B, H, D] and store block j at table[j].
    rng = np.random.default_rng(B)
    H, D, N = 2, 4, 40
    for L in (1, B, B + 1, 3 * B - 1, 37):
        hist = rng.standard_normal((L, H, D))
        nb = -(-L // B)
        table = rng.permutation(N)[:nb]
        pool = np.full((N, B, H, D), np.nan)
        padded = np.full((nb * B, H, D), np.nan)
        padded[:L] = hist
        pool[table] = padded.reshape(nb, B, H, D)
        got = paging.gather_contiguous(pool, table, L, B)
        assert np.array_equal(got, hist)


def test_gather_rejects_out_of_range_ids():
    pool = np.zeros((4, 2, 1, 1))
    with pytest.raises(IndexError):
        paging.gather_contiguous(pool, [0, 9], 3, 2)
    with pytest.raises(IndexError):
        paging.gather_contiguous(pool, [0, -1], 3, 2)
