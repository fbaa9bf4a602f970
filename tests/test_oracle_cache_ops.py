"""Pins for oracle.cache_ops: append and whole-block copy are byte moves."""

import json
import os

import numpy as np
import pytest

from oracle import cache_ops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_append_into_ten_token_table():
    # Ten-token example: the token at position 9 is the second slot of the
    # third logical block, physical block 11 (positions 8-9 live in 11).
    with open(os.path.join(GOLDEN, "ten_token_example.json")) as f:
        g = json.load(f)
    B = g["block_size"]
    rng = np.random.default_rng(0)
    kp = rng.standard_normal((16, B, 2, 3))
    vp = rng.standard_normal((16, B, 2, 3))
    k_new = rng.standard_normal((1, 2, 3))
    v_new = rng.standard_normal((1, 2, 3))
    k2, v2 = cache_ops.append_token(kp, vp, k_new, v_new, np.array([g["table"]]), [9], B)
    last_block = g["position_ranges"][-1][2]
    expected_k = kp.copy()
    expected_k[last_block, 9 - g["position_ranges"][-1][0]] = k_new[0]
    expected_v = vp.copy()
    expected_v[last_block, 1] = v_new[0]
    assert np.array_equal(k2, expected_k) and np.array_equal(v2, expected_v)
    # The original pools are untouched (the oracle works on copies).
    assert not np.array_equal(kp, k2)


def test_append_first_token_of_new_block_and_padding_rows():
    rng = np.random.default_rng(1)
    B = 4
    kp = rng.standard_normal((8, B, 1, 2)).astype(np.float32)
    vp = rng.standard_normal((8, B, 1, 2)).astype(np.float32)
    k_new = rng.standard_normal((3, 1, 2)).astype(np.float32)
    v_new = rng.standard_normal((3, 1, 2)).astype(np.float32)
    # seq 0 has 12 tokens in [7, 2, 11]: its 13th token opens block 5;
    # seq 1 is a padding row (negative length); seq 2 writes slot 0 of block 3.
    tables = np.array([[7, 2, 11 % 8, 5], [0, -1, -1, -1], [3, -1, -1, -1]])
    k2, v2 = cache_ops.append_token(kp, vp, k_new, v_new, tables, [12, -1, 0], B)
    changed = np.argwhere((k2 != kp).any(axis=(2, 3)))
    assert sorted(map(tuple, changed)) == [(3, 0), (5, 0)]
    assert np.array_equal(k2[5, 0], k_new[0]) and np.array_equal(v2[3, 0], v_new[2])


def test_copy_blocks_whole_block_and_rejects_overlap():
    rng = np.random.default_rng(2)
    kp = rng.standard_normal((6, 4, 2, 3))
    vp = rng.standard_normal((6, 4, 2, 3))
    k2, v2 = cache_ops.copy_blocks(kp, vp, [1, 4], [0, 5])
    assert np.array_equal(k2[0], kp[1]) and np.array_equal(v2[5], vp[4])
    untouched = [1, 2, 3, 4]
    assert np.array_equal(k2[untouched], kp[untouched])
    with pytest.raises(ValueError):
        cache_ops.copy_blocks(kp, vp, [1, 2], [2, 3])
    with pytest.raises(ValueError):
        cache_ops.copy_blocks(kp, vp, [1, 2], [3, 3])
