"""Pins for the chunked-prefill oracle and the multi-token append.

prefill_attention is checked against torch's scaled_dot_product_attention in
float64 on the CPU (a routine the oracle does not use) with an explicit mask
built from the reading "query at position p sees positions 0..p"; against
is_causal=True when the chunk is the whole history (the two mask alignments
coincide there); against the decode oracle when the chunk is one token; and
against closed forms.  append_tokens is checked against the ten-token
example of [note] "Map a ten-token sequence into pages" and against repeated
single-token appends.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention, cache_ops


def build_paged(hists, B, N, seed):
    """Store contiguous histories [L, H, D] in a pool by numpy reshape, block
    ids from a seeded permutation; returns pool, tables."""
    rng = np.random.default_rng(seed)
    H, D = hists[0].shape[1:]
    pool = np.full((N, B, H, D), np.nan)
    nbs = [-(-h.shape[0] // B) for h in hists]
    tables = np.full((len(hists), max(nbs)), -1, dtype=np.int64)
    perm = rng.permutation(N)
    pos = 0
    for s, h in enumerate(hists):
        ids = perm[pos:pos + nbs[s]]
        pos += nbs[s]
        padded = np.full((nbs[s] * B, H, D), np.nan)
        padded[: h.shape[0]] = h
        pool[ids] = padded.reshape(nbs[s], B, H, D)
        tables[s, : nbs[s]] = ids
    return pool, tables


def sdpa_chunk(q, k_hist, v_hist, mask=None, is_causal=False):
    """q [n, Hq, D], K/V [L, Hkv, D] -> [n, Hq, D] via torch SDPA (float64)."""
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))        # [Hq, n, D]
    kt = torch.from_numpy(np.ascontiguousarray(k_hist.transpose(1, 0, 2)))   # [Hkv, L, D]
    vt = torch.from_numpy(np.ascontiguousarray(v_hist.transpose(1, 0, 2)))
    m = None if mask is None else torch.from_numpy(mask)
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=is_causal,
                                         enable_gqa=True)
    return out.numpy().transpose(1, 0, 2)


def make_case(Hq, Hkv, D, B, lens, chunks, seed):
    rng = np.random.default_rng(seed)
    k_h = [rng.standard_normal((L, Hkv, D)) for L in lens]
    v_h = [rng.standard_normal((L, Hkv, D)) for L in lens]
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    q = rng.standard_normal((int(cu[-1]), Hq, D))
    N = sum(-(-L // B) for L in lens) + 5
    k_pool, tables = build_paged(k_h, B, N, seed + 1)
    v_pool, _ = build_paged(v_h, B, N, seed + 1)
    return q, k_h, v_h, k_pool, v_pool, tables, cu


@pytest.mark.parametrize("Hq,Hkv,D,B", [(2, 1, 16, 4), (8, 2, 32, 16), (6, 6, 8, 8),
                                        (16, 2, 64, 32)])
def test_prefill_equals_dense_sdpa_with_bottom_right_mask(Hq, Hkv, D, B):
    lens = [1, 7, 3 * B + 5, 40, 2 * B]
    chunks = [1, 7, 9, 1, 5]
    q, k_h, v_h, kp, vp, tables, cu = make_case(Hq, Hkv, D, B, lens, chunks, Hq + D + B)
    out = attention.prefill_attention(q, kp, vp, tables, lens, cu, B)
    for s, (L, n) in enumerate(zip(lens, chunks)):
        pos = L - n + np.arange(n)
        mask = np.arange(L)[None, :] <= pos[:, None]                          # [n, L]
        ref = sdpa_chunk(q[cu[s]:cu[s + 1]], k_h[s], v_h[s], mask=mask)
        np.testing.assert_allclose(out[cu[s]:cu[s + 1]], ref, rtol=1e-12, atol=1e-13)


def test_whole_history_chunk_is_ordinary_causal_attention():
    lens = [13, 32, 5]
    q, k_h, v_h, kp, vp, tables, cu = make_case(4, 2, 16, 8, lens, lens, 7)
    out = attention.prefill_attention(q, kp, vp, tables, lens, cu, 8)
    for s in range(len(lens)):
        ref = sdpa_chunk(q[cu[s]:cu[s + 1]], k_h[s], v_h[s], is_causal=True)
        np.testing.assert_allclose(out[cu[s]:cu[s + 1]], ref, rtol=1e-12, atol=1e-13)


def test_one_token_chunk_is_decode_attention():
    lens = [1, 9, 33, 17]
    q, k_h, v_h, kp, vp, tables, cu = make_case(8, 2, 16, 4, lens, [1, 1, 1, 1], 11)
    out = attention.prefill_attention(q, kp, vp, tables, lens, cu, 4)
    ref = attention.decode_attention(q, kp, vp, tables, lens, 4)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-14)


def test_closed_forms():
    # Position 0 sees only itself: output = v_0 exactly.  Equal keys: the
    # output of the query at position p is the mean of V over 0..p.
    B, D, L = 4, 8, 11
    rng = np.random.default_rng(3)
    k = np.tile(rng.standard_normal((1, 1, D)), (L, 1, 1))
    v = rng.standard_normal((L, 1, D))
    kp, tables = build_paged([k], B, 5, 9)
    vp, _ = build_paged([v], B, 5, 9)
    q = rng.standard_normal((L, 1, D))
    out = attention.prefill_attention(q, kp, vp, tables, [L], [0, L], B)
    assert np.array_equal(out[0, 0], v[0, 0])
    for p in range(L):
        np.testing.assert_allclose(out[p, 0], v[: p + 1, 0].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_relabelling_blocks_changes_nothing():
    lens = [21, 6]
    q, k_h, v_h, kp, vp, tables, cu = make_case(4, 1, 8, 4, lens, [5, 6], 13)
    out = attention.prefill_attention(q, kp, vp, tables, lens, cu, 4)
    kp2, t2 = build_paged(k_h, 4, kp.shape[0], 99)
    vp2, _ = build_paged(v_h, 4, kp.shape[0], 99)
    assert not np.array_equal(t2, tables)
    assert np.array_equal(attention.prefill_attention(q, kp2, vp2, t2, lens, cu, 4), out)


def test_planted_mask_mistakes_fail():
    # A top-left aligned mask (query j sees 0..j) and an exclusive one
    # (positions < p) both differ from the oracle when the chunk is shorter
    # than the history.
    L, n, B, D = 12, 4, 4, 8
    q, k_h, v_h, kp, vp, tables, cu = make_case(2, 1, D, B, [L], [n], 17)
    out = attention.prefill_attention(q, kp, vp, tables, [L], cu, B)
    top_left = sdpa_chunk(q, k_h[0], v_h[0], is_causal=True)
    assert np.abs(out - top_left).max() > 1e-3
    pos = L - n + np.arange(n)
    exclusive = sdpa_chunk(q, k_h[0], v_h[0], mask=np.arange(L)[None, :] < pos[:, None])
    assert np.abs(out - exclusive).max() > 1e-3


def test_prefill_rejects_chunks_longer_than_the_history():
    q, k_h, v_h, kp, vp, tables, cu = make_case(2, 1, 8, 4, [3], [3], 5)
    with pytest.raises(ValueError):
        attention.prefill_attention(q, kp, vp, tables, [2], cu, 4)


def test_append_tokens_ten_token_example():
    # [note] "Map a ten-token sequence into pages": B = 4, table [7, 2, 11],
    # positions 0-3 -> block 7, 4-7 -> block 2, 8-9 -> block 11.  Appending
    # three tokens at length 7 writes (2, 3), (11, 0), (11, 1) and nothing else.
    N, B, H, D = 16, 4, 1, 2
    kp = np.arange(N * B * H * D, dtype=np.float64).reshape(N, B, H, D)
    vp = -kp
    tables = np.array([[7, 2, 11, -1]])
    k_new = np.full((3, H, D), 0.5) + np.arange(3)[:, None, None]
    v_new = -k_new
    ko, vo = cache_ops.append_tokens(kp, vp, k_new, v_new, tables, [7], [0, 3], B)
    expect = kp.copy()
    expect[2, 3] = k_new[0]
    expect[11, 0] = k_new[1]
    expect[11, 1] = k_new[2]
    assert np.array_equal(ko, expect)
    assert np.array_equal(vo, -expect)


def test_append_tokens_equals_repeated_single_appends():
    rng = np.random.default_rng(21)
    N, B, H, D = 40, 4, 2, 4
    kp = rng.standard_normal((N, B, H, D))
    vp = rng.standard_normal((N, B, H, D))
    tables = rng.permutation(N)[:30].reshape(3, 10)
    lens_pre = [0, 5, 13]
    chunks = [6, 0, 9]
    cu = np.concatenate([[0], np.cumsum(chunks)])
    k_new = rng.standard_normal((cu[-1], H, D))
    v_new = rng.standard_normal((cu[-1], H, D))
    ko, vo = cache_ops.append_tokens(kp, vp, k_new, v_new, tables, lens_pre, cu, B)
    k2, v2 = kp, vp
    for j in range(max(chunks)):
        rows = [s for s in range(3) if j < chunks[s]]
        sub_lens = [lens_pre[s] + j if s in rows else -1 for s in range(3)]
        kn = np.zeros((3, H, D))
        vn = np.zeros((3, H, D))
        for s in rows:
            kn[s] = k_new[cu[s] + j]
            vn[s] = v_new[cu[s] + j]
        k2, v2 = cache_ops.append_token(k2, v2, kn, vn, tables, sub_lens, B)
    assert np.array_equal(ko, k2)
    assert np.array_equal(vo, v2)


def test_append_tokens_padding_rows_write_nothing():
    rng = np.random.default_rng(2)
    kp = rng.standard_normal((8, 4, 1, 2))
    vp = rng.standard_normal((8, 4, 1, 2))
    ko, vo = cache_ops.append_tokens(kp, vp, np.ones((2, 1, 2)), np.ones((2, 1, 2)),
                                     np.array([[1, 2], [3, 4]]), [-1, 3], [0, 2, 2], 4)
    assert np.array_equal(ko, kp) and np.array_equal(vo, vp)
