"""Pins for oracle.attention.

The paged result must equal dense attention on the contiguous history
([pofe] "How it works": only the addresses change).  The dense reference is
torch's scaled_dot_product_attention in float64 on the CPU (a library routine
the oracle does not use; it fixes the 1/sqrt(D) scale and, with enable_gqa,
the grouped-query head mapping), plus closed forms that a dropped term, a
wrong index or a transposed operand would break.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention


def build_paged(hists, B, N, rng):
    """Store each contiguous history [L, H, D] in a pool by numpy reshape."""
    H, D = hists[0].shape[1:]
    pool = np.full((N, B, H, D), np.nan)
    nbs = [-(-h.shape[0] // B) for h in hists]
    tables = np.full((len(hists), max(nbs)), -1, dtype=np.int64)
    perm = rng.permutation(N)
    pos = 0
    for s, h in enumerate(hists):
        nb = nbs[s]
        ids = perm[pos:pos + nb]
        pos += nb
        padded = np.full((nb * B, H, D), np.nan)
        padded[: h.shape[0]] = h
        pool[ids] = padded.reshape(nb, B, H, D)
        tables[s, :nb] = ids
    return pool, tables


def sdpa_reference(q, k_hist, v_hist):
    """Dense attention of one query row per head: q [Hq, D], K/V [L, Hkv, D]."""
    qt = torch.from_numpy(q)[:, None, :]                      # [Hq, 1, D]
    kt = torch.from_numpy(np.ascontiguousarray(k_hist.transpose(1, 0, 2)))  # [Hkv, L, D]
    vt = torch.from_numpy(np.ascontiguousarray(v_hist.transpose(1, 0, 2)))
    out = F.scaled_dot_product_attention(qt, kt, vt, enable_gqa=True)
    return out[:, 0, :].numpy()


@pytest.mark.parametrize("Hq,Hkv,D,B", [(2, 1, 16, 4), (4, 4, 8, 8), (8, 2, 32, 16),
                                        (6, 3, 16, 1), (16, 2, 64, 32)])
def test_paged_equals_dense_sdpa(Hq, Hkv, D, B):
    rng = np.random.default_rng(Hq * 100 + D + B)
    lens = [1, 2, B, B + 1, 3 * B + 5, 47]
    k_h = [rng.standard_normal((L, Hkv, D)) for L in lens]
    v_h = [rng.standard_normal((L, Hkv, D)) for L in lens]
    q = rng.standard_normal((len(lens), Hq, D))
    N = sum(-(-L // B) for L in lens) + 7
    k_pool, tables = build_paged(k_h, B, N, np.random.default_rng(5))
    v_pool, tables2 = build_paged(v_h, B, N, np.random.default_rng(5))
    assert (tables == tables2).all()
    out = attention.decode_attention(q, k_pool, v_pool, tables, lens, B)
    for s in range(len(lens)):
        ref = sdpa_reference(q[s], k_h[s], v_h[s])
        np.testing.assert_allclose(out[s], ref, rtol=1e-12, atol=1e-13)


def test_gqa_head_mapping_is_floor_division():
    # Two KV heads whose V rows are all 0 and all 1: query heads 0,1 use
    # KV head 0 and heads 2,3 use KV head 1 (h // g); h % H_kv would give 0,1,0,1.
    B, L, D = 4, 6, 8
    rng = np.random.default_rng(1)
    k = rng.standard_normal((L, 2, D))
    v = np.zeros((L, 2, D))
    v[:, 1, :] = 1.0
    k_pool, tables = build_paged([k], B, 4, rng)
    v_pool, _ = build_paged([v], B, 4, np.random.default_rng(1))
    # rebuild v with the same table
    v_pool = np.full_like(k_pool, np.nan)
    pad = np.full((2 * B, 2, D), np.nan)
    pad[:L] = v
    v_pool[tables[0, :2]] = pad.reshape(2, B, 2, D)
    q = rng.standard_normal((1, 4, D))
    out = attention.decode_attention(q, k_pool, v_pool, tables, [L], B)
    np.testing.assert_allclose(out[0, :2], 0.0, atol=1e-15)
    np.testing.assert_allclose(out[0, 2:], 1.0, atol=1e-14)


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(2)
    k_pool = rng.standard_normal((3, 4, 1, 8))
    v_pool = rng.standard_normal((3, 4, 1, 8))
    q = rng.standard_normal((1, 2, 8))
    out = attention.decode_attention(q, k_pool, v_pool, np.array([[2]]), [1], 4)
    assert np.array_equal(out[0, 0], v_pool[2, 0, 0])
    assert np.array_equal(out[0, 1], v_pool[2, 0, 0])


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(3)
    L, B, D = 13, 4, 16
    k = rng.standard_normal((L, 1, D))
    v = rng.standard_normal((L, 1, D))
    kp, tables = build_paged([k], B, 9, np.random.default_rng(7))
    vp, _ = build_paged([v], B, 9, np.random.default_rng(7))
    out = attention.decode_attention(np.zeros((1, 1, D)), kp, vp, tables, [L], B)
    np.testing.assert_allclose(out[0, 0], v[:, 0, :].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_dominant_logit_selects_its_value():
    rng = np.random.default_rng(4)
    L, B, D = 20, 8, 16
    q = rng.standard_normal(D)
    k = rng.standard_normal((L, 1, D)) * 0.01
    k[11, 0] = 200.0 * q / np.linalg.norm(q)
    v = rng.standard_normal((L, 1, D))
    kp, tables = build_paged([k], B, 5, np.random.default_rng(9))
    vp, _ = build_paged([v], B, 5, np.random.default_rng(9))
    out = attention.decode_attention(q[None, None, :], kp, vp, tables, [L], B)
    np.testing.assert_allclose(out[0, 0], v[11, 0], atol=1e-12)


def test_scale_argument_and_default():
    rng = np.random.default_rng(6)
    L, B, D = 9, 4, 16
    k = rng.standard_normal((L, 1, D))
    v = rng.standard_normal((L, 1, D))
    q = rng.standard_normal((1, 1, D))
    kp, tables = build_paged([k], B, 6, np.random.default_rng(2))
    vp, _ = build_paged([v], B, 6, np.random.default_rng(2))
    a = attention.decode_attention(q, kp, vp, tables, [L], B)
    b = attention.decode_attention(q, kp, vp, tables, [L], B, scale=1.0 / math.sqrt(D))
    c = attention.decode_attention(q / math.sqrt(D), kp, vp, tables, [L], B, scale=1.0)
    assert np.array_equal(a, b)
    np.testing.assert_allclose(a, c, rtol=1e-13)


def test_empty_sequence_gives_zeros():
    kp = np.zeros((2, 4, 1, 4))
    out = attention.decode_attention(np.ones((1, 2, 4)), kp, kp, np.array([[-1]]), [0], 4)
    assert (out == 0).all()


def test_relabelling_blocks_changes_nothing():
    # [note] "Try it": moving a block to another physical address changes
    # where the data is found, not the result.
    rng = np.random.default_rng(8)
    B, H, D, N = 4, 2, 8, 20
    lens = [7, 13, 4]
    k_h = [rng.standard_normal((L, H, D)) for L in lens]
    v_h = [rng.standard_normal((L, H, D)) for L in lens]
    q = rng.standard_normal((3, 4, D))
    kp, tables = build_paged(k_h, B, N, np.random.default_rng(0))
    vp, _ = build_paged(v_h, B, N, np.random.default_rng(0))
    base = attention.decode_attention(q, kp, vp, tables, lens, B)
    relabel = rng.permutation(N)                   # old id -> new id
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[relabel] = kp
    vp2[relabel] = vp
    tables2 = np.where(tables >= 0, relabel[np.maximum(tables, 0)], -1)
    moved = attention.decode_attention(q, kp2, vp2, tables2, lens, B)
    assert np.array_equal(base, moved)


def test_shared_prefix_equals_private_copies():
    # Two tables pointing at the same prefix blocks give the same result as
    # tables holding private bitwise copies of them.
    rng = np.random.default_rng(10)
    B, H, D, N = 4, 1, 8, 16
    kp = rng.standard_normal((N, B, H, D))
    vp = rng.standard_normal((N, B, H, D))
    kp[[2, 3]] = kp[[0, 1]]
    vp[[2, 3]] = vp[[0, 1]]
    shared = np.array([[0, 1, 5], [0, 1, 6]])
    private = np.array([[0, 1, 5], [2, 3, 6]])
    q = rng.standard_normal((2, 2, D))
    a = attention.decode_attention(q, kp, vp, shared, [11, 10], B)
    b = attention.decode_attention(q, kp, vp, private, [11, 10], B)
    assert np.array_equal(a, b)


def test_tail_slots_are_never_read():
    rng = np.random.default_rng(11)
    B, D = 8, 8
    kp = rng.standard_normal((4, B, 1, D))
    vp = rng.standard_normal((4, B, 1, D))
    kp[1, 3:] = np.nan
    vp[1, 3:] = np.nan
    kp[[0, 2]] = np.nan
    vp[[0, 2]] = np.nan
    out = attention.decode_attention(rng.standard_normal((1, 1, D)), kp, vp,
                                     np.array([[3, 1, -1]]), [B + 3], B)
    assert np.isfinite(out).all()


@pytest.mark.parametrize("B,P", [(4, 4), (4, 8), (8, 24), (16, 512), (16, 32)])
def test_online_recurrence_and_merge_equal_two_pass(B, P):
    rng = np.random.default_rng(B + P)
    lens = [1, B - 1 if B > 1 else 1, 2 * P + 3, P, 5 * B + 1]
    H, D = 2, 16
    k_h = [rng.standard_normal((L, H, D)) * 2 for L in lens]
    v_h = [rng.standard_normal((L, H, D)) for L in lens]
    q = rng.standard_normal((len(lens), 4, D))
    N = sum(-(-L // B) for L in lens) + 3
    kp, tables = build_paged(k_h, B, N, np.random.default_rng(1))
    vp, _ = build_paged(v_h, B, N, np.random.default_rng(1))
    two_pass = attention.decode_attention(q, kp, vp, tables, lens, B)
    split = attention.split_k_decode_attention(q, kp, vp, tables, lens, B, P)
    np.testing.assert_allclose(split, two_pass, rtol=1e-12, atol=1e-14)
    # the whole sequence as one run of the recurrence: o / l
    for s, L in enumerate(lens):
        m, l, o = attention.online_softmax_blocks(q[s, 0], kp, vp, tables[s], L, B, 0,
                                                  1 / math.sqrt(D))
        np.testing.assert_allclose(o / l, two_pass[s, 0], rtol=1e-12, atol=1e-14)
        assert l >= 1.0


def test_merge_states_closed_form():
    # Two halves with equal logits c: each state is (c, n_p, sum of its v);
    # the merge must be the plain mean over both halves, whatever c is.
    v = np.arange(12.0).reshape(6, 2)
    for c in (0.0, 50.0, -700.0):
        a = (c, 4.0, v[:4].sum(axis=0))
        b = (c + 3.0, 2.0 * math.exp(0.0), v[4:].sum(axis=0))  # logits c+3 for b
        out = attention.merge_states([a, b])
        w = np.array([1.0] * 4 + [math.exp(3.0)] * 2)
        np.testing.assert_allclose(out, (w[:, None] * v).sum(0) / w.sum(), rtol=1e-13)
    empty = (-math.inf, 0.0, np.zeros(2))
    np.testing.assert_allclose(attention.merge_states([empty, (0.0, 1.0, np.ones(2))]), 1.0)
    assert (attention.merge_states([empty]) == 0).all()


def test_large_logits_are_stable():
    # Softmax is shift invariant: adding 1000 to every logit (a key component
    # along q) must not change the result, and nothing may overflow.  Without
    # the max subtraction of the stable two-pass form exp(1000) is inf.
    rng = np.random.default_rng(12)
    L, B, D = 10, 4, 16
    q = np.zeros((1, 1, D))
    q[0, 0, 0] = 1.0
    k = rng.standard_normal((L, 1, D))
    v = rng.standard_normal((L, 1, D))
    k_big = k.copy()
    k_big[:, 0, 0] += 1000.0 * math.sqrt(D)
    kp, tables = build_paged([k], B, 5, np.random.default_rng(3))
    kp_big, _ = build_paged([k_big], B, 5, np.random.default_rng(3))
    vp, _ = build_paged([v], B, 5, np.random.default_rng(3))
    a = attention.decode_attention(q, kp, vp, tables, [L], B)
    b = attention.decode_attention(q, kp_big, vp, tables, [L], B)
    assert np.isfinite(b).all()
    np.testing.assert_allclose(b, a, rtol=1e-9, atol=1e-10)
    m, l, o = attention.online_softmax_blocks(q[0, 0], kp_big, vp, tables[0], L, B, 0,
                                              1 / math.sqrt(D))
    np.testing.assert_allclose(o / l, a[0, 0], rtol=1e-9, atol=1e-10)


def test_recurrence_keeps_the_running_maximum():
    # The first block holds logits near +700, later blocks near -700.  The
    # running maximum must not drop back to a later block's maximum: if it
    # did, the rescale factor exp(m_old - m_new) = exp(1400) would overflow.
    rng = np.random.default_rng(13)
    L, B, D = 12, 4, 4
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    k = rng.standard_normal((L, 1, D)) * 0.1
    k[:B, 0, 0] += 700.0 * math.sqrt(D)
    k[B:, 0, 0] -= 700.0 * math.sqrt(D)
    v = rng.standard_normal((L, 1, D))
    kp, tables = build_paged([k], B, 4, np.random.default_rng(4))
    vp, _ = build_paged([v], B, 4, np.random.default_rng(4))
    ref = attention.decode_attention(q, kp, vp, tables, [L], B)
    assert np.isfinite(ref).all()
    m, l, o = attention.online_softmax_blocks(q[0, 0], kp, vp, tables[0], L, B, 0,
                                              1 / math.sqrt(D))
    np.testing.assert_allclose(o / l, ref[0, 0], rtol=1e-12, atol=1e-13)
    split = attention.split_k_decode_attention(q, kp, vp, tables, [L], B, B)
    np.testing.assert_allclose(split, ref, rtol=1e-12, atol=1e-13)


def test_log_normaliser_matches_scipy_and_recombines():
    # scipy's logsumexp is an independent routine; and the normalised halves
    # of a split history, weighted by e^lse, give the whole result.
    from scipy.special import logsumexp
    rng = np.random.default_rng(41)
    B, D, Hq, Hkv = 4, 8, 4, 2
    lens = [1, 7, 13]
    k_h = [rng.standard_normal((L, Hkv, D)) * 3 for L in lens]
    v_h = [rng.standard_normal((L, Hkv, D)) for L in lens]
    q = rng.standard_normal((3, Hq, D))
    kp, tables = build_paged(k_h, B, 12, np.random.default_rng(2))
    vp, _ = build_paged(v_h, B, 12, np.random.default_rng(2))
    lse = attention.decode_log_normaliser(q, kp, tables, lens, B)
    scale = 1 / math.sqrt(D)
    for s, L in enumerate(lens):
        for h in range(Hq):
            z = scale * k_h[s][:, h // 2, :] @ q[s, h]
            assert abs(lse[s, h] - logsumexp(z)) < 1e-12
    # Split sequence 2 (13 tokens) at 8 = two blocks: prefix and suffix.
    s, cut = 2, 8
    pre = attention.decode_attention(q[s:s + 1], kp, vp, tables[s:s + 1], [cut], B)
    lp = attention.decode_log_normaliser(q[s:s + 1], kp, tables[s:s + 1], [cut], B)
    suf_tab = np.concatenate([tables[s:s + 1, cut // B:], np.full((1, cut // B), -1)], axis=1)
    suf = attention.decode_attention(q[s:s + 1], kp, vp, suf_tab, [13 - cut], B)
    ls = attention.decode_log_normaliser(q[s:s + 1], kp, suf_tab, [13 - cut], B)
    m = np.maximum(lp, ls)[..., None]
    wa, wb = np.exp(lp[..., None] - m), np.exp(ls[..., None] - m)
    comb = (wa * pre + wb * suf) / (wa + wb)
    full = attention.decode_attention(q[s:s + 1], kp, vp, tables[s:s + 1], [13], B)
    np.testing.assert_allclose(comb, full, rtol=1e-12, atol=1e-13)
    assert np.isneginf(attention.decode_log_normaliser(q[:1], kp, tables[:1], [0], B)).all()
