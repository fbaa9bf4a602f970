"""Pins of oracle/fp8.py: the E4M3FN field definition, ties, saturation,
an independent library cast, and the FP8 cache append."""

import math

import numpy as np
import pytest
import torch

from oracle import cache_ops, fp8


def test_decode_closed_forms():
    # Values fixed by the field layout (bias 7, 3 mantissa bits, subnormals
    # at exponent 0, S.1111.111 = NaN, no infinities).
    assert fp8.decode_e4m3(0x00) == 0.0 and math.copysign(1, fp8.decode_e4m3(0x80)) < 0
    assert fp8.decode_e4m3(0x01) == 2.0 ** -9            # smallest subnormal
    assert fp8.decode_e4m3(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert fp8.decode_e4m3(0x08) == 2.0 ** -6            # smallest normal
    assert fp8.decode_e4m3(0x38) == 1.0
    assert fp8.decode_e4m3(0x3F) == 1.875
    assert fp8.decode_e4m3(0x40) == 2.0
    assert fp8.decode_e4m3(0x7E) == 448.0 and fp8.decode_e4m3(0xFE) == -448.0
    assert math.isnan(fp8.decode_e4m3(0x7F)) and math.isnan(fp8.decode_e4m3(0xFF))
    mags = fp8.DECODE_TABLE[:0x7F]
    assert np.all(np.diff(mags) > 0)                      # codes 0..0x7E increase
    assert np.isfinite(fp8.DECODE_TABLE).sum() == 254
    assert np.array_equal(fp8.DECODE_TABLE[0x80:0xFF], -fp8.DECODE_TABLE[:0x7F])


def test_decode_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = fp8.DECODE_TABLE
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0, 1, 3000), rng.normal(0, 100, 3000),
                        rng.uniform(-448, 448, 3000), rng.normal(0, 1e-3, 1000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([fp8.encode_e4m3(v) for v in x], dtype=np.uint8)
    assert np.array_equal(ref, got)


def test_ties_go_to_even_and_saturation():
    assert fp8.encode_e4m3(1.0 + 1 / 16) == 0x38          # between 1.0 and 1.125: even is 1.0
    assert fp8.encode_e4m3(1.0 + 3 / 16) == 0x3A          # between 1.125 and 1.25: even is 1.25
    assert fp8.encode_e4m3(2.0 ** -10) == 0x00            # between 0 and 2^-9
    assert fp8.encode_e4m3(3 * 2.0 ** -10) == 0x02        # between 2^-9 and 2^-8
    assert fp8.encode_e4m3(-(1.0 + 1 / 16)) == 0xB8
    assert fp8.encode_e4m3(1.0 + 1 / 16 + 1e-9) == 0x39   # just above the tie
    for big in (448.0, 449.0, 464.0, 1e6, math.inf):
        assert fp8.encode_e4m3(big) == 0x7E
        assert fp8.encode_e4m3(-big) == 0xFE
    assert fp8.encode_e4m3(math.nan) == 0x7F


def test_round_trip_of_every_code():
    for c in range(256):
        v = fp8.decode_e4m3(c)
        if not math.isnan(v):
            assert fp8.encode_e4m3(v) == c


def test_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(9)
    finite = fp8.DECODE_TABLE[np.isfinite(fp8.DECODE_TABLE)]
    for v in rng.uniform(-460, 460, 2000):
        c = fp8.encode_e4m3(v)
        best = np.min(np.abs(finite - min(max(v, -448), 448)))
        assert abs(fp8.decode_e4m3(c) - min(max(v, -448), 448)) == best


def test_quantise_divides_in_float32():
    x = np.array([1.1, -3.3, 500.0, 0.0], dtype=np.float32)
    s = 0.7
    q = fp8.quantise(x, s)
    for xi, qi in zip(x, q):
        assert qi == fp8.encode_e4m3(float(np.float32(xi) / np.float32(s)))
    assert np.array_equal(fp8.dequantise(q, 1.0), fp8.DECODE_TABLE[q])


def test_fp8_append_writes_the_same_slots_as_the_plain_append():
    rng = np.random.default_rng(3)
    N, B, H, D = 12, 4, 2, 16
    tables = np.array([[7, 2, 11, -1], [3, 5, -1, -1]])
    lens_pre = np.array([9, 4])
    k_new = rng.normal(0, 1, (2, H, D)).astype(np.float32)
    v_new = rng.normal(0, 3, (2, H, D)).astype(np.float32)
    kp = rng.integers(0, 256, (N, B, H, D)).astype(np.uint8)
    vp = rng.integers(0, 256, (N, B, H, D)).astype(np.uint8)
    k2, v2 = fp8.append_token_fp8(kp, vp, k_new, v_new, tables, lens_pre, B, 0.05, 0.5)
    kf, vf = cache_ops.append_token(kp.astype(np.int64), vp.astype(np.int64),
                                    fp8.quantise(k_new, 0.05).astype(np.int64),
                                    fp8.quantise(v_new, 0.5).astype(np.int64), tables,
                                    lens_pre, B)
    assert np.array_equal(k2, kf) and np.array_equal(v2, vf)
    assert np.array_equal(k2[11, 1], fp8.quantise(k_new[0], 0.05))     # token 9 -> block 11, slot 1
    changed = np.argwhere((k2 != kp).any(axis=(2, 3)))
    assert sorted(map(tuple, changed.tolist())) == [(5, 0), (11, 1)]


def test_planted_encoder_mistakes_fail():
    # A round-half-up encoder and a non-saturating one differ from the pins.
    def half_up(x):
        mags = fp8.DECODE_TABLE[:0x7F]
        a = abs(x)
        lo = int(np.searchsorted(mags, a, side="right")) - 1
        if lo == 0x7E or mags[lo] == a:
            return lo
        return lo + 1 if a - mags[lo] >= mags[lo + 1] - a else lo
    assert half_up(1.0 + 1 / 16) != fp8.encode_e4m3(1.0 + 1 / 16)
    assert fp8.encode_e4m3(500.0) != 0x7F


def test_fp8_append_tokens_equals_repeated_single_appends_and_plain_slots():
    """Multi-token FP8 append: (1) the same codes as appending the chunk one
    token at a time with append_token_fp8 (pinned above), and (2) the same
    slots as the plain multi-token append, holding quantise() of the rows."""
    rng = np.random.default_rng(21)
    N, B, H, D = 12, 4, 2, 8
    tables = np.array([[3, 7, 1, -1], [0, 5, 9, 2], [11, -1, -1, -1]], np.int32)
    lens_pre = np.array([2, 5, -1])
    chunks = np.array([7, 6, 3])                       # the padding row's chunk writes nothing
    cu = np.concatenate([[0], np.cumsum(chunks)])
    T = int(cu[-1])
    k_new = rng.normal(0, 40, (T, H, D)).astype(np.float32)
    v_new = rng.normal(0, 0.3, (T, H, D)).astype(np.float32)
    pool = rng.integers(0, 256, (N, B, H, D)).astype(np.uint8)
    ks, vs = 0.5, 0.0625
    kc, vc = fp8.append_tokens_fp8(pool, pool, k_new, v_new, tables, lens_pre, cu, B, ks, vs)
    # (1) one token at a time
    ek, ev = pool.copy(), pool.copy()
    for s in range(len(chunks)):
        if lens_pre[s] < 0:
            continue
        for j in range(chunks[s]):
            t = cu[s] + j
            ek, ev = fp8.append_token_fp8(ek, ev, k_new[t:t + 1], v_new[t:t + 1], tables[s:s + 1],
                                          [lens_pre[s] + j], B, ks, vs)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)
    # (2) the plain append's slots, holding the quantised rows
    pk, pv = cache_ops.append_tokens(pool.astype(np.float64), pool.astype(np.float64),
                                     fp8.quantise(k_new, ks).astype(np.float64),
                                     fp8.quantise(v_new, vs).astype(np.float64),
                                     tables, lens_pre, cu, B)
    assert np.array_equal(kc, pk.astype(np.uint8)) and np.array_equal(vc, pv.astype(np.uint8))
