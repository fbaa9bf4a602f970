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


def e4m3_half_step(y: float) -> float:
    """Half the spacing of E4M3FN values around |y| (|y| <= 448), from the field
    layout: 3 mantissa bits, so normal numbers in [2^e, 2^(e+1)) are 2^(e-3)
    apart; below 2^-6 (subnormals) the spacing is 2^-9."""
    a = abs(y)
    if a < 2.0 ** -6:
        return 2.0 ** -10
    return 2.0 ** (math.floor(math.log2(a)) - 4)


SCALES = (0.05, 0.0625, 0.125, 0.7, 3.0)


def scale_convention_holds(quantise, dequantise) -> bool:
    """The scale reading: a code stands for decode(code) * scale, and the code
    stored for x is the nearest one to x / scale.  Checked without the
    oracle's formulas: (1) the code of 1.0 (0x38) stands for the scale itself;
    (2) every finite code survives dequantise -> quantise unchanged; (3) an
    in-range x comes back within half an E4M3 step of x / scale, times the
    scale (the closed-form rounding bound)."""
    rng = np.random.default_rng(17)
    finite = [c for c in range(256) if not math.isnan(fp8.decode_e4m3(c))]
    for s in SCALES:
        s32 = float(np.float32(s))
        if dequantise(np.array([0x38], np.uint8), s)[0] != s32:
            return False
        codes = np.array(finite, np.uint8)
        if not np.array_equal(quantise(dequantise(codes, s), s), codes):
            return False
        x = (rng.uniform(-440, 440, 400) * s32).astype(np.float32)
        back = dequantise(quantise(x, s), s)
        for xi, bi in zip(x.astype(np.float64), back):
            y = xi / s32
            if abs(bi - xi) > e4m3_half_step(y) * s32 * (1 + 1e-6) + 1e-30:
                return False
    return True


def test_scale_convention_round_trip():
    # [pofe] "Fine-tuned models and adapters": FP8 changes the bytes per
    # block and nothing else, so a stored code must give back the value it
    # was written for, to within the format's rounding, at any scale.
    assert scale_convention_holds(fp8.quantise, fp8.dequantise)


def test_planted_scale_inversion_fails():
    # A dequantiser that divides by the scale, or a quantiser that multiplies,
    # must fail the convention pin at non-unit scales.
    def dequantise_divides(codes, scale):
        return fp8.DECODE_TABLE[np.asarray(codes, np.uint8)] / np.float64(np.float32(scale))

    def quantise_multiplies(x, scale):
        return fp8.quantise(np.asarray(x, np.float64) * float(np.float32(scale)) ** 2, scale)

    assert not scale_convention_holds(fp8.quantise, dequantise_divides)
    assert not scale_convention_holds(quantise_multiplies, fp8.dequantise)


def test_quantise_divides_in_float32():
    # torch divides two float32 tensors in float32 and casts with its own
    # float8_e4m3fn encoder (an independent routine).  The inputs are chosen
    # so that the float32 quotient lands exactly on a tie between two codes
    # while the exact quotient does not: a float64 division would pick the
    # other code.
    cases = [(2.5823814868927, 2.430476665496826), (3.468320846557617, 2.9206912517547607),
             (7.949495315551758, 3.740938901901245), (0.01111726462841034, 0.020926615223288536)]
    for x, s in cases:
        x32 = torch.tensor([x], dtype=torch.float32)
        s32 = torch.tensor([s], dtype=torch.float32)
        ref = (x32 / s32).to(torch.float8_e4m3fn).view(torch.uint8).item()
        got = int(fp8.quantise(np.array([x], np.float32), s)[0])
        assert got == ref
        assert fp8.encode_e4m3(float(np.float64(np.float32(x)) / np.float64(np.float32(s)))) != ref
    rng = np.random.default_rng(23)
    for s in SCALES:
        x = rng.normal(0, 50 * s, 2000).astype(np.float32)
        ref = (torch.from_numpy(x) / torch.tensor(s, dtype=torch.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(fp8.quantise(x, s), ref)
    q = fp8.quantise(np.array([1.1, -3.3, 500.0, 0.0], np.float32), 0.7)
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


# --- per-head scales ---------------------------------------------------------

def test_per_head_scales_reduce_to_the_per_pool_rule():
    # Every head at the same scale: exactly the per-pool codes and values,
    # which the round-trip and torch pins above fix.
    rng = np.random.default_rng(31)
    x = rng.normal(0, 4, (5, 3, 16)).astype(np.float32)
    for s in SCALES:
        q = fp8.quantise_heads(x, [s] * 3)
        assert np.array_equal(q, fp8.quantise(x, s))
        assert np.array_equal(fp8.dequantise_heads(q, [s] * 3), fp8.dequantise(q, s))


def per_head_convention_holds(quantise_heads, dequantise_heads) -> bool:
    """Distinct scales per head: (1) the code of 1.0 in head h stands for
    scale h itself, whatever the other axes; (2) every finite code survives
    dequantise -> quantise in every head."""
    scales = np.array([0.05, 3.0, 0.0625, 0.7], np.float32)
    H = len(scales)
    ones = np.full((2, 3, H, 4), 0x38, np.uint8)
    vals = dequantise_heads(ones, scales)
    for h in range(H):
        if not np.all(vals[:, :, h, :] == np.float64(scales[h])):
            return False
    finite = np.array([c for c in range(256) if not math.isnan(fp8.decode_e4m3(c))], np.uint8)
    codes = np.stack([np.roll(finite, 37 * h) for h in range(H)], axis=0)[None]   # [1, H, 254]
    return np.array_equal(quantise_heads(dequantise_heads(codes, scales), scales), codes)


def test_per_head_scale_convention():
    assert per_head_convention_holds(fp8.quantise_heads, fp8.dequantise_heads)


def test_planted_per_head_mistakes_fail():
    # Scales applied along the wrong axis (the channel axis instead of the
    # head axis, or the heads in reverse order) must fail the pin.
    def deq_reversed(codes, scales):
        return fp8.dequantise_heads(codes, np.asarray(scales)[::-1])

    def deq_channel_axis(codes, scales):
        codes = np.asarray(codes, np.uint8)
        sc = np.asarray(scales, np.float32)
        return fp8.DECODE_TABLE[codes] * np.resize(sc, codes.shape[-1]).astype(np.float64)

    assert not per_head_convention_holds(fp8.quantise_heads, deq_reversed)
    assert not per_head_convention_holds(fp8.quantise_heads, deq_channel_axis)


def test_per_head_invalid_scale_gives_nan_codes_in_that_head_only():
    rng = np.random.default_rng(32)
    x = rng.normal(0, 1, (4, 3, 8)).astype(np.float32)
    for bad in (0.0, -1.0, math.nan, math.inf):
        q = fp8.quantise_heads(x, [0.5, bad, 2.0])
        assert np.all(q[:, 1, :] == 0x7F)
        assert np.array_equal(q[:, 0, :], fp8.quantise(x[:, 0, :], 0.5))
        assert np.array_equal(q[:, 2, :], fp8.quantise(x[:, 2, :], 2.0))
        v = fp8.dequantise_heads(q, [0.5, bad, 2.0])
        assert np.all(np.isnan(v[:, 1, :])) and not np.any(np.isnan(v[:, 0, :]))


def test_fp8_append_with_per_head_scales_is_the_per_pool_append_head_by_head():
    # Head h of the per-head append equals head h of the per-pool append at
    # scale h (pinned above against the plain append's slots).
    rng = np.random.default_rng(33)
    N, B, H, D = 10, 4, 3, 8
    tables = np.array([[4, 1, 9], [2, 6, -1]])
    lens_pre = np.array([6, 3])
    k_new = rng.normal(0, 2, (2, H, D)).astype(np.float32)
    v_new = rng.normal(0, 5, (2, H, D)).astype(np.float32)
    kp = rng.integers(0, 256, (N, B, H, D)).astype(np.uint8)
    vp = rng.integers(0, 256, (N, B, H, D)).astype(np.uint8)
    ks, vs = [0.05, 1.0, 3.0], [0.7, 0.0625, 2.0]
    k2, v2 = fp8.append_token_fp8(kp, vp, k_new, v_new, tables, lens_pre, B, ks, vs)
    for h in range(H):
        kh, vh = fp8.append_token_fp8(kp, vp, k_new, v_new, tables, lens_pre, B, ks[h], vs[h])
        assert np.array_equal(k2[:, :, h], kh[:, :, h]) and np.array_equal(v2[:, :, h], vh[:, :, h])
