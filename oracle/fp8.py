"""FP8 (E4M3FN) cache blocks: encoding, decoding, append and dequantisation (oracle).

Test infrastructure only; see the package docstring for who may use it.

[pofe] "Fine-tuned models and adapters": an FP8 cache halves the bytes per
block and nothing else about paging changes; [pofe] "Failure modes": fewer
bytes per token is the lever once the cache dominates step time.  The pages
name no FP8 format and no scale convention.  Readings taken here:

* Format: E4M3FN of the OCP 8-bit floating point specification, the
  format gfx950's conversion instructions implement: 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent 0 is subnormal
  (value m/8 * 2^-6); no infinities; S.1111.111 is NaN; the largest finite
  magnitude is 1.75 * 2^8 = 448.
* Encoding: round to nearest, ties to even; magnitudes beyond 448 saturate
  to +-448 (the cache must not turn a large activation into NaN); NaN stays
  NaN (0x7F with the input's sign).
* Scale: one float32 per pool (K and V separately), a per-tensor scale.
  The stored code is encode(fp32(x) / fp32(scale)), the division done in
  float32 so that both sides reach the same code; the value a code stands
  for is decode(code) * scale.  Pinned without these formulas: at scales
  other than 1 every finite code survives dequantise then quantise, the
  code of 1.0 stands for the scale, and a value comes back within half an
  E4M3 step (times the scale) of what was written.
* Per-head scales (the other option the survey of FP8 caches names; the
  pages are silent): one float32 per KV head and pool, head h's codes
  following the rule above with its own scale.  A head whose scale is not
  finite and positive has no defined codes: its rows store the NaN code
  0x7F.  Pinned by reduction to the per-pool rule when every head has the
  same scale, by the code of 1.0 in head h standing for scale h, and by the
  round trip at distinct scales per head.
"""

from __future__ import annotations

import math

import numpy as np

from .paging import resolve

E4M3_MAX = 448.0


def decode_e4m3(code: int) -> float:
    """The real value of one E4M3FN byte, from the field definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


DECODE_TABLE = np.array([decode_e4m3(c) for c in range(256)], dtype=np.float64)


def encode_e4m3(x: float) -> int:
    """Nearest E4M3FN code to x (ties to the even mantissa), saturating.

    Works on the exact value of x: every finite code is a multiple of 2^-9,
    so x is compared with the two neighbouring codes of the same sign.
    """
    x = float(x)
    if math.isnan(x):
        return 0xFF if math.copysign(1.0, x) < 0 else 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0x00
    a = abs(x)
    if a >= E4M3_MAX:
        return sign | 0x7E
    # Magnitude codes 0x00 .. 0x7E are increasing in value; find the largest
    # code whose value is <= a, then compare with the next one.
    mags = DECODE_TABLE[:0x7F]
    lo = int(np.searchsorted(mags, a, side="right")) - 1
    if mags[lo] == a or lo == 0x7E:
        return sign | lo
    hi = lo + 1
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    if d_lo < d_hi:
        pick = lo
    elif d_hi < d_lo:
        pick = hi
    else:
        pick = lo if lo % 2 == 0 else hi   # tie: the even mantissa
    return sign | pick


def quantise(x: np.ndarray, scale: float) -> np.ndarray:
    """Codes of encode(fp32(x) / fp32(scale)), elementwise, uint8."""
    xs = np.asarray(x, dtype=np.float32) / np.float32(scale)
    flat = [encode_e4m3(v) for v in xs.reshape(-1)]
    return np.array(flat, dtype=np.uint8).reshape(xs.shape)


def dequantise(codes: np.ndarray, scale: float) -> np.ndarray:
    """float64 values decode(code) * scale."""
    return DECODE_TABLE[np.asarray(codes, dtype=np.uint8)] * np.float64(np.float32(scale))


NAN_CODE = 0x7F


def scale_is_valid(scale) -> bool:
    s = float(np.float32(scale))
    return math.isfinite(s) and s > 0.0


def quantise_heads(x: np.ndarray, scales) -> np.ndarray:
    """Codes of x [..., H_kv, D] with per-head scales [H_kv]: head h is
    quantise(x[..., h, :], scales[h]), or all NAN_CODE when scales[h] is not
    finite and positive."""
    x = np.asarray(x, dtype=np.float32)
    scales = np.asarray(scales, dtype=np.float32).reshape(-1)
    if x.shape[-2] != scales.shape[0]:
        raise ValueError("one scale per KV head")
    out = np.empty(x.shape, dtype=np.uint8)
    for h, sc in enumerate(scales):
        out[..., h, :] = quantise(x[..., h, :], sc) if scale_is_valid(sc) else NAN_CODE
    return out


def dequantise_heads(codes: np.ndarray, scales) -> np.ndarray:
    """float64 values of codes [..., H_kv, D]: decode(code) * scales[h] in
    head h (NaN throughout a head whose scale is not finite and positive)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float32).reshape(-1)
    if codes.shape[-2] != scales.shape[0]:
        raise ValueError("one scale per KV head")
    out = np.empty(codes.shape, dtype=np.float64)
    for h, sc in enumerate(scales):
        out[..., h, :] = dequantise(codes[..., h, :], sc) if scale_is_valid(sc) else math.nan
    return out


def _quantise_row(x: np.ndarray, scale) -> np.ndarray:
    """A [H_kv, D] row: per-pool scale (a number) or per-head scales (a
    sequence of H_kv numbers)."""
    if np.ndim(scale) == 0:
        return quantise(x, scale)
    return quantise_heads(x, scale)


def append_token_fp8(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
                     v_new: np.ndarray, tables: np.ndarray, lens_pre, block_size: int,
                     k_scale: float, v_scale: float):
    """Cache append into uint8 code pools: the [pofe] "How it works" decode-step
    write (slot len mod b of the block listed at len / b), with the new
    token's k and v quantised as above.  Every other byte is unchanged.

    k_new, v_new: [S, H_kv, D] (float32-representable values); pools uint8
    [N, B, H_kv, D]; lens_pre: [S] (negative: padding row, no write).
    k_scale, v_scale: one number per pool, or one per KV head ([H_kv],
    quantise_heads).
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    num_blocks = k_pool.shape[0]
    for s, length in enumerate(lens_pre):
        length = int(length)
        if length < 0:
            continue
        physical, offset = resolve(tables[s], block_size, length)
        if not (0 <= physical < num_blocks):
            raise IndexError(f"sequence {s}: block id {physical} outside the pool")
        k_out[physical, offset] = _quantise_row(k_new[s], k_scale)
        v_out[physical, offset] = _quantise_row(v_new[s], v_scale)
    return k_out, v_out


def append_tokens_fp8(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
                      v_new: np.ndarray, tables: np.ndarray, lens_pre, cu_seqlens,
                      block_size: int, k_scale: float, v_scale: float):
    """The multi-token append of prefill chunks into uint8 code pools: sequence
    s writes the packed rows k_new[cu_seqlens[s] + j], j < n_s, at positions
    lens_pre[s] + j ([pofe] "How it works": prefill writes the prompt into its
    blocks), each row quantised as in append_token_fp8.  A negative lens_pre
    marks a padding row.

    k_new, v_new: [T, H_kv, D] packed (float32-representable values); pools
    uint8 [N, B, H_kv, D]; lens_pre [S]; cu_seqlens [S + 1].
    """
    k_out = k_pool.copy()
    v_out = v_pool.copy()
    num_blocks = k_pool.shape[0]
    cu = [int(x) for x in cu_seqlens]
    for s, start in enumerate(lens_pre):
        start = int(start)
        if start < 0:
            continue
        for j in range(cu[s + 1] - cu[s]):
            physical, offset = resolve(tables[s], block_size, start + j)
            if not (0 <= physical < num_blocks):
                raise IndexError(f"sequence {s}: block id {physical} outside the pool")
            k_out[physical, offset] = quantise(k_new[cu[s] + j], k_scale)
            v_out[physical, offset] = quantise(v_new[cu[s] + j], v_scale)
    return k_out, v_out

