"""Number formats the cache is stored in (oracle side, test infrastructure).

bf16: the upper 16 bits of an IEEE-754 binary32.
fp8 e4m3 ("e4m3fn" of the OCP 8-bit floating point specification): 1 sign
bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
subnormals m/8 * 2^-6; there are no infinities; S.1111.111 is NaN; the
largest finite magnitude is 1.75 * 2^8 = 448.

The fp8 cache stores, per token, codes of c_j / s_j with s_j = amax_j / 448
(amax over the token's d_c content lanes, computed in fp32), and the rope
key in bf16. Reading the cache back is c_j = s_j * decode(code_j), exact in
float64.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_decode(codes) -> np.ndarray:
    """e4m3fn codes (uint8) -> float64, from the field definitions."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, sub, normal)
    nan = (e == 0xF) & ((c & 0x7) == 0x7)
    return np.where(nan, np.nan, val)


def e4m3_encode_f32(x) -> np.ndarray:
    """float32 values -> e4m3fn codes, round to nearest (ties to even code),
    saturating at +-448. The rounding decision is taken on the float32 value.

    Enumerates every finite code and picks the nearest: slow, obviously
    correct, meant for small arrays.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    codes = np.arange(0x7F, dtype=np.uint8)           # +0 .. +448
    vals = e4m3_decode(codes)
    even = (codes % 2 == 0)
    step = 1 << 15
    for i in range(0, flat.size, step):
        xs = flat[i:i + step]
        a = np.minimum(np.abs(xs), 448.0)
        dist = np.abs(a[:, None] - vals)               # [n, 127]
        cand = dist == dist.min(axis=1, keepdims=True)
        # ties: the even code (its mantissa LSB is 0)
        pick_even = cand & even
        choice = np.where(pick_even.any(axis=1, keepdims=True), pick_even, cand)
        code = np.argmax(choice, axis=1).astype(np.uint8)
        out[i:i + step] = np.where(np.signbit(xs), code | 0x80, code)
    return out.reshape(x.shape)


def fp8_cache_dequant(codes, scales) -> np.ndarray:
    """Stored fp8 latents [T, d_c] with per-token scales [T] -> float64."""
    return e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def fp8_quantize_tokens(c) -> tuple[np.ndarray, np.ndarray]:
    """Per-token e4m3 storage of latents c [T, d_c], decided in float32:
    amax in fp32, scale = amax / 448 in fp32 (1.0 if amax is 0), code of
    fp32(c) / scale in fp32. Returns (codes uint8, scales float32)."""
    c32 = np.asarray(c, dtype=np.float32)
    amax = np.abs(c32).max(axis=1)
    scale = np.where(amax == 0, np.float32(1.0), amax / np.float32(448.0)).astype(np.float32)
    q = (c32 / scale[:, None]).astype(np.float32)
    return e4m3_encode_f32(q), scale
