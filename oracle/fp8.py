"""E4M3 8-bit float codes for a quantised KV cache, from the format's definition.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

[P3 §4.1 量化: storing tensors in 8 bits instead of 16 halves their memory
and the bytes moved, GPUs compute on FP8; §1.5: the KV cache size is linear in
the bytes per element.] The pages name FP8 but fix no format; the reading
taken is the OCP 8-bit floating point "E4M3" encoding:

* bit 7 sign, bits 6..3 exponent ``e`` (bias 7), bits 2..0 mantissa ``m``;
* ``e == 0``: subnormal, value ``m / 8 * 2^-6``;
* ``e == 15 and m == 7``: NaN (there are no infinities);
* otherwise ``(1 + m / 8) * 2^(e - 7)``; the largest finite value is 448.

A cache of codes holds ``value / scale``: element = code's value * scale, one
fp32 scale for all K and one for all V of a layer. Writing a bf16 row
computes ``x / scale`` in fp32 (correctly rounded, the precision the write
takes its decision in) and stores the nearest E4M3 value, ties to the even
code, magnitudes beyond 448 saturating to 448, NaN kept as NaN.
"""

from __future__ import annotations

import numpy as np


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> float64 values, exactly, field by field."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# every non-negative finite value with its code, in code order (increasing value)
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = decode(_POS_CODES)


def encode(y: np.ndarray) -> np.ndarray:
    """float64 values -> uint8 codes: nearest representable value, ties to the
    even code, saturating at +-448, NaN -> sign | 0x7f. Brute force over the
    127 non-negative finite values."""
    y = np.asarray(y, dtype=np.float64)
    flat = y.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    neg = np.signbit(flat)
    mag = np.abs(flat)
    nan = np.isnan(flat)
    safe = np.where(nan, 0.0, np.minimum(mag, 448.0))
    chunk = 1 << 16
    for lo in range(0, flat.size, chunk):
        s = safe[lo:lo + chunk]
        dist = np.abs(s[:, None] - _POS_VALUES[None, :])          # [n, 127]
        best = dist.min(axis=1, keepdims=True)
        tied = dist == best
        # among the nearest codes prefer the even one (at most two are nearest)
        even = tied & ((_POS_CODES[None, :] & 1) == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), tied.argmax(axis=1))
        out[lo:lo + chunk] = _POS_CODES[pick]
    out = np.where(nan, np.uint8(0x7F), out)
    out = out | np.where(neg, np.uint8(0x80), np.uint8(0))
    return out.astype(np.uint8).reshape(y.shape)


def quantize_bf16(bits: np.ndarray, scale: float) -> np.ndarray:
    """Raw bf16 bits -> E4M3 codes of ``value / scale`` (the division in fp32)."""
    x32 = (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        y = x32 / np.float32(scale)
    return encode(y.astype(np.float64))


def write_kv(k_cache, v_cache, k_new_bits, v_new_bits, slot_mapping, block_size: int,
             k_scale: float, v_scale: float) -> None:
    """The E4M3 cache write [P1 §02 slot_mapping]: quantise each new bf16 row
    and store its codes in the named slot (negative slot: no write)."""
    kq = quantize_bf16(k_new_bits, k_scale)
    vq = quantize_bf16(v_new_bits, v_scale)
    for i, s in enumerate(np.asarray(slot_mapping).tolist()):
        if s < 0:
            continue
        block, offset = divmod(int(s), block_size)
        k_cache[block][offset] = kq[i]
        v_cache[block][offset] = vq[i]
