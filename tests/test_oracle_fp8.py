"""Pins of the E4M3 codec and the quantised-cache attention oracle (CPU only).

* decode of all 256 codes agrees with torch's own float8_e4m3fn widening (an
  implementation independent of the oracle), NaN codes included;
* constants the format fixes: 1.0, 2.0, 1.5, the largest finite value 448,
  the smallest normal 2^-6 and the smallest subnormal 2^-9;
* encode agrees with torch's float -> float8_e4m3fn conversion on every bf16
  value inside the finite range, and on fp32 midpoints between codes;
* ties go to the even code, magnitudes at or beyond 448 saturate, NaN stays
  NaN, signs survive (including -0);
* encode(decode(c)) == c for every finite code;
* the quantised write divides in fp32 before rounding;
* attention over a quantised cache equals attention over the dequantised
  values (the scales applied to K and to V respectively).
A planted mistake (ties away from zero) is caught by the tie pin.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_encode(values_f32):
    t = torch.from_numpy(np.asarray(values_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got, want = fp8.decode(codes), _torch_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.isnan(got).sum() == 2                     # 0x7f and 0xff
    ok = ~np.isnan(got)
    assert np.array_equal(got[ok], want[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))


def test_format_constants():
    d = fp8.decode(np.array([0x38, 0x40, 0x3C, 0x7E, 0x08, 0x01, 0x00, 0x80, 0xFE],
                            dtype=np.uint8))
    assert d[:6].tolist() == [1.0, 2.0, 1.5, 448.0, 2.0 ** -6, 2.0 ** -9]
    assert d[6] == 0.0 and not np.signbit(d[6]) and d[7] == 0.0 and np.signbit(d[7])
    assert d[8] == -448.0
    finite = fp8.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(finite) > 0)                  # codes ordered by value
    assert finite.max() == 448.0


def test_encode_matches_torch_on_all_bf16_values():
    bits = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    x = bits.view(np.float32)
    inside = np.isfinite(x) & (np.abs(x) < 448.0)
    got = fp8.encode(x[inside].astype(np.float64))
    assert np.array_equal(got, _torch_encode(x[inside]))


def test_encode_matches_torch_on_midpoints():
    pos = fp8.decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)       # exact in fp32
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    vals = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(np.inf))])
    assert np.array_equal(fp8.encode(vals.astype(np.float64)), _torch_encode(vals))


def test_ties_to_even_code():
    y = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 0.5 * (2 ** -6 + 9 * 2 ** -9)])
    # 1.0625 between 0x38 (1.0) and 0x39 (1.125) -> 0x38; 1.1875 -> 0x3a (1.25);
    # half the smallest subnormal -> 0; 1.5 subnormal steps -> 0x02;
    # between 2^-6 (0x08) and 2^-6 + 2^-9 (0x09) -> 0x08
    assert fp8.encode(y).tolist() == [0x38, 0x3A, 0x00, 0x02, 0x08]


def test_saturation_nan_and_sign():
    y = np.array([448.0, 449.0, 464.0, 1e30, np.inf, -500.0, -np.inf, np.nan, -np.nan,
                  -0.0, -2.0 ** -11, -1.0])
    assert fp8.encode(y).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0xFF,
                                      0x80, 0x80, 0xB8]


def test_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(fp8.encode(fp8.decode(codes)), codes)


def test_quantize_divides_in_fp32():
    rng = np.random.Generator(np.random.PCG64(11))
    bits = (rng.normal(size=5000).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    for scale in (0.5, 0.0371, 3.3):
        x = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).float()
        y = (x / scale).clamp(-448, 448)                  # torch fp32 division
        assert np.array_equal(fp8.quantize_bf16(bits, scale), _torch_encode(y.numpy()))


def test_planted_ties_away_is_caught():
    def wrong(y):
        pos = fp8.decode(np.arange(0x7F, dtype=np.uint8))
        idx = np.searchsorted(pos, np.abs(y))              # first value >= |y|
        lo = np.clip(idx - 1, 0, 0x7E)
        hi = np.clip(idx, 0, 0x7E)
        pick = np.where(np.abs(y) - pos[lo] < pos[hi] - np.abs(y), lo, hi)
        return pick.astype(np.uint8)
    y = np.array([1.0625, 1.1875])
    assert wrong(y).tolist() != fp8.encode(y).tolist()


@pytest.mark.parametrize("k_scale,v_scale", [(0.75, 0.375), (1.0, 2.0)])
def test_attention_over_quantised_cache(k_scale, v_scale):
    rng = np.random.Generator(np.random.PCG64(12))
    nb, bs, hkv, hq, d = 6, 4, 2, 4, 8
    codes = lambda: rng.integers(0, 0x7F, size=(nb, bs, hkv, d), dtype=np.uint8) | \
        (rng.integers(0, 2, size=(nb, bs, hkv, d), dtype=np.uint8) << 7)
    kc, vc = codes(), codes()
    kc = np.where((kc & 0x7F) > 0x50, kc & 0xBF, kc)        # keep scores moderate
    q = (rng.normal(size=(3, hq, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    table = np.array([[5, 1, 3], [0, 2, 4], [4, 4, 4]], dtype=np.int32)
    lens = np.array([10, 7, 0])
    got, glse = oracle.paged_decode(q, kc, vc, table, lens, 0.3, bs, "bf16",
                                    kv_dtype="e4m3", k_scale=k_scale, v_scale=v_scale)
    # the same attention over the dequantised values, stored exactly as fp32
    kf = (fp8.decode(kc) * k_scale).astype(np.float32).view(np.uint32)
    vf = (fp8.decode(vc) * v_scale).astype(np.float32).view(np.uint32)
    qf = oracle.widen(q, "bf16").astype(np.float32).view(np.uint32)
    want, wlse = oracle.paged_decode(qf, kf, vf, table, lens, 0.3, bs, "f32")
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(glse[:2], wlse[:2], rtol=1e-13)
    assert np.all(np.isneginf(glse[2]))
