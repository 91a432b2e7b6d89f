"""Pins of the oracle's bit widening and of its two remaining scatters (CPU only).

* ``widen`` turns stored bits into float64. It is compared with torch's own
  reinterpretation of the same bits (``Tensor.view(dtype)`` followed by a
  conversion to float64), an implementation that shares nothing with the
  oracle, on every one of the 2^16 bf16 and fp16 codes and on a seeded sample
  of fp32 codes with the special values (zeros, infinities, NaNs,
  subnormals, the extremes). NaN must map to NaN and every other code to the
  same number with the same sign. Planted mistakes (a bf16 shift of 15, fp16
  bits read as bf16, fp32 bits read as integers) fail the comparison.
* ``rope.rope_write_kv`` rotates q and K and scatters the rotated K and the
  raw V bits to ``slot_mapping`` [P2 步骤 3 RoPE; P1 §02 slot_mapping]. A
  hand-built fixture fixes each rule: the slot -> (block, row) split, a
  negative slot writes nothing but still rotates q, a position outside the
  angle table leaves q as it is and writes nothing, every other slot keeps
  its sentinel, and the rotated values are the exact products of the table
  entries (quarter and half turns, a 3-4-5 turn).
* ``fp8.write_kv`` quantises bf16 rows to E4M3 codes of x / scale and
  scatters them [P3 §4.1; P1 §02]. A hand-built fixture with values whose
  quotients are exact E4M3 numbers gives the codes from the format's fields,
  checks the slot split and the skipped negative slot, and that untouched
  slots keep their sentinel.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8
from oracle.rope import rope_write_kv


def _same_numbers(got: np.ndarray, want: np.ndarray) -> bool:
    """NaN where NaN, otherwise equal values with equal sign bits."""
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    if not np.array_equal(nan_g, nan_w):
        return False
    ok = ~nan_w
    return bool(np.array_equal(got[ok], want[ok]) and
                np.array_equal(np.signbit(got[ok]), np.signbit(want[ok])))


def _torch_widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        t = torch.from_numpy(bits.astype(np.uint32).view(np.int32)).view(torch.float32)
    else:
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        t = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(tdt)
    return t.to(torch.float64).numpy()


pytestmark = pytest.mark.filterwarnings("ignore:invalid value encountered in cast:RuntimeWarning")

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_widen_matches_torch_on_every_16_bit_code(dtype):
    got = oracle.widen(ALL16, dtype)
    want = _torch_widen(ALL16, dtype)
    assert got.dtype == np.float64
    assert _same_numbers(got, want)
    # the count of NaN codes the formats fix: exponent all ones, mantissa != 0
    mant_bits = 7 if dtype == "bf16" else 10
    assert int(np.isnan(got).sum()) == 2 * ((1 << mant_bits) - 1)


def test_widen_matches_torch_on_fp32_codes():
    rng = np.random.Generator(np.random.PCG64(77))
    sample = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000,
                        0xFFC00001, 0x7F800001, 0x00000001, 0x80000001, 0x007FFFFF,
                        0x00800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x3F800000, 0xBF800000],
                       dtype=np.uint32)
    bits = np.concatenate([sample, special])
    assert _same_numbers(oracle.widen(bits, "f32"), _torch_widen(bits, "f32"))


def test_widen_known_values():
    # values the formats fix: 1.0, -2.0, the largest finite and -0.0
    assert oracle.widen(np.array([0x3F80, 0xC000, 0x7F7F], np.uint16), "bf16").tolist() == \
        [1.0, -2.0, float(np.float32(3.3895313892515355e38))]
    assert oracle.widen(np.array([0x3C00, 0xC000, 0x7BFF, 0x0001], np.uint16), "f16").tolist() == \
        [1.0, -2.0, 65504.0, 2.0 ** -24]
    z = oracle.widen(np.array([0x8000], np.uint16), "bf16")
    assert z[0] == 0.0 and np.signbit(z[0])


@pytest.mark.parametrize("mistake", ["bf16_shift_15", "f16_as_bf16", "f32_as_int"])
def test_planted_widen_mistakes_are_caught(mistake):
    if mistake == "bf16_shift_15":
        bad = (ALL16.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
        assert not _same_numbers(bad, _torch_widen(ALL16, "bf16"))
    elif mistake == "f16_as_bf16":
        assert not _same_numbers(oracle.widen(ALL16, "bf16"), _torch_widen(ALL16, "f16"))
    else:
        bits = np.arange(1, 1 << 12, dtype=np.uint32) * np.uint32(999_983)
        bad = bits.astype(np.float64)
        assert not _same_numbers(bad, _torch_widen(bits, "f32"))


# --------------------------------------------------------- RoPE write scatter
def _bf16_bits(values) -> np.ndarray:
    """bf16 bits of values that bf16 holds exactly."""
    f = np.asarray(values, dtype=np.float32)
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(oracle.widen(bits, "bf16"), f.astype(np.float64))
    return bits


def test_rope_write_kv_scatter_fixture():
    # 4 tokens, 2 query heads, 1 KV head, head_dim 4 (rotary_dim 4, NeoX pairs
    # (0, 2) and (1, 3)), block_size 2, 3 blocks; angle table of 4 positions:
    # p0 identity, p1 quarter turn, p2 half turn, p3 cos 0.6 / sin 0.8
    cos_sin = np.array([[1.0, 1.0, 0.0, 0.0],
                        [0.0, 0.0, 1.0, 1.0],
                        [-1.0, -1.0, 0.0, 0.0],
                        [0.6, 0.6, 0.8, 0.8]])
    q = np.array([[[1, 2, 3, 4], [5, 6, 7, 8]],
                  [[1, 2, 3, 4], [-1, 0, 2, 0.5]],
                  [[9, 8, 7, 6], [1, 1, 1, 1]],
                  [[1, 0, 0, 1], [2, 2, 2, 2]]], dtype=np.float64)
    k = np.array([[[1, 2, 3, 4]], [[5, 6, 7, 8]], [[-1, -2, 0.5, 0.25]], [[3, 0, 4, 0]]],
                 dtype=np.float64)
    v_vals = np.array([[[10, 11, 12, 13]], [[14, 15, 16, 17]], [[18, 19, 20, 21]],
                       [[22, 23, 24, 25]]], dtype=np.float64)
    q_bits, k_bits, v_bits = _bf16_bits(q), _bf16_bits(k), _bf16_bits(v_vals)
    positions = np.array([2, 1, 7, 3])           # token 2's position is outside the table
    slots = np.array([3, -1, 1, 4], dtype=np.int64)
    sentinel = -123.0
    k_cache = np.full((3, 2, 1, 4), sentinel)
    v_cache = np.full((3, 2, 1, 4), 0xABCD, dtype=np.uint16)
    q_rot, k_rot = rope_write_kv(q_bits, k_bits, v_bits, slots, positions, cos_sin, 4, True,
                                 "bf16", k_cache, v_cache, 2)
    # q: token 0 half turn (every rotated dim negated), token 1 quarter turn
    # (a, b) -> (-b, a) on pairs (0, 2) and (1, 3), token 2 untouched
    # (outside the table), token 3 turned by (0.6, 0.8)
    assert q_rot[0].tolist() == (-q[0]).tolist()
    assert q_rot[1, 0].tolist() == [-3, -4, 1, 2] and q_rot[1, 1].tolist() == [-2, -0.5, -1, 0]
    assert q_rot[2].tolist() == q[2].tolist()
    np.testing.assert_allclose(q_rot[3, 0], [0.6, -0.8, 0.8, 0.6], rtol=0, atol=1e-15)
    np.testing.assert_allclose(q_rot[3, 1], [-0.4, -0.4, 2.8, 2.8], rtol=0, atol=1e-15)
    # slots: 3 -> block 1 row 1 (half turn: K negated); -1 -> nothing; 1
    # (token 2) -> nothing (position outside the table); 4 -> block 2 row 0
    # (pair (3, 4) turned by (0.6, 0.8) -> (-1.4, 4.8))
    assert k_cache[1, 1, 0].tolist() == [-1, -2, -3, -4]
    assert np.array_equal(v_cache[1, 1], v_bits[0])
    np.testing.assert_allclose(k_cache[2, 0, 0], [-1.4, 0, 4.8, 0], rtol=0, atol=1e-15)
    assert np.array_equal(v_cache[2, 0], v_bits[3])
    written = np.zeros((3, 2), dtype=bool)
    written[1, 1] = written[2, 0] = True
    assert np.all(k_cache[~written] == sentinel)
    assert np.all(v_cache[~written] == 0xABCD)
    # the returned K rotation covers every token (written or not)
    assert k_rot[1, 0].tolist() == [-7, -8, 5, 6]


def test_rope_write_kv_gptj_pairs_and_partial_rotary_dim():
    # GPT-J pairs (2i, 2i+1) with rotary_dim 2 of head_dim 4: only dims 0, 1 turn
    cos_sin = np.array([[0.0, 1.0]])               # one position, a quarter turn
    k = np.array([[[1, 2, 3, 4]]], dtype=np.float64)
    bits = _bf16_bits(k)
    k_cache = np.zeros((1, 16, 1, 4))
    v_cache = np.zeros((1, 16, 1, 4), dtype=np.uint16)
    q_rot, _ = rope_write_kv(bits, bits, bits, np.array([5]), np.array([0]), cos_sin, 2, False,
                             "bf16", k_cache, v_cache, 16)
    assert q_rot[0, 0].tolist() == [-2, 1, 3, 4]
    assert k_cache[0, 5, 0].tolist() == [-2, 1, 3, 4]
    assert np.array_equal(v_cache[0, 5], bits[0])


# ----------------------------------------------------------- E4M3 write scatter
def test_fp8_write_kv_scatter_fixture():
    # scale 0.5: x / 0.5 = 2x, chosen so every quotient is an E4M3 value;
    # codes from the fields (sign, exponent e with bias 7, mantissa m):
    #   1.0  -> 2.0  = 1.0 * 2^1      -> e 8,  m 0 -> 0x40
    #  -0.75 -> -1.5 = 1.5 * 2^0      -> e 7,  m 4 -> 0xBC
    #   0.0  -> 0                              -> 0x00
    #   224  -> 448  = 1.75 * 2^8     -> e 15, m 6 -> 0x7E
    #   2^-10 -> 2^-9 (smallest subnormal, m 1)    -> 0x01
    #  -3.25 -> -6.5 = 1.625 * 2^2    -> e 9,  m 5 -> 0xCD
    k_vals = np.array([[[1.0, -0.75, 0.0]], [[224.0, 2.0 ** -10, -3.25]], [[1, 1, 1]]])
    v_vals = np.array([[[-3.25, 224.0, 1.0]], [[0.0, -0.75, 2.0 ** -10]], [[1, 1, 1]]])
    kb, vb = _bf16_bits(k_vals), _bf16_bits(v_vals)
    k_cache = np.full((2, 4, 1, 3), 0x55, dtype=np.uint8)
    v_cache = np.full((2, 4, 1, 3), 0x55, dtype=np.uint8)
    slots = np.array([6, 1, -5], dtype=np.int64)     # block 1 row 2, block 0 row 1, skipped
    fp8.write_kv(k_cache, v_cache, kb, vb, slots, 4, 0.5, 0.5)
    assert k_cache[1, 2, 0].tolist() == [0x40, 0xBC, 0x00]
    assert v_cache[1, 2, 0].tolist() == [0xCD, 0x7E, 0x40]
    assert k_cache[0, 1, 0].tolist() == [0x7E, 0x01, 0xCD]
    assert v_cache[0, 1, 0].tolist() == [0x00, 0xBC, 0x01]
    written = np.zeros((2, 4), dtype=bool)
    written[1, 2] = written[0, 1] = True
    assert np.all(k_cache[~written] == 0x55) and np.all(v_cache[~written] == 0x55)
    # the codes decode back to the quotients
    assert fp8.decode(k_cache[1, 2, 0]).tolist() == [2.0, -1.5, 0.0]
