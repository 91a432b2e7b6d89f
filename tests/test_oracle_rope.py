"""Pins of the RoPE oracle to closed forms of the rotation (CPU only).

* a quarter turn maps the pair (1, 0) to (0, 1), in both pairings;
* angle 0 is the identity, and dimensions past rotary_dim never change;
* each rotated pair keeps its length;
* with the RoFormer angle table, q.k after rotation depends only on the
  distance between the two positions (the relative-position property the
  pages name);
* the NeoX and GPT-J pairings are the same rotation under a fixed reordering
  of dimensions.
A planted sign error is caught by the length pin.
"""

import numpy as np
import pytest

from oracle.rope import pair_index, rope, standard_table


def _table(angles):
    angles = np.asarray(angles, dtype=np.float64)
    return np.concatenate([np.cos(angles), np.sin(angles)], axis=1)


@pytest.mark.parametrize("neox", [True, False])
def test_quarter_turn(neox):
    x = np.zeros((1, 1, 4))
    first, second = pair_index(4, neox)
    x[0, 0, first[0]] = 1.0
    t = _table([[np.pi / 2, 0.0]])
    y = rope(x, np.array([0]), t, 4, neox)
    assert abs(y[0, 0, first[0]]) < 1e-15 and abs(y[0, 0, second[0]] - 1.0) < 1e-15


@pytest.mark.parametrize("neox", [True, False])
def test_identity_and_pass_through(neox):
    rng = np.random.Generator(np.random.PCG64(1))
    x = rng.normal(size=(5, 3, 16))
    y = rope(x, np.zeros(5, int), _table(np.zeros((1, 4))), 8, neox)
    assert np.array_equal(y, x)
    y = rope(x, rng.integers(0, 7, 5), _table(rng.uniform(-3, 3, (7, 4))), 8, neox)
    assert np.array_equal(y[..., 8:], x[..., 8:])


def _pair_lengths(x, rotary_dim, neox):
    first, second = pair_index(rotary_dim, neox)
    return np.hypot(x[..., first], x[..., second])


@pytest.mark.parametrize("neox", [True, False])
def test_pair_lengths_kept(neox):
    rng = np.random.Generator(np.random.PCG64(2))
    x = rng.normal(size=(6, 4, 64))
    t = _table(rng.uniform(-10, 10, (9, 32)))
    y = rope(x, rng.integers(0, 9, 6), t, 64, neox)
    np.testing.assert_allclose(_pair_lengths(y, 64, neox), _pair_lengths(x, 64, neox),
                               rtol=1e-13)


@pytest.mark.parametrize("neox", [True, False])
def test_relative_position(neox):
    rng = np.random.Generator(np.random.PCG64(3))
    d = 32
    t = standard_table(200, d)
    q = rng.normal(size=(1, 1, d))
    k = rng.normal(size=(1, 1, d))

    def score(m, n):
        return float(np.sum(rope(q, np.array([m]), t, d, neox) *
                            rope(k, np.array([n]), t, d, neox)))
    for m, n in ((10, 3), (57, 57), (4, 90)):
        for shift in (1, 17, 100):
            assert abs(score(m, n) - score(m + shift, n + shift)) < 1e-10
    assert abs(score(10, 3) - score(3, 10)) > 1e-6   # the direction matters


def test_pairings_are_one_rotation():
    rng = np.random.Generator(np.random.PCG64(4))
    d = 16
    x = rng.normal(size=(3, 2, d))
    t = _table(rng.uniform(-3, 3, (5, d // 2)))
    pos = rng.integers(0, 5, 3)
    # NeoX pair (i, i + d/2) sits at GPT-J positions (2i, 2i + 1)
    perm = np.empty(d, int)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    y_neox = rope(x, pos, t, d, True)
    y_gptj = rope(x[..., perm], pos, t, d, False)
    assert np.allclose(y_gptj, y_neox[..., perm], atol=1e-14)


def test_planted_sign_error_is_caught():
    def wrong(x, positions, cos_sin, rotary_dim, neox):
        half = rotary_dim // 2
        first, second = pair_index(rotary_dim, neox)
        out = x.copy()
        c = cos_sin[positions, :half][:, None, :]
        s = cos_sin[positions, half:][:, None, :]
        a, b = x[..., first], x[..., second]
        out[..., first] = a * c - b * s
        out[..., second] = b * c - a * s
        return out
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.normal(size=(4, 2, 8))
    t = _table(rng.uniform(-3, 3, (4, 4)))
    y = wrong(x, np.arange(4), t, 8, True)
    assert not np.allclose(_pair_lengths(y, 8, True), _pair_lengths(x, 8, True))
