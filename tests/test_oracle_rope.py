"""Pins of the oracle's 3D RoPE and relocation (CPU only).

RoPE: Vidu S2 paper read, abbreviation table (RoPE: rotary positions over
space and time).  Relocation: "Vidu S2 vs PixVerse R2" blog, section "Choice 3:
bounded memory" (positions kept inside the trained range).  The split over
(t, h, w), pairing and frequencies are the stated reading of the oracle; the
worked example under tests/golden/ fixes them by hand.
"""
import math

import numpy as np
import pytest

from oracle import rope

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def test_axis_split_and_frequencies():
    assert rope.axis_split(128) == (22, 21, 21)
    assert rope.axis_split(64) == (12, 10, 10)
    assert rope.axis_split(6) == (1, 1, 1)
    np.testing.assert_allclose(rope.axis_frequencies(4, 10000.0), [1.0, 0.1, 0.01, 0.001], rtol=1e-15)


def _load_golden(name):
    rows = []
    for line in open(f"{GOLDEN}/{name}"):
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append([float(v) for v in line.split()])
    return [np.array(r) for r in rows]


def test_worked_example_d6():
    """d=6: one pair per axis, every frequency 1, so each pair turns by its raw coordinate."""
    g = _load_golden("rope_d6_worked_example.txt")
    x, pos, expected = g[0], g[1], g[2]
    got = rope.rotate(x, rope.angles(pos[0], pos[1], pos[2], 6))
    np.testing.assert_allclose(got, expected, atol=1e-15)


def test_worked_example_d12_frequencies():
    """d=12: two pairs per axis with omega = (1, theta^-1/2) = (1, 0.01)."""
    g = _load_golden("rope_d12_worked_example.txt")
    x, pos, expected = g[0], g[1], g[2]
    got = rope.rotate(x, rope.angles(pos[0], pos[1], pos[2], 12))
    np.testing.assert_allclose(got, expected, atol=1e-15)


def test_norm_identity_composition_relative():
    rng = np.random.default_rng(1)
    d = 128
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    a = np.array([7.0, 11.0, 23.0])
    b = np.array([2.0, 30.0, 5.0])
    ra = rope.angles(*a, d)
    rb = rope.angles(*b, d)
    # norm preserved, identity at the origin
    assert abs(np.linalg.norm(rope.rotate(q, ra)) - np.linalg.norm(q)) < 1e-12
    np.testing.assert_array_equal(rope.rotate(q, rope.angles(0, 0, 0, d)), q)
    # composition R(a) R(b) = R(a + b)
    np.testing.assert_allclose(rope.rotate(rope.rotate(q, ra), rb), rope.rotate(q, rope.angles(*(a + b), d)),
                               atol=1e-12)
    # relative: <R(a) q, R(b) k> = <q, R(b - a) k>
    lhs = rope.rotate(q, ra) @ rope.rotate(k, rb)
    rhs = q @ rope.rotate(k, rope.angles(*(b - a), d))
    assert abs(lhs - rhs) < 1e-12


def test_axes_touch_only_their_pairs():
    d = 128
    pt, ph, pw = rope.axis_split(d)
    x = np.arange(d, dtype=np.float64) + 1.0
    base = rope.rotate(x, rope.angles(3, 4, 5, d))
    for axis, (lo, hi) in enumerate([(0, 2 * pt), (2 * pt, 2 * (pt + ph)), (2 * (pt + ph), d)]):
        pos = [3, 4, 5]
        pos[axis] += 9
        moved = rope.rotate(x, rope.angles(*pos, d))
        changed = np.nonzero(np.abs(moved - base) > 1e-12)[0]
        assert changed.min() >= lo and changed.max() < hi


def test_block_grid_order():
    f, h, w = rope.block_grid(3, 2, 4)
    assert list(f[:9]) == [0, 0, 0, 0, 0, 0, 0, 0, 1]
    assert list(h[:5]) == [0, 0, 0, 0, 1]
    assert list(w[:5]) == [0, 1, 2, 3, 0]


@pytest.mark.parametrize("S,W,F", [(1, 3, 3), (2, 2, 3), (0, 4, 2), (3, 0, 1)])
def test_relocation_closed_forms(S, W, F):
    for n_s in range(S + 1):
        for n_w in range(W + 1):
            s1 = rope.relocation_bases("s1", n_s, n_w, F)
            rel = rope.relocation_bases("relative", n_s, n_w, F)
            assert s1 == [F * l for l in range(n_s + n_w + 1)]
            # relative-time = the S1 layout shifted so the window starts at 0
            assert rel == [b - n_s * F for b in s1]
            assert rel[n_s:n_s + n_w] == [F * j for j in range(n_w)]
            # positions stay bounded however long the stream is
            assert all(-S * F <= t < (S + W + 1) * F for t in s1 + rel)
    with pytest.raises(ValueError):
        rope.relocation_bases("absolute", 1, 1, F)


def test_worked_example_custom_split():
    """A caller-given split (2, 0, 2) at d = 8, theta = 100: no pair follows the row."""
    g = _load_golden("rope_d8_custom_split.txt")
    x, pos, expected, params = g[0], g[1], g[2], g[3]
    theta, split = params[0], tuple(int(v) for v in params[1:])
    got = rope.rotate(x, rope.angles(pos[0], pos[1], pos[2], 8, theta, split))
    np.testing.assert_allclose(got, expected, atol=1e-15)
    assert rope.axis_split(8, split) == (2, 0, 2)
    with pytest.raises(ValueError):
        rope.axis_split(8, (2, 1, 2))      # does not cover the 4 pairs
