"""Pins of the oracle's fp8 attention (CPU only).

Scheme (an own design for CDNA4's scaled fp8 matrix instructions; the pages only say
that quantised attention is chosen per layer -- Vidu S2 paper read, section 2.4):
OCP E4M3 elements, round to nearest even; power-of-two scales per group of 32 values,
e = ceil(log2(amax / 448)); K groups = 32 channels of a key after block-local RoPE, V
groups = the first and the last 32 keys of a 64-key block, per channel; Q groups =
32 channels of a query after its rotation for each slot.

Pinned against torch's float8_e4m3fn conversion (a library routine), closed forms of
the scale exponent, structural properties of the groups, and the exact fp64 oracle
(the fp8 oracle must reduce to it when element rounding is switched off).
"""
import numpy as np
import pytest
import torch

import synth
from oracle import fp8
from oracle import stream as ostream


def test_e4m3_round_matches_torch():
    rng = np.random.default_rng(0)
    mant = rng.integers(0, 1 << 12, 20000)
    ex = rng.integers(-13, 9, 20000)
    x = np.ldexp(1.0 + mant / 4096.0, ex) * np.where(rng.random(20000) < 0.5, -1, 1)
    # exact midpoints between neighbouring codes, subnormals, the top of the range
    codes = np.arange(0, 127, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, vals, mids, -mids, [0.0, 2.0 ** -10, 3 * 2.0 ** -11, 440.0, 447.5, 448.0]])
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.all(x.astype(np.float32) == x)            # the inputs are exact in fp32
    np.testing.assert_array_equal(fp8.e4m3_round(x), ref)


def test_scale_exponent_closed_form():
    for e in (-20, -3, 0, 5, 40):
        top = 448.0 * 2.0 ** e
        assert fp8.e8m0_exponent(top) == e                 # exactly at the limit
        assert fp8.e8m0_exponent(top * (1 + 2.0 ** -30)) == e + 1
        assert fp8.e8m0_exponent(top / 2 * (1 + 2.0 ** -30)) == e   # just above half the limit
        assert fp8.e8m0_exponent(top / 2) == e - 1
    assert fp8.e8m0_exponent(0.0) == -127
    assert fp8.e8m0_exponent(1e-300) == -127               # clipped
    assert fp8.e8m0_exponent(1e300) == 127


def test_group_scales_are_tight_and_idempotent():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 128)) * np.exp(rng.uniform(-8, 8, (50, 1)))
    y = fp8.quantize_groups(x)
    g = x.reshape(50, 4, 32)
    e = fp8.e8m0_exponent(np.abs(g).max(axis=-1))
    scaled = np.abs(g).max(axis=-1) / np.ldexp(1.0, e)
    assert np.all(scaled <= 448.0) and np.all(scaled > 224.0)
    np.testing.assert_array_equal(fp8.quantize_groups(y), y)
    # element error within half an E4M3 step of the group's scale (3 mantissa bits)
    assert np.all(np.abs(y - x) <= np.maximum(np.abs(x) * 2.0 ** -4, np.ldexp(2.0 ** -10, e).repeat(32, axis=1)))


def test_v_groups_are_block_halves():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((100, 3)) * 0.01                # a full block and a short one
    base = fp8.quantize_v(v)
    big = v.copy()
    big[40, 1] = 50.0                                      # key 40: second half of block 0
    q = fp8.quantize_v(big)
    grp = np.zeros(100, dtype=bool)
    grp[32:64] = True
    assert np.array_equal(q[~grp], base[~grp])             # other groups are untouched
    assert np.array_equal(q[:, [0, 2]], base[:, [0, 2]])   # other channels untouched
    assert not np.array_equal(q[grp, 1], base[grp, 1])     # its own group lost precision
    assert np.array_equal(fp8.quantize_v(v[64:]), base[64:])   # blocks are independent


W = synth.tiny(8, name="fp8_tiny", n_heads=2, lat_h=6, lat_w=10, n_chunks=6)


def test_reduces_to_exact_attention_without_element_rounding(monkeypatch):
    exact = ostream.Stream(W.replace(attn_fp8=False))
    monkeypatch.setattr(fp8, "e4m3_round", lambda x: np.asarray(x, dtype=np.float64))
    q8 = ostream.Stream(W)
    for n in (0, 2, 5):
        o8, l8, _ = q8.call(n, 1)
        oe, le, _ = exact.call(n, 1)
        np.testing.assert_allclose(o8, oe, atol=1e-12)
        np.testing.assert_allclose(l8, le, atol=1e-12)


def test_fp8_close_to_exact_but_not_equal():
    exact = ostream.Stream(W.replace(attn_fp8=False))
    q8 = ostream.Stream(W)
    for n in (3, 5):
        o8, l8, _ = q8.call(n, 1)
        oe, le, _ = exact.call(n, 1)
        rel = np.linalg.norm(o8 - oe) / np.linalg.norm(oe)
        assert 1e-4 < rel < 3e-2, rel
        assert np.abs(l8 - le).max() < 2e-2


@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_planted_unquantised_operand_fails(monkeypatch, which):
    """Leaving out the quantisation of any one operand changes the result (each step is there)."""
    from oracle import rope
    o_ref, _, _ = ostream.Stream(W).call(4, 1)

    def rotated(w, stored, head, delta, as_f64):
        x = as_f64(w, stored[:, head, :])
        f, hh, ww = rope.block_grid(stored.shape[0] // (w.lat_h * w.lat_w), w.lat_h, w.lat_w)
        return rope.rotate(x, rope.angles(f + delta, hh, ww, w.head_dim, w.rope_theta))

    if which == "q":   # rotated and scaled, not quantised
        monkeypatch.setattr(fp8, "query_for_slot",
                            lambda w, q, h, d, as_f64: rotated(w, q, h, d, as_f64) * fp8.score_scale(w))
    elif which == "k":
        monkeypatch.setattr(fp8, "key_local", lambda w, k, h, as_f64: rotated(w, k, h, 0, as_f64))
    else:
        monkeypatch.setattr(fp8, "quantize_v", lambda v: np.asarray(v, dtype=np.float64))
    o_bad, _, _ = ostream.Stream(W).call(4, 1)
    assert not np.allclose(o_bad, o_ref, atol=1e-9)


def _plain_fp8(x):
    """The plain definition of fp8 attention operands: the whole tensor scaled by amax / 448 and
    rounded to E4M3 by torch's float8_e4m3fn conversion (a library routine), read back."""
    s = np.abs(x).max() / 448.0
    return torch.from_numpy((x / s).astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy() * s


def test_scheme_agrees_with_plain_per_tensor_fp8():
    """Against an fp8 attention written from the plain definition -- Q rotated at its relocated
    positions, K at its slot's relocated positions and V, each quantised with one scale per head
    -- the oracle's scheme (K quantised at block-local positions, Q per slot, 32-value groups) is
    no less accurate, and the two differ by about their independent rounding errors added in
    quadrature (E4M3 keeps 3 mantissa bits: about 3% relative error on the output here)."""
    exact = ostream.Stream(W.replace(attn_fp8=False))
    q8 = ostream.Stream(W)
    for n in (2, 5):
        o8, _, _ = q8.call(n, 1)
        oe, _, _ = exact.call(n, 1)
        q, slots = exact.slot_inputs(n, 1)
        bases = exact.bases(n)
        op = np.empty_like(oe)
        for h in range(W.n_heads):
            qr = _plain_fp8(ostream.relocated_head(W, q, h, bases[-1]))
            kr = _plain_fp8(np.concatenate([ostream.relocated_head(W, k, h, bases[l])
                                            for l, (_, _, k, _) in enumerate(slots)]))
            vr = _plain_fp8(np.concatenate([synth.as_f64(W, v[:, h, :]) for (_, _, _, v) in slots]))
            sc = qr @ kr.T / np.sqrt(W.head_dim)
            e = np.exp(sc - sc.max(axis=1, keepdims=True))
            op[:, h] = (e @ vr) / e.sum(axis=1, keepdims=True)

        def rel(a, b):
            return np.linalg.norm(a - b) / np.linalg.norm(b)
        e_or, e_pl, d = rel(o8, oe), rel(op, oe), rel(o8, op)
        assert 1e-3 < e_pl < 5e-2, e_pl
        assert e_or <= 1.25 * e_pl, (e_or, e_pl)
        assert d <= 1.6 * max(e_or, e_pl), (d, e_or, e_pl)
