"""Pins of the oracle for variable-length blocks (CPU only).

"Vidu S2 vs PixVerse R2" blog, section "Choice 5: how people control it": in R2
the length of a block follows the active control signal, up to a cap (short
blocks for a key press, longer ones for an event or an audio segment).  Section
"Choice 3: bounded memory": positions stay in the trained range (relative-time
RoPE for R2).  Readings: the sink and window sizes still count blocks; a slot
starts where the previous one in [sinks, window, current] ends; relative time
puts the window from 0 and the sinks just before it.

Pinned against the brute-force full-stream attention (explicit block mask,
positions from the visible layout, complex RoPE, torch SDPA), against the
fixed-length formulas they must reduce to, and against hand-worked bases.
"""
import numpy as np
import pytest

import synth
from oracle import bruteforce, rope, stream

VAR = synth.tiny(1, n_heads=2, lat_h=4, lat_w=6, n_chunks=9, frame_pattern=(3, 1, 2, 1, 3, 2))


def test_bases_reduce_to_fixed_length():
    for policy in ("s1", "relative"):
        for S, W, F in ((1, 2, 3), (2, 3, 1), (0, 4, 2), (3, 0, 3)):
            assert rope.relocation_bases_frames(policy, [F] * S, [F] * W, F) == \
                rope.relocation_bases(policy, S, W, F)


def test_bases_worked_example():
    # sinks [3 frames], window [1, 2, 3] oldest -> newest, current 2 frames
    assert rope.relocation_bases_frames("s1", [3], [1, 2, 3], 2) == [0, 3, 4, 6, 9]
    assert rope.relocation_bases_frames("relative", [3], [1, 2, 3], 2) == [-3, 0, 1, 3, 6]
    assert rope.relocation_bases_frames("relative", [], [2], 1) == [0, 2]


def test_frames_of_pattern_and_cap():
    assert [synth.frames_of(VAR, b) for b in range(8)] == [3, 1, 2, 1, 3, 2, 3, 1]
    assert synth.block_shape(VAR, 1) == (24, 2, 64)
    with pytest.raises(ValueError):
        synth.frames_of(VAR.replace(frame_pattern=(4,)), 0)


@pytest.mark.parametrize("policy", ["s1", "relative"])
def test_varlen_stream_equals_bruteforce(policy):
    w = VAR.replace(policy=policy)
    st = stream.Stream(w)
    for n in range(w.n_chunks):
        o, lse, _ = st.call(n, 1)
        ob, lb = bruteforce.chunk(w, n, 1)
        assert o.shape[0] == synth.block_shape(w, n)[0]
        np.testing.assert_allclose(o, ob, atol=1e-12, err_msg=f"chunk {n}")
        np.testing.assert_allclose(lse, lb, atol=1e-12, err_msg=f"chunk {n}")


def test_varlen_twin_and_window_variants_equal_bruteforce():
    for kw in (dict(n_sink=2, n_window=1), dict(twin=True, n_steps=2, dtype="bf16", scale=0.5)):
        w = VAR.replace(**kw)
        st = stream.Stream(w)
        for n in range(w.n_chunks):
            for s in range(1, w.n_steps + 1):
                o, lse, _ = st.call(n, s)
                ob, lb = bruteforce.chunk(w, n, s)
                np.testing.assert_allclose(o, ob, atol=1e-12, err_msg=f"{kw} chunk {n} step {s}")


def test_constant_pattern_is_the_fixed_length_stream():
    w = VAR.replace(frame_pattern=None)
    wc = VAR.replace(frame_pattern=(3,))
    a, b = stream.Stream(w), stream.Stream(wc)
    for n in (0, 3, 8):
        oa, la, _ = a.call(n, 1)
        ob, lb, _ = b.call(n, 1)
        assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_relative_and_s1_agree_on_varlen():
    a = stream.Stream(VAR)
    b = stream.Stream(VAR.replace(policy="relative"))
    for n in range(VAR.n_chunks):
        oa, la, _ = a.call(n, 1)
        ob, lb, _ = b.call(n, 1)
        np.testing.assert_allclose(oa, ob, atol=1e-12)
        np.testing.assert_allclose(la, lb, atol=1e-12)


def test_cap_spaced_bases_fail_the_pin(monkeypatch):
    """Placing slots at multiples of the cap (ignoring the real block lengths) is caught."""
    def wrong(policy, sink_frames, window_frames, current_frames):
        n = len(sink_frames) + len(window_frames) + 1
        return [l * VAR.frames for l in range(n)]
    monkeypatch.setattr(rope, "relocation_bases_frames", wrong)
    st = stream.Stream(VAR)
    bad = False
    for n in range(VAR.n_chunks):
        o, _, _ = st.call(n, 1)
        ob, _ = bruteforce.chunk(VAR, n, 1)
        bad |= not np.allclose(o, ob, atol=1e-6)
    assert bad
