"""Pins of the oracle for frame-aligned editing attention (CPU only).

Vidu S2 paper read, section 2.6 (the editing model): source video and reference
image enter as condition tokens; each generated frame exchanges information only
with the source frame of the same instant, the reference is visible to all
frames, and source frames are consumed with their target frame, never cached.
BloomBook Vidu S2 tutorial, section "S2-Editing": the same, with the causal
history of target frames in the figure.  Readings: the reference is block 0 of
the stream, kept as a sink; the source frame of instant t has the (t, h, w)
positions of target frame t.

Pinned against the brute-force stream (every arrived source frame laid out, a
same-instant predicate on global frame indices, complex RoPE, torch SDPA), the
cross-instant independence the pages state, and planted mistakes.
"""
import numpy as np
import pytest

import synth
from oracle import bruteforce, stream

ED = synth.tiny(1, n_heads=2, lat_h=3, lat_w=5, n_chunks=7, editing=True, ref_frames=1)   # F = 3


def _check_stream(w, chunks=None, steps=None):
    st = stream.Stream(w)
    for n in (range(w.n_chunks) if chunks is None else chunks):
        for s in (range(1, w.n_steps + 1) if steps is None else steps):
            o, lse, _ = st.call(n, s)
            ob, lb = bruteforce.chunk(w, n, s)
            np.testing.assert_allclose(o, ob, atol=1e-12, err_msg=f"{w.name} chunk {n} step {s}")
            np.testing.assert_allclose(lse, lb, atol=1e-12, err_msg=f"{w.name} chunk {n} step {s}")


@pytest.mark.parametrize("policy", ["s1", "relative"])
def test_editing_stream_equals_bruteforce(policy):
    _check_stream(ED.replace(policy=policy))


def test_editing_variants_equal_bruteforce():
    for kw in (dict(n_sink=2, n_window=1), dict(n_window=0), dict(frame_pattern=(3, 1, 2, 3, 1)),
               dict(twin=True, n_steps=2, dtype="bf16", scale=0.5), dict(ref_frames=2)):
        _check_stream(ED.replace(**kw, name=f"ed{sorted(kw)}"))


def test_reference_block_has_one_frame_and_no_source():
    assert synth.block_shape(ED, 0) == (15, 2, 64)
    assert synth.block_shape(ED, 1) == (45, 2, 64)
    with pytest.raises(ValueError):
        synth.source_kv(ED, 0)
    # chunk 0 (the reference itself) is plain block-causal attention
    plain = ED.replace(editing=False, frame_pattern=(1, 3))
    a, _, _ = stream.Stream(ED).call(0, 1)
    b, _, _ = stream.Stream(plain).call(0, 1)
    np.testing.assert_array_equal(a, b)


def test_no_cross_instant_mixing():
    """Changing source frame j of chunk n changes exactly the rows of target frame j."""
    n, hw = 3, ED.lat_h * ED.lat_w
    base = stream.Stream(ED)
    o0, _, _ = base.call(n, 1)
    ks, vs = synth.source_kv(ED, n)
    for j in range(ED.frames):
        ks2, vs2 = ks.copy(), vs.copy()
        ks2[j * hw:(j + 1) * hw] = synth.draw(ED, 99, 0, synth.TAG_KS)[j * hw:(j + 1) * hw]
        vs2[j * hw:(j + 1) * hw] = synth.draw(ED, 99, 0, synth.TAG_VS)[j * hw:(j + 1) * hw]
        st = stream.Stream(ED, contents=lambda b, kind: (ks2, vs2) if (b, kind) == (n, "source") else None)
        o1, _, _ = st.call(n, 1)
        frame_of_row = np.arange(o0.shape[0]) // hw
        changed = np.any(o1 != o0, axis=(1, 2))
        assert np.array_equal(changed, frame_of_row == j), j


def test_source_is_consumed_with_its_chunk():
    """A chunk's output does not depend on the source frames of earlier chunks."""
    n = 4
    st0 = stream.Stream(ED)
    o0, l0, _ = st0.call(n, 1)
    other = synth.source_kv(ED, 1)
    st1 = stream.Stream(ED, contents=lambda b, kind: other if (kind == "source" and b < n) else None)
    o1, l1, _ = st1.call(n, 1)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)


def test_one_frame_blocks_see_the_whole_source_block():
    """With one frame per block, frame alignment is the whole source block: dropping the mask
    must not change anything (the mask reduces to no mask)."""
    w = ED.replace(frames=1)
    a, la, _ = stream.Stream(w).call(3, 1)
    orig = stream._frame_aligned
    try:
        stream._frame_aligned = lambda w_, rows, lengths: np.ones((len(rows), sum(lengths)), dtype=bool)
        b, lb, _ = stream.Stream(w).call(3, 1)
    finally:
        stream._frame_aligned = orig
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def _fails_bruteforce(monkeypatch, target, attr, wrong):
    monkeypatch.setattr(target, attr, wrong)
    st = stream.Stream(ED)
    bad = False
    for n in (1, 3, 5):
        o, _, _ = st.call(n, 1)
        ob, _ = bruteforce.chunk(ED, n, 1)
        bad |= not np.allclose(o, ob, atol=1e-6)
    return bad


def test_planted_whole_source_visible_fails(monkeypatch):
    wrong = lambda w, rows, lengths: np.ones((len(rows), sum(lengths)), dtype=bool)
    assert _fails_bruteforce(monkeypatch, stream, "_frame_aligned", wrong)


def test_planted_shifted_source_positions_fail(monkeypatch):
    orig = stream.relocated_head
    calls = {"n": 0}

    def shifted(w, stored, head, base):
        # the source is the last slot: shift its time base by one frame
        calls["n"] += 1
        return orig(w, stored, head, base + (1 if stored is calls.get("src") else 0))

    orig_source = stream.Stream.source

    def source(self, n):
        kv = orig_source(self, n)
        calls["src"] = kv[0]
        return kv

    monkeypatch.setattr(stream.Stream, "source", source)
    assert _fails_bruteforce(monkeypatch, stream, "relocated_head", shifted)
    assert calls["n"] > 0


def test_planted_previous_frame_alignment_fails(monkeypatch):
    """Aligning each query with the source frame one instant earlier is caught."""
    def wrong(w, rows, lengths):
        hw = w.lat_h * w.lat_w
        rows = np.asarray(rows)
        n_other = sum(lengths[:-1])
        vis = np.ones((rows.size, n_other + lengths[-1]), dtype=bool)
        vis[:, n_other:] = (rows // hw - 1)[:, None] == (np.arange(lengths[-1]) // hw)[None, :]
        vis[rows // hw == 0, n_other:] = False
        return vis
    assert _fails_bruteforce(monkeypatch, stream, "_frame_aligned", wrong)
