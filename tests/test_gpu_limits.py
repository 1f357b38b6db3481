"""GPU parity at the library's limits: the largest slot count (S + W + 1 = 16) and the largest
block (65536 tokens), against the fp64 oracle.

Cache model: "Vidu S2 vs PixVerse R2" blog, section "Choice 3: bounded memory" (sinks plus a
sliding window).  The limits are the library's (include/swattn.h): n_sink + n_window + 1 <= 16
slots (n_sink + n_window + 2 with editing), and F * lat_h * lat_w <= 65536 tokens per block.
"""
import numpy as np
import pytest

import synth
from oracle import stream as ostream

from .helpers import commit_block, compare, config_for, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)


def _stream(w, check, rows=None, heads=None):
    from streaming_block_causal_amd.cache import Cache
    c = Cache(config_for(w), device="cuda")
    st = ostream.Stream(w)
    for n in range(w.n_chunks):
        fn = synth.frames_of(w, n)
        q, k, v = synth.qkv(w, n, w.n_steps)
        c.append("current", to_dev(w, k), to_dev(w, v), n, n_frames=fn)
        if n in check:
            B = synth.block_shape(w, n)[0]
            lse = torch.empty((w.n_heads, B), dtype=torch.float32, device="cuda")
            out = c.attend(to_dev(w, q), "final", lse=lse)
            torch.cuda.synchronize()
            r = np.arange(B) if rows is None else np.asarray(rows)
            ref, rl, _ = st.call(n, w.n_steps, rows=r, heads=heads, workers=8)
            got, gl = to_f64(out)[r], to_f64(lse)[:, r]
            if heads is not None:
                got, gl = got[:, heads], gl[heads]
            ok, m = compare(got, ref, "fp8" if w.attn_fp8 else w.dtype, gl, rl)
            _say(f"  chunk {n}: {m}")
            assert ok, (n, m)
        commit_block(c, w, n, n)
    return c


@pytest.mark.parametrize("base", [1, 2, 8])
def test_sixteen_slots(base):
    """One sink and a 14-block window: every attention call sees 16 slots once the window is full."""
    w = synth.tiny(base, name="limit_slots", frames=1, lat_h=8, lat_w=10, n_heads=2, n_sink=1, n_window=14,
                   n_chunks=19, n_steps=1, **({} if base == 1 else {"head_dim": 128}))
    _say(f"[16 slots, {w.dtype}{' fp8' if w.attn_fp8 else ''}]")
    c = _stream(w, check={3, 15, 16, 18})
    assert len(c.inspect()) == 15            # after the last commit: the sink and a full window


def test_editing_sixteen_slots():
    """Editing caches hold one slot less: sink + 13 window blocks + current + the source frames."""
    w = synth.tiny(7, name="limit_edit", frames=2, lat_h=6, lat_w=10, n_heads=2, n_sink=1, n_window=13,
                   n_chunks=17, n_steps=1, ref_frames=1)
    _say("[editing, 16 slots]")
    from streaming_block_causal_amd.cache import Cache
    c = Cache(config_for(w), device="cuda")
    st = ostream.Stream(w)
    for n in range(w.n_chunks):
        fn = synth.frames_of(w, n)
        q, k, v = synth.qkv(w, n, 1)
        c.append("current", to_dev(w, k), to_dev(w, v), n, n_frames=fn)
        if n >= 1:
            ks, vs = synth.source_kv(w, n)
            c.append("source", to_dev(w, ks), to_dev(w, vs), n, n_frames=fn)
        if n >= 15:
            assert len(c.inspect()) == 16
            B = synth.block_shape(w, n)[0]
            lse = torch.empty((w.n_heads, B), dtype=torch.float32, device="cuda")
            out = c.attend(to_dev(w, q), "final", lse=lse)
            torch.cuda.synchronize()
            ref, rl, _ = st.call(n, 1)
            ok, m = compare(to_f64(out), ref, w.dtype, to_f64(lse), rl)
            _say(f"  chunk {n}: {m}")
            assert ok, (n, m)
        commit_block(c, w, n, n)


def test_largest_block():
    """A 65536-token block (one 256 x 256 frame), sink + one window block: 196608 keys per query."""
    w = synth.tiny(2, name="limit_block", frames=1, lat_h=256, lat_w=256, n_heads=1, n_sink=1, n_window=1,
                   n_chunks=3, n_steps=1)
    assert w.block_tokens == 65536
    _say("[65536-token blocks]")
    B = w.block_tokens
    rows = list(range(0, 40)) + list(range(B // 2 - 20, B // 2 + 20)) + list(range(B - 40, B))
    _stream(w, check={2}, rows=rows)
