"""GPU parity for frame-aligned editing attention: the HIP path through the C ABI against the
fp64 oracle.

Editing model (Vidu S2 paper read, section 2.6; BloomBook Vidu S2 tutorial, section
"S2-Editing"): each target frame reads the source frame of its own instant, the
reference (first block, a sink) and the causal target history; source frames are
consumed with their chunk.  Every chunk and row of small streams (fp32 and bf16, query
tiles and key blocks straddling frame boundaries, split key ranges opening on source
blocks of another frame), all rows of two heads at 540p, the read-back of staged source
frames, and that a commit drops them.
"""
import numpy as np
import pytest

import synth
from oracle import stream as ostream

from .helpers import compare, config_for, to_dev, to_f64, window_len_after

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)


def _run_stream(w, chunks, heads=None, steps=None, check_from=0, rows=None):
    from streaming_block_causal_amd.cache import Cache
    c = Cache(config_for(w), device="cuda")
    st = ostream.Stream(w)
    S, W = w.n_sink, w.n_window
    for n in chunks:
        fn = synth.frames_of(w, n)
        if n >= 1:
            ks, vs = synth.source_kv(w, n)
        for s in (steps or range(1, w.n_steps + 1)):
            q, k, v = synth.qkv(w, n, s)
            c.append("current", to_dev(w, k), to_dev(w, v), n, n_frames=fn)
            if n >= 1 and s == (steps or [1])[0]:
                c.append("source", to_dev(w, ks), to_dev(w, vs), n, n_frames=fn)
            if n < check_from:
                continue
            B = synth.block_shape(w, n)[0]
            lse = torch.empty((w.n_heads, B), dtype=torch.float32, device="cuda")
            out = c.attend(to_dev(w, q), "final" if s == w.n_steps else "intermediate", lse=lse)
            torch.cuda.synchronize()
            got, gl = to_f64(out), to_f64(lse)
            r = np.arange(B) if rows is None else np.asarray([x for x in rows if x < B])
            ref, rl, _ = st.call(n, s, heads=heads, rows=r,
                                 workers=8 if heads is None or len(heads) > 1 else 1)
            if heads is not None:
                got, gl = got[:, heads], gl[heads]
            ok, m = compare(got[r], ref, w.dtype, gl[:, r], rl)
            _say(f"  chunk {n} ({fn} frames, B={B}) step {s}: {m}")
            assert ok, (n, s, m)
        if n >= S and W > 0 and window_len_after(n, S, W) == W:
            c.evict()
        c.append("clean", None, None, n)
        if w.twin:
            kn, vn = synth.noisy_kv(w, n)
            c.append("noisy", to_dev(w, kn), to_dev(w, vn), n, n_frames=fn)
    return c


@pytest.mark.parametrize("policy", ["s1", "relative"])
def test_editing_fp32_full_stream(policy):
    w = synth.tiny(1, n_chunks=8, policy=policy, editing=True, ref_frames=1)
    _say(f"[editing fp32 {policy}] hw={w.lat_h * w.lat_w}")
    _run_stream(w, range(w.n_chunks))


def test_editing_fp32_odd_frames_varlen():
    # 5 x 7 frames: fp32 workgroups of 64 rows and 32-key sub-blocks both straddle frames
    w = synth.tiny(1, n_chunks=8, lat_h=5, lat_w=7, editing=True, ref_frames=2, frame_pattern=(3, 1, 2))
    _say("[editing fp32 5x7 varlen]")
    _run_stream(w, range(w.n_chunks))


def test_editing_bf16_small_stream():
    # 16 x 20 = 320 tokens per frame: 256-row query tiles and 64-key blocks straddle frames, and
    # the few tiles of this shape are cut into key ranges, some opening on another frame's source
    w = synth.tiny(7, name="editing_small_bf16", lat_h=16, lat_w=20, n_heads=4, n_chunks=8, n_steps=2)
    _say(f"[editing bf16 small] hw={w.lat_h * w.lat_w}")
    _run_stream(w, range(w.n_chunks))


def test_editing_bf16_twin_varlen():
    w = synth.tiny(7, name="editing_twin_bf16", lat_h=9, lat_w=13, n_heads=2, n_chunks=9, n_steps=2,
                   twin=True, policy="relative", frame_pattern=(3, 1, 2))
    _say(f"[editing bf16 twin varlen] hw={w.lat_h * w.lat_w}")
    _run_stream(w, range(w.n_chunks))


def test_editing_bf16_frames_shorter_than_a_key_block():
    # 4 x 6 = 24 tokens per frame: one 64-key block holds several frames
    w = synth.tiny(7, name="editing_tiny_bf16", lat_h=4, lat_w=6, n_heads=2, n_chunks=6, n_steps=1)
    _say("[editing bf16 4x6]")
    _run_stream(w, range(w.n_chunks))


def test_editing_540p_steady_state_two_heads():
    w = synth.WORKLOADS[7]
    hw = w.lat_h * w.lat_w
    rows = sorted(set(list(range(0, 48)) + list(range(hw - 40, hw + 40)) + list(range(2 * hw - 40, 2 * hw + 40))
                      + list(range(w.block_tokens - 40, w.block_tokens))))
    _say(f"[c7] {w.name} rows {len(rows)}")
    _run_stream(w, range(8), heads=[0, 17], steps=[w.n_steps], check_from=5, rows=rows)


def test_source_readback_and_commit_drops_it():
    from streaming_block_causal_amd.cache import Cache
    w = synth.tiny(7, name="editing_rb", lat_h=8, lat_w=12, n_heads=2, n_chunks=4, n_steps=1)
    c = Cache(config_for(w), device="cuda")
    plain = Cache(config_for(w.replace(editing=False)), device="cuda")
    for n in range(3):
        fn = synth.frames_of(w, n)
        q, k, v = synth.qkv(w, n, 1)
        for cc in (c, plain):
            cc.append("current", to_dev(w, k), to_dev(w, v), n, n_frames=fn)
        if n == 1:
            # source frames equal to the block's own K/V are stored exactly like it
            c.append("source", to_dev(w, k), to_dev(w, v), n)
            kc, vc = c.read_slot(0, "current")
            ks, vs = c.read_slot(0, "source")
            assert torch.equal(kc, ks) and torch.equal(vc, vs)
        if n == 2:
            # block 1's source was dropped by its commit: no source, the plain result exactly
            assert all(d["role"] != "source" for d in c.inspect())
            o1 = c.attend(to_dev(w, q), "final")
            o2 = plain.attend(to_dev(w, q), "final")
            torch.cuda.synchronize()
            assert torch.equal(o1, o2)
        for cc in (c, plain):
            cc.append("clean", None, None, n)
