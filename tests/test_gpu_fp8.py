"""GPU parity for fp8 attention: the HIP path through the C ABI against the fp64 oracle of the
same scheme (E4M3 values, power-of-two scales per 32 values; quantised attention chosen per
layer -- Vidu S2 paper read, section 2.4).

The stored K (after block-local RoPE) and V are compared with the oracle's quantisation value
by value; the attention output with the oracle's fp8 attention, whose only difference from the
kernel is the E4M3 rounding of the probabilities (the fp8 tolerance in helpers.py).
"""
import numpy as np
import pytest

import synth
from oracle import fp8 as ofp8
from oracle import stream as ostream

from .helpers import advance, commit_block, compare, config_for, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)


def _quant_check(got, ref, label):
    """Equal except where fp32 vs fp64 rounding of the pre-quantisation value crosses a rounding
    boundary: at most 1 in 1000 values, each within one E4M3 step (2^-3 relative)."""
    diff = np.abs(got - ref)
    bad = diff > 0
    n_bad = int(bad.sum())
    _say(f"  {label}: {n_bad} of {got.size} values differ")
    assert n_bad <= max(1, got.size // 1000), (label, n_bad)
    assert np.all(diff[bad] <= 2.0 ** -3 * np.maximum(np.abs(ref[bad]), np.abs(got[bad])) + 1e-30), label


def test_fp8_quantised_cache_matches_oracle():
    from streaming_block_causal_amd.cache import Cache
    w = synth.tiny(8, name="fp8_q", lat_h=16, lat_w=20, n_heads=4, n_chunks=3)
    c = Cache(config_for(w), device="cuda")
    q, k, v = synth.qkv(w, 0, 1)
    c.append("current", to_dev(w, k), to_dev(w, v), 0)
    kc, vc = c.read_slot(0, "current")
    torch.cuda.synchronize()
    kc, vc = to_f64(kc), to_f64(vc)
    for h in range(w.n_heads):
        _quant_check(kc[:, h], ofp8.key_local(w, k, h, synth.as_f64), f"K head {h}")
        _quant_check(vc[:, h], ofp8.quantize_v(synth.as_f64(w, v[:, h, :])), f"V head {h}")


def _run(w, chunks, heads=None, rows=None, steps=(1,), check_from=0):
    """The last of `steps` must be the final step: its K/V are what the commit keeps."""
    assert steps[-1] == w.n_steps
    from streaming_block_causal_amd.cache import Cache
    c = Cache(config_for(w), device="cuda")
    st = ostream.Stream(w)
    for n in chunks:
        for s in steps:
            q, k, v = synth.qkv(w, n, s)
            c.append("current", to_dev(w, k), to_dev(w, v), n)
            if n < check_from:
                continue
            lse = torch.empty((w.n_heads, w.block_tokens), dtype=torch.float32, device="cuda")
            out = c.attend(to_dev(w, q), "final" if s == w.n_steps else "intermediate", lse=lse)
            torch.cuda.synchronize()
            r = np.arange(w.block_tokens) if rows is None else np.asarray(rows)
            ref, rl, _ = st.call(n, s, heads=heads, rows=r, workers=8)
            got, gl = to_f64(out), to_f64(lse)
            if heads is not None:
                got, gl = got[:, heads], gl[heads]
            ok, m = compare(got[r], ref, "fp8", gl[:, r], rl)
            _say(f"  chunk {n} step {s}: {m}")
            assert ok, (n, s, m)
        commit_block(c, w, n, n)


def test_fp8_small_stream_all_rows():
    # 320 tokens per frame, 960 per block: ragged 64-key blocks, split tiles, evictions
    w = synth.tiny(8, name="fp8_small", lat_h=16, lat_w=20, n_heads=4, n_chunks=7, n_steps=1)
    _say("[fp8 small stream]")
    _run(w, range(w.n_chunks))


def test_fp8_relative_time_twin():
    w = synth.tiny(8, name="fp8_twin", lat_h=9, lat_w=13, n_heads=2, n_chunks=7, n_steps=2, twin=True,
                   policy="relative")
    _say("[fp8 twin relative]")
    from streaming_block_causal_amd.cache import Cache
    c = Cache(config_for(w), device="cuda")
    st = ostream.Stream(w)
    for n in range(w.n_chunks):
        for s in (1, 2):
            q, k, v = synth.qkv(w, n, s)
            c.append("current", to_dev(w, k), to_dev(w, v), n)
            lse = torch.empty((w.n_heads, w.block_tokens), dtype=torch.float32, device="cuda")
            out = c.attend(to_dev(w, q), "final" if s == 2 else "intermediate", lse=lse)
            torch.cuda.synchronize()
            ref, rl, _ = st.call(n, s)
            ok, m = compare(to_f64(out), ref, "fp8", to_f64(lse), rl)
            _say(f"  chunk {n} step {s}: {m}")
            assert ok, (n, s, m)
        commit_block(c, w, n, n)


def test_fp8_540p_steady_state_two_heads():
    w = synth.WORKLOADS[8]
    rows = sorted(set(list(range(0, 40)) + list(range(2040 - 20, 2040 + 20)) + list(range(6120 - 40, 6120))))
    _say(f"[c8] {w.name}")
    _run(w, range(w.n_sink + w.n_window + 2), heads=[0, 17], rows=rows, steps=(w.n_steps,),
         check_from=w.n_sink + w.n_window)


def test_fp8_variable_length_blocks():
    """Blocks of 3, 1 and 2 frames (per-slot key counts, cumulative-frame relocation) in fp8."""
    from streaming_block_causal_amd.cache import Cache
    w = synth.tiny(8, name="fp8_varlen", lat_h=9, lat_w=13, n_heads=2, n_chunks=8, n_steps=1, policy="relative",
                   frame_pattern=(3, 1, 2))
    _say("[fp8 varlen]")
    c = Cache(config_for(w), device="cuda")
    st = ostream.Stream(w)
    for n in range(w.n_chunks):
        fn = synth.frames_of(w, n)
        q, k, v = synth.qkv(w, n, 1)
        c.append("current", to_dev(w, k), to_dev(w, v), n, n_frames=fn)
        B = synth.block_shape(w, n)[0]
        lse = torch.empty((w.n_heads, B), dtype=torch.float32, device="cuda")
        out = c.attend(to_dev(w, q), "final", lse=lse)
        torch.cuda.synchronize()
        ref, rl, _ = st.call(n, 1)
        ok, m = compare(to_f64(out), ref, "fp8", to_f64(lse), rl)
        _say(f"  chunk {n} ({fn} frames): {m}")
        assert ok, (n, m)
        commit_block(c, w, n, n)
