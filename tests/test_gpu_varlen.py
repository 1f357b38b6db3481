"""GPU parity for variable-length blocks: the HIP path through the C ABI against the fp64 oracle.

Block length follows the control signal up to a cap ("Vidu S2 vs PixVerse R2" blog,
section "Choice 5: how people control it"); positions per section "Choice 3: bounded
memory".  Every chunk and row of small streams (fp32 and bf16, ragged 64-key blocks of
different lengths per slot), and all rows of two heads at 540p.
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


def _run_stream(w, chunks, heads=None, steps=None, check_from=0):
    from streaming_block_causal_amd.cache import Cache
    c = Cache(config_for(w), device="cuda")
    st = ostream.Stream(w)
    S, W = w.n_sink, w.n_window
    worst = {}
    for n in chunks:
        fn = synth.frames_of(w, n)
        for s in (steps or range(1, w.n_steps + 1)):
            q, k, v = synth.qkv(w, n, s)
            c.append("current", to_dev(w, k), to_dev(w, v), n, n_frames=fn)
            if n < check_from:
                continue
            B = synth.block_shape(w, n)[0]
            lse = torch.empty((w.n_heads, B), dtype=torch.float32, device="cuda")
            out = c.attend(to_dev(w, q), "final" if s == w.n_steps else "intermediate", lse=lse)
            torch.cuda.synchronize()
            got, gl = to_f64(out), to_f64(lse)
            ref, rl, _ = st.call(n, s, heads=heads, workers=8 if heads is None or len(heads) > 1 else 1)
            if heads is not None:
                got, gl = got[:, heads], gl[heads]
            ok, m = compare(got, ref, w.dtype, gl, rl)
            _say(f"  chunk {n} ({fn} frames, B={B}) step {s}: {m}")
            assert ok, (n, s, m)
            for key, val in m.items():
                worst[key] = max(worst.get(key, 0.0), val)
        # commit the final-step K/V (staged by the last step above)
        if n >= S and W > 0 and window_len_after(n, S, W) == W:
            c.evict()
        c.append("clean", None, None, n)
        if w.twin:
            kn, vn = synth.noisy_kv(w, n)
            c.append("noisy", to_dev(w, kn), to_dev(w, vn), n, n_frames=fn)
    return worst


@pytest.mark.parametrize("policy", ["s1", "relative"])
def test_varlen_fp32_full_stream(policy):
    w = synth.tiny(1, n_chunks=10, policy=policy, frame_pattern=(3, 1, 2, 1, 3, 2))
    _say(f"[varlen fp32 {policy}]")
    _run_stream(w, range(w.n_chunks))


def test_varlen_bf16_small_stream_twin():
    w = synth.tiny(2, name="varlen_small_bf16", lat_h=16, lat_w=20, n_heads=4, n_chunks=10, n_steps=2,
                   twin=True, policy="relative", frame_pattern=(3, 1, 2, 1, 3, 2))
    _say(f"[varlen bf16 small] B per frame {w.lat_h * w.lat_w}")
    _run_stream(w, range(w.n_chunks))


def test_varlen_540p_steady_state_two_heads():
    w = synth.WORKLOADS[6]
    _say(f"[c6] {w.name} pattern {w.frame_pattern}")
    # chunks 8..11: full window, slots of 3, 1, 1, 2 frames and current blocks of 3, 1, 1, 2
    _run_stream(w, range(12), heads=[0, 17], steps=[w.n_steps], check_from=8)
