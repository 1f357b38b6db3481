"""GPU: the fused QKV epilogue (per-head RMSNorm of q and k + RoPE + append) against the oracle.

Vidu S2 paper read, section 2.4: adjacent operators such as RMSNorm and elementwise work are
fused into one kernel.  The normalised q, the stored (normalised, rotated) k and v are compared
with the fp64 oracle's RMSNorm and RoPE, and the attention call that consumes them with the
oracle's attention over the normalised block.
"""
import numpy as np
import pytest

import synth
from oracle import qknorm, rope
from oracle import stream as ostream

from .helpers import advance, compare, config_for, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

EPS = 1e-6


def _gammas(d, seed=11):
    g = np.random.default_rng(seed)
    return g.uniform(0.5, 1.5, d), g.uniform(0.5, 1.5, d)


def _store(w, x64):
    """fp64 values -> the workload's storage form (the oracle's inputs are stored tensors)."""
    return synth.round_bf16(x64.astype(np.float32)) if w.dtype == "bf16" else x64.astype(np.float32)


@pytest.mark.parametrize("base,kw", [(2, dict(lat_h=16, lat_w=20, n_heads=4, n_chunks=6)),
                                     (1, dict(head_dim=128, n_heads=2, n_chunks=6))])
def test_qkv_epilogue_against_oracle(base, kw):
    from streaming_block_causal_amd.cache import Cache
    w = synth.tiny(base, name="qkv_epilogue", **kw)
    print(f"[qkv epilogue {w.dtype}] B={w.block_tokens}", flush=True)
    c = Cache(config_for(w), device="cuda")
    n = w.n_sink + w.n_window + 1            # steady state: full window
    advance(c, w, n)
    q, k, v = synth.qkv(w, n, 1)
    gq, gk = _gammas(w.head_dim)
    qkv = np.stack([q, k, v], axis=1)        # [B][3][H][d], storage form
    q_out = c.append_qkv(to_dev(w, qkv), torch.tensor(gq, dtype=torch.float32, device="cuda"),
                         torch.tensor(gk, dtype=torch.float32, device="cuda"), EPS, n)
    kc, vc = c.read_slot(0, "current")
    torch.cuda.synchronize()
    qn = qknorm.rms_norm(synth.as_f64(w, q), gq, EPS)
    kn = qknorm.rms_norm(synth.as_f64(w, k), gk, EPS)
    k_ref = rope.rotate_block(kn, 0, w.frames, w.lat_h, w.lat_w, w.rope_theta)
    # one rounding of an fp32 result to the storage type (bf16: within one ulp, 2^-8 relative)
    rtol, atol = (2.0 ** -8, 1e-6) if w.dtype == "bf16" else (1e-5, 1e-6)
    np.testing.assert_allclose(to_f64(q_out), qn, rtol=rtol, atol=atol)
    np.testing.assert_allclose(to_f64(kc), k_ref, rtol=rtol, atol=atol * 10)
    assert np.array_equal(to_f64(vc), synth.as_f64(w, v))
    # the attention call over the fused block, against the oracle fed the normalised block
    lse = torch.empty((w.n_heads, w.block_tokens), dtype=torch.float32, device="cuda")
    out = c.attend(q_out, "final" if w.n_steps == 1 else "intermediate", lse=lse)
    torch.cuda.synchronize()
    ref, rl, _ = ostream.Stream(w).call(n, 1, current=(_store(w, qn), _store(w, kn), v))
    ok, m = compare(to_f64(out), ref, w.dtype, to_f64(lse), rl)
    print(f"  attention: {m}", flush=True)
    assert ok, m


def test_qkv_epilogue_short_block_and_restage():
    """A 1-frame block through the epilogue, restaged for a second step with new values."""
    from streaming_block_causal_amd.cache import Cache
    w = synth.tiny(6, name="qkv_varlen", lat_h=9, lat_w=13, n_heads=2, n_chunks=4, n_steps=2)
    c = Cache(config_for(w), device="cuda")
    gq, gk = _gammas(w.head_dim, 5)
    tq = torch.tensor(gq, dtype=torch.float32, device="cuda")
    tk = torch.tensor(gk, dtype=torch.float32, device="cuda")
    for n in range(3):
        fn = synth.frames_of(w, n)
        for s in (1, 2):
            q, k, v = synth.qkv(w, n, s)
            q_out = c.append_qkv(to_dev(w, np.stack([q, k, v], axis=1)), tq, tk, EPS, n, n_frames=fn)
            kc, _ = c.read_slot(0, "current")
            torch.cuda.synchronize()
            k_ref = rope.rotate_block(qknorm.rms_norm(synth.as_f64(w, k), gk, EPS), 0, fn, w.lat_h, w.lat_w,
                                      w.rope_theta)
            np.testing.assert_allclose(to_f64(q_out), qknorm.rms_norm(synth.as_f64(w, q), gq, EPS),
                                       rtol=2.0 ** -8, atol=1e-6)
            np.testing.assert_allclose(to_f64(kc), k_ref, rtol=2.0 ** -8, atol=1e-5)
        c.append("clean", None, None, n)
