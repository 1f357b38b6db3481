"""Shared test plumbing: workload -> cache config, numpy <-> torch, stream driving, tolerances."""
from __future__ import annotations

import numpy as np

import synth

# Tolerances.  Max-abs bounds: 2e-2 for bf16 arithmetic, 1e-4 for fp32.
# At bf16 the outputs are so small (|O| ~ 3e-3 at 30600 keys) that 2e-2 would pass an
# all-zero output, so a relative-RMS bound is added: bf16 rounding of Q, K (after
# rotation) and P gives ~3e-3; 1e-2 leaves margin.  LSE ~ ln(#keys) is bounded in
# absolute terms.
TOL = {
    "bf16": dict(max_abs=2e-2, rel_rms=1e-2, lse=1e-2),
    "f32": dict(max_abs=1e-4, rel_rms=1e-5, lse=1e-5),
    # fp8 attention against the oracle fed the same quantised Q, K, V: what is left is the E4M3
    # rounding of the probabilities (relative error uniform in +-2^-4, rms 2^-4/sqrt(3) = 3.6%
    # per probability, averaged over the keys of a row) -- bounded at 5% relative RMS
    "fp8": dict(max_abs=2e-2, rel_rms=5e-2, lse=1e-2),
}


def config_for(w: synth.Workload):
    from streaming_block_causal_amd.cache import CacheConfig
    return CacheConfig(n_heads=w.n_heads, head_dim=w.head_dim, frames_per_block=w.frames, lat_h=w.lat_h,
                       lat_w=w.lat_w, n_sink=w.n_sink, n_window=w.n_window, twin=w.twin,
                       sparse=w.sparse_keep is not None, dtype="fp8" if w.attn_fp8 else w.dtype,
                       rope_theta=w.rope_theta,
                       policy=w.policy, tile=w.tile, editing=w.editing, rope_pairs=w.rope_split)


def to_dev(w: synth.Workload, stored: np.ndarray, device="cuda"):
    import torch
    if w.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).to(device)


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def window_len_after(n_committed: int, S: int, W: int) -> int:
    return min(max(n_committed - S, 0), W)


def commit_block(cache, w: synth.Workload, b: int, n_committed: int, seed: int = 0, device="cuda",
                 contents=None):
    """Commit block b as the stream would: evict if the window is full, promote, noisy twin."""
    S, W = w.n_sink, w.n_window
    if n_committed >= S and W > 0 and window_len_after(n_committed, S, W) == W:
        cache.evict()
    cache.append("clean", None, None, b)
    if w.twin:
        kn, vn = contents(b, "noisy") if contents else synth.noisy_kv(w, b, seed)
        cache.append("noisy", to_dev(w, kn, device), to_dev(w, vn, device), b)


def advance(cache, w: synth.Workload, upto: int, seed: int = 0, device="cuda", contents=None):
    """Stage + commit chunks 0..upto-1 with their final-step K/V (what the history keeps)."""
    for b in range(upto):
        k, v = contents(b, "clean") if contents else synth.committed_kv(w, b, seed)
        cache.append("current", to_dev(w, k, device), to_dev(w, v, device), b)
        commit_block(cache, w, b, b, seed, device, contents)


def compare(got: np.ndarray, ref: np.ndarray, dtype: str, got_lse=None, ref_lse=None):
    """Return error metrics and whether they are inside the tolerances."""
    tol = TOL[dtype]
    diff = got - ref
    m = dict(max_abs=float(np.abs(diff).max()),
             rel_rms=float(np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-300)))
    ok = m["max_abs"] <= tol["max_abs"] and m["rel_rms"] <= tol["rel_rms"]
    if got_lse is not None:
        m["lse"] = float(np.abs(got_lse - ref_lse).max())
        ok = ok and m["lse"] <= tol["lse"]
    return ok, m
