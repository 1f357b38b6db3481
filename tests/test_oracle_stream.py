"""Pins of the oracle's streaming call against brute force and invariants (CPU only).

Brute force: every token of blocks 0..n with an explicit block-causal visibility
mask, closed-form relocated positions, complex-exponential RoPE and torch SDPA
(``oracle/bruteforce.py``), which shares no step with ``oracle/stream.py``
beyond the seeded inputs.  Invariants from "Vidu S2 vs PixVerse R2" blog,
section "Choice 3: bounded memory": cost per block is flat, and positions (hence
outputs) do not depend on how long the stream has run; TwinCache reads noisy
copies at intermediate steps and clean ones at the final step.
"""
import numpy as np
import pytest

import synth
from oracle import bruteforce, stream

C1 = synth.WORKLOADS[1]


def _check_against_bruteforce(w, chunks, steps=None, tol=1e-12):
    st = stream.Stream(w)
    for n in chunks:
        for s in (steps or range(1, w.n_steps + 1)):
            o, lse, _ = st.call(n, s)
            ob, lb = bruteforce.chunk(w, n, s)
            np.testing.assert_allclose(o, ob, atol=tol, err_msg=f"chunk {n} step {s}")
            np.testing.assert_allclose(lse, lb, atol=tol, err_msg=f"chunk {n} step {s}")


def test_c1_all_chunks_equal_bruteforce():
    _check_against_bruteforce(C1, range(C1.n_chunks))


@pytest.mark.parametrize("variant", [
    dict(policy="relative"),
    dict(n_sink=2, n_window=1),
    dict(n_sink=0, n_window=3),
    dict(n_sink=2, n_window=0),
    dict(twin=True, n_steps=2, dtype="bf16", scale=0.5),
    dict(lat_h=5, lat_w=7, frames=2, head_dim=128, n_heads=2, dtype="bf16", scale=0.5),
    dict(rope_split=(8, 12, 12)),                     # a caller-given RoPE split (d = 64)
    dict(rope_split=(20, 0, 12), policy="relative"),  # no pair follows the row
])
def test_variants_equal_bruteforce(variant):
    w = synth.tiny(1, **{**dict(n_heads=2, lat_h=4, lat_w=6, n_chunks=7), **variant})
    _check_against_bruteforce(w, range(w.n_chunks))


def test_relocation_policies_agree():
    """Relative-time RoPE is the S1 layout shifted in time: same attention."""
    a = stream.Stream(C1)
    b = stream.Stream(C1.replace(policy="relative"))
    for n in range(C1.n_chunks):
        oa, la, _ = a.call(n, 1)
        ob, lb, _ = b.call(n, 1)
        np.testing.assert_allclose(oa, ob, atol=1e-12)
        np.testing.assert_allclose(la, lb, atol=1e-12)


def test_block_10_equals_block_1000():
    """Same cache contents at chunk 10 and chunk 1000 -> identical output, exactly."""
    w = C1
    pool = {i: synth.committed_kv(w, 500 + i) for i in range(w.n_sink + w.n_window)}
    cur = synth.qkv(w, 777, 1)

    def contents_for(n):
        def f(b, kind):
            if b < w.n_sink:
                return pool[b]
            return pool[w.n_sink + (b - (n - w.n_window))]
        return f

    o10, l10, _ = stream.Stream(w, contents=contents_for(10)).call(10, 1, current=cur)
    o1k, l1k, _ = stream.Stream(w, contents=contents_for(1000)).call(1000, 1, current=cur)
    np.testing.assert_array_equal(o10, o1k)
    np.testing.assert_array_equal(l10, l1k)


def test_logical_slots_flat_in_stream_length():
    st = stream.Stream(synth.WORKLOADS[2])
    sizes = [len(st.logical(n)) for n in range(0, 300)]
    assert sizes[:4] == [1, 2, 3, 4] and set(sizes[4:]) == {5}


# ---- TwinCache --------------------------------------------------------------------
TWIN = synth.tiny(3, n_heads=2, head_dim=64, lat_h=4, lat_w=6, n_chunks=6, n_steps=3)


def test_twin_zero_noise_equals_dense():
    dense = stream.Stream(TWIN.replace(twin=False))
    twin0 = stream.Stream(TWIN, sigma_override=0.0)
    for n in range(TWIN.n_chunks):
        for s in range(1, TWIN.n_steps + 1):
            np.testing.assert_array_equal(twin0.call(n, s)[0], dense.call(n, s)[0])


def test_twin_final_step_reads_clean_intermediate_reads_noisy():
    dense = stream.Stream(TWIN.replace(twin=False))
    twin = stream.Stream(TWIN)
    T = TWIN.n_steps
    for n in range(1, TWIN.n_chunks):
        np.testing.assert_array_equal(twin.call(n, T)[0], dense.call(n, T)[0])
        for s in range(1, T):
            diff = np.abs(twin.call(n, s)[0] - dense.call(n, s)[0]).max()
            assert diff > 1e-3, (n, s)
    # chunk 0 has no history: noisy or clean makes no difference
    np.testing.assert_array_equal(twin.call(0, 1)[0], dense.call(0, 1)[0])


def test_twin_noise_recipe():
    k, v = synth.committed_kv(TWIN, 2)
    kn, vn = synth.noisy_kv(TWIN, 2)
    sig = synth.sigma(TWIN, 2)
    assert 0.3 <= sig <= 0.8
    dk = synth.as_f64(TWIN, kn) - synth.as_f64(TWIN, k)
    assert abs(dk.std() / sig - 1) < 0.05
