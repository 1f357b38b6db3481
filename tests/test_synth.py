"""The seeded input generators (CPU only): bf16 rounding is round-to-nearest-even, the same as
torch's float32 -> bfloat16 conversion, and draws are reproducible per (seed, chunk, step, tag)."""
import numpy as np
import torch

import synth


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(0.5),
        rng.standard_normal(1000).astype(np.float32) * np.float32(1e30),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4028235e38, -3.4028235e38, 1e-45, -1e-45, 1.1754944e-38],
                 dtype=np.float32)])
    # exact ties: a bf16 value plus half its last place, both parities of the kept bit
    base = rng.integers(0, 0x7F7F, 2000, dtype=np.uint32) << np.uint32(16)       # finite values
    ties = (base | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.round_bf16(x), want)


def test_draws_are_reproducible_and_independent():
    w = synth.WORKLOADS[1]
    a = synth.draw(w, 3, 1, synth.TAG_K)
    b = synth.draw(w, 3, 1, synth.TAG_K)
    c = synth.draw(w, 3, 1, synth.TAG_V)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    k, v = synth.committed_kv(w, 3)
    assert np.array_equal(k, synth.draw(w, 3, w.n_steps, synth.TAG_K))
