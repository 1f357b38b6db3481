"""Pins of the oracle's RMSNorm (CPU only): closed forms and torch's own rms_norm.

Source: Vidu S2 paper read, section 2.4 (RMSNorm fused with elementwise operators);
textbook definition y = x / sqrt(mean(x^2) + eps) * g over the head dimension.
"""
import numpy as np
import torch

from oracle import qknorm


def test_constant_vector_closed_form():
    d, c, eps = 128, 0.37, 1e-6
    g = np.linspace(0.5, 1.5, d)
    y = qknorm.rms_norm(np.full((3, d), c), g, eps)
    np.testing.assert_allclose(y, np.broadcast_to(g * c / np.sqrt(c * c + eps), (3, d)), rtol=1e-15)


def test_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 7, 128))
    y = qknorm.rms_norm(x, np.ones(128), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(qknorm.rms_norm(4.5 * x, np.ones(128), 0.0), y, rtol=1e-13)


def test_matches_torch_rms_norm():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 3, 128)) * 0.5
    g = rng.uniform(0.5, 1.5, 128)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(g), eps=1e-6).numpy()
    np.testing.assert_allclose(qknorm.rms_norm(x, g, 1e-6), ref, rtol=1e-12, atol=1e-14)


def test_planted_mean_of_abs_fails():
    """Normalising by mean |x| instead of the root mean square is caught by the closed form."""
    x = np.array([[3.0, 4.0] + [0.0] * 126])
    wrong = x / np.mean(np.abs(x), axis=-1, keepdims=True)
    right = qknorm.rms_norm(x, np.ones(128), 0.0)
    assert not np.allclose(wrong, right)
    np.testing.assert_allclose(right[0, :2], np.array([3.0, 4.0]) / np.sqrt(25.0 / 128.0))
