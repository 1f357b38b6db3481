"""Pins of the oracle's cache model and attention core (CPU only).

Cache: "Vidu S2 vs PixVerse R2" blog, section "Choice 3: bounded memory"
(permanent first blocks, window of recent blocks, the rest dropped; cost per
block does not grow).  Attention: textbook scaled dot-product softmax, pinned to
torch's scaled_dot_product_attention and closed-form special cases.
"""
import numpy as np
import pytest
import torch

from oracle import attention, cache


@pytest.mark.parametrize("S,W", [(1, 3), (1, 2), (2, 2), (0, 3), (3, 0), (0, 0), (4, 1)])
def test_cache_model_matches_closed_form(S, W):
    m = cache.CacheModel(S, W)
    for n in range(0, 1001):
        sinks, window = cache.closed_form(n, S, W)
        assert m.sinks == sinks, n
        assert list(m.window) == window, n
        lg = m.logical(n)
        assert [b for r, b in lg] == sinks + window + [n]
        assert len(lg) * 7 == cache.key_count(n, S, W, 7)
        m.commit(n)


def test_key_count_is_flat_after_warmup():
    S, W, B = 1, 3, 6120
    counts = [cache.key_count(n, S, W, B) for n in range(0, 2000)]
    assert counts[:5] == [B, 2 * B, 3 * B, 4 * B, 5 * B]
    assert set(counts[S + W:]) == {30600}


def test_attend_matches_torch_sdpa():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((70, 32)), rng.standard_normal((133, 32)), rng.standard_normal((133, 24))
    vis = rng.random((70, 133)) < 0.7
    vis[:, 0] = True
    o, lse = attention.attend(q, k, v, vis, row_block=16)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(vis)[None])[0].numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)
    s = (q @ k.T) / np.sqrt(32)
    s[~vis] = -np.inf
    np.testing.assert_allclose(lse, torch.logsumexp(torch.from_numpy(s), dim=1).numpy(), atol=1e-12)


def test_attend_special_cases():
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((9, 16)), rng.standard_normal((40, 16))
    # constant values -> output is that value
    v = np.tile(rng.standard_normal(5), (40, 1))
    o, _ = attention.attend(q, k, v)
    np.testing.assert_allclose(o, np.tile(v[0], (9, 1)), atol=1e-13)
    # one visible key -> output is its value, LSE is its score
    vis = np.zeros((9, 40), dtype=bool)
    vis[:, 17] = True
    v2 = rng.standard_normal((40, 5))
    o, lse = attention.attend(q, k, v2, vis)
    np.testing.assert_allclose(o, np.tile(v2[17], (9, 1)), atol=1e-13)
    np.testing.assert_allclose(lse, q @ k[17] / 4.0, atol=1e-13)
    # identity values -> rows of the softmax matrix, which sum to 1
    o, _ = attention.attend(q, k, np.eye(40))
    np.testing.assert_allclose(o.sum(axis=1), 1.0, atol=1e-13)
    assert (o >= 0).all()
    # masked keys contribute nothing: same as dropping them
    vis = np.ones((9, 40), dtype=bool)
    vis[:, 5:12] = False
    keep = np.r_[0:5, 12:40]
    o1, l1 = attention.attend(q, k, v2, vis)
    o2, l2 = attention.attend(q, k[keep], v2[keep])
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
