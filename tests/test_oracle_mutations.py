"""Planted mistakes in the oracle must fail a pin (CPU only).

Each case monkeypatches one plausible slip into the oracle -- a flipped sign,
a swapped axis split, an off-by-one relocation, the wrong eviction end, a
dropped scale, a misindexed operand, the wrong TwinCache copy, a tie broken the
wrong way -- and checks that one of the pins in the other oracle tests catches
it.  The mistakes live in the oracle on the CPU only.
"""
import numpy as np
import pytest

import synth
from oracle import attention, bruteforce, cache, rope, stream, tilemask

C1 = synth.WORKLOADS[1]
TWIN = synth.tiny(3, n_heads=2, head_dim=64, lat_h=4, lat_w=6, n_chunks=4, n_steps=2)


def _bruteforce_pin(w, chunks=(0, 3, 5), steps=(1,)):
    st = stream.Stream(w)
    for n in chunks:
        for s in steps:
            o, lse, _ = st.call(n, s)
            ob, lb = bruteforce.chunk(w, n, s)
            np.testing.assert_allclose(o, ob, atol=1e-12)
            np.testing.assert_allclose(lse, lb, atol=1e-12)


def test_pin_passes_unmutated():
    _bruteforce_pin(C1)
    _bruteforce_pin(TWIN, chunks=(1, 3), steps=(1, 2))


def test_flipped_rotation_sign_is_caught(monkeypatch):
    def bad_rotate(x, ang):
        return _orig_rotate(x, -ang)
    _orig_rotate = rope.rotate
    monkeypatch.setattr(rope, "rotate", bad_rotate)
    with pytest.raises(AssertionError):
        _bruteforce_pin(C1)


def test_swapped_axis_split_is_caught(monkeypatch):
    orig = rope.axis_split
    monkeypatch.setattr(rope, "axis_split", lambda d, split=None: tuple(orig(d, split)[i] for i in (1, 0, 2)))
    with pytest.raises(AssertionError):
        _bruteforce_pin(C1)


def test_pairs_of_neighbouring_dims_not_halves(monkeypatch):
    """Rotating (i, i + d/2) instead of (2p, 2p+1) is a different RoPE layout."""
    def half_rotate(x, ang):
        x = np.asarray(x, dtype=np.float64)
        h = x.shape[-1] // 2
        y = np.empty_like(x)
        c, s = np.cos(ang), np.sin(ang)
        y[..., :h] = x[..., :h] * c - x[..., h:] * s
        y[..., h:] = x[..., :h] * s + x[..., h:] * c
        return y
    monkeypatch.setattr(rope, "rotate", half_rotate)
    with pytest.raises(AssertionError):
        _bruteforce_pin(C1)


def test_off_by_one_relocation_is_caught(monkeypatch):
    orig = rope.relocation_bases
    monkeypatch.setattr(rope, "relocation_bases", lambda *a: [b + (1 if i == 1 else 0)
                                                              for i, b in enumerate(orig(*a))])
    with pytest.raises(AssertionError):
        _bruteforce_pin(C1)


def test_evicting_newest_is_caught(monkeypatch):
    def bad_commit(self, block):
        if len(self.sinks) < self.n_sink:
            self.sinks.append(block)
        elif len(self.window) < self.n_window:
            self.window.append(block)
        # full window: the newest block is the one dropped
    monkeypatch.setattr(cache.CacheModel, "commit", bad_commit)
    with pytest.raises(AssertionError):
        _bruteforce_pin(C1)


def test_missing_scale_is_caught(monkeypatch):
    orig = attention.attend
    monkeypatch.setattr(attention, "attend", lambda q, k, v, vis=None, row_block=512:
                        orig(q * np.sqrt(q.shape[1]), k, v, vis, row_block))
    with pytest.raises(AssertionError):
        _bruteforce_pin(C1)


def test_misindexed_values_are_caught(monkeypatch):
    orig = attention.attend
    monkeypatch.setattr(attention, "attend", lambda q, k, v, vis=None, row_block=512:
                        orig(q, k, np.roll(v, 1, axis=0), vis, row_block))
    with pytest.raises(AssertionError):
        _bruteforce_pin(C1)


def test_wrong_twin_copy_is_caught(monkeypatch):
    orig = stream.Stream.slot_inputs

    def always_noisy(self, n, s, current=None):
        w = self.w
        self.w = w.replace(n_steps=w.n_steps + 1)      # final step now looks intermediate
        try:
            return orig(self, n, s, current)
        finally:
            self.w = w
    monkeypatch.setattr(stream.Stream, "slot_inputs", always_noisy)
    with pytest.raises(AssertionError):
        _bruteforce_pin(TWIN, chunks=(2,), steps=(2,))


def test_current_block_wrong_step_is_caught(monkeypatch):
    orig = stream.Stream.slot_inputs

    def stale_current(self, n, s, current=None):
        q, slots = orig(self, n, s, current)
        _, k_last, v_last = synth.qkv(self.w, n, self.w.n_steps, self.seed)
        role, b, _, _ = slots[-1]
        return q, slots[:-1] + [(role, b, k_last, v_last)]
    monkeypatch.setattr(stream.Stream, "slot_inputs", stale_current)
    with pytest.raises(AssertionError):
        _bruteforce_pin(TWIN, chunks=(2,), steps=(1,))


def test_tie_to_higher_index_is_caught(monkeypatch):
    def bad_select(scores, always, budget):
        rest = sorted((i for i in range(len(scores)) if i not in always),
                      key=lambda i: (-float(scores[i]), -i))
        return sorted(set(always) | set(rest[:max(0, budget - len(always))]))
    monkeypatch.setattr(tilemask, "select", bad_select)
    from tests.test_oracle_tilemask import test_select_properties
    with pytest.raises(AssertionError):
        test_select_properties()


def test_dropped_forced_tile_is_caught(monkeypatch):
    monkeypatch.setattr(tilemask, "forced", lambda i, roles, tpb: {(len(roles) - 1) * tpb + i})
    from tests.test_oracle_tilemask import test_c5_steady_state_sparsity
    with pytest.raises(AssertionError):
        test_c5_steady_state_sparsity()


def test_ragged_tile_pooled_over_full_tile_is_caught(monkeypatch):
    """Averaging a ragged last tile over 128 rows (zero pads counted) instead of its valid tokens."""
    def padded_mean(x, tile=128):
        return np.stack([x[a:b].sum(axis=0) / tile for a, b in tilemask.tile_bounds(x.shape[0], tile)])
    monkeypatch.setattr(tilemask, "pooled", padded_mean)
    from tests.test_oracle_tilemask import test_golden_kept_tiles_through_stream
    with pytest.raises(AssertionError):
        test_golden_kept_tiles_through_stream()


def test_unrelocated_tile_scores_are_caught(monkeypatch):
    """Scoring key tiles with block-local (un-relocated) vectors."""
    orig = stream.relocated_head
    monkeypatch.setattr(stream, "relocated_head", lambda w, stored, head, base: orig(w, stored, head, 0))
    from tests.test_oracle_tilemask import test_golden_kept_tiles_through_stream
    with pytest.raises(AssertionError):
        test_golden_kept_tiles_through_stream()
