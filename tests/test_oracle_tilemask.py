"""Pins of the oracle's block-sparse tile mask (CPU only).

Source: "Vidu S2 vs PixVerse R2" blog, section "Choice 4: where the speed comes
from" (block-sparse attention above 90% sparsity).  Mask recipe: top-k of
mean-pooled tile scores with forced tiles (stated reading in oracle/tilemask.py).
"""
import math
import os

import numpy as np
import pytest

import synth
from oracle import attention, rope, stream, tilemask


def test_tile_geometry_and_budget():
    assert tilemask.n_tiles(6120) == 48 and tilemask.tile_bounds(6120)[-1] == (6016, 6120)
    assert tilemask.n_tiles(10800) == 85 and tilemask.tile_bounds(10800)[-1] == (10752, 10800)
    # budgets of the 540p block-sparse stream as the window fills: 48, 96, ..., 240 key tiles
    assert [tilemask.row_budget(48 * L, 0.08, 2) for L in range(1, 6)] == [4, 8, 12, 15, 19]
    assert 19 / 240 < 0.10            # >90% sparse at steady state
    assert tilemask.row_budget(10, 0.08, 2) == 2   # forced tiles always fit


def test_select_properties():
    rng = np.random.default_rng(5)
    scores = np.round(rng.standard_normal(240), 1)        # many exact ties
    f = {0, 200}
    kept = tilemask.select(scores, f, 19)
    assert kept == sorted(kept) and len(kept) == 19 and f <= set(kept)
    free_kept = [i for i in kept if i not in f]
    dropped = [i for i in range(240) if i not in kept]
    worst = min(scores[i] for i in free_kept)
    assert all(scores[i] <= worst for i in dropped)
    # ties at the boundary go to the lower index
    tie = [i for i in dropped if scores[i] == worst]
    assert all(i > max(j for j in free_kept if scores[j] == worst) for i in tie)
    # all scores equal: the free picks are the lowest indices
    assert tilemask.select(np.zeros(240), {7, 100}, 6) == [0, 1, 2, 3, 7, 100]
    flat = np.zeros(240)
    flat[50:60] = 1.0
    assert tilemask.select(flat, {0}, 6) == [0, 50, 51, 52, 53, 54]


def test_pooled_relocated_score_identity():
    """Pooling commutes with the per-slot time rotation (what a kernel may exploit)."""
    w = synth.tiny(5, n_heads=1, lat_h=6, lat_w=10)
    q, k, _ = synth.qkv(w, 3, 1)
    base_q, base_k = 12, 3
    f, hh, ww = rope.block_grid(w.frames, w.lat_h, w.lat_w)
    qx, kx = synth.as_f64(w, q[:, 0]), synth.as_f64(w, k[:, 0])
    q_rel = rope.rotate(qx, rope.angles(base_q + f, hh, ww, 128))
    k_rel = rope.rotate(kx, rope.angles(base_k + f, hh, ww, 128))
    q_loc = rope.rotate(qx, rope.angles(f, hh, ww, 128))
    k_loc = rope.rotate(kx, rope.angles(f, hh, ww, 128))
    lhs = tilemask.pooled(q_rel, 128) @ tilemask.pooled(k_rel, 128).T
    qbar = rope.rotate(tilemask.pooled(q_loc, 128), rope.angles(base_q - base_k, 0, 0, 128))
    rhs = qbar @ tilemask.pooled(k_loc, 128).T
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)


SMALL = synth.tiny(5, n_heads=2, lat_h=16, lat_w=16, n_chunks=6, n_steps=1)   # B = 768 = 6 tiles


def test_keep_all_equals_dense():
    w = SMALL.replace(sparse_keep=1.0)
    for n in range(SMALL.n_chunks):
        o, l, kept = stream.Stream(w).call(n, 1)
        od, ld, _ = stream.Stream(w.replace(sparse_keep=None)).call(n, 1)
        np.testing.assert_allclose(o, od, atol=1e-12)
        np.testing.assert_allclose(l, ld, atol=1e-12)


# B = 480: three full tiles and a ragged one of 96 tokens
RAGGED = synth.tiny(5, n_heads=2, lat_h=8, lat_w=20, n_chunks=6, n_steps=1)


@pytest.mark.parametrize("base", [SMALL, RAGGED], ids=["full_tiles", "ragged_tile"])
def test_gather_equals_mask_and_forced_present(base):
    w = base.replace(sparse_keep=0.25)
    st = stream.Stream(w)
    for n in (0, 1, 4, 5):
        o, lse, kept = st.call(n, 1)
        q, slots = st.slot_inputs(n, 1)
        bases = st.bases(n)
        roles = [r for r, _, _, _ in slots]
        tpb = tilemask.n_tiles(w.block_tokens)
        for h in range(w.n_heads):
            q_rel = stream.relocated_head(w, q, h, bases[-1])
            k_rel = [stream.relocated_head(w, k, h, bases[l]) for l, (_, _, k, _) in enumerate(slots)]
            v = [synth.as_f64(w, vv[:, h]) for (_, _, _, vv) in slots]
            for i, lst in enumerate(kept[h]):
                assert tilemask.forced(i, roles, tpb) <= set(lst)
                assert len(lst) == tilemask.row_budget(len(slots) * tpb, 0.25, len(tilemask.forced(i, roles, tpb)))
                ka = np.concatenate([k_rel[t // tpb][128 * (t % tpb):128 * (t % tpb + 1)] for t in lst])
                va = np.concatenate([v[t // tpb][128 * (t % tpb):128 * (t % tpb + 1)] for t in lst])
                og, lg = attention.attend(q_rel[128 * i:128 * (i + 1)], ka, va)
                np.testing.assert_allclose(o[128 * i:128 * (i + 1), h], og, atol=1e-12)
                np.testing.assert_allclose(lse[h, 128 * i:128 * (i + 1)], lg, atol=1e-12)


def test_c5_steady_state_sparsity():
    """Full-size 540p block-sparse stream, one head: 19 of 240 tiles per row (92.1% sparse)."""
    w = synth.WORKLOADS[5]
    st = stream.Stream(w)
    _, _, kept = st.call(5, 1, heads=[0], rows=np.arange(4))
    rows = kept[0]
    assert len(rows) == 48 and all(len(r) == 19 for r in rows)
    frac = sum(len(r) for r in rows) / (48 * 240)
    assert frac < 0.10
    assert all(0 in r and (4 * 48 + i) in r for i, r in enumerate(rows))


# ---- hand-derived worked example: a ragged key tile, a query tile that is ragged too, and a sink
# slot whose relocation turns the time pair by one radian (tests/golden/tilemask_ragged_relocated.txt)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tilemask_ragged_relocated.txt")


def _golden():
    rec = {}
    with open(GOLDEN) as fh:
        for ln in fh:
            if ln.startswith("#") or not ln.strip():
                continue
            key, vals = ln.split(":", 1)
            rec[key.strip()] = [float(x) for x in vals.split()]
    return rec


def _golden_case():
    g = _golden()
    d = int(g["d"][0])
    frames, lat_h, lat_w = (int(x) for x in g["grid"])
    w = synth.tiny(5, name="tilemask_golden", n_heads=1, head_dim=d, frames=frames, lat_h=lat_h,
                   lat_w=lat_w, n_sink=1, n_window=0, n_chunks=2, n_steps=1, dtype="f32", scale=1.0,
                   sparse_keep=g["keep"][0], policy="s1")
    B = w.block_tokens

    def fill(name):
        x = np.zeros((B, 1, d), dtype=np.float32)
        for j, (a, b) in enumerate(tilemask.tile_bounds(B)):
            pat = np.asarray(g[f"pattern {name} {j}"], dtype=np.float32).reshape(-1, 2)
            x[a:b, 0, 0:2] = pat[np.arange(b - a) % len(pat)]
        return x
    zero = np.zeros((B, 1, d), dtype=np.float32)
    return g, w, fill("q"), fill("k_sink"), fill("k_cur"), zero


def test_golden_tile_scores_ragged_and_relocated():
    """Pooled scores and kept tiles of the hand-worked example, from the oracle's relocation and
    tilemask.build."""
    g, w, q, k_sink, k_cur, _ = _golden_case()
    bases = stream.Stream(w).bases(1)
    assert bases == [0, 1]
    q_rel = stream.relocated_head(w, q, 0, bases[1])
    k_rel = [stream.relocated_head(w, k_sink, 0, bases[0]), stream.relocated_head(w, k_cur, 0, bases[1])]
    kept, scores, budget = tilemask.build(q_rel, k_rel, ["sink", "current"], g["keep"][0], w.tile)
    want = np.array([g["scores_x_sqrt_d 0"], g["scores_x_sqrt_d 1"]]) / math.sqrt(w.head_dim)
    np.testing.assert_allclose(scores, want, rtol=0, atol=1e-12)
    assert budget == 3
    assert kept == [[int(x) for x in g["kept 0"]], [int(x) for x in g["kept 1"]]]


def test_golden_kept_tiles_through_stream():
    """The same example through the stream oracle: its mask (and the attention restricted to it)."""
    g, w, q, k_sink, k_cur, v0 = _golden_case()
    st = stream.Stream(w, contents=lambda b, kind: (k_sink, v0) if b == 0 else None)
    o, lse, kept = st.call(1, 1, current=(q, k_cur, v0))
    assert kept[0] == [[int(x) for x in g["kept 0"]], [int(x) for x in g["kept 1"]]]
    assert np.all(o == 0.0)                          # V is zero
    # every query sees 128 + 32 + (its diagonal tile) keys -> LSE = log(sum exp(score)) is finite
    assert np.all(np.isfinite(lse))
