"""GPU parity for parts of the C ABI beyond the plain dense call: the tile mask of a TwinCache
stream (the noisy copies are scored on intermediate steps), tile lists with repeated or
out-of-order entries (each key tile counts at most once), and RoPE splits over (t, h, w) given
by the caller.  HIP path through the C ABI against the fp64 oracle; tolerances in helpers.py.

Sources: "Vidu S2 vs PixVerse R2" blog, sections "Choice 3: bounded memory" (TwinCache reads)
and "Choice 4: where the speed comes from" (block-sparse attention); Vidu S2 paper read,
abbreviation table (3D RoPE over time, height and width).
"""
import numpy as np
import pytest

import synth
from oracle import stream as ostream
from oracle import tilemask as otm

from .helpers import advance, commit_block, compare, config_for, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)


def _cache(w):
    from streaming_block_causal_amd.cache import Cache
    return Cache(config_for(w), device="cuda")


def _mask_vs_oracle(w, c, qd, n, s, step, contents=None):
    """GPU tile mask against the oracle's (kept sets equal except at fp64 near-ties)."""
    idx, k_row = c.build_tile_mask(qd, w.sparse_keep, step=step)
    torch.cuda.synchronize()
    st = ostream.Stream(w, contents=contents)
    q, slots = st.slot_inputs(n, s)
    bases = st.bases(n)
    roles = [r for r, _, _, _ in slots]
    gpu = idx.cpu().numpy()
    kept_all, flips = [], 0
    for h in range(w.n_heads):
        q_rel = ostream.relocated_head(w, q, h, bases[-1])
        k_rel = [ostream.relocated_head(w, k, h, bases[l]) for l, (_, _, k, _) in enumerate(slots)]
        kept, scores, budget = otm.build(q_rel, k_rel, roles, w.sparse_keep, w.tile)
        assert k_row == budget
        for i, ref in enumerate(kept):
            g = list(gpu[h, i])
            if g != ref:
                sc = scores[i]
                a, b = set(g) - set(ref), set(ref) - set(g)
                gap = max(abs(sc[x] - sc[y]) for x in a for y in b)
                assert gap <= 1e-5 * np.abs(sc).max() + 1e-7, (h, i, a, b, gap)
                flips += len(a)
        kept_all.append(kept)
    return idx, k_row, kept_all, flips


def test_twincache_sparse_mask_and_attention():
    """A TwinCache + block-sparse stream: intermediate steps score (and attend) the noisy copies,
    the final step the clean ones; mask and attention against the oracle, every row."""
    w = synth.tiny(3, name="twin_sparse", n_heads=3, lat_h=16, lat_w=20, n_chunks=6, n_steps=3,
                   sparse_keep=0.3)                                           # B = 960
    _say(f"[twin + sparse] B={w.block_tokens}")
    c = _cache(w)
    st = ostream.Stream(w)
    for n in range(w.n_chunks):
        for s in range(1, w.n_steps + 1):
            q, k, v = synth.qkv(w, n, s)
            c.append("current", to_dev(w, k), to_dev(w, v), n)
            step = "final" if s == w.n_steps else "intermediate"
            qd = to_dev(w, q)
            idx, k_row, kept, flips = _mask_vs_oracle(w, c, qd, n, s, step)
            ref, rl, okept = st.call(n, s)
            assert okept == kept
            # attention on the oracle's mask (the GPU mask may differ at near-ties)
            tiles = torch.tensor(np.array(kept, dtype=np.int32), device="cuda")
            lse = torch.empty((w.n_heads, w.block_tokens), dtype=torch.float32, device="cuda")
            out = c.attend(qd, step, tile_idx=tiles, k_row=tiles.shape[2], lse=lse)
            torch.cuda.synchronize()
            ok, m = compare(to_f64(out), ref, w.dtype, to_f64(lse), rl)
            _say(f"  chunk {n} step {s} ({step}): flips={flips} {m}")
            assert ok, (n, s, m)
        commit_block(c, w, n, n)


def test_twincache_mask_reads_the_step_copy():
    """The same queries scored against the noisy and the clean copies give different masks (the
    noise is large), and each equals the oracle's for its step."""
    w = synth.tiny(3, name="twin_sparse_copy", n_heads=2, lat_h=16, lat_w=20, n_chunks=5, n_steps=2,
                   sparse_keep=0.3)
    n = 4
    c = _cache(w)
    advance(c, w, n)
    q, k, v = synth.qkv(w, n, 1)
    c.append("current", to_dev(w, k), to_dev(w, v), n)
    qd = to_dev(w, q)
    i1, _, _, _ = _mask_vs_oracle(w, c, qd, n, 1, "intermediate")
    i1 = i1.clone()
    # the step-1 queries scored on the clean copies: an oracle stream in which step 1 is the
    # final step, fed the blocks this cache committed
    w2 = w.replace(n_steps=1)
    i2, _, _, _ = _mask_vs_oracle(w2, c, qd, n, 1, "final",
                                  contents=lambda b, kind: synth.committed_kv(w, b) if kind == "clean" else None)
    assert not torch.equal(i1, i2)


def test_repeated_and_unordered_tile_entries_count_once():
    """Every key tile of a row counts at most once: a list whose entries repeat, or step back
    below an entry already taken, gives the attention of the list without them, bit for bit."""
    w = synth.tiny(5, n_heads=2, lat_h=16, lat_w=20, n_chunks=4, n_steps=1, sparse_keep=0.3)
    n = 3
    c = _cache(w)
    advance(c, w, n)
    q, k, v = synth.qkv(w, n, 1)
    c.append("current", to_dev(w, k), to_dev(w, v), n)
    qd = to_dev(w, q)
    idx, k_row = c.build_tile_mask(qd, w.sparse_keep)
    torch.cuda.synchronize()
    base = idx.cpu().numpy()
    twice = np.repeat(base, 2, axis=2)                               # a0 a0 a1 a1 ...
    back = np.concatenate([base, base[:, :, :1], base[:, :, :1]], axis=2)   # ... then a0 again
    o_ref = c.attend(qd, "final", tile_idx=idx, k_row=k_row)
    for name, lst in (("repeated", twice), ("stepping back", back)):
        t = torch.tensor(np.ascontiguousarray(lst), dtype=torch.int32, device="cuda")
        o = c.attend(qd, "final", tile_idx=t, k_row=t.shape[2])
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), name
    # an unordered row: the entries below the running maximum are skipped
    rev = np.ascontiguousarray(base[:, :, ::-1])
    kept_first = np.full_like(base, -1)
    kept_first[:, :, 0] = rev[:, :, 0]                              # only the largest survives
    o1 = c.attend(qd, "final", tile_idx=torch.tensor(rev, device="cuda"), k_row=k_row)
    o2 = c.attend(qd, "final", tile_idx=torch.tensor(kept_first, device="cuda"), k_row=k_row)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("base, split, kw", [
    (1, (8, 12, 12), dict(n_chunks=6)),                                          # fp32, d = 64
    (1, (40, 12, 12), dict(n_chunks=5, head_dim=128, lat_h=5, lat_w=7)),         # fp32: > 24 time pairs
    (2, (16, 24, 24), dict(n_heads=3, lat_h=8, lat_w=20, n_chunks=6, n_steps=2)),   # bf16
    (2, (24, 0, 40), dict(n_heads=2, lat_h=8, lat_w=20, n_chunks=5, n_steps=1, policy="relative")),
], ids=["f32_d64", "f32_d128_long_time", "bf16", "bf16_no_row_pairs"])
def test_custom_rope_split_stream(base, split, kw):
    w = synth.tiny(base, name="split", rope_split=split, **kw)
    _say(f"[rope split {split}] {w.dtype} d={w.head_dim} B={w.block_tokens}")
    c = _cache(w)
    st = ostream.Stream(w)
    for n in range(w.n_chunks):
        for s in range(1, w.n_steps + 1):
            q, k, v = synth.qkv(w, n, s)
            c.append("current", to_dev(w, k), to_dev(w, v), n)
            lse = torch.empty((w.n_heads, w.block_tokens), dtype=torch.float32, device="cuda")
            out = c.attend(to_dev(w, q), "final" if s == w.n_steps else "intermediate", lse=lse)
            torch.cuda.synchronize()
            ref, rl, _ = st.call(n, s)
            ok, m = compare(to_f64(out), ref, w.dtype, to_f64(lse), rl)
            _say(f"  chunk {n} step {s}: {m}")
            assert ok, (n, s, m)
        commit_block(c, w, n, n)


@pytest.mark.parametrize("split, policy", [((0, 32, 32), "relative"), ((24, 20, 20), "relative"),
                                           ((24, 20, 20), "s1")], ids=["no_time_pairs", "max_time_pairs", "max_s1"])
def test_sparse_relocation_rows(split, policy):
    """The tile mask stages each slot's row of the time table (pt entries, 0..24) before scoring:
    a split with no time pairs (no relocation at all) and one with the most a bf16 cache allows,
    against the oracle's mask and then the attention over that mask, every row."""
    w = synth.tiny(5, name="reloc_rows", rope_split=split, n_heads=2, lat_h=16, lat_w=20, n_chunks=6,
                   n_steps=1, sparse_keep=0.3, policy=policy)
    n = 5                                                       # past the first eviction
    c = _cache(w)
    advance(c, w, n)
    q, k, v = synth.qkv(w, n, 1)
    c.append("current", to_dev(w, k), to_dev(w, v), n)
    qd = to_dev(w, q)
    _, _, kept, flips = _mask_vs_oracle(w, c, qd, n, 1, "final")
    # attention on the oracle's mask (the GPU mask may differ at near-ties)
    tiles = torch.tensor(np.array(kept, dtype=np.int32), device="cuda")
    lse = torch.empty((w.n_heads, w.block_tokens), dtype=torch.float32, device="cuda")
    out = c.attend(qd, "final", tile_idx=tiles, k_row=tiles.shape[2], lse=lse)
    torch.cuda.synchronize()
    ref, rl, _ = ostream.Stream(w).call(n, 1, kept=kept)
    ok, m = compare(to_f64(out), ref, w.dtype, to_f64(lse), rl)
    _say(f"[sparse relocation rows {split} {policy}] flips={flips} {m}")
    assert ok, m


def test_custom_rope_split_sparse_and_fp8():
    """The tile mask and the fp8 attention take the split too."""
    w = synth.tiny(5, name="split_sparse", rope_split=(18, 23, 23), n_heads=2, lat_h=16, lat_w=20,
                   n_chunks=5, n_steps=1, sparse_keep=0.3)
    n = 4
    c = _cache(w)
    advance(c, w, n)
    q, k, v = synth.qkv(w, n, 1)
    c.append("current", to_dev(w, k), to_dev(w, v), n)
    _, _, _, flips = _mask_vs_oracle(w, c, to_dev(w, q), n, 1, "final")
    _say(f"[rope split sparse] flips={flips}")
    wf = synth.tiny(8, name="split_fp8", rope_split=(20, 22, 22), lat_h=16, lat_w=20, n_heads=2, n_chunks=5,
                    n_steps=1)
    cf = _cache(wf)
    st = ostream.Stream(wf)
    for n in range(wf.n_chunks):
        q, k, v = synth.qkv(wf, n, 1)
        cf.append("current", to_dev(wf, k), to_dev(wf, v), n)
        lse = torch.empty((wf.n_heads, wf.block_tokens), dtype=torch.float32, device="cuda")
        out = cf.attend(to_dev(wf, q), "final", lse=lse)
        torch.cuda.synchronize()
        ref, rl, _ = st.call(n, 1)
        ok, m = compare(to_f64(out), ref, "fp8", to_f64(lse), rl)
        _say(f"  fp8 chunk {n}: {m}")
        assert ok, (n, m)
        commit_block(cf, wf, n, n)
