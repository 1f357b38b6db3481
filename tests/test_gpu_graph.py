"""GPU: a chunk's launches recorded once per ring phase and replayed match eager calls exactly.

The steady launch sequence of a chunk (appends and attention calls of every denoising
step) is captured and replayed (Vidu S2 paper read, section 2.4, the kernel-level cut).
In steady state the ring layout repeats every n_window + 1 chunks, so one graph per
phase, replayed in turn with each chunk's inputs copied into the recorded buffers,
continues the stream.  Every replay is compared bit for bit with an eager cache fed
the same inputs, with eager work and synchronisations between replays, and the last
replayed chunk with the fp64 oracle.
"""
import pytest

import synth
from oracle import stream as ostream

from .helpers import compare, config_for, to_dev, to_f64, window_len_after

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _commit(c, w, n):
    if n >= w.n_sink and w.n_window > 0 and window_len_after(n, w.n_sink, w.n_window) == w.n_window:
        c.evict()
    c.append("clean", None, None, n)


@pytest.mark.parametrize("kind", ["dense", "twin", "sparse", "editing", "fp8"])
def test_graph_replay_equals_eager(kind):
    from streaming_block_causal_amd.cache import Cache
    kw = dict(lat_h=16, lat_w=20, n_heads=4, n_chunks=14, n_steps=2)
    w = {"dense": synth.tiny(2, name="g_dense", **kw),
         "twin": synth.tiny(3, name="g_twin", **kw),
         "sparse": synth.tiny(5, name="g_sparse", sparse_keep=0.3, **kw),
         "editing": synth.tiny(7, name="g_edit", ref_frames=3, **kw),
         "fp8": synth.tiny(8, name="g_fp8", **kw)}[kind]
    print(f"[graph {kind}]", flush=True)
    side = torch.cuda.Stream()
    eager = Cache(config_for(w), device="cuda")
    rec = Cache(config_for(w), device="cuda", stream=side)
    B, T = w.block_tokens, w.n_steps
    shape = (B, w.n_heads, w.head_dim)
    dt = torch.bfloat16
    sq = [torch.empty(shape, dtype=dt, device="cuda") for _ in range(T)]
    sk = [torch.empty(shape, dtype=dt, device="cuda") for _ in range(T)]
    sv = [torch.empty(shape, dtype=dt, device="cuda") for _ in range(T)]
    so = [torch.empty(shape, dtype=dt, device="cuda") for _ in range(T)]
    skn, svn = torch.empty(shape, dtype=dt, device="cuda"), torch.empty(shape, dtype=dt, device="cuda")
    sks, svs = torch.empty(shape, dtype=dt, device="cuda"), torch.empty(shape, dtype=dt, device="cuda")
    nt = -(-B // 128)
    first = w.n_sink + w.n_window        # the first chunk with a full window (steady state)
    state = {"k_row": 0}

    def inputs(n):
        qkv = [synth.qkv(w, n, s + 1) for s in range(T)]
        extra = {}
        if w.twin:
            extra["noisy"] = synth.noisy_kv(w, n)
        if w.editing and n >= 1:
            extra["source"] = synth.source_kv(w, n)
        return qkv, extra

    def chunk_calls(c, n, q, k, v, out, kn=None, vn=None, ks=None, vs=None, idx=None):
        for s in range(T):
            c.append("current", k[s], v[s], n)
            if ks is not None and s == 0:
                c.append("source", ks, vs, n)
            step = "final" if s == T - 1 else "intermediate"
            if idx is not None and n >= first:   # block-sparse in steady state (fixed budget)
                _, kr = c.build_tile_mask(q[s], w.sparse_keep, out=idx, k_cap=state["k_row"], step=step)
                assert kr == state["k_row"]
                c.attend(q[s], step, tile_idx=idx, k_row=kr, out=out[s])
            else:
                c.attend(q[s], step, out=out[s])
        _commit(c, w, n)
        if kn is not None:
            c.append("noisy", kn, vn, n)

    def eager_chunk(n, qkv, extra, cache=None):
        q = [to_dev(w, x[0]) for x in qkv]
        k = [to_dev(w, x[1]) for x in qkv]
        v = [to_dev(w, x[2]) for x in qkv]
        out = [torch.empty(shape, dtype=dt, device="cuda") for _ in range(T)]
        kn, vn = (to_dev(w, x) for x in extra["noisy"]) if "noisy" in extra else (None, None)
        ks, vs = (to_dev(w, x) for x in extra["source"]) if "source" in extra else (None, None)
        idx = torch.empty_like(state["sidx"]) if kind == "sparse" and n >= first else None
        chunk_calls(eager if cache is None else cache, n, q, k, v, out, kn, vn, ks, vs, idx)
        torch.cuda.synchronize()
        return out

    def fill_static(qkv, extra):
        for s in range(T):
            for dst, src in ((sq[s], qkv[s][0]), (sk[s], qkv[s][1]), (sv[s], qkv[s][2])):
                dst.copy_(to_dev(w, src))
        if "noisy" in extra:
            skn.copy_(to_dev(w, extra["noisy"][0]))
            svn.copy_(to_dev(w, extra["noisy"][1]))
        if "source" in extra:
            sks.copy_(to_dev(w, extra["source"][0]))
            svs.copy_(to_dev(w, extra["source"][1]))
        torch.cuda.synchronize()

    # both caches run eagerly up to steady state (full window: the first evicting chunk)
    for n in range(first):
        qkv, extra = inputs(n)
        eager_chunk(n, qkv, extra)
        fill_static(qkv, extra)
        chunk_calls(rec, n, sq, sk, sv, so, skn if w.twin else None, svn, sks if "source" in extra else None,
                    svs)
        torch.cuda.synchronize()
    state["k_row"] = rec.mask_budget(w.sparse_keep) if kind == "sparse" else 1
    state["sidx"] = torch.empty((w.n_heads, nt, state["k_row"]), dtype=torch.int32, device="cuda")
    sidx = state["sidx"]
    # record one chunk per ring phase (nothing runs while recording)
    period = rec.ring_period()
    graphs = []
    for p in range(period):
        rec.graph_begin()
        chunk_calls(rec, first + p, sq, sk, sv, so, skn if w.twin else None, svn,
                    sks if w.editing else None, svs, sidx if kind == "sparse" else None)
        graphs.append(rec.graph_end())
    # replay two periods and a half, chunk by chunk, against the eager cache
    for n in range(first, first + 2 * period + period // 2 + 1):
        qkv, extra = inputs(n)
        ref = eager_chunk(n, qkv, extra)
        fill_static(qkv, extra)
        graphs[(n - first) % period].launch()
        side.synchronize()
        for s in range(T):
            assert torch.equal(so[s], ref[s]), (kind, n, s)
        print(f"  chunk {n} phase {(n - first) % period}: equal", flush=True)
    # the last replayed chunk against the fp64 oracle, every row of every step (block-sparse: the
    # final step, on the mask the replay built -- it holds that step's mask, and may differ from
    # the oracle's own only at near-ties)
    kept, steps = None, range(T)
    if kind == "sparse":
        g = sidx.cpu().numpy()
        kept = [[[int(x) for x in row if x >= 0] for row in g[h]] for h in range(w.n_heads)]
        steps = [T - 1]
    st = ostream.Stream(w)
    for s in steps:
        ref, _, _ = st.call(n, s + 1, kept=kept)
        ok, m = compare(to_f64(so[s]), ref, "fp8" if w.attn_fp8 else w.dtype)
        print(f"  chunk {n} step {s + 1} vs oracle: {m}", flush=True)
        assert ok, (kind, n, s, m)
    # Replays do not move the host bookkeeping: it stays at the end of the recorded chunks.  After a
    # whole number of ring periods of replays the device ring is back in that layout, and eager
    # calls on the recording cache continue the stream: the next eager chunk equals the eager
    # cache's bit for bit.
    n += 1
    while (n - first) % period:
        qkv, extra = inputs(n)
        eager_chunk(n, qkv, extra)
        fill_static(qkv, extra)
        graphs[(n - first) % period].launch()
        side.synchronize()
        n += 1
    qkv, extra = inputs(n)
    ref = eager_chunk(n, qkv, extra)
    got = eager_chunk(n, qkv, extra, cache=rec)
    for s in range(T):
        assert torch.equal(got[s], ref[s]), (kind, "eager after replays", n, s)
    print(f"  chunk {n}: eager call after {(n - first) // period} periods of replays equal", flush=True)
    for g in graphs:
        g.close()
