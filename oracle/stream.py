"""One attention call of a streaming workload, computed plainly in float64.

For chunk n, denoising step s (1..T) and head h:

    O = softmax_k( <R(p_q) q, R(p_k) k> / sqrt(d) + M ) V

over the materialised keys [sink blocks, window blocks oldest->newest, current
block], positions p = (t, h, w) relocated as in ``rope.relocation_bases``, and
M = -inf only on key tiles the block-sparse mask drops.

Editing streams (frame-aligned attention: Vidu S2 paper read, section 2.6 on
the editing model; the BloomBook Vidu S2 tutorial, section "S2-Editing" and the
figure caption on the input structure; "Vidu S2 vs PixVerse R2" blog, section
"Choice 5: how people control it"): block 0 holds the reference image and stays
as a sink, seen by every frame; chunk n >= 1 also sees the source-video frames
that arrive with it, a query of frame f only the source frame of the same
instant f, at the same (t, h, w) positions as the target frame.  Source frames
are consumed with their chunk and never enter the history.

Sources: "Vidu S2 vs PixVerse R2" blog (orkas.ai), sections "What real-time
changes" (blocks in time order, each sees only the past), "Choice 3: bounded
memory" (sinks + sliding window, RoPE relocation / relative-time RoPE,
TwinCache noisy/clean reads) and "Choice 4: where the speed comes from"
(block-sparse attention).  Readings used: the current block attends to itself
bidirectionally; the block a chunk commits is its final-step K/V; with
TwinCache, steps 1..T-1 read the noisy copy of every history block (sinks
included) and step T reads the clean copy, while the current block always uses
its own step-s K/V.
"""
from __future__ import annotations

import os
from typing import Callable, Optional, Sequence

import numpy as np

import synth

from . import attention, cache, fp8, rope, tilemask


class Stream:
    """Walks a workload's cache model and computes any (chunk, step) call in fp64.

    `contents(block_id, kind)` may replace the stored K/V of a history block
    ('clean' or 'noisy') or a chunk's source frames ('source'); where it returns None
    (or is not given) blocks are the seeded draws.
    """

    def __init__(self, w: synth.Workload, seed: int = 0,
                 contents: Optional[Callable] = None, sigma_override: Optional[float] = None):
        self.w, self.seed = w, seed
        self.contents = contents
        self.sigma_override = sigma_override
        self._memo = {}

    # ---- cache state -------------------------------------------------------------
    def logical(self, n: int):
        model = cache.CacheModel(self.w.n_sink, self.w.n_window)
        for b in range(n):
            model.commit(b)
        return model.logical(n)

    def bases(self, n: int):
        lg = self.logical(n)
        w = self.w
        if w.frame_pattern is None and not w.editing:
            n_s = sum(1 for r, _ in lg if r == "sink")
            n_w = sum(1 for r, _ in lg if r == "window")
            return rope.relocation_bases(w.policy, n_s, n_w, w.frames)
        return rope.relocation_bases_frames(
            w.policy, [synth.frames_of(w, b) for r, b in lg if r == "sink"],
            [synth.frames_of(w, b) for r, b in lg if r == "window"], synth.frames_of(w, n))

    # ---- inputs ------------------------------------------------------------------
    def _kv(self, block: int, kind: str):
        key = (block, kind)
        if key not in self._memo:
            kv = self.contents(block, kind) if self.contents is not None else None
            if kv is None and kind == "clean":
                kv = synth.committed_kv(self.w, block, self.seed)
            elif kv is None:
                kv = synth.noisy_kv(self.w, block, self.seed, self.sigma_override)
            self._memo[key] = kv
        return self._memo[key]

    def slot_inputs(self, n: int, s: int, current=None):
        """[(role, block, K_stored, V_stored)] in logical order, plus Q_stored.

        current: optional (Q, K, V) storage arrays replacing the seeded draw.
        """
        w = self.w
        q, kc, vc = synth.qkv(w, n, s, self.seed) if current is None else current
        out = []
        for role, b in self.logical(n):
            if role == "current":
                out.append((role, b, kc, vc))
            else:
                kind = "noisy" if (w.twin and s < w.n_steps) else "clean"
                k, v = self._kv(b, kind)
                out.append((role, b, k, v))
        if w.editing and n >= 1:
            ks, vs = self.source(n)
            out.append(("source", n, ks, vs))
        return q, out

    def source(self, n: int):
        """Source-frame K/V of chunk n (replaceable through `contents(n, 'source')`)."""
        if self.contents is not None:
            kv = self.contents(n, "source")
            if kv is not None:
                return kv
        return synth.source_kv(self.w, n, self.seed)

    # ---- the call ----------------------------------------------------------------
    def call(self, n: int, s: int, heads: Optional[Sequence[int]] = None,
             rows: Optional[Sequence[int]] = None, kept=None, workers: int = 1,
             current=None):
        """Return (O [rows, heads, d], LSE [heads, rows], kept) for chunk n, step s.

        kept: None -> the workload decides (dense, or the oracle's own tile mask);
        otherwise a per-head list of per-query-tile kept key-tile lists.
        """
        w = self.w
        heads = list(range(w.n_heads)) if heads is None else list(heads)
        rows = np.arange(synth.block_shape(w, n)[0]) if rows is None else np.asarray(rows)
        q, slots = self.slot_inputs(n, s, current)
        bases = self.bases(n)
        if slots[-1][0] == "source":
            bases = bases + [bases[-1]]   # source frames sit at the current block's positions
        job = dict(w=w, q=q, slots=slots, bases=bases, rows=rows, kept=kept)
        if workers > 1 and len(heads) > 1:
            res = _pool_map(job, heads, workers)
        else:
            res = [_one_head(job, h) for h in heads]
        o = np.stack([r[0] for r in res], axis=1)
        lse = np.stack([r[1] for r in res], axis=0)
        return o, lse, [r[2] for r in res]


def relocated_head(w: synth.Workload, stored: np.ndarray, head: int, base: int) -> np.ndarray:
    """[B, d] float64 RoPE of one head of a stored block placed at time `base`."""
    x = synth.as_f64(w, stored[:, head, :])
    f, hh, ww = rope.block_grid(stored.shape[0] // (w.lat_h * w.lat_w), w.lat_h, w.lat_w)
    return rope.rotate(x, rope.angles(base + f, hh, ww, w.head_dim, w.rope_theta, w.rope_split))


def _one_head(job, h):
    w, q, slots, bases, rows = job["w"], job["q"], job["slots"], job["bases"], job["rows"]
    if w.attn_fp8:
        if job["kept"] is not None or w.sparse_keep is not None or slots[-1][0] == "source":
            raise ValueError("fp8 attention is built for the dense stream")
        o, lse = fp8.attend_head(w, h, q, slots, bases, rows, synth.as_f64)
        return o, lse, None
    q_rel = relocated_head(w, q, h, bases[-1])
    k_rel = [relocated_head(w, k, h, bases[l]) for l, (_, _, k, _) in enumerate(slots)]
    v_all = np.concatenate([synth.as_f64(w, v[:, h, :]) for (_, _, _, v) in slots], axis=0)
    k_all = np.concatenate(k_rel, axis=0)
    kept = None
    vis = None
    if slots[-1][0] == "source":
        if job["kept"] is not None or w.sparse_keep is not None:
            raise ValueError("frame-aligned editing attention is dense only")
        vis = _frame_aligned(w, rows, [k.shape[0] for (_, _, k, _) in slots])
    elif job["kept"] is not None:
        kept = job["kept"][h]
    elif w.sparse_keep is not None:
        kept, _, _ = tilemask.build(q_rel, k_rel, [r for r, _, _, _ in slots], w.sparse_keep, w.tile)
    if kept is not None:
        vis = tilemask.visible(kept, w.block_tokens, len(slots), w.tile)[rows]
    o, lse = attention.attend(q_rel[rows], k_all, v_all, vis)
    return o, lse, kept


def _frame_aligned(w: synth.Workload, rows, lengths):
    """Visibility [rows, keys] with the source block last: every history and current key is
    visible, a source key only to the queries of its own frame."""
    hw = w.lat_h * w.lat_w
    rows = np.asarray(rows)
    n_other = sum(lengths[:-1])
    src_frame = np.arange(lengths[-1]) // hw
    vis = np.ones((rows.size, n_other + lengths[-1]), dtype=bool)
    vis[:, n_other:] = (rows // hw)[:, None] == src_frame[None, :]
    return vis


_JOB = None


def _worker(h):
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        return _one_head(_JOB, h)


def _pool_map(job, heads, workers):
    import multiprocessing as mp
    global _JOB
    _JOB = job
    ctx = mp.get_context("fork")
    with ctx.Pool(min(workers, len(heads), os.cpu_count() or 1)) as pool:
        return pool.map(_worker, heads)
