"""Brute-force check of the streaming call: full attention over the whole stream.

Independent of the cache model in ``cache.py`` and of ``attention.attend``: it
lays out every token of blocks 0..n, decides visibility of each key block by a
predicate on (block id, query block id), places visible blocks at the times a
training clip of the same visible length would give them, rotates with complex
exponentials, and runs torch's scaled_dot_product_attention in float64 under
an explicit boolean mask.  Meant for tiny workloads only.

Sources: "Vidu S2 vs PixVerse R2" blog (orkas.ai), sections "What real-time
changes" (each block sees only earlier blocks) and "Choice 3: bounded memory"
(permanent first blocks, a window of recent blocks, positions kept inside the
trained range).  Editing streams (Vidu S2 paper read, section 2.6): every source
frame that has arrived is laid out too, and a source frame is visible to a query
exactly when both belong to the same instant of the stream (the same global
frame index), never across instants.
"""
from __future__ import annotations

import numpy as np
import torch

import synth


def visible_block(b: int, n: int, n_sink: int, n_window: int) -> bool:
    """Is block b part of the context of query block n?"""
    if b == n:
        return True
    if b > n:
        return False                      # the future is never visible
    if b < n_sink:
        return True                       # sink blocks are pinned for good
    return n_window > 0 and b >= n - n_window


def start_times(n: int, w: synth.Workload):
    """Start time of each visible block b <= n (dict), from the visible layout: a visible block
    starts where the visible blocks before it end; relative time puts the visible sinks before 0."""
    vis = [b for b in range(n + 1) if visible_block(b, n, w.n_sink, w.n_window)]
    sink_frames = sum(synth.frames_of(w, b) for b in vis if b < w.n_sink and b != n)
    shift = -sink_frames if w.policy == "relative" else 0
    return {b: sum(synth.frames_of(w, c) for c in vis if c < b) + shift for b in vis}


def instant(w: synth.Workload, b: int, f):
    """Global frame index (instant of the stream) of frame f of block b."""
    return sum(synth.frames_of(w, c) for c in range(b)) + f


def _pair_angles(t, h, wcol, head_dim, theta, split=None):
    p_all = head_dim // 2
    if split is None:
        ph = pw = p_all // 3
        pt = p_all - ph - pw
    else:
        pt, ph, pw = split
    out = np.empty(t.shape + (p_all,), dtype=np.float64)
    for p in range(p_all):
        if p < pt:
            out[..., p] = t * theta ** (-p / pt)
        elif p < pt + ph:
            out[..., p] = h * theta ** (-(p - pt) / ph)
        else:
            out[..., p] = wcol * theta ** (-(p - pt - ph) / pw)
    return out


def _rope_complex(x, t, h, wcol, theta, split=None):
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * np.exp(1j * _pair_angles(t, h, wcol, x.shape[-1], theta, split))
    y = np.empty_like(x)
    y[..., 0::2], y[..., 1::2] = z.real, z.imag
    return y


def chunk(w: synth.Workload, n: int, s: int, seed: int = 0, contents=None):
    """(O [B, H, d], LSE [H, B]) of query block n at step s, by brute force."""
    H, d = w.n_heads, w.head_dim

    def grid(b):
        tok = np.arange(synth.block_shape(w, b)[0])
        return tok // (w.lat_h * w.lat_w), (tok // w.lat_w) % w.lat_h, tok % w.lat_w

    B = synth.block_shape(w, n)[0]
    times = start_times(n, w)
    q_st, k_cur, v_cur = synth.qkv(w, n, s, seed)
    ks, vs, key_block = [], [], []
    for b in range(n + 1):
        if b == n:
            k_st, v_st = k_cur, v_cur
        else:
            kind = "noisy" if (w.twin and s < w.n_steps) else "clean"
            if contents is not None:
                k_st, v_st = contents(b, kind)
            elif kind == "clean":
                k_st, v_st = synth.committed_kv(w, b, seed)
            else:
                k_st, v_st = synth.noisy_kv(w, b, seed)
        t0 = times.get(b, 0)
        f, hh, wc = grid(b)
        ks.append(_rope_complex(synth.as_f64(w, k_st), (t0 + f)[:, None], hh[:, None], wc[:, None],
                                w.rope_theta, w.rope_split))
        vs.append(synth.as_f64(w, v_st))
        key_block.append(np.full(f.size, b))
    f, hh, wc = grid(n)
    q = _rope_complex(synth.as_f64(w, q_st), (times[n] + f)[:, None], hh[:, None], wc[:, None],
                      w.rope_theta, w.rope_split)
    k = np.concatenate(ks, 0)
    v = np.concatenate(vs, 0)
    kb = np.concatenate(key_block)
    allowed = np.array([visible_block(int(b), n, w.n_sink, w.n_window) for b in kb])
    mask = np.broadcast_to(allowed, (B, kb.size))
    if w.editing and n >= 1:
        # source frames of every block that has arrived, at their target block's positions
        sk, sv, s_inst = [], [], []
        for b in range(1, n + 1):
            k_src, v_src = synth.source_kv(w, b, seed) if contents is None else contents(b, "source")
            t0 = times.get(b, 0)
            fb, hb, wb = grid(b)
            sk.append(_rope_complex(synth.as_f64(w, k_src), (t0 + fb)[:, None], hb[:, None], wb[:, None],
                                    w.rope_theta, w.rope_split))
            sv.append(synth.as_f64(w, v_src))
            s_inst.append(instant(w, b, fb))
        s_inst = np.concatenate(s_inst)
        q_inst = instant(w, n, f)
        k = np.concatenate([k] + sk, 0)
        v = np.concatenate([v] + sv, 0)
        mask = np.concatenate([mask, q_inst[:, None] == s_inst[None, :]], axis=1)
    mask = torch.from_numpy(np.ascontiguousarray(mask))
    qt = torch.from_numpy(q).permute(1, 0, 2)          # [H, B, d]
    kt = torch.from_numpy(k).permute(1, 0, 2)
    vt = torch.from_numpy(v).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    # LSE from the same masked scores, for the normaliser check
    sc = (qt @ kt.transpose(1, 2)) / np.sqrt(d)
    sc = sc.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(sc, dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.numpy()
