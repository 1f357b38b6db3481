"""3D rotary position embedding and its relocation, in float64.

Sources: Vidu S2 paper read (yingwang.github.io), abbreviation table, RoPE
entry -- rotary positions tell attention where each token sits in space and
time.  "Vidu S2 vs PixVerse R2" blog, section "Choice 3: bounded memory" -- S1
relocates RoPE and R2 uses relative-time RoPE so that positions stay in the
range seen in training, however long the session runs.

The pages fix neither the split of the head dimension over (t, h, w), nor the
frequencies, nor the relocation formula.  Readings used (plainest ones):

* P = d/2 rotation pairs; pair p rotates dims (2p, 2p+1), time pairs first,
  then height, then width.  By default height and width get floor(P/3) pairs
  each and time the rest; a workload may give its own split (P_t, P_h, P_w).
* Inside an axis with P_a pairs, pair j turns at omega_j = theta^(-j/P_a),
  theta = 10000, by angle pos * omega_j; (x0, x1) -> (x0 cos - x1 sin,
  x0 sin + x1 cos).
* S1 relocation: the l-th block of the materialised sequence [sinks, window
  oldest->newest, current] starts at time l*F.  Relative-time: window j starts
  at j*F, the current block at n_w*F, sink i at (i - n_s)*F.  Both are the
  positions a training clip of the same length would have (up to a shift).
"""
from __future__ import annotations

import numpy as np


def axis_split(head_dim: int, split=None):
    """(pairs for time, height, width): the given split, or the default one."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    p = head_dim // 2
    if split is not None:
        pt, ph, pw = (int(x) for x in split)
        if min(pt, ph, pw) < 0 or pt + ph + pw != p:
            raise ValueError(f"RoPE split {split} does not cover {p} pairs")
        return pt, ph, pw
    third = p // 3
    return p - 2 * third, third, third


def axis_frequencies(n_pairs: int, theta: float) -> np.ndarray:
    j = np.arange(n_pairs, dtype=np.float64)
    return np.power(float(theta), -j / n_pairs) if n_pairs else np.zeros(0)


def angles(t, h, w, head_dim: int, theta: float = 10000.0, split=None) -> np.ndarray:
    """Rotation angle of every pair for tokens at positions (t, h, w) -> [..., d/2]."""
    pt, ph, pw = axis_split(head_dim, split)
    t = np.asarray(t, dtype=np.float64)[..., None]
    h = np.asarray(h, dtype=np.float64)[..., None]
    w = np.asarray(w, dtype=np.float64)[..., None]
    return np.concatenate([t * axis_frequencies(pt, theta),
                           h * axis_frequencies(ph, theta),
                           w * axis_frequencies(pw, theta)], axis=-1)


def rotate(x: np.ndarray, ang: np.ndarray) -> np.ndarray:
    """Apply the pair rotations: x [..., d], ang broadcastable to [..., d/2]."""
    x = np.asarray(x, dtype=np.float64)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    c, s = np.cos(ang), np.sin(ang)
    y = np.empty(np.broadcast_shapes(x.shape, x.shape), dtype=np.float64)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


def block_grid(frames: int, lat_h: int, lat_w: int):
    """Per-token (f, h, w) of one block in (frame, row, column) row-major order."""
    f, h, w = np.meshgrid(np.arange(frames), np.arange(lat_h), np.arange(lat_w), indexing="ij")
    return f.reshape(-1), h.reshape(-1), w.reshape(-1)


def relocation_bases(policy: str, n_sink: int, n_window: int, frames: int):
    """Start time of each logical slot [sinks..., window oldest->newest..., current]."""
    if policy == "s1":
        return [l * frames for l in range(n_sink + n_window + 1)]
    if policy == "relative":
        return ([(i - n_sink) * frames for i in range(n_sink)]
                + [j * frames for j in range(n_window)]
                + [n_window * frames])
    raise ValueError(f"unknown relocation policy {policy!r}")


def relocation_bases_frames(policy: str, sink_frames, window_frames, current_frames: int):
    """Start times of the logical slots when blocks have their own frame counts.

    S1: each slot starts where the previous one ends (cumulative frames in logical order, from 0).
    Relative-time: the window starts at 0 and runs oldest -> newest, the current block follows
    it, and the sinks sit just before time 0, back to back.  With every block at F frames these
    are ``relocation_bases`` exactly.
    """
    fr = [int(f) for f in sink_frames] + [int(f) for f in window_frames] + [int(current_frames)]
    starts = [0]
    for f in fr[:-1]:
        starts.append(starts[-1] + f)
    if policy == "s1":
        return starts
    if policy == "relative":
        shift = sum(int(f) for f in sink_frames)
        return [t - shift for t in starts]
    raise ValueError(f"unknown relocation policy {policy!r}")


def rotate_block(x: np.ndarray, base: int, frames: int, lat_h: int, lat_w: int,
                 theta: float = 10000.0, split=None) -> np.ndarray:
    """RoPE of a whole block [B, H, d] whose first frame sits at time `base`."""
    f, h, w = block_grid(frames, lat_h, lat_w)
    ang = angles(base + f, h, w, x.shape[-1], theta, split)      # [B, d/2]
    return rotate(x, ang[:, None, :])
