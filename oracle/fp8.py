"""Reduced-precision (fp8) chunk attention, plainly in float64 (test infrastructure).

The pages' stack chooses quantised attention per layer (Vidu S2 paper read,
section 2.4, the attention cut: SageAttention and relatives where a layer
tolerates the approximation; "Vidu S2 vs PixVerse R2" blog, section "Choice 4:
where the speed comes from").  They give no scheme; this one is built for the
scaled fp8 matrix instructions of CDNA4 and is defined here step by step:

* Element format: OCP FP8 E4M3 (bias 7, no infinities, largest finite 448,
  subnormals down to 2^-9), round to nearest, ties to even.
* Groups of 32 values share a power-of-two scale 2^e (an E8M0 exponent),
  e = ceil(log2(amax / 448)) for the group's largest magnitude amax (e = -127
  for an all-zero group), so the scaled values never exceed 448.  A value x
  is stored as the E4M3 rounding of x / 2^e and read back as that times 2^e.
* K is quantised after its rotation at block-local positions (t = frame in the
  block, h, w), in groups of 32 consecutive channels of one key and head.
* V is quantised per channel and head within each 64-key block, in two groups:
  its first 32 keys and its last 32 keys.
* Q is quantised for each cache slot separately, after its rotation at the
  relocated time of that slot (the query carries the relocation) and its
  multiplication by the softmax scale in base 2, log2(e) / sqrt(d), in groups of
  32 consecutive channels of one query and head: its products with K are then
  scores in base-2 units, and the softmax takes powers of two.
* Scores, softmax and the weighted sum of V are exact (float64) on the
  dequantised values.  (The GPU kernel also rounds the probabilities to E4M3
  before the product with V; that rounding is what the GPU tolerance covers.)
"""
from __future__ import annotations

import numpy as np

from . import rope

E4M3_MAX = 448.0


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value (ties to even), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # quantum: 2^(e-3) for a normal magnitude in [2^e, 2^(e+1)), 2^-9 below the normal range
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    q = np.ldexp(1.0, e - 3)
    y = np.round(a / q) * q                              # numpy rounds halves to even
    y = np.minimum(y, E4M3_MAX)
    return np.where(x < 0, -y, y)


def e8m0_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer e with amax / 2^e <= 448 (-127 for amax = 0), clipped to [-127, 127]."""
    amax = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(np.where(amax > 0, amax, 1.0))     # amax = m * 2^ex, 448 = 0.875 * 2^9
    e = ex - 9 + (m > 0.875).astype(np.int64)
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127)


def quantize_groups(x: np.ndarray, axis: int = -1, group: int = 32) -> np.ndarray:
    """Dequantised values of x after E4M3 + E8M0 quantisation in groups of `group` consecutive
    entries along `axis` (its length must be a multiple of `group`)."""
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    shp = xm.shape
    g = xm.reshape(shp[:-1] + (shp[-1] // group, group))
    e = e8m0_exponent(np.abs(g).max(axis=-1, keepdims=True))
    y = e4m3_round(np.ldexp(g, -e)) * np.ldexp(1.0, e)
    return np.moveaxis(y.reshape(shp), -1, axis)


def quantize_v(v: np.ndarray) -> np.ndarray:
    """V [N, ...] (keys first): per channel, per 64-key block, the first 32 keys form one group
    and the last 32 the other.  A short last block pads with zeros."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    n64 = -(-n // 64) * 64
    vp = np.zeros((n64,) + v.shape[1:])
    vp[:n] = v
    blk = vp.reshape((n64 // 64, 64) + v.shape[1:])
    out = quantize_groups(blk, axis=1, group=32)          # keys 0..31 and 32..63 of each block
    return out.reshape(vp.shape)[:n]


def key_local(w, stored_k: np.ndarray, head: int, as_f64) -> np.ndarray:
    """Dequantised K [B, d] of one head: rotated at block-local positions, then quantised."""
    x = as_f64(w, stored_k[:, head, :])
    f, hh, ww = rope.block_grid(stored_k.shape[0] // (w.lat_h * w.lat_w), w.lat_h, w.lat_w)
    return quantize_groups(rope.rotate(x, rope.angles(f, hh, ww, w.head_dim, w.rope_theta, w.rope_split)))


def score_scale(w) -> float:
    """The softmax scale in base 2: exp(q.k / sqrt(d)) = 2^(q.k * log2(e) / sqrt(d))."""
    return float(np.log2(np.e) / np.sqrt(w.head_dim))


def query_for_slot(w, stored_q: np.ndarray, head: int, delta: int, as_f64) -> np.ndarray:
    """Dequantised Q [B, d] of one head, rotated at block-local time + delta (the slot's
    relocation: time base of the current block minus that of the slot), multiplied by the
    softmax scale in base 2, then quantised."""
    x = as_f64(w, stored_q[:, head, :])
    f, hh, ww = rope.block_grid(stored_q.shape[0] // (w.lat_h * w.lat_w), w.lat_h, w.lat_w)
    rotated = rope.rotate(x, rope.angles(f + delta, hh, ww, w.head_dim, w.rope_theta, w.rope_split))
    return quantize_groups(rotated * score_scale(w))


def attend_head(w, head: int, q_stored, slots, bases, rows, as_f64, row_block: int = 512):
    """(O [rows, d], LSE [rows]) of one head with fp8-quantised Q, K, V (see the module notes).

    slots: [(role, block, K_stored, V_stored)] in logical order, the current block last; bases:
    their time bases.  The scores against slot l use the queries quantised for that slot; they
    are in base-2 units (the scale is in Q), and the LSE is returned in natural units."""
    rows = np.asarray(rows)
    ks = [key_local(w, k, head, as_f64) for (_, _, k, _) in slots]
    vs = np.concatenate([quantize_v(as_f64(w, v[:, head, :])) for (_, _, _, v) in slots], axis=0)
    qs = [query_for_slot(w, q_stored, head, bases[-1] - bases[l], as_f64)[rows] for l in range(len(slots))]
    o = np.empty((rows.size, w.head_dim))
    lse = np.empty(rows.size)
    for r0 in range(0, rows.size, row_block):
        r1 = min(rows.size, r0 + row_block)
        sc = np.concatenate([qs[l][r0:r1] @ ks[l].T for l in range(len(slots))], axis=1)
        m = sc.max(axis=1, keepdims=True)
        e = np.exp2(sc - m)
        den = e.sum(axis=1, keepdims=True)
        o[r0:r1] = (e @ vs) / den
        lse[r0:r1] = ((m + np.log2(den)) * np.log(2.0))[:, 0]
    return o, lse
