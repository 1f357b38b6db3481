"""Seeded synthetic inputs for streaming block-causal chunk attention.

This module describes the synthetic workloads (shapes, cache sizes,
stream lengths, value distributions) and draws their Q/K/V tensors from a
seed.  It computes no step of the attention method: it only draws numbers and
rounds fp32 draws to bfloat16 bit patterns, so that the fp64 oracle and the
GPU library consume exactly the same inputs.  Both sides import it; it imports
neither.

Every tensor of a workload is drawn from its own independent stream,
``numpy.random.default_rng([seed, cfg_id, chunk, step, tag])``, so any
(chunk, step) can be regenerated alone without replaying the stream.

Value recipe (the pages give no shapes; the workload descriptions do):

* Q, K, V ~ N(0, 1) * scale, shape ``[B, H, d]`` token-major, B = F * lat_h *
  lat_w tokens in (frame, row, column) row-major order.  bf16 workloads round
  the fp32 draw to nearest-even bfloat16.
* Steps are numbered 1..T; step T is the final denoising step.  The block a
  chunk commits to the history is its step-T K/V.
* TwinCache noisy copies: clean committed K (or V) upcast to fp32, plus
  sigma_b * N(0, 1) with sigma_b ~ U[0.3, 0.8] drawn once per block, then
  rounded to bfloat16.
* Variable-length blocks: a workload may give a frame pattern; block b then
  has pattern[b % len(pattern)] latent frames (at most `frames`, the cap) and
  every tensor of that block is drawn at its own length.
* Editing streams: block 0 holds the reference-image latents (`ref_frames`
  frames) and every later block b comes with the K/V of its source-video frames,
  drawn like a block's K/V at block b's shape, independent of the step.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "TAG_Q", "TAG_K", "TAG_V", "TAG_KN", "TAG_VN",
    "TAG_SIGMA", "rng", "round_bf16", "bf16_to_f32", "draw", "qkv",
    "committed_kv", "noisy_kv", "source_kv", "as_f64", "tiny", "frames_of", "block_shape",
]

TAG_Q, TAG_K, TAG_V, TAG_KN, TAG_VN, TAG_SIGMA, TAG_KS, TAG_VS = 0, 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic streaming workload (what the stream looks like, not how it is computed)."""

    name: str
    cfg_id: int
    n_heads: int
    head_dim: int
    frames: int            # latent frames per block (F)
    lat_h: int
    lat_w: int
    n_sink: int            # S
    n_window: int          # W
    n_chunks: int
    n_steps: int           # denoising steps per chunk (T)
    dtype: str             # "f32" or "bf16"
    scale: float           # std of the Q/K/V draws
    twin: bool = False
    sparse_keep: Optional[float] = None   # kept fraction of 128x128 tiles, None = dense
    policy: str = "s1"     # "s1" (slot relocation) or "relative" (relative-time)
    sigma_range: Tuple[float, float] = (0.3, 0.8)
    rope_theta: float = 10000.0
    rope_split: Optional[Tuple[int, int, int]] = None   # RoPE pairs (time, height, width); None: default
    tile: int = 128
    frame_pattern: Optional[Tuple[int, ...]] = None   # frames of block b = pattern[b % len]; None: `frames`
    editing: bool = False            # block 0 is the reference, blocks >= 1 carry source frames
    ref_frames: Optional[int] = None  # editing: latent frames of the reference block (None: as block 0)
    attn_fp8: bool = False           # attention on fp8 (E4M3, power-of-two group scales) Q, K, V

    @property
    def block_tokens(self) -> int:
        return self.frames * self.lat_h * self.lat_w

    @property
    def shape(self) -> Tuple[int, int, int]:
        return (self.block_tokens, self.n_heads, self.head_dim)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[int, Workload] = {
    1: Workload("c1_tiny_f32", 1, n_heads=4, head_dim=64, frames=3, lat_h=8, lat_w=8,
                n_sink=1, n_window=2, n_chunks=8, n_steps=1, dtype="f32", scale=1.0),
    2: Workload("c2_540p_dense_bf16", 2, n_heads=24, head_dim=128, frames=3, lat_h=34, lat_w=60,
                n_sink=1, n_window=3, n_chunks=32, n_steps=4, dtype="bf16", scale=0.5),
    3: Workload("c3_540p_twincache_bf16", 3, n_heads=24, head_dim=128, frames=3, lat_h=34,
                lat_w=60, n_sink=1, n_window=3, n_chunks=32, n_steps=4, dtype="bf16",
                scale=0.5, twin=True),
    4: Workload("c4_720p_refiner_bf16", 4, n_heads=24, head_dim=128, frames=3, lat_h=45,
                lat_w=80, n_sink=1, n_window=2, n_chunks=16, n_steps=1, dtype="bf16",
                scale=0.5, policy="relative"),
    5: Workload("c5_540p_blocksparse_bf16", 5, n_heads=24, head_dim=128, frames=3, lat_h=34,
                lat_w=60, n_sink=1, n_window=3, n_chunks=64, n_steps=4, dtype="bf16",
                scale=0.5, sparse_keep=0.08),
    # variable-length blocks (block length follows the control signal, capped): 1-frame blocks
    # for short controls, 2-3 frames for longer events; relative-time RoPE
    6: Workload("c6_540p_varlen_bf16", 6, n_heads=24, head_dim=128, frames=3, lat_h=34, lat_w=60,
                n_sink=1, n_window=3, n_chunks=32, n_steps=4, dtype="bf16", scale=0.5,
                policy="relative", frame_pattern=(3, 1, 1, 2, 3, 2, 1, 3)),
    # streaming video editing: a one-frame reference image pinned as the sink, a window of edited
    # (target) blocks, and per chunk the source-video frames of the same instants
    7: Workload("c7_540p_editing_bf16", 7, n_heads=24, head_dim=128, frames=3, lat_h=34, lat_w=60,
                n_sink=1, n_window=3, n_chunks=32, n_steps=4, dtype="bf16", scale=0.5,
                editing=True, ref_frames=1),
    # the 540p dense stream with attention on fp8-quantised Q, K, V (inputs still bf16)
    8: Workload("c8_540p_fp8", 8, n_heads=24, head_dim=128, frames=3, lat_h=34, lat_w=60,
                n_sink=1, n_window=3, n_chunks=32, n_steps=4, dtype="bf16", scale=0.5, attn_fp8=True),
}


def frames_of(w: Workload, block: int) -> int:
    """Latent frames of block `block` (the cap `w.frames` unless the workload has a pattern, or the
    block is an editing stream's reference)."""
    if w.editing and block == 0 and w.ref_frames is not None:
        f = int(w.ref_frames)
    elif w.frame_pattern is None:
        return w.frames
    else:
        f = int(w.frame_pattern[block % len(w.frame_pattern)])
    if not 1 <= f <= w.frames:
        raise ValueError(f"frame pattern entry {f} outside [1, {w.frames}]")
    return f


def block_shape(w: Workload, block: int) -> Tuple[int, int, int]:
    return (frames_of(w, block) * w.lat_h * w.lat_w, w.n_heads, w.head_dim)


def tiny(base: int = 1, **kw) -> Workload:
    """A small variant of a workload (for unit tests); keyword overrides win."""
    w = WORKLOADS[base]
    kw.setdefault("name", w.name + "_variant")
    return w.replace(**kw)


def rng(seed: int, cfg_id: int, chunk: int, step: int, tag: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(cfg_id), int(chunk), int(step), int(tag)])


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even (finite values:
    the 32-bit sum below cannot wrap for them)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return b.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(w: Workload, x32: np.ndarray) -> np.ndarray:
    return round_bf16(x32) if w.dtype == "bf16" else np.ascontiguousarray(x32, dtype=np.float32)


def as_f64(w: Workload, stored: np.ndarray) -> np.ndarray:
    """Exact value of a stored tensor (uint16 bf16 bits or float32) as float64."""
    if w.dtype == "bf16":
        return bf16_to_f32(stored).astype(np.float64)
    return np.asarray(stored, dtype=np.float64)


def as_f32(w: Workload, stored: np.ndarray) -> np.ndarray:
    return bf16_to_f32(stored) if w.dtype == "bf16" else np.asarray(stored, dtype=np.float32)


def draw(w: Workload, chunk: int, step: int, tag: int, seed: int = 0) -> np.ndarray:
    """One [B, H, d] tensor in storage form (uint16 bf16 bits, or float32)."""
    g = rng(seed, w.cfg_id, chunk, step, tag)
    x = g.standard_normal(size=block_shape(w, chunk), dtype=np.float32) * np.float32(w.scale)
    return _store(w, x)


def qkv(w: Workload, chunk: int, step: int, seed: int = 0):
    """(Q, K, V) of chunk `chunk` at denoising step `step` (1..T), storage form."""
    return (draw(w, chunk, step, TAG_Q, seed), draw(w, chunk, step, TAG_K, seed),
            draw(w, chunk, step, TAG_V, seed))


def committed_kv(w: Workload, block: int, seed: int = 0):
    """The clean K/V a block leaves in the history: its final-step draw."""
    return draw(w, block, w.n_steps, TAG_K, seed), draw(w, block, w.n_steps, TAG_V, seed)


def sigma(w: Workload, block: int, seed: int = 0) -> float:
    g = rng(seed, w.cfg_id, block, 0, TAG_SIGMA)
    lo, hi = w.sigma_range
    return float(g.uniform(lo, hi))


def source_kv(w: Workload, block: int, seed: int = 0):
    """K/V of the source-video frames that come with block `block` (>= 1) of an editing stream."""
    if not w.editing or block < 1:
        raise ValueError("source frames exist for blocks >= 1 of an editing workload")
    return draw(w, block, 0, TAG_KS, seed), draw(w, block, 0, TAG_VS, seed)


def noisy_kv(w: Workload, block: int, seed: int = 0, sigma_override: Optional[float] = None):
    """Noisy twin of a committed block: clean + sigma_b * N(0,1), rounded to storage."""
    kc, vc = committed_kv(w, block, seed)
    s = np.float32(sigma(w, block, seed) if sigma_override is None else sigma_override)
    out = []
    for stored, tag in ((kc, TAG_KN), (vc, TAG_VN)):
        g = rng(seed, w.cfg_id, block, w.n_steps, tag)
        n = g.standard_normal(size=block_shape(w, block), dtype=np.float32)
        out.append(_store(w, as_f32(w, stored) + s * n))
    return out[0], out[1]
