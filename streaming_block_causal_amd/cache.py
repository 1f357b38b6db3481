"""torch-facing wrapper of the C ABI: owns the device pool, checks tensors, calls native.

Marshalling only -- device memory and streams come from PyTorch, all compute runs
in libswattn's HIP kernels.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import torch

from . import native

# cache dtype -> (C enum, torch dtype of inputs and outputs); fp8 caches take and return bf16
_DTYPES = {"bf16": (native.SW_BF16, torch.bfloat16), "f32": (native.SW_F32, torch.float32),
           "fp8": (native.SW_FP8, torch.bfloat16)}
_POLICY = {"s1": native.SW_ROPE_S1_RELOCATE, "relative": native.SW_ROPE_RELATIVE_TIME}
KIND = {"current": native.SW_KV_CURRENT, "clean": native.SW_KV_CLEAN, "noisy": native.SW_KV_NOISY,
        "source": native.SW_KV_SOURCE}
STEP = {"intermediate": native.SW_STEP_INTERMEDIATE, "final": native.SW_STEP_FINAL}


@dataclasses.dataclass
class CacheConfig:
    n_heads: int
    head_dim: int
    frames_per_block: int
    lat_h: int
    lat_w: int
    n_sink: int
    n_window: int
    twin: bool = False
    sparse: bool = False
    dtype: str = "bf16"
    rope_theta: float = 10000.0
    policy: str = "s1"
    tile: int = 128
    editing: bool = False
    rope_pairs: Optional[Tuple[int, int, int]] = None   # (time, height, width) pairs; None: default split

    @property
    def block_tokens(self) -> int:
        return self.frames_per_block * self.lat_h * self.lat_w

    def to_c(self) -> native.sw_cache_config:
        return native.sw_cache_config(
            n_heads=self.n_heads, head_dim=self.head_dim, frames_per_block=self.frames_per_block,
            lat_h=self.lat_h, lat_w=self.lat_w, n_sink=self.n_sink, n_window=self.n_window,
            twin=int(self.twin), sparse=int(self.sparse), dtype=_DTYPES[self.dtype][0],
            rope_theta=self.rope_theta, policy=_POLICY[self.policy], tile=self.tile, editing=int(self.editing),
            **dict(zip(("rope_pairs_t", "rope_pairs_h", "rope_pairs_w"), self.rope_pairs or (0, 0, 0))))


class Cache:
    """A sink + window KV cache on one GPU (or metadata-only with device=None)."""

    def __init__(self, cfg: CacheConfig, device: Optional[str] = "cuda", stream: Optional[torch.cuda.Stream] = None):
        self.cfg = cfg
        self._c = cfg.to_c()
        self.nbytes = native.sw_cache_required_bytes(self._c)
        self.torch_dtype = _DTYPES[cfg.dtype][1]
        self.shape = (cfg.block_tokens, cfg.n_heads, cfg.head_dim)
        self.cur_frames = cfg.frames_per_block   # frames of the staged current block
        self.device = device
        if device is None:
            self.pool = None
            self.stream = None
            self.handle = native.sw_cache_create(self._c, 0, 0, 0)
        else:
            self.stream = stream if stream is not None else torch.cuda.current_stream(device)
            # the pool belongs to the stream its kernels run on: the allocator hands it back only
            # after that stream's work
            with torch.cuda.stream(self.stream):
                self.pool = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
            self.handle = native.sw_cache_create(self._c, self.pool.data_ptr(), self.nbytes,
                                                 self.stream.cuda_stream)
        self._capturing = False

    def close(self):
        if getattr(self, "handle", None):
            native.sw_cache_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ---- checks -----------------------------------------------------------------
    def _tensor(self, t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
        if self.device is None:
            return 1 if t is not None else 0          # metadata-only: only NULL-ness matters
        dtype = dtype or self.torch_dtype
        shape = shape or self.shape
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != dtype or tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}: expected {dtype} {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous CUDA tensor")
        if t.device != self.pool.device:
            raise ValueError(f"{name} is on {t.device}, the cache on {self.pool.device}")
        return t.data_ptr()

    # ---- stream order ------------------------------------------------------------
    # The kernels run on the cache's stream.  When the caller's current stream is another one,
    # the cache's stream first waits for the current stream (inputs written there), and after the
    # call the current stream waits for the cache's (outputs read there); tensors the kernels use
    # are recorded on the cache's stream so that the allocator does not reuse them early.  Not
    # while a graph is being recorded: the recording covers the cache's stream only.
    def _enter(self):
        if self.device is None or self._capturing:
            return None
        cur = torch.cuda.current_stream(self.pool.device)
        if cur == self.stream:
            return None
        self.stream.wait_stream(cur)
        return cur

    def _leave(self, cur, *tensors):
        if cur is None:
            return
        for t in tensors:
            if isinstance(t, torch.Tensor):
                t.record_stream(self.stream)
        cur.wait_stream(self.stream)

    # ---- the C calls -----------------------------------------------------------
    def shape_of(self, frames: int):
        return (frames * self.cfg.lat_h * self.cfg.lat_w, self.cfg.n_heads, self.cfg.head_dim)

    def append(self, kind: str, k: Optional[torch.Tensor], v: Optional[torch.Tensor], block_id: int,
               n_frames: Optional[int] = None):
        """Append a block (see sw_cache_append_block); n_frames: a block shorter than the cap."""
        shape = self.shape_of(n_frames) if n_frames is not None else self.shape
        kp = self._tensor(k, "k", shape=shape) if k is not None else 0
        vp = self._tensor(v, "v", shape=shape) if v is not None else 0
        cur = self._enter()
        if n_frames is None:
            native.sw_cache_append_block(self.handle, KIND[kind], kp, vp, block_id)
        else:
            native.sw_cache_append_block_frames(self.handle, KIND[kind], kp, vp, block_id, n_frames)
        self._leave(cur, k, v)
        if kind == "current":
            self.cur_frames = self.cfg.frames_per_block if n_frames is None else n_frames

    def append_qkv(self, qkv: torch.Tensor, gamma_q: torch.Tensor, gamma_k: torch.Tensor, eps: float,
                   block_id: int, q_out: Optional[torch.Tensor] = None, n_frames: Optional[int] = None):
        """Stage the current block from a packed QKV projection output [B][3][H][d], RMSNorm of q
        and k fused in (see sw_cache_append_qkv); returns the normalised q [B][H][d]."""
        n_frames = self.cfg.frames_per_block if n_frames is None else n_frames
        shape = self.shape_of(n_frames)
        if q_out is None and self.device is not None:
            q_out = torch.empty(shape, dtype=self.torch_dtype, device=self.device)
        qkv_shape = (shape[0], 3, shape[1], shape[2])
        args = (self._tensor(qkv, "qkv", shape=qkv_shape), self._tensor(gamma_q, "gamma_q", torch.float32, (shape[2],)),
                self._tensor(gamma_k, "gamma_k", torch.float32, (shape[2],)), eps,
                self._tensor(q_out, "q_out", shape=shape), block_id, n_frames)
        cur = self._enter()
        native.sw_cache_append_qkv(self.handle, *args)
        self._leave(cur, qkv, gamma_q, gamma_k, q_out)
        self.cur_frames = n_frames
        return q_out

    def evict(self):
        native.sw_cache_evict(self.handle)

    def relocate(self, policy: str):
        native.sw_rope_relocate(self.handle, _POLICY[policy])

    def mask_budget(self, keep_frac: float) -> int:
        return native.sw_tile_mask_budget(self.handle, keep_frac)

    def build_tile_mask(self, q: torch.Tensor, keep_frac: float, out: Optional[torch.Tensor] = None,
                        k_cap: Optional[int] = None, step: str = "final"):
        """Tile mask of this step's queries over the keys `step` reads (see sw_build_tile_mask)."""
        nt = -(-self.cfg.block_tokens // self.cfg.tile)
        k_cap = k_cap or self.mask_budget(keep_frac)
        if out is None:
            out = torch.empty((self.cfg.n_heads, nt, k_cap), dtype=torch.int32, device=self.device)
        op = self._tensor(out, "tile_idx_out", torch.int32, (self.cfg.n_heads, nt, k_cap))
        qp = self._tensor(q, "q")
        cur = self._enter()
        k_row = native.sw_build_tile_mask(self.handle, qp, STEP[step], keep_frac, op, k_cap)
        self._leave(cur, q, out)
        return out, k_row

    def attend(self, q: torch.Tensor, step: str = "final", tile_idx: Optional[torch.Tensor] = None,
               k_row: int = 0, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
        shape = self.shape_of(self.cur_frames)
        if out is None:
            out = torch.empty(shape, dtype=self.torch_dtype, device=self.device)
        tp = 0
        if tile_idx is not None:
            if tile_idx.dtype != torch.int32 or not tile_idx.is_cuda or not tile_idx.is_contiguous():
                raise ValueError("tile_idx must be a contiguous int32 CUDA tensor")
            if self.pool is not None and tile_idx.device != self.pool.device:
                raise ValueError(f"tile_idx is on {tile_idx.device}, the cache on {self.pool.device}")
            nt = -(-self.cfg.block_tokens // self.cfg.tile)
            if tuple(tile_idx.shape) != (self.cfg.n_heads, nt, k_row):
                raise ValueError(f"tile_idx shape {tuple(tile_idx.shape)} != {(self.cfg.n_heads, nt, k_row)}")
            tp = tile_idx.data_ptr()
        lp = self._tensor(lse, "lse", torch.float32, (self.cfg.n_heads, shape[0])) if lse is not None else 0
        qp, outp = self._tensor(q, "q", shape=shape), self._tensor(out, "out", shape=shape)
        cur = self._enter()
        native.sw_chunk_attend(self.handle, qp, STEP[step], tp, k_row, outp, lp)
        self._leave(cur, q, out, lse, tile_idx)
        return out

    def inspect(self):
        return native.sw_cache_inspect(self.handle)

    def read_slot(self, logical_slot: int, kind: str = "clean"):
        info = self.inspect()
        if kind in ("current", "source"):
            frames = self.cur_frames
        else:
            frames = info[logical_slot]["frames"]
        out_dtype = torch.float32 if self.cfg.dtype == "fp8" else self.torch_dtype   # fp8: dequantised
        k = torch.empty(self.shape_of(frames), dtype=out_dtype, device=self.device)
        v = torch.empty_like(k)
        cur = self._enter()
        native.sw_cache_read_slot(self.handle, logical_slot, KIND[kind], k.data_ptr(), v.data_ptr())
        self._leave(cur, k, v)
        return k, v

    # ---- graph replay (see sw_graph_begin) ------------------------------------------
    def ring_period(self) -> int:
        return native.sw_cache_ring_period(self.handle)

    def graph_begin(self):
        """Start recording this cache's stream; pass `out=` to attend while recording (no allocation)."""
        native.sw_graph_begin(self.handle)
        self._capturing = True

    def graph_end(self) -> "Graph":
        self._capturing = False
        return Graph(native.sw_graph_end(self.handle))


class Graph:
    """An instantiated recording of library calls; launch() replays it on the recorded stream."""

    def __init__(self, handle: int):
        self.handle = handle

    def launch(self, stream: Optional[torch.cuda.Stream] = None):
        native.sw_graph_launch(self.handle, stream.cuda_stream if stream is not None else None)

    def close(self):
        if getattr(self, "handle", None):
            native.sw_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
