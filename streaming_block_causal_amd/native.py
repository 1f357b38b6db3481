"""ctypes binding of libswattn.so -- argument marshalling only.

Every function here has the name of the C entry point it wraps (include/swattn.h)
and does nothing but check/convert arguments and raise on a non-zero status.
All computation happens in the HIP kernels behind the C ABI; when the library
is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# SWATTN_LIB: another build of the same library (the sanitizer build of the host code)
LIB_PATH = os.environ.get("SWATTN_LIB") or os.path.join(HERE, "libswattn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "swattn.h")

SW_OK, SW_ERR_INVALID_ARG, SW_ERR_SHAPE, SW_ERR_STATE, SW_ERR_CAPACITY, SW_ERR_UNSUPPORTED, SW_ERR_HIP = range(7)
STATUS_NAMES = ["SW_OK", "SW_ERR_INVALID_ARG", "SW_ERR_SHAPE", "SW_ERR_STATE", "SW_ERR_CAPACITY",
                "SW_ERR_UNSUPPORTED", "SW_ERR_HIP"]
SW_BF16, SW_F32, SW_FP8 = 0, 1, 2
SW_KV_CURRENT, SW_KV_CLEAN, SW_KV_NOISY, SW_KV_SOURCE = 0, 1, 2, 3
SW_STEP_INTERMEDIATE, SW_STEP_FINAL = 0, 1
SW_ROPE_S1_RELOCATE, SW_ROPE_RELATIVE_TIME = 0, 1


class sw_cache_config(ctypes.Structure):
    _fields_ = [
        ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("frames_per_block", ctypes.c_int32), ("lat_h", ctypes.c_int32), ("lat_w", ctypes.c_int32),
        ("n_sink", ctypes.c_int32), ("n_window", ctypes.c_int32),
        ("twin", ctypes.c_int32), ("sparse", ctypes.c_int32),
        ("dtype", ctypes.c_int), ("rope_theta", ctypes.c_double),
        ("rope_pairs_t", ctypes.c_int32), ("rope_pairs_h", ctypes.c_int32), ("rope_pairs_w", ctypes.c_int32),
        ("policy", ctypes.c_int),
        ("tile", ctypes.c_int32), ("editing", ctypes.c_int32),
    ]


class sw_slot_info(ctypes.Structure):
    _fields_ = [("role", ctypes.c_int32), ("block_id", ctypes.c_int64), ("physical_slot", ctypes.c_int32),
                ("time_base", ctypes.c_int32), ("twin_complete", ctypes.c_int32), ("frames", ctypes.c_int32)]


class SwError(RuntimeError):
    def __init__(self, status: int, fn: str, message: str):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{fn}: {name}: {message}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libswattn.so (raises ImportError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m streaming_block_causal_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        H = ctypes.c_void_p
        sigs = {
            "sw_last_error": ([], ctypes.c_char_p),
            "sw_cache_required_bytes": ([ctypes.POINTER(sw_cache_config), ctypes.POINTER(SZ)], ctypes.c_int),
            "sw_cache_create": ([ctypes.POINTER(sw_cache_config), P, SZ, P, ctypes.POINTER(H)], ctypes.c_int),
            "sw_cache_destroy": ([H], ctypes.c_int),
            "sw_cache_append_block": ([H, ctypes.c_int, P, P, I64], ctypes.c_int),
            "sw_cache_append_block_frames": ([H, ctypes.c_int, P, P, I64, I32], ctypes.c_int),
            "sw_cache_append_qkv": ([H, P, P, P, F32, P, I64, I32], ctypes.c_int),
            "sw_cache_evict": ([H], ctypes.c_int),
            "sw_rope_relocate": ([H, ctypes.c_int], ctypes.c_int),
            "sw_tile_mask_budget": ([H, F32, ctypes.POINTER(I32)], ctypes.c_int),
            "sw_build_tile_mask": ([H, P, ctypes.c_int, F32, P, I32, ctypes.POINTER(I32)], ctypes.c_int),
            "sw_chunk_attend": ([H, P, ctypes.c_int, P, I32, P, P], ctypes.c_int),
            "sw_chunk_attend_noalloc": ([H, P, ctypes.c_int, P, I32, P, P], ctypes.c_int),
            "sw_cache_inspect": ([H, ctypes.POINTER(sw_slot_info), I32, ctypes.POINTER(I32)], ctypes.c_int),
            "sw_cache_read_slot": ([H, I32, ctypes.c_int, P, P], ctypes.c_int),
            "sw_graph_begin": ([H], ctypes.c_int),
            "sw_graph_end": ([H, ctypes.POINTER(H)], ctypes.c_int),
            "sw_graph_launch": ([H, P], ctypes.c_int),
            "sw_graph_destroy": ([H], ctypes.c_int),
            "sw_cache_ring_period": ([H, ctypes.POINTER(I32)], ctypes.c_int),
            "sw_probe_mfma": ([P, ctypes.c_int, I32, P, I32, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def declared_symbols(header: str = HEADER):
    """Names of the entry points include/swattn.h declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|sw_status)\s+(sw_\w+)\s*\(", text, re.M)))


def _check(status: int, fn: str):
    if status != SW_OK:
        raise SwError(status, fn, lib().sw_last_error().decode())


# ---- thin wrappers with the C names -------------------------------------------------
def sw_last_error() -> str:
    return lib().sw_last_error().decode()


def sw_cache_required_bytes(cfg: sw_cache_config) -> int:
    n = ctypes.c_size_t()
    _check(lib().sw_cache_required_bytes(ctypes.byref(cfg), ctypes.byref(n)), "sw_cache_required_bytes")
    return n.value


def sw_cache_create(cfg: sw_cache_config, pool_ptr: int, pool_bytes: int, stream_ptr: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().sw_cache_create(ctypes.byref(cfg), pool_ptr or None, pool_bytes, stream_ptr or None,
                                 ctypes.byref(h)), "sw_cache_create")
    return h.value


def sw_cache_destroy(handle: int) -> None:
    _check(lib().sw_cache_destroy(handle), "sw_cache_destroy")


def sw_cache_append_block(handle: int, kind: int, k_ptr: Optional[int], v_ptr: Optional[int], block_id: int):
    _check(lib().sw_cache_append_block(handle, kind, k_ptr or None, v_ptr or None, block_id),
           "sw_cache_append_block")


def sw_cache_append_block_frames(handle: int, kind: int, k_ptr: Optional[int], v_ptr: Optional[int],
                                 block_id: int, n_frames: int):
    _check(lib().sw_cache_append_block_frames(handle, kind, k_ptr or None, v_ptr or None, block_id, n_frames),
           "sw_cache_append_block_frames")


def sw_cache_append_qkv(handle: int, qkv_ptr: int, gq_ptr: int, gk_ptr: int, eps: float, q_out_ptr: int,
                        block_id: int, n_frames: int) -> None:
    _check(lib().sw_cache_append_qkv(handle, qkv_ptr or None, gq_ptr or None, gk_ptr or None, eps,
                                     q_out_ptr or None, block_id, n_frames), "sw_cache_append_qkv")


def sw_cache_evict(handle: int) -> None:
    _check(lib().sw_cache_evict(handle), "sw_cache_evict")


def sw_rope_relocate(handle: int, policy: int) -> None:
    _check(lib().sw_rope_relocate(handle, policy), "sw_rope_relocate")


def sw_tile_mask_budget(handle: int, keep_frac: float) -> int:
    k = ctypes.c_int32()
    _check(lib().sw_tile_mask_budget(handle, keep_frac, ctypes.byref(k)), "sw_tile_mask_budget")
    return k.value


def sw_build_tile_mask(handle: int, q_ptr: int, step: int, keep_frac: float, out_ptr: int, k_cap: int) -> int:
    k = ctypes.c_int32()
    _check(lib().sw_build_tile_mask(handle, q_ptr, step, keep_frac, out_ptr, k_cap, ctypes.byref(k)),
           "sw_build_tile_mask")
    return k.value


def sw_chunk_attend(handle: int, q_ptr: int, step: int, tile_ptr: Optional[int], k_row: int, out_ptr: int,
                    lse_ptr: Optional[int]) -> None:
    _check(lib().sw_chunk_attend(handle, q_ptr, step, tile_ptr or None, k_row, out_ptr, lse_ptr or None),
           "sw_chunk_attend")


def sw_chunk_attend_noalloc(handle: int, q_ptr: int, step: int, tile_ptr: Optional[int], k_row: int, out_ptr: int,
                            lse_ptr: Optional[int]) -> None:
    _check(lib().sw_chunk_attend_noalloc(handle, q_ptr, step, tile_ptr or None, k_row, out_ptr, lse_ptr or None),
           "sw_chunk_attend_noalloc")


def sw_cache_inspect(handle: int, cap: int = 16):
    arr = (sw_slot_info * cap)()
    n = ctypes.c_int32()
    _check(lib().sw_cache_inspect(handle, arr, cap, ctypes.byref(n)), "sw_cache_inspect")
    return [dict(role=("sink", "window", "current", "source")[s.role], block_id=s.block_id, physical_slot=s.physical_slot,
                 time_base=s.time_base, twin_complete=bool(s.twin_complete), frames=s.frames)
            for s in arr[:min(cap, n.value)]]


def sw_cache_read_slot(handle: int, logical_slot: int, kind: int, k_ptr: int, v_ptr: int) -> None:
    _check(lib().sw_cache_read_slot(handle, logical_slot, kind, k_ptr, v_ptr), "sw_cache_read_slot")


def sw_graph_begin(handle: int) -> None:
    _check(lib().sw_graph_begin(handle), "sw_graph_begin")


def sw_graph_end(handle: int) -> int:
    g = ctypes.c_void_p()
    _check(lib().sw_graph_end(handle, ctypes.byref(g)), "sw_graph_end")
    return g.value


def sw_graph_launch(graph: int, stream_ptr: Optional[int] = None) -> None:
    _check(lib().sw_graph_launch(graph, stream_ptr or None), "sw_graph_launch")


def sw_graph_destroy(graph: int) -> None:
    _check(lib().sw_graph_destroy(graph), "sw_graph_destroy")


def sw_cache_ring_period(handle: int) -> int:
    p = ctypes.c_int32()
    _check(lib().sw_cache_ring_period(handle, ctypes.byref(p)), "sw_cache_ring_period")
    return p.value


def sw_probe_mfma(stream_ptr: Optional[int], dtype: int, iters: int, sink_ptr: int, sink_floats: int) -> float:
    """Enqueue the matrix-core rate probe; returns the launch's flops (time it on the stream)."""
    f = ctypes.c_double()
    st = lib().sw_probe_mfma(stream_ptr or None, dtype, iters, sink_ptr, sink_floats, ctypes.byref(f))
    if st != SW_OK:
        raise SwError(st, "sw_probe_mfma", "invalid arguments, short sink or launch failure")
    return f.value
