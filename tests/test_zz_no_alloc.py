"""GPU: the allocation-free attention entry point against sw_chunk_attend, through the C ABI.

sw_chunk_attend_noalloc takes the split workspace (partial results of the query tiles the
dense launch cuts into key ranges) from a static device array instead of the cache pool and
makes the same work split, so its output and LSE must equal sw_chunk_attend's bit for bit --
which is inside the parity bar (helpers.TOL) a fortiori.  Calls in a row on one device: a
540p dense chunk (64 tiles cut into 256 pieces), then a smaller block (2 frames, 4080 tokens),
then a 540p fp8 chunk (512 pieces of 128 rows); each reuses the array the previous call
left.  A block too small to fill the device with query tiles would need a larger split than
the array holds: SW_ERR_CAPACITY, while the pool call still works.
"""
import ctypes

import numpy as np
import pytest

import synth

from .helpers import advance, compare, config_for, to_dev, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _noalloc():
    from streaming_block_causal_amd import native
    fn = native.lib().sw_chunk_attend_noalloc
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int32,
                   ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn, native


def _pair(w, n=5, s=1):
    """(pool call, allocation-free call) outputs and LSEs of chunk n, step s of workload w."""
    from streaming_block_causal_amd.cache import Cache
    fn, native = _noalloc()
    c = Cache(config_for(w), device="cuda")
    advance(c, w, n)
    q, k, v = synth.qkv(w, n, s)
    c.append("current", to_dev(w, k), to_dev(w, v), n)
    qd = to_dev(w, q)
    step = "final" if s == w.n_steps else "intermediate"
    lse_a = torch.empty((w.n_heads, w.block_tokens), dtype=torch.float32, device="cuda")
    out_a = c.attend(qd, step, lse=lse_a)
    out_b = torch.full_like(out_a, float("nan"))
    lse_b = torch.full_like(lse_a, float("nan"))
    st = fn(c.handle, qd.data_ptr(), 1 if step == "final" else 0, None, 0, out_b.data_ptr(), lse_b.data_ptr())
    torch.cuda.synchronize()
    assert st == native.SW_OK, native.sw_last_error()
    return c, out_a, lse_a, out_b, lse_b


def _same(w, label, **kw):
    print(f"[noalloc] {label} B={w.block_tokens}", flush=True)
    c, oa, la, ob, lb = _pair(w, **kw)
    ok, m = compare(to_f64(ob), to_f64(oa), "fp8" if w.attn_fp8 else w.dtype, to_f64(lb), to_f64(la))
    print(f"  vs sw_chunk_attend: {m}", flush=True)
    assert ok, m
    assert torch.equal(oa, ob) and torch.equal(la, lb), label


def test_noalloc_equals_pool_call_twice_then_fp8():
    _same(synth.WORKLOADS[2], "540p dense chunk 5")
    _same(synth.WORKLOADS[2].replace(frames=2), "540p 2-frame block (smaller)", n=4, s=2)
    _same(synth.WORKLOADS[8], "540p fp8 chunk 5")


def test_noalloc_rejects_a_split_larger_than_the_array():
    from streaming_block_causal_amd.cache import Cache
    fn, native = _noalloc()
    w = synth.WORKLOADS[2].replace(frames=1)            # 2040 tokens: 192 query tiles < 256 CUs
    c = Cache(config_for(w), device="cuda")
    advance(c, w, 4)
    q, k, v = synth.qkv(w, 4, 1)
    c.append("current", to_dev(w, k), to_dev(w, v), 4)
    qd = to_dev(w, q)
    out = torch.empty_like(qd)
    st = fn(c.handle, qd.data_ptr(), 0, None, 0, out.data_ptr(), None)
    assert st == native.SW_ERR_CAPACITY, (st, native.sw_last_error())
    assert "static scratch" in native.sw_last_error()
    ref = c.attend(qd, "intermediate")                  # the pool call still works
    torch.cuda.synchronize()
    assert bool(torch.isfinite(ref.float()).all())
