"""sw_cache_append_qkv on metadata-only handles (CPU only): it stages the current block like
SW_KV_CURRENT, and its argument checks (Vidu S2 paper read, section 2.4: RMSNorm fused with
elementwise work into one kernel)."""
import pytest

import synth
from streaming_block_causal_amd import native
from streaming_block_causal_amd.cache import Cache

from .helpers import config_for


def _dry(w):
    return Cache(config_for(w), device=None)


def test_stages_like_current_append():
    w = synth.WORKLOADS[2]
    a, b = _dry(w), _dry(w)
    for n in range(12):
        a.append("current", 1, 1, n)
        native.sw_cache_append_qkv(b.handle, 1, 1, 1, 1e-6, 1, n, w.frames)
        assert a.inspect() == b.inspect()
        if n >= 4:
            a.evict()
            b.evict()
        a.append("clean", None, None, n)
        b.append("clean", None, None, n)


def test_argument_checks():
    w = synth.WORKLOADS[2]
    c = _dry(w)
    for args, status in (((0, 1, 1, 1e-6, 1, 0, 3), native.SW_ERR_INVALID_ARG),    # NULL qkv
                         ((1, 0, 1, 1e-6, 1, 0, 3), native.SW_ERR_INVALID_ARG),    # NULL gamma_q
                         ((1, 1, 0, 1e-6, 1, 0, 3), native.SW_ERR_INVALID_ARG),    # NULL gamma_k
                         ((1, 1, 1, 1e-6, 0, 0, 3), native.SW_ERR_INVALID_ARG),    # NULL q_out
                         ((1, 1, 1, -1.0, 1, 0, 3), native.SW_ERR_INVALID_ARG),    # eps < 0
                         ((1, 1, 1, float("nan"), 1, 0, 3), native.SW_ERR_INVALID_ARG),
                         ((1, 1, 1, 1e-6, 1, 0, 4), native.SW_ERR_INVALID_ARG),    # n_frames > cap
                         ((1, 1, 1, 1e-6, 1, -1, 3), native.SW_ERR_INVALID_ARG)):  # block id
        with pytest.raises(native.SwError) as e:
            native.sw_cache_append_qkv(c.handle, *args)
        assert e.value.status == status, args
    assert c.inspect() == []                                   # nothing was staged
    native.sw_cache_append_qkv(c.handle, 1, 1, 1, 1e-6, 1, 0, 3)
    with pytest.raises(native.SwError) as e:                   # another id while 0 is staged
        native.sw_cache_append_qkv(c.handle, 1, 1, 1, 1e-6, 1, 1, 3)
    assert e.value.status == native.SW_ERR_STATE
    d64 = _dry(synth.WORKLOADS[1])
    with pytest.raises(native.SwError) as e:
        native.sw_cache_append_qkv(d64.handle, 1, 1, 1, 1e-6, 1, 0, 3)
    assert e.value.status == native.SW_ERR_UNSUPPORTED
