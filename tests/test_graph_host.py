"""Graph-replay entry points on metadata-only handles (CPU only): argument and state checks.

Replaying a stable launch sequence (Vidu S2 paper read, section 2.4, the kernel-level
cut: adjacent operators fused and the steady sequence captured once and replayed)."""
import ctypes

import pytest

import synth
from streaming_block_causal_amd import native
from streaming_block_causal_amd.cache import Cache

from .helpers import config_for


@pytest.mark.parametrize("W", [0, 1, 3, 14])
def test_ring_period_is_window_plus_one(W):
    c = Cache(config_for(synth.WORKLOADS[2].replace(n_window=W)), device=None)
    assert c.ring_period() == W + 1


def test_graph_calls_refuse_bad_state():
    c = Cache(config_for(synth.WORKLOADS[2]), device=None)
    with pytest.raises(native.SwError) as e:
        c.graph_begin()                       # metadata-only: nothing to record
    assert e.value.status == native.SW_ERR_STATE
    with pytest.raises(native.SwError) as e:
        c.graph_end()                         # no capture in progress
    assert e.value.status == native.SW_ERR_STATE
    L = native.lib()
    assert L.sw_graph_launch(None, None) == native.SW_ERR_INVALID_ARG
    assert L.sw_graph_destroy(None) == native.SW_ERR_INVALID_ARG
    assert L.sw_cache_ring_period(None, ctypes.byref(ctypes.c_int32())) == native.SW_ERR_INVALID_ARG
