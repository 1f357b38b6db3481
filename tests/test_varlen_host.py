"""Host bookkeeping of variable-length blocks on a metadata-only handle (CPU only).

Block length follows the control signal up to a cap ("Vidu S2 vs PixVerse R2" blog,
section "Choice 5: how people control it"); time bases are compared with the
oracle's cumulative-frame relocation over a long stream, and the error paths of
sw_cache_append_block_frames are exercised.
"""
import pytest

import synth
from oracle import cache as ocache
from oracle import rope as orope
from streaming_block_causal_amd import native
from streaming_block_causal_amd.cache import Cache

from .helpers import config_for, window_len_after


@pytest.mark.parametrize("policy", ["s1", "relative"])
@pytest.mark.parametrize("S,W", [(1, 3), (2, 1), (0, 2)])
def test_varlen_bases_match_oracle(policy, S, W):
    w = synth.WORKLOADS[6].replace(policy=policy, n_sink=S, n_window=W)
    c = Cache(config_for(w), device=None)
    model = ocache.CacheModel(S, W)
    for n in range(300):
        fn = synth.frames_of(w, n)
        c.append("current", 1, 1, n, n_frames=fn)
        lg = model.logical(n)
        info = c.inspect()
        assert [(d["role"], d["block_id"]) for d in info] == lg
        assert [d["frames"] for d in info] == [synth.frames_of(w, b) for _, b in lg]
        ref = orope.relocation_bases_frames(policy, [synth.frames_of(w, b) for r, b in lg if r == "sink"],
                                            [synth.frames_of(w, b) for r, b in lg if r == "window"], fn)
        assert [d["time_base"] for d in info] == ref, n
        if n >= S and W > 0 and window_len_after(n, S, W) == W:
            c.evict()
        c.append("clean", None, None, n)
        model.commit(n)


def test_varlen_error_paths():
    w = synth.WORKLOADS[6].replace(twin=True)
    c = Cache(config_for(w), device=None)

    def err(fn, code):
        before = c.inspect()
        with pytest.raises(native.SwError) as e:
            fn()
        assert e.value.status == code, str(e.value)
        assert c.inspect() == before

    err(lambda: c.append("current", 1, 1, 0, n_frames=0), native.SW_ERR_INVALID_ARG)
    err(lambda: c.append("current", 1, 1, 0, n_frames=4), native.SW_ERR_INVALID_ARG)
    c.append("current", 1, 1, 0, n_frames=2)
    err(lambda: c.append("current", 1, 1, 0, n_frames=3), native.SW_ERR_STATE)   # restage keeps the length
    c.append("clean", None, None, 0)
    assert c.inspect()[0]["frames"] == 2
    err(lambda: c.append("noisy", 1, 1, 0, n_frames=3), native.SW_ERR_STATE)     # twin matches the block
    c.append("noisy", 1, 1, 0, n_frames=2)
    sparse = Cache(config_for(synth.WORKLOADS[5]), device=None)
    with pytest.raises(native.SwError) as e:
        sparse.append("current", 1, 1, 0, n_frames=1)
    assert e.value.status == native.SW_ERR_UNSUPPORTED


def test_full_length_frames_call_equals_plain_append():
    w = synth.WORKLOADS[2]
    a, b = Cache(config_for(w), device=None), Cache(config_for(w), device=None)
    for n in range(12):
        a.append("current", 1, 1, n)
        b.append("current", 1, 1, n, n_frames=w.frames)
        assert a.inspect() == b.inspect()
        if n >= 4:
            a.evict()
            b.evict()
        a.append("clean", None, None, n)
        b.append("clean", None, None, n)
