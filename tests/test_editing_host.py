"""Host bookkeeping of frame-aligned editing on metadata-only handles (CPU only).

Editing model (Vidu S2 paper read, section 2.6): the reference image is visible to
every frame, each target frame reads only the source frame of its instant, and
source frames are consumed with their frame, never cached.  Here: the reference
is the first committed block (a sink of its own length), source frames are staged
beside the current block, listed after it at its time base, and dropped by its
commit; the error paths of SW_KV_SOURCE are exercised.
"""
import pytest

import synth
from oracle import cache as ocache
from oracle import rope as orope
from streaming_block_causal_amd import native
from streaming_block_causal_amd.cache import Cache

from .helpers import config_for, window_len_after

ED = synth.WORKLOADS[7]


def _frames_bases(w, lg, n):
    return orope.relocation_bases_frames(w.policy, [synth.frames_of(w, b) for r, b in lg if r == "sink"],
                                         [synth.frames_of(w, b) for r, b in lg if r == "window"],
                                         synth.frames_of(w, n))


@pytest.mark.parametrize("policy", ["s1", "relative"])
def test_editing_stream_bookkeeping(policy):
    w = ED.replace(policy=policy)
    c = Cache(config_for(w), device=None)
    model = ocache.CacheModel(w.n_sink, w.n_window)
    for n in range(200):
        fn = synth.frames_of(w, n)
        for _ in range(w.n_steps):
            c.append("current", 1, 1, n, n_frames=fn)
            if n >= 1:
                c.append("source", 1, 1, n, n_frames=fn)
        lg = model.logical(n)
        info = c.inspect()
        bases = _frames_bases(w, lg, n)
        want = [(r, b) for r, b in lg] + ([("source", n)] if n >= 1 else [])
        assert [(d["role"], d["block_id"]) for d in info] == want
        assert [d["time_base"] for d in info] == bases + ([bases[-1]] if n >= 1 else [])
        assert info[0]["frames"] == w.ref_frames and info[0]["role"] == ("sink" if n >= 1 else "current")
        if n >= 1:
            assert info[-1]["frames"] == fn and info[-1]["physical_slot"] == -1
        if n >= w.n_sink and w.n_window > 0 and window_len_after(n, w.n_sink, w.n_window) == w.n_window:
            c.evict()
        c.append("clean", None, None, n)
        model.commit(n)
        assert all(d["role"] != "source" for d in c.inspect())   # consumed with its block


def test_source_error_paths():
    c = Cache(config_for(ED), device=None)
    c.append("current", 1, 1, 0, n_frames=1)
    c.append("clean", None, None, 0)                              # the reference
    with pytest.raises(native.SwError) as e:
        c.append("source", 1, 1, 1)                               # nothing staged
    assert e.value.status == native.SW_ERR_STATE
    c.append("current", 1, 1, 1)
    for args, status in (((1, 1, 2), native.SW_ERR_STATE),        # another block id
                         ((None, 1, 1), native.SW_ERR_INVALID_ARG),  # NULL K
                         ((1, None, 1), native.SW_ERR_INVALID_ARG)):
        with pytest.raises(native.SwError) as e:
            c.append("source", *args)
        assert e.value.status == status, args
    with pytest.raises(native.SwError) as e:
        c.append("source", 1, 1, 1, n_frames=2)                   # not the staged length
    assert e.value.status == native.SW_ERR_STATE
    assert all(d["role"] != "source" for d in c.inspect())        # failed calls change nothing
    c.append("source", 1, 1, 1)
    c.append("current", 1, 1, 1)                                  # the next step keeps the source
    assert c.inspect()[-1]["role"] == "source"
    c.append("source", 1, 1, 1)                                   # re-staging overwrites
    assert sum(d["role"] == "source" for d in c.inspect()) == 1
    plain = Cache(config_for(ED.replace(editing=False)), device=None)
    plain.append("current", 1, 1, 0)
    with pytest.raises(native.SwError) as e:
        plain.append("source", 1, 1, 0)
    assert e.value.status == native.SW_ERR_STATE


def test_editing_config_validation_and_bytes():
    base = config_for(ED)
    plain = config_for(ED.replace(editing=False))
    slot = 24 * 6144 * 128 * 2
    assert native.sw_cache_required_bytes(base.to_c()) == native.sw_cache_required_bytes(plain.to_c()) + 2 * slot
    for kw, status in ((dict(sparse=True), native.SW_ERR_UNSUPPORTED),
                       (dict(n_sink=1, n_window=14), native.SW_ERR_SHAPE)):
        cfg = config_for(ED)
        for k, v in kw.items():
            setattr(cfg, k, v)
        with pytest.raises(native.SwError) as e:
            native.sw_cache_required_bytes(cfg.to_c())
        assert e.value.status == status, kw
    cfg = config_for(ED.replace(n_window=13))                   # S + W + 2 = 16 fits
    native.sw_cache_required_bytes(cfg.to_c())
    bad = config_for(ED).to_c()
    bad.editing = 2
    with pytest.raises(native.SwError) as e:
        native.sw_cache_required_bytes(bad)
    assert e.value.status == native.SW_ERR_INVALID_ARG
