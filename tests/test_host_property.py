"""Property-based check of the host bookkeeping (CPU only, metadata-only caches).

Random cache shapes (sinks, window, frames per block, TwinCache), random block lengths,
block ids with gaps and policy switches mid-stream: after every call the slot table must be
the oracle's -- logical order from the cache model, time bases from the relocation closed
forms -- with distinct physical slots.  Source: "Vidu S2 vs PixVerse R2" blog, sections
"Choice 3: bounded memory" (sinks, window, relocation) and "Choice 5: how people control it"
(block length follows the control signal up to a cap).
"""
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import synth
from oracle import cache as ocache
from oracle import rope as orope
from streaming_block_causal_amd.cache import Cache

from .helpers import config_for


@st.composite
def streams(draw):
    S = draw(st.integers(0, 4))
    W = draw(st.integers(0, 10 - S))
    F = draw(st.integers(1, 3))
    twin = draw(st.booleans())
    n = draw(st.integers(1, 30))
    frames = draw(st.lists(st.integers(1, F), min_size=n, max_size=n))
    gaps = draw(st.lists(st.integers(1, 3), min_size=n, max_size=n))
    switches = draw(st.lists(st.sampled_from(["s1", "relative", None, None, None]), min_size=n, max_size=n))
    return S, W, F, twin, frames, gaps, switches


@settings(max_examples=60, deadline=None)
@given(streams())
def test_slot_table_matches_the_oracle(stream):
    S, W, F, twin, frames, gaps, switches = stream
    w = synth.tiny(1, n_sink=S, n_window=W, frames=F, lat_h=2, lat_w=3, twin=twin)
    c = Cache(config_for(w), device=None)
    model = ocache.CacheModel(S, W)
    held_frames = {}
    policy = w.policy
    block = -1
    for i, (fr, gap, sw) in enumerate(zip(frames, gaps, switches)):
        block += gap
        if sw is not None:
            c.relocate(sw)
            policy = sw
        c.append("current", 1, 1, block, n_frames=fr)
        lg = model.logical(block)
        info = c.inspect()
        assert [(d["role"], d["block_id"]) for d in info] == lg
        sink_f = [held_frames[b] for r, b in lg if r == "sink"]
        win_f = [held_frames[b] for r, b in lg if r == "window"]
        assert [d["time_base"] for d in info] == orope.relocation_bases_frames(policy, sink_f, win_f, fr)
        assert [d["frames"] for d in info] == sink_f + win_f + [fr]
        phys = [d["physical_slot"] for d in info]
        assert len(set(phys)) == len(phys) and all(0 <= p < S + W + 1 for p in phys)
        # commit (evict first when the window is full)
        if len(model.sinks) == S and W > 0 and len(model.window) == W:
            c.evict()
        c.append("clean", None, None, block)
        if twin and (len(model.sinks) < S or W > 0):
            c.append("noisy", 1, 1, block, n_frames=fr)
        model.commit(block)
        held_frames[block] = fr
