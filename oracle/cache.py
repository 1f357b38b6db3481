"""Logical model of the bounded KV cache: permanent sinks plus a rolling window.

Source: "Vidu S2 vs PixVerse R2" blog (orkas.ai), section "Choice 3: bounded
memory" -- the first few blocks are kept for good as anchors (sinks), a sliding
window keeps the most recent blocks and the rest is dropped, so generating a
block costs the same however long the stream is.  The Vidu S2 tutorial
(bloombook.cn), section "What Vidu S2 is", pairs the sliding-window context with
a rolling KV cache whose memory does not grow with the conversation.

Reading used: the first S committed blocks become the sinks; later blocks go to
the window, which keeps the W most recent and evicts oldest first.  The
materialised key sequence of a call is [sinks, window oldest->newest, current].
"""
from __future__ import annotations

from collections import deque
from typing import List, Tuple


class CacheModel:
    """Plain list + deque model; holds block ids only (contents are looked up by id)."""

    def __init__(self, n_sink: int, n_window: int):
        self.n_sink, self.n_window = n_sink, n_window
        self.sinks: List[int] = []
        self.window: deque = deque()

    def commit(self, block: int) -> None:
        if len(self.sinks) < self.n_sink:
            self.sinks.append(block)
            return
        if self.n_window == 0:
            return                      # no window: the block is dropped at once
        if len(self.window) == self.n_window:
            self.window.popleft()
        self.window.append(block)

    def logical(self, current: int) -> List[Tuple[str, int]]:
        """[(role, block_id)] in attention order; role in {'sink','window','current'}."""
        return ([("sink", b) for b in self.sinks] + [("window", b) for b in self.window]
                + [("current", current)])


def closed_form(n: int, n_sink: int, n_window: int):
    """Cache contents seen by chunk n of a stream that commits every chunk.

    sinks = 0..min(n,S)-1, window = max(S, n-W)..n-1 (empty when W = 0).
    """
    sinks = list(range(min(n, n_sink)))
    window = list(range(max(n_sink, n - n_window), n)) if n_window > 0 else []
    return sinks, window


def key_count(n: int, n_sink: int, n_window: int, block_tokens: int) -> int:
    return (min(n, n_sink) + min(max(n - n_sink, 0), n_window) + 1) * block_tokens
