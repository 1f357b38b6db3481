"""Block-sparse tile mask: which 128x128 (query tile, key tile) pairs are computed.

Source: "Vidu S2 vs PixVerse R2" blog (orkas.ai), section "Choice 4: where the
speed comes from" -- R2 learns block-sparse attention in training, above 90%
sparsity.  The learned selector needs trained weights, so the mask here is the
plain stand-in the block-sparse workload describes: per head and per query
tile, keep the key tiles with the largest mean-pooled Q.K score, plus tiles that
are always kept.

Readings used (the pages give none of these details):

* Tiles never straddle a block: a block of B tokens has ceil(B/128) tiles, the
  last one partial.  Pooling averages the valid tokens of a tile only.
* Pooled score of query tile i and key tile (slot l, j) = <mean of relocated
  rotated queries, mean of relocated rotated keys> / sqrt(d).
* Always kept: key tile 0 of the first sink (the stream's first tokens), when a
  sink exists, and the diagonal tile j = i of the current block.  Keeping every
  sink tile would already exceed 8% of the tiles, which the >90% sparsity rules
  out.
* Row budget k = max(#forced, floor(keep * n_kv_tiles + 0.5)); the forced tiles
  count inside it; the rest are the highest scores, ties to the lower linear
  index l * tiles_per_block + j.  Kept indices are returned ascending.
"""
from __future__ import annotations

import math

import numpy as np


def n_tiles(block_tokens: int, tile: int = 128) -> int:
    return -(-block_tokens // tile)


def tile_bounds(block_tokens: int, tile: int = 128):
    return [(j * tile, min(block_tokens, (j + 1) * tile)) for j in range(n_tiles(block_tokens, tile))]


def pooled(x: np.ndarray, tile: int = 128) -> np.ndarray:
    """Mean over the valid tokens of each tile: x [B, d] -> [n_tiles, d]."""
    return np.stack([x[a:b].mean(axis=0) for a, b in tile_bounds(x.shape[0], tile)])


def row_budget(n_kv_tiles: int, keep: float, n_forced: int) -> int:
    return max(n_forced, int(math.floor(keep * n_kv_tiles + 0.5)))


def forced(q_tile: int, roles, tiles_per_block: int):
    """Linear key-tile indices always kept for query tile `q_tile`."""
    out = set()
    if roles and roles[0] == "sink":
        out.add(0)
    out.add((len(roles) - 1) * tiles_per_block + q_tile)
    return out


def select(scores: np.ndarray, always, budget: int):
    """Forced tiles plus the best remaining scores (ties -> lower index), ascending."""
    rest = sorted((i for i in range(len(scores)) if i not in always),
                  key=lambda i: (-float(scores[i]), i))
    kept = set(always) | set(rest[:max(0, budget - len(always))])
    return sorted(kept)


def build(q_rel: np.ndarray, k_rel_slots, roles, keep: float, tile: int = 128):
    """Per-query-tile kept key tiles for one head.

    q_rel: [B, d] relocated rotated queries of the current block.
    k_rel_slots: list (logical order) of [B, d] relocated rotated keys.
    Returns (kept: list of ascending index lists, scores [n_q_tiles, n_kv_tiles], budget).
    """
    d = q_rel.shape[1]
    tpb = n_tiles(q_rel.shape[0], tile)
    qbar = pooled(q_rel, tile)
    kbar = np.concatenate([pooled(k, tile) for k in k_rel_slots], axis=0)
    scores = (qbar @ kbar.T) / math.sqrt(d)
    n_kv = kbar.shape[0]
    kept, budget = [], None
    for i in range(tpb):
        f = forced(i, roles, tpb)
        budget = row_budget(n_kv, keep, len(f))
        kept.append(select(scores[i], f, budget))
    return kept, scores, budget


def visible(kept, block_tokens: int, n_slots: int, tile: int = 128) -> np.ndarray:
    """Dense bool mask [B, n_slots*B] equivalent to the kept tile lists."""
    tpb = n_tiles(block_tokens, tile)
    bounds = tile_bounds(block_tokens, tile)
    m = np.zeros((block_tokens, n_slots * block_tokens), dtype=bool)
    for i, lst in enumerate(kept):
        qa, qb = bounds[i]
        for t in lst:
            l, j = divmod(t, tpb)
            ka, kb = bounds[j]
            m[qa:qb, l * block_tokens + ka:l * block_tokens + kb] = True
    return m
