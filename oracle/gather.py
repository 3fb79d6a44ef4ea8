"""The consumer of the selection: gathering the selected positions' rows of a
latent cache, oracle side (test infrastructure: only tests/ and the smoke
check use it).

What the pages fix: the positions the indexer selects are where the sparse
attention reads the latent cache c^KV (d_c = 512 per token), so a decode
step moves k * d_c elements instead of the whole context (Study MLA
Indexer, the data-flow diagram's last step and the first of its "three
whys"; Lightning Indexer explained, section 1 on the indexer's role).  What
they leave open, and the readings taken here:

* The latent cache is paged like the indexer cache and shares its block
  table: position s of sequence b is page block_table[b][s // page_size],
  slot s % page_size.
* A row is opaque bytes (the element type does not matter to a gather).
* A padding index (-1), or any index outside [0, max_pages * page_size),
  yields a zero row.

Index Share (Lightning Indexer explained, section 1, question 4 of the Q&A,
and section 3): the top-k computed at one layer is reused by the layers that
follow it.  Each reusing layer then reads its own latent cache at the shared
positions, so the multi-layer gather is the single-layer gather applied to
each layer's cache with one index set.
"""
from __future__ import annotations

import numpy as np


def topk_gather(latent_cache: np.ndarray, block_table: np.ndarray, topk_idx: np.ndarray,
                page_size: int = 64) -> np.ndarray:
    """latent_cache [pages][page_size][row_bytes] uint8, block_table [B][max_pages]
    int32, topk_idx [B][K] int32 -> out [B][K][row_bytes] uint8."""
    B, K = topk_idx.shape
    row = latent_cache.shape[2]
    out = np.zeros((B, K, row), dtype=np.uint8)
    limit = block_table.shape[1] * page_size
    for b in range(B):
        for j in range(K):
            s = int(topk_idx[b, j])
            if 0 <= s < limit:
                out[b, j] = latent_cache[int(block_table[b, s // page_size]), s % page_size]
    return out


def topk_gather_layers(latent_caches, block_table: np.ndarray, topk_idx: np.ndarray,
                       page_size: int = 64) -> list:
    """One selection served to several layers: layer l's rows are gathered
    from latent_caches[l] at the same positions (and with the same table)."""
    return [topk_gather(c, block_table, topk_idx, page_size) for c in latent_caches]
