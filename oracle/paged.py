"""Paged KV cache gather (test infrastructure only).

The pages describe K/V kept in fixed-size pages addressed through a per-sequence
block table (FlexAttention/DFlash article, sections 1 and 4: PagedAttention and
the block_table argument).  Pool layout [num_pages, page_size, Hkv, D].  Logical
key j of sequence b lives in page block_table[b, j // page_size], slot
j % page_size.
"""
from __future__ import annotations

import numpy as np


def gather(pool: np.ndarray, block_table: np.ndarray, b: int, seq_len: int) -> np.ndarray:
    """Logical [Hkv, seq_len, D] K (or V) of sequence b, gathered from the pool."""
    pool = np.asarray(pool)
    bt = np.asarray(block_table)
    page_size = pool.shape[1]
    j = np.arange(seq_len)
    pages = bt[b, j // page_size]
    rows = pool[pages, j % page_size]  # [seq_len, Hkv, D]
    return np.transpose(rows, (1, 0, 2))
