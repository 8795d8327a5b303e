"""BlockMask tile classes and tile lists from a dense mask (test infrastructure only).

A BlockMask marks each (query tile, key tile) pair as EMPTY (skipped), PARTIAL
(the predicate decides per element) or FULL (every pair visible, no predicate),
the block-sparsity the FlexAttention article describes in section 1.  Here the
classes come from the explicit dense mask: a tile is EMPTY if no in-range pair
is visible, FULL if every in-range pair is visible, PARTIAL otherwise.  Pairs
beyond the query or key length do not count.
"""
from __future__ import annotations

import numpy as np

from . import masks as _masks

EMPTY, PARTIAL, FULL = 0, 1, 2


def classify(mask_mod, b: int, h: int, Nq: int, Nk: int, tile: int) -> np.ndarray:
    """uint8 [ceil(Nq/tile), ceil(Nk/tile)] tile classes of one (batch, head)."""
    nqt = -(-Nq // tile)
    nkt = -(-Nk // tile)
    out = np.zeros((nqt, nkt), dtype=np.uint8)
    for i in range(nqt):
        rows = np.arange(i * tile, min(Nq, (i + 1) * tile))
        dm = _masks.dense(mask_mod, b, h, Nq, Nk, rows)
        for j in range(nkt):
            blk = dm[:, j * tile:min(Nk, (j + 1) * tile)]
            if not blk.any():
                out[i, j] = EMPTY
            elif blk.all():
                out[i, j] = FULL
            else:
                out[i, j] = PARTIAL
    return out


def tile_lists(classes: np.ndarray):
    """Per query-tile row: (part_num [nqt], part_idx [nqt, nkt], full_num, full_idx),
    indices ascending and zero-padded past the count."""
    classes = np.asarray(classes)
    nqt, nkt = classes.shape
    part_num = np.zeros(nqt, dtype=np.int32)
    full_num = np.zeros(nqt, dtype=np.int32)
    part_idx = np.zeros((nqt, nkt), dtype=np.int32)
    full_idx = np.zeros((nqt, nkt), dtype=np.int32)
    for i in range(nqt):
        p = np.nonzero(classes[i] == PARTIAL)[0]
        f = np.nonzero(classes[i] == FULL)[0]
        part_num[i], full_num[i] = len(p), len(f)
        part_idx[i, :len(p)] = p
        full_idx[i, :len(f)] = f
    return part_num, part_idx, full_num, full_idx
