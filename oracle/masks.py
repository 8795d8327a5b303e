"""mask_mod predicates for the oracle (test infrastructure only).

Each builder returns ``mask_mod(b, h, q_idx, kv_idx) -> bool ndarray``, the
form the FlexAttention article gives (section 1: a predicate saying which keys a
query can see).  ``q_idx`` and ``kv_idx`` are integer arrays that broadcast
against each other (typically a column of query rows and a row of key columns).

Query positions are aligned bottom-right when the query and key lengths differ:
query i sits at absolute position i + (Nk - Nq).  The pages warn that a
misaligned causal mask shifts the output (FlashAttention 2 principles and
PyTorch practice, section 7) but do not fix the convention; bottom-right is the
only reading under which a few draft queries appended after a long context can
be "causal among themselves".
"""
from __future__ import annotations

import numpy as np


def _pos(q_idx, Nq, Nk):
    return np.asarray(q_idx) + (Nk - Nq)


def causal(Nq: int, Nk: int):
    """Key k visible iff k <= aligned query position (FlashAttention 2 article,
    section 2, is_causal=True / causal=True)."""
    def mod(b, h, q_idx, kv_idx):
        return np.asarray(kv_idx) <= _pos(q_idx, Nq, Nk)
    return mod


def window(left: int, right: int, Nq: int, Nk: int):
    """Sliding window: p - left <= k <= p + right, both ends inclusive; a negative
    width means unbounded on that side.  The symmetric (w, w) window is the one the
    FlexAttention/DFlash article (section 3, finding 1) describes as the causal
    (w, 0) window made symmetric so bidirectional queries see both ways."""
    def mod(b, h, q_idx, kv_idx):
        p = _pos(q_idx, Nq, Nk)
        k = np.asarray(kv_idx)
        ok = np.ones(np.broadcast(p, k).shape, dtype=bool)
        if left >= 0:
            ok &= k >= p - left
        if right >= 0:
            ok &= k <= p + right
        return ok
    return mod


def document(doc_lengths_per_batch, Nq: int, Nk: int):
    """Same-document mask (FlexAttention article, section 1, document masks):
    visible iff the query's document id equals the key's.  Documents are
    contiguous runs of tokens with the given lengths; ids are assigned here by
    repeating the document index over its length."""
    ids = [np.repeat(np.arange(len(lens)), lens) for lens in doc_lengths_per_batch]
    for i, lens in zip(ids, doc_lengths_per_batch):
        if i.shape[0] != Nk:
            raise ValueError("document lengths must cover the key sequence")

    def mod(b, h, q_idx, kv_idx):
        doc_id = ids[int(b)]
        p = _pos(q_idx, Nq, Nk)
        return doc_id[p] == doc_id[np.asarray(kv_idx)]
    return mod


def block_causal(block_size: int, Nq: int, Nk: int):
    """Block-diffusion draft mask: bidirectional inside each block of block_size
    tokens, causal towards earlier blocks (FlexAttention/DFlash article,
    summary and section 3): visible iff floor(k/bs) <= floor(p/bs)."""
    def mod(b, h, q_idx, kv_idx):
        p = _pos(q_idx, Nq, Nk)
        return (np.asarray(kv_idx) // block_size) <= (p // block_size)
    return mod


def key_range(lo: int, hi: int):
    """Keys in [lo, hi) only: the part of the key sequence one split-KV chunk covers."""
    def mod(b, h, q_idx, kv_idx):
        k = np.asarray(kv_idx)
        q = np.asarray(q_idx)
        return np.broadcast_to((k >= lo) & (k < hi), np.broadcast(q, k).shape)
    return mod


def blockmask(tile_map, tile: int, partial_mod):
    """BlockMask semantics (FlexAttention article, section 1: block-level
    sparsity with fully-masked blocks skipped): the tile (q // tile, k // tile)
    decides -- EMPTY (0) hides the pair, FULL (2) shows it without consulting
    any predicate, PARTIAL (1) defers to ``partial_mod``.

    ``tile_map`` is [n_q_tiles, n_k_tiles] or [Bm, Hm, n_q_tiles, n_k_tiles]
    with size-1 batch/head dimensions broadcast.
    """
    tm = np.asarray(tile_map)
    if tm.ndim == 2:
        tm = tm[None, None]

    def mod(b, h, q_idx, kv_idx):
        t = tm[int(b) if tm.shape[0] > 1 else 0, int(h) if tm.shape[1] > 1 else 0]
        qi = np.asarray(q_idx)
        ki = np.asarray(kv_idx)
        state = t[qi // tile, ki // tile]
        part = partial_mod(b, h, qi, ki)
        return (state == 2) | ((state == 1) & part)
    return mod


def and_(*mods):
    """AND-composition of predicates (a pair is visible iff every predicate allows it)."""
    def mod(b, h, q_idx, kv_idx):
        out = None
        for m in mods:
            r = m(b, h, q_idx, kv_idx)
            out = r if out is None else (out & r)
        return out
    return mod


def full():
    """No mask: every key visible (the non-causal / bidirectional case)."""
    def mod(b, h, q_idx, kv_idx):
        return np.ones(np.broadcast(np.asarray(q_idx), np.asarray(kv_idx)).shape, dtype=bool)
    return mod


def dense(mod, b: int, h: int, Nq: int, Nk: int, rows=None) -> np.ndarray:
    """Materialise the boolean mask [len(rows), Nk] of one (batch, head)."""
    r = np.arange(Nq) if rows is None else np.asarray(rows)
    return np.asarray(mod(b, h, r[:, None], np.arange(Nk)[None, :]), dtype=bool)
