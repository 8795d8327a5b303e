"""score_mod functions for the oracle (test infrastructure only).

The FlexAttention article (section 1) pairs mask_mod with
``score_mod(score, b, h, q_idx, kv_idx) -> score``: a change of the scaled
score before the softmax, its examples being ALiBi, a position bias and a
learnable bias.  The builders here return that form for the modifications
the library implements (the score is scale * q.k, and query i sits at
position p = i + (Nk - Nq), as for the masks):

    alibi(slopes)        score + slopes[h] * (k - p)
    alibi_sym(slopes)    score - slopes[h] * |k - p|
    rel_bias(table, R)   score + table[h][clamp(k - p, -R, R) + R]
    softcap(cap)         cap * tanh(score / cap)

``combine`` applies several in turn (the library's order: softcap first, then
the additive terms).  Every builder's function also carries ``dscore``, the
derivative of its output with respect to its score argument (1 for the
additive terms, 1 - tanh^2(score / cap) for softcap), which oracle.backward
uses for the chain rule.  Tanh-capping of the logits is not in the pages; it
is the standard saturating change of the same score_mod form (parity
unpinned against any published figure: pinned by brute force, limits and
finite differences instead).
"""
from __future__ import annotations

import numpy as np


def _dist(q_idx, kv_idx, Nq, Nk):
    return np.asarray(kv_idx) - (np.asarray(q_idx) + (Nk - Nq))


def _additive(mod):
    """Mark an additive score_mod: d(score + bias)/d(score) = 1."""
    mod.dscore = lambda score, b, h, q_idx, kv_idx: np.ones_like(np.asarray(score, dtype=np.float64))
    return mod


def alibi(slopes, Nq: int, Nk: int):
    """ALiBi with a per-head slope: + slope_h (k - p), which is <= 0 on and left of the diagonal."""
    sl = np.asarray(slopes, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        return score + sl[h] * _dist(q_idx, kv_idx, Nq, Nk)
    return _additive(mod)


def alibi_sym(slopes, Nq: int, Nk: int):
    """Symmetric ALiBi for bidirectional attention: - slope_h |k - p|."""
    sl = np.asarray(slopes, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        return score - sl[h] * np.abs(_dist(q_idx, kv_idx, Nq, Nk))
    return _additive(mod)


def rel_bias(table, R: int, Nq: int, Nk: int):
    """A learnable bias per head and relative distance, distances beyond R clamped:
    + table[h][clamp(k - p, -R, R) + R], table of shape [H, 2R + 1]."""
    tb = np.asarray(table, dtype=np.float64)
    if tb.shape[-1] != 2 * R + 1:
        raise ValueError("rel_bias table must have 2R + 1 columns")

    def mod(score, b, h, q_idx, kv_idx):
        return score + tb[h][np.clip(_dist(q_idx, kv_idx, Nq, Nk), -R, R) + R]
    return _additive(mod)


def softcap(cap: float):
    """Tanh capping of the scaled score: cap * tanh(score / cap), which keeps every score
    in (-cap, cap) and is close to the identity for |score| << cap."""
    c = float(cap)
    if not c > 0.0:
        raise ValueError("softcap needs cap > 0")

    def mod(score, b, h, q_idx, kv_idx):
        return c * np.tanh(np.asarray(score, dtype=np.float64) / c)

    def dscore(score, b, h, q_idx, kv_idx):
        t = np.tanh(np.asarray(score, dtype=np.float64) / c)
        return 1.0 - t * t
    mod.dscore = dscore
    return mod


def combine(*mods):
    """Apply score_mods one after another (None entries are skipped); dscore by the chain
    rule, the product of each step's derivative at that step's input."""
    mods = [m for m in mods if m is not None]

    def mod(score, b, h, q_idx, kv_idx):
        for m in mods:
            score = m(score, b, h, q_idx, kv_idx)
        return score

    def dscore(score, b, h, q_idx, kv_idx):
        d = np.ones_like(np.asarray(score, dtype=np.float64))
        for m in mods:
            d = d * m.dscore(score, b, h, q_idx, kv_idx)
            score = m(score, b, h, q_idx, kv_idx)
        return d
    mod.dscore = dscore
    return mod


def dense(mod, b: int, h: int, s: np.ndarray, rows, Nk: int) -> np.ndarray:
    """Apply ``mod`` to a block of scores s [len(rows), Nk] of one (batch, head)."""
    r = np.asarray(rows)
    return np.asarray(mod(s, b, h, r[:, None], np.arange(Nk)[None, :]), dtype=np.float64)


def dense_dscore(mod, b: int, h: int, s: np.ndarray, rows, Nk: int) -> np.ndarray:
    """d mod(s) / d s for a block of scores s [len(rows), Nk] of one (batch, head)."""
    r = np.asarray(rows)
    d = mod.dscore(s, b, h, r[:, None], np.arange(Nk)[None, :])
    return np.broadcast_to(np.asarray(d, dtype=np.float64), s.shape)
