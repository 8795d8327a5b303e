"""score_mod functions for the oracle (test infrastructure only).

The FlexAttention article (section 1) pairs mask_mod with
``score_mod(score, b, h, q_idx, kv_idx) -> score``: a change of the scaled
score before the softmax, its examples being ALiBi, a position bias and a
learnable bias.  The builders here return that form for the additive
modifications the library implements (the score is scale * q.k, and query i
sits at position p = i + (Nk - Nq), as for the masks):

    alibi(slopes)        score + slopes[h] * (k - p)
    alibi_sym(slopes)    score - slopes[h] * |k - p|
    rel_bias(table, R)   score + table[h][clamp(k - p, -R, R) + R]

``combine`` applies several in turn.  All are additive, so d(score')/d(score)
is 1 and the gradients of oracle.backward keep their form.
"""
from __future__ import annotations

import numpy as np


def _dist(q_idx, kv_idx, Nq, Nk):
    return np.asarray(kv_idx) - (np.asarray(q_idx) + (Nk - Nq))


def alibi(slopes, Nq: int, Nk: int):
    """ALiBi with a per-head slope: + slope_h (k - p), which is <= 0 on and left of the diagonal."""
    sl = np.asarray(slopes, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        return score + sl[h] * _dist(q_idx, kv_idx, Nq, Nk)
    return mod


def alibi_sym(slopes, Nq: int, Nk: int):
    """Symmetric ALiBi for bidirectional attention: - slope_h |k - p|."""
    sl = np.asarray(slopes, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        return score - sl[h] * np.abs(_dist(q_idx, kv_idx, Nq, Nk))
    return mod


def rel_bias(table, R: int, Nq: int, Nk: int):
    """A learnable bias per head and relative distance, distances beyond R clamped:
    + table[h][clamp(k - p, -R, R) + R], table of shape [H, 2R + 1]."""
    tb = np.asarray(table, dtype=np.float64)
    if tb.shape[-1] != 2 * R + 1:
        raise ValueError("rel_bias table must have 2R + 1 columns")

    def mod(score, b, h, q_idx, kv_idx):
        return score + tb[h][np.clip(_dist(q_idx, kv_idx, Nq, Nk), -R, R) + R]
    return mod


def combine(*mods):
    """Apply score_mods one after another (None entries are skipped)."""
    mods = [m for m in mods if m is not None]

    def mod(score, b, h, q_idx, kv_idx):
        for m in mods:
            score = m(score, b, h, q_idx, kv_idx)
        return score
    return mod


def dense(mod, b: int, h: int, s: np.ndarray, rows, Nk: int) -> np.ndarray:
    """Apply ``mod`` to a block of scores s [len(rows), Nk] of one (batch, head)."""
    r = np.asarray(rows)
    return np.asarray(mod(s, b, h, r[:, None], np.arange(Nk)[None, :]), dtype=np.float64)
