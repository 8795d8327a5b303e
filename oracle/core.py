"""Plain float64 attention and LSE combine (test infrastructure only).

attention_rows -- the definition for chosen query rows of one (batch, head):
    s = scale * Q K^T,  P = softmax over visible keys,  O = P V,  LSE = log sum exp s
  (FlashAttention 2 principles and PyTorch practice, section 1; the running
  max M / exp-sum L of its section 3.2 are what LSE = M + log L summarises).
attention      -- every row of every (batch, head), row block by row block.
combine        -- merges partial results over disjoint key sets by their LSE:
    LSE = log sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s
  which is exact because each partial is a softmax over its own key set (the
  split-KV decoding the FlexAttention article, section 1, names).

Conventions (readings where the pages are silent):
* LSE is in natural-log units and includes the softmax scale.
* A row that sees no key has O = 0 and LSE = -inf.
* GQA: query head hq reads KV head hq // (Hq // Hkv) (consecutive grouping).
"""
from __future__ import annotations

import numpy as np

from . import masks as _masks
from . import score_mods as _score_mods


def scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """scale * Q K^T for the given query rows [r, D] against keys [Nk, D], in float64."""
    return scale * (np.asarray(q_rows, dtype=np.float64) @ np.asarray(k, dtype=np.float64).T)


def masked_softmax(s: np.ndarray, visible: np.ndarray):
    """Row softmax restricted to ``visible`` keys.  Returns (P, LSE); rows with no
    visible key get P = 0 and LSE = -inf."""
    s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.where(visible, np.exp(s - m_safe), 0.0)
    l = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        p = np.where(empty, 0.0, e / np.where(empty, 1.0, l))
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return p, lse[..., 0]


def attention_rows(q, k, v, scale: float, mask_mod, b: int, hq: int, rows, score_mod=None):
    """O [len(rows), D] and LSE [len(rows)] for query rows ``rows`` of (b, hq).

    q: [B, Hq, Nq, D]; k, v: [B, Hkv, Nk, D]; any float dtype (upcast exactly).
    ``score_mod`` (oracle.score_mods) changes the scaled scores before the
    softmax; LSE is then the log-sum-exp of the changed scores.
    """
    Hq, Nq = q.shape[1], q.shape[2]
    Hkv, Nk = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    kvh = hq // (Hq // Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    qr = np.asarray(q[b, hq], dtype=np.float64)[rows]
    kk = np.asarray(k[b, kvh], dtype=np.float64)
    vv = np.asarray(v[b, kvh], dtype=np.float64)
    s = scores(qr, kk, scale)
    if score_mod is not None:
        s = _score_mods.dense(score_mod, b, hq, s, rows, Nk)
    if mask_mod is None:
        vis = np.ones_like(s, dtype=bool)
    else:
        vis = _masks.dense(mask_mod, b, hq, Nq, Nk, rows)
    p, lse = masked_softmax(s, vis)
    return p @ vv, lse


def attention(q, k, v, scale: float | None = None, mask_mod=None, row_block: int = 512,
              score_mod=None):
    """Full O [B, Hq, Nq, D] and LSE [B, Hq, Nq] in float64."""
    B, Hq, Nq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros((B, Hq, Nq, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, Hq, Nq), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, Nq, row_block):
                rows = np.arange(r0, min(Nq, r0 + row_block))
                o[b, h, rows], lse[b, h, rows] = attention_rows(q, k, v, scale, mask_mod, b, h, rows,
                                                                score_mod)
    return o, lse


def combine(o_parts: np.ndarray, lse_parts: np.ndarray, axis: int = 0):
    """Merge partial attention results over disjoint key sets.

    o_parts [..., S, ..., D] (split axis ``axis``), lse_parts the same without D.
    Splits with LSE = -inf carry no weight; if every split is -inf the row is
    empty (O = 0, LSE = -inf).
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = np.max(lse_parts, axis=axis, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - m_safe), 0.0)
    tot = np.sum(w, axis=axis, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
        wn = np.where(empty, 0.0, w / np.where(empty, 1.0, tot))
    o = np.sum(np.expand_dims(wn, -1) * o_parts, axis=axis)
    return o, np.squeeze(lse, axis=axis)
