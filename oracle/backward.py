"""Gradients of masked exact attention in float64 (test infrastructure only).

The pages keep only the inputs and the per-row softmax statistics from the
forward pass and rebuild P piece by piece when the gradients are taken (the
DeepSeek v2->v4 attention article, section 2, segmented recomputation; the
recompute-instead-of-store argument of "Flash Attention原理与DeepSeek V4.1实战部署指南",
section 2.2).  What that reaches is the gradient of the definition of
"FlashAttention 2 principles and PyTorch practice", section 1,

    O = P V,   P = softmax over visible keys of s,   s = scale * Q K^T,

for an upstream gradient dO (the loss is sum(dO * O)).  By the chain rule,
with the softmax Jacobian taken row by row:

    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))
    dQ = scale * dS K,     dK = scale * dS^T Q

With a score_mod (oracle.score_mods: the modified score is s' = f(s) for
each (h, q, k)) P is the softmax of the modified scores and dS above is the
gradient with respect to s'; by the chain rule the gradient with respect to
s is dS * f'(s).  For the additive changes f'(s) = 1; for softcap
f(s) = cap tanh(s / cap) and f'(s) = 1 - tanh^2(s / cap).  The bias terms
and the cap get no gradient here.

GQA (query head hq reads KV head hq // G): dK and dV of a KV head sum the
contributions of all G query heads that read it.  A row with no visible key
has P = 0 and contributes nothing.  No tiling, no recomputation order: the
whole row block's P is formed at once.

``attention_bwd(..., bound=True)`` also returns, per gradient, the sum of
absolute values of the terms that make up each element (with the rows'
rowsum(P*dP) term counted through |O|): the scale a rounding-error bound for
bf16 operands is built from.  ``o_used`` is the O a caller hands to a
kernel instead of the exact one; its error enters that bound with a factor
2^8.
"""
from __future__ import annotations

import numpy as np

from . import core as _core
from . import masks as _masks
from . import score_mods as _score_mods


def softmax_grad(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """dS = J^T dP for a row softmax: p * (dp - sum_k p dp), row by row."""
    return p * (dp - np.sum(p * dp, axis=-1, keepdims=True))


def bwd_rows(q, k, v, do, scale: float, mask_mod, b: int, hq: int, rows, score_mod=None):
    """For query rows ``rows`` of (b, hq): (dQ rows, dK part, dV part, P, dS).

    dK part / dV part are this row block's contributions to the gradients of
    KV head hq // G, shape [Nk, D].
    """
    Hq, Nq = q.shape[1], q.shape[2]
    Hkv, Nk = k.shape[1], k.shape[2]
    kvh = hq // (Hq // Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    qr = np.asarray(q[b, hq], dtype=np.float64)[rows]
    dor = np.asarray(do[b, hq], dtype=np.float64)[rows]
    kk = np.asarray(k[b, kvh], dtype=np.float64)
    vv = np.asarray(v[b, kvh], dtype=np.float64)
    s = _core.scores(qr, kk, scale)
    jac = None
    if score_mod is not None:
        jac = _score_mods.dense_dscore(score_mod, b, hq, s, rows, Nk)
        s = _score_mods.dense(score_mod, b, hq, s, rows, Nk)
    if mask_mod is None:
        vis = np.ones_like(s, dtype=bool)
    else:
        vis = _masks.dense(mask_mod, b, hq, Nq, Nk, rows)
    p, _ = _core.masked_softmax(s, vis)
    dp = dor @ vv.T
    ds = softmax_grad(p, dp)
    if jac is not None:
        ds = ds * jac
    return scale * (ds @ kk), scale * (ds.T @ qr), p.T @ dor, p, ds


def attention_bwd(q, k, v, do, scale: float | None = None, mask_mod=None, row_block: int = 512,
                  bound: bool = False, o_used=None, score_mod=None):
    """dQ [B, Hq, Nq, D], dK and dV [B, Hkv, Nk, D] in float64.

    With ``bound``, also (mQ, mK, mV) of the same shapes: mV = sum_q P |dO|,
    mQ = scale * sum_k m_S |K|, mK = scale * sum_q m_S |Q|, where
    m_S = |dS| + P * f'(s) * sum_d |dO| (|O| + 2^8 |o_used - O|), f'(s) = 1 without a
    score_mod.
    """
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.zeros((B, Hq, Nq, D), dtype=np.float64)
    dk = np.zeros((B, Hkv, Nk, D), dtype=np.float64)
    dv = np.zeros((B, Hkv, Nk, v.shape[-1]), dtype=np.float64)
    if bound:
        mq, mk, mv = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            kvh = h // G
            for r0 in range(0, Nq, row_block):
                rows = np.arange(r0, min(Nq, r0 + row_block))
                dqr, dkp, dvp, p, ds = bwd_rows(q, k, v, do, scale, mask_mod, b, h, rows, score_mod)
                dq[b, h, rows] = dqr
                dk[b, kvh] += dkp
                dv[b, kvh] += dvp
                if bound:
                    dor = np.abs(np.asarray(do[b, h], dtype=np.float64)[rows])
                    o = p @ np.asarray(v[b, kvh], dtype=np.float64)
                    oerr = 0.0
                    if o_used is not None:
                        oerr = np.abs(np.asarray(o_used[b, h], dtype=np.float64)[rows] - o)
                    dterm = np.sum(dor * (np.abs(o) + 256.0 * oerr), axis=-1, keepdims=True)
                    jac = 1.0
                    if score_mod is not None:  # the Delta error reaches dS through f'(s) too
                        sr = _core.scores(np.asarray(q[b, h], dtype=np.float64)[rows],
                                          np.asarray(k[b, kvh], dtype=np.float64), scale)
                        jac = _score_mods.dense_dscore(score_mod, b, h, sr, rows, Nk)
                    ms = np.abs(ds) + p * dterm * jac
                    mq[b, h, rows] = scale * (ms @ np.abs(np.asarray(k[b, kvh], dtype=np.float64)))
                    mk[b, kvh] += scale * (ms.T @ np.abs(np.asarray(q[b, h], dtype=np.float64)[rows]))
                    mv[b, kvh] += p.T @ dor
    if bound:
        return dq, dk, dv, (mq, mk, mv)
    return dq, dk, dv
