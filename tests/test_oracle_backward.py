"""Pins for oracle.backward, each against something other than its own formula.

* finite differences: central differences of sum(dO * O) with O from the
  pure-Python brute force of tests/brute.py (no Jacobian, no oracle code)
* library special case: torch float64 CPU autograd through
  scaled_dot_product_attention with boolean masks built from torch primitives
* closed forms of the softmax Jacobian: the gradient rows of dS sum to zero, so
  sum_k dK = 0; sum_k dV = sum of dO over rows that see a key; constant V or a
  single visible key per row gives dQ = dK = 0 (and dV = dO for the diagonal)
* GQA equals MHA on repeated K/V with the repeated heads' dK/dV summed

test_oracle_mutants.py plants mistakes in oracle.backward and checks that one of
these pins catches each.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as OBW, masks as M
import brute
import workloads as W
from test_oracle_pins import _tiny, _oracle_mod, _torch_mask


def _rand(seed, shape):
    g = W.generator(seed)
    return W.randn_bf16(g, shape).to(torch.float64).numpy()


# ---- finite differences of the brute force -------------------------------------------------

BWD_FD_CASES = [
    # (name, B, Hq, Hkv, Nq, Nk, D, spec)
    ("none", 1, 1, 1, 4, 5, 3, {}),
    ("causal_bottom_right_gqa", 1, 2, 1, 3, 6, 3, {"causal": True}),
    ("window_sym", 1, 1, 1, 7, 7, 2, {"window": (2, 2)}),
    ("documents", 1, 2, 2, 7, 7, 2, {"docs": [2, 4, 1]}),
    ("block_diffusion", 1, 1, 1, 7, 7, 3, {"block": 3}),
    ("empty_rows", 1, 1, 1, 5, 5, 2, {"docs": [5], "key_range": (3, 5), "causal": True}),
]


def _brute_loss(q, k, v, do, scale, spec):
    o, _ = brute.attention(q.tolist(), k.tolist(), v.tolist(), scale, spec)
    return math.fsum(a * c for a, c in zip(np.asarray(o).ravel().tolist(), do.ravel().tolist()))


def pin_bwd_finite_differences(case):
    name, B, Hq, Hkv, Nq, Nk, D, spec = case
    seed = zlib.crc32(name.encode()) % 1000
    q, k, v = _tiny(seed, B, Hq, Hkv, Nq, Nk, D)
    do = _rand(seed + 1, (B, Hq, Nq, D))
    scale = 1.0 / math.sqrt(D)
    dq, dk, dv = OBW.attention_bwd(q, k, v, do, scale, _oracle_mod(spec, Nq, Nk, B), row_block=2)
    h = 1e-5
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            fp = _brute_loss(q, k, v, do, scale, spec)
            x[idx] = x0 - h
            fm = _brute_loss(q, k, v, do, scale, spec)
            x[idx] = x0
            fd[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(fd - g)) < 1e-7, (name, np.max(np.abs(fd - g)))


@pytest.mark.parametrize("case", BWD_FD_CASES, ids=[c[0] for c in BWD_FD_CASES])
def test_bwd_finite_differences(case):
    pin_bwd_finite_differences(case)


# ---- torch float64 autograd ------------------------------------------------------------------

def _autograd(q, k, v, do, scale, bool_mask):
    qt, kt, vt = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=bool_mask, scale=scale, enable_gqa=qt.shape[1] != kt.shape[1])
    o.backward(torch.from_numpy(do))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def _check_autograd(seed, B, Hq, Hkv, N, D, scale, oracle_mod, torch_mask):
    q, k, v = _tiny(seed, B, Hq, Hkv, N, N, D)
    do = _rand(seed + 7, (B, Hq, N, D))
    ref = _autograd(q, k, v, do, scale, torch_mask)
    got = OBW.attention_bwd(q, k, v, do, scale, oracle_mod, row_block=96)
    for a, b in zip(got, ref):
        assert np.max(np.abs(a - b)) < 1e-10, np.max(np.abs(a - b))


def pin_bwd_autograd_causal_gqa():
    _check_autograd(31, 2, 4, 2, 200, 32, 0.2, M.causal(200, 200), _torch_mask("causal", 200))


def pin_bwd_autograd_window_docs():
    lens = [50, 90, 60]
    _check_autograd(32, 1, 2, 2, 200, 16, 0.3,
                    M.and_(M.window(20, 20, 200, 200), M.document([lens], 200, 200)),
                    _torch_mask("window_docs", 200, w=20, lengths=lens))


def pin_bwd_autograd_block():
    _check_autograd(33, 1, 2, 1, 150, 16, 0.25, M.block_causal(16, 150, 150),
                    _torch_mask("block", 150, bs=16))


def test_bwd_autograd_causal_gqa():
    pin_bwd_autograd_causal_gqa()


def test_bwd_autograd_window_docs():
    pin_bwd_autograd_window_docs()


def test_bwd_autograd_block():
    pin_bwd_autograd_block()


# ---- closed forms ----------------------------------------------------------------------------

def pin_bwd_invariants():
    N, G = 60, 2
    q, k, v = _tiny(34, 1, 4, 2, N, N, 8)
    do = _rand(35, (1, 4, N, 8))
    # a mask with rows that see nothing (keys 40.. only, causal) and a document cut
    mod = M.and_(M.causal(N, N), M.key_range(40, N), M.document([[25, 35]], N, N))
    dq, dk, dv = OBW.attention_bwd(q, k, v, do, 0.4, mod, row_block=17)
    vis = M.dense(mod, 0, 0, N, N, np.arange(N))
    sees = vis.any(1)
    assert np.max(np.abs(dk.sum(2))) < 1e-12
    want = do[0][:, sees].reshape(2, G, -1, 8).sum(axis=(1, 2))
    assert np.max(np.abs(dv[0].sum(1) - want)) < 1e-12
    assert np.all(dq[0][:, ~sees] == 0)
    # constant V rows: every dS is zero
    vc = np.full_like(v, -1.25)
    dq2, dk2, _ = OBW.attention_bwd(q, k, vc, do, 0.4, M.causal(N, N), row_block=32)
    assert np.max(np.abs(dq2)) < 1e-12 and np.max(np.abs(dk2)) < 1e-12
    # one visible key per row (window 0): P = 1, dS = 0, dV = dO (MHA)
    q1, k1, v1 = _tiny(36, 1, 2, 2, N, N, 8)
    dq3, dk3, dv3 = OBW.attention_bwd(q1, k1, v1, do[:, :2], 0.4, M.window(0, 0, N, N), row_block=32)
    assert np.max(np.abs(dq3)) < 1e-12 and np.max(np.abs(dk3)) < 1e-12
    assert np.max(np.abs(dv3 - do[:, :2])) < 1e-12


def pin_bwd_gqa_equals_repeated():
    N = 40
    q, k, v = _tiny(37, 1, 4, 2, N, N, 8)
    do = _rand(38, (1, 4, N, 8))
    dq, dk, dv = OBW.attention_bwd(q, k, v, do, 0.4, M.causal(N, N))
    dq_r, dk_r, dv_r = OBW.attention_bwd(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), do, 0.4,
                                         M.causal(N, N))
    assert np.max(np.abs(dq - dq_r)) < 1e-12
    assert np.max(np.abs(dk - dk_r.reshape(1, 2, 2, N, 8).sum(2))) < 1e-12
    assert np.max(np.abs(dv - dv_r.reshape(1, 2, 2, N, 8).sum(2))) < 1e-12


def test_bwd_invariants():
    pin_bwd_invariants()


def test_bwd_gqa_equals_repeated():
    pin_bwd_gqa_equals_repeated()


def test_bwd_bound_dominates_gradients():
    """The error-bound magnitudes are sums of |terms|, so they bound |gradient|."""
    N = 50
    q, k, v = _tiny(39, 1, 2, 1, N, N, 8)
    do = _rand(40, (1, 2, N, 8))
    dq, dk, dv, (mq, mk, mv) = OBW.attention_bwd(q, k, v, do, 0.4, M.causal(N, N), bound=True)
    for g, m in ((dq, mq), (dk, mk), (dv, mv)):
        assert np.all(np.abs(g) <= m + 1e-12)
    _, _, _, (mq2, _, _) = OBW.attention_bwd(q, k, v, do, 0.4, M.causal(N, N), bound=True,
                                             o_used=np.zeros((1, 2, N, 8)))
    assert np.all(mq2 >= mq)


BWD_PINS = [
    lambda: [pin_bwd_finite_differences(c) for c in BWD_FD_CASES],
    pin_bwd_autograd_causal_gqa, pin_bwd_autograd_window_docs, pin_bwd_autograd_block,
    pin_bwd_invariants, pin_bwd_gqa_equals_repeated,
]


def test_bwd_bound_rejects_plausible_kernel_mistakes():
    """The GPU bar |g - g_ref| <= 2^-7 m (m from ``bound=True``) must reject the mistakes a
    tiled backward kernel could plausibly make: each mistaken gradient, computed here in
    float64, exceeds the bar somewhere."""
    N, D, G = 300, 64, 2
    q, k, v = _tiny(41, 1, 2 * G, 2, N, N, D)
    do = _rand(42, (1, 2 * G, N, D))
    sc = 1.0 / math.sqrt(D)
    mod = M.causal(N, N)
    dq, dk, dv, (mq, mk, mv) = OBW.attention_bwd(q, k, v, do, sc, mod, bound=True)
    tol = (2.0 ** -7) * np.asarray(mq), (2.0 ** -7) * np.asarray(mk), (2.0 ** -7) * np.asarray(mv)

    def rejected(g, t):
        return bool(np.any(np.abs(g[0] - g[1]) > t))

    # a skipped 64-row step in dK / dV (rows 128..191 of every head)
    skip = M.and_(mod, lambda b, h, qi, ki: ~((np.asarray(qi) >= 128) & (np.asarray(qi) < 192))
                  & np.ones(np.broadcast(np.asarray(qi), np.asarray(ki)).shape, dtype=bool))
    _, dk_s, dv_s = OBW.attention_bwd(q, k, v, do, sc, skip)
    assert rejected((dk_s, dk), tol[1]) and rejected((dv_s, dv), tol[2])
    # a skipped 128-key step in dQ (keys 0..127), everything else exact
    dq_s = dq.copy()
    for h in range(2 * G):
        kvh = h // G
        p = np.zeros((N, N))
        s = sc * q[0, h] @ k[0, kvh].T
        vis = np.tril(np.ones((N, N), dtype=bool))
        s = np.where(vis, s, -np.inf)
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        dp = do[0, h] @ v[0, kvh].T
        ds = OBW.softmax_grad(p, dp)
        dq_s[0, h] -= sc * ds[:, :128] @ k[0, kvh, :128]
    assert rejected((dq_s, dq), tol[0])
    # GQA: dK / dV of a KV head from its first query head only
    dq1, dk1, dv1 = OBW.attention_bwd(q[:, ::G], k, v, do[:, ::G], sc, mod)
    assert rejected((dk1, dk), tol[1]) and rejected((dv1, dv), tol[2])
    # dS without the rowsum term, and P taken with the neighbouring row's LSE
    orig = OBW.softmax_grad
    try:
        OBW.softmax_grad = lambda p, dp: p * dp
        dq2, dk2, _ = OBW.attention_bwd(q, k, v, do, sc, mod)
        assert rejected((dq2, dq), tol[0]) and rejected((dk2, dk), tol[1])
        OBW.softmax_grad = lambda p, dp: orig(np.roll(p, 1, axis=0) * p.sum(1, keepdims=True), dp)
        dq3, dk3, dv3 = OBW.attention_bwd(q, k, v, do, sc, mod)
        assert rejected((dq3, dq), tol[0]) and rejected((dk3, dk), tol[1])
    finally:
        OBW.softmax_grad = orig
    # dK without the softmax scale
    assert rejected((dk / sc, dk), tol[1])
