"""Pins for oracle.score_mods (and the score_mod path of oracle.core / oracle.backward).

* brute force: tests/brute.py adds each bias in scalar Python loops
* library special case: torch float64 CPU scaled_dot_product_attention with a
  float attn_mask (bias, -inf where masked) built from torch.arange
  differences, forward and autograd
* closed forms with Q = 0 (all scores are the bias): ALiBi over keys 0..p is a
  geometric series, LSE_p = log((1 - e^{-a (p+1)}) / (1 - e^{-a})); a bias
  table that is one large entry selects a single key
* identities: slope 0 is no change; a constant table shifts LSE by the
  constant and leaves O alone
* softcap (cap * tanh(score / cap), applied before the additive terms):
  brute force with math.tanh; central finite differences of the brute-force
  loss for the gradients (this pins the chain-rule factor 1 - tanh^2); the
  saturated closed form LSE = log(n+ e^cap + n- e^-cap) when every score is
  far beyond +-cap; a cap far above every score is no change
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as OBW, masks as M, score_mods as SM
import brute
from test_oracle_pins import _tiny, _oracle_mod
from test_oracle_backward import _rand

SLOPES4 = [0.5, 0.25, 0.125, 0.0625]


def _oracle_smod(sspec, Nq, Nk):
    mods = []
    if "softcap" in sspec:
        mods.append(SM.softcap(sspec["softcap"]))
    if "alibi" in sspec:
        mods.append(SM.alibi(sspec["alibi"], Nq, Nk))
    if "alibi_sym" in sspec:
        mods.append(SM.alibi_sym(sspec["alibi_sym"], Nq, Nk))
    if "rel" in sspec:
        mods.append(SM.rel_bias(np.asarray(sspec["rel"][0]), sspec["rel"][1], Nq, Nk))
    return SM.combine(*mods)


SCORE_BRUTE = [
    # (name, B, Hq, Hkv, Nq, Nk, D, mask spec, score spec)
    ("alibi_causal", 1, 2, 1, 7, 7, 3, {"causal": True}, {"alibi": [0.5, 0.125]}),
    ("alibi_bottom_right", 1, 2, 2, 3, 8, 3, {"causal": True}, {"alibi": [0.3, 1.0]}),
    ("alibi_sym_window", 1, 1, 1, 9, 9, 2, {"window": (3, 3)}, {"alibi_sym": [0.7]}),
    ("rel_bias_nomask", 1, 2, 1, 6, 6, 3, {}, {"rel": ([[0.1, -0.4, 0.9, 0.3, -1.2], [2.0, 0.0, -0.5, 0.25, 1.5]], 2)}),
    ("alibi_and_rel_docs", 1, 1, 1, 8, 8, 2, {"docs": [3, 5]},
     {"alibi_sym": [0.2], "rel": ([[0.3, -0.2, 0.5, 0.0, 0.1, -0.7, 0.4]], 3)}),
]


def pin_score_brute(case):
    name, B, Hq, Hkv, Nq, Nk, D, mspec, sspec = case
    q, k, v = _tiny(zlib.crc32(name.encode()) % 1000, B, Hq, Hkv, Nq, Nk, D)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale, _oracle_mod(mspec, Nq, Nk, B), row_block=3,
                              score_mod=_oracle_smod(sspec, Nq, Nk))
    ob, lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), scale, mspec, sspec)
    ob, lb = np.array(ob), np.array(lb)
    fin = np.isfinite(lb)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb)), name
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0) < 1e-12, name
    assert np.max(np.abs(o - ob)) < 1e-12, name


@pytest.mark.parametrize("case", SCORE_BRUTE, ids=[c[0] for c in SCORE_BRUTE])
def test_score_brute_force(case):
    pin_score_brute(case)


def _torch_bias(kind, Hq, N, **kw):
    """[Hq, N, N] float bias from torch primitives (square, positions = indices)."""
    d = (torch.arange(N)[None, :] - torch.arange(N)[:, None]).double()   # k - p
    if kind == "alibi":
        return torch.tensor(kw["slopes"], dtype=torch.float64)[:, None, None] * d
    if kind == "alibi_sym":
        return -torch.tensor(kw["slopes"], dtype=torch.float64)[:, None, None] * d.abs()
    if kind == "rel":
        R = kw["R"]
        idx = d.clamp(-R, R).long() + R
        return torch.stack([torch.tensor(kw["table"][h], dtype=torch.float64)[idx] for h in range(Hq)])
    raise ValueError(kind)


def _sdpa_bias(q, k, v, do, scale, bias, bool_mask):
    qt, kt, vt = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    am = bias.masked_fill(~bool_mask, -math.inf) if bool_mask is not None else bias
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, scale=scale,
                                                         enable_gqa=qt.shape[1] != kt.shape[1])
    G = qt.shape[1] // kt.shape[1]
    s = scale * torch.matmul(qt, kt.repeat_interleave(G, 1).transpose(-1, -2)) + am
    lse = torch.logsumexp(s, dim=-1)
    o.backward(torch.from_numpy(do))
    return o.detach().numpy(), lse.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def _check_sdpa(seed, Hq, Hkv, N, D, kind, kw, mspec, tmask):
    q, k, v = _tiny(seed, 1, Hq, Hkv, N, N, D)
    do = _rand(seed + 3, (1, Hq, N, D))
    scale = 1.0 / math.sqrt(D)
    sspec = {kind: kw["slopes"]} if kind != "rel" else {"rel": (kw["table"], kw["R"])}
    smod = _oracle_smod(sspec, N, N)
    mod = _oracle_mod(mspec, N, N, 1)
    o, lse = oracle.attention(q, k, v, scale, mod, row_block=64, score_mod=smod)
    dq, dk, dv = OBW.attention_bwd(q, k, v, do, scale, mod, row_block=64, score_mod=smod)
    ro, rl, rq, rk, rv = _sdpa_bias(q, k, v, do, scale, _torch_bias(kind, Hq, N, **kw)[None], tmask)
    for a, b in ((o, ro), (lse, rl), (dq, rq), (dk, rk), (dv, rv)):
        assert np.max(np.abs(a - b)) < 1e-10, np.max(np.abs(a - b))


def pin_score_sdpa():
    N = 150
    causal = torch.ones(N, N).tril().bool()
    _check_sdpa(51, 4, 2, N, 16, "alibi", {"slopes": SLOPES4}, {"causal": True}, causal)
    _check_sdpa(52, 4, 4, N, 16, "alibi_sym", {"slopes": SLOPES4}, {}, None)
    rng = np.random.default_rng(5)
    table = rng.normal(size=(2, 2 * 40 + 1)).tolist()
    _check_sdpa(53, 2, 1, N, 16, "rel", {"table": table, "R": 40}, {"causal": True}, causal)


def test_score_sdpa():
    pin_score_sdpa()


def pin_score_closed_forms():
    N, D = 60, 8
    _, k, v = _tiny(54, 1, 1, 1, N, N, D)
    q = np.zeros((1, 1, N, D))
    a = 0.3
    o, lse = oracle.attention(q, k, v, 0.5, M.causal(N, N), score_mod=SM.alibi([a], N, N))
    p = np.arange(N)
    want = np.log((1 - np.exp(-a * (p + 1))) / (1 - np.exp(-a)))
    assert np.max(np.abs(lse[0, 0] - want)) < 1e-12
    w = np.exp(-a * (5 - np.arange(6)))
    assert np.max(np.abs(o[0, 0, 5] - (w[:, None] * v[0, 0, :6]).sum(0) / w.sum())) < 1e-12
    # symmetric ALiBi, no mask: sum over both sides of the row
    o2, l2 = oracle.attention(q, k, v, 0.5, None, score_mod=SM.alibi_sym([a], N, N))
    want2 = np.log(np.array([np.exp(-a * np.abs(np.arange(N) - i)).sum() for i in range(N)]))
    assert np.max(np.abs(l2[0, 0] - want2)) < 1e-12
    # a table that is one large entry at distance +3 selects key p + 3
    R = 5
    tb = np.zeros((1, 2 * R + 1))
    tb[0, 3 + R] = 60.0
    o3, l3 = oracle.attention(q, k, v, 0.5, None, score_mod=SM.rel_bias(tb, R, N, N))
    # every other key weighs e^-60 of it: O = V[p + 3] up to N e^-60 |V| < 1e-20
    assert np.max(np.abs(o3[0, 0, :N - 3] - v[0, 0, 3:])) < 1e-20


def pin_score_identities():
    N = 40
    q, k, v = _tiny(55, 1, 2, 1, N, N, 8)
    base = oracle.attention(q, k, v, 0.4, M.causal(N, N))
    z = oracle.attention(q, k, v, 0.4, M.causal(N, N), score_mod=SM.alibi([0.0, 0.0], N, N))
    assert np.max(np.abs(z[0] - base[0])) < 1e-12 and np.max(np.abs(z[1] - base[1])) < 1e-12
    c = oracle.attention(q, k, v, 0.4, M.causal(N, N),
                         score_mod=SM.rel_bias(np.full((2, 7), 1.75), 3, N, N))
    assert np.max(np.abs(c[0] - base[0])) < 1e-12 and np.max(np.abs(c[1] - base[1] - 1.75)) < 1e-12


def test_score_closed_forms():
    pin_score_closed_forms()


def test_score_identities():
    pin_score_identities()


SOFTCAP_BRUTE = [
    # (name, B, Hq, Hkv, Nq, Nk, D, mask spec, score spec)
    ("softcap_causal", 1, 2, 1, 7, 7, 3, {"causal": True}, {"softcap": 0.8}),
    ("softcap_alibi_sym_window", 1, 1, 1, 9, 9, 2, {"window": (3, 3)}, {"softcap": 1.5, "alibi_sym": [0.7]}),
    ("softcap_rel_bottom_right", 1, 2, 2, 3, 8, 3, {"causal": True},
     {"softcap": 0.5, "rel": ([[0.1, -0.4, 0.9, 0.3, -1.2], [2.0, 0.0, -0.5, 0.25, 1.5]], 2)}),
]


@pytest.mark.parametrize("case", SOFTCAP_BRUTE, ids=[c[0] for c in SOFTCAP_BRUTE])
def test_softcap_brute_force(case):
    pin_score_brute(case)


SOFTCAP_FD = [
    # (name, Hq, Hkv, Nq, Nk, D, mask spec, score spec)
    ("softcap_gqa_bottom_right", 2, 1, 3, 5, 3, {"causal": True}, {"softcap": 0.7}),
    ("softcap_alibi_window", 1, 1, 5, 5, 2, {"window": (2, 2)}, {"softcap": 1.2, "alibi": [0.4]}),
]


def _brute_loss_smod(q, k, v, do, scale, spec, sspec):
    o, _ = brute.attention(q.tolist(), k.tolist(), v.tolist(), scale, spec, sspec)
    return math.fsum(a * c for a, c in zip(np.asarray(o).ravel().tolist(), do.ravel().tolist()))


def pin_softcap_finite_differences():
    for name, Hq, Hkv, Nq, Nk, D, mspec, sspec in SOFTCAP_FD:
        seed = zlib.crc32(name.encode()) % 1000
        q, k, v = _tiny(seed, 1, Hq, Hkv, Nq, Nk, D)
        q *= 2.0  # scores of a few units: well into the curved part of tanh at these caps
        do = _rand(seed + 1, (1, Hq, Nq, D))
        scale = 1.0 / math.sqrt(D)
        dq, dk, dv = OBW.attention_bwd(q, k, v, do, scale, _oracle_mod(mspec, Nq, Nk, 1), row_block=2,
                                       score_mod=_oracle_smod(sspec, Nq, Nk))
        h = 1e-5
        for x, g in ((q, dq), (k, dk), (v, dv)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                x0 = x[idx]
                x[idx] = x0 + h
                fp = _brute_loss_smod(q, k, v, do, scale, mspec, sspec)
                x[idx] = x0 - h
                fm = _brute_loss_smod(q, k, v, do, scale, mspec, sspec)
                x[idx] = x0
                fd[idx] = (fp - fm) / (2 * h)
            assert np.max(np.abs(fd - g)) < 1e-7, (name, np.max(np.abs(fd - g)))


def test_softcap_finite_differences():
    pin_softcap_finite_differences()


def pin_softcap_closed_forms():
    # Saturation: q = (A, 0, ...) and keys (+-1, x, ...) give scores +-scale A = +-50 cap, where
    # tanh is +-1 to within 1e-40: LSE_p = log(n+ e^cap + n- e^-cap) over the keys up to p.
    N, D, cap = 12, 4, 2.0
    rng = np.random.default_rng(9)
    sign = np.where(rng.random(N) < 0.5, 1.0, -1.0)
    sign[0] = 1.0
    k = rng.normal(size=(1, 1, N, D))
    k[0, 0, :, 0] = sign
    v = rng.normal(size=(1, 1, N, D))
    scale = 0.5
    q = np.zeros((1, 1, N, D))
    q[0, 0, :, 0] = 50.0 * cap / scale
    o, lse = oracle.attention(q, k, v, scale, M.causal(N, N), score_mod=SM.softcap(cap))
    for p in range(N):
        npos = int((sign[:p + 1] > 0).sum())
        nneg = p + 1 - npos
        assert abs(lse[0, 0, p] - math.log(npos * math.exp(cap) + nneg * math.exp(-cap))) < 1e-12
        w = np.where(sign[:p + 1] > 0, math.exp(cap), math.exp(-cap))
        assert np.max(np.abs(o[0, 0, p] - (w[:, None] * v[0, 0, :p + 1]).sum(0) / w.sum())) < 1e-12
    # A cap far above every score: cap tanh(s / cap) = s - s^3 / (3 cap^2) + ..., no change to 1e-9.
    q2, k2, v2 = _tiny(56, 1, 2, 1, 30, 30, 8)
    base = oracle.attention(q2, k2, v2, 0.4, M.causal(30, 30))
    big = oracle.attention(q2, k2, v2, 0.4, M.causal(30, 30), score_mod=SM.softcap(1e6))
    assert np.max(np.abs(big[0] - base[0])) < 1e-9 and np.max(np.abs(big[1] - base[1])) < 1e-9


def test_softcap_closed_forms():
    pin_softcap_closed_forms()


SCORE_PINS = [
    lambda: [pin_score_brute(c) for c in SCORE_BRUTE + SOFTCAP_BRUTE],
    pin_score_sdpa, pin_score_closed_forms, pin_score_identities,
    pin_softcap_finite_differences, pin_softcap_closed_forms,
]
