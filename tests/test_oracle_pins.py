"""Pins for the CPU oracle: each check compares it with something other than itself.

* brute force: scalar loops over closed-form visible-key ranges (tests/brute.py)
* library special case: torch's float64 CPU scaled_dot_product_attention with
  boolean masks built from torch primitives (tril / triu / block_diag / kron)
* hand-worked values (tests/golden/hand_worked.json)
* invariants and closed forms: rows of P sum to 1, constant V, one visible key,
  Q = 0 gives LSE = ln(#visible keys) and O = mean of the visible V rows
* identities between masks, GQA vs repeated K/V, split + combine vs unsplit,
  paged gather vs contiguous

The ``pin_*`` functions raise AssertionError on a mismatch; test_oracle_mutants.py
plants mistakes in the oracle and checks that some pin catches each one.
"""
import json
import math
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import masks as M
from oracle import paged, blockmask as OB
import brute
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def _np(t):
    return t.to(torch.float64).numpy()


def _tiny(seed, B, Hq, Hkv, Nq, Nk, D):
    g = W.generator(seed)
    q = W.randn_bf16(g, (B, Hq, Nq, D))
    k = W.randn_bf16(g, (B, Hkv, Nk, D))
    v = W.randn_bf16(g, (B, Hkv, Nk, D))
    return _np(q), _np(k), _np(v)


def _oracle_mod(spec, Nq, Nk, B):
    mods = []
    if spec.get("causal"):
        mods.append(M.causal(Nq, Nk))
    if "window" in spec:
        mods.append(M.window(spec["window"][0], spec["window"][1], Nq, Nk))
    if "docs" in spec:
        mods.append(M.document([spec["docs"]] * B, Nq, Nk))
    if "block" in spec:
        mods.append(M.block_causal(spec["block"], Nq, Nk))
    if "key_range" in spec:
        mods.append(M.key_range(*spec["key_range"]))
    if "tiles" in spec:
        tmap, T, inner = spec["tiles"]
        mods.append(M.blockmask(np.asarray(tmap), T, _oracle_mod(inner, Nq, Nk, B)))
    return M.and_(*mods) if mods else M.full()


BRUTE_CASES = [
    # (name, B, Hq, Hkv, Nq, Nk, D, spec)
    ("none", 1, 2, 2, 5, 7, 4, {}),
    ("causal_square", 1, 1, 1, 9, 9, 4, {"causal": True}),
    ("causal_bottom_right", 2, 2, 1, 4, 11, 3, {"causal": True}),
    ("window_sym", 1, 1, 1, 13, 13, 4, {"window": (2, 2)}),
    ("window_asym_causal", 1, 1, 1, 12, 12, 3, {"window": (3, 1), "causal": True}),
    ("window_left_unbounded", 1, 1, 1, 10, 10, 3, {"window": (-1, 1)}),
    ("window_bottom_right", 1, 1, 1, 5, 12, 3, {"window": (2, 1)}),
    ("documents", 1, 2, 2, 14, 14, 4, {"docs": [3, 6, 5]}),
    ("window_and_documents", 1, 1, 1, 16, 16, 4, {"window": (2, 2), "docs": [5, 4, 7]}),
    ("block_diffusion", 1, 1, 1, 13, 13, 4, {"block": 4}),
    ("gqa_4_2", 1, 4, 2, 6, 6, 4, {"causal": True}),
    ("key_range", 1, 1, 1, 6, 10, 3, {"key_range": (3, 8)}),
    ("blockmask", 1, 2, 1, 12, 12, 3,
     {"tiles": ([[1, 0, 2], [2, 1, 0], [0, 2, 1]], 4, {"causal": True})}),
    ("blockmask_ragged", 1, 1, 1, 10, 10, 3,
     {"tiles": ([[1, 0, 0], [0, 1, 0], [2, 0, 1]], 4, {"causal": True})}),
    ("empty_rows", 1, 1, 1, 6, 6, 3, {"docs": [6], "key_range": (4, 6), "causal": True}),
    ("blockmask_per_batch_and_head", 2, 2, 1, 8, 8, 3,
     {"tiles": ([[[[1, 0], [2, 1]], [[1, 2], [0, 0]]], [[[0, 0], [0, 1]], [[2, 2], [2, 2]]]], 4,
                {"window": (1, 1)})}),
]


def pin_brute(case):
    name, B, Hq, Hkv, Nq, Nk, D, spec = case
    q, k, v = _tiny(zlib.crc32(name.encode()) % 1000, B, Hq, Hkv, Nq, Nk, D)
    scale = 1.0 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale, _oracle_mod(spec, Nq, Nk, B), row_block=3)
    ob, lb = brute.attention(q.tolist(), k.tolist(), v.tolist(), scale, spec)
    ob, lb = np.array(ob), np.array(lb)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb)), name
    fin = np.isfinite(lb)
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0) < 1e-12, name
    assert np.max(np.abs(o - ob)) < 1e-12, name


@pytest.mark.parametrize("case", BRUTE_CASES, ids=[c[0] for c in BRUTE_CASES])
def test_brute_force(case):
    pin_brute(case)


def test_brute_force_paged_two_splits():
    """Paged decode with a permuted 3-page pool, 2 key splits combined by LSE."""
    g = W.generator(5)
    B, Hq, Hkv, Lq, Nk, D, P = 1, 2, 1, 3, 11, 4, 4
    wl = W.paged_decode("t", B, Hq, Hkv, Lq, Nk, D, page_size=P, pool_pages=5, seed=5)
    t = wl.tensors
    kp, vp, bt = _np(t["k_pool"]), _np(t["v_pool"]), t["block_table"].numpy()
    kl = paged.gather(kp, bt, 0, Nk)[None]
    vl = paged.gather(vp, bt, 0, Nk)[None]
    q = _np(t["q"])
    scale = 0.5
    # split into [0, 8) and [8, 11)
    parts = [oracle.attention(q, kl, vl, scale, M.and_(M.causal(Lq, Nk), M.key_range(lo, hi)))
             for lo, hi in ((0, 8), (8, 11))]
    o, lse = oracle.combine(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    ob, lb = brute.attention(q.tolist(), _np(t["k_logical"]).tolist(), _np(t["v_logical"]).tolist(),
                             scale, {"causal": True})
    assert np.max(np.abs(o - np.array(ob))) < 1e-12
    assert np.max(np.abs(lse - np.array(lb))) < 1e-12


def test_hand_worked_golden():
    cases = json.load(open(os.path.join(HERE, "golden", "hand_worked.json")))["cases"]
    for c in cases:
        q, k, v = (np.array(c[x], dtype=np.float64) for x in ("q", "k", "v"))
        mod = None if c["mask"] == "none" else M.causal(q.shape[2], k.shape[2])
        o, lse = oracle.attention(q, k, v, c["scale"], mod)
        assert np.max(np.abs(o - np.array(c["O"]))) < 1e-12, c["name"]
        assert np.max(np.abs(lse - np.array(c["LSE"]))) < 1e-12, c["name"]


# ---- torch float64 CPU SDPA (library special case) ---------------------------------------

def _sdpa(q, k, v, scale, bool_mask, is_causal=False):
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    gqa = qt.shape[1] != kt.shape[1]
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=None if bool_mask is None else bool_mask, is_causal=is_causal,
        scale=scale, enable_gqa=gqa)
    G = qt.shape[1] // kt.shape[1]
    kr = kt.repeat_interleave(G, dim=1)
    s = scale * torch.matmul(qt, kr.transpose(-1, -2))
    if is_causal:
        bool_mask = torch.ones(s.shape[-2], s.shape[-1], dtype=torch.bool).tril()
    if bool_mask is not None:
        s = s.masked_fill(~bool_mask, -math.inf)
    lse = torch.logsumexp(s, dim=-1)
    return o.numpy(), lse.numpy()


def _torch_mask(kind, N, **kw):
    one = torch.ones(N, N)
    if kind == "causal":
        return one.tril().bool()
    if kind == "window":
        w = kw["w"]
        return one.triu(-w).tril(w).bool()
    if kind == "docs":
        return torch.block_diag(*[torch.ones(L, L) for L in kw["lengths"]]).bool()
    if kind == "window_docs":
        return _torch_mask("window", N, w=kw["w"]) & _torch_mask("docs", N, lengths=kw["lengths"])
    if kind == "block":
        bs = kw["bs"]
        nb = -(-N // bs)
        return torch.kron(torch.ones(nb, nb).tril(), torch.ones(bs, bs))[:N, :N].bool()
    if kind == "tiles":
        tm, T = torch.as_tensor(kw["tmap"]), kw["T"]
        full = torch.kron((tm == 2).double(), torch.ones(T, T))[:N, :N].bool()
        part = torch.kron((tm == 1).double(), torch.ones(T, T))[:N, :N].bool()
        return full | (part & one.tril().bool())
    raise ValueError(kind)


def pin_sdpa_causal():
    q, k, v = _tiny(11, 2, 3, 3, 300, 300, 64)
    o, lse = oracle.attention(q, k, v, 0.125, M.causal(300, 300), row_block=128)
    os_, ls = _sdpa(q, k, v, 0.125, None, is_causal=True)
    assert np.max(np.abs(o - os_)) < 1e-10 and np.max(np.abs(lse - ls)) < 1e-10


def pin_sdpa_window_docs():
    N = 257
    q, k, v = _tiny(12, 1, 2, 2, N, N, 16)
    lengths = [40, 100, 17, 100]
    o, lse = oracle.attention(q, k, v, 0.25, M.and_(M.window(9, 9, N, N), M.document([lengths], N, N)))
    os_, ls = _sdpa(q, k, v, 0.25, _torch_mask("window_docs", N, w=9, lengths=lengths))
    assert np.max(np.abs(o - os_)) < 1e-10 and np.max(np.abs(lse - ls)) < 1e-10


def pin_sdpa_block():
    N = 100
    q, k, v = _tiny(13, 1, 2, 2, N, N, 8)
    o, lse = oracle.attention(q, k, v, 0.3, M.block_causal(16, N, N))
    os_, ls = _sdpa(q, k, v, 0.3, _torch_mask("block", N, bs=16))
    assert np.max(np.abs(o - os_)) < 1e-10 and np.max(np.abs(lse - ls)) < 1e-10


def pin_sdpa_tiles_gqa():
    N, T = 70, 16
    q, k, v = _tiny(14, 1, 4, 2, N, N, 8)
    tm = np.array([[1, 0, 0, 2, 0], [2, 1, 0, 0, 0], [0, 0, 1, 0, 0], [2, 2, 0, 1, 0], [0, 2, 0, 0, 1]])
    o, lse = oracle.attention(q, k, v, 0.3, M.blockmask(tm, T, M.causal(N, N)))
    os_, ls = _sdpa(q, k, v, 0.3, _torch_mask("tiles", N, tmap=tm, T=T))
    assert np.max(np.abs(o - os_)) < 1e-10 and np.max(np.abs(lse - ls)) < 1e-10


def pin_sdpa_decode_paged():
    wl = W.paged_decode("t", 2, 4, 2, 5, 45, 8, page_size=4, pool_pages=30, seed=3)
    t = wl.tensors
    q = _np(t["q"])
    kp, vp, bt = _np(t["k_pool"]), _np(t["v_pool"]), t["block_table"].numpy()
    kl = np.stack([paged.gather(kp, bt, b, 45) for b in range(2)])
    vl = np.stack([paged.gather(vp, bt, b, 45) for b in range(2)])
    o, lse = oracle.attention(q, kl, vl, 0.3, M.causal(5, 45))
    # torch's own gather: whole pages by reshape, then drop the padding
    kt = torch.from_numpy(kp)[torch.from_numpy(bt).long()]  # [B, pages, P, Hkv, D]
    vt = torch.from_numpy(vp)[torch.from_numpy(bt).long()]
    kt = kt.flatten(1, 2)[:, :45].permute(0, 2, 1, 3).contiguous().numpy()
    vt = vt.flatten(1, 2)[:, :45].permute(0, 2, 1, 3).contiguous().numpy()
    bm = torch.ones(5, 45).tril(diagonal=40).bool()
    os_, ls = _sdpa(q, kt, vt, 0.3, bm)
    assert np.max(np.abs(o - os_)) < 1e-10 and np.max(np.abs(lse - ls)) < 1e-10


def test_sdpa_causal():
    pin_sdpa_causal()


def test_sdpa_window_docs():
    pin_sdpa_window_docs()


def test_sdpa_block_diffusion():
    pin_sdpa_block()


def test_sdpa_blockmask_gqa():
    pin_sdpa_tiles_gqa()


def test_sdpa_decode_paged():
    pin_sdpa_decode_paged()


# ---- invariants and closed forms ----------------------------------------------------------

def pin_probs_sum_to_one():
    rng = np.random.default_rng(0)
    s = rng.normal(size=(40, 50)) * 5
    vis = rng.random((40, 50)) < 0.3
    vis[3] = False
    p, lse = oracle.masked_softmax(s, vis)
    rows = vis.any(1)
    assert np.max(np.abs(p[rows].sum(1) - 1)) < 1e-12
    assert np.all(p[~vis] == 0) and np.all(p[3] == 0) and np.isneginf(lse[3])


def pin_constant_v():
    q, k, _ = _tiny(21, 1, 2, 2, 33, 33, 8)
    v = np.full_like(k, 0.75)
    o, _ = oracle.attention(q, k, v, 0.35, M.and_(M.window(4, 4, 33, 33), M.document([[10, 23]], 33, 33)))
    assert np.max(np.abs(o - 0.75)) < 1e-12


def pin_one_visible_key():
    q, k, v = _tiny(22, 1, 1, 1, 20, 20, 8)
    o, lse = oracle.attention(q, k, v, 0.35, M.window(0, 0, 20, 20))
    assert np.max(np.abs(o[0, 0] - v[0, 0])) < 1e-12
    sc = 0.35 * np.einsum("nd,nd->n", q[0, 0], k[0, 0])
    assert np.max(np.abs(lse[0, 0] - sc)) < 1e-12
    o2, l2 = oracle.attention(q, k, v, 0.35, M.causal(20, 20))
    assert np.max(np.abs(o2[0, 0, 0] - v[0, 0, 0])) < 1e-12
    assert abs(l2[0, 0, 0] - 0.35 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-12


def _q0_check(mod, counts, ranges, N, D=8, Hq=1):
    _, k, v = _tiny(23, 1, Hq, 1, N, N, D)
    q = np.zeros((1, Hq, N, D))
    o, lse = oracle.attention(q, k, v, 0.5, mod)
    for i in range(N):
        c = counts[i]
        if c == 0:
            assert np.isneginf(lse[0, 0, i]) and np.all(o[0, 0, i] == 0)
            continue
        assert abs(lse[0, 0, i] - math.log(c)) < 1e-12, (i, c)
        lo, hi = ranges[i]
        assert np.max(np.abs(o[0, 0, i] - v[0, 0, lo:hi].mean(0))) < 1e-12


def pin_q0_counts():
    N = 50
    _q0_check(M.causal(N, N), [i + 1 for i in range(N)], [(0, i + 1) for i in range(N)], N)
    w = 6
    _q0_check(M.window(w, w, N, N), [min(i + w, N - 1) - max(i - w, 0) + 1 for i in range(N)],
              [(max(i - w, 0), min(i + w, N - 1) + 1) for i in range(N)], N)
    lens = [7, 20, 23]
    starts = np.cumsum([0] + lens)
    doc_of = [int(np.searchsorted(starts, i, side="right") - 1) for i in range(N)]
    _q0_check(M.document([lens], N, N), [lens[d] for d in doc_of],
              [(starts[d], starts[d + 1]) for d in doc_of], N)
    bs = 8
    _q0_check(M.block_causal(bs, N, N), [min(N, (i // bs + 1) * bs) for i in range(N)],
              [(0, min(N, (i // bs + 1) * bs)) for i in range(N)], N)


def pin_identities():
    N = 40
    q, k, v = _tiny(24, 1, 4, 2, N, N, 8)
    base_full = oracle.attention(q, k, v, 0.4, M.full())
    base_causal = oracle.attention(q, k, v, 0.4, M.causal(N, N))
    for o, l in (oracle.attention(q, k, v, 0.4, M.window(N, N, N, N)),
                 oracle.attention(q, k, v, 0.4, M.document([[N]], N, N)),
                 oracle.attention(q, k, v, 0.4, None)):
        assert np.max(np.abs(o - base_full[0])) < 1e-12 and np.max(np.abs(l - base_full[1])) < 1e-12
    for o, l in (oracle.attention(q, k, v, 0.4, M.block_causal(1, N, N)),
                 oracle.attention(q, k, v, 0.4, M.blockmask(np.ones((5, 5), dtype=np.uint8), 8, M.causal(N, N)))):
        assert np.max(np.abs(o - base_causal[0])) < 1e-12 and np.max(np.abs(l - base_causal[1])) < 1e-12
    # GQA == MHA on repeated K/V
    o_r, l_r = oracle.attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), 0.4, M.causal(N, N))
    assert np.max(np.abs(o_r - base_causal[0])) < 1e-12 and np.max(np.abs(l_r - base_causal[1])) < 1e-12


def pin_split_combine():
    N = 64
    q, k, v = _tiny(25, 1, 2, 2, 10, N, 8)
    o, l = oracle.attention(q, k, v, 0.4, M.causal(10, N))
    bounds = [0, 13, 30, 55, 64]
    parts = [oracle.attention(q, k, v, 0.4, M.and_(M.causal(10, N), M.key_range(a, b)))
             for a, b in zip(bounds[:-1], bounds[1:])]
    oc, lc = oracle.combine(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    assert np.max(np.abs(oc - o)) < 1e-12 and np.max(np.abs(lc - l)) < 1e-12
    # a split that sees nothing carries no weight; S = 1 is the identity
    empty = oracle.attention(q, k, v, 0.4, M.key_range(0, 0))
    oc2, lc2 = oracle.combine(np.stack([o, empty[0]]), np.stack([l, empty[1]]))
    assert np.max(np.abs(oc2 - o)) < 1e-12 and np.max(np.abs(lc2 - l)) < 1e-12
    o1, l1 = oracle.combine(o[None], l[None])
    assert np.max(np.abs(o1 - o)) < 1e-15 and np.max(np.abs(l1 - l)) < 1e-15
    oe, le = oracle.combine(np.stack([empty[0]] * 3), np.stack([empty[1]] * 3))
    assert np.all(oe == 0) and np.all(np.isneginf(le))


def pin_paged_equals_contiguous():
    wl = W.paged_decode("t", 2, 2, 1, 3, 37, 4, page_size=4, pool_pages=25, seed=9)
    t = wl.tensors
    for b in range(2):
        for pool, logical in ((t["k_pool"], t["k_logical"]), (t["v_pool"], t["v_logical"])):
            g = paged.gather(_np(pool), t["block_table"].numpy(), b, 37)
            assert np.array_equal(g, _np(logical)[b])
            assert not np.isnan(g).any()


def pin_blockmask_classes():
    N, T = 40, 8
    cls = OB.classify(M.causal(N, N), 0, 0, N, N, T)
    # closed form: causal tiles -- FULL strictly below the diagonal, PARTIAL on it, EMPTY above
    nt = 5
    want = np.array([[2 if j < i else (1 if j == i else 0) for j in range(nt)] for i in range(nt)])
    assert np.array_equal(cls, want)
    # ragged tail: N=37, last row/column tiles hold 5 elements
    cls2 = OB.classify(M.window(3, 3, 37, 37), 0, 0, 37, 37, 8)
    assert cls2.shape == (5, 5)
    # tile (i, j) is EMPTY iff the closest pair is farther than 3
    for i in range(5):
        for j in range(5):
            qs, ks = range(8 * i, min(37, 8 * i + 8)), range(8 * j, min(37, 8 * j + 8))
            d = [abs(a - b) for a in qs for b in ks]
            exp = 0 if min(d) > 3 else (2 if max(d) <= 3 else 1)
            assert cls2[i, j] == exp
    # ragged causal, N=37: the last query tile holds 5 rows and the last key tile 5 keys;
    # pairs past N do not count, so the last row's tiles left of the diagonal stay FULL
    cls3 = OB.classify(M.causal(37, 37), 0, 0, 37, 37, 8)
    assert np.array_equal(cls3, want)
    pn, pi, fn, fi = OB.tile_lists(want)
    assert list(pn) == [1] * 5 and list(fn) == [0, 1, 2, 3, 4]
    assert list(fi[4, :4]) == [0, 1, 2, 3] and list(pi[:, 0]) == [0, 1, 2, 3, 4]


def test_probs_sum_to_one():
    pin_probs_sum_to_one()


def test_constant_v():
    pin_constant_v()


def test_one_visible_key():
    pin_one_visible_key()


def test_q0_counts():
    pin_q0_counts()


def test_identities():
    pin_identities()


def test_split_combine():
    pin_split_combine()


def test_paged_equals_contiguous():
    pin_paged_equals_contiguous()


def test_blockmask_classes():
    pin_blockmask_classes()
