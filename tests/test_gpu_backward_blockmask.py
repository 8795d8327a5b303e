"""GPU parity: the backward pass over a BlockMask (attn_bwd_blockmask) against the fp64
oracle's gradients with the BlockMask mask_mod, and the key-tile-major lists
(attn_blockmask_transpose) bitwise against the transposed tile classes.

The gradient bar is the one of test_gpu_backward (2^-7 times the oracle's sum of |terms|
per element; keys no row sees exactly 0)."""
import math

import numpy as np
import pytest
import torch

from oracle import backward as OBW, masks as M, blockmask as OB
import workloads as W
from gpu_util import f64, assert_close, announce
from test_gpu_backward import assert_grad_close, fp16_floor
from test_gpu_blockmask import _gm_mod

pytestmark = pytest.mark.gpu
if torch.cuda.is_available():
    import tiled_attention_attn_amd as T
DEV = "cuda"


def _tile_map(g, nq_t, nk_t, frac_full, frac_part, causal_diag):
    """uint8 [nq_t, nk_t] classes: random FULL / PARTIAL tiles, plus PARTIAL diagonal tiles."""
    r = torch.rand(nq_t, nk_t, generator=g)
    tm = torch.zeros(nq_t, nk_t, dtype=torch.uint8)
    tm[r < frac_full] = W.TILE_FULL
    tm[(r >= frac_full) & (r < frac_full + frac_part)] = W.TILE_PARTIAL
    if causal_diag:
        for i in range(min(nq_t, nk_t)):
            tm[i, i] = W.TILE_PARTIAL
    return tm


CASES = [
    # (id, B, Hq, Hkv, Nq, Nk, D, per-head maps, spec of the PARTIAL predicate, dtype)
    ("causal_tiles_d64_n700_gqa", 1, 4, 2, 700, 700, 64, False, {"causal": True}, "bf16"),
    ("causal_tiles_d128_n700_gqa", 1, 4, 2, 700, 700, 128, False, {"causal": True}, "bf16"),
    ("per_head_maps_d64_n600", 1, 4, 2, 600, 600, 64, True, {"causal": True}, "bf16"),
    ("per_head_maps_d128_b2_n520", 2, 2, 1, 520, 520, 128, True, {"window": (100, 100)}, "bf16"),
    ("no_predicate_d128_q300_k900", 1, 2, 2, 300, 900, 128, False, {}, "bf16"),
    ("causal_tiles_d64_fp16", 1, 2, 2, 500, 500, 64, False, {"causal": True}, "fp16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_blockmask_matches_oracle(case):
    name, B, Hq, Hkv, Nq, Nk, D, per_head, spec, dt = case
    announce(f"backward blockmask {name}")
    dtype = torch.float16 if dt == "fp16" else torch.bfloat16
    g = W.generator(len(name) * 7 + 1)
    q = W.randn_half(g, (B, Hq, Nq, D), dtype)
    k = W.randn_half(g, (B, Hkv, Nk, D), dtype)
    v = W.randn_half(g, (B, Hkv, Nk, D), dtype)
    do = W.randn_half(g, (B, Hq, Nq, D), dtype)
    nq_t, nk_t = (Nq + 127) // 128, (Nk + 127) // 128
    Bm, Hm = (B, Hq) if per_head else (1, 1)
    tm = torch.stack([torch.stack([_tile_map(g, nq_t, nk_t, 0.25, 0.2, bool(spec.get("causal")))
                                   for _ in range(Hm)]) for _ in range(Bm)])
    gm, pmod = _gm_mod(spec, Nq, Nk)
    scale = 1.0 / math.sqrt(D)
    qg, kg, vg, dog = (x.to(DEV) for x in (q, k, v, do))
    bm = T.BlockMask(Bm, Hm, Nq, Nk)
    T.attn_build_blockmask(bm, B, Nq, Nk, tile_map=tm.contiguous().to(DEV))
    bm_t = T.attn_blockmask_transpose(bm)
    o = torch.empty_like(qg)
    lse = torch.empty(B, Hq, Nq, dtype=torch.float32, device=DEV)
    T.attn_fwd_blockmask(qg, kg, vg, o, bm, lse, scale, gm)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (qg, kg, vg))
    T.attn_bwd_blockmask(qg, kg, vg, o, dog, lse, dq, dk, dv, bm, bm_t, None, scale, gm)
    torch.cuda.synchronize()
    # key-tile-major lists: bitwise the lists of the transposed class map
    for bb in range(Bm):
        for hh in range(Hm):
            pn, pi, fn, fi = OB.tile_lists(tm[bb, hh].numpy().T.copy())
            assert np.array_equal(bm_t.part_num[bb, hh].cpu().numpy(), pn), name
            assert np.array_equal(bm_t.full_num[bb, hh].cpu().numpy(), fn), name
            assert np.array_equal(bm_t.part_idx[bb, hh].cpu().numpy(), pi), name
            assert np.array_equal(bm_t.full_idx[bb, hh].cpu().numpy(), fi), name
    mod = M.blockmask(tm.numpy(), 128, pmod)
    ro, rl = __import__("oracle").attention(f64(q), f64(k), f64(v), scale, mod)
    assert_close(f64(o), f64(lse), ro, rl, f"{name} forward")
    rq, rk, rv, (mq, mk, mv) = OBW.attention_bwd(f64(q), f64(k), f64(v), f64(do), scale, mod,
                                                 row_block=256, bound=True, o_used=f64(o))
    fq, fk, fv = fp16_floor(f64(q), f64(k), f64(do), scale, mod) if dt == "fp16" else (0.0,) * 3
    assert_grad_close(f64(dq), rq, mq, f"{name} dQ", fq)
    assert_grad_close(f64(dk), rk, mk, f"{name} dK", fk)
    assert_grad_close(f64(dv), rv, mv, f"{name} dV", fv)
    # keys no row sees: exactly zero
    seen = np.zeros((B, Hkv, Nk), dtype=bool)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            seen[b, h // G] |= M.dense(mod, b, h, Nq, Nk).any(0)
    assert torch.all(dk.cpu()[torch.from_numpy(~seen)] == 0)
    assert torch.all(dv.cpu()[torch.from_numpy(~seen)] == 0)


def test_backward_blockmask_all_partial_causal_equals_dense_causal():
    """Every tile PARTIAL with the causal predicate is the dense causal mask: the gradients of
    the two backward paths agree within the gradient bar of each other's oracle."""
    announce("backward blockmask all-partial == causal")
    B, H, N, D = 1, 2, 1000, 128
    g = W.generator(21)
    q, k, v, do = (W.randn_bf16(g, (B, H, N, D)) for _ in range(4))
    qg, kg, vg, dog = (x.to(DEV) for x in (q, k, v, do))
    nt = (N + 127) // 128
    tm = torch.full((1, 1, nt, nt), W.TILE_PARTIAL, dtype=torch.uint8)
    bm = T.BlockMask(1, 1, N, N)
    T.attn_build_blockmask(bm, 1, N, N, tile_map=tm.to(DEV))
    bm_t = T.attn_blockmask_transpose(bm)
    o = torch.empty_like(qg)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    T.attn_fwd(qg, kg, vg, o, lse, None, T.Mask(causal=True))
    g1 = tuple(torch.empty_like(x) for x in (qg, kg, vg))
    g2 = tuple(torch.empty_like(x) for x in (qg, kg, vg))
    T.attn_bwd(qg, kg, vg, o, dog, lse, *g1, None, None, T.Mask(causal=True))
    T.attn_bwd_blockmask(qg, kg, vg, o, dog, lse, *g2, bm, bm_t, None, None, T.Mask(causal=True))
    torch.cuda.synchronize()
    rq, rk, rv, (mq, mk, mv) = OBW.attention_bwd(f64(q), f64(k), f64(v), f64(do), 1 / math.sqrt(D),
                                                 M.causal(N, N), row_block=250, bound=True,
                                                 o_used=f64(o))
    for got, ref, mag, what in zip(g2, (rq, rk, rv), (mq, mk, mv), ("dQ", "dK", "dV")):
        assert_grad_close(f64(got), ref, mag, f"blockmask {what}")
    # the dQ kernel visits the tiles in the same ascending order on both paths: bitwise
    assert torch.equal(g1[0], g2[0])


def test_backward_blockmask_rejects_score_changes():
    q = torch.zeros(1, 2, 128, 128, dtype=torch.bfloat16, device=DEV)
    bm = T.BlockMask(1, 1, 128, 128)
    bm_t = T.attn_blockmask_transpose(bm)
    lse = torch.zeros(1, 2, 128, device=DEV)
    sm = T.ScoreMod(softcap=20.0)
    with pytest.raises(T.AttnError) as e:
        T.attn_bwd_blockmask(q, q, q, q, q, lse, q.clone(), q.clone(), q.clone(), bm, bm_t, smod=sm)
    assert e.value.status == -13
