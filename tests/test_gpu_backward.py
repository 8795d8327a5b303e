"""GPU parity: attn_bwd (dQ, dK, dV) against the fp64 CPU oracle's gradients.

Bar, per element (derived from the arithmetic of the kernels):  every gradient
element is a sum of products whose bf16-rounded factor (P or dS, each rounded
once, relative error <= 2^-9) multiplies an exact bf16 input, accumulated in
fp32, and written as bf16 (another 2^-9).  dS also carries the error of
Delta = rowsum(dO * O) through the O the kernel is given.  So
|g - g_ref| <= 2^-8 * m, with m the oracle's sum of |terms| of that element
(oracle.backward, ``bound=True``; the given O's error enters m with factor
2^8).  The tests allow 2^-7 * m: a factor 2 for the exp2 approximation, the
fp32 LSE and fp32 accumulation.  A key seen by no row must get exactly 0.

fp16 inputs (P, dS and the gradients rounded to fp16): below 2^-14 the fp16
grid is absolute (subnormal spacing 2^-24), so a value rounded there is off
by up to 2^-25, not 2^-11 relative.  The fp16 bar adds that floor once for
the written gradient and once per rounded P or dS, times the sum of |other
factor| over the element's terms (``fp16_floor``).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as OBW, masks as M
import workloads as W
from gpu_util import f64, LazyF64, announce
from test_gpu_prefill import _mask_pair

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # with a GPU present the HIP library must load: no fallback
    import tiled_attention_attn_amd as T
DEV = "cuda"
REL = 2.0 ** -7


def assert_grad_close(got, ref, mag, what, floor=0.0):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    err = np.abs(got - ref)
    bar = REL * mag + floor
    bad = err > bar
    if bad.any():
        i = np.unravel_index(np.argmax(err - bar), err.shape)
        fl = float(np.broadcast_to(floor, err.shape)[i])
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} elements over 2^-7 * m + floor; "
                             f"worst at {i}: got {got[i]:.6g} ref {ref[i]:.6g} m {mag[i]:.3g} floor {fl:.3g}")
    scale = max(float(np.max(np.abs(ref))), 1e-30)
    return float(np.max(err)) / scale


def fp16_floor(q, k, do, scale, mod):
    """Absolute error floor of fp16 rounding (subnormal spacing 2^-24, so at most 2^-25 per
    rounded value): 2^-25 for the written gradient, plus 2^-25 per fp16-rounded P / dS times
    the other factor of each term: dV sums P |dO| over the rows seeing the key, dK sums
    scale dS |Q|, dQ sums scale dS |K| over the row's keys."""
    q, k, do = (np.abs(np.asarray(x, dtype=np.float64)) for x in (q, k, do))
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    fq, fk, fv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(k)
    u = 2.0 ** -25
    for b in range(B):
        for h in range(Hq):
            vis = (M.dense(mod, b, h, Nq, Nk, np.arange(Nq)) if mod is not None
                   else np.ones((Nq, Nk), dtype=bool)).astype(np.float64)
            fq[b, h] = u * scale * (vis @ k[b, h // G])
            fk[b, h // G] += u * scale * (vis.T @ q[b, h])
            fv[b, h // G] += u * (vis.T @ do[b, h])
    return fq + u, fk + u, fv + u


def _to_dev(x, layout):
    if layout == "bnhd":
        return x.transpose(1, 2).contiguous().to(DEV).transpose(1, 2)
    return x.to(DEV)


def _empty_like_layout(B, H, N, D, layout, dtype=torch.bfloat16):
    if layout == "bnhd":
        return torch.full((B, N, H, D), float("nan"), dtype=dtype, device=DEV).transpose(1, 2)
    return torch.full((B, H, N, D), float("nan"), dtype=dtype, device=DEV)


def _fwd_bwd(q, k, v, do, scale, gm, layout="bhnd"):
    """GPU attn_fwd then attn_bwd; inputs CPU bf16.  Returns CPU (o, lse, dq, dk, dv)."""
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    qg, kg, vg, dog = (_to_dev(x, layout) for x in (q, k, v, do))
    o = _empty_like_layout(B, Hq, Nq, D, layout, q.dtype)
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=DEV)
    T.attn_fwd(qg, kg, vg, o, lse, scale, gm)
    dq = _empty_like_layout(B, Hq, Nq, D, layout, q.dtype)
    dk = _empty_like_layout(B, Hkv, Nk, D, layout, q.dtype)
    dv = _empty_like_layout(B, Hkv, Nk, D, layout, q.dtype)
    ws = torch.full((max(T.attn_bwd_workspace_bytes(B, Hq, Nq) // 4, 1),), float("nan"),
                    dtype=torch.float32, device=DEV)
    T.attn_bwd(qg, kg, vg, o, dog, lse, dq, dk, dv, ws, scale, gm)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu(), dq.cpu(), dk.cpu(), dv.cpu()


CASES = [
    # (id, B, Hq, Hkv, Nq, Nk, D, spec)
    ("none_d64", 1, 2, 2, 200, 200, 64, {}),
    ("none_d128_q200_k333", 1, 2, 1, 200, 333, 128, {}),
    ("causal_d64_n300", 2, 2, 2, 300, 300, 64, {"causal": True}),
    ("causal_d64_n1", 1, 1, 1, 1, 1, 64, {"causal": True}),
    ("causal_d128_n257_gqa", 1, 4, 2, 257, 257, 128, {"causal": True}),
    ("causal_d64_n640_gqa8", 1, 8, 1, 640, 640, 64, {"causal": True}),
    ("causal_bottom_right_d64", 1, 2, 2, 100, 300, 64, {"causal": True}),
    ("causal_empty_rows_d128", 1, 2, 2, 300, 100, 128, {"causal": True}),
    ("window_d128_n700_w40", 1, 2, 2, 700, 700, 128, {"window": (40, 40)}),
    ("window_asym_d64", 1, 2, 2, 500, 500, 64, {"window": (37, 5)}),
    ("docs_d64", 1, 2, 1, 600, 600, 64, {"docs": [[1, 255, 100, 244]]}),
    ("window_docs_d128", 2, 2, 2, 520, 520, 128, {"window": (64, 64), "docs": [[130, 250, 140], [520]]}),
    ("block_diffusion_d128", 1, 2, 2, 400, 400, 128, {"block": 16}),
    ("block_diffusion_d64_bs5", 1, 1, 1, 333, 333, 64, {"block": 5}),
    ("causal_window_d64", 1, 2, 2, 640, 640, 64, {"causal": True, "window": (200, 0)}),
    # A window mask without documents whose dK/dV row searches once branched into the
    # document search and read through the null offsets pointer (work group 1).
    ("window_b2_gqa2_d64_n520", 2, 2, 1, 520, 520, 64, {"window": (100, 100)}),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("layout", ["bhnd", "bnhd", "fp16"])
def test_backward_matches_oracle(case, layout):
    """bhnd / bnhd: bf16 in the two memory layouts; fp16: fp16 inputs in [B, H, N, D]."""
    name, B, Hq, Hkv, Nq, Nk, D, spec = case
    if layout == "bnhd" and name not in ("causal_d64_n300", "causal_d128_n257_gqa", "window_docs_d128"):
        pytest.skip("strided layout checked on a subset")
    if layout == "fp16" and name not in ("causal_d64_n300", "causal_d128_n257_gqa", "window_docs_d128",
                                         "causal_empty_rows_d128", "block_diffusion_d64_bs5"):
        pytest.skip("fp16 checked on a subset")
    announce(f"bwd {name} {layout}")
    dtype = torch.float16 if layout == "fp16" else torch.bfloat16
    g = W.generator(len(name) * 7 + Nq)
    q = W.randn_half(g, (B, Hq, Nq, D), dtype)
    k = W.randn_half(g, (B, Hkv, Nk, D), dtype)
    v = W.randn_half(g, (B, Hkv, Nk, D), dtype)
    do = W.randn_half(g, (B, Hq, Nq, D), dtype)
    scale = 1.0 / math.sqrt(D)
    gm, mod = _mask_pair(spec, B, Nq, Nk)
    o, lse, dq, dk, dv = _fwd_bwd(q, k, v, do, scale, gm, "bnhd" if layout == "bnhd" else "bhnd")
    assert dq.dtype == dtype
    rq, rk, rv, (mq, mk, mv) = OBW.attention_bwd(f64(q), f64(k), f64(v), f64(do), scale, mod,
                                                 row_block=256, bound=True, o_used=f64(o))
    fq, fk, fv = fp16_floor(f64(q), f64(k), f64(do), scale, mod) if layout == "fp16" else (0.0,) * 3
    eq = assert_grad_close(f64(dq), rq, mq, f"{name} dQ", fq)
    ek = assert_grad_close(f64(dk), rk, mk, f"{name} dK", fk)
    ev = assert_grad_close(f64(dv), rv, mv, f"{name} dV", fv)
    print(f"  normalised max err dQ {eq:.2e} dK {ek:.2e} dV {ev:.2e}")


def test_keys_and_rows_that_see_nothing():
    """A key no row sees gets dK = dV = 0 exactly; a row that sees no key gets dQ = 0
    exactly; one visible key per row gives P = 1, so dV = dO exactly."""
    announce("bwd unseen keys and rows")
    B, H, D = 1, 2, 64
    g = W.generator(5)
    q, do = (W.randn_bf16(g, (B, H, 100, D)) for _ in range(2))
    k, v = (W.randn_bf16(g, (B, H, 300, D)) for _ in range(2))
    # window (0, 0), 100 rows at positions 200..299: keys 0..199 are seen by no row
    gm, mod = _mask_pair({"window": (0, 0)}, B, 100, 300)
    o, _, dq, dk, dv = _fwd_bwd(q, k, v, do, 0.125, gm)
    assert torch.all(dk[:, :, :200] == 0) and torch.all(dv[:, :, :200] == 0)
    assert torch.equal(dv[:, :, 200:], do)
    rq, rk, _, (mq, mk, _) = OBW.attention_bwd(f64(q), f64(k), f64(v), f64(do), 0.125, mod,
                                               bound=True, o_used=f64(o))
    assert_grad_close(f64(dq), rq, mq, "window0 dQ")
    assert_grad_close(f64(dk), rk, mk, "window0 dK")
    # causal with Nq > Nk: rows 0..99 sit at positions < 0 and see no key
    q2, do2 = (W.randn_bf16(g, (B, H, 200, D)) for _ in range(2))
    gm2, _ = _mask_pair({"causal": True}, B, 200, 100)
    _, lse2, dq2, _, _ = _fwd_bwd(q2, k[:, :, :100], v[:, :, :100], do2, 0.125, gm2)
    assert torch.all(torch.isneginf(lse2[:, :, :100]))
    assert torch.all(dq2[:, :, :100] == 0)


def test_empty_sequences():
    announce("bwd empty")
    q = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.randn(1, 2, 50, 64, device=DEV).to(torch.bfloat16)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(k, float("nan"))
    lse = torch.zeros(1, 2, 0, dtype=torch.float32, device=DEV)
    T.attn_bwd(q, k, k, q, q, lse, q, dk, dv, None, 0.125, T.Mask(causal=True))
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
    q2 = torch.randn(1, 2, 40, 64, device=DEV).to(torch.bfloat16)
    k0 = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device=DEV)
    o = torch.zeros_like(q2)
    lse2 = torch.full((1, 2, 40), -math.inf, dtype=torch.float32, device=DEV)
    dq = torch.full_like(q2, float("nan"))
    T.attn_bwd(q2, k0, k0, o, q2, lse2, dq, k0, k0, None, 0.125, None)
    torch.cuda.synchronize()
    assert torch.all(dq == 0)


def test_backward_deterministic():
    announce("bwd deterministic")
    B, Hq, Hkv, N, D = 1, 4, 1, 700, 128
    g = W.generator(9)
    q = W.randn_bf16(g, (B, Hq, N, D)).to(DEV)
    k, v = (W.randn_bf16(g, (B, Hkv, N, D)).to(DEV) for _ in range(2))
    do = W.randn_bf16(g, (B, Hq, N, D)).to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty(B, Hq, N, dtype=torch.float32, device=DEV)
    T.attn_fwd(q, k, v, o, lse, 0.1, T.Mask(causal=True))
    outs = []
    for _ in range(2):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        T.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, None, 0.1, T.Mask(causal=True))
        outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_causal_b2h16n4096d64_sampled_heads():
    """The benchmark's backward workload at full size; two (batch, head) pairs checked
    against the oracle over every row and key of that head."""
    announce("bwd causal_b2h16n4096d64")
    wl = W.causal_b2h16n4096d64()
    t = wl.tensors
    g = W.generator(1234)
    do = W.randn_bf16(g, tuple(t["q"].shape))
    q, k, v = (t[x].to(DEV) for x in ("q", "k", "v"))
    dog = do.to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty(2, 16, 4096, dtype=torch.float32, device=DEV)
    gm = T.Mask(causal=True)
    T.attn_fwd(q, k, v, o, lse, wl.scale, gm)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    T.attn_bwd(q, k, v, o, dog, lse, dq, dk, dv, None, wl.scale, gm)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 13)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv, (mq, mk, mv) = OBW.attention_bwd(
            f64(t["q"][sl]), f64(t["k"][sl]), f64(t["v"][sl]), f64(do[sl]), wl.scale,
            M.causal(4096, 4096), row_block=512, bound=True, o_used=f64(o[sl]))
        assert_grad_close(f64(dq[sl]), rq, mq, f"b{b}h{h} dQ")
        assert_grad_close(f64(dk[sl]), rk, mk, f"b{b}h{h} dK")
        assert_grad_close(f64(dv[sl]), rv, mv, f"b{b}h{h} dV")
