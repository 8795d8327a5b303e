"""GPU parity: attn_fwd_auto, the shape-based switch between the prefill kernels and
split-KV + combine over contiguous K/V, against the fp64 CPU oracle; plus bitwise
agreement of the contiguous split-KV path with the paged one at full size."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import masks as M, paged as OP, score_mods as SM
import workloads as W
from gpu_util import (f64, assert_close, bf16_bits, bits_to_f64, announce, COUNT_LSE_TOL)
from test_gpu_prefill import _mask_pair

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # with a GPU present the HIP library must load: no fallback
    import tiled_attention_attn_amd as T
DEV = "cuda"


def _auto(q, k, v, scale, gm, layout="bhnd", smod=None, expect=None):
    """q/k/v CPU tensors [B,H,N,D]; runs attn_fwd_auto and returns (O, LSE) on the CPU."""
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if expect is not None:
        assert T.attn_fwd_auto_plan(B, Hq, Hkv, Nq, Nk, D, smod).path == expect
    if layout == "bnhd":
        qg, kg, vg = (x.transpose(1, 2).contiguous().to(DEV).transpose(1, 2) for x in (q, k, v))
        o = torch.empty(B, Nq, Hq, D, dtype=q.dtype, device=DEV).transpose(1, 2)
    else:
        qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
        o = torch.empty_like(qg)
    o.fill_(float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=DEV)
    need = T.attn_fwd_auto_plan(B, Hq, Hkv, Nq, Nk, D, smod).workspace_bytes
    ws = torch.full((max(need // 4, 1),), float("nan"), dtype=torch.float32, device=DEV)
    T.attn_fwd_auto(qg, kg, vg, o, lse, scale, gm, workspace=ws, smod=smod)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


SPLIT = [
    # (id, B, Hq, Hkv, Nq, Nk, D, mask spec, layout)
    ("bidir_gqa4_d128", 2, 8, 2, 16, 1500, 128, {}, "bhnd"),
    ("causal_d64", 1, 4, 4, 16, 700, 64, {"causal": True}, "bhnd"),
    ("draft_window_d128", 2, 4, 1, 8, 3000, 128, {"window": (1000, 1000)}, "bnhd"),
    ("causal_docs_d128", 2, 4, 2, 16, 2000, 128, {"causal": True, "docs": [[500, 1499, 1], [2000]]}, "bhnd"),
    ("block_diffusion_d64", 1, 2, 2, 32, 1024, 64, {"block": 16}, "bnhd"),
    ("rows64_g64_d128", 1, 64, 1, 1, 600, 128, {"causal": True}, "bhnd"),
    ("ragged_d64", 3, 6, 3, 5, 777, 64, {"causal": True, "window": (300, 0)}, "bhnd"),
    ("one_query_d128", 4, 8, 8, 1, 513, 128, {"causal": True}, "bnhd"),
    ("min_keys_d64", 2, 4, 2, 3, 512, 64, {"causal": True}, "bhnd"),          # Nk at the threshold
    ("single_split_d64", 64, 8, 8, 1, 700, 64, {"causal": True}, "bhnd"),     # B * Hkv = 512: S = 1
]


@pytest.mark.parametrize("case", SPLIT, ids=[c[0] for c in SPLIT])
def test_split_path_vs_oracle(case):
    name, B, Hq, Hkv, Nq, Nk, D, spec, layout = case
    announce(f"auto split {name}")
    g = W.generator(zlib.crc32(name.encode()) % 9973)
    q = W.randn_bf16(g, (B, Hq, Nq, D))
    k = W.randn_bf16(g, (B, Hkv, Nk, D))
    v = W.randn_bf16(g, (B, Hkv, Nk, D))
    scale = 1.0 / math.sqrt(D)
    gm, mod = _mask_pair(spec, B, Nq, Nk)
    o, lse = _auto(q, k, v, scale, gm, layout, expect=T.PATH_SPLITKV)
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), scale, mod)
    assert_close(f64(o), f64(lse), ro, rl, name)


@pytest.mark.parametrize("name", ["causal_docs_d128", "ragged_d64"])
def test_split_path_key_counts(name):
    """Q = 0: LSE = ln(#visible keys) to 1e-5 on every row, so a key lost or counted twice
    at a split boundary shows."""
    name_, B, Hq, Hkv, Nq, Nk, D, spec, layout = next(c for c in SPLIT if c[0] == name)
    announce(f"auto split counts {name}")
    g = W.generator(5)
    k = W.randn_bf16(g, (B, Hkv, Nk, D))
    v = W.randn_bf16(g, (B, Hkv, Nk, D))
    q = torch.zeros(B, Hq, Nq, D, dtype=torch.bfloat16)
    gm, mod = _mask_pair(spec, B, Nq, Nk)
    _, lse = _auto(q, k, v, 0.1, gm, layout, expect=T.PATH_SPLITKV)
    cnt = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            vis = M.dense(mod, b, h, Nq, Nk, np.arange(Nq))
            cnt[b, h] = vis.sum(axis=1)
    assert np.max(np.abs(f64(lse) - np.log(cnt))) <= COUNT_LSE_TOL


def test_split_path_fp16_alibi_softcap():
    """fp16 inputs, ALiBi and the soft-cap (D = 64 and 128) on the split-KV path."""
    from test_gpu_score_mod import alibi_slopes, CAP
    for D, dtype, sym, cap in ((128, torch.float16, False, False), (64, torch.bfloat16, True, False),
                               (128, torch.bfloat16, False, True)):
        announce(f"auto split D={D} {dtype} alibi sym={sym} cap={cap}")
        B, Hq, Hkv, Nq, Nk = 2, 8, 2, 12, 2100
        g = W.generator(31 + D)
        q = W.randn_half(g, (B, Hq, Nq, D), dtype)
        k = W.randn_half(g, (B, Hkv, Nk, D), dtype)
        v = W.randn_half(g, (B, Hkv, Nk, D), dtype)
        slopes = alibi_slopes(Hq)
        smod = T.ScoreMod(alibi_slopes=slopes.to(DEV), symmetric=sym, softcap=CAP if cap else None)
        spec = {"window": (900, 900)} if sym else {"causal": True}
        gm, mod = _mask_pair(spec, B, Nq, Nk)
        o, lse = _auto(q, k, v, 1.0 / math.sqrt(D), gm, smod=smod, expect=T.PATH_SPLITKV)
        assert o.dtype == dtype
        sm = (SM.alibi_sym if sym else SM.alibi)(slopes.double().numpy(), Nq, Nk)
        if cap:
            sm = SM.combine(SM.softcap(CAP), sm)
        ro, rl = oracle.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), mod, score_mod=sm)
        assert_close(f64(o), f64(lse), ro, rl, f"alibi D={D} cap={cap}")


def test_split_path_bias_table():
    """A relative-position bias table (with ALiBi) on the split-KV path, against the oracle."""
    from test_gpu_score_mod import alibi_slopes
    B, Hq, Hkv, Nq, Nk, D, R = 2, 8, 2, 12, 1800, 128, 40
    announce("auto split bias table")
    g = W.generator(91)
    q = W.randn_bf16(g, (B, Hq, Nq, D))
    k = W.randn_bf16(g, (B, Hkv, Nk, D))
    v = W.randn_bf16(g, (B, Hkv, Nk, D))
    slopes = alibi_slopes(Hq)
    table = (0.5 * torch.randn(Hq, 2 * R + 1, generator=torch.Generator().manual_seed(3))).float()
    smod = T.ScoreMod(alibi_slopes=slopes.to(DEV), rel_bias=table.to(DEV))
    gm, mod = _mask_pair({"causal": True}, B, Nq, Nk)
    o, lse = _auto(q, k, v, 1.0 / math.sqrt(D), gm, smod=smod, expect=T.PATH_SPLITKV)
    sm = SM.combine(SM.alibi(slopes.double().numpy(), Nq, Nk), SM.rel_bias(table.double().numpy(), R, Nq, Nk))
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), 1.0 / math.sqrt(D), mod, score_mod=sm)
    assert_close(f64(o), f64(lse), ro, rl, "auto split bias table")


def test_prefill_path_is_attn_fwd():
    """Prefill-shaped calls (80 query rows a KV head: too many for one split-KV group; one with
    a bias table) run attn_fwd itself: bitwise the same O and LSE."""
    for (B, Hq, Hkv, Nq, Nk, D) in ((1, 4, 2, 300, 300, 64), (2, 4, 1, 20, 900, 128)):
        announce(f"auto prefill {B}x{Hq}x{Hkv} {Nq}x{Nk} D={D}")
        g = W.generator(Nq + D)
        q = W.randn_bf16(g, (B, Hq, Nq, D)).to(DEV)
        k = W.randn_bf16(g, (B, Hkv, Nk, D)).to(DEV)
        v = W.randn_bf16(g, (B, Hkv, Nk, D)).to(DEV)
        smod = None
        if D == 128:
            tb = (0.3 * torch.randn(Hq, 9, generator=torch.Generator().manual_seed(1))).float().to(DEV)
            smod = T.ScoreMod(rel_bias=tb)
        assert T.attn_fwd_auto_plan(B, Hq, Hkv, Nq, Nk, D, smod).path == T.PATH_PREFILL
        gm = T.Mask(causal=True)
        o1, o2 = torch.empty_like(q), torch.empty_like(q)
        l1 = torch.empty(B, Hq, Nq, dtype=torch.float32, device=DEV)
        l2 = torch.empty_like(l1)
        T.attn_fwd(q, k, v, o1, l1, None, gm, smod=smod)
        T.attn_fwd_auto(q, k, v, o2, l2, None, gm, smod=smod)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_shape_b16h32kv8q16k32768d128_contiguous():
    """The full decode workload with K/V gathered into contiguous [B, Hkv, Nk, D] tensors:
    attn_fwd_auto takes split-KV with the same 4 splits of 8192 keys as the paged call, so
    O and LSE are bitwise those of attn_decode_splitkv + combine over the page pool; sampled
    (sequence, head) rows also against the oracle."""
    announce("auto decode_b16h32kv8q16k32768d128 contiguous")
    wl = W.decode_b16h32kv8q16k32768d128()
    t = wl.tensors
    B, Hq, Hkv, Lq, Nk, D = 16, 32, 8, 16, 32768, 128
    plan = T.attn_fwd_auto_plan(B, Hq, Hkv, Lq, Nk, D)
    S = T.attn_decode_num_splits(B, Hkv, 2048)
    assert plan.path == T.PATH_SPLITKV and plan.num_splits == S == 4
    q = t["q"].to(DEV)
    bt = t["block_table"].to(DEV)
    kp, vp = t["k_pool"].to(DEV), t["v_pool"].to(DEV)
    # logical key j of sequence b: pool[bt[b, j // 16], j % 16]
    j = torch.arange(Nk, device=DEV)
    kc = kp[bt[:, j // 16].long(), (j % 16)[None]].permute(0, 2, 1, 3).contiguous()  # [B, Hkv, Nk, D]
    vc = vp[bt[:, j // 16].long(), (j % 16)[None]].permute(0, 2, 1, 3).contiguous()
    ws_o = torch.empty(B, Hq, Lq, S, D, dtype=torch.float32, device=DEV)
    ws_l = torch.empty(B, Hq, Lq, S, dtype=torch.float32, device=DEV)
    T.attn_decode_splitkv(q, kp, vp, bt, t["seq_lens"].to(DEV), 2048, S, ws_o, ws_l, wl.scale)
    o_p = torch.empty(B, Hq, Lq, D, dtype=torch.bfloat16, device=DEV)
    l_p = torch.empty(B, Hq, Lq, dtype=torch.float32, device=DEV)
    T.attn_decode_combine(ws_o, ws_l, o_p, l_p)
    del kp, vp, ws_o, ws_l
    o_a = torch.empty_like(o_p)
    l_a = torch.empty_like(l_p)
    T.attn_fwd_auto(q, kc, vc, o_a, l_a, wl.scale, T.Mask(causal=True))
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_p) and torch.equal(l_a, l_p)
    kbits, vbits = bf16_bits(kc[[0, 15]].cpu()), bf16_bits(vc[[0, 15]].cpu())
    qf, o_c, l_c = f64(t["q"]), o_a.cpu(), l_a.cpu()
    for bi, b in enumerate((0, 15)):
        for hq in (0, 31):
            kvh = hq // 4
            ro, rl = oracle.attention(qf[b:b + 1, hq:hq + 1], bits_to_f64(kbits[bi:bi + 1, kvh:kvh + 1]),
                                      bits_to_f64(vbits[bi:bi + 1, kvh:kvh + 1]), wl.scale, M.causal(Lq, Nk))
            assert_close(f64(o_c[b:b + 1, hq:hq + 1]), f64(l_c[b:b + 1, hq:hq + 1]), ro, rl,
                         f"auto cfg5 b{b} hq{hq}")
