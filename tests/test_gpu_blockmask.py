"""GPU parity: the BlockMask builder (bitwise vs tile classes from the oracle's dense mask)
and attn_fwd_blockmask (vs the oracle with the BlockMask mask_mod)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import masks as M, blockmask as OB
import workloads as W
from gpu_util import f64, LazyF64, assert_close, sample_rows, doc_offsets, announce

pytestmark = pytest.mark.gpu
if torch.cuda.is_available():
    import tiled_attention_attn_amd as T
DEV = "cuda"

BUILD_CASES = [
    ("causal", 1, 1000, 1000, {"causal": True}),
    ("causal_bottom_right", 1, 300, 1000, {"causal": True}),
    ("window", 1, 1100, 1100, {"window": (200, 200)}),
    ("window_docs", 2, 1500, 1500, {"window": (300, 300), "docs": [[100, 900, 500], [1500]]}),
    ("block16", 1, 700, 700, {"block": 16}),
    ("none", 1, 129, 257, {}),
]


def _gm_mod(spec, Nq, Nk):
    gm = T.Mask(causal=spec.get("causal", False), window=spec.get("window"), block_size=spec.get("block"))
    mods = []
    if spec.get("causal"):
        mods.append(M.causal(Nq, Nk))
    if spec.get("window"):
        mods.append(M.window(*spec["window"], Nq, Nk))
    if spec.get("block"):
        mods.append(M.block_causal(spec["block"], Nq, Nk))
    if spec.get("docs"):
        gm.doc_offsets = doc_offsets(spec["docs"], DEV)
        mods.append(M.document(spec["docs"], Nq, Nk))
    return gm, (M.and_(*mods) if mods else M.full())


@pytest.mark.parametrize("case", BUILD_CASES, ids=[c[0] for c in BUILD_CASES])
def test_builder_from_predicate_bitwise(case):
    name, B, Nq, Nk, spec = case
    announce(f"blockmask build {name}")
    gm, mod = _gm_mod(spec, Nq, Nk)
    bm = T.BlockMask(B, 1, Nq, Nk)
    T.attn_build_blockmask(bm, B, Nq, Nk, mask=gm)
    torch.cuda.synchronize()
    for b in range(B):
        cls = OB.classify(mod, b, 0, Nq, Nk, 128)
        pn, pi, fn, fi = OB.tile_lists(cls)
        assert np.array_equal(bm.part_num[b, 0].cpu().numpy(), pn), name
        assert np.array_equal(bm.full_num[b, 0].cpu().numpy(), fn), name
        assert np.array_equal(bm.part_idx[b, 0].cpu().numpy(), pi), name
        assert np.array_equal(bm.full_idx[b, 0].cpu().numpy(), fi), name


def test_builder_from_tile_map_bitwise():
    announce("blockmask build from map")
    g = W.generator(3)
    tm = W.blockmask_tile_map(g, 40, 0.3)
    tm[3, 30] = W.TILE_FULL  # an upper tile too
    tm_b = tm[None, None].expand(1, 2, 40, 40).contiguous().clone()
    tm_b[0, 1, 5, 1] = 7  # unknown codes are EMPTY
    bm = T.BlockMask(1, 2, 40 * 128, 40 * 128)
    T.attn_build_blockmask(bm, 1, 40 * 128, 40 * 128, tile_map=tm_b.to(DEV))
    torch.cuda.synchronize()
    for h in range(2):
        ref = tm_b[0, h].numpy().copy()
        ref[ref > 2] = 0
        pn, pi, fn, fi = OB.tile_lists(ref)
        assert np.array_equal(bm.part_num[0, h].cpu().numpy(), pn)
        assert np.array_equal(bm.part_idx[0, h].cpu().numpy(), pi)
        assert np.array_equal(bm.full_num[0, h].cpu().numpy(), fn)
        assert np.array_equal(bm.full_idx[0, h].cpu().numpy(), fi)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("D,Hq,Hkv,N", [(64, 4, 2, 1000), (128, 4, 1, 1300)])
def test_fwd_blockmask_small_vs_oracle(D, Hq, Hkv, N, dtype):
    announce(f"fwd_blockmask small D{D} N{N} {dtype}")
    g = W.generator(D + N)
    q = W.randn_half(g, (1, Hq, N, D), dtype)
    k = W.randn_half(g, (1, Hkv, N, D), dtype)
    v = W.randn_half(g, (1, Hkv, N, D), dtype)
    nt = (N + 127) // 128
    tm = W.blockmask_tile_map(g, nt, 0.3)
    tm[1, nt - 1] = W.TILE_FULL
    bm = T.BlockMask(1, 1, N, N)
    T.attn_build_blockmask(bm, 1, N, N, tile_map=tm[None, None].contiguous().to(DEV))
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.empty_like(qg)
    lse = torch.empty(1, Hq, N, dtype=torch.float32, device=DEV)
    T.attn_fwd_blockmask(qg, kg, vg, o, bm, lse, 1 / math.sqrt(D), T.Mask(causal=True))
    torch.cuda.synchronize()
    mod = M.blockmask(tm.numpy(), 128, M.causal(N, N))
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), 1 / math.sqrt(D), mod)
    assert_close(f64(o), f64(lse), ro, rl, "fwd_blockmask small")


def test_fwd_blockmask_from_predicate_matches_dense():
    """A BlockMask built from a predicate gives the oracle's dense-mask result."""
    announce("fwd_blockmask predicate")
    N = 1500
    spec = {"window": (300, 300), "docs": [[100, 900, 500]]}
    gm, mod = _gm_mod(spec, N, N)
    g = W.generator(5)
    q = W.randn_bf16(g, (1, 2, N, 128))
    k = W.randn_bf16(g, (1, 2, N, 128))
    v = W.randn_bf16(g, (1, 2, N, 128))
    bm = T.BlockMask(1, 1, N, N)
    T.attn_build_blockmask(bm, 1, N, N, mask=gm)
    qg, kg, vg = q.to(DEV), k.to(DEV), v.to(DEV)
    o = torch.empty_like(qg)
    lse = torch.empty(1, 2, N, dtype=torch.float32, device=DEV)
    T.attn_fwd_blockmask(qg, kg, vg, o, bm, lse, 0.1, gm)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), 0.1, mod)
    assert_close(f64(o), f64(lse), ro, rl, "predicate blockmask")


def test_config4_blockmask_gqa_b1h32kv8n32768d128_every_head_sampled_rows():
    """Block-sparse GQA prefill at full size: builder bitwise vs the map, every head on sampled
    rows (first and last 8, 32 random) vs the oracle, and every row of the first and the last
    head (KV heads 0 and 7)."""
    announce("blockmask_gqa_b1h32kv8n32768d128")
    wl = W.blockmask_gqa_b1h32kv8n32768d128()
    tm = wl.mask["tile_map"]
    assert int((tm == W.TILE_FULL).sum()) == 3264 and int((tm == W.TILE_PARTIAL).sum()) == 256
    q, k, v = (wl.tensors[x].to(DEV) for x in ("q", "k", "v"))
    N = 32768
    bm = T.BlockMask(1, 1, N, N)
    T.attn_build_blockmask(bm, 1, N, N, tile_map=tm[None, None].contiguous().to(DEV))
    o = torch.empty_like(q)
    lse = torch.empty(1, 32, N, dtype=torch.float32, device=DEV)
    T.attn_fwd_blockmask(q, k, v, o, bm, lse, wl.scale, T.Mask(causal=True))
    torch.cuda.synchronize()
    pn, pi, fn, fi = OB.tile_lists(tm.numpy())
    assert np.array_equal(bm.full_num[0, 0].cpu().numpy(), fn)
    assert np.array_equal(bm.full_idx[0, 0].cpu().numpy(), fi)
    mod = M.blockmask(tm.numpy(), 128, M.causal(N, N))
    qa, ka, va = (f64(wl.tensors[x]) for x in ("q", "k", "v"))
    for h in range(32):
        rows = sample_rows(N, 32, h)
        ro, rl = oracle.attention_rows(qa, ka, va, wl.scale, mod, 0, h, rows)
        assert_close(f64(o[0, h, rows]), f64(lse[0, h, rows]), ro, rl, f"cfg4 h{h}")
    for h in (0, 31):
        for r0 in range(0, N, 2048):
            rows = np.arange(r0, r0 + 2048)
            ro, rl = oracle.attention_rows(qa, ka, va, wl.scale, mod, 0, h, rows)
            assert_close(f64(o[0, h, rows]), f64(lse[0, h, rows]), ro, rl, f"cfg4 h{h} rows {r0}+2048")
