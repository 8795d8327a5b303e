"""GPU parity at the address limits of the boundary:

* row strides of 2^24 - 8 elements, the largest the boundary accepts for streamed tiles:
  a 128-row tile's copies then span almost 2^32 bytes, the limit of the kernels' 32-bit
  tile offsets (attn_fwd, attn_fwd_blockmask and attn_bwd at D=64 and D=128);
* a paged decode whose used pages all lie past the first 4 GiB of a 4.6 GB page pool, so
  the page addresses must be 64-bit.

The tensors are allocated at their full strided size on the GPU (about 6.7 GB each for
the wide rows) and only their logical elements are written.  Each case was replayed
clean on the CPU from the compiled kernels first (tests/test_isa_replay.py)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as OBW, masks as M, paged as OP
import workloads as W
from gpu_util import f64, assert_close, announce
from test_gpu_backward import assert_grad_close

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():  # with a GPU present the HIP library must load: no fallback
    import tiled_attention_attn_amd as T
DEV = "cuda"
ROW_STRIDE = 2**24 - 8


def _wide_rows(g, B, H, N, D):
    """[B, H, N, D] bf16 on the GPU with rows ROW_STRIDE elements apart (heads interleaved
    inside a row); only the logical elements are written."""
    t = torch.empty_strided((B, H, N, D), (N * ROW_STRIDE, D, ROW_STRIDE, 1), dtype=torch.bfloat16,
                            device=DEV)
    src = W.randn_bf16(g, (B, H, N, D))
    t.copy_(src.to(DEV))
    return t, src


@pytest.mark.parametrize("D", [64, 128])
def test_largest_row_stride_forward(D):
    B, H, N = 1, 2, 200
    announce(f"largest row stride forward D={D}")
    g = W.generator(D)
    (q, q_h), (k, k_h), (v, v_h) = (_wide_rows(g, B, H, N, D) for _ in range(3))
    assert q.stride(2) == ROW_STRIDE and k.stride(2) == ROW_STRIDE
    scale = 1.0 / math.sqrt(D)
    ro, rl = oracle.attention(f64(q_h), f64(k_h), f64(v_h), scale, M.causal(N, N))
    o = torch.full((B, H, N, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    T.attn_fwd(q, k, v, o, lse, scale, T.Mask(causal=True))
    torch.cuda.synchronize()
    assert_close(f64(o), f64(lse), ro, rl, f"attn_fwd, row stride 2^24 - 8, D={D}")
    # the BlockMask kernel on the same tensors: every tile PARTIAL under the causal predicate
    nt = (N + 127) // 128
    bm = T.BlockMask(1, 1, N, N)
    T.attn_build_blockmask(bm, B, N, N, tile_map=torch.ones(1, 1, nt, nt, dtype=torch.uint8, device=DEV))
    o2 = torch.full_like(o, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    T.attn_fwd_blockmask(q, k, v, o2, bm, lse2, scale, T.Mask(causal=True))
    torch.cuda.synchronize()
    assert_close(f64(o2), f64(lse2), ro, rl, f"attn_fwd_blockmask, row stride 2^24 - 8, D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_largest_row_stride_backward(D):
    B, H, N = 1, 2, 200
    announce(f"largest row stride backward D={D}")
    g = W.generator(100 + D)
    (q, q_h), (k, k_h), (v, v_h), (do, do_h) = (_wide_rows(g, B, H, N, D) for _ in range(4))
    scale = 1.0 / math.sqrt(D)
    mod = M.causal(N, N)
    o = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H, N), device=DEV)
    T.attn_fwd(q, k, v, o, lse, scale, T.Mask(causal=True))
    dq, dk, dv = (torch.full((B, H, N, D), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in range(3))
    T.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, None, scale, T.Mask(causal=True))
    torch.cuda.synchronize()
    rq, rk, rv, (mq, mk, mv) = OBW.attention_bwd(f64(q_h), f64(k_h), f64(v_h), f64(do_h), scale, mod,
                                                 row_block=256, bound=True, o_used=f64(o))
    for got, ref, mag, what in ((dq, rq, mq, "dQ"), (dk, rk, mk, "dK"), (dv, rv, mv, "dV")):
        assert_grad_close(f64(got), ref, mag, f"{what}, row stride 2^24 - 8, D={D}")


def test_paged_decode_pool_beyond_4gib():
    B, Hq, Hkv, Lq, D, ps, S, P = 2, 16, 8, 4, 128, 16, 3, 140_000
    sl = [300, 170]
    announce("paged decode, pool of 4.6 GB, pages past 4 GiB")
    g = W.generator(4)
    per_seq = (max(sl) + ps - 1) // ps
    first = P - 2000
    assert first * ps * Hkv * D * 2 > 2**32
    bt = (first + torch.randperm(2000, generator=g)[: B * per_seq]).reshape(B, per_seq).to(torch.int32)
    q = W.randn_bf16(g, (B, Hq, Lq, D))
    kp = torch.empty((P, ps, Hkv, D), dtype=torch.bfloat16, device=DEV)
    vp = torch.empty((P, ps, Hkv, D), dtype=torch.bfloat16, device=DEV)
    used = {}
    for name, pool in (("k", kp), ("v", vp)):
        pages = W.randn_bf16(g, (B * per_seq, ps, Hkv, D))
        pool[bt.flatten().long().to(DEV)] = pages.to(DEV)
        used[name] = torch.zeros((2000, ps, Hkv, D), dtype=torch.bfloat16)
        used[name][(bt.flatten() - first).long()] = pages
    ws_o = torch.empty((B, Hq, Lq, S, D), device=DEV)
    ws_l = torch.empty((B, Hq, Lq, S), device=DEV)
    o = torch.full((B, Hq, Lq, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, Hq, Lq), float("nan"), device=DEV)
    scale = 1.0 / math.sqrt(D)
    T.attn_decode_splitkv(q.to(DEV), kp, vp, bt.to(DEV), torch.tensor(sl, dtype=torch.int32, device=DEV),
                          per_seq, S, ws_o, ws_l, scale)
    T.attn_decode_combine(ws_o, ws_l, o, lse)
    torch.cuda.synchronize()
    bt_used = (bt - first).numpy()
    for b in range(B):
        kl = OP.gather(f64(used["k"]), bt_used, b, sl[b])[None]
        vl = OP.gather(f64(used["v"]), bt_used, b, sl[b])[None]
        ro, rl = oracle.attention(f64(q[b:b + 1]), kl, vl, scale, M.causal(Lq, sl[b]))
        assert_close(f64(o[b:b + 1]), f64(lse[b:b + 1]), ro, rl, f"sequence {b}")
    del kp, vp
    torch.cuda.empty_cache()
