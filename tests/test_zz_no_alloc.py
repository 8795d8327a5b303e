"""GPU: attn_decode_noalloc (split-KV + combine with the partials in the library's static
per-GPU buffer, no allocation) gives exactly the outputs of attn_decode_splitkv +
attn_decode_combine with a caller workspace, called through the C ABI: two calls in a row
on one GPU, the second with a smaller input, so the buffer's leftovers from the first call
cannot leak into the second."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import masks as M, paged as OP
import workloads as W
from gpu_util import f64, assert_close, announce

pytestmark = pytest.mark.gpu
if torch.cuda.is_available():
    import tiled_attention_attn_amd as T
DEV = "cuda"


def _strides(t):
    return (ctypes.c_int64 * 3)(*t.stride()[:3])


def _reference(t, S, max_pages, scale, dtype):
    """The existing two-call path with a caller workspace."""
    B, Hq, Lq, D = t["q"].shape
    ws_o = torch.empty(B, Hq, Lq, S, D, dtype=torch.float32, device=DEV)
    ws_l = torch.empty(B, Hq, Lq, S, dtype=torch.float32, device=DEV)
    T.attn_decode_splitkv(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], max_pages,
                          S, ws_o, ws_l, scale)
    o = torch.empty(B, Hq, Lq, D, dtype=dtype, device=DEV)
    lse = torch.empty(B, Hq, Lq, dtype=torch.float32, device=DEV)
    T.attn_decode_combine(ws_o, ws_l, o, lse)
    return o, lse


def _noalloc(t, S, max_pages, scale, dtype):
    """attn_decode_noalloc called directly through the C ABI (ctypes)."""
    lib = T.lib_handle()
    q, kp, vp, bt, sl = t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"]
    B, Hq, Lq, D = q.shape
    n_pages, ps, Hkv, _ = kp.shape
    o = torch.full((B, Hq, Lq, D), float("nan"), dtype=dtype, device=DEV)
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device=DEV)
    st = lib.attn_decode_noalloc(q.data_ptr(), _strides(q), kp.data_ptr(), vp.data_ptr(), n_pages,
                                 bt.data_ptr(), bt.stride(0), sl.data_ptr(), max_pages, B, Hq, Hkv, Lq,
                                 D, T.DTYPE_BF16 if dtype == torch.bfloat16 else T.DTYPE_F16, ps, S,
                                 scale, None, None, o.data_ptr(), _strides(o), lse.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0, T.attn_status_str(st)
    return o, lse


# (name, B, Hq, Hkv, Lq, Nk, D, seq_lens, S): the first call fills most of the buffer
CALLS = [
    ("large_b8h32kv8q16k4096d128", 8, 32, 8, 16, 4096, 128, None, 7),
    ("small_b2h8kv2q5k300d64", 2, 8, 2, 5, 300, 64, [300, 171], 3),
]


def test_noalloc_two_calls_match_the_workspace_path():
    outs = []
    for name, B, Hq, Hkv, Lq, Nk, D, sl, S in CALLS:
        announce(f"decode noalloc {name} S={S}")
        pages = (Nk + 15) // 16
        wl = W.paged_decode(name, B, Hq, Hkv, Lq, Nk, D, page_size=16, pool_pages=B * pages + 5, seed=3,
                            seq_lens=sl)
        t = {k: v.to(DEV) for k, v in wl.tensors.items() if k != "k_logical" and k != "v_logical"}
        assert B * Hq * Lq * S * (D + 1) * 4 <= T.attn_decode_noalloc_max_bytes()
        o_na, l_na = _noalloc(t, S, pages, wl.scale, torch.bfloat16)
        torch.cuda.synchronize()
        o_ref, l_ref = _reference(t, S, pages, wl.scale, torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ref), f"{name}: O differs from the workspace path"
        assert torch.equal(l_na, l_ref), f"{name}: LSE differs from the workspace path"
        # and the oracle's bar on a few sequences
        kp, vp, bt = f64(wl.tensors["k_pool"]), f64(wl.tensors["v_pool"]), wl.tensors["block_table"].numpy()
        lens = wl.tensors["seq_lens"].tolist()
        for b in (0, B - 1):
            kl = OP.gather(kp, bt, b, lens[b])[None]
            vl = OP.gather(vp, bt, b, lens[b])[None]
            ro, rl = oracle.attention(f64(wl.tensors["q"])[b:b + 1], kl, vl, wl.scale,
                                      M.causal(Lq, lens[b]))
            assert_close(f64(o_na[b:b + 1]), f64(l_na[b:b + 1]), ro, rl, f"{name} b{b}")
        outs.append((o_na, l_na))
