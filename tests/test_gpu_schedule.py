"""GPU race check: one call under two work-group schedules gives bitwise-equal outputs.

Every output row (every dK / dV key in the backward pass) is produced by exactly one work
group, with a fixed order of its sums, so the schedule flags -- no tile pairing, no XCD
remap, work groups numbered in reverse -- may change which work group computes what and
which work groups share a CU at the same time, but never a bit of the result.  A missing
barrier or wait (an LDS read racing the copy that fills it) would make the result depend
on that timing and show up as a difference here."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import announce

pytestmark = pytest.mark.gpu
if torch.cuda.is_available():
    import tiled_attention_attn_amd as T
DEV = "cuda"



def _alts():
    return [T.SCHED_NO_PAIRING | T.SCHED_NO_XCD_REMAP | T.SCHED_REVERSE, T.SCHED_REVERSE]


def _bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int16 if a.element_size() == 2 else torch.int32),
                       b.contiguous().view(torch.int16 if b.element_size() == 2 else torch.int32))


def _mask_for(wl, sched):
    m = wl.mask
    if "doc_lengths" in m:
        starts = np.concatenate([[0], np.cumsum(m["doc_lengths"][0])]).astype(np.int32)
        off = torch.tensor(starts, dtype=torch.int32, device=DEV)[None]
        return T.Mask(window=(m["window"], m["window"]), doc_offsets=off, schedule=sched)
    if m.get("block_size"):
        return T.Mask(block_size=m["block_size"], schedule=sched)
    return T.Mask(causal=True, schedule=sched)


@pytest.mark.parametrize("name", ["causal_b2h16n4096d64", "window_doc_b1h32n8192d128",
                                  "blockdiff_b1h32n8192d128"])
def test_prefill_schedules_bitwise(name):
    announce(f"schedules prefill {name}")
    wl = W.FULL_SIZE[name]()
    q, k, v = (wl.tensors[x].to(DEV) for x in ("q", "k", "v"))
    B, H, N, D = q.shape
    outs = []
    for sched in [0] + _alts():
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
        T.attn_fwd(q, k, v, o, lse, wl.scale, _mask_for(wl, sched))
        outs.append((o, lse))
    torch.cuda.synchronize()
    for (o, lse), sched in zip(outs[1:], _alts()):
        assert _bits_equal(o, outs[0][0]) and _bits_equal(lse, outs[0][1]), f"{name} sched {sched:#x}"


def test_blockmask_schedules_bitwise():
    announce("schedules blockmask_gqa_b1h32kv8n32768d128")
    wl = W.blockmask_gqa_b1h32kv8n32768d128()
    q, k, v = (wl.tensors[x].to(DEV) for x in ("q", "k", "v"))
    N = 32768
    bm = T.BlockMask(1, 1, N, N)
    T.attn_build_blockmask(bm, 1, N, N, tile_map=wl.mask["tile_map"][None, None].contiguous().to(DEV))
    outs = []
    for sched in [0] + _alts():
        o = torch.full_like(q, float("nan"))
        lse = torch.full((1, 32, N), float("nan"), dtype=torch.float32, device=DEV)
        T.attn_fwd_blockmask(q, k, v, o, bm, lse, wl.scale, T.Mask(causal=True, schedule=sched))
        outs.append((o, lse))
    torch.cuda.synchronize()
    for (o, lse), sched in zip(outs[1:], _alts()):
        assert _bits_equal(o, outs[0][0]) and _bits_equal(lse, outs[0][1]), f"sched {sched:#x}"


@pytest.mark.parametrize("name", ["causal_b2h16n4096d64", "blockdiff_b1h8n2048d128"])
def test_backward_schedules_bitwise(name):
    announce(f"schedules backward {name}")
    if name == "causal_b2h16n4096d64":
        wl = W.causal_b2h16n4096d64()
    else:
        wl = W.dense(name, 1, 8, 8, 2048, 128, dict(block_size=16), seed=4)
    q, k, v = (wl.tensors[x].to(DEV) for x in ("q", "k", "v"))
    B, H, N, D = q.shape
    do = W.randn_bf16(W.generator(9), tuple(q.shape)).to(DEV)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, dtype=torch.float32, device=DEV)
    T.attn_fwd(q, k, v, o, lse, wl.scale, _mask_for(wl, 0))
    outs = []
    for sched in [0] + _alts():
        grads = tuple(torch.full_like(x, float("nan")) for x in (q, k, v))
        T.attn_bwd(q, k, v, o, do, lse, *grads, None, wl.scale, _mask_for(wl, sched))
        outs.append(grads)
    torch.cuda.synchronize()
    for g, sched in zip(outs[1:], _alts()):
        for a, b, what in zip(g, outs[0], ("dQ", "dK", "dV")):
            assert _bits_equal(a, b), f"{name} {what} sched {sched:#x}"


def test_decode_schedules_bitwise():
    announce("schedules decode_b16h32kv8q16k32768d128")
    wl = W.decode_b16h32kv8q16k32768d128()
    t = {x: wl.tensors[x].to(DEV) for x in ("q", "k_pool", "v_pool", "block_table", "seq_lens")}
    B, Hq, Lq, D = t["q"].shape
    S = T.attn_decode_num_splits(B, 8, 2048)
    outs = []
    for sched in [0] + _alts():
        ws_o = torch.full((B, Hq, Lq, S, D), float("nan"), dtype=torch.float32, device=DEV)
        ws_l = torch.full((B, Hq, Lq, S), float("nan"), dtype=torch.float32, device=DEV)
        T.attn_decode_splitkv(t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"], 2048, S,
                              ws_o, ws_l, wl.scale, T.Mask(causal=True, schedule=sched))
        outs.append((ws_o, ws_l))
    torch.cuda.synchronize()
    for (a, b), sched in zip(outs[1:], _alts()):
        assert _bits_equal(a, outs[0][0]) and _bits_equal(b, outs[0][1]), f"sched {sched:#x}"
