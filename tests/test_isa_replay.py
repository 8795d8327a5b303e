"""CPU replays of compiled kernels (tests/isa_replay): the prefill kernels, the backward
pass, the BlockMask backward and the paged decode; a static check of every kernel; and
pins of the replay's and the check's own logic.

The dK/dV kernel's row searches once compiled to code that evaluated the "mask has
documents" test as a lane mask inside a loop whose lanes leave one by one, and branched
on it in the next loop under another EXEC.  For the window-masked call below the two
lane sets were disjoint: the kernel took the document search and read through the null
offsets pointer.  These tests replay the library's compiled kernels, with the launch
arguments its host code computes, and require no out-of-bounds access, no lane-mask
reuse and results within the GPU tests' bars of the fp64 oracle.
"""
import ctypes
import math
import os
import shutil
import tempfile

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as OBW, masks as M
import workloads as W
from gpu_util import assert_close

HAVE_HIPCC = shutil.which("hipcc") is not None or os.path.exists("/opt/rocm/bin/hipcc")
REL = 2.0 ** -7  # the gradient bar of the GPU backward tests: 2^-7 times the oracle's sum of |terms|


def _strides(t):
    return (ctypes.c_int64 * 3)(*t.stride()[:3])


def _check_grad(got, ref, mag, what):
    err = np.abs(got.to(torch.float64).numpy() - ref)
    bad = err > REL * mag
    assert not bad.any(), f"{what}: {int(bad.sum())} of {err.size} elements over the bar"


def _backward_replay(B, Hq, Hkv, N, D, mask_flags, window=None, docs=None, kernels=None, seed=0, schedule=0):
    """attn_bwd through the recorded host library, then a replay of its launches."""
    from isa_replay.host import Replay
    from tiled_attention_attn_amd import _lib
    rp = Replay(("bwd",))
    g = W.generator(seed)
    q, k, v, do = (W.randn_bf16(g, s) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D), (B, Hq, N, D)))
    scale = 1.0 / math.sqrt(D)
    mods, desc = [], _lib.attn_mask_desc(flags=mask_flags | schedule, window_left=-1, window_right=-1)
    if mask_flags & 1:
        mods.append(M.causal(N, N))
    if window is not None:
        desc.window_left, desc.window_right = window
        mods.append(M.window(window[0], window[1], N, N))
    off = None
    if docs is not None:
        nd = max(len(d) for d in docs)
        rows = [np.concatenate([[0], np.cumsum(d), np.full(nd - len(d), sum(d))]) for d in docs]
        off = torch.tensor(np.stack(rows), dtype=torch.int32)
        desc.doc_offsets, desc.num_docs, desc.doc_stride = off.data_ptr(), nd, off.stride(0)
        mods.append(M.document(docs, N, N))
    mod = M.and_(*mods)
    ro, rl = oracle.attention(*(x.to(torch.float64).numpy() for x in (q, k, v)), scale, mod)
    o = torch.from_numpy(ro).to(torch.bfloat16)
    lse = torch.from_numpy(rl).to(torch.float32)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    ws = torch.zeros(max(int(rp.lib.attn_bwd_workspace_bytes(B, Hq, N)) // 4, 1))
    rp.register(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, ws=ws, doc_offsets=off)
    st = rp.lib.attn_bwd(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
                         o.data_ptr(), _strides(o), do.data_ptr(), _strides(do), lse.data_ptr(),
                         dq.data_ptr(), _strides(dq), dk.data_ptr(), _strides(dk), dv.data_ptr(), _strides(dv),
                         B, Hq, Hkv, N, N, D, 0, scale, ctypes.byref(desc), None, ws.data_ptr(), ws.numel() * 4,
                         None)
    assert st == 0, st
    rp.run(only=kernels)
    ref = OBW.attention_bwd(*(x.to(torch.float64).numpy() for x in (q, k, v, do)), scale, mod,
                            row_block=256, bound=True, o_used=o.to(torch.float64).numpy())
    return rp, (dq, dk, dv), ref


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_window_mask_backward_d64_replays_clean():
    """The shape whose dK/dV row search read through the null document pointer: every
    kernel of the call replays without a fault or a lane-mask note, within the bar."""
    rp, (dq, dk, dv), (rq, rk, rv, (mq, mk, mv)) = _backward_replay(
        2, 2, 1, 520, 64, 2, window=(100, 100), seed=11)
    assert [r[0].split("kernel")[0] for r in rp.ran] == ["_ZN5tattn14bwd_pre_", "_ZN5tattn13bwd_kv_",
                                                          "_ZN5tattn12bwd_q_"]
    assert not rp.notes, rp.notes
    _check_grad(dq, rq, mq, "dQ")
    _check_grad(dk, rk, mk, "dK")
    _check_grad(dv, rv, mv, "dV")


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_window_and_documents_backward_d128_replays_clean():
    """D = 128 with documents (the search's document steps run): the dK/dV kernel replays
    without a fault or a lane-mask note, within the bar."""
    rp, (dq, dk, dv), (rq, rk, rv, (mq, mk, mv)) = _backward_replay(
        2, 2, 2, 520, 128, 2 | 4, window=(64, 64), docs=[[130, 250, 140], [520]], kernels=["bwd_pre", "bwd_kv"],
        seed=12)
    assert not rp.notes, rp.notes
    _check_grad(dk, rk, mk, "dK")
    _check_grad(dv, rv, mv, "dV")


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_backward_schedules_replay_bitwise():
    """The causal backward under the default schedule and under all three schedule flags
    (no tile pairing, no XCD remap, work groups numbered in reverse).  Gradients start as
    NaN, so a tile no work group covers would show; the two calls must agree bit for bit,
    within the bar of the oracle.  With 8 heads of 256 rows both schedules launch a
    multiple of 8 work groups, so the XCD remap is in play."""
    from tiled_attention_attn_amd import _lib
    runs = []
    for sched in (0, _lib.SCHED_ALL):
        rp, grads, ref = _backward_replay(1, 8, 8, 256, 64, 1, seed=14, schedule=sched)
        assert not rp.notes, rp.notes
        runs.append(([(r[0], r[1]) for r in rp.ran], grads, ref))
    (ran0, g0, (rq, rk, rv, (mq, mk, mv))), (ran1, g1, _) = runs
    assert [r[0] for r in ran0] == [r[0] for r in ran1]
    assert ran0 != ran1, "the schedule flags left every grid unchanged"
    for a, b, what in zip(g0, g1, ("dQ", "dK", "dV")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"{what} differs between schedules"
    _check_grad(g0[0], rq, mq, "dQ")
    _check_grad(g0[1], rk, mk, "dK")
    _check_grad(g0[2], rv, mv, "dV")


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_blockmask_backward_per_head_maps_d128_replays_clean():
    """The BlockMask backward call that faulted on a GPU before the row-search fix: B=2,
    one tile map per (batch, head), a window predicate on PARTIAL tiles.  The list builder,
    the transposition and the dK/dV kernel replay without a fault or a lane-mask note;
    the transposed lists equal the oracle's and dK, dV are within the bar."""
    from isa_replay.host import Replay
    from tiled_attention_attn_amd import _lib
    from oracle import blockmask as OB
    rp = Replay(("bwd", "blockmask"))
    B, Hq, Hkv, N, D = 2, 2, 1, 520, 128
    g = W.generator(13)
    q, k, v, do = (W.randn_bf16(g, s) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D), (B, Hq, N, D)))
    nt = (N + 127) // 128
    tm = torch.stack([torch.stack([W.blockmask_tile_map(g, nt, 0.3) for _ in range(Hq)]) for _ in range(B)])
    tm = tm.contiguous()
    i32 = dict(dtype=torch.int32)
    fwd_lists = [torch.zeros(B, Hq, nt, **i32), torch.zeros(B, Hq, nt, nt, **i32),
                 torch.zeros(B, Hq, nt, **i32), torch.zeros(B, Hq, nt, nt, **i32)]
    key_lists = [torch.zeros_like(x) for x in fwd_lists]
    tmp = torch.zeros(B * Hq * nt * nt, dtype=torch.uint8)

    def desc(ls):
        return _lib.attn_blockmask(Bm=B, Hm=Hq, nQt=nt, nKt=nt, part_num=ls[0].data_ptr(), part_idx=ls[1].data_ptr(),
                                   full_num=ls[2].data_ptr(), full_idx=ls[3].data_ptr())
    bm, bm_t = desc(fwd_lists), desc(key_lists)
    scale = 1.0 / math.sqrt(D)
    mask = _lib.attn_mask_desc(flags=2, window_left=100, window_right=100)
    mod = M.blockmask(tm.numpy(), 128, M.window(100, 100, N, N))
    ro, rl = oracle.attention(*(x.to(torch.float64).numpy() for x in (q, k, v)), scale, mod)
    o, lse = torch.from_numpy(ro).to(torch.bfloat16), torch.from_numpy(rl).to(torch.float32)
    dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
    ws = torch.zeros(max(int(rp.lib.attn_bwd_workspace_bytes(B, Hq, N)) // 4, 1))
    rp.register(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, ws=ws, tm=tm, tmp=tmp,
                **{f"lists{i}": t for i, t in enumerate(fwd_lists + key_lists)})
    assert rp.lib.attn_build_blockmask(None, tm.data_ptr(), B, N, N, ctypes.byref(bm), None) == 0
    assert rp.lib.attn_blockmask_transpose(ctypes.byref(bm), ctypes.byref(bm_t), tmp.data_ptr(), tmp.numel(),
                                           None) == 0
    rp.run()
    st = rp.lib.attn_bwd_blockmask(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
                                   o.data_ptr(), _strides(o), do.data_ptr(), _strides(do), lse.data_ptr(),
                                   dq.data_ptr(), _strides(dq), dk.data_ptr(), _strides(dk), dv.data_ptr(),
                                   _strides(dv), B, Hq, Hkv, N, N, D, 0, scale, ctypes.byref(mask), None,
                                   ctypes.byref(bm), ctypes.byref(bm_t), ws.data_ptr(), ws.numel() * 4, None)
    assert st == 0, st
    rp.run(only=["bwd_pre", "bwd_kv"])
    assert not rp.notes, rp.notes
    for b in range(B):
        for h in range(Hq):
            pn, pi, fn, fi = OB.tile_lists(tm[b, h].numpy().T.copy())
            got = [x[b, h].numpy() for x in key_lists]
            assert all(np.array_equal(a, e) for a, e in zip(got, (pn, pi, fn, fi))), (b, h)
    _, rk, rv, (_, mk, mv) = OBW.attention_bwd(*(x.to(torch.float64).numpy() for x in (q, k, v, do)), scale, mod,
                                               row_block=256, bound=True, o_used=o.to(torch.float64).numpy())
    _check_grad(dk, rk, mk, "dK")
    _check_grad(dv, rv, mv, "dV")


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_paged_decode_with_empty_splits_replays_clean():
    """Split-KV decode + combine over ragged sequences where most splits of the short ones
    are empty (seq_lens 130, 1, 64 in 16-token pages, 9 splits): no fault, no race, no
    lane-mask note, and O / LSE equal to the oracle's within the GPU tests' bars."""
    from isa_replay.host import Replay
    from oracle import paged as OP
    rp = Replay(("decode",))
    B, Hq, Hkv, Lq, Nk, D, ps, S = 3, 4, 2, 2, 130, 64, 16, 9
    sl = [130, 1, 64]
    wl = W.paged_decode("replay", B, Hq, Hkv, Lq, Nk, D, page_size=ps, pool_pages=B * 9 + 7, seed=3, seq_lens=sl)
    t = wl.tensors
    q, kp, vp, bt, lens = t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"]
    ws_o = torch.full((B, Hq, Lq, S, D), float("nan"))
    ws_l = torch.full((B, Hq, Lq, S), float("nan"))
    o = torch.full((B, Hq, Lq, D), float("nan"), dtype=torch.bfloat16)
    lse = torch.full((B, Hq, Lq), float("nan"))
    rp.register(q=q, kp=kp, vp=vp, bt=bt, lens=lens, ws_o=ws_o, ws_l=ws_l, o=o, lse=lse)
    st = rp.lib.attn_decode_splitkv(q.data_ptr(), _strides(q), kp.data_ptr(), vp.data_ptr(), kp.shape[0],
                                    bt.data_ptr(), bt.stride(0), lens.data_ptr(), bt.shape[1], B, Hq, Hkv, Lq, D,
                                    0, ps, S, wl.scale, None, None, ws_o.data_ptr(), ws_l.data_ptr(), None)
    assert st == 0, st
    st = rp.lib.attn_decode_combine(ws_o.data_ptr(), ws_l.data_ptr(), B, Hq, Lq, S, D, 0, o.data_ptr(),
                                    _strides(o), lse.data_ptr(), None)
    assert st == 0, st
    rp.run()
    assert [r[0].split("kernel")[0] for r in rp.ran] == ["_ZN5tattn13decode_", "_ZN5tattn14combine_"]
    assert not rp.notes, rp.notes
    for b in range(B):
        kl = OP.gather(kp.to(torch.float64).numpy(), bt.numpy(), b, sl[b])[None]
        vl = OP.gather(vp.to(torch.float64).numpy(), bt.numpy(), b, sl[b])[None]
        ro, rl = oracle.attention(q[b:b + 1].to(torch.float64).numpy(), kl, vl, wl.scale, M.causal(Lq, sl[b]))
        assert_close(o[b:b + 1].to(torch.float64).numpy(), lse[b:b + 1].numpy(), ro, rl, f"sequence {b}")


_FWD_CASES = [
    # (id, B, Hq, Hkv, N, D, mask flags, window, documents, per-head BlockMask maps)
    ("causal_d64_gqa", 1, 4, 2, 700, 64, 1, None, None, False),            # fwd_kernel<64>
    ("window_docs_d128_b2", 2, 2, 1, 600, 128, 2 | 4, (64, 64), [[100, 300, 200], [600]], False),  # ping-pong
    ("blockmask_per_head_d128_b2", 2, 2, 1, 520, 128, 2, (100, 100), None, True),  # fwd_kernel<128, BlockMask>
]


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
@pytest.mark.parametrize("case", _FWD_CASES, ids=[c[0] for c in _FWD_CASES])
def test_forward_replays_clean(case):
    """One replay per prefill kernel family: no fault, race or lane-mask note, and O / LSE
    within the GPU tests' bars of the oracle."""
    from isa_replay.host import Replay
    from tiled_attention_attn_amd import _lib
    name, B, Hq, Hkv, N, D, flags, window, docs, blockmask = case
    rp = Replay(("fwd", "fwd_pp", "blockmask"))
    g = W.generator(len(name))
    q, k, v = (W.randn_bf16(g, s) for s in ((B, Hq, N, D), (B, Hkv, N, D), (B, Hkv, N, D)))
    desc = _lib.attn_mask_desc(flags=flags, window_left=-1, window_right=-1)
    mods = [M.causal(N, N)] if flags & 1 else []
    if window is not None:
        desc.window_left, desc.window_right = window
        mods.append(M.window(window[0], window[1], N, N))
    off = None
    if docs is not None:
        nd = max(len(d) for d in docs)
        rows = [np.concatenate([[0], np.cumsum(d), np.full(nd - len(d), sum(d))]) for d in docs]
        off = torch.tensor(np.stack(rows), dtype=torch.int32)
        desc.doc_offsets, desc.num_docs, desc.doc_stride = off.data_ptr(), nd, off.stride(0)
        mods.append(M.document(docs, N, N))
    mod = M.and_(*mods)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, N), float("nan"))
    rp.register(q=q, k=k, v=v, o=o, lse=lse, doc_offsets=off)
    scale = 1.0 / math.sqrt(D)
    if blockmask:
        nt = (N + 127) // 128
        tm = torch.stack([torch.stack([W.blockmask_tile_map(g, nt, 0.3) for _ in range(Hq)]) for _ in range(B)])
        tm = tm.contiguous()
        lists = [torch.zeros(B, Hq, nt, dtype=torch.int32), torch.zeros(B, Hq, nt, nt, dtype=torch.int32),
                 torch.zeros(B, Hq, nt, dtype=torch.int32), torch.zeros(B, Hq, nt, nt, dtype=torch.int32)]
        rp.register(tm=tm, **{f"lists{i}": t for i, t in enumerate(lists)})
        bm = _lib.attn_blockmask(Bm=B, Hm=Hq, nQt=nt, nKt=nt, part_num=lists[0].data_ptr(),
                                 part_idx=lists[1].data_ptr(), full_num=lists[2].data_ptr(),
                                 full_idx=lists[3].data_ptr())
        assert rp.lib.attn_build_blockmask(None, tm.data_ptr(), B, N, N, ctypes.byref(bm), None) == 0
        st = rp.lib.attn_fwd_blockmask(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(),
                                       _strides(v), o.data_ptr(), _strides(o), lse.data_ptr(), B, Hq, Hkv, N, N, D,
                                       0, scale, ctypes.byref(desc), None, ctypes.byref(bm), None)
        mod = M.blockmask(tm.numpy(), 128, mod)
    else:
        st = rp.lib.attn_fwd(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
                             o.data_ptr(), _strides(o), lse.data_ptr(), B, Hq, Hkv, N, N, D, 0, scale,
                             ctypes.byref(desc), None, None)
    assert st == 0, st
    rp.run()
    assert not rp.notes, rp.notes
    ro, rl = oracle.attention(*(x.to(torch.float64).numpy() for x in (q, k, v)), scale, mod)
    assert_close(o.to(torch.float64).numpy(), lse.numpy(), ro, rl, name)



def _wide_rows(g, B, H, N, D, n_stride):
    """A [B, H, N, D] bf16 tensor whose rows lie n_stride elements apart (heads interleaved
    inside a row): storage of about N * n_stride elements, of which only the logical ones
    are ever written, so the untouched pages cost no memory."""
    t = torch.empty_strided((B, H, N, D), (N * n_stride, D, n_stride, 1), dtype=torch.bfloat16)
    t.copy_(W.randn_bf16(g, (B, H, N, D)))
    return t


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
@pytest.mark.parametrize("D", [64, 128])
def test_largest_row_stride_replays_clean(D):
    """Row strides of 2^24 - 8 elements, the largest the boundary accepts for streamed
    tiles: the copies of a 128-row tile then span almost 2^32 bytes, the limit of the
    kernels' 32-bit tile offsets.  attn_fwd (fwd_kernel at D=64, the ping-pong kernel at
    D=128), attn_fwd_blockmask and attn_bwd (all three kernels; Q and dO with the same
    stride) replay without a fault, race or lane-mask note, within the oracle bars."""
    from isa_replay.host import Replay
    from tiled_attention_attn_amd import _lib
    B, H, N, ns = 1, 2, 200, 2**24 - 8
    g = W.generator(D)
    q, k, v, do = (_wide_rows(g, B, H, N, D, ns) for _ in range(4))
    scale = 1.0 / math.sqrt(D)
    desc = _lib.attn_mask_desc(flags=1, window_left=-1, window_right=-1)
    mod = M.causal(N, N)
    rp = Replay(("fwd", "fwd_pp", "bwd", "blockmask"))
    o = torch.full((B, H, N, D), float("nan"), dtype=torch.bfloat16)
    lse = torch.full((B, H, N), float("nan"))
    rp.register(q=q, k=k, v=v, do=do, o=o, lse=lse)
    assert rp.lib.attn_fwd(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
                           o.data_ptr(), _strides(o), lse.data_ptr(), B, H, H, N, N, D, 0, scale,
                           ctypes.byref(desc), None, None) == 0
    rp.run()
    assert not rp.notes, rp.notes
    f64 = lambda x: x.to(torch.float64).numpy()  # noqa: E731
    ro, rl = oracle.attention(f64(q), f64(k), f64(v), scale, mod)
    assert_close(f64(o), lse.numpy(), ro, rl, f"row stride 2^24 - 8, D={D}")

    # the BlockMask kernel on the same tensors: every tile PARTIAL under the causal predicate
    nt = (N + 127) // 128
    tm = torch.ones(1, 1, nt, nt, dtype=torch.uint8)
    lists = [torch.zeros(1, 1, nt, dtype=torch.int32), torch.zeros(1, 1, nt, nt, dtype=torch.int32),
             torch.zeros(1, 1, nt, dtype=torch.int32), torch.zeros(1, 1, nt, nt, dtype=torch.int32)]
    o_bm = torch.full_like(o, float("nan"))
    lse_bm = torch.full_like(lse, float("nan"))
    rp.register(tm=tm, o_bm=o_bm, lse_bm=lse_bm, **{f"lists{i}": t for i, t in enumerate(lists)})
    bm = _lib.attn_blockmask(Bm=1, Hm=1, nQt=nt, nKt=nt, part_num=lists[0].data_ptr(),
                             part_idx=lists[1].data_ptr(), full_num=lists[2].data_ptr(),
                             full_idx=lists[3].data_ptr())
    assert rp.lib.attn_build_blockmask(None, tm.data_ptr(), B, N, N, ctypes.byref(bm), None) == 0
    assert rp.lib.attn_fwd_blockmask(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(),
                                     _strides(v), o_bm.data_ptr(), _strides(o_bm), lse_bm.data_ptr(), B, H, H, N, N,
                                     D, 0, scale, ctypes.byref(desc), None, ctypes.byref(bm), None) == 0
    rp.run()
    assert not rp.notes, rp.notes
    assert_close(f64(o_bm), lse_bm.numpy(), ro, rl, f"BlockMask, row stride 2^24 - 8, D={D}")

    dq, dk, dv = (torch.full((B, H, N, D), float("nan"), dtype=torch.bfloat16) for _ in range(3))
    ws = torch.zeros(max(int(rp.lib.attn_bwd_workspace_bytes(B, H, N)) // 4, 1))
    rp.register(dq=dq, dk=dk, dv=dv, ws=ws)
    assert rp.lib.attn_bwd(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
                           o.data_ptr(), _strides(o), do.data_ptr(), _strides(do), lse.data_ptr(),
                           dq.data_ptr(), _strides(dq), dk.data_ptr(), _strides(dk), dv.data_ptr(), _strides(dv),
                           B, H, H, N, N, D, 0, scale, ctypes.byref(desc), None, ws.data_ptr(), ws.numel() * 4,
                           None) == 0
    rp.run()
    assert not rp.notes, rp.notes
    rq, rk, rv, (mq, mk, mv) = OBW.attention_bwd(f64(q), f64(k), f64(v), f64(do), scale, mod, row_block=256,
                                                 bound=True, o_used=f64(o))
    _check_grad(dq, rq, mq, "dQ")
    _check_grad(dk, rk, mk, "dK")
    _check_grad(dv, rv, mv, "dV")


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_paged_decode_pool_beyond_4gib_replays_clean():
    """A page pool of 4.6 GB (140000 pages of [16, 8, 128] bf16) whose used pages all lie
    past its first 4 GiB: the decode kernel's page addresses must be 64-bit.  Only the used
    pages are ever written, so the rest of the pool costs no memory.  Split-KV + combine
    replay without a fault, race or lane-mask note, and O / LSE match the oracle's paged
    gather within the GPU tests' bars."""
    from isa_replay.host import Replay
    from oracle import paged as OP
    B, Hq, Hkv, Lq, D, ps, S, P = 2, 16, 8, 4, 128, 16, 3, 140_000
    sl = [300, 170]
    g = W.generator(4)
    per_seq = (max(sl) + ps - 1) // ps
    first = P - 2000                                   # byte offset of page `first` > 2^32
    assert first * ps * Hkv * D * 2 > 2**32
    bt = (first + torch.randperm(2000, generator=g)[: B * per_seq]).reshape(B, per_seq).to(torch.int32)
    q = W.randn_bf16(g, (B, Hq, Lq, D))
    kp = torch.empty((P, ps, Hkv, D), dtype=torch.bfloat16)
    vp = torch.empty((P, ps, Hkv, D), dtype=torch.bfloat16)
    for pool in (kp, vp):
        pool[bt.flatten().long()] = W.randn_bf16(g, (B * per_seq, ps, Hkv, D))
    lens = torch.tensor(sl, dtype=torch.int32)
    ws_o = torch.full((B, Hq, Lq, S, D), float("nan"))
    ws_l = torch.full((B, Hq, Lq, S), float("nan"))
    o = torch.full((B, Hq, Lq, D), float("nan"), dtype=torch.bfloat16)
    lse = torch.full((B, Hq, Lq), float("nan"))
    rp = Replay(("decode",))
    rp.register(q=q, kp=kp, vp=vp, bt=bt, lens=lens, ws_o=ws_o, ws_l=ws_l, o=o, lse=lse)
    scale = 1.0 / math.sqrt(D)
    assert rp.lib.attn_decode_splitkv(q.data_ptr(), _strides(q), kp.data_ptr(), vp.data_ptr(), P, bt.data_ptr(),
                                      bt.stride(0), lens.data_ptr(), per_seq, B, Hq, Hkv, Lq, D, 0, ps, S, scale,
                                      None, None, ws_o.data_ptr(), ws_l.data_ptr(), None) == 0
    assert rp.lib.attn_decode_combine(ws_o.data_ptr(), ws_l.data_ptr(), B, Hq, Lq, S, D, 0, o.data_ptr(),
                                      _strides(o), lse.data_ptr(), None) == 0
    rp.run()
    assert not rp.notes, rp.notes
    used_k = kp[first:].to(torch.float64).numpy()       # the oracle gathers from the used part
    used_v = vp[first:].to(torch.float64).numpy()
    bt_used = (bt - first).numpy()
    for b in range(B):
        kl = OP.gather(used_k, bt_used, b, sl[b])[None]
        vl = OP.gather(used_v, bt_used, b, sl[b])[None]
        ro, rl = oracle.attention(q[b:b + 1].to(torch.float64).numpy(), kl, vl, scale, M.causal(Lq, sl[b]))
        assert_close(o[b:b + 1].to(torch.float64).numpy(), lse[b:b + 1].numpy(), ro, rl, f"sequence {b}")

# SQ counters per dispatch, read with rocprofv3 --pmc on an MI355X for the causal
# 2x16x4096x64 prefill (fwd_kernel<64>) and the paged decode (decode_kernel<128>); both
# dispatches ran 2048 waves.  Values as profiles/sq_counters_causal_b2h16n4096d64_and_decode.md
# lists them, to six or more significant digits.
_SQ_COUNTERS = {
    "prefill": dict(MFMA=2_162_688, VALU=19_935_200, TRANS=4_343_810, LDS=3_244_030),
    "decode": dict(MFMA=8_388_608, VALU=141_860_000, TRANS=4_728_830, LDS=14_712_800),
}
def _compare_with_counters(which, counts, waves):
    from isa_replay.mix import classes  # MFMAs count as VALU too; TRANS: the f32 transcendentals
    hw = _SQ_COUNTERS[which]
    got = classes(counts)
    for c in ("MFMA", "TRANS", "LDS"):
        # equal, to the listed digits
        assert abs(got[c] / waves - hw[c] / 2048) <= 0.05, f"{which} {c}: {got[c] / waves} vs {hw[c] / 2048} a wave"
    # the prefill's VALU count is equal to the listed digits too; the decode's is 1.9 a wave
    # (0.003%) above the listed count, a difference not traced to an instruction
    assert abs(got["VALU"] / waves / (hw["VALU"] / 2048) - 1) <= 1e-4, f"{which} VALU: {got['VALU'] / waves}"


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_replay_instruction_counts_match_hardware_counters():
    """The replay executes the instructions the GPU executed: per wave, its MFMA, VALU,
    transcendental and LDS instruction counts over sampled work groups of the causal
    2x16x4096x64 prefill (every work group runs 33 key steps) and of one (sequence, KV
    head) row of the paged decode (all four splits; every row holds 32768 keys) agree with
    the hardware counters of the full dispatches.  A wrong branch or loop trip in the replay
    would move them.  The kernels are those the counters were read on; a kernel change
    that moves these counts fails here until the counters are read again."""
    from isa_replay.host import Replay
    from tiled_attention_attn_amd import _lib
    wl = W.causal_b2h16n4096d64()
    q, k, v = (wl.tensors[x] for x in ("q", "k", "v"))
    B, H, N, D = q.shape
    rp = Replay(("fwd",))
    o, lse = torch.zeros_like(q), torch.zeros(B, H, N)
    rp.register(q=q, k=k, v=v, o=o, lse=lse)
    desc = _lib.attn_mask_desc(flags=1, window_left=-1, window_right=-1)
    assert rp.lib.attn_fwd(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
                           o.data_ptr(), _strides(o), lse.data_ptr(), B, H, H, N, N, D, 0, wl.scale,
                           ctypes.byref(desc), None, None) == 0
    (L,) = rp.recorded()
    assert L["grid"] == (512, 1, 1) and L["block"] == (256, 1, 1)
    groups = [0, 333]
    m = rp.run_launch(L, groups)
    assert not m.notes, m.notes
    _compare_with_counters("prefill", m.op_counts(), len(groups) * 4)

    d = W.decode_b16h32kv8q16k32768d128()
    t = d.tensors
    q, kp, vp, bt, sl = t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"]
    B, Hq, Lq, D = q.shape
    Hkv = kp.shape[2]
    rp = Replay(("decode",))
    S = int(rp.lib.attn_decode_num_splits(B, Hkv, bt.shape[1], 256))
    ws_o, ws_l = torch.zeros(B, Hq, Lq, S, D), torch.zeros(B, Hq, Lq, S)
    rp.register(q=q, kp=kp, vp=vp, bt=bt, sl=sl, ws_o=ws_o, ws_l=ws_l)
    assert rp.lib.attn_decode_splitkv(q.data_ptr(), _strides(q), kp.data_ptr(), vp.data_ptr(), kp.shape[0],
                                      bt.data_ptr(), bt.stride(0), sl.data_ptr(), bt.shape[1], B, Hq, Hkv, Lq, D,
                                      0, kp.shape[1], S, d.scale, None, None, ws_o.data_ptr(), ws_l.data_ptr(),
                                      None) == 0
    (L,) = rp.recorded()
    assert L["grid"] == (S, Hkv, B) and L["block"] == (256, 1, 1)
    m = rp.run_launch(L, list(range(S)))  # the splits of sequence 0, KV head 0
    assert not m.notes, m.notes
    _compare_with_counters("decode", m.op_counts(), S * 4)


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_no_kernel_branches_on_a_lane_mask_from_a_lane_by_lane_loop():
    """Every kernel of the library, statically: no compare made inside a loop whose lanes
    leave one by one has its lane mask used with EXEC after that loop (the row-search
    defect, which this check finds at 12 sites in the unfixed dK/dV kernels)."""
    import glob
    from isa_replay.host import Kernels, build
    from isa_replay.static_checks import lane_mask_reuse_sites
    from tiled_attention_attn_amd import build as B
    names = tuple(os.path.basename(p)[:-4] for p in sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
                  if not p.endswith("attn_api.hip"))
    _, asm = build(names)
    kernels = Kernels(list(asm.values()))
    assert len(kernels.where) > 60
    found = {n: lane_mask_reuse_sites(p, n) for n, p in kernels.where.items()}
    assert not any(found.values()), {n: s for n, s in found.items() if s}



# Scratch bytes a lane may spill, per kernel family with a score change (SM): the only
# variants whose registers overflow at their two-waves-per-SIMD budget.  Every other kernel
# must not spill.
_SPILL_LIMITS = {
    ("fwd_kernel<64,", True): 140,
    ("bwd_kv_kernel<64,", True): 224,
    ("bwd_q_kernel<128,", True): 24,
}


@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_every_kernel_keeps_the_lds_rule_and_the_recorded_spills():
    """From the compiled kernel descriptors of every kernel: no work group uses more than
    72 KB of LDS (two groups per CU, and the footprint rule of every kernel's LDS
    declaration), and only the score-change variants listed above spill, by at most the
    listed bytes.  A kernel change that starts a new spill, or grows one, fails here."""
    import glob
    from isa_replay.host import Kernels, build
    from isa_replay.mix import demangle
    from tiled_attention_attn_amd import build as B
    names = tuple(os.path.basename(p)[:-4] for p in sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))
                  if not p.endswith("attn_api.hip"))
    _, asm = build(names)
    kernels = Kernels(list(asm.values()))
    assert len(kernels.desc) > 60
    for name, d in kernels.desc.items():
        k = demangle(name)
        assert d["group_segment_fixed_size"] <= 72 * 1024, (k, d["group_segment_fixed_size"])
        # the SM template argument is the third of fwd_kernel / bwd_*_kernel and the last of decode
        args = [a.strip() for a in k[k.find("<") + 1:k.rfind(">")].split(",")] if "<" in k else []
        sm = len(args) >= 3 and args[2] == "true" if k.startswith(("bwd_kv", "bwd_q")) else (
            len(args) >= 4 and args[3] == "true" if k.startswith("fwd_kernel") else False)
        limit = next((v for (pre, s_), v in _SPILL_LIMITS.items() if k.startswith(pre) and s_ == sm), 0)
        assert d["private_segment_fixed_size"] <= limit, (k, d["private_segment_fixed_size"], limit)

_LOOP_ASM = """\
probe:
\ts_mov_b64 s[8:9], 0
.LBB0_1:                                ; =>This Loop Header: Depth=1
\tv_cmp_ne_u32_e64 s[6:7], 1, v1
\tv_add_u32_e32 v2, 1, v2
\tv_cmp_ge_u32_e32 vcc, v2, v0
\ts_or_b64 s[8:9], vcc, s[8:9]
\t{exit}
\ts_cbranch_execnz .LBB0_1
; %bb.2:
\ts_or_b64 exec, exec, s[8:9]
\ts_and_b64 vcc, exec, s[6:7]
\ts_cbranch_vccnz .LBB0_3
.LBB0_3:
\ts_endpgm
.Lfunc_end0:
"""


def test_static_check_flags_only_lane_by_lane_loops():
    from isa_replay.static_checks import lane_mask_reuse_sites
    for exit_idiom, expected in (("s_andn2_b64 exec, exec, s[8:9]", 1), ("s_and_b64 s[10:11], exec, s[8:9]", 0)):
        with tempfile.NamedTemporaryFile("w", suffix=".s", delete=False) as fh:
            fh.write(_LOOP_ASM.format(exit=exit_idiom))
        try:
            sites = lane_mask_reuse_sites(fh.name, "probe")
        finally:
            os.unlink(fh.name)
        assert len(sites) == expected, (exit_idiom, sites)


# ---- pins of the replay's own checks, on hand-written assembly ----------------------
_ASM = """\
probe:
\ts_load_dwordx2 s[4:5], s[0:1], 0x0
\tv_cmp_gt_u32_e64 s[6:7], 8, v0
\ts_and_saveexec_b64 s[8:9], s[6:7]
\tv_cmp_ne_u32_e64 s[10:11], 1, v0
\ts_or_b64 exec, exec, s[8:9]
\ts_and_b64 vcc, exec, s[10:11]
\ts_waitcnt lgkmcnt(0)
\tv_mov_b32_e32 v1, s4
\tv_mov_b32_e32 v2, s5
\tv_lshlrev_b32_e32 v3, 2, v0
\tv_add_co_u32_e32 v1, vcc, v1, v3
\tv_addc_co_u32_e32 v2, vcc, 0, v2, vcc
\tglobal_load_dword v4, v[1:2], off
\t{use}
\ts_endpgm
.Lfunc_end0:
"""


def _probe(use, n_words):
    from isa_replay import emulator as E
    mem = E.Memory()
    data = np.arange(n_words, dtype=np.uint32)
    buf_addr = mem.alloc(data.tobytes(), "buffer")
    ka = mem.alloc(np.array([buf_addr], dtype=np.uint64).tobytes(), "kernarg")
    with tempfile.NamedTemporaryFile("w", suffix=".s", delete=False) as fh:
        fh.write(_ASM.format(use=use))
    try:
        m = E.Machine(fh.name, "probe", mem, ka, 0, 64)
        m.run_group((0, 0, 0), [0])
    finally:
        os.unlink(fh.name)
    return m


def test_replay_flags_a_lane_mask_used_under_a_wider_exec():
    """A mask made under EXEC = lanes 0..7 and tested under all 64 lanes is reported."""
    m = _probe("s_waitcnt vmcnt(0)", 64)
    assert len(m.notes) == 1 and "lane mask" in m.notes[0] and "00000000000000ff" in m.notes[0]


def test_replay_flags_out_of_bounds_and_unwaited_loads():
    from isa_replay import emulator as E
    with pytest.raises(E.Fault, match="outside every allocation"):
        _probe("s_waitcnt vmcnt(0)", 63)          # lane 63 reads one word past the buffer
    with pytest.raises(E.Hazard, match="outstanding"):
        _probe("v_mov_b32_e32 v5, v4", 64)        # uses the load's register before its wait



_DMA_ASM = """\
probe:
\ts_load_dwordx2 s[4:5], s[0:1], 0x0
\tv_lshlrev_b32_e32 v1, 4, v0
\ts_mov_b32 m0, {m0}
\ts_waitcnt lgkmcnt(0)
\ts_nop 0
\tglobal_load_lds_dwordx4 v1, s[4:5]
\ts_waitcnt vmcnt(0)
\ts_endpgm
.Lfunc_end0:
"""


def test_replay_flags_lds_copies_above_64_kib():
    """The replay enforces the LDS copy rule: one wave's 1 KB LDS-DMA copy ending at the
    64 KB mark runs, the same copy starting there is a fault (in a 128 KB allocation, so
    only the rule, not the bounds check, can object)."""
    from isa_replay import emulator as E

    def run(m0):
        mem = E.Memory()
        buf = mem.alloc(np.arange(256, dtype=np.uint32).tobytes(), "buffer")
        ka = mem.alloc(np.array([buf], dtype=np.uint64).tobytes(), "kernarg")
        with tempfile.NamedTemporaryFile("w", suffix=".s", delete=False) as fh:
            fh.write(_DMA_ASM.format(m0=hex(m0)))
        try:
            m = E.Machine(fh.name, "probe", mem, ka, 128 * 1024, 64)
            m.run_group((0, 0, 0), [0])
        finally:
            os.unlink(fh.name)

    run(0x10000 - 1024)
    with pytest.raises(E.Fault, match="copies below"):
        run(0x10000)



@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_gpu_address_limit_tests_dry_run_on_the_cpu():
    """tests/test_gpu_large_addresses.py, the GPU tests themselves, run on the CPU through
    isa_replay.dryrun: the binding's calls reach the compiled kernels' replay, and every
    comparison of the test file passes (row stride 2^24 - 8 forward, BlockMask and
    backward at D=64 and 128; paged decode over a 4.6 GB pool)."""
    import subprocess
    import sys
    env = dict(os.environ, PYTHONPATH=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    r = subprocess.run([sys.executable, "-m", "isa_replay.dryrun", "test_gpu_large_addresses",
                        "test_largest_row_stride_forward", "test_largest_row_stride_backward",
                        "test_paged_decode_pool_beyond_4gib"],
                       cwd=os.path.dirname(os.path.abspath(__file__)), env=env, capture_output=True, text=True,
                       timeout=1200)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert r.stdout.count("dry run passed") == 5, r.stdout



@pytest.mark.skipif(not HAVE_HIPCC, reason="needs hipcc to compile the kernels' assembly")
def test_score_change_backward_that_faulted_dry_runs_on_the_cpu():
    """test_gpu_score_mod.py::test_backward_score_mod[alibi_sym_window_d64], the GPU case
    that faulted before the dK/dV row-search fix, run as written on the CPU through
    isa_replay.dryrun: attn_fwd then attn_bwd with symmetric ALiBi and a bias table at
    D=64, every gradient within the test's bar (scratch filled with 0x7F)."""
    import subprocess
    import sys
    env = dict(os.environ, PYTHONPATH=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    r = subprocess.run([sys.executable, "-m", "isa_replay.dryrun", "test_gpu_score_mod",
                        "test_backward_score_mod[2]"],
                       cwd=os.path.dirname(os.path.abspath(__file__)), env=env, capture_output=True, text=True,
                       timeout=1200)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "dry run passed: test_gpu_score_mod::test_backward_score_mod[alibi_sym_window_d64]" in r.stdout, r.stdout
