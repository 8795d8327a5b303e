"""Per-wave instruction mix of the library's kernels on the benchmark workloads, counted
by the CPU replay of their compiled code.

Every benchmark mask is the same for every head, so one head carries a dispatch's whole
per-head work: the replay runs each call on head 0 of the workload's own tensors (for the
GQA workload: KV head 0 and its four query heads), through the library's host code, and
runs every work group of every launch (the paged decode, whose rows all hold 32768 keys:
the splits of one row).  Per-wave means are then those of the full
dispatch, except for a few scalar instructions of the work-group numbering and for
branches that depend on the data.  The backward calls take O and the LSE from the
replayed forward call and the upstream gradient the benchmark draws.

The replay's instruction counts agree with the SQ counters of two dispatches
(tests/test_isa_replay.py, test_replay_instruction_counts_match_hardware_counters).  They
count instructions, not cycles: they say how much VALU work a kernel issues per MFMA, not
how well the two overlap.

Usage, from tests/:  python -m isa_replay.mix [workload ...]   (all five by default: the
forward calls of the prefill benchmarks, the backward calls of the causal and the
block-diffusion one, and the paged decode; the block-diffusion call and the BlockMask
prefill take about an hour each)
"""
from __future__ import annotations

import ctypes
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

from .host import Replay  # noqa: E402

# flops of one MFMA instruction (2 * M * N * K)
MFMA_FLOP = {"v_mfma_f32_32x32x16_bf16": 32768, "v_mfma_f32_32x32x16_f16": 32768,
             "v_mfma_f32_16x16x32_bf16": 16384, "v_mfma_f32_16x16x32_f16": 16384}
TRANS = ("v_exp_f32", "v_log_f32", "v_rcp_f32", "v_rcp_iflag_f32", "v_rsq_f32", "v_sqrt_f32", "v_sin_f32",
         "v_cos_f32")
FLAG_CAUSAL, FLAG_WINDOW, FLAG_DOCUMENT, FLAG_BLOCK = 1, 2, 4, 8


def _s3(t):
    return (ctypes.c_int64 * 3)(*t.stride()[:3])


def classes(counts):
    """Mnemonic counts -> instruction classes (MFMAs are VALU instructions too)."""
    c = dict(MFMA=0, mfma_flop=0, VALU=0, TRANS=0, LDS=0, VMEM=0, SMEM=0, SALU=0, waitcnt=0, branch=0, total=0)
    for op, n in counts.items():
        c["total"] += n
        if op.startswith("v_"):
            c["VALU"] += n
            if op.startswith("v_mfma"):
                c["MFMA"] += n
                c["mfma_flop"] += n * MFMA_FLOP[op]
            c["TRANS"] += n * op.startswith(TRANS)
        elif op.startswith("ds_"):
            c["LDS"] += n
        elif op.startswith(("global_", "buffer_")):
            c["VMEM"] += n
        elif op.startswith(("s_load", "s_buffer_load")):
            c["SMEM"] += n
        elif op.startswith("s_waitcnt"):
            c["waitcnt"] += n
        elif op.startswith(("s_cbranch", "s_branch")):
            c["branch"] += n
        elif op.startswith("s_") and not op.startswith(("s_barrier", "s_endpgm", "s_nop", "s_setprio", "s_sleep")):
            c["SALU"] += n
    return c


class _Run:
    def __init__(self, sources):
        self.rp = Replay(sources)
        self.rows = []

    def launches(self, label, heads_in_dispatch, groups=None):
        """Runs the launches recorded since the last call: every work group, or those
        ``groups(launch)`` names (work groups that stand for the whole grid)."""
        for L in self.rp.recorded():
            t0 = time.time()
            ids = groups(L) if groups else None
            m = self.rp.run_launch(L, ids)
            if m.notes:
                raise RuntimeError(f"{L['name']}: {m.notes}")
            n_groups = L["grid"][0] * L["grid"][1] * L["grid"][2]
            per_group = (L["block"][0] + 63) // 64
            waves = (len(ids) if ids is not None else n_groups) * per_group
            row = dict(label=label, kernel=L["name"], grid=L["grid"], waves=waves,
                       scale=heads_in_dispatch * n_groups * per_group / waves,
                       seconds=time.time() - t0, **classes(m.op_counts()))
            self.rows.append(row)
            print(format_row(row), flush=True)


def format_row(r):
    w = r["waves"]
    per = lambda k: r[k] / w  # noqa: E731
    ratio = f"{(r['VALU'] - r['MFMA']) / r['MFMA']:.2f}" if r["MFMA"] else "-"
    return (f"| {r['label']} | `{demangle(r['kernel'])}` | {r['grid'][0]}x{r['grid'][1]}x{r['grid'][2]} "
            f"| {w} | {per('MFMA'):.1f} | {per('VALU') - per('MFMA'):.1f} | {ratio} | {per('TRANS'):.1f} "
            f"| {per('LDS'):.1f} | {per('VMEM'):.1f} | {per('SALU'):.1f} | {per('total'):.1f} "
            f"| {r['mfma_flop'] * r['scale'] / 1e9:.2f} |")


def demangle(name):
    """Kernel name without namespaces and parameters (the 16-bit float types written as
    vendor types first: GNU c++filt does not know their mangling)."""
    import subprocess
    plain = name.replace("DF16b", "u4bf16").replace("DF16_", "u3f16")
    out = subprocess.run(["c++filt", plain], capture_output=True, text=True).stdout.strip() or name
    out = out.replace("tattn::", "").replace("(anonymous namespace)::", "").split("(")[0]
    return out[5:] if out.startswith("void ") else out


HEADER = ("| call | kernel | grid of the replayed call | waves replayed | MFMA a wave | other VALU a wave | other VALU per MFMA "
          "| f32 transcendental a wave | LDS a wave | global memory a wave | scalar ALU a wave "
          "| all instructions a wave | MFMA GFLOP, whole dispatch |\n"
          "|---|---|---|---|---|---|---|---|---|---|---|---|---|")


def _fwd(run, q, k, v, scale, desc, Hkv):
    B, Hq, N, D = q.shape
    o, lse = torch.zeros_like(q), torch.zeros(B, Hq, N)
    run.rp.register(q=q, k=k, v=v, o=o, lse=lse)
    st = run.rp.lib.attn_fwd(q.data_ptr(), _s3(q), k.data_ptr(), _s3(k), v.data_ptr(), _s3(v), o.data_ptr(),
                             _s3(o), lse.data_ptr(), B, Hq, Hkv, N, N, D, 0, scale, ctypes.byref(desc), None, None)
    assert st == 0, st
    return o, lse


def _bwd(run, q, k, v, o, lse, do, scale, desc):
    B, H, N, D = q.shape
    dq, dk, dv = (torch.zeros_like(x) for x in (q, k, v))
    ws = torch.zeros(max(int(run.rp.lib.attn_bwd_workspace_bytes(B, H, N)) // 4, 1))
    run.rp.register(do=do, dq=dq, dk=dk, dv=dv, ws=ws)
    st = run.rp.lib.attn_bwd(q.data_ptr(), _s3(q), k.data_ptr(), _s3(k), v.data_ptr(), _s3(v), o.data_ptr(),
                             _s3(o), do.data_ptr(), _s3(do), lse.data_ptr(), dq.data_ptr(), _s3(dq),
                             dk.data_ptr(), _s3(dk), dv.data_ptr(), _s3(dv), B, H, H, N, N, D, 0, scale,
                             ctypes.byref(desc), None, ws.data_ptr(), ws.numel() * 4, None)
    assert st == 0, st


def _head0(wl):
    return [wl.tensors[x][:, :1].contiguous() for x in ("q", "k", "v")]


def _desc(**kw):
    from tiled_attention_attn_amd import _lib
    d = _lib.attn_mask_desc(flags=0, window_left=-1, window_right=-1)
    for key, val in kw.items():
        setattr(d, key, val)
    return d


def _dense_desc(wl):
    m = wl.mask
    if m.get("causal"):
        return _desc(flags=FLAG_CAUSAL), None
    if m.get("block_size"):
        return _desc(flags=FLAG_BLOCK, block_size=int(m["block_size"])), None
    starts = np.concatenate([[0], np.cumsum(m["doc_lengths"][0])]).astype(np.int32)
    off = torch.tensor(starts, dtype=torch.int32)[None].contiguous()
    d = _desc(flags=FLAG_WINDOW | FLAG_DOCUMENT, window_left=int(m["window"]), window_right=int(m["window"]),
              doc_offsets=off.data_ptr(), num_docs=len(starts) - 1, doc_stride=off.stride(0))
    return d, off


def dense_prefill(name, backward=False):
    wl = W.FULL_SIZE[name]()
    H = wl.Hq
    run = _Run(("fwd", "fwd_pp", "bwd"))
    q, k, v = _head0(wl)
    desc, off = _dense_desc(wl)
    run.rp.register(doc_offsets=off)
    o, lse = _fwd(run, q, k, v, wl.scale, desc, 1)
    run.launches(name, H)
    if backward:
        # the upstream gradient bench.py draws for its backward calls
        do = W.randn_bf16(W.generator(77), tuple(wl.tensors["q"].shape))[:, :1].contiguous()
        _bwd(run, q, k, v, o, lse, do, wl.scale, desc)
        run.launches(name + " backward", H)
    return run.rows


def blockmask_prefill(name="blockmask_gqa_b1h32kv8n32768d128"):
    from tiled_attention_attn_amd import _lib
    wl = W.blockmask_gqa_b1h32kv8n32768d128()
    G = wl.Hq // wl.Hkv
    q = wl.tensors["q"][:, :G].contiguous()
    k, v = (wl.tensors[x][:, :1].contiguous() for x in ("k", "v"))
    B, Hq, N, D = q.shape
    run = _Run(("fwd", "blockmask"))
    tm = wl.mask["tile_map"][None, None].contiguous()
    nt = tm.shape[-1]
    lists = [torch.zeros(1, 1, nt, dtype=torch.int32), torch.zeros(1, 1, nt, nt, dtype=torch.int32),
             torch.zeros(1, 1, nt, dtype=torch.int32), torch.zeros(1, 1, nt, nt, dtype=torch.int32)]
    run.rp.register(tm=tm, **{f"lists{i}": t for i, t in enumerate(lists)})
    bm = _lib.attn_blockmask(Bm=1, Hm=1, nQt=nt, nKt=nt, part_num=lists[0].data_ptr(), part_idx=lists[1].data_ptr(),
                             full_num=lists[2].data_ptr(), full_idx=lists[3].data_ptr())
    assert run.rp.lib.attn_build_blockmask(None, tm.data_ptr(), 1, N, N, ctypes.byref(bm), None) == 0
    run.launches(name + " (list build)", 1)
    o, lse = torch.zeros_like(q), torch.zeros(B, Hq, N)
    run.rp.register(q=q, k=k, v=v, o=o, lse=lse)
    desc = _desc(flags=FLAG_CAUSAL)
    st = run.rp.lib.attn_fwd_blockmask(q.data_ptr(), _s3(q), k.data_ptr(), _s3(k), v.data_ptr(), _s3(v),
                                       o.data_ptr(), _s3(o), lse.data_ptr(), B, Hq, 1, N, N, D, 0, wl.scale,
                                       ctypes.byref(desc), None, ctypes.byref(bm), None)
    assert st == 0, st
    run.launches(name, wl.Hkv)
    return run.rows


def paged_decode(name="decode_b16h32kv8q16k32768d128"):
    """Split-KV + combine.  Every (sequence, KV head) row holds 32768 keys, so the splits of
    row 0 stand for the split-KV grid; the combine runs whole."""
    wl = W.decode_b16h32kv8q16k32768d128()
    t = wl.tensors
    q, kp, vp, bt, sl = t["q"], t["k_pool"], t["v_pool"], t["block_table"], t["seq_lens"]
    B, Hq, Lq, D = q.shape
    Hkv = kp.shape[2]
    run = _Run(("decode",))
    S = int(run.rp.lib.attn_decode_num_splits(B, Hkv, bt.shape[1], 256))
    ws_o, ws_l = torch.zeros(B, Hq, Lq, S, D), torch.zeros(B, Hq, Lq, S)
    o, lse = torch.zeros(B, Hq, Lq, D, dtype=q.dtype), torch.zeros(B, Hq, Lq)
    run.rp.register(q=q, kp=kp, vp=vp, bt=bt, sl=sl, ws_o=ws_o, ws_l=ws_l, o=o, lse=lse)
    st = run.rp.lib.attn_decode_splitkv(q.data_ptr(), _s3(q), kp.data_ptr(), vp.data_ptr(), kp.shape[0],
                                        bt.data_ptr(), bt.stride(0), sl.data_ptr(), bt.shape[1], B, Hq, Hkv, Lq,
                                        D, 0, kp.shape[1], S, wl.scale, None, None, ws_o.data_ptr(),
                                        ws_l.data_ptr(), None)
    assert st == 0, st
    st = run.rp.lib.attn_decode_combine(ws_o.data_ptr(), ws_l.data_ptr(), B, Hq, Lq, S, D, 0, o.data_ptr(),
                                        _s3(o), lse.data_ptr(), None)
    assert st == 0, st
    run.launches(name, 1, groups=lambda L: list(range(S)) if "decode_kernel" in L["name"] else None)
    return run.rows


CALLS = {
    "causal_b2h16n4096d64": lambda: dense_prefill("causal_b2h16n4096d64", backward=True),
    "window_doc_b1h32n8192d128": lambda: dense_prefill("window_doc_b1h32n8192d128"),
    "blockdiff_b1h32n8192d128": lambda: dense_prefill("blockdiff_b1h32n8192d128", backward=True),
    "blockmask_gqa_b1h32kv8n32768d128": blockmask_prefill,
    "decode_b16h32kv8q16k32768d128": paged_decode,
}


def main(argv):
    names = argv or list(CALLS)
    print(HEADER, flush=True)
    for n in names:
        CALLS[n]()


if __name__ == "__main__":
    main(sys.argv[1:])
