"""Benchmark of the fused attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--quick]

Headline: causal prefill B=2 H=16 N=4096 D=64 (bf16 in, fp32 accumulate),
useful (unmasked) TFLOP/s = 4 * D * (#visible (q, k) pairs) / kernel time, as a
fraction of the MI355X dense bf16 MFMA peak (2.5 PFLOP/s).  The same run also
times, each on its own seeded synthetic inputs with inputs resident in HBM:

* decode: split-KV paged decode B=16 Hq=32 Hkv=8, 16 queries over 32768 keys,
  D=128, 16-token pages (splitkv + combine), KV-read GB/s = B*Hkv*Nk*D*2 bytes
  * 2 (K and V) / time, as a fraction of the 8 TB/s HBM peak; and the same
  keys in contiguous K/V through attn_fwd_auto (split-KV chosen by shape)
  against attn_fwd's prefill kernels on that call;
* the other prefill workloads (window+document and block-diffusion at
  B=1 H=32 N=8192 D=128, block-sparse GQA at N=32768), in TFLOP/s;
* the backward pass (attn_bwd: dQ, dK, dV) on the causal headline shape and
  on block-diffusion N=8192 D=128, in useful TFLOP/s (2.5x the forward's
  FLOP: the five products S, dP, dV, dK, dQ).

Each kernel is timed with HIP events recorded on the stream it is launched on
(torch's current stream, which the binding passes to the library) around K
back-to-back launches after W warm-up launches, bracketed by synchronisation;
the per-launch figure is that time / K.  The CPU
baseline is the fp64 oracle timed on this host's cores over a bounded sample
of the headline workload.  One JSON line is printed on stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(key):
    """HBM bytes per launch recorded in profiles/traffic.json for `key`, or None when
    the kernel's sources changed since those counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        ent = json.load(open(path))["kernels"][key]
    except (OSError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in ent["sources"]:
        with open(os.path.join(ROOT, "tiled_attention_attn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return ent["hbm_bytes_per_launch"] if h.hexdigest()[:16] == ent["source_sha256_16"] else None


def time_launches(fn, steps, warmup):
    """Kernel time per launch (ms): HIP events recorded on the current stream
    (the stream the binding launches on) around `steps` back-to-back launches,
    divided by `steps`; plus the shortest single launch of a second, event-
    bracketed pass (informational), and the wall time of the timed region."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    outer0 = torch.cuda.Event(enable_timing=True)
    outer1 = torch.cuda.Event(enable_timing=True)
    outer0.record(stream)
    for _ in range(steps):
        fn()
    outer1.record(stream)
    torch.cuda.synchronize()
    wall = outer0.elapsed_time(outer1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(steps, 10))]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    best = min(a.elapsed_time(b) for a, b in ev)
    return wall / steps, best, wall


def causal_pairs(N):
    return N * (N + 1) // 2


def visible_pairs_dense(lo, hi):
    import numpy as np
    return int(np.maximum(hi - lo + 1, 0).sum())


def bench_prefill_causal(T, W, steps, warmup):
    import torch
    wl = W.causal_b2h16n4096d64()
    q, k, v = (wl.tensors[x].cuda() for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty(2, 16, 4096, dtype=torch.float32, device="cuda")
    mask = T.Mask(causal=True)
    desc = mask.desc()
    fn = lambda: T.attn_fwd(q, k, v, o, lse, wl.scale, desc)
    avg, best, wall = time_launches(fn, steps, warmup)
    flops = 4.0 * 64 * 2 * 16 * causal_pairs(4096)
    # Executed work: each 128-row query tile t runs t + 1 steps of 128 keys in full
    # (the diagonal step's masked half included).
    executed = 4.0 * 64 * 2 * 16 * sum((t + 1) * 128 * 128 for t in range(4096 // 128))
    return wl, dict(avg_ms=avg, min_ms=best, wall_ms=wall, flops=flops, executed_flops=executed)


def bench_prefill_others(T, W, steps, warmup):
    import numpy as np
    import torch
    out = []
    # window + document and block-diffusion, B=1 H=32 N=8192 D=128
    for name in ("window_doc_b1h32n8192d128", "blockdiff_b1h32n8192d128"):
        wl = W.FULL_SIZE[name]()
        q, k, v = (wl.tensors[x].cuda() for x in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty(1, 32, 8192, dtype=torch.float32, device="cuda")
        N = 8192
        p = np.arange(N)
        if name.startswith("window"):
            lens = wl.mask["doc_lengths"][0]
            starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            off = torch.tensor(starts, dtype=torch.int32, device="cuda")[None]
            mask = T.Mask(window=(512, 512), doc_offsets=off)
            d = np.searchsorted(starts, p, side="right") - 1
            lo = np.maximum(p - 512, starts[d])
            hi = np.minimum(p + 512, starts[d + 1] - 1)
        else:
            mask = T.Mask(block_size=16)
            lo = np.zeros(N, dtype=np.int64)
            hi = np.minimum((p // 16 + 1) * 16 - 1, N - 1)
        desc = mask.desc()
        fn = lambda: T.attn_fwd(q, k, v, o, lse, wl.scale, desc)
        avg, best, wall = time_launches(fn, steps, warmup)
        flops = 4.0 * 128 * 32 * visible_pairs_dense(lo, hi)
        out.append(dict(workload=name, avg_ms=avg, min_ms=best, tflops=flops / avg / 1e9,
                        frac=flops / avg / 1e9 / PEAK_BF16_TFLOPS))
        del q, k, v, o, lse
    # block-sparse GQA, N=32768
    wl = W.blockmask_gqa_b1h32kv8n32768d128()
    q, k, v = (wl.tensors[x].cuda() for x in ("q", "k", "v"))
    N = 32768
    o = torch.empty_like(q)
    lse = torch.empty(1, 32, N, dtype=torch.float32, device="cuda")
    tm = wl.mask["tile_map"]
    bm = T.BlockMask(1, 1, N, N)
    tmg = tm[None, None].contiguous().cuda()
    build = lambda: T.attn_build_blockmask(bm, 1, N, N, tile_map=tmg)
    b_avg, _, _ = time_launches(build, steps, warmup)
    desc = T.Mask(causal=True).desc()
    fn = lambda: T.attn_fwd_blockmask(q, k, v, o, bm, lse, wl.scale, desc)
    avg, best, wall = time_launches(fn, steps, warmup)
    n_full = int((tm == W.TILE_FULL).sum())
    n_diag = int((tm == W.TILE_PARTIAL).sum())
    pairs = n_full * 128 * 128 + n_diag * (128 * 129 // 2)
    flops = 4.0 * 128 * 32 * pairs
    out.append(dict(workload=wl.name, avg_ms=avg, min_ms=best, tflops=flops / avg / 1e9,
                    frac=flops / avg / 1e9 / PEAK_BF16_TFLOPS, blockmask_build_ms=b_avg))
    return out


def bench_decode(T, W, steps, warmup):
    import torch
    wl = W.decode_b16h32kv8q16k32768d128()
    t = wl.tensors
    B, Hq, Hkv, Lq, Nk, D = 16, 32, 8, 16, 32768, 128
    q = t["q"].cuda()
    kp, vp = t["k_pool"].cuda(), t["v_pool"].cuda()
    bt, sl = t["block_table"].cuda(), t["seq_lens"].cuda()
    del wl, t
    S = T.attn_decode_num_splits(B, Hkv, 2048)
    ws_o = torch.empty(B, Hq, Lq, S, D, dtype=torch.float32, device="cuda")
    ws_l = torch.empty(B, Hq, Lq, S, dtype=torch.float32, device="cuda")
    o = torch.empty(B, Hq, Lq, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, Hq, Lq, dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(D)

    def split():
        T.attn_decode_splitkv(q, kp, vp, bt, sl, 2048, S, ws_o, ws_l, scale)

    def comb():
        T.attn_decode_combine(ws_o, ws_l, o, lse)

    def both():
        split()
        comb()
    s_avg, s_min, _ = time_launches(split, steps, warmup)
    c_avg, _, _ = time_launches(comb, steps, warmup)
    avg, best, wall = time_launches(both, steps, warmup)
    kv_bytes = float(B * Hkv * Nk * D * 2 * 2)
    # The same keys gathered into contiguous [B, Hkv, Nk, D] K/V: attn_fwd_auto (split-KV +
    # combine, chosen by shape) against attn_fwd (the prefill kernels) on that call.
    j = torch.arange(Nk, device="cuda")
    page, slot = bt[:, j // 16].long(), (j % 16)[None]
    kc = kp[page, slot].permute(0, 2, 1, 3).contiguous()
    vc = vp[page, slot].permute(0, 2, 1, 3).contiguous()
    del kp, vp, page
    plan = T.attn_fwd_auto_plan(B, Hq, Hkv, Lq, Nk, D)
    ws = torch.empty(plan.workspace_bytes // 4, dtype=torch.float32, device="cuda")
    cm = T.Mask(causal=True).desc()
    a_avg, a_min, _ = time_launches(lambda: T.attn_fwd_auto(q, kc, vc, o, lse, scale, cm, ws), steps,
                                    warmup)
    p_avg, _, _ = time_launches(lambda: T.attn_fwd(q, kc, vc, o, lse, scale, cm), steps, warmup)
    return dict(avg_ms=avg, min_ms=best, wall_ms=wall, splitkv_ms=s_avg, splitkv_min_ms=s_min,
                combine_ms=c_avg, splits=S, kv_bytes=kv_bytes, auto_ms=a_avg, auto_min_ms=a_min,
                auto_path=int(plan.path), auto_splits=int(plan.num_splits), auto_prefill_ms=p_avg)


def bench_backward(T, W, steps, warmup):
    """attn_bwd (three kernels) on the causal 2x16x4096x64 workload and on block-diffusion
    1x32x8192x128; upstream gradient dO is seeded N(0,1) bf16.  Useful FLOP = 2.5x the forward's
    4 D (#visible pairs): the five products S, dP, dV, dK, dQ of 2 D per pair each."""
    import numpy as np
    import torch
    out = []
    for name in ("causal_b2h16n4096d64", "blockdiff_b1h32n8192d128"):
        wl = W.FULL_SIZE[name]()
        q, k, v = (wl.tensors[x].cuda() for x in ("q", "k", "v"))
        B, H, N, D = q.shape
        g = W.generator(77)
        do = W.randn_bf16(g, tuple(q.shape)).cuda()
        o = torch.empty_like(q)
        lse = torch.empty(B, H, N, dtype=torch.float32, device="cuda")
        if name.startswith("causal"):
            mask = T.Mask(causal=True)
            pairs = B * H * causal_pairs(N)
        else:
            mask = T.Mask(block_size=16)
            p = np.arange(N)
            pairs = B * H * visible_pairs_dense(np.zeros(N, dtype=np.int64),
                                                np.minimum((p // 16 + 1) * 16 - 1, N - 1))
        desc = mask.desc()
        T.attn_fwd(q, k, v, o, lse, wl.scale, desc)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(T.attn_bwd_workspace_bytes(B, H, N) // 4, dtype=torch.float32, device="cuda")
        fn = lambda: T.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, wl.scale, desc)
        avg, best, wall = time_launches(fn, steps, warmup)
        flops = 10.0 * D * pairs
        out.append(dict(workload=name, avg_ms=avg, min_ms=best, tflops=flops / avg / 1e9,
                        frac=flops / avg / 1e9 / PEAK_BF16_TFLOPS))
        del q, k, v, o, lse, do, dq, dk, dv, ws
    return out


def cpu_baseline(budget_s=12.0):
    """The fp64 oracle on this host, on a bounded sample of the headline workload:
    whole (batch, head) slices of causal B=2 H=16 N=4096 D=64, in order, until the
    time budget is spent.  Useful FLOP as for the GPU."""
    import numpy as np
    import oracle
    from oracle import masks as M
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    wl = W.causal_b2h16n4096d64()
    q = wl.tensors["q"].double().numpy()
    k = wl.tensors["k"].double().numpy()
    v = wl.tensors["v"].double().numpy()
    mod = M.causal(4096, 4096)
    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    for b in range(2):
        for h in range(16):
            for r0 in range(0, 4096, 512):
                rows = np.arange(r0, r0 + 512)
                oracle.attention_rows(q, k, v, wl.scale, mod, b, h, rows)
            flops += 4.0 * 64 * causal_pairs(4096)
            heads += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), model)
    except OSError:
        pass
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=int(threads), cpu_model=model,
                seconds=round(dt, 2), kind="oracle",
                sample=f"{heads} of 32 (batch, head) slices of causal_b2h16n4096d64, fp64 NumPy, "
                       f"{dt:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline prefill only")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "backward", "copy"], default="all",
                    help="profiling helper: run one kernel family only (copy = a plain "
                         "device-to-device copy of 1 GiB, for calibrating HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import tiled_attention_attn_amd as T
    import workloads as W
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({props.gcnArchName}), {props.multi_processor_count} CUs")
    if args.only == "copy":
        n = 1 << 29  # 1 GiB of bf16 read + 1 GiB written per copy
        src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        # an elementwise kernel (torch.mul) that reads 1 GiB and writes 1 GiB
        avg, _, _ = time_launches(lambda: torch.mul(src, 1.0, out=dst), args.steps, args.warmup)
        log(f"copy 1 GiB: {avg*1e3:.1f} us, {2 * n * 2 / avg / 1e6:.0f} GB/s (read + write)")
        return
    if args.only == "decode":
        dec = bench_decode(T, W, args.steps, args.warmup)
        log(f"decode: {dec['avg_ms']*1e3:.1f} us (splitkv {dec['splitkv_ms']*1e3:.1f} + combine "
            f"{dec['combine_ms']*1e3:.1f}), {dec['kv_bytes'] / dec['avg_ms'] / 1e6:.0f} GB/s")
        log(f"auto (contiguous K/V): {dec['auto_ms']*1e3:.1f} us on path {dec['auto_path']}, "
            f"prefill kernels {dec['auto_prefill_ms']*1e3:.1f} us")
        return

    if args.only == "backward":
        for b in bench_backward(T, W, args.steps, args.warmup):
            log(f"backward {b['workload']}: {b['avg_ms']*1e3:.1f} us, {b['tflops']:.1f} TFLOP/s")
        return

    wl, pf = bench_prefill_causal(T, W, args.steps, args.warmup)
    tflops = pf["flops"] / pf["avg_ms"] / 1e9
    log(f"prefill causal_b2h16n4096d64: {pf['avg_ms']*1e3:.1f} us/launch, {tflops:.1f} TFLOP/s")
    result = {
        "metric": "attention TFLOP/s (unmasked) & % bf16 MFMA peak; decode KV GB/s & % HBM peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["wall_ms"] / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal_b2h16n4096d64", "B": 2, "H": 16, "N": 4096, "D": 64,
                   "mask": "causal", "seed": 0},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic("fwd_kernel<64,false>/causal_b2h16n4096d64"),
                     "traffic_unit": "bytes/launch", "kernel": "fwd_kernel<64, false, bf16, false>",
                     "kernel_us": round(pf["avg_ms"] * 1e3, 2),
                     "useful_gflop": round(pf["flops"] / 1e9, 3),
                     "executed_gflop": round(pf["executed_flops"] / 1e9, 3),
                     "executed_tflops": round(pf["executed_flops"] / pf["avg_ms"] / 1e9, 2)},
    }
    if not args.quick and args.only == "all":
        dec = bench_decode(T, W, args.steps, args.warmup)
        gbs = dec["kv_bytes"] / dec["avg_ms"] / 1e6
        log(f"decode: {dec['avg_ms']*1e3:.1f} us (splitkv {dec['splitkv_ms']*1e3:.1f} + combine "
            f"{dec['combine_ms']*1e3:.1f}), {gbs:.0f} GB/s, S={dec['splits']}")
        s_gbs = dec["kv_bytes"] / dec["splitkv_ms"] / 1e6
        result["decode"] = {
            "workload": "decode_b16h32kv8q16k32768d128", "value": round(gbs, 1), "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "us_per_step": round(dec["avg_ms"] * 1e3, 2),
            "splitkv_us": round(dec["splitkv_ms"] * 1e3, 2),
            "splitkv_min_us": round(dec["splitkv_min_ms"] * 1e3, 2),
            "combine_us": round(dec["combine_ms"] * 1e3, 2), "num_splits": dec["splits"],
            "roofline": {"bound": "hbm", "achieved": round(s_gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(s_gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode_kernel<128>/decode_b16h32kv8q16k32768d128"),
                         "traffic_unit": "bytes/launch",
                         "kernel": "decode_kernel<128, bf16, false, true>"},
            "auto_contiguous": {
                "what": "attn_fwd_auto on the same keys in contiguous [B, Hkv, Nk, D] K/V "
                        "(split-KV + combine, chosen by shape) vs attn_fwd (prefill kernels)",
                "path": "splitkv" if dec["auto_path"] == 1 else "prefill",
                "num_splits": dec["auto_splits"], "us": round(dec["auto_ms"] * 1e3, 2),
                "min_us": round(dec["auto_min_ms"] * 1e3, 2),
                "GB/s": round(dec["kv_bytes"] / dec["auto_ms"] / 1e6, 1),
                "prefill_kernels_us": round(dec["auto_prefill_ms"] * 1e3, 2),
                "speedup": round(dec["auto_prefill_ms"] / dec["auto_ms"], 2)},
        }
    if not args.quick:
        others = bench_prefill_others(T, W, args.steps, args.warmup)
        for o in others:
            log(f"prefill {o['workload']}: {o['avg_ms']*1e3:.1f} us, {o['tflops']:.1f} TFLOP/s")
        result["prefill_other"] = [{k: (round(v, 4) if isinstance(v, float) else v)
                                    for k, v in o.items()} for o in others]
        bwd = bench_backward(T, W, args.steps, args.warmup)
        for b in bwd:
            log(f"backward {b['workload']}: {b['avg_ms']*1e3:.1f} us, {b['tflops']:.1f} TFLOP/s")
        result["backward"] = [{k: (round(v, 4) if isinstance(v, float) else v)
                               for k, v in b.items()} for b in bwd]
    if not args.no_cpu_baseline:
        cb = cpu_baseline()
        log(f"cpu oracle: {cb['value']:.4f} TFLOP/s on {cb['cores']} threads ({cb['sample']})")
        cb["value"] = round(cb["value"], 6)
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
