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

Timing.  Every kernel is timed with HIP events recorded on the stream it is
launched on (torch's current stream, which the binding passes to the library).
The headline ``value`` comes from K back-to-back launches after W warm-up
launches, bracketed by synchronisation (per-launch time = event time / K).
Every workload also gets a second series: 10 warm-up launches, then at least
100 launches, each bracketed by its own event pair, reported as the median
and the minimum.  Decode splits its series per kernel (split-KV, combine) from
the same launches, so its rate and its roofline come from one timing.

Also in the line: the HBM read ceiling of a plain streaming kernel
(attn_probe_stream_read over 2 GiB, same series), and the fp64 oracle timed on
this host's cores: the headline workload (whole (batch, head) slices within a
time budget) plus a stated sample of every other workload.  One JSON line is
printed on stdout.
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


SERIES_REPS = 100
SERIES_WARMUP = 10


def time_series(fn, reps=SERIES_REPS, warmup=SERIES_WARMUP, split=None):
    """Per-launch times (ms) of `reps` back-to-back launches after `warmup`, each launch
    bracketed by its own event pair on the current stream.  With `split` = a list of
    callables run in order, each one gets its own pair: returns one list per callable."""
    import torch
    parts = split if split is not None else [fn]
    for _ in range(warmup):
        for f in parts:
            f()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
           for _ in range(reps)]
    for row in evs:
        row[0].record(stream)
        for i, f in enumerate(parts):
            f()
            row[i + 1].record(stream)
    torch.cuda.synchronize()
    out = [[row[i].elapsed_time(row[i + 1]) for row in evs] for i in range(len(parts))]
    return out if split is not None else out[0]


def stats(ts):
    import numpy as np
    a = np.asarray(ts, dtype=np.float64)
    return dict(median_ms=float(np.median(a)), min_ms=float(a.min()), mean_ms=float(a.mean()),
                reps=int(a.size))


def host_cores():
    return len(os.sched_getaffinity(0))


def causal_pairs(N):
    return N * (N + 1) // 2


def visible_pairs_dense(lo, hi):
    import numpy as np
    return int(np.maximum(hi - lo + 1, 0).sum())


def executed_pp_flops(lo, hi, D, rows=256, kblk=64, wave_rows=32):
    """FLOP the D=128 dense-mask prefill kernel executes for one head: 256-row tiles,
    64-key steps from the tile's first row's lo to its last row's hi, and a 32-row wave
    runs a step unless none of its rows sees a key of it (every MFMA of a run step is
    counted in full, masked elements included)."""
    N = len(lo)
    total = 0
    for q0 in range(0, N, rows):
        last = min(q0 + rows, N) - 1
        lo_first, hi_last = int(lo[q0]), int(hi[last])
        if hi_last < lo_first:
            continue
        kb_begin = (lo_first // kblk) * kblk
        n_steps = (hi_last + 1 - kb_begin + kblk - 1) // kblk
        for w0 in range(q0, last + 1, wave_rows):
            wl, wh = int(lo[w0]), int(hi[min(w0 + wave_rows, N) - 1])
            for j in range(n_steps):
                kb = kb_begin + j * kblk
                if not (kb > wh or kb + kblk - 1 < wl):
                    total += 1
    return 4.0 * D * wave_rows * kblk * total


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
    ser = stats(time_series(fn))
    flops = 4.0 * 64 * 2 * 16 * causal_pairs(4096)
    # Executed work: each 128-row query tile t runs t + 1 steps of 128 keys in full
    # (the diagonal step's masked half included).
    executed = 4.0 * 64 * 2 * 16 * sum((t + 1) * 128 * 128 for t in range(4096 // 128))
    return wl, dict(avg_ms=avg, min_ms=best, wall_ms=wall, flops=flops, executed_flops=executed,
                    series=ser)


def _rate_fields(flops, executed, avg_ms, ser):
    return dict(avg_ms=avg_ms, median_ms=ser["median_ms"], min_ms=ser["min_ms"], reps=ser["reps"],
                tflops=flops / avg_ms / 1e9, frac=flops / avg_ms / 1e9 / PEAK_BF16_TFLOPS,
                median_tflops=flops / ser["median_ms"] / 1e9,
                useful_gflop=flops / 1e9, executed_gflop=executed / 1e9,
                executed_tflops=executed / avg_ms / 1e9)


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
        ser = stats(time_series(fn))
        flops = 4.0 * 128 * 32 * visible_pairs_dense(lo, hi)
        executed = 32 * executed_pp_flops(lo, hi, 128)
        out.append(dict(workload=name, kernel="fwd_pp_kernel<128>",
                        **_rate_fields(flops, executed, avg, ser)))
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
    b_ser = stats(time_series(build))
    desc = T.Mask(causal=True).desc()
    fn = lambda: T.attn_fwd_blockmask(q, k, v, o, bm, lse, wl.scale, desc)
    avg, best, wall = time_launches(fn, steps, warmup)
    ser = stats(time_series(fn))
    n_full = int((tm == W.TILE_FULL).sum())
    n_diag = int((tm == W.TILE_PARTIAL).sum())
    pairs = n_full * 128 * 128 + n_diag * (128 * 129 // 2)
    flops = 4.0 * 128 * 32 * pairs
    # every listed tile runs both of its 64-key steps for all 128 rows
    executed = 4.0 * 128 * 32 * (n_full + n_diag) * 128 * 128
    out.append(dict(workload=wl.name, kernel="fwd_kernel<128, blockmask>",
                    **_rate_fields(flops, executed, avg, ser),
                    blockmask_build_median_ms=b_ser["median_ms"]))
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
    avg, best, wall = time_launches(both, steps, warmup)
    # one series, each launch of each kernel bracketed by its own events
    ts_split, ts_comb = time_series(None, split=[split, comb])
    step_ser = stats([a + b for a, b in zip(ts_split, ts_comb)])
    split_ser, comb_ser = stats(ts_split), stats(ts_comb)
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
    a_ser = stats(time_series(lambda: T.attn_fwd_auto(q, kc, vc, o, lse, scale, cm, ws)))
    p_ser = stats(time_series(lambda: T.attn_fwd(q, kc, vc, o, lse, scale, cm), reps=20, warmup=3))
    return dict(avg_ms=avg, wall_ms=wall, step=step_ser, split=split_ser, comb=comb_ser, splits=S,
                kv_bytes=kv_bytes, auto=a_ser, auto_path=int(plan.path),
                auto_splits=int(plan.num_splits), auto_prefill=p_ser)


def bench_stream(T):
    """Read ceiling: the streaming probe over 2 GiB (one 256-thread group per CU, eight
    16-byte loads in flight per lane), same series as the kernels."""
    import torch
    n = 2 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    ser = stats(time_series(lambda: T.attn_probe_stream_read(src, sink, blocks)))
    del src
    return dict(bytes=n, blocks=blocks, median_gbs=n / ser["median_ms"] / 1e6,
                best_gbs=n / ser["min_ms"] / 1e6, median_us=ser["median_ms"] * 1e3)


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
        ser = stats(time_series(fn))
        flops = 10.0 * D * pairs
        out.append(dict(workload=name, avg_ms=avg, median_ms=ser["median_ms"], min_ms=ser["min_ms"],
                        reps=ser["reps"], tflops=flops / avg / 1e9,
                        frac=flops / avg / 1e9 / PEAK_BF16_TFLOPS,
                        median_tflops=flops / ser["median_ms"] / 1e9))
        del q, k, v, o, lse, do, dq, dk, dv, ws
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            return next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")),
                        "unknown")
    except OSError:
        return "unknown"


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return host_cores()


def cpu_baseline(budget_s=8.0):
    """The fp64 oracle on this host, on a bounded sample of the headline workload:
    whole (batch, head) slices of causal B=2 H=16 N=4096 D=64, in order, until the
    time budget is spent.  Useful FLOP as for the GPU."""
    import numpy as np
    import oracle
    from oracle import masks as M
    import workloads as W
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
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=int(_blas_threads()),
                host_cores=host_cores(), cpu_model=_cpu_model(), seconds=round(dt, 2),
                kind="oracle",
                sample=f"{heads} of 32 (batch, head) slices of causal_b2h16n4096d64, fp64 NumPy, "
                       f"{dt:.1f} s")


def cpu_oracle_samples():
    """The fp64 oracle timed on a stated sample of every other workload (same process,
    same host threads): one head of each N=8192 workload (all 8192 rows), 32 query tiles
    of one head of the block-sparse workload (the first, the last and the 30 densest,
    against all 32768 keys), and one sequence of the decode workload (all 32 heads x 16
    queries over its 32768 paged keys)."""
    import numpy as np
    import oracle
    from oracle import masks as M, paged as OP
    import workloads as W
    out = []

    def timed(name, sample, fn, flops):
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
        out.append(dict(workload=name, sample=sample, seconds=round(dt, 2),
                        useful_gflop=round(flops / 1e9, 3), tflops=round(flops / dt / 1e12, 6)))
    N = 8192
    p = np.arange(N)
    for name in ("window_doc_b1h32n8192d128", "blockdiff_b1h32n8192d128"):
        wl = W.FULL_SIZE[name]()
        q, k, v = (wl.tensors[x][:, :1].double().numpy() for x in ("q", "k", "v"))
        if name.startswith("window"):
            lens = wl.mask["doc_lengths"][0]
            mod = M.and_(M.window(512, 512, N, N), M.document([lens], N, N))
            starts = np.concatenate([[0], np.cumsum(lens)])
            d = np.searchsorted(starts, p, side="right") - 1
            pairs = int((np.minimum(p + 512, starts[d + 1] - 1)
                         - np.maximum(p - 512, starts[d]) + 1).sum())
        else:
            mod = M.block_causal(16, N, N)
            pairs = int((np.minimum((p // 16 + 1) * 16 - 1, N - 1) + 1).sum())
        timed(name, "head 0 of 32, all 8192 rows",
              lambda: oracle.attention(q, k, v, wl.scale, mod, row_block=1024), 4.0 * 128 * pairs)
        del wl, q, k, v
    wl = W.blockmask_gqa_b1h32kv8n32768d128()
    tm = wl.mask["tile_map"].numpy()
    nt = tm.shape[0]
    dens = (tm != W.TILE_EMPTY).sum(1)
    order = [0, nt - 1] + [int(i) for i in np.argsort(-dens, kind="stable")
                           if i not in (0, nt - 1)][:30]
    q = wl.tensors["q"][:, :1].double().numpy()
    k = wl.tensors["k"][:, :1].double().numpy()
    v = wl.tensors["v"][:, :1].double().numpy()
    mod = M.blockmask(tm, 128, M.causal(32768, 32768))
    pairs = sum(int((tm[t] == W.TILE_FULL).sum()) * 128 * 128 + 128 * 129 // 2 for t in order)

    def bm_rows():
        for t in order:
            oracle.attention_rows(q, k, v, wl.scale, mod, 0, 0, np.arange(t * 128, (t + 1) * 128))
    timed(wl.name, "32 query tiles of head 0 (first, last, 30 densest) against all 32768 keys",
          bm_rows, 4.0 * 128 * pairs)
    del wl, q, k, v
    wl = W.decode_b16h32kv8q16k32768d128()
    t = wl.tensors
    bt0 = t["block_table"][0].long()
    # sequence 0's 2048 pages, re-indexed 0..2047, gathered by the oracle's own page walk
    kp = t["k_pool"][bt0].double().numpy()
    vp = t["v_pool"][bt0].double().numpy()
    table = np.arange(2048)[None]
    qd = t["q"][:1].double().numpy()
    del wl, t

    def dec():
        kl = OP.gather(kp, table, 0, 32768)[None]
        vl = OP.gather(vp, table, 0, 32768)[None]
        oracle.attention(qd, kl, vl, 1.0 / math.sqrt(128), M.causal(16, 32768))
    pairs = 32 * sum(32768 - 16 + i + 1 for i in range(16))
    timed("decode_b16h32kv8q16k32768d128",
          "sequence 0 of 16: all 32 heads x 16 queries over its 32768 paged keys", dec,
          4.0 * 128 * pairs)
    return out


def _leg(result, key, fn):
    """Runs one secondary leg.  A Python-level failure there (an argument error, a shape
    mistake) is recorded under result[key] = {"error": ...} instead of losing the
    headline line; it is logged and returns None."""
    try:
        return fn()
    except Exception as e:  # noqa: BLE001 - reported in the JSON line, not swallowed
        log(f"{key} failed: {type(e).__name__}: {e}")
        result[key] = {"error": f"{type(e).__name__}: {e}"}
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="headline prefill only")
    ap.add_argument("--only", choices=["all", "prefill", "others", "decode", "backward", "copy",
                                       "stream"], default="all",
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
    if args.only == "stream":
        st = bench_stream(T)
        log(f"stream read 2 GiB: {st['median_us']:.1f} us, {st['median_gbs']:.0f} GB/s median")
        return
    if args.only == "decode":
        dec = bench_decode(T, W, args.steps, args.warmup)
        log(f"decode: {dec['step']['median_ms']*1e3:.1f} us median (splitkv "
            f"{dec['split']['median_ms']*1e3:.1f} + combine {dec['comb']['median_ms']*1e3:.1f})")
        return
    if args.only == "backward":
        for b in bench_backward(T, W, args.steps, args.warmup):
            log(f"backward {b['workload']}: {b['avg_ms']*1e3:.1f} us, {b['tflops']:.1f} TFLOP/s")
        return
    if args.only == "others":
        for o in bench_prefill_others(T, W, args.steps, args.warmup):
            log(f"prefill {o['workload']}: {o['avg_ms']*1e3:.1f} us, {o['tflops']:.1f} TFLOP/s")
        return

    wl, pf = bench_prefill_causal(T, W, args.steps, args.warmup)
    tflops = pf["flops"] / pf["avg_ms"] / 1e9
    ser = pf["series"]
    log(f"prefill causal_b2h16n4096d64: {pf['avg_ms']*1e3:.1f} us/launch, {tflops:.1f} TFLOP/s "
        f"(series median {ser['median_ms']*1e3:.1f} us, min {ser['min_ms']*1e3:.1f} us)")
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
                     "median_us": round(ser["median_ms"] * 1e3, 2),
                     "min_us": round(ser["min_ms"] * 1e3, 2), "series_reps": ser["reps"],
                     "median_frac": round(pf["flops"] / ser["median_ms"] / 1e9 / PEAK_BF16_TFLOPS, 4),
                     "useful_gflop": round(pf["flops"] / 1e9, 3),
                     "executed_gflop": round(pf["executed_flops"] / 1e9, 3),
                     "executed_tflops": round(pf["executed_flops"] / pf["avg_ms"] / 1e9, 2)},
    }
    dec = others = bwd = None
    if not args.quick and args.only == "all":
        dec = _leg(result, "decode", lambda: bench_decode(T, W, args.steps, args.warmup))
    if dec is not None:
        kvb = dec["kv_bytes"]
        step_ms, split_ms = dec["step"]["median_ms"], dec["split"]["median_ms"]
        gbs = kvb / step_ms / 1e6
        s_gbs = kvb / split_ms / 1e6
        log(f"decode: {step_ms*1e3:.1f} us median (splitkv {split_ms*1e3:.1f} + combine "
            f"{dec['comb']['median_ms']*1e3:.1f}), {gbs:.0f} GB/s, S={dec['splits']}; "
            f"{dec['avg_ms']*1e3:.1f} us mean over {args.steps} back-to-back steps")
        err = {}
        st = _leg(err, "read_ceiling", lambda: bench_stream(T))
        if st is not None:
            log(f"stream read ceiling: {st['median_gbs']:.0f} GB/s median, {st['best_gbs']:.0f} best")
        result["decode"] = {
            "workload": "decode_b16h32kv8q16k32768d128", "value": round(gbs, 1), "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "timing": f"median of {dec['step']['reps']} event-bracketed steps after "
                      f"{SERIES_WARMUP} warm-ups; value and roofline from the same launches",
            "us_per_step_median": round(step_ms * 1e3, 2),
            "us_per_step_min": round(dec["step"]["min_ms"] * 1e3, 2),
            "us_per_step_backtoback_mean": round(dec["avg_ms"] * 1e3, 2),
            "splitkv_median_us": round(split_ms * 1e3, 2),
            "splitkv_min_us": round(dec["split"]["min_ms"] * 1e3, 2),
            "combine_median_us": round(dec["comb"]["median_ms"] * 1e3, 2),
            "num_splits": dec["splits"],
            "roofline": {"bound": "hbm", "achieved": round(s_gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(s_gbs / PEAK_HBM_GBS, 4),
                         "traffic": measured_traffic("decode_kernel<128>/decode_b16h32kv8q16k32768d128"),
                         "traffic_unit": "bytes/launch",
                         "kernel": "decode_kernel<128, bf16, false, true>",
                         "kernel_median_us": round(split_ms * 1e3, 2)},
            "read_ceiling": err.get("read_ceiling") if st is None else {
                "what": "attn_probe_stream_read: plain streaming read of 2 GiB, one "
                        "256-thread group per CU, median of the same series",
                "median_gbs": round(st["median_gbs"], 1),
                "best_gbs": round(st["best_gbs"], 1),
                "decode_frac_of_ceiling": round(gbs / st["median_gbs"], 4)},
            "auto_contiguous": {
                "what": "attn_fwd_auto on the same keys in contiguous [B, Hkv, Nk, D] K/V "
                        "(split-KV + combine, chosen by shape) vs attn_fwd (prefill kernels)",
                "path": "splitkv" if dec["auto_path"] == 1 else "prefill",
                "num_splits": dec["auto_splits"],
                "median_us": round(dec["auto"]["median_ms"] * 1e3, 2),
                "GB/s": round(kvb / dec["auto"]["median_ms"] / 1e6, 1),
                "prefill_kernels_median_us": round(dec["auto_prefill"]["median_ms"] * 1e3, 2),
                "speedup": round(dec["auto_prefill"]["median_ms"] / dec["auto"]["median_ms"], 2)},
        }
    if not args.quick:
        others = _leg(result, "prefill_other", lambda: bench_prefill_others(T, W, args.steps, args.warmup))
    if not args.quick and others is not None:
        for o in others:
            log(f"prefill {o['workload']}: {o['avg_ms']*1e3:.1f} us, {o['tflops']:.1f} TFLOP/s "
                f"(median {o['median_ms']*1e3:.1f} us; executed {o['executed_gflop']:.1f} of "
                f"useful {o['useful_gflop']:.1f} GFLOP)")
        result["prefill_other"] = [{k: (round(v, 4) if isinstance(v, float) else v)
                                    for k, v in o.items()} for o in others]
    if not args.quick:
        bwd = _leg(result, "backward", lambda: bench_backward(T, W, args.steps, args.warmup))
    if not args.quick and bwd is not None:
        for b in bwd:
            log(f"backward {b['workload']}: {b['avg_ms']*1e3:.1f} us, {b['tflops']:.1f} TFLOP/s "
                f"(median {b['median_ms']*1e3:.1f} us)")
        result["backward"] = [{k: (round(v, 4) if isinstance(v, float) else v)
                               for k, v in b.items()} for b in bwd]
    if not args.no_cpu_baseline:
        cb = cpu_baseline()
        log(f"cpu oracle: {cb['value']:.4f} TFLOP/s on {cb['cores']} threads of {cb['host_cores']} "
            f"host cores ({cb['sample']})")
        cb["value"] = round(cb["value"], 6)
        if not args.quick:
            cb["other_workloads"] = _leg(cb, "other_workloads", cpu_oracle_samples) or cb.get("other_workloads", [])
            for o in (cb["other_workloads"] if isinstance(cb["other_workloads"], list) else []):
                log(f"cpu oracle {o['workload']}: {o['seconds']} s, {o['tflops']:.4f} TFLOP/s "
                    f"({o['sample']})")
        result["cpu_baseline"] = cb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
