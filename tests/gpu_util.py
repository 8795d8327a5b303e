"""Helpers for the GPU parity tests: tolerance constants, conversions, comparisons."""
import math

import numpy as np
import torch

# Parity bar: max |O_gpu - O_oracle| on bf16 outputs, |LSE_gpu - LSE_oracle| on fp32 LSE.
O_TOL = 2e-2
LSE_TOL = 1e-3
# Q = 0 makes every visible score 0, so LSE = ln(count) is an exact small sum of ones in fp32.
COUNT_LSE_TOL = 1e-5


def f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


class LazyF64:
    """Indexable view of a (CPU or GPU) torch tensor that converts only the indexed part
    to float64 NumPy -- lets the oracle read one (batch, head) of a huge tensor."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        return self.t[idx].to(torch.float64).cpu().numpy()


def bf16_bits(t):
    """int16 NumPy view of a bf16 tensor's bits (for exact gathers on huge pools)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy()


def bits_to_f64(a):
    u = np.asarray(a).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, what="", o_tol=O_TOL, lse_tol=LSE_TOL):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert o_gpu.shape == o_ref.shape, (what, o_gpu.shape, o_ref.shape)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    eo = float(np.max(np.abs(o_gpu - o_ref))) if o_gpu.size else 0.0
    assert eo <= o_tol, f"{what}: max |O err| {eo:.3e} > {o_tol}"
    el = 0.0
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
        lse_ref = np.asarray(lse_ref, dtype=np.float64)
        ninf_g, ninf_r = np.isneginf(lse_gpu), np.isneginf(lse_ref)
        assert np.array_equal(ninf_g, ninf_r), f"{what}: -inf LSE pattern differs"
        fin = ~ninf_r
        el = float(np.max(np.abs(lse_gpu[fin] - lse_ref[fin]))) if fin.any() else 0.0
        assert el <= lse_tol, f"{what}: max |LSE err| {el:.3e} > {lse_tol}"
    print(f"[err] {what}: max |O err| {eo:.3e}, max |LSE err| {el:.3e}", flush=True)
    return eo, el


def sample_rows(n, k, seed):
    """First 8, last 8 and k random rows of [0, n)."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(8, n))) | set(range(max(0, n - 8), n))
    rows |= set(rng.choice(n, size=min(k, n), replace=False).tolist())
    return np.array(sorted(rows))


def doc_offsets(lengths_per_batch, device):
    nd = max(len(l) for l in lengths_per_batch)
    rows = []
    for lens in lengths_per_batch:
        off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        off = np.concatenate([off, np.full(nd + 1 - len(off), off[-1], dtype=np.int32)])
        rows.append(off)
    return torch.tensor(np.stack(rows), dtype=torch.int32, device=device)


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
