"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic. It only draws tensors and structure:

* Q/K/V: fp32 samples of N(0, 1) from a CPU ``torch.Generator`` seeded per
  workload, rounded to bfloat16 with round-to-nearest-even.  The pages build
  their test tensors the same way (``torch.randn`` in bf16; FlashAttention 2
  principles and PyTorch practice, section 2 code and section 5 code).
* document lengths: i.i.d. uniform integers in [lo, hi] until they cover the
  sequence; the last document is truncated to fit.
* BlockMask tile picks: a seeded choice, without replacement, of strictly
  lower-triangular 128x128 tiles.
* paged KV cache: a seeded permutation of a page pool gives the block table;
  the logical K/V rows are scattered into the pool and every page that no
  sequence uses is filled with NaN (poison).

Draw order is fixed: Q, K, V (logical shapes), then the structure.  Both the
CPU oracle's tests and the HIP path's tests and benchmark take their inputs
from here, so the two sides see the same bytes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Tile-map codes shared by every BlockMask consumer (interface format, not arithmetic).
TILE_EMPTY = 0
TILE_PARTIAL = 1
TILE_FULL = 2
BLOCKMASK_TILE = 128


def generator(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def randn_bf16(gen: torch.Generator, shape) -> torch.Tensor:
    """fp32 N(0,1) draw rounded to bf16 (RNE), on the CPU."""
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(torch.bfloat16)


def randn_half(gen: torch.Generator, shape, dtype=torch.bfloat16) -> torch.Tensor:
    """fp32 N(0,1) draw rounded (RNE) to a 16-bit float type (bf16 or fp16), on the CPU."""
    return torch.randn(*shape, generator=gen, dtype=torch.float32).to(dtype)


def doc_lengths(gen: torch.Generator, n: int, lo: int = 512, hi: int = 2048) -> list[int]:
    """Document lengths drawn uniform on the integers [lo, hi] until they cover n tokens."""
    out: list[int] = []
    total = 0
    while total < n:
        ln = int(torch.randint(lo, hi + 1, (1,), generator=gen).item())
        ln = min(ln, n - total)
        out.append(ln)
        total += ln
    return out


def blockmask_tile_map(gen: torch.Generator, n_tiles: int, frac: float = 0.1) -> torch.Tensor:
    """uint8 [n_tiles, n_tiles] map: diagonal tiles PARTIAL, round(frac * #strictly-lower)
    strictly-lower tiles FULL (seeded, without replacement), everything else EMPTY."""
    tmap = torch.zeros(n_tiles, n_tiles, dtype=torch.uint8)
    idx = torch.arange(n_tiles)
    tmap[idx, idx] = TILE_PARTIAL
    lower_i, lower_j = torch.tril_indices(n_tiles, n_tiles, offset=-1)
    n_lower = lower_i.numel()
    n_pick = int(round(frac * n_lower))
    pick = torch.randperm(n_lower, generator=gen)[:n_pick]
    tmap[lower_i[pick], lower_j[pick]] = TILE_FULL
    return tmap


@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    D: int
    scale: float
    mask: dict = field(default_factory=dict)
    tensors: dict = field(default_factory=dict)


def _qkv(gen, B, Hq, Hkv, Nq, Nk, D):
    q = randn_bf16(gen, (B, Hq, Nq, D))
    k = randn_bf16(gen, (B, Hkv, Nk, D))
    v = randn_bf16(gen, (B, Hkv, Nk, D))
    return q, k, v


def dense(name: str, B: int, Hq: int, Hkv: int, N: int, D: int, mask: dict, seed: int = 0,
          Nk: int | None = None, doc_range=(512, 2048)) -> Workload:
    """A prefill workload with a dense (interval) mask.

    ``mask`` keys: causal (bool), window (int w for |q-k| <= w, or None),
    document (bool: draw document lengths), block_size (block-diffusion, or None).
    """
    gen = generator(seed)
    Nk = N if Nk is None else Nk
    q, k, v = _qkv(gen, B, Hq, Hkv, N, Nk, D)
    m = dict(mask)
    if m.get("document"):
        m["doc_lengths"] = [doc_lengths(gen, Nk, *doc_range) for _ in range(B)]
    return Workload(name, B, Hq, Hkv, N, Nk, D, 1.0 / math.sqrt(D), m, dict(q=q, k=k, v=v))


def blocksparse(name: str, B: int, Hq: int, Hkv: int, N: int, D: int, frac: float = 0.1,
                seed: int = 0) -> Workload:
    """Block-sparse prefill: a 128x128 tile map (diagonal PARTIAL with causal inside,
    ``frac`` of the strictly-lower tiles FULL), shared by every batch and head."""
    gen = generator(seed)
    q, k, v = _qkv(gen, B, Hq, Hkv, N, N, D)
    n_t = (N + BLOCKMASK_TILE - 1) // BLOCKMASK_TILE
    tmap = blockmask_tile_map(gen, n_t, frac)
    return Workload(name, B, Hq, Hkv, N, N, D, 1.0 / math.sqrt(D),
                    dict(causal=True, tile_map=tmap), dict(q=q, k=k, v=v))


def paged_decode(name: str, B: int, Hq: int, Hkv: int, Lq: int, Nk: int, D: int,
                 page_size: int = 16, pool_pages: int = 40000, seed: int = 0,
                 seq_lens: list[int] | None = None) -> Workload:
    """Split-KV paged decode: Lq new queries per sequence over Nk keys (the Lq new tokens
    included), K/V in ``page_size``-token pages of a shared pool [pages, page_size, Hkv, D].

    The block table is a seeded permutation of the pool; pages no sequence uses hold NaN.
    ``seq_lens`` (optional) gives ragged per-sequence key lengths (<= Nk).
    """
    gen = generator(seed)
    q = randn_bf16(gen, (B, Hq, Lq, D))
    k_log = randn_bf16(gen, (B, Hkv, Nk, D))
    v_log = randn_bf16(gen, (B, Hkv, Nk, D))
    pages_per_seq = (Nk + page_size - 1) // page_size
    if B * pages_per_seq > pool_pages:
        raise ValueError("page pool too small")
    perm = torch.randperm(pool_pages, generator=gen)
    block_table = perm[: B * pages_per_seq].reshape(B, pages_per_seq).to(torch.int32)
    if seq_lens is None:
        seq_lens = [Nk] * B
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
    k_pool = torch.full((pool_pages, page_size, Hkv, D), nan.item(), dtype=torch.bfloat16)
    v_pool = torch.full((pool_pages, page_size, Hkv, D), nan.item(), dtype=torch.bfloat16)
    pad = pages_per_seq * page_size - Nk
    for b in range(B):
        kb = k_log[b]  # [Hkv, Nk, D]
        vb = v_log[b]
        if pad:
            kb = torch.cat([kb, torch.full((Hkv, pad, D), nan.item(), dtype=torch.bfloat16)], 1)
            vb = torch.cat([vb, torch.full((Hkv, pad, D), nan.item(), dtype=torch.bfloat16)], 1)
        # [Hkv, pages, page_size, D] -> [pages, page_size, Hkv, D]
        kb = kb.reshape(Hkv, pages_per_seq, page_size, D).permute(1, 2, 0, 3)
        vb = vb.reshape(Hkv, pages_per_seq, page_size, D).permute(1, 2, 0, 3)
        rows = block_table[b].long()
        k_pool[rows] = kb
        v_pool[rows] = vb
        # rows beyond this sequence's length are poison as well
        sl = seq_lens[b]
        if sl < Nk:
            for j in range(sl, pages_per_seq * page_size):
                k_pool[rows[j // page_size], j % page_size] = nan.item()
                v_pool[rows[j // page_size], j % page_size] = nan.item()
    return Workload(name, B, Hq, Hkv, Lq, Nk, D, 1.0 / math.sqrt(D),
                    dict(causal=True, page_size=page_size),
                    dict(q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table,
                         seq_lens=torch.tensor(seq_lens, dtype=torch.int32),
                         k_logical=k_log, v_logical=v_log))


# The five workloads at full size (seed 0 for all of them).
def causal_b1h1n256d64(seed: int = 0) -> Workload:
    """Single-head causal attention, B=1 H=1 N=256 D=64 (small correctness case)."""
    return dense("causal_b1h1n256d64", 1, 1, 1, 256, 64, dict(causal=True), seed)


def causal_b2h16n4096d64(seed: int = 0) -> Workload:
    """Causal prefill B=2 H=16 N=4096 D=64 (the pages' SDPA / flash_attn example shape)."""
    return dense("causal_b2h16n4096d64", 2, 16, 16, 4096, 64, dict(causal=True), seed)


def window_doc_b1h32n8192d128(seed: int = 0) -> Workload:
    """Bidirectional symmetric window |q-k| <= 512 AND same document, docs U[512, 2048]."""
    return dense("window_doc_b1h32n8192d128", 1, 32, 32, 8192, 128,
                 dict(window=512, document=True), seed)


def blockdiff_b1h32n8192d128(seed: int = 0) -> Workload:
    """Block-diffusion: 16-token blocks bidirectional inside, causal to the prior context."""
    return dense("blockdiff_b1h32n8192d128", 1, 32, 32, 8192, 128, dict(block_size=16), seed)


def blockmask_gqa_b1h32kv8n32768d128(seed: int = 0) -> Workload:
    """Block-sparse long prefill with GQA 32/8, N=32768, 128x128 tiles."""
    return blocksparse("blockmask_gqa_b1h32kv8n32768d128", 1, 32, 8, 32768, 128, 0.1, seed)


def decode_b16h32kv8q16k32768d128(seed: int = 0) -> Workload:
    """Split-KV paged decode: B=16, Hq=32, Hkv=8, 16 draft queries, 32768 keys, 16-token pages."""
    return paged_decode("decode_b16h32kv8q16k32768d128", 16, 32, 8, 16, 32768, 128, 16, 40000, seed)


FULL_SIZE = {
    "causal_b1h1n256d64": causal_b1h1n256d64,
    "causal_b2h16n4096d64": causal_b2h16n4096d64,
    "window_doc_b1h32n8192d128": window_doc_b1h32n8192d128,
    "blockdiff_b1h32n8192d128": blockdiff_b1h32n8192d128,
    "blockmask_gqa_b1h32kv8n32768d128": blockmask_gqa_b1h32kv8n32768d128,
    "decode_b16h32kv8q16k32768d128": decode_b16h32kv8q16k32768d128,
}
