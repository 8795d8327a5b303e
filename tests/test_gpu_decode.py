"""GPU parity: split-KV paged decode (attn_decode_splitkv) and the LSE combine
(attn_decode_combine) against the fp64 CPU oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import masks as M, paged as OP
import workloads as W
from gpu_util import (f64, assert_close, bf16_bits, bits_to_f64, sample_rows, announce,
                      COUNT_LSE_TOL)

pytestmark = pytest.mark.gpu
if torch.cuda.is_available():
    import tiled_attention_attn_amd as T
DEV = "cuda"


def _decode(wl, S, max_pages=None, mask=None, q=None):
    t = wl.tensors
    B, Hq, Lq, D = t["q"].shape
    max_pages = t["block_table"].shape[1] if max_pages is None else max_pages
    qg = (t["q"] if q is None else q).to(DEV)
    ws_o = torch.full((B, Hq, Lq, S, D), float("nan"), dtype=torch.float32, device=DEV)
    ws_l = torch.full((B, Hq, Lq, S), float("nan"), dtype=torch.float32, device=DEV)
    T.attn_decode_splitkv(qg, t["k_pool"].to(DEV), t["v_pool"].to(DEV), t["block_table"].to(DEV),
                          t["seq_lens"].to(DEV), max_pages, S, ws_o, ws_l, wl.scale, mask)
    o = torch.empty(B, Hq, Lq, D, dtype=qg.dtype, device=DEV)
    lse = torch.empty(B, Hq, Lq, dtype=torch.float32, device=DEV)
    T.attn_decode_combine(ws_o, ws_l, o, lse)
    torch.cuda.synchronize()
    return ws_o.cpu(), ws_l.cpu(), o.cpu(), lse.cpu()


CASES = [
    # (id, B, Hq, Hkv, Lq, Nk, D, page, seq_lens, S)
    ("ps16_s3", 2, 8, 2, 5, 300, 128, 16, [300, 171], 3),
    ("ps16_s1", 2, 4, 4, 16, 200, 64, 16, [200, 16], 1),
    ("ps8_s5_gqa8", 1, 8, 1, 4, 333, 128, 8, [333], 5),
    ("ps16_many_splits", 3, 4, 2, 2, 130, 64, 16, [130, 1, 64], 9),
    ("ps32_rows80", 1, 20, 2, 8, 500, 128, 32, [500], 2),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "fp16"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_small_decode_partials_and_combine(case, dtype):
    name, B, Hq, Hkv, Lq, Nk, D, ps, sl, S = case
    if dtype == torch.float16 and name not in ("ps16_s3", "ps16_s1", "ps32_rows80"):
        pytest.skip("fp16 checked on a subset")
    announce(f"decode {name} {dtype}")
    pages_per_seq = (Nk + ps - 1) // ps
    wl = W.paged_decode(name, B, Hq, Hkv, Lq, Nk, D, page_size=ps,
                        pool_pages=B * pages_per_seq + 7, seed=len(name), seq_lens=sl)
    if dtype != torch.bfloat16:  # the same draws, rounded from bf16 to fp16
        for key in ("q", "k_pool", "v_pool"):
            wl.tensors[key] = wl.tensors[key].to(dtype)
    ws_o, ws_l, o, lse = _decode(wl, S)
    t = wl.tensors
    kp, vp, bt = f64(t["k_pool"]), f64(t["v_pool"]), t["block_table"].numpy()
    C = ps * math.ceil(pages_per_seq / S)
    q = f64(t["q"])
    for b in range(B):
        kl = OP.gather(kp, bt, b, sl[b])[None]
        vl = OP.gather(vp, bt, b, sl[b])[None]
        qb = q[b:b + 1]
        ro, rl = oracle.attention(qb, kl, vl, wl.scale, M.causal(Lq, sl[b]))
        assert_close(f64(o[b:b + 1]), f64(lse[b:b + 1]), ro, rl, f"{name} b{b}")
        for s in range(S):
            po, pl = oracle.attention(qb, kl, vl, wl.scale,
                                      M.and_(M.causal(Lq, sl[b]), M.key_range(s * C, (s + 1) * C)))
            assert_close(f64(ws_o[b:b + 1, :, :, s]), f64(ws_l[b:b + 1, :, :, s]), po, pl,
                         f"{name} b{b} split{s}")


def test_paged_equals_contiguous_bitwise():
    """The same logical K/V in a permuted page pool or in pages in order: bitwise equal."""
    announce("paged == contiguous")
    wl = W.paged_decode("perm", 2, 8, 2, 4, 1000, 128, page_size=16, pool_pages=200, seed=2)
    ident = W.paged_decode("perm", 2, 8, 2, 4, 1000, 128, page_size=16, pool_pages=200, seed=2)
    t = ident.tensors
    pps = t["block_table"].shape[1]
    bt = torch.arange(2 * pps, dtype=torch.int32).reshape(2, pps)
    for name in ("k_pool", "v_pool"):
        logical = t["k_logical" if name == "k_pool" else "v_logical"]
        pool = torch.full_like(t[name], float("nan"))
        pad = pps * 16 - logical.shape[2]
        logical = torch.cat([logical, torch.full((2, 2, pad, 128), float("nan"), dtype=logical.dtype)], 2)
        for b in range(2):
            pool[bt[b].long()] = logical[b].reshape(2, pps, 16, 128).permute(1, 2, 0, 3)
        t[name] = pool
    t["block_table"] = bt
    a = _decode(wl, 4)
    c = _decode(ident, 4)
    for x, y in zip(a, c):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x.view(torch.int16),
                           y.view(torch.int32) if y.dtype == torch.float32 else y.view(torch.int16))


WINDOW_CASES = [
    # (id, B, Hq, Hkv, Lq, Nk, seq_lens, S): the draft model's sliding-window
    # call over a paged cache, grouped by where the sequence ends against the
    # (2048, 2048) window.
    ("mixed_b2", 2, 4, 2, 8, 3000, [3000, 3000], 4),
    ("short", 2, 4, 2, 8, 40, [40, 9], 2),
    ("single_stream", 1, 8, 2, 8, 2100, [2100], 3),
    ("window_edge", 2, 4, 1, 8, 2064, [2056, 2057], 4),
    ("beyond_window", 2, 4, 2, 8, 6000, [6000, 4500], 6),
]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=[c[0] for c in WINDOW_CASES])
def test_window_mask_decode(case):
    """Non-causal symmetric window over a paged cache (the draft-model call shape);
    beyond the window the first splits see no key and must get weight 0."""
    name, B, Hq, Hkv, Lq, Nk, sl, S = case
    announce(f"decode window {name}")
    pages = (Nk + 15) // 16
    wl = W.paged_decode("win" + name, B, Hq, Hkv, Lq, Nk, 128, page_size=16,
                        pool_pages=B * pages + 5, seed=4 + len(name), seq_lens=sl)
    ws_o, ws_l, o, lse = _decode(wl, S, mask=T.Mask(window=(2048, 2048)))
    t = wl.tensors
    kp, vp, bt = f64(t["k_pool"]), f64(t["v_pool"]), t["block_table"].numpy()
    C = 16 * math.ceil(pages / S)
    for b in range(B):
        kl = OP.gather(kp, bt, b, sl[b])[None]
        vl = OP.gather(vp, bt, b, sl[b])[None]
        qb = f64(t["q"])[b:b + 1]
        ro, rl = oracle.attention(qb, kl, vl, wl.scale, M.window(2048, 2048, Lq, sl[b]))
        assert_close(f64(o[b:b + 1]), f64(lse[b:b + 1]), ro, rl, f"window {name} b{b}")
        for s in range(S):
            po, pl = oracle.attention(qb, kl, vl, wl.scale,
                                      M.and_(M.window(2048, 2048, Lq, sl[b]), M.key_range(s * C, (s + 1) * C)))
            assert_close(f64(ws_o[b:b + 1, :, :, s]), f64(ws_l[b:b + 1, :, :, s]), po, pl,
                         f"window {name} b{b} split{s}")


def test_config5_decode_b16h32kv8q16k32768d128_every_row():
    """Full-size paged decode: every (sequence, head, query) row vs the oracle, element by
    element, plus the Q = 0 count test on every row (LSE = ln(#visible keys) to 1e-5)."""
    announce("decode_b16h32kv8q16k32768d128")
    wl = W.decode_b16h32kv8q16k32768d128()
    t = wl.tensors
    B, Hq, Lq, D, Nk = 16, 32, 16, 128, 32768
    S = T.attn_decode_num_splits(B, 8, 2048)
    ws_o, ws_l, o, lse = _decode(wl, S)
    kbits, vbits, bt = bf16_bits(t["k_pool"]), bf16_bits(t["v_pool"]), t["block_table"].numpy()
    q = f64(t["q"])
    eo = el = 0.0
    for b in range(B):
        kl = bits_to_f64(OP.gather(kbits, bt, b, Nk))
        vl = bits_to_f64(OP.gather(vbits, bt, b, Nk))
        ro, rl = oracle.attention(q[b:b + 1], kl[None], vl[None], wl.scale, M.causal(Lq, Nk))
        e = assert_close(f64(o[b:b + 1]), f64(lse[b:b + 1]), ro, rl, f"cfg5 b{b}, all 32 heads x 16 rows")
        eo, el = max(eo, e[0]), max(el, e[1])
        del kl, vl
    print(f"[err] cfg5 every row: max |O err| {eo:.3e}, max |LSE err| {el:.3e}")
    # Q = 0: every row of every sequence and head sees exactly Nk - Lq + 1 + t keys
    _, _, o0, lse0 = _decode(wl, S, q=torch.zeros_like(t["q"]))
    cnt = Nk - Lq + 1 + np.arange(Lq)
    assert np.max(np.abs(f64(lse0) - np.log(cnt)[None, None])) <= COUNT_LSE_TOL


def test_planted_peak_decode():
    """Scaled queries aligned with one key per page make O dominated by those V rows, so an
    O error (not only an LSE error) becomes visible."""
    announce("planted peak")
    wl = W.paged_decode("peak", 1, 4, 1, 3, 640, 128, page_size=16, pool_pages=50, seed=6)
    t = wl.tensors
    kl = t["k_logical"]
    # query i copies key (100 + 200 i) scaled by 8
    q = torch.stack([kl[0, 0, 100 + 200 * i].float() * 8 for i in range(3)]).to(torch.bfloat16)
    q = q[None, None].expand(1, 4, 3, 128).contiguous()
    ws_o, ws_l, o, lse = _decode(wl, 3, q=q)
    bt = t["block_table"].numpy()
    kk = OP.gather(f64(t["k_pool"]), bt, 0, 640)[None]
    vv = OP.gather(f64(t["v_pool"]), bt, 0, 640)[None]
    ro, rl = oracle.attention(f64(q), kk, vv, wl.scale, M.causal(3, 640))
    assert np.max(np.abs(ro)) > 0.5  # the peak dominates
    assert_close(f64(o), f64(lse), ro, rl, "planted peak")
