"""The C-ABI library loads, exports every symbol include/tiled_attn.h declares, and
rejects bad arguments on the host before any launch (no GPU needed: no compute call
is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tiled_attn.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def T():
    import tiled_attention_attn_amd as T
    return T


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("attn_fwd", "attn_fwd_blockmask", "attn_build_blockmask", "attn_decode_splitkv",
              "attn_decode_combine"):
        assert n in names


def test_library_exports_every_declared_symbol(T):
    lib = ctypes.CDLL(T.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(T.EXPORTS)


def test_status_strings(T):
    assert T.attn_status_str(0) == "ok"
    for code in range(-13, 0):
        assert T.attn_status_str(code) != "unknown status"
    assert T.attn_abi_version() >= 1


def _strides(*v):
    return (ctypes.c_int64 * 3)(*v)


def _fwd(T, **kw):
    lib = T.lib_handle()
    a = dict(q=16, k=32, v=48, o=64, qs=(64 * 256, 64 * 256, 64), ks=None, vs=None, os=None, lse=None,
             B=1, Hq=1, Hkv=1, Nq=256, Nk=256, D=64, dtype=0, scale=0.125, mask=None, smod=None)
    a.update(kw)
    s = lambda x: _strides(*(x or a["qs"]))
    mk = None if a["mask"] is None else ctypes.byref(a["mask"])
    sm = None if a["smod"] is None else ctypes.byref(a["smod"])
    return lib.attn_fwd(a["q"], s(a["qs"]), a["k"], s(a["ks"]), a["v"], s(a["vs"]), a["o"], s(a["os"]),
                        a["lse"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["D"], a["dtype"], a["scale"],
                        mk, sm, None)


def test_fwd_argument_errors(T):
    # every case fails validation, so nothing is launched
    assert _fwd(T, q=None) == -1
    assert _fwd(T, k=None) == -1
    assert _fwd(T, D=96) == -3
    assert _fwd(T, dtype=2) == -12 and _fwd(T, dtype=-1) == -12
    SMD = T.attn_score_mod
    qs128 = (128 * 256, 128 * 256, 128)
    f128 = lambda **kw: _fwd(T, D=128, qs=qs128, **kw)
    assert f128(smod=SMD(flags=16)) == -13                                   # unknown flag
    for cap in (0.0, -3.0, float("inf"), float("nan")):                      # SOFTCAP needs a cap > 0
        assert f128(smod=SMD(flags=8, softcap=cap)) == -13
    assert _fwd(T, smod=SMD(flags=8, softcap=30.0), B=0) == 0               # D = 64 takes a cap
    assert f128(smod=SMD(flags=3, slopes=16)) == -13                         # ALIBI and ALIBI_SYM
    assert f128(smod=SMD(flags=1, slopes=None)) == -1
    assert f128(smod=SMD(flags=4, rel_bias=None, rel_radius=3)) == -1
    assert f128(smod=SMD(flags=4, rel_bias=16, rel_radius=1024)) == -13     # 2R+1 > 2048
    assert f128(smod=SMD(flags=4, rel_bias=16, rel_radius=-1)) == -13
    assert _fwd(T, smod=SMD(flags=1, slopes=16), B=0) == 0                  # and ALiBi (validated, B = 0)
    assert f128(smod=SMD(flags=0), B=0) == 0
    assert _fwd(T, Hq=3, Hkv=2) == -4
    assert _fwd(T, Hkv=0) == -4
    assert _fwd(T, qs=(64 * 256, 64 * 256, 60)) == -5
    assert _fwd(T, ks=(1 << 30, 1 << 30, 1 << 24)) == -5  # 128-row tiles, 32-bit offsets
    assert _fwd(T, q=18) == -6
    assert _fwd(T, Nq=-1) == -2
    assert _fwd(T, scale=0.0) == -11
    assert _fwd(T, scale=float("nan")) == -11
    m = T.attn_mask_desc(flags=64)
    assert _fwd(T, mask=m) == -7
    m = T.attn_mask_desc(flags=T.MASK_BLOCK_CAUSAL, block_size=0)
    assert _fwd(T, mask=m) == -7
    m = T.attn_mask_desc(flags=T.MASK_DOCUMENT, doc_offsets=None, num_docs=1, doc_stride=2)
    assert _fwd(T, mask=m) == -1
    m = T.attn_mask_desc(flags=T.MASK_DOCUMENT, doc_offsets=1024, num_docs=2, doc_stride=2)
    assert _fwd(T, mask=m) == -7
    m = T.attn_mask_desc(flags=T.MASK_DOCUMENT, doc_offsets=1024, num_docs=1, doc_stride=2)
    assert _fwd(T, mask=m, Nq=300, Nk=256) == -7


def test_schedule_flags_are_accepted_beside_the_mask(T):
    m = T.attn_mask_desc(flags=T.MASK_CAUSAL | T.SCHED_ALL)
    assert _fwd(T, Nq=0, mask=m) == 0                                # accepted, nothing to launch
    assert _fwd(T, Nq=0, mask=T.attn_mask_desc(flags=1 << 20)) == -7
    with pytest.raises(ValueError):
        T.Mask(causal=True, schedule=1 << 20).desc()


def test_empty_problems_launch_nothing(T):
    # B = 0 or Nq = 0: valid, nothing to do, returns OK without touching the GPU
    assert _fwd(T, B=0) == 0
    assert _fwd(T, Nq=0) == 0


def test_blockmask_and_decode_argument_errors(T):
    lib = T.lib_handle()
    bm = T.attn_blockmask(Bm=1, Hm=1, nQt=2, nKt=2, part_num=16, part_idx=32, full_num=48, full_idx=64)
    assert lib.attn_build_blockmask(None, None, 1, 256, 256, ctypes.byref(bm), None) == -1  # no map, no mask
    bad = T.attn_blockmask(Bm=1, Hm=1, nQt=3, nKt=2, part_num=16, part_idx=32, full_num=48, full_idx=64)
    m = T.attn_mask_desc(flags=T.MASK_CAUSAL)
    assert lib.attn_build_blockmask(ctypes.byref(m), None, 1, 256, 256, ctypes.byref(bad), None) == -10
    assert lib.attn_blockmask_bytes(1, 1, 2, 2) == 2 * 4 * 2 + 2 * 2 * 4 * 2
    qs = _strides(32 * 16 * 128, 16 * 128, 128)
    args = lambda **kw: dict(dict(q=16, qs=qs, kc=32, vc=48, pages=10, bt=64, bts=4, sl=80, maxp=4, B=1,
                                  Hq=4, Hkv=2, Lq=2, D=128, dt=0, ps=16, S=2, scale=0.1, mask=None, wo=96,
                                  wl=112, smod=None), **kw)

    def dec(**kw):
        a = args(**kw)
        mk = None if a["mask"] is None else ctypes.byref(a["mask"])
        sm = None if a["smod"] is None else ctypes.byref(a["smod"])
        return lib.attn_decode_splitkv(a["q"], a["qs"], a["kc"], a["vc"], a["pages"], a["bt"], a["bts"],
                                       a["sl"], a["maxp"], a["B"], a["Hq"], a["Hkv"], a["Lq"], a["D"],
                                       a["dt"], a["ps"], a["S"], a["scale"], mk, sm, a["wo"], a["wl"], None)
    assert dec(wo=None) == -1
    assert dec(S=0) == -8
    assert dec(bts=3) == -2
    assert dec(D=80) == -3
    assert dec(dt=5) == -12
    assert dec(smod=T.attn_score_mod(flags=4, rel_bias=16, rel_radius=1024)) == -13  # 2R + 1 > 2048
    assert dec(smod=T.attn_score_mod(flags=4, rel_bias=None, rel_radius=2)) == -1
    assert dec(smod=T.attn_score_mod(flags=8, softcap=0.0)) == -13
    assert dec(Hq=3) == -4
    md = T.attn_mask_desc(flags=T.MASK_DOCUMENT, doc_offsets=16, num_docs=1, doc_stride=2)
    assert dec(mask=md) == -7
    assert dec(B=0) == 0
    assert lib.attn_decode_combine(None, 16, 1, 1, 1, 1, 64, 0, 32, qs, None, None) == -1
    assert lib.attn_decode_combine(16, 16, 1, 1, 1, 0, 64, 0, 32, qs, None, None) == -8
    assert lib.attn_decode_combine(16, 16, 1, 1, 1, 1, 64, 3, 32, qs, None, None) == -12
    assert lib.attn_decode_num_splits(16, 8, 2048, 256) == 4   # two work groups per CU
    assert lib.attn_decode_num_splits(1, 1, 3, 256) == 3        # never more splits than pages
    assert lib.attn_decode_num_splits(1, 300, 10000, 256) == 5  # at most 2048 pages per split
    assert dec(S=1, maxp=4097, bts=4097) == -8                  # 4097 pages in one split
    assert dec(Hq=65536 * 2, Hkv=2) == -2                       # Hq bounded like every entry point
    # the allocation-free variant: partials beyond its static buffer are refused before any launch
    assert lib.attn_decode_noalloc_max_bytes() == 32 << 20

    def dec_na(**kw):
        a = args(**kw)
        return lib.attn_decode_noalloc(a["q"], a["qs"], a["kc"], a["vc"], a["pages"], a["bt"], a["bts"],
                                       a["sl"], a["maxp"], a["B"], a["Hq"], a["Hkv"], a["Lq"], a["D"],
                                       a["dt"], a["ps"], a["S"], a["scale"], None, None, 128, qs, None,
                                       None)
    assert dec_na(B=16, Hq=32, Hkv=8, Lq=16, S=8) == -8    # 16*32*16*8*129*4 B > 32 MiB
    assert dec_na(B=16, Hq=32, Hkv=8, Lq=16, S=65536) == -8
    assert dec_na(S=0) == -8
    assert dec_na(D=80) == -3
    assert lib.attn_decode_noalloc(16, qs, 32, 48, 10, 64, 4, 80, 4, 1, 4, 2, 2, 128, 0, 16, 2, 0.1,
                                   None, None, None, qs, None, None) == -1      # no output
    assert lib.attn_decode_noalloc(16, qs, 32, 48, 10, 64, 4, 80, 4, 1, 4, 2, 2, 128, 0, 16, 2, 0.1,
                                   None, None, 8, qs, None, None) == -6         # misaligned output
    assert dec(Hq=60000, Hkv=1, Lq=65536) == -2                 # G * Lq rows kept inside int
    assert lib.attn_decode_ws_o_bytes(16, 32, 16, 128, 4) == 16 * 32 * 16 * 4 * 128 * 4



def test_extreme_sizes_are_rejected_without_overflow(T):
    """Sizes whose products pass 32 or 64 bits: the checks compute them without overflow
    (cases found by the UBSan run of tests/test_host_ub.py) and refuse them before any
    launch, or the size helpers answer 0 ("invalid sizes")."""
    lib = T.lib_handle()
    IMAX = 2**31 - 1
    qs = _strides(32 * 16 * 128, 16 * 128, 128)
    # num_docs + 1 and 2 * rel_radius + 1 at INT_MAX
    md = T.attn_mask_desc(flags=T.MASK_DOCUMENT, doc_offsets=16, num_docs=IMAX, doc_stride=IMAX)
    assert lib.attn_fwd(16, qs, 32, qs, 48, qs, 64, qs, None, 1, 4, 4, 16, 16, 128, 0, 0.1,
                        ctypes.byref(md), None, None) == -7
    sm = T.attn_score_mod(flags=T.SCORE_REL_BIAS, rel_bias=16, rel_radius=IMAX)
    assert lib.attn_fwd(16, qs, 32, qs, 48, qs, 64, qs, None, 1, 4, 4, 16, 16, 128, 0, 0.1, None,
                        ctypes.byref(sm), None) == -13
    # size helpers: products beyond 2^64 give 0
    assert lib.attn_decode_ws_o_bytes(IMAX, IMAX, IMAX, 128, 65536) == 0
    assert lib.attn_decode_ws_lse_bytes(IMAX, IMAX, IMAX, IMAX) == 0
    assert lib.attn_bwd_workspace_bytes(IMAX, IMAX, IMAX) == 0
    assert lib.attn_blockmask_bytes(65535, 65535, 2**21, 2**21) == 0
    assert lib.attn_blockmask_bytes(1, 1, 256, 256) == 256 * 8 + 256 * 256 * 8
    assert lib.attn_decode_num_splits(1, 1, IMAX, 256) == -(-IMAX // 2048)
    # split-KV partials of more bytes than a size_t holds: no workspace can exist
    assert lib.attn_decode_splitkv(16, qs, 32, 48, 10, 64, 65536, 80, 65536, 65535, 65535, 65535, 65536,
                                   128, 0, 16, 65536, 0.1, None, None, 96, 112, None) == -2
    # combine: B * Hq * Lq past 2^31 - 4 rows (the product itself past 2^63 too)
    assert lib.attn_decode_combine(16, 16, IMAX, IMAX, IMAX, 1, 64, 0, 32, qs, None, None) == -2
    assert lib.attn_decode_combine(16, 16, 1, 1, IMAX - 2, 1, 64, 0, 32, qs, None, None) == -2
    # transposition of a map with more than 2^64 entries
    bm = T.attn_blockmask(Bm=65535, Hm=65535, nQt=2**21, nKt=2**21, part_num=16, part_idx=32,
                          full_num=48, full_idx=64)
    bt = T.attn_blockmask(Bm=65535, Hm=65535, nQt=2**21, nKt=2**21, part_num=16, part_idx=32,
                          full_num=48, full_idx=64)
    assert lib.attn_blockmask_transpose(ctypes.byref(bm), ctypes.byref(bt), 16, 2**63, None) == -10
    # a decode-shaped auto call whose combine would number more than 2^31 - 4 rows stays on
    # the prefill path; one just below the bound takes split-KV
    P = T.attn_fwd_auto_plan
    assert P(65535, 65535, 65535, 1, 512, 64).path == T.PATH_PREFILL
    assert P(32767, 65535, 65535, 1, 512, 64).path == T.PATH_SPLITKV

def test_bwd_argument_errors(T):
    lib = T.lib_handle()
    qs = _strides(64 * 256, 64 * 256, 64)
    ws = T.attn_bwd_workspace_bytes(1, 1, 256)
    assert ws == 2 * 256 * 4 and T.attn_bwd_workspace_bytes(2, 3, 65) == 2 * 2 * 3 * 128 * 4

    def bwd(**kw):
        a = dict(q=16, k=32, v=48, o=64, do=80, lse=96, dq=112, dk=128, dv=144, s=qs, ks=qs, B=1, Hq=1,
                 Hkv=1, Nq=256, Nk=256, D=64, dt=1, scale=0.125, mask=None, ws=160, wsb=ws, smod=None)
        a.update(kw)
        mk = None if a["mask"] is None else ctypes.byref(a["mask"])
        sm = None if a["smod"] is None else ctypes.byref(a["smod"])
        s, ks = a["s"], a["ks"]
        return lib.attn_bwd(a["q"], s, a["k"], ks, a["v"], s, a["o"], s, a["do"], s, a["lse"], a["dq"], s,
                            a["dk"], s, a["dv"], s, a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["D"],
                            a["dt"], a["scale"], mk, sm, a["ws"], a["wsb"], None)
    assert bwd(do=None) == -1
    assert bwd(lse=None) == -1
    assert bwd(dk=None) == -1
    assert bwd(ws=None) == -1
    assert bwd(D=32) == -3
    assert bwd(dt=7) == -12
    # G (2R + 1) bias-table floats over 8192 for one work group
    q128 = _strides(128 * 256, 128 * 256, 128)
    assert bwd(D=128, s=q128, ks=q128, Hq=8, Hkv=1,
               smod=T.attn_score_mod(flags=4, rel_bias=16, rel_radius=512)) == -13
    assert bwd(smod=T.attn_score_mod(flags=1, slopes=16), B=0) == 0   # D = 64 takes a score change
    assert bwd(Hq=2, Hkv=3) == -4
    assert bwd(s=_strides(64 * 256, 64 * 256, 68)) == -5
    assert bwd(ks=_strides(1 << 30, 1 << 30, 1 << 24)) == -5  # streamed row stride over 2^24
    assert bwd(dv=150) == -6
    assert bwd(scale=-1.0) == -11
    assert bwd(mask=T.attn_mask_desc(flags=32)) == -7
    assert bwd(mask=T.attn_mask_desc(flags=1 << 19)) == -7           # not a schedule bit either
    assert bwd(wsb=ws - 4) == -8
    assert bwd(B=0) == 0
    # no rows and no keys: nothing to compute; row-less tensors may be NULL
    assert bwd(Nq=0, Nk=0, q=None, o=None, do=None, dq=None, lse=None, ws=None, k=None, v=None,
               dk=None, dv=None) == 0


def test_bwd_blockmask_and_transpose_argument_errors(T):
    lib = T.lib_handle()
    qs = _strides(64 * 256, 64 * 256, 64)
    ws = T.attn_bwd_workspace_bytes(1, 1, 256)
    BM = T.attn_blockmask

    def lists(Bm=1, Hm=1, nQt=2, nKt=2, base=512, **kw):
        a = dict(part_num=base, part_idx=base + 16, full_num=base + 32, full_idx=base + 48)
        a.update(kw)
        return BM(Bm=Bm, Hm=Hm, nQt=nQt, nKt=nKt, **a)

    def bwd(bm="d", bm_t="d", **kw):
        a = dict(B=1, Hq=1, Hkv=1, Nq=256, Nk=256, D=64, smod=None, wsb=ws)
        a.update(kw)
        bm = lists() if bm == "d" else bm
        bm_t = lists(base=1024) if bm_t == "d" else bm_t
        sm = None if a["smod"] is None else ctypes.byref(a["smod"])
        ref = lambda x: None if x is None else ctypes.byref(x)
        return lib.attn_bwd_blockmask(16, qs, 32, qs, 48, qs, 64, qs, 80, qs, 96, 112, qs, 128, qs, 144, qs,
                                      a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["D"], 0, 0.125, None, sm,
                                      ref(bm), ref(bm_t), 160, a["wsb"], None)
    assert bwd(bm=None) == -1 and bwd(bm_t=None) == -1
    assert bwd(bm_t=lists(base=1024, full_idx=None)) == -1
    assert bwd(bm=lists(nQt=3)) == -10                     # tile counts must match Nq / Nk
    assert bwd(bm=lists(Bm=2)) == -10                      # Bm is 1 or B
    assert bwd(bm_t=lists(base=1024, Hm=2)) == -10         # the transpose must match bm
    assert bwd(bm=lists(nKt=3), bm_t=lists(base=1024, nKt=3), Nk=300) == -10  # bm_t is bm's nKt x nQt
    assert bwd(smod=T.attn_score_mod(flags=1, slopes=16)) == -13  # no score change on this path
    assert bwd(D=96) == -3
    assert bwd(wsb=ws - 4) == -8
    assert bwd(B=0) == 0
    tp = lambda bm, out, tmp=2048, n=1 << 20: lib.attn_blockmask_transpose(
        None if bm is None else ctypes.byref(bm), None if out is None else ctypes.byref(out), tmp, n, None)
    assert tp(None, lists()) == -1 and tp(lists(), None) == -1
    assert tp(lists(nQt=3, nKt=2), lists(base=1024, nQt=3, nKt=2)) == -10   # out must be nKt x nQt
    assert tp(lists(Hm=2), lists(base=1024)) == -10
    assert tp(lists(), lists(base=1024), tmp=None) == -1
    assert tp(lists(), lists(base=1024), n=3) == -8                           # map_tmp holds 4 bytes
    assert tp(lists(nQt=0, nKt=0), lists(base=1024, nQt=0, nKt=0), tmp=None) == 0


def test_grids_beyond_the_launch_limit_are_rejected(T):
    """Shapes whose work-group count passes 2^31 - 1 fail on the host (ATTN_ERR_SHAPE)
    instead of launching a truncated grid."""
    big = dict(B=65535, Hq=65535, Hkv=65535, Nq=1 << 20, Nk=256)
    assert _fwd(T, **big) == -2
    lib = T.lib_handle()
    qs = _strides(64 * 256, 64 * 256, 64)
    bm = T.attn_blockmask(Bm=1, Hm=1, nQt=(1 << 20) // 128, nKt=2, part_num=16, part_idx=32, full_num=48,
                          full_idx=64)
    assert lib.attn_fwd_blockmask(16, qs, 32, qs, 48, qs, 64, qs, None, 65535, 65535, 65535, 1 << 20, 256, 64,
                                  0, 0.125, None, None, ctypes.byref(bm), None) == -2
    assert lib.attn_bwd(16, qs, 32, qs, 48, qs, 64, qs, 80, qs, 96, 112, qs, 128, qs, 144, qs,
                        65535, 65535, 65535, 1 << 20, 256, 64, 0, 0.125, None, None, 160, 1 << 62, None) == -2
    # just inside the limit the same calls would launch, so they are not made here


def test_auto_plan_rule(T):
    """attn_fwd_auto's choice: split-KV for G * Nq <= 64 rows per KV head and Nk >= 512;
    the split count targets 512 work groups with >= 256 keys each,
    in whole 64-key steps; workspace = fp32 partial O (padded to 256 B) + partial LSE."""
    P = T.attn_fwd_auto_plan
    pl = P(16, 32, 8, 16, 32768, 128)
    assert (pl.path, pl.num_splits) == (T.PATH_SPLITKV, 4)
    parts = 16 * 32 * 16 * 4
    assert pl.workspace_bytes == parts * 128 * 4 + parts * 4
    assert P(1, 32, 8, 16, 32768, 128).num_splits == 64      # 8 units: 64 splits of 512 keys
    assert P(1, 1, 1, 1, 1000, 64).num_splits == 3           # <= Nk / 256 splits, chunks of 384
    assert P(128, 32, 8, 1, 4096, 128).num_splits == 1       # 1024 units already fill the GPU
    assert P(1, 8, 8, 1, 512, 64).path == T.PATH_SPLITKV
    assert P(1, 8, 8, 1, 511, 64).path == T.PATH_PREFILL     # too few keys
    assert P(16, 32, 8, 17, 32768, 128).path == T.PATH_PREFILL  # 68 rows per KV head
    assert P(1, 64, 1, 1, 32768, 128).path == T.PATH_SPLITKV    # G = 64, one row each
    assert P(2, 16, 16, 4096, 4096, 64).path == T.PATH_PREFILL
    assert P(1, 8, 8, 0, 4096, 64).path == T.PATH_PREFILL
    rel = T.attn_score_mod(flags=T.SCORE_REL_BIAS, rel_bias=16, rel_radius=4)
    assert P(16, 32, 8, 16, 32768, 128, rel).path == T.PATH_SPLITKV   # every score change runs on both
    ali = T.attn_score_mod(flags=T.SCORE_ALIBI, slopes=16)
    assert P(16, 32, 8, 16, 32768, 128, ali).path == T.PATH_SPLITKV
    for B, Hq, Hkv, Nq, Nk in [(3, 12, 4, 5, 700), (1, 2, 1, 32, 99999), (7, 8, 2, 16, 4097)]:
        pl = P(B, Hq, Hkv, Nq, Nk, 64)
        assert pl.path == T.PATH_SPLITKV
        chunk = (-(-Nk // pl.num_splits) + 63) // 64 * 64
        assert -(-Nk // chunk) == pl.num_splits and (pl.num_splits - 1) * chunk < Nk
    lib = T.lib_handle()
    assert lib.attn_fwd_auto_plan(1, 4, 3, 1, 1, 64, None, ctypes.byref(T.attn_auto_plan())) == -4
    assert lib.attn_fwd_auto_plan(1, 4, 4, 1, 1, 96, None, ctypes.byref(T.attn_auto_plan())) == -3
    assert lib.attn_fwd_auto_plan(-1, 4, 4, 1, 1, 64, None, ctypes.byref(T.attn_auto_plan())) == -2
    assert lib.attn_fwd_auto_plan(1, 4, 4, 1, 1, 64, None, None) == -1


def test_auto_argument_errors(T):
    lib = T.lib_handle()
    qs = _strides(32 * 16 * 128, 16 * 128, 128)
    ks = _strides(8 * 4096 * 128, 4096 * 128, 128)
    need = T.attn_fwd_auto_plan(2, 32, 8, 16, 4096, 128).workspace_bytes

    def auto(**kw):
        a = dict(q=16, k=32, v=48, o=64, lse=None, B=2, Hq=32, Hkv=8, Nq=16, Nk=4096, D=128, dt=0,
                 scale=0.1, mask=None, smod=None, ws=80, wsb=need)
        a.update(kw)
        mk = None if a["mask"] is None else ctypes.byref(a["mask"])
        sm = None if a["smod"] is None else ctypes.byref(a["smod"])
        return lib.attn_fwd_auto(a["q"], qs, a["k"], ks, a["v"], ks, a["o"], qs, a["lse"], a["B"], a["Hq"],
                                 a["Hkv"], a["Nq"], a["Nk"], a["D"], a["dt"], a["scale"], mk, sm, a["ws"],
                                 a["wsb"], None)
    assert auto(ws=None) == -1
    assert auto(wsb=need - 1) == -8
    assert auto(ws=88) == -6
    assert auto(k=None) == -1
    assert auto(D=80) == -3
    assert auto(dt=4) == -12
    assert auto(Hkv=5) == -4
    assert auto(scale=float("nan")) == -11
    assert auto(mask=T.attn_mask_desc(flags=64)) == -7
    assert auto(smod=T.attn_score_mod(flags=1, slopes=None)) == -1
    # the prefill path keeps attn_fwd's rules: a score change at D = 64 is validated like any other
    assert auto(Nq=4096, D=64, smod=T.attn_score_mod(flags=16)) == -13
    assert auto(Nq=4096, D=64, B=0, smod=T.attn_score_mod(flags=1, slopes=16)) == 0
    assert auto(B=0) == 0 and auto(Nq=0, ws=None) == 0


def test_product_path_does_not_reach_the_oracle():
    """The package and its C sources never import or include the oracle or the workloads."""
    pkg = os.path.join(ROOT, "tiled_attention_attn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.replace("Oracle", ""), f
                assert "import workloads" not in src and "from workloads" not in src, f


def test_binding_rejects_bad_tensors_before_any_call(T):
    """The Python binding checks every tensor argument the C ABI cannot see (shapes the
    kernels index with, one slope / table row per query head, a block-table row per
    sequence, device placement) and raises before calling into the library.  CPU
    tensors reach the shape checks first, then fail the device check."""
    import torch
    bf = dict(dtype=torch.bfloat16)
    q = torch.zeros(1, 4, 64, 64, **bf)
    k = torch.zeros(1, 2, 64, 64, **bf)
    o = torch.zeros_like(q)
    lse = torch.zeros(1, 4, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        T.attn_fwd(q, k, k, o, lse)                                # all on the CPU
    with pytest.raises(ValueError, match="shape"):
        T.attn_fwd(q, k, torch.zeros(1, 2, 63, 64, **bf), o)      # v != k
    with pytest.raises(ValueError, match="shape"):
        T.attn_fwd(q, k, k, torch.zeros(1, 4, 64, 128, **bf))      # o != q
    with pytest.raises(ValueError, match="shape"):
        T.attn_fwd(q, k, k, o, torch.zeros(1, 4, 65))               # lse rows
    with pytest.raises(TypeError, match="lse"):
        T.attn_fwd(q, k, k, o, torch.zeros(1, 4, 64, dtype=torch.float64))
    with pytest.raises(ValueError, match="alibi_slopes"):
        T.attn_fwd(q, k, k, o, lse, smod=T.ScoreMod(alibi_slopes=torch.zeros(3)))
    with pytest.raises(ValueError, match="rel_bias"):
        T.attn_fwd(q, k, k, o, lse, smod=T.ScoreMod(rel_bias=torch.zeros(2, 9)))
    with pytest.raises(ValueError, match="doc_offsets"):
        T.attn_fwd(q, k, k, o, lse, mask=T.Mask(doc_offsets=torch.zeros(2, 3, dtype=torch.int32)))
    # backward: gradients shaped like their inputs, lse required
    with pytest.raises(ValueError, match="shape"):
        T.attn_bwd(q, k, k, o, q, lse, q, torch.zeros(1, 4, 64, 64, **bf), k)
    with pytest.raises(TypeError, match="lse"):
        T.attn_bwd(q, k, k, o, q, None, q, k, k)
    # decode: block table and seq_lens cover every sequence
    qd = torch.zeros(3, 4, 2, 64, **bf)
    pool = torch.zeros(10, 16, 2, 64, **bf)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    sl = torch.zeros(3, dtype=torch.int32)
    ws_o, ws_l = torch.zeros(3, 4, 2, 2, 64), torch.zeros(3, 4, 2, 2)
    with pytest.raises(ValueError, match="block_table"):
        T.attn_decode_splitkv(qd, pool, pool, bt, sl, 4, 2, ws_o, ws_l)
    with pytest.raises(ValueError, match="seq_lens"):
        T.attn_decode_splitkv(qd, pool, pool, torch.zeros(3, 4, dtype=torch.int32), sl[:2], 4, 2,
                              ws_o, ws_l)
    with pytest.raises(ValueError, match="GPU tensor"):
        T.attn_decode_splitkv(qd, pool, pool, torch.zeros(3, 4, dtype=torch.int32), sl, 4, 2,
                              ws_o, ws_l)
    with pytest.raises(ValueError, match="shape"):
        T.attn_decode_combine(ws_o, ws_l, torch.zeros(3, 4, 2, 128, **bf))
    with pytest.raises(ValueError, match="shape"):
        T.attn_decode_combine(ws_o, torch.zeros(3, 4, 2, 3), torch.zeros(3, 4, 2, 64, **bf))


def test_header_compiles_as_c_and_matches_the_binding(T, tmp_path):
    """tests/abi_from_c.c, plain C11 built with gcc -Wall -Wextra -Werror against the
    header and linked against the library, reports the header's struct layouts,
    constants and a few host-only results; each must equal what the ctypes binding
    uses, so a field or constant changed on one side only fails here."""
    import json
    import shutil
    import subprocess
    from tiled_attention_attn_amd import _lib as L
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("needs gcc")
    pkg = os.path.dirname(T.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "abi_from_c.c"), "-L", pkg, "-ltiled_attn",
           f"-Wl,-rpath,{pkg}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = json.loads(subprocess.run([exe], capture_output=True, text=True, check=True).stdout)

    for cname, cls in (("attn_mask_desc", L.attn_mask_desc), ("attn_score_mod", L.attn_score_mod),
                       ("attn_blockmask", L.attn_blockmask), ("attn_auto_plan", L.attn_auto_plan)):
        assert out[f"sizeof {cname}"] == ctypes.sizeof(cls), cname
        c_fields = {k.split(".", 1)[1] for k in out if k.startswith(cname + ".")}
        assert c_fields == {f for f, _ in cls._fields_}, cname
        for f, _ in cls._fields_:
            fld = getattr(cls, f)
            assert out[f"{cname}.{f}"] == [fld.offset, fld.size], f"{cname}.{f}"

    for c, py in (("ATTN_DTYPE_BF16", T.DTYPE_BF16), ("ATTN_DTYPE_F16", T.DTYPE_F16),
                  ("ATTN_MASK_CAUSAL", L.MASK_CAUSAL), ("ATTN_MASK_WINDOW", L.MASK_WINDOW),
                  ("ATTN_MASK_DOCUMENT", L.MASK_DOCUMENT), ("ATTN_MASK_BLOCK_CAUSAL", L.MASK_BLOCK_CAUSAL),
                  ("ATTN_SCHED_NO_PAIRING", L.SCHED_NO_PAIRING), ("ATTN_SCHED_NO_XCD_REMAP", L.SCHED_NO_XCD_REMAP),
                  ("ATTN_SCHED_REVERSE", L.SCHED_REVERSE), ("ATTN_SCORE_ALIBI", L.SCORE_ALIBI),
                  ("ATTN_SCORE_ALIBI_SYM", L.SCORE_ALIBI_SYM), ("ATTN_SCORE_REL_BIAS", L.SCORE_REL_BIAS),
                  ("ATTN_SCORE_SOFTCAP", L.SCORE_SOFTCAP), ("ATTN_BLOCKMASK_TILE", L.BLOCKMASK_TILE),
                  ("ATTN_PATH_PREFILL", L.PATH_PREFILL), ("ATTN_PATH_SPLITKV", L.PATH_SPLITKV)):
        assert out[c] == py, c

    lib = T.lib_handle()
    assert out["fwd_null"] == out["ATTN_ERR_NULL"]
    plan = L.attn_auto_plan()
    assert lib.attn_fwd_auto_plan(16, 32, 8, 16, 32768, 128, None, ctypes.byref(plan)) == 0
    assert out["plan"] == [0, plan.path, plan.num_splits, plan.workspace_bytes]
    assert out["plan"][1] == out["ATTN_PATH_SPLITKV"]
    assert out["bwd_ws"] == T.attn_bwd_workspace_bytes(2, 16, 4096)
    assert out["bm_bytes"] == T.attn_blockmask_bytes(1, 1, 256, 256)
    assert out["noalloc_max"] == T.attn_decode_noalloc_max_bytes()
    assert out["status_head_dim"] == T.attn_status_str(out["ATTN_ERR_HEAD_DIM"])
