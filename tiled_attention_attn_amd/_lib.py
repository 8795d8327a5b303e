"""ctypes binding of libtiled_attn.so (include/tiled_attn.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI.  Functions keep the C names; torch tensors (on the
GPU) supply the device pointers, shapes and element strides, and the current
torch stream is used unless one is passed.  A non-zero status raises
``AttnError`` with the library's own message.  If the library is missing the
import fails: there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtiled_attn.so")

DTYPE_BF16 = 0
DTYPE_F16 = 1
_DTYPES = {torch.bfloat16: DTYPE_BF16, torch.float16: DTYPE_F16}

MASK_CAUSAL = 1
MASK_WINDOW = 2
MASK_DOCUMENT = 4
MASK_BLOCK_CAUSAL = 8
SCHED_NO_PAIRING = 1 << 16
SCHED_NO_XCD_REMAP = 1 << 17
SCHED_REVERSE = 1 << 18
SCHED_ALL = SCHED_NO_PAIRING | SCHED_NO_XCD_REMAP | SCHED_REVERSE
BLOCKMASK_TILE = 128
TILE_EMPTY, TILE_PARTIAL, TILE_FULL = 0, 1, 2


class AttnError(RuntimeError):
    def __init__(self, func: str, status: int, msg: str):
        super().__init__(f"{func}: status {status}: {msg}")
        self.status = status


class attn_mask_desc(ctypes.Structure):
    _fields_ = [
        ("flags", ctypes.c_uint32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("doc_offsets", ctypes.c_void_p),
        ("num_docs", ctypes.c_int32),
        ("doc_stride", ctypes.c_int32),
    ]


class attn_score_mod(ctypes.Structure):
    _fields_ = [
        ("flags", ctypes.c_uint32),
        ("slopes", ctypes.c_void_p),
        ("rel_bias", ctypes.c_void_p),
        ("rel_radius", ctypes.c_int32),
        ("softcap", ctypes.c_float),
    ]


SCORE_ALIBI = 1
SCORE_ALIBI_SYM = 2
SCORE_REL_BIAS = 4
SCORE_SOFTCAP = 8


PATH_PREFILL = 0
PATH_SPLITKV = 1


class attn_auto_plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)]


class attn_blockmask(ctypes.Structure):
    _fields_ = [
        ("Bm", ctypes.c_int32), ("Hm", ctypes.c_int32),
        ("nQt", ctypes.c_int32), ("nKt", ctypes.c_int32),
        ("part_num", ctypes.c_void_p), ("part_idx", ctypes.c_void_p),
        ("full_num", ctypes.c_void_p), ("full_idx", ctypes.c_void_p),
    ]


def declare_signatures(lib):
    """Sets the C ABI's argument and result types on a loaded copy of the library."""
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    I64 = ctypes.c_int64
    STR = ctypes.POINTER(ctypes.c_int64)
    MP = ctypes.POINTER(attn_mask_desc)
    SP = ctypes.POINTER(attn_score_mod)
    BP = ctypes.POINTER(attn_blockmask)
    sig = {
        "attn_fwd": (I, [P, STR, P, STR, P, STR, P, STR, P, I, I, I, I, I, I, I, F, MP, SP, P]),
        "attn_fwd_blockmask": (I, [P, STR, P, STR, P, STR, P, STR, P, I, I, I, I, I, I, I, F, MP, SP, BP, P]),
        "attn_build_blockmask": (I, [MP, P, I, I, I, BP, P]),
        "attn_blockmask_bytes": (S, [I, I, I, I]),
        "attn_decode_splitkv": (I, [P, STR, P, P, I64, P, I64, P, I, I, I, I, I, I, I, I, I, F, MP, SP, P, P, P]),
        "attn_decode_combine": (I, [P, P, I, I, I, I, I, I, P, STR, P, P]),
        "attn_decode_noalloc": (I, [P, STR, P, P, I64, P, I64, P, I, I, I, I, I, I, I, I, I, F, MP, SP,
                                    P, STR, P, P]),
        "attn_decode_noalloc_max_bytes": (S, []),
        "attn_decode_ws_o_bytes": (S, [I, I, I, I, I]),
        "attn_decode_ws_lse_bytes": (S, [I, I, I, I]),
        "attn_decode_num_splits": (I, [I, I, I, I]),
        "attn_bwd": (I, [P, STR, P, STR, P, STR, P, STR, P, STR, P, P, STR, P, STR, P, STR,
                         I, I, I, I, I, I, I, F, MP, SP, P, S, P]),
        "attn_bwd_workspace_bytes": (S, [I, I, I]),
        "attn_bwd_blockmask": (I, [P, STR, P, STR, P, STR, P, STR, P, STR, P, P, STR, P, STR, P, STR,
                                   I, I, I, I, I, I, I, F, MP, SP, BP, BP, P, S, P]),
        "attn_blockmask_transpose": (I, [BP, BP, P, S, P]),
        "attn_fwd_auto_plan": (I, [I, I, I, I, I, I, SP, ctypes.POINTER(attn_auto_plan)]),
        "attn_fwd_auto": (I, [P, STR, P, STR, P, STR, P, STR, P, I, I, I, I, I, I, I, F, MP, SP, P, S, P]),
        "attn_probe_stream_read": (I, [P, S, I, P, P]),
        "attn_status_str": (ctypes.c_char_p, [I]),
        "attn_abi_version": (I, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    return declare_signatures(ctypes.CDLL(LIB_PATH))


_lib = _load()
EXPORTS = ("attn_fwd", "attn_fwd_blockmask", "attn_build_blockmask", "attn_blockmask_bytes",
           "attn_decode_splitkv", "attn_decode_combine", "attn_decode_noalloc",
           "attn_decode_noalloc_max_bytes", "attn_decode_ws_o_bytes",
           "attn_decode_ws_lse_bytes", "attn_decode_num_splits", "attn_bwd",
           "attn_bwd_workspace_bytes", "attn_bwd_blockmask", "attn_blockmask_transpose",
           "attn_fwd_auto_plan", "attn_fwd_auto",
           "attn_probe_stream_read", "attn_status_str", "attn_abi_version")


def _check(func: str, status: int):
    if status != 0:
        raise AttnError(func, status, _lib.attn_status_str(status).decode())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _strides(t: torch.Tensor):
    if t.dim() != 4:
        raise ValueError("expected a 4-d [B, H, N, D] tensor")
    arr = (ctypes.c_int64 * 3)(*t.stride()[:3])
    return arr


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _half(*ts):
    """The library dtype code shared by all of ``ts`` (bf16 or fp16, D contiguous)."""
    dt = ts[0].dtype
    for t in ts:
        if t.dtype != dt or dt not in _DTYPES:
            raise TypeError("attention tensors must all be bfloat16 or all float16")
        if t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
    return _DTYPES[dt]


def _shape(name, t, want):
    """``t`` must have exactly shape ``want``."""
    if tuple(t.shape) != tuple(want):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(want)}")


def _on_device(*named):
    """Every (name, tensor) pair with a tensor must live on the GPU, on one device.  Checked
    after the shapes, so a shape error is reported first wherever it can be seen."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def _check_lse(lse, B, H, N):
    if lse is None:
        return
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 [B, Hq, Nq] tensor")
    _shape("lse", lse, (B, H, N))


def _check_qkvo(q, k, v, o):
    """Shapes of a prefill call: q/o [B,Hq,Nq,D], k/v [B,Hkv,Nk,D]; returns B, Hq, Hkv, Nq, Nk, D."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be a 4-d [B, H, N, D] tensor")
    B, Hq, Nq, D = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    _shape("k", k, (B, Hkv, Nk, D))
    _shape("v", v, (B, Hkv, Nk, D))
    _shape("o", o, (B, Hq, Nq, D))
    return B, Hq, Hkv, Nq, Nk, D


def _mask_tensors(mask, B):
    """The device tensors a Mask brings (doc_offsets must have one row per batch row)."""
    if isinstance(mask, Mask) and mask.doc_offsets is not None:
        if mask.doc_offsets.dim() != 2 or mask.doc_offsets.shape[0] != B:
            raise ValueError(f"doc_offsets must have one row per batch row ({B}), "
                             f"got shape {tuple(mask.doc_offsets.shape)}")
        return [("doc_offsets", mask.doc_offsets)]
    return []


def _smod_tensors(smod, Hq):
    """The device tensors a ScoreMod brings (one slope / one table row per query head)."""
    if not isinstance(smod, ScoreMod):
        return []
    out = []
    if smod.alibi_slopes is not None:
        if smod.alibi_slopes.numel() < Hq:
            raise ValueError(f"alibi_slopes needs {Hq} entries (one per query head), "
                             f"got {smod.alibi_slopes.numel()}")
        out.append(("alibi_slopes", smod.alibi_slopes))
    if smod.rel_bias is not None:
        if smod.rel_bias.dim() != 2 or smod.rel_bias.shape[0] < Hq:
            raise ValueError(f"rel_bias needs {Hq} rows (one per query head), "
                             f"got shape {tuple(smod.rel_bias.shape)}")
        out.append(("rel_bias", smod.rel_bias))
    return out


@dataclass
class Mask:
    """The mask menu of attn_mask_desc (AND-composed).

    causal: k <= p;  window=(left, right): p-left <= k <= p+right (negative =
    unbounded side);  block_size: block-diffusion k < bs*(p//bs + 1);
    doc_offsets: int32 [B, num_docs+1] cumulative document starts on the GPU.
    """
    causal: bool = False
    window: tuple | None = None
    block_size: int | None = None
    doc_offsets: torch.Tensor | None = None
    schedule: int = 0  # ATTN_SCHED_* bits: another work-group schedule, results bitwise unchanged

    def desc(self) -> attn_mask_desc:
        d = attn_mask_desc()
        d.flags = 0
        d.window_left = d.window_right = -1
        d.block_size = 0
        d.doc_offsets = None
        d.num_docs = 0
        d.doc_stride = 0
        if self.schedule & ~SCHED_ALL:
            raise ValueError("unknown schedule bits")
        d.flags |= self.schedule
        if self.causal:
            d.flags |= MASK_CAUSAL
        if self.window is not None:
            d.flags |= MASK_WINDOW
            d.window_left, d.window_right = int(self.window[0]), int(self.window[1])
        if self.block_size is not None:
            d.flags |= MASK_BLOCK_CAUSAL
            d.block_size = int(self.block_size)
        if self.doc_offsets is not None:
            off = self.doc_offsets
            if off.dtype != torch.int32 or off.dim() != 2 or off.stride(1) != 1:
                raise TypeError("doc_offsets must be int32 [B, num_docs+1] with rows contiguous")
            d.flags |= MASK_DOCUMENT
            d.doc_offsets = off.data_ptr()
            d.num_docs = off.shape[1] - 1
            d.doc_stride = off.stride(0)
        return d


def _mask_ptr(mask):
    if mask is None:
        return None, None
    d = mask.desc() if isinstance(mask, Mask) else mask
    return d, ctypes.byref(d)


@dataclass
class ScoreMod:
    """Score changes of attn_score_mod (s = scale * q.k, d = key index - query position):

    softcap: float > 0 -> s becomes softcap * tanh(s / softcap), before the additive terms;
    alibi_slopes: float32 [Hq] on the GPU -> + slope * d (or - slope * |d| with
    symmetric=True);  rel_bias: float32 [Hq, 2R+1] on the GPU -> + rel_bias[h][clamp(d, -R, R) + R].
    """
    alibi_slopes: torch.Tensor | None = None
    symmetric: bool = False
    rel_bias: torch.Tensor | None = None
    softcap: float | None = None

    def desc(self) -> attn_score_mod:
        d = attn_score_mod()
        d.flags = 0
        d.slopes = d.rel_bias = None
        d.rel_radius = 0
        d.softcap = 0.0
        if self.softcap is not None:
            d.flags |= SCORE_SOFTCAP
            d.softcap = float(self.softcap)
        if self.alibi_slopes is not None:
            t = self.alibi_slopes
            if t.dtype != torch.float32 or t.dim() != 1 or not t.is_contiguous():
                raise TypeError("alibi_slopes must be a contiguous float32 [Hq] tensor")
            d.flags |= SCORE_ALIBI_SYM if self.symmetric else SCORE_ALIBI
            d.slopes = t.data_ptr()
        if self.rel_bias is not None:
            t = self.rel_bias
            if t.dtype != torch.float32 or t.dim() != 2 or not t.is_contiguous() or t.shape[1] % 2 != 1:
                raise TypeError("rel_bias must be a contiguous float32 [Hq, 2R+1] tensor")
            d.flags |= SCORE_REL_BIAS
            d.rel_bias = t.data_ptr()
            d.rel_radius = (t.shape[1] - 1) // 2
        return d


def _smod_ptr(smod):
    if smod is None:
        return None, None
    d = smod.desc() if isinstance(smod, ScoreMod) else smod
    return d, ctypes.byref(d)


def attn_fwd(q, k, v, o, lse=None, scale=None, mask=None, stream=None, smod=None):
    """O (and LSE) for q [B,Hq,Nq,D], k/v [B,Hkv,Nk,D] bf16 or fp16 CUDA tensors (any B/H/N
    strides)."""
    dt = _half(q, k, v, o)
    B, Hq, Hkv, Nq, Nk, D = _check_qkvo(q, k, v, o)
    _check_lse(lse, B, Hq, Nq)
    _on_device(("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), *_mask_tensors(mask, B),
               *_smod_tensors(smod, Hq))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    keep, mp = _mask_ptr(mask)
    keep_s, sp = _smod_ptr(smod)
    st = _lib.attn_fwd(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                       _ptr(o), _strides(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, D, dt, scale, mp, sp,
                       _stream(stream))
    _check("attn_fwd", st)
    return o, lse


class BlockMask:
    """Device buffers of one attn_blockmask (allocated with torch on ``device``)."""

    def __init__(self, Bm, Hm, Nq, Nk, device="cuda"):
        self.Bm, self.Hm = Bm, Hm
        self.nQt = (Nq + BLOCKMASK_TILE - 1) // BLOCKMASK_TILE
        self.nKt = (Nk + BLOCKMASK_TILE - 1) // BLOCKMASK_TILE
        i32 = dict(dtype=torch.int32, device=device)
        self.part_num = torch.zeros(Bm, Hm, self.nQt, **i32)
        self.full_num = torch.zeros(Bm, Hm, self.nQt, **i32)
        self.part_idx = torch.zeros(Bm, Hm, self.nQt, max(self.nKt, 1), **i32)
        self.full_idx = torch.zeros(Bm, Hm, self.nQt, max(self.nKt, 1), **i32)

    def struct(self) -> attn_blockmask:
        s = attn_blockmask()
        s.Bm, s.Hm, s.nQt, s.nKt = self.Bm, self.Hm, self.nQt, self.nKt
        s.part_num, s.part_idx = self.part_num.data_ptr(), self.part_idx.data_ptr()
        s.full_num, s.full_idx = self.full_num.data_ptr(), self.full_idx.data_ptr()
        return s


def attn_blockmask_transpose(bm: "BlockMask", stream=None) -> "BlockMask":
    """The key-tile-major BlockMask of ``bm`` (a new BlockMask whose rows are key tiles), built on
    the GPU by attn_blockmask_transpose; the backward pass over a BlockMask takes both."""
    out = BlockMask.__new__(BlockMask)
    out.Bm, out.Hm, out.nQt, out.nKt = bm.Bm, bm.Hm, bm.nKt, bm.nQt
    dev = bm.part_num.device
    i32 = dict(dtype=torch.int32, device=dev)
    out.part_num = torch.zeros(bm.Bm, bm.Hm, out.nQt, **i32)
    out.full_num = torch.zeros(bm.Bm, bm.Hm, out.nQt, **i32)
    out.part_idx = torch.zeros(bm.Bm, bm.Hm, out.nQt, max(out.nKt, 1), **i32)
    out.full_idx = torch.zeros(bm.Bm, bm.Hm, out.nQt, max(out.nKt, 1), **i32)
    tmp = torch.empty(max(bm.Bm * bm.Hm * bm.nQt * bm.nKt, 1), dtype=torch.uint8, device=dev)
    _on_device(("part_num", bm.part_num), ("out", out.part_num), ("tmp", tmp))
    s_in, s_out = bm.struct(), out.struct()
    _check("attn_blockmask_transpose",
           _lib.attn_blockmask_transpose(ctypes.byref(s_in), ctypes.byref(s_out), _ptr(tmp),
                                         tmp.numel(), _stream(stream)))
    out._tmp = tmp  # the map is overwritten by the kernel; kept alive until the stream uses it
    return out


def attn_blockmask_bytes(Bm, Hm, nQt, nKt):
    return int(_lib.attn_blockmask_bytes(Bm, Hm, nQt, nKt))


def attn_build_blockmask(bm: BlockMask, B, Nq, Nk, mask=None, tile_map=None, stream=None):
    """Fill ``bm`` from a uint8 tile map [Bm, Hm, nQt, nKt] (CUDA) or from ``mask``."""
    if tile_map is not None and (tile_map.dtype != torch.uint8 or not tile_map.is_contiguous()):
        raise TypeError("tile_map must be a contiguous uint8 tensor")
    if tile_map is not None:
        _shape("tile_map", tile_map, (bm.Bm, bm.Hm, bm.nQt, bm.nKt))
    if (bm.nQt, bm.nKt) != ((Nq + BLOCKMASK_TILE - 1) // BLOCKMASK_TILE,
                            (Nk + BLOCKMASK_TILE - 1) // BLOCKMASK_TILE):
        raise ValueError("BlockMask tile counts do not match Nq / Nk")
    _on_device(("tile_map", tile_map), ("part_num", bm.part_num), ("part_idx", bm.part_idx),
               ("full_num", bm.full_num), ("full_idx", bm.full_idx), *_mask_tensors(mask, B))
    keep, mp = _mask_ptr(mask)
    s = bm.struct()
    st = _lib.attn_build_blockmask(mp, _ptr(tile_map), B, Nq, Nk, ctypes.byref(s), _stream(stream))
    _check("attn_build_blockmask", st)
    return bm


def attn_fwd_blockmask(q, k, v, o, bm: BlockMask, lse=None, scale=None, mask=None, stream=None,
                       smod=None):
    dt = _half(q, k, v, o)
    B, Hq, Hkv, Nq, Nk, D = _check_qkvo(q, k, v, o)
    _check_lse(lse, B, Hq, Nq)
    _on_device(("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("part_num", bm.part_num),
               ("part_idx", bm.part_idx), ("full_num", bm.full_num), ("full_idx", bm.full_idx),
               *_mask_tensors(mask, B), *_smod_tensors(smod, Hq))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    keep, mp = _mask_ptr(mask)
    keep_s, sp = _smod_ptr(smod)
    s = bm.struct()
    st = _lib.attn_fwd_blockmask(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                 _ptr(o), _strides(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, D, dt, scale,
                                 mp, sp, ctypes.byref(s), _stream(stream))
    _check("attn_fwd_blockmask", st)
    return o, lse


def attn_decode_num_splits(B, Hkv, max_pages, num_cus=None):
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    return int(_lib.attn_decode_num_splits(B, Hkv, max_pages, num_cus))


def attn_decode_ws_o_bytes(B, Hq, Lq, D, S):
    return int(_lib.attn_decode_ws_o_bytes(B, Hq, Lq, D, S))


def attn_decode_ws_lse_bytes(B, Hq, Lq, S):
    return int(_lib.attn_decode_ws_lse_bytes(B, Hq, Lq, S))


def attn_decode_splitkv(q, k_cache, v_cache, block_table, seq_lens, max_pages, num_splits,
                        ws_o, ws_lse, scale=None, mask=None, stream=None, smod=None):
    """Split-KV partials: q [B,Hq,Lq,D]; caches [pages, page_size, Hkv, D] (contiguous);
    block_table int32 [B, >=max_pages]; seq_lens int32 [B]; ws_o float [B,Hq,Lq,S,D];
    ws_lse float [B,Hq,Lq,S]."""
    dt = _half(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("KV caches must have the dtype of q")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("KV caches must be contiguous [pages, page_size, Hkv, D]")
    if k_cache.shape != v_cache.shape:
        raise ValueError("K and V caches differ in shape")
    if block_table.dtype != torch.int32 or block_table.stride(1) != 1:
        raise TypeError("block_table must be int32 with contiguous rows")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise TypeError("seq_lens must be contiguous int32")
    if ws_o.dtype != torch.float32 or ws_lse.dtype != torch.float32:
        raise TypeError("workspaces must be float32")
    if q.dim() != 4 or k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q and the caches must be 4-d, block_table 2-d")
    B, Hq, Lq, D = q.shape
    n_pages, page_size, Hkv, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("head dim mismatch")
    if block_table.shape[0] < B or block_table.shape[1] < max_pages:
        raise ValueError(f"block_table must be at least [{B}, {max_pages}], "
                         f"got {tuple(block_table.shape)}")
    if seq_lens.numel() < B:
        raise ValueError(f"seq_lens needs {B} entries, got {seq_lens.numel()}")
    if ws_o.numel() * 4 < attn_decode_ws_o_bytes(B, Hq, Lq, D, num_splits) or \
            ws_lse.numel() * 4 < attn_decode_ws_lse_bytes(B, Hq, Lq, num_splits):
        raise ValueError("workspace too small")
    if not (ws_o.is_contiguous() and ws_lse.is_contiguous()):
        raise TypeError("workspaces must be contiguous")
    _on_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
               ("seq_lens", seq_lens), ("ws_o", ws_o), ("ws_lse", ws_lse),
               *_smod_tensors(smod, Hq))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    keep, mp = _mask_ptr(mask)
    keep_s, sp = _smod_ptr(smod)
    st = _lib.attn_decode_splitkv(_ptr(q), _strides(q), _ptr(k_cache), _ptr(v_cache), n_pages,
                                  _ptr(block_table), block_table.stride(0), _ptr(seq_lens),
                                  int(max_pages), B, Hq, Hkv, Lq, D, dt, page_size, int(num_splits),
                                  scale, mp, sp, _ptr(ws_o), _ptr(ws_lse), _stream(stream))
    _check("attn_decode_splitkv", st)
    return ws_o, ws_lse


def attn_decode_combine(ws_o, ws_lse, o, lse=None, stream=None):
    """O [B,Hq,Lq,D] bf16 / fp16 (and LSE [B,Hq,Lq]) from ws_o [B,Hq,Lq,S,D], ws_lse [B,Hq,Lq,S]."""
    dt = _half(o)
    if ws_o.dim() != 5:
        raise ValueError("ws_o must be a 5-d [B, Hq, Lq, S, D] tensor")
    B, Hq, Lq, S, D = ws_o.shape
    if ws_o.dtype != torch.float32 or ws_lse.dtype != torch.float32 or not ws_o.is_contiguous() \
            or not ws_lse.is_contiguous():
        raise TypeError("workspaces must be contiguous float32")
    _shape("ws_lse", ws_lse, (B, Hq, Lq, S))
    if o.dim() != 4:
        raise ValueError("o must be a 4-d [B, Hq, Lq, D] tensor")
    _shape("o", o, (B, Hq, Lq, D))
    _check_lse(lse, B, Hq, Lq)
    _on_device(("ws_o", ws_o), ("ws_lse", ws_lse), ("o", o), ("lse", lse))
    st = _lib.attn_decode_combine(_ptr(ws_o), _ptr(ws_lse), B, Hq, Lq, S, D, dt, _ptr(o),
                                  _strides(o), _ptr(lse), _stream(stream))
    _check("attn_decode_combine", st)
    return o, lse


def attn_decode_noalloc_max_bytes():
    return int(_lib.attn_decode_noalloc_max_bytes())


def attn_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, max_pages, num_splits, o,
                        lse=None, scale=None, mask=None, stream=None, smod=None):
    """attn_decode_splitkv + attn_decode_combine in one call that allocates nothing (the split
    partials live in the library's static per-GPU buffer); o [B,Hq,Lq,D], lse [B,Hq,Lq] or None."""
    dt = _half(q, o)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("KV caches must have the dtype of q")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()) or k_cache.shape != v_cache.shape:
        raise ValueError("KV caches must be contiguous [pages, page_size, Hkv, D] of one shape")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise TypeError("block_table must be int32 [B, >= max_pages] with contiguous rows")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise TypeError("seq_lens must be contiguous int32")
    if q.dim() != 4 or k_cache.dim() != 4 or o.dim() != 4:
        raise ValueError("q, o and the caches must be 4-d")
    B, Hq, Lq, D = q.shape
    n_pages, page_size, Hkv, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("head dim mismatch")
    _shape("o", o, (B, Hq, Lq, D))
    _check_lse(lse, B, Hq, Lq)
    if block_table.shape[0] < B or block_table.shape[1] < max_pages:
        raise ValueError(f"block_table must be at least [{B}, {max_pages}]")
    if seq_lens.numel() < B:
        raise ValueError(f"seq_lens needs {B} entries")
    _on_device(("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("block_table", block_table),
               ("seq_lens", seq_lens), ("o", o), ("lse", lse), *_smod_tensors(smod, Hq))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    keep, mp = _mask_ptr(mask)
    keep_s, sp = _smod_ptr(smod)
    st = _lib.attn_decode_noalloc(_ptr(q), _strides(q), _ptr(k_cache), _ptr(v_cache), n_pages,
                                  _ptr(block_table), block_table.stride(0), _ptr(seq_lens),
                                  int(max_pages), B, Hq, Hkv, Lq, D, dt, page_size, int(num_splits),
                                  scale, mp, sp, _ptr(o), _strides(o), _ptr(lse), _stream(stream))
    _check("attn_decode_noalloc", st)
    return o, lse


def attn_bwd_workspace_bytes(B, Hq, Nq):
    return int(_lib.attn_bwd_workspace_bytes(B, Hq, Nq))


def attn_bwd(q, k, v, o, d_o, lse, dq, dk, dv, workspace=None, scale=None, mask=None, stream=None,
             smod=None):
    """dQ, dK, dV (written into dq / dk / dv) for q/o/d_o [B,Hq,Nq,D], k/v [B,Hkv,Nk,D] (bf16 or fp16)
    and the forward pass's lse float [B,Hq,Nq]; ``workspace`` is a float32 CUDA tensor of at
    least attn_bwd_workspace_bytes(B, Hq, Nq) bytes (allocated here if None)."""
    dt = _half(q, k, v, o, d_o, dq, dk, dv)
    B, Hq, Hkv, Nq, Nk, D = _check_qkvo(q, k, v, o)
    for name, t, want in (("d_o", d_o, q.shape), ("dq", dq, q.shape), ("dk", dk, k.shape),
                          ("dv", dv, k.shape)):
        _shape(name, t, want)
    if lse is None:
        raise TypeError("lse (the forward pass's float32 [B, Hq, Nq]) is required")
    _check_lse(lse, B, Hq, Nq)
    _on_device(("q", q), ("k", k), ("v", v), ("o", o), ("d_o", d_o), ("lse", lse), ("dq", dq),
               ("dk", dk), ("dv", dv), ("workspace", workspace), *_mask_tensors(mask, B),
               *_smod_tensors(smod, Hq))
    need = attn_bwd_workspace_bytes(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=q.device)
    if workspace.dtype != torch.float32 or not workspace.is_contiguous():
        raise TypeError("workspace must be contiguous float32")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    keep, mp = _mask_ptr(mask)
    keep_s, sp = _smod_ptr(smod)
    st = _lib.attn_bwd(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                       _ptr(o), _strides(o), _ptr(d_o), _strides(d_o), _ptr(lse),
                       _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv), _strides(dv),
                       B, Hq, Hkv, Nq, Nk, D, dt, scale, mp, sp, _ptr(workspace), workspace.numel() * 4,
                       _stream(stream))
    _check("attn_bwd", st)
    return dq, dk, dv


def attn_bwd_blockmask(q, k, v, o, d_o, lse, dq, dk, dv, bm: "BlockMask", bm_t: "BlockMask",
                       workspace=None, scale=None, mask=None, stream=None, smod=None):
    """dQ, dK, dV of attn_fwd_blockmask's O: ``bm`` the forward BlockMask, ``bm_t`` its
    key-tile-major lists (attn_blockmask_transpose(bm)); otherwise as attn_bwd."""
    dt = _half(q, k, v, o, d_o, dq, dk, dv)
    B, Hq, Hkv, Nq, Nk, D = _check_qkvo(q, k, v, o)
    for name, t, want in (("d_o", d_o, q.shape), ("dq", dq, q.shape), ("dk", dk, k.shape),
                          ("dv", dv, k.shape)):
        _shape(name, t, want)
    if lse is None:
        raise TypeError("lse (the forward pass's float32 [B, Hq, Nq]) is required")
    _check_lse(lse, B, Hq, Nq)
    _on_device(("q", q), ("k", k), ("v", v), ("o", o), ("d_o", d_o), ("lse", lse), ("dq", dq),
               ("dk", dk), ("dv", dv), ("workspace", workspace), ("bm", bm.part_num),
               ("bm_t", bm_t.part_num), *_mask_tensors(mask, B), *_smod_tensors(smod, Hq))
    need = attn_bwd_workspace_bytes(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need // 4, 1), dtype=torch.float32, device=q.device)
    if workspace.dtype != torch.float32 or not workspace.is_contiguous():
        raise TypeError("workspace must be contiguous float32")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    keep, mp = _mask_ptr(mask)
    keep_s, sp = _smod_ptr(smod)
    s1, s2 = bm.struct(), bm_t.struct()
    st = _lib.attn_bwd_blockmask(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                 _ptr(o), _strides(o), _ptr(d_o), _strides(d_o), _ptr(lse),
                                 _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv), _strides(dv),
                                 B, Hq, Hkv, Nq, Nk, D, dt, scale, mp, sp, ctypes.byref(s1),
                                 ctypes.byref(s2), _ptr(workspace), workspace.numel() * 4,
                                 _stream(stream))
    _check("attn_bwd_blockmask", st)
    return dq, dk, dv


def attn_fwd_auto_plan(B, Hq, Hkv, Nq, Nk, D, smod=None) -> attn_auto_plan:
    """The path attn_fwd_auto takes for a shape (PATH_PREFILL / PATH_SPLITKV), its key split
    count and the workspace bytes it needs (host only)."""
    keep_s, sp = _smod_ptr(smod)
    out = attn_auto_plan()
    _check("attn_fwd_auto_plan", _lib.attn_fwd_auto_plan(B, Hq, Hkv, Nq, Nk, D, sp, ctypes.byref(out)))
    return out


def attn_fwd_auto(q, k, v, o, lse=None, scale=None, mask=None, workspace=None, stream=None,
                  smod=None):
    """attn_fwd with the kernel chosen by shape: split-KV + combine for decode-shaped calls
    (G * Nq <= 64 query rows per KV head and Nk >= 512), the prefill kernels otherwise.
    ``workspace`` is a CUDA tensor of at least attn_fwd_auto_plan(...).workspace_bytes bytes
    (allocated here if None)."""
    dt = _half(q, k, v, o)
    B, Hq, Hkv, Nq, Nk, D = _check_qkvo(q, k, v, o)
    _check_lse(lse, B, Hq, Nq)
    _on_device(("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("workspace", workspace),
               *_mask_tensors(mask, B), *_smod_tensors(smod, Hq))
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    keep, mp = _mask_ptr(mask)
    keep_s, sp = _smod_ptr(smod)
    if workspace is None:
        need = attn_fwd_auto_plan(B, Hq, Hkv, Nq, Nk, D, smod).workspace_bytes
        workspace = torch.empty(max((need + 3) // 4, 1), dtype=torch.float32, device=q.device)
    if not workspace.is_contiguous():
        raise TypeError("workspace must be contiguous")
    st = _lib.attn_fwd_auto(_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                            _ptr(o), _strides(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, D, dt, scale, mp,
                            sp, _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(stream))
    _check("attn_fwd_auto", st)
    return o, lse


def attn_probe_stream_read(src, sink, blocks=None, stream=None):
    """Read all of ``src`` (a contiguous GPU tensor, size a multiple of 16 bytes) once with the
    streaming probe kernel; ``sink`` is a GPU int32 tensor of at least ``blocks`` entries."""
    if blocks is None:
        blocks = sink.numel()
    if not src.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < blocks:
        raise ValueError("src must be contiguous and sink an int32 tensor of >= blocks entries")
    _on_device(("src", src), ("sink", sink))
    _check("attn_probe_stream_read",
           _lib.attn_probe_stream_read(_ptr(src), src.numel() * src.element_size(), int(blocks),
                                       _ptr(sink), _stream(stream)))


def attn_status_str(status: int) -> str:
    return _lib.attn_status_str(status).decode()


def attn_abi_version() -> int:
    return int(_lib.attn_abi_version())


def lib_handle():
    """The loaded ctypes library (for direct C-ABI calls in tests)."""
    return _lib
