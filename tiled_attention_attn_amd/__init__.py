"""Fused exact attention for one AMD MI355X (gfx950), from hand-written HIP kernels.

O = softmax(scale * Q K^T + mask) V computed tile by tile with an online
softmax, so the N x N score matrix never reaches HBM (the method of
"FlashAttention 2 principles and PyTorch practice", sections 1 and 3), with the
mask menu of the FlexAttention / DFlash article: causal, symmetric sliding
window, document, block-diffusion, BlockMask block sparsity, GQA, and
split-KV decoding over a paged KV cache merged by log-sum-exp, a shape-based
switch to split-KV for decode-shaped calls; and the backward pass (dQ, dK,
dV by recomputation from the saved LSE).

The package is a thin ctypes binding over the C ABI of ``include/tiled_attn.h``
(``libtiled_attn.so``); importing it fails if the library has not been built.
"""
from ._lib import (  # noqa: F401
    AttnError, Mask, ScoreMod, BlockMask, LIB_PATH, EXPORTS, DTYPE_BF16, DTYPE_F16,
    SCORE_ALIBI, SCORE_ALIBI_SYM, SCORE_REL_BIAS, SCORE_SOFTCAP, attn_score_mod,
    MASK_CAUSAL, MASK_WINDOW, MASK_DOCUMENT, MASK_BLOCK_CAUSAL, BLOCKMASK_TILE,
    SCHED_NO_PAIRING, SCHED_NO_XCD_REMAP, SCHED_REVERSE, SCHED_ALL,
    TILE_EMPTY, TILE_PARTIAL, TILE_FULL,
    attn_fwd, attn_fwd_blockmask, attn_build_blockmask, attn_blockmask_bytes,
    attn_decode_splitkv, attn_decode_combine, attn_decode_num_splits,
    attn_decode_noalloc, attn_decode_noalloc_max_bytes,
    attn_decode_ws_o_bytes, attn_decode_ws_lse_bytes, attn_bwd, attn_bwd_workspace_bytes,
    attn_bwd_blockmask, attn_blockmask_transpose,
    attn_fwd_auto, attn_fwd_auto_plan, attn_auto_plan, PATH_PREFILL, PATH_SPLITKV,
    attn_probe_stream_read, attn_status_str, attn_abi_version,
    attn_mask_desc, attn_blockmask, lib_handle,
)
