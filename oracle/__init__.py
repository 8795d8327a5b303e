"""CPU oracle for masked exact attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
does, and nothing here imports the product path: the two share no code.

What it computes is the plain definition, in float64 NumPy, with no tiling and
no online softmax:

    s[q, k] = scale * <Q[q], K[k]>            (scale defaults to 1/sqrt(d))
    P       = softmax over the keys the mask lets q see
    O[q]    = sum_k P[q, k] V[k],   LSE[q] = log sum_k exp(s[q, k])

(FlashAttention 2 principles and PyTorch practice, section 1: standard attention
softmax(QK^T/sqrt(d))V and the N x N matrices S and P).  The tiled method on
the pages reaches this same result up to rounding order, so the definition is
the oracle.  Masks are explicit dense boolean predicates in the mask_mod form
(b, h, q_idx, kv_idx) -> bool that the FlexAttention article (section 1)
describes.

Modules:
    masks      -- mask_mod predicates: causal, symmetric window, document,
                  block-diffusion, BlockMask, key range, AND-composition
    core       -- attention(), attention_rows(), combine(), scores(), masked_softmax()
    paged      -- logical K/V gathered from a paged pool through a block table
    blockmask  -- tile classes (EMPTY / PARTIAL / FULL) from a dense mask, and
                  the compacted per-row tile lists
    backward   -- dQ, dK, dV of the same definition (softmax Jacobian, chain rule)
    score_mods -- additive score modifications: ALiBi, symmetric ALiBi, a
                  relative-position bias table (FlexAttention article, section 1)

Every function is pinned by CPU tests (brute force on tiny inputs, torch's
float64 CPU scaled_dot_product_attention, closed forms, invariants and
identities); no function here is "parity unpinned".
"""
from . import masks, core, paged, blockmask, backward, score_mods
from .core import attention, attention_rows, combine, scores, masked_softmax

__all__ = ["masks", "core", "paged", "blockmask", "backward", "score_mods", "attention", "attention_rows", "combine",
           "scores", "masked_softmax"]
