/*
 * tiled_attn.h -- C ABI of the MI355X (gfx950) fused exact-attention library.
 *
 * What the library computes, for every batch row b and query head hq:
 *
 *     s[q, k] = scale * <Q[b, hq, q, :], K[b, kvh, k, :]>,   kvh = hq / (Hq / Hkv)
 *     O[b, hq, q, :] = sum over visible k of softmax_k(s[q, k]) * V[b, kvh, k, :]
 *     LSE[b, hq, q]  = log sum over visible k of exp(s[q, k])       (natural log)
 *
 * the plain attention softmax(QK^T / sqrt(d)) V of "FlashAttention 2 principles
 * and PyTorch practice" (section 1), computed the way its sections 1 and 3
 * describe: Q in blocks, K/V streamed block by block through on-chip memory,
 * an online softmax (running max and exp-sum, accumulator rescaled), so the
 * N x N score matrix never reaches HBM.  Which keys a query sees comes from
 * the mask menu of the FlexAttention / DFlash article (section 1: mask_mod,
 * BlockMask, GQA, split-KV decoding over a paged cache; section 3: the
 * symmetric sliding window).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Q, K, V, O (and dO, dQ, dK, dV) are 16-bit floats of one type, named by
 *   the `dtype` argument: ATTN_DTYPE_BF16 or ATTN_DTYPE_F16 (the two kernel
 *   dtypes the FlashAttention 2 article, section 7, allows; fp32 callers
 *   convert first).  P is rounded to the same type for the P V product.
 *   Accumulation is fp32.
 * - Tensors are logical [B, H, N, D] with D contiguous (stride 1).  Each
 *   tensor comes with three element strides for (b, h, n); any order of the
 *   B/H/N dimensions in memory is accepted, so both [B, H, N, D] and
 *   [B, N, H, D] layouts pass without a copy (FlashAttention 2 article,
 *   section 2).  Strides must be multiples of 8 elements and base pointers
 *   16-byte aligned; the sequence (n) strides of K and V (and, for attn_bwd,
 *   of Q and dO) stay below 2^24.
 * - LSE is fp32 [B, Hq, Nq], contiguous, natural log, scale included.  A row
 *   that sees no key gets O = 0 and LSE = -inf.  LSE pointers may be NULL
 *   where noted (then it is not written).
 * - D is 64 or 128.  Hq must be a multiple of Hkv (GQA, consecutive
 *   grouping: query head hq reads KV head hq / (Hq / Hkv)).
 * - A call whose one-dimensional work-group count would pass 2^31 - 1
 *   (B * Hq * ceil(Nq / 128) for the prefill and dQ kernels, B * Hkv *
 *   ceil(Nk / 128) for dK/dV) fails with ATTN_ERR_SHAPE before any launch.
 * - scale must be finite and > 0 (callers wanting 1/sqrt(D) pass it).
 * - Every pointer to tensor data is a DEVICE pointer owned by the caller.
 *   The library allocates nothing, frees nothing, keeps no state between
 *   calls and never synchronises: each call validates its arguments on the
 *   host, then enqueues its kernels on `stream` and returns.  The one
 *   exception is attn_decode_noalloc's static per-GPU buffer (see there).
 * - Return value: ATTN_OK (0) or a negative ATTN_ERR_* code.  Arguments are
 *   checked before any launch; on an error nothing is launched and no output
 *   is touched.  ATTN_ERR_LAUNCH reports hipGetLastError() after a launch.
 * - Results are deterministic: no atomics in any reduction; the reduction
 *   order depends only on logical positions, never on memory placement.
 */
#ifndef TILED_ATTN_H
#define TILED_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define ATTN_OK 0
#define ATTN_ERR_NULL (-1)      /* a required pointer is NULL                  */
#define ATTN_ERR_SHAPE (-2)     /* negative size, or a size over a limit       */
#define ATTN_ERR_HEAD_DIM (-3)  /* D is not 64 or 128                          */
#define ATTN_ERR_GQA (-4)       /* Hq not a positive multiple of Hkv           */
#define ATTN_ERR_STRIDE (-5)    /* stride not a multiple of 8 elements         */
#define ATTN_ERR_ALIGN (-6)     /* tensor base not 16-byte aligned             */
#define ATTN_ERR_MASK (-7)      /* unknown mask flag or bad mask parameter     */
#define ATTN_ERR_WORKSPACE (-8) /* workspace / split arguments inconsistent    */
#define ATTN_ERR_LAUNCH (-9)    /* the HIP runtime reported a launch error     */
#define ATTN_ERR_BLOCKMASK (-10)/* BlockMask descriptor inconsistent           */
#define ATTN_ERR_SCALE (-11)    /* scale not finite and > 0                    */
#define ATTN_ERR_DTYPE (-12)    /* dtype is not ATTN_DTYPE_BF16 / ATTN_DTYPE_F16 */
#define ATTN_ERR_SCORE_MOD (-13)/* bad score_mod flags / parameters, or not supported here */

/* ---- element types ------------------------------------------------------ */
#define ATTN_DTYPE_BF16 0
#define ATTN_DTYPE_F16 1

/* ---- masks --------------------------------------------------------------
 * A query row q is placed at the absolute position p = q + (Nk - Nq)
 * (bottom-right alignment; the FlashAttention 2 article, section 7, warns
 * that a misaligned causal mask shifts the output).  The flags are
 * AND-composed; flags == 0 means every key is visible (non-causal /
 * bidirectional).  Every flag keeps the visible keys of a row one contiguous
 * interval [lo(p), hi(p)], and both ends never decrease as p grows.
 */
#define ATTN_MASK_CAUSAL 1u       /* k <= p                                       */
#define ATTN_MASK_WINDOW 2u       /* p - window_left <= k <= p + window_right     */
#define ATTN_MASK_DOCUMENT 4u     /* k in the same document as p                  */
#define ATTN_MASK_BLOCK_CAUSAL 8u /* k < block_size * (p / block_size + 1)        */
#define ATTN_MASK_ALL 15u

/* Schedule flags, carried in attn_mask_desc.flags beside the mask bits.  They
 * change only which work group covers which tile and how the work groups are
 * numbered on the GPU -- never a bit of any result, because every output row
 * (and every dK / dV key) is produced by exactly one work group with a fixed
 * order of its key (or row) sums.  They exist so a test can run one call
 * under two schedules and require bitwise-equal outputs (a missing
 * synchronisation would show up as a difference).
 *   NO_PAIRING      causal-like masks: one query (key) tile per work group
 *                   instead of the pair (i, n-1-i)
 *   NO_XCD_REMAP    work groups numbered in launch order instead of whole
 *                   heads per XCD
 *   REVERSE         work groups numbered from the last to the first
 */
#define ATTN_SCHED_NO_PAIRING (1u << 16)
#define ATTN_SCHED_NO_XCD_REMAP (1u << 17)
#define ATTN_SCHED_REVERSE (1u << 18)
#define ATTN_SCHED_ALL (7u << 16)

typedef struct attn_mask_desc {
  uint32_t flags;       /* ATTN_MASK_* bits (and optional ATTN_SCHED_* bits)       */
  int32_t window_left;  /* WINDOW: inclusive widths; a negative width leaves that  */
  int32_t window_right; /*   side unbounded.  Symmetric (w, w) is the pages' case. */
  int32_t block_size;   /* BLOCK_CAUSAL: block length (> 0)                        */
  /* DOCUMENT: device int32 [B][doc_stride] of cumulative document starts.
   * Row b holds num_docs + 1 entries: doc d covers keys [off[d], off[d+1]).
   * off[0] = 0, non-decreasing, off[num_docs] = Nk; rows with fewer documents
   * repeat their final offset.  DOCUMENT requires Nq <= Nk (every query
   * position then lies inside the key sequence).  Offsets that break these
   * rules give unspecified values but never an out-of-range access
   * (positions are clamped to [0, Nk)).                                         */
  const int32_t* doc_offsets;
  int32_t num_docs;     /* documents per row (>= 1)                                */
  int32_t doc_stride;   /* elements between rows of doc_offsets (>= num_docs + 1)  */
} attn_mask_desc;

/* ---- score modification -------------------------------------------------
 * Changes of the scaled score before the softmax, the score_mod of the
 * FlexAttention article (section 1: ALiBi, a position bias, a learnable
 * bias), plus tanh capping.  With s = scale * q.k and d = k - p (key index
 * minus the query's aligned position), the score becomes
 *     SOFTCAP    s -> softcap * tanh(s / softcap)      (applied first)
 *     ALIBI      + slopes[hq] * d                      (<= 0 where k <= p)
 *     ALIBI_SYM  - slopes[hq] * |d|
 *     REL_BIAS   + rel_bias[hq][clamp(d, -R, R) + R]
 * ALIBI and ALIBI_SYM exclude each other; the others combine freely.  LSE is
 * then the log-sum-exp of the changed scores.  The bias arrays are device
 * memory; the backward pass applies the cap's derivative 1 - tanh^2(s / cap)
 * and treats the biases and the cap as constants (no gradient for them).
 * SOFTCAP needs a finite softcap > 0.
 * REL_BIAS needs 0 <= R <= 1023 and, in attn_bwd, (Hq / Hkv) * (2R + 1) <=
 * 8192.  attn_fwd, attn_fwd_blockmask, attn_bwd and attn_decode_splitkv take
 * every score change at D = 64 and 128.
 */
#define ATTN_SCORE_ALIBI 1u
#define ATTN_SCORE_ALIBI_SYM 2u
#define ATTN_SCORE_REL_BIAS 4u
#define ATTN_SCORE_SOFTCAP 8u
#define ATTN_SCORE_ALL 15u

typedef struct attn_score_mod {
  uint32_t flags;         /* ATTN_SCORE_* bits (0 = no change)                    */
  const float* slopes;    /* ALIBI / ALIBI_SYM: device float [Hq]                 */
  const float* rel_bias;  /* REL_BIAS: device float [Hq][2 * rel_radius + 1]      */
  int32_t rel_radius;     /* REL_BIAS: R                                          */
  float softcap;          /* SOFTCAP: the cap (> 0)                               */
} attn_score_mod;

/* ---- dense-mask prefill ---------------------------------------------------
 * attn_fwd: O = softmax(scale * Q K^T restricted by `mask`) V, plus LSE.
 *   q  [B, Hq,  Nq, D], k/v [B, Hkv, Nk, D], o [B, Hq, Nq, D] (strides (b,h,n))
 *   lse float [B, Hq, Nq] contiguous, or NULL.
 *   mask may be NULL (no mask); smod may be NULL (no score change).  Nq or Nk
 *   may be 0 (Nk = 0: every row empty; k and v may then be NULL).
 * The key blocks of a query block are chosen analytically from the mask's
 * per-row intervals: blocks outside every row's interval are skipped, blocks
 * inside every row's interval run unmasked, the rest apply the interval
 * per element in registers.
 */
int attn_fwd(const void* q, const int64_t q_stride[3],
             const void* k, const int64_t k_stride[3],
             const void* v, const int64_t v_stride[3],
             void* o, const int64_t o_stride[3], float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int D, int dtype, float scale,
             const attn_mask_desc* mask, const attn_score_mod* smod, hipStream_t stream);

/* ---- BlockMask -----------------------------------------------------------
 * Block-level sparsity over 128 x 128 tiles (FlexAttention article,
 * section 1).  Per (batch row, head, query tile) the BlockMask lists the key
 * tiles to visit: FULL tiles run with no predicate, PARTIAL tiles apply the
 * `mask` intervals per element, tiles in neither list are skipped.
 * Bm / Hm are 1 when one BlockMask is shared by every batch row / head.
 */
#define ATTN_BLOCKMASK_TILE 128
#define ATTN_TILE_EMPTY 0
#define ATTN_TILE_PARTIAL 1
#define ATTN_TILE_FULL 2

typedef struct attn_blockmask {
  int32_t Bm, Hm;     /* 1 (shared) or B / Hq                                   */
  int32_t nQt, nKt;   /* ceil(Nq / 128), ceil(Nk / 128)                          */
  int32_t* part_num;  /* device [Bm][Hm][nQt]: number of PARTIAL tiles           */
  int32_t* part_idx;  /* device [Bm][Hm][nQt][nKt]: their key-tile indices, ascending */
  int32_t* full_num;  /* device [Bm][Hm][nQt]                                    */
  int32_t* full_idx;  /* device [Bm][Hm][nQt][nKt]                               */
} attn_blockmask;

/* Bytes of device memory the four arrays of one attn_blockmask need in total
 * (the caller allocates them; 0 on invalid sizes, and when the count would not
 * fit a size_t). */
size_t attn_blockmask_bytes(int Bm, int Hm, int nQt, int nKt);

/* attn_build_blockmask: fills `out` (whose pointers and Bm, Hm, nQt, nKt the
 * caller has set) on `stream`.
 *   tile_map: device uint8 [Bm][Hm][nQt][nKt] of ATTN_TILE_* codes, or NULL.
 *     Given: each tile takes its class from the map (the `mask` predicate is
 *     applied to PARTIAL tiles at attention time, FlexAttention semantics).
 *     NULL: classes come from `mask` (required then): a tile is EMPTY when no
 *     in-range (q, k) pair of it is visible, FULL when every in-range pair is,
 *     PARTIAL otherwise.  With a DOCUMENT mask Bm must equal B.
 *   B is the batch size the mask's doc_offsets describe (ignored otherwise).
 * Lists are written in ascending key-tile order; entries past a row's count
 * are set to 0, so the output is fully determined.
 */
int attn_build_blockmask(const attn_mask_desc* mask, const uint8_t* tile_map,
                         int B, int Nq, int Nk, attn_blockmask* out,
                         hipStream_t stream);

/* attn_fwd_blockmask: attn_fwd restricted to the tiles `bm` lists.
 * bm->nQt / nKt must equal ceil(Nq/128) / ceil(Nk/128); bm->Bm in {1, B},
 * bm->Hm in {1, Hq}.  `mask` (may be NULL) is applied on PARTIAL tiles only.
 */
int attn_fwd_blockmask(const void* q, const int64_t q_stride[3],
                       const void* k, const int64_t k_stride[3],
                       const void* v, const int64_t v_stride[3],
                       void* o, const int64_t o_stride[3], float* lse,
                       int B, int Hq, int Hkv, int Nq, int Nk, int D, int dtype, float scale,
                       const attn_mask_desc* mask, const attn_score_mod* smod,
                       const attn_blockmask* bm, hipStream_t stream);

/* ---- split-KV paged decode -------------------------------------------------
 * "Short query, long KV" decoding split over the key sequence and merged by
 * log-sum-exp (FlexAttention article, section 1: FlashDecoding-style split-KV
 * with GQA and a paged cache addressed through a block table).
 *
 * attn_decode_splitkv: for each sequence b, KV head, split s and query row,
 * the attention over split s's keys only, normalised, in fp32:
 *   q           [B, Hq, Lq, D] of `dtype` (strides (b, h, n))
 *   k_cache,    [num_pages, page_size, Hkv, D] of `dtype`, contiguous pool
 *   v_cache
 *   block_table device int32 [B][bt_stride]; logical key j of sequence b
 *               lives in page block_table[b][j / page_size], slot j % page_size
 *   seq_lens    device int32 [B]: key count of each sequence, the Lq new
 *               tokens included (0 <= seq_lens[b] <= max_pages * page_size)
 *   max_pages   pages of the block table a sequence may use (<= bt_stride)
 *   num_splits  S >= 1 with ceil(max_pages / S) <= 2048 (a split's block-
 *               table entries are staged on chip).  Split s covers keys
 *               [s*C, min((s+1)*C, seq_len)) with C = page_size * ceil(max_pages / S).
 *   mask        NULL = causal; else CAUSAL / WINDOW / BLOCK_CAUSAL flags
 *               (DOCUMENT is rejected).  Query t of sequence b sits at
 *               position seq_lens[b] - Lq + t.
 *   ws_o        float [B][Hq][Lq][S][D] (caller-allocated workspace)
 *   ws_lse      float [B][Hq][Lq][S]
 * A split with no visible key writes O_s = 0, LSE_s = -inf.  Pages past a
 * sequence's length are never read.  Out-of-contract inputs give unspecified
 * values but no out-of-range access: seq_lens are clamped to
 * [0, max_pages * page_size] and page indices to [0, num_pages).
 */
int attn_decode_splitkv(const void* q, const int64_t q_stride[3],
                        const void* k_cache, const void* v_cache, int64_t num_pages,
                        const int32_t* block_table, int64_t bt_stride,
                        const int32_t* seq_lens, int max_pages,
                        int B, int Hq, int Hkv, int Lq, int D, int dtype, int page_size,
                        int num_splits, float scale, const attn_mask_desc* mask,
                        const attn_score_mod* smod, float* ws_o, float* ws_lse,
                        hipStream_t stream);

/* attn_decode_combine: O = sum_s exp(LSE_s - LSE) O_s with
 * LSE = log sum_s exp(LSE_s) (max-shifted); splits with LSE_s = -inf weigh 0.
 *   o   [B, Hq, Lq, D] of `dtype` (strides (b, h, n)); lse float [B, Hq, Lq] or NULL.
 * o and ws_o must be 16-byte aligned (ATTN_ERR_ALIGN otherwise).  B * Hq * Lq
 * rows must stay below 2^31 - 3 (ATTN_ERR_SHAPE otherwise).
 */
int attn_decode_combine(const float* ws_o, const float* ws_lse,
                        int B, int Hq, int Lq, int S, int D, int dtype,
                        void* o, const int64_t o_stride[3], float* lse,
                        hipStream_t stream);

/* attn_decode_noalloc: attn_decode_splitkv followed by attn_decode_combine in
 * one call that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Arguments are attn_decode_splitkv's without ws_o /
 * ws_lse, plus attn_decode_combine's outputs o / o_stride / lse; results are
 * bit for bit those of the two calls with the same num_splits.
 * The split partials live in a library-owned static device buffer of
 * attn_decode_noalloc_max_bytes() = 32 MiB per GPU, held until the process
 * ends: B * Hq * Lq * num_splits * (D + 1) * 4 bytes (plus alignment) must fit
 * in it, else ATTN_ERR_WORKSPACE before any launch.  Every call on one GPU
 * shares that GPU's buffer, so calls that overlap on one GPU (two streams, two
 * host threads) race; calls ordered on one stream are safe.  The buffer's
 * device address is looked up on a device's first call.
 */
int attn_decode_noalloc(const void* q, const int64_t q_stride[3],
                        const void* k_cache, const void* v_cache, int64_t num_pages,
                        const int32_t* block_table, int64_t bt_stride,
                        const int32_t* seq_lens, int max_pages,
                        int B, int Hq, int Hkv, int Lq, int D, int dtype, int page_size,
                        int num_splits, float scale, const attn_mask_desc* mask,
                        const attn_score_mod* smod, void* o, const int64_t o_stride[3],
                        float* lse, hipStream_t stream);
size_t attn_decode_noalloc_max_bytes(void);

/* Workspace sizes of attn_decode_splitkv in bytes (0 on invalid sizes, and when
 * the count would not fit a size_t; attn_decode_splitkv refuses such shapes with
 * ATTN_ERR_SHAPE). */
size_t attn_decode_ws_o_bytes(int B, int Hq, int Lq, int D, int num_splits);
size_t attn_decode_ws_lse_bytes(int B, int Hq, int Lq, int num_splits);

/* A split count that fills the GPU: enough (sequence, KV head, split) work
 * groups for every compute unit, never more splits than pages. */
int attn_decode_num_splits(int B, int Hkv, int max_pages, int num_cus);

/* ---- shape-based dispatch ----------------------------------------------------
 * The FlexAttention article (section 1) describes a decode backend that
 * notices the "short query, long KV" shape and switches to a FlashDecoding-
 * style split-KV kernel.  attn_fwd_auto is attn_fwd with that choice made by
 * shape: same tensors, strides, mask, score_mod and results (O, LSE) as
 * attn_fwd, on contiguous (non-paged) K/V.
 *
 * The split-KV path is taken when all G * Nq query rows of a KV head fit one
 * 64-row group (G = Hq / Hkv, so G * Nq <= 64), Nk >= 512 and the combine's
 * B * Hq * Nq rows stay below 2^31 - 3.  It runs the
 * split-KV kernel over K/V in place and
 * then the combine: K/V are read once per KV head rather than once per query
 * head, and the key splits fill the GPU.  Every other shape runs attn_fwd.
 *
 * attn_fwd_auto_plan: the path (ATTN_PATH_*), the key split count and the
 * workspace bytes attn_fwd_auto needs for a shape; host only, launches
 * nothing.  Size errors as attn_fwd; ATTN_ERR_NULL when out is NULL.
 *
 * attn_fwd_auto: `workspace` is device memory of at least
 * plan.workspace_bytes, 16-byte aligned, overwritten (fp32 partial O and LSE
 * of every split); it may be NULL when that is 0.  ATTN_ERR_WORKSPACE when
 * workspace_bytes is smaller.  On the split-KV path the mask menu is
 * attn_fwd's (DOCUMENT included) and smod may carry any score change at
 * D = 64 and 128; on the prefill path every attn_fwd rule holds.  Results match attn_fwd to
 * rounding (a different order of the key sums), not bit for bit.
 */
#define ATTN_PATH_PREFILL 0
#define ATTN_PATH_SPLITKV 1

typedef struct attn_auto_plan {
  int32_t path;             /* ATTN_PATH_PREFILL or ATTN_PATH_SPLITKV       */
  int32_t num_splits;       /* key splits of the split-KV path, else 0      */
  uint64_t workspace_bytes; /* bytes attn_fwd_auto needs, 0 on the prefill path */
} attn_auto_plan;

int attn_fwd_auto_plan(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                       const attn_score_mod* smod, attn_auto_plan* out);

int attn_fwd_auto(const void* q, const int64_t q_stride[3],
                  const void* k, const int64_t k_stride[3],
                  const void* v, const int64_t v_stride[3],
                  void* o, const int64_t o_stride[3], float* lse,
                  int B, int Hq, int Hkv, int Nq, int Nk, int D, int dtype, float scale,
                  const attn_mask_desc* mask, const attn_score_mod* smod,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- backward pass ---------------------------------------------------------
 * Gradients of attn_fwd's O for an upstream gradient dO, by recomputation:
 * only Q, K, V, O and the forward pass's LSE are read, and P is rebuilt tile
 * by tile on chip (the segmented recomputation of the DeepSeek v2->v4
 * attention article, section 2).  With P = exp(scale Q K^T + mask - LSE) and
 * Delta = rowsum(dO * O):
 *     dV = P^T dO,  dS = P * (dO V^T - Delta),  dQ = scale dS K,  dK = scale dS^T Q.
 *   q, o, d_o, dq   [B, Hq, Nq, D] of `dtype` (strides (b, h, n))
 *   k, v, dk, dv    [B, Hkv, Nk, D] of `dtype`
 *   lse             float [B, Hq, Nq] contiguous, as attn_fwd wrote it
 *                   (-inf for rows that see no key)
 *   mask            the dense mask of the forward call (NULL = none)
 *   workspace       device memory of at least attn_bwd_workspace_bytes(B, Hq,
 *                   Nq) bytes, 16-byte aligned, overwritten (per-row Delta
 *                   and LSE in base 2); may be NULL when Nq = 0
 * dq, dk and dv are fully written: rows and keys that see nothing get 0.
 * With GQA, dk / dv of a KV head sum the G query heads that read it (no
 * atomics: one work group owns each key tile).  Outputs must not overlap the
 * inputs or the workspace.  Nq or Nk may be 0; tensors without rows may then
 * be NULL.  Three kernels run on `stream`, in order.
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq);

int attn_bwd(const void* q, const int64_t q_stride[3],
             const void* k, const int64_t k_stride[3],
             const void* v, const int64_t v_stride[3],
             const void* o, const int64_t o_stride[3],
             const void* d_o, const int64_t do_stride[3], const float* lse,
             void* dq, const int64_t dq_stride[3],
             void* dk, const int64_t dk_stride[3],
             void* dv, const int64_t dv_stride[3],
             int B, int Hq, int Hkv, int Nq, int Nk, int D, int dtype, float scale,
             const attn_mask_desc* mask, const attn_score_mod* smod,
             float* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---- measurement helper -----------------------------------------------------
 * attn_probe_stream_read: reads `bytes` of device memory at `src` once with a
 * plain streaming kernel (16-byte loads, `blocks` work groups of 256 threads,
 * grid-stride) and writes one 32-bit fold per work group to `sink` (device
 * uint32 [blocks]).  No attention arithmetic: it gives the read rate a bare
 * stream reaches on the device, the ceiling the decode kernel's KV-read rate
 * is compared against.  src and bytes must be 16-byte aligned / a multiple of
 * 16 (ATTN_ERR_ALIGN); 1 <= blocks <= 2^20 (ATTN_ERR_SHAPE).
 */
int attn_probe_stream_read(const void* src, size_t bytes, int blocks, uint32_t* sink,
                           hipStream_t stream);

/* ---- backward pass over a BlockMask ------------------------------------------
 * attn_bwd_blockmask: the gradients of attn_fwd_blockmask's O (same Q, K, V,
 * mask, score_mod, BlockMask), by the same recomputation as attn_bwd.  The dQ
 * kernel walks a query tile's FULL / PARTIAL key tiles from `bm` (the forward
 * lists); the dK / dV kernel walks a key tile's FULL / PARTIAL query tiles from
 * `bm_t`, the key-tile-major lists attn_blockmask_transpose builds from `bm`.
 * FULL tiles apply no predicate, PARTIAL tiles the `mask` intervals (the
 * FlexAttention article, section 1: BlockMask block sparsity; the DeepSeek
 * v2->v4 article, section 2: segmented recomputation).  Arguments and
 * workspace as attn_bwd; bm as attn_fwd_blockmask's; bm_t->Bm / Hm equal
 * bm's and bm_t->nQt = bm->nKt, bm_t->nKt = bm->nQt (ATTN_ERR_BLOCKMASK
 * otherwise).  No score change is taken here (ATTN_ERR_SCORE_MOD).
 */
int attn_bwd_blockmask(const void* q, const int64_t q_stride[3],
                       const void* k, const int64_t k_stride[3],
                       const void* v, const int64_t v_stride[3],
                       const void* o, const int64_t o_stride[3],
                       const void* d_o, const int64_t do_stride[3], const float* lse,
                       void* dq, const int64_t dq_stride[3],
                       void* dk, const int64_t dk_stride[3],
                       void* dv, const int64_t dv_stride[3],
                       int B, int Hq, int Hkv, int Nq, int Nk, int D, int dtype, float scale,
                       const attn_mask_desc* mask, const attn_score_mod* smod,
                       const attn_blockmask* bm, const attn_blockmask* bm_t,
                       float* workspace, size_t workspace_bytes, hipStream_t stream);

/* attn_blockmask_transpose: fills `out` with the key-tile-major lists of `bm`:
 * row kt of (batch row, head) lists, ascending, the query tiles whose tile
 * (qt, kt) is PARTIAL / FULL in `bm`.  out->Bm / Hm must equal bm's, out->nQt
 * = bm->nKt and out->nKt = bm->nQt; its arrays are caller-allocated
 * (attn_blockmask_bytes(Bm, Hm, bm->nKt, bm->nQt)).  map_tmp is device memory
 * of at least Bm * Hm * nQt * nKt bytes, overwritten (a class map); a count
 * that would not fit a size_t gives ATTN_ERR_BLOCKMASK.
 */
int attn_blockmask_transpose(const attn_blockmask* bm, attn_blockmask* out, uint8_t* map_tmp,
                             size_t map_tmp_bytes, hipStream_t stream);

/* Human-readable text of a status code (static storage). */
const char* attn_status_str(int status);

/* ABI version, bumped on any signature or semantic change. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TILED_ATTN_H */
