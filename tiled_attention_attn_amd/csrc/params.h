// Kernel parameter blocks (passed by value to the kernels), shared by the
// kernel sources and the host-side C ABI that fills them.  Tensor pointers
// are untyped: each kernel is instantiated for its element type (bf16 or
// fp16) and casts them.
#pragma once

#include "common.h"

namespace tattn {

// Prefill (dense-mask and BlockMask variants).
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_sb, q_sh, q_sn, k_sb, k_sh, k_sn, v_sb, v_sh, v_sn, o_sb, o_sh, o_sn;
  int B, Hq, Hkv, G, Nq, Nk;
  float c2;  // scale * log2(e): scores live in base-2 units inside the kernel
  MaskParams mask;
  ScoreParams smod;
  const int32_t* part_num;
  const int32_t* part_idx;
  const int32_t* full_num;
  const int32_t* full_idx;
  int bm_B, bm_H, nKt;
  int n_qt;     // query tiles of 128 rows
  int n_slots;  // work groups per (batch, head)
  int paired;   // slot i also does tile n_qt-1-i
  int xcd_remap;
  uint32_t sched;  // ATTN_SCHED_* bits of the call
};

// BlockMask transposition: class map [Bm][Hm][nKt][nQt] from the lists.
struct BmTransposeParams {
  const int32_t* part_num;
  const int32_t* part_idx;
  const int32_t* full_num;
  const int32_t* full_idx;
  int Bm, Hm, nQt, nKt;
  uint8_t* map_t;
};

// BlockMask builder.
struct BmBuildParams {
  MaskParams mask;
  const uint8_t* tile_map;
  int Nq, Nk;
  int64_t shift;  // Nk - Nq
  int Bm, Hm, nQt, nKt;
  int32_t* part_num;
  int32_t* part_idx;
  int32_t* full_num;
  int32_t* full_idx;
};

// Split-KV decode, over a paged KV pool (block table) or over contiguous,
// strided K/V tensors [B, Hkv, Nk, D].
struct DecParams {
  const void* q;
  int64_t q_sb, q_sh, q_sn;
  const void* kc;
  const void* vc;
  // Element strides of K and V.  Paged: sn = slot stride inside a page
  // (Hkv * D), sh = head stride (D), sb unused.  Contiguous: batch, head and
  // token strides of the caller's tensors.
  int64_t k_sb, k_sh, k_sn, v_sb, v_sh, v_sn;
  const int32_t* bt;        // paged only
  int64_t bt_stride;
  const int32_t* seq_lens;  // paged only; contiguous sequences all have max_keys keys
  int B, Hq, Hkv, G, Lq, ps, S, chunk;  // chunk: keys per split (multiple of ps)
  int rows, n_rg;                       // G*Lq query rows per KV head, groups of 64
  int max_keys;                         // max_pages * page_size
  int64_t num_pages;                    // pool size (page indices are clamped to it)
  float c2;
  MaskParams mask;
  ScoreParams smod;
  float* ws_o;
  float* ws_lse;
  uint32_t sched;  // ATTN_SCHED_* bits of the call
};

// Backward pass (dQ, dK, dV by recomputation).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int64_t q_sb, q_sh, q_sn, k_sb, k_sh, k_sn, v_sb, v_sh, v_sn, o_sb, o_sh, o_sn;
  int64_t do_sb, do_sh, do_sn, dq_sb, dq_sh, dq_sn, dk_sb, dk_sh, dk_sn, dv_sb, dv_sh, dv_sn;
  int B, Hq, Hkv, G, Nq, Nk;
  int nq_pad;  // workspace rows per (batch, head): Nq rounded up to 64
  float c2;    // scale * log2(e)
  float scale;
  MaskParams mask;
  ScoreParams smod;
  float* ws_l2;     // [B*Hq][nq_pad]: LSE * log2(e); +inf for empty rows and padding
  float* ws_delta;  // [B*Hq][nq_pad]: rowsum(dO * O); 0 for padding
  int n_kt, kv_slots, kv_paired, kv_xcd_remap;  // 128-key tiles (dK / dV kernel)
  int n_qt, q_slots, q_paired, q_xcd_remap;     // 128-row tiles (dQ kernel)
  // BlockMask (attn_bwd_blockmask): the forward lists [bm_B][bm_H][n_qt][n_kt]
  // (dQ kernel) and the key-tile-major lists [bm_B][bm_H][n_kt][n_qt] (dK / dV).
  const int32_t* part_num;
  const int32_t* part_idx;
  const int32_t* full_num;
  const int32_t* full_idx;
  const int32_t* tpart_num;
  const int32_t* tpart_idx;
  const int32_t* tfull_num;
  const int32_t* tfull_idx;
  int bm_B, bm_H;
  uint32_t sched;  // ATTN_SCHED_* bits of the call
};

}  // namespace tattn
