// C ABI of the attention library: argument validation, launch geometry and
// status codes.  Everything here runs on the host; the work itself is in the
// kernels of fwd.hip, blockmask.hip and decode.hip.  Nothing is allocated,
// freed or synchronised here (see include/tiled_attn.h for the contract).
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "params.h"

namespace tattn {
int launch_fwd(const FwdParams& p, int D, bool blockmask, int dtype, hipStream_t stream);
int launch_blockmask(const BmBuildParams& p, hipStream_t stream);
int launch_decode(const DecParams& p, int D, int dtype, hipStream_t stream);
int launch_combine(const float* ws_o, const float* ws_lse, int B, int Hq, int Lq, int S, int D,
                   int dtype, void* o, int64_t o_sb, int64_t o_sh, int64_t o_sn, float* lse,
                   hipStream_t stream);
int launch_bwd(const BwdParams& p, int D, int dtype, bool blockmask, hipStream_t stream);
int launch_blockmask_transpose(const BmTransposeParams& p, hipStream_t stream);
}  // namespace tattn

using namespace tattn;

namespace {

constexpr int kMaxLen = 1 << 28;  // keeps every key / row index and product in range
constexpr int64_t kMaxRowStride = (int64_t)1 << 24;  // sequence stride of streamed tiles

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Product of byte-count factors, or 0 when it does not fit a size_t (the size
// helpers' "invalid sizes" answer).
size_t checked_product(std::initializer_list<size_t> factors) {
  size_t r = 1;
  for (size_t f : factors)
    if (__builtin_mul_overflow(r, f, &r)) return 0;
  return r;
}

int check_strides(const int64_t s[3]) {
  if (s == nullptr) return ATTN_ERR_NULL;
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || (s[i] & 7) != 0) return ATTN_ERR_STRIDE;
  return ATTN_OK;
}

int check_scale(float scale) {
  return (std::isfinite(scale) && scale > 0.f) ? ATTN_OK : ATTN_ERR_SCALE;
}

int check_dtype(int dtype) {
  return (dtype == ATTN_DTYPE_BF16 || dtype == ATTN_DTYPE_F16) ? ATTN_OK : ATTN_ERR_DTYPE;
}

// Converts the public mask descriptor; `allow_doc` is false for decode.  The
// schedule bits go to `sched` (0 when there are none).
int make_mask(const attn_mask_desc* m, int Nq, int Nk, bool allow_doc, MaskParams& out,
              uint32_t* sched = nullptr) {
  out = MaskParams{0u, -1, -1, 1, nullptr, 1, 2};
  if (sched) *sched = 0u;
  if (m == nullptr) return ATTN_OK;
  if (m->flags & ~(ATTN_MASK_ALL | ATTN_SCHED_ALL)) return ATTN_ERR_MASK;
  out.flags = m->flags & ATTN_MASK_ALL;
  if (sched) *sched = m->flags & ATTN_SCHED_ALL;
  out.wl = m->window_left < 0 ? -1 : m->window_left;
  out.wr = m->window_right < 0 ? -1 : m->window_right;
  if (m->flags & ATTN_MASK_BLOCK_CAUSAL) {
    if (m->block_size <= 0) return ATTN_ERR_MASK;
    out.bs = m->block_size;
  }
  if (m->flags & ATTN_MASK_DOCUMENT) {
    if (!allow_doc) return ATTN_ERR_MASK;
    if (m->doc_offsets == nullptr) return ATTN_ERR_NULL;
    if (m->num_docs < 1 || (int64_t)m->doc_stride < (int64_t)m->num_docs + 1) return ATTN_ERR_MASK;
    if (Nq > Nk) return ATTN_ERR_MASK;
    out.doc = m->doc_offsets;
    out.num_docs = m->num_docs;
    out.doc_stride = m->doc_stride;
  }
  return ATTN_OK;
}

// Converts the public score_mod descriptor.  `G_bwd` > 0 (the backward
// pass) also bounds the G bias tables one work group stages.
int make_smod(const attn_score_mod* m, float scale, int G_bwd, ScoreParams& out) {
  out = ScoreParams{0u, nullptr, nullptr, 0, 0.f, 0.f};
  if (m == nullptr || m->flags == 0) return ATTN_OK;
  const uint32_t f = m->flags;
  if (f & ~ATTN_SCORE_ALL) return ATTN_ERR_SCORE_MOD;
  if ((f & ATTN_SCORE_ALIBI) && (f & ATTN_SCORE_ALIBI_SYM)) return ATTN_ERR_SCORE_MOD;
  if ((f & (ATTN_SCORE_ALIBI | ATTN_SCORE_ALIBI_SYM)) && m->slopes == nullptr) return ATTN_ERR_NULL;
  if (f & ATTN_SCORE_REL_BIAS) {
    if (m->rel_bias == nullptr) return ATTN_ERR_NULL;
    if (m->rel_radius < 0 || m->rel_radius > (kMaxRelTable - 1) / 2) return ATTN_ERR_SCORE_MOD;
    if (G_bwd > 0 && (int64_t)G_bwd * (2 * m->rel_radius + 1) > 8192) return ATTN_ERR_SCORE_MOD;
  }
  if (f & ATTN_SCORE_SOFTCAP) {
    if (!(std::isfinite(m->softcap) && m->softcap > 0.f)) return ATTN_ERR_SCORE_MOD;
    out.cap_in = scale / m->softcap;
    out.cap_out = m->softcap * 1.4426950408889634f;
  }
  out.flags = f;
  out.slopes = m->slopes;
  out.rel = m->rel_bias;
  out.R = m->rel_radius;
  return ATTN_OK;
}

int check_common(const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                 const void* v, const int64_t* vs, const void* o, const int64_t* os, int B,
                 int Hq, int Hkv, int Nq, int Nk, int D, int dtype, float scale) {
  // K and V may be NULL when there are no keys (an empty tensor has no storage).
  if (!q || !o || (Nk > 0 && (!k || !v))) return ATTN_ERR_NULL;
  int st;
  if ((st = check_strides(qs)) || (st = check_strides(ks)) || (st = check_strides(vs)) ||
      (st = check_strides(os)))
    return st;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SHAPE;
  if (Nq > kMaxLen || Nk > kMaxLen || B > 65535 || Hq > 65535) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if ((st = check_dtype(dtype))) return st;
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (!aligned16(q) || !aligned16(o) || (Nk > 0 && (!aligned16(k) || !aligned16(v))))
    return ATTN_ERR_ALIGN;
  // The prefill kernels address a K/V tile of up to 128 rows with 32-bit
  // byte offsets: 127 rows of 2^24 - 8 elements stay below 2^32 bytes.
  if (ks[2] >= kMaxRowStride || vs[2] >= kMaxRowStride) return ATTN_ERR_STRIDE;
  return check_scale(scale);
}

void fill_fwd(FwdParams& p, const void* q, const int64_t* qs, const void* k, const int64_t* ks,
              const void* v, const int64_t* vs, void* o, const int64_t* os, float* lse, int B,
              int Hq, int Hkv, int Nq, int Nk, float scale) {
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.q_sb = qs[0]; p.q_sh = qs[1]; p.q_sn = qs[2];
  p.k_sb = ks[0]; p.k_sh = ks[1]; p.k_sn = ks[2];
  p.v_sb = vs[0]; p.v_sh = vs[1]; p.v_sn = vs[2];
  p.o_sb = os[0]; p.o_sh = os[1]; p.o_sn = os[2];
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.Nq = Nq; p.Nk = Nk;
  p.c2 = scale * 1.4426950408889634f;
  p.n_qt = (Nq + 127) / 128;
  p.part_num = p.part_idx = p.full_num = p.full_idx = nullptr;
  p.bm_B = p.bm_H = 1;
  p.nKt = (Nk + 127) / 128;
}

// Work-group counts (and the (batch, head, tile) indices the kernels derive
// from them in 32-bit arithmetic) must stay within a 1-D grid: at most
// 2^31 - 1 groups.
bool grid_fits(int64_t groups) { return groups <= 0x7fffffffLL; }

bool causal_like(const MaskParams& m) {
  return (m.flags & (ATTN_MASK_CAUSAL | ATTN_MASK_BLOCK_CAUSAL)) != 0 &&
         !(m.flags & (ATTN_MASK_WINDOW | ATTN_MASK_DOCUMENT));
}

void set_slots(FwdParams& p, bool paired) {
  p.paired = paired && p.n_qt > 1 && !(p.sched & ATTN_SCHED_NO_PAIRING);
  p.n_slots = p.paired ? (p.n_qt + 1) / 2 : p.n_qt;
  const long units = (long)p.B * p.Hq * p.n_slots;
  p.xcd_remap = (units % 8) == 0 && !(p.sched & ATTN_SCHED_NO_XCD_REMAP);
}

// Shape-based choice of attn_fwd_auto.  A decode-shaped call -- all G * Nq
// query rows of a KV head fit one 64-row group of the split-KV kernel, and
// there are at least kAutoMinKeys keys -- runs split-KV + combine: K/V are
// read once per KV head instead of once per query head, and the key splits
// fill the GPU even when B * Hkv cannot.
constexpr int kAutoMinKeys = 512;
constexpr int kAutoSplitKeys = 256;  // fewest keys per split
constexpr long kAutoTargetGroups = 2L * 256;  // two work groups per CU on 256 CUs

struct AutoPlan {
  int path, S, chunk;
  size_t ws_o_bytes, ws_bytes;
};

AutoPlan auto_plan(int B, int Hq, int Hkv, int Nq, int Nk, int D, const attn_score_mod* smod) {
  (void)smod;  // every score change runs on both paths
  AutoPlan pl{ATTN_PATH_PREFILL, 0, 0, 0, 0};
  const long rows = (long)(Hq / Hkv) * Nq;
  if (Nq < 1 || rows > 64 || Nk < kAutoMinKeys) return pl;
  // the combine numbers its B * Hq * Nq rows in int (as attn_decode_combine bounds them)
  if ((long)B * Hq * Nq > 0x7fffffffL - 3) return pl;
  const long units = (long)B * Hkv;
  long S = units > 0 ? (kAutoTargetGroups + units - 1) / units : 1;
  const long max_s = Nk / kAutoSplitKeys;
  if (S > max_s) S = max_s;
  if (S < 1) S = 1;
  // keys per split, a whole number of 64-key steps; no split left empty
  const long chunk = ((Nk + S - 1) / S + 63) / 64 * 64;
  S = (Nk + chunk - 1) / chunk;
  pl.path = ATTN_PATH_SPLITKV;
  pl.S = (int)S;
  pl.chunk = (int)chunk;
  const size_t parts = (size_t)B * Hq * Nq * S;
  pl.ws_o_bytes = (parts * D * sizeof(float) + 255) / 256 * 256;
  pl.ws_bytes = pl.ws_o_bytes + parts * sizeof(float);
  return pl;
}

}  // namespace

namespace {

int bwd_impl(const void* q, const int64_t q_stride[3], const void* k, const int64_t k_stride[3],
             const void* v, const int64_t v_stride[3], const void* o, const int64_t o_stride[3],
             const void* d_o, const int64_t do_stride[3], const float* lse, void* dq,
             const int64_t dq_stride[3], void* dk, const int64_t dk_stride[3], void* dv,
             const int64_t dv_stride[3], int B, int Hq, int Hkv, int Nq, int Nk, int D,
             int dtype, float scale, const attn_mask_desc* mask, const attn_score_mod* smod,
             float* workspace, size_t workspace_bytes, const attn_blockmask* bm,
             const attn_blockmask* bm_t, hipStream_t stream) {
  // Tensors without rows may be NULL (an empty tensor has no storage).
  if (Nq > 0 && (!q || !o || !d_o || !dq || !lse)) return ATTN_ERR_NULL;
  if (Nk > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL;
  if (!workspace && Nq > 0) return ATTN_ERR_NULL;
  const int64_t* all[8] = {q_stride, k_stride, v_stride, o_stride, do_stride, dq_stride, dk_stride,
                           dv_stride};
  int st;
  for (const int64_t* s : all)
    if ((st = check_strides(s))) return st;
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SHAPE;
  if (Nq > kMaxLen || Nk > kMaxLen || B > 65535 || Hq > 65535) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if ((st = check_dtype(dtype))) return st;
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  const void* ptrs[9] = {q, k, v, o, d_o, dq, dk, dv, workspace};
  for (const void* x : ptrs)
    if (x && !aligned16(x)) return ATTN_ERR_ALIGN;
  // K / V tiles (dQ kernel) and Q / dO tiles (dK / dV kernel) are streamed
  // with 32-bit byte offsets.
  if (k_stride[2] >= kMaxRowStride || v_stride[2] >= kMaxRowStride ||
      q_stride[2] >= kMaxRowStride || do_stride[2] >= kMaxRowStride)
    return ATTN_ERR_STRIDE;
  if ((st = check_scale(scale))) return st;
  if (bm != nullptr) {
    // the forward lists (dQ) and their key-tile-major transpose (dK / dV)
    if (bm_t == nullptr) return ATTN_ERR_NULL;
    if (!bm->part_num || !bm->part_idx || !bm->full_num || !bm->full_idx || !bm_t->part_num ||
        !bm_t->part_idx || !bm_t->full_num || !bm_t->full_idx)
      return ATTN_ERR_NULL;
    if (bm->nQt != (Nq + 127) / 128 || bm->nKt != (Nk + 127) / 128) return ATTN_ERR_BLOCKMASK;
    if (!(bm->Bm == 1 || bm->Bm == B) || !(bm->Hm == 1 || bm->Hm == Hq)) return ATTN_ERR_BLOCKMASK;
    if (bm_t->Bm != bm->Bm || bm_t->Hm != bm->Hm || bm_t->nQt != bm->nKt || bm_t->nKt != bm->nQt)
      return ATTN_ERR_BLOCKMASK;
  }
  BwdParams p;
  if ((st = make_mask(mask, Nq, Nk, true, p.mask, &p.sched))) return st;
  if ((st = make_smod(smod, scale, Hq / Hkv, p.smod))) return st;
  // The BlockMask backward kernels take no score change.
  if (bm != nullptr && p.smod.flags != 0) return ATTN_ERR_SCORE_MOD;
  if (workspace_bytes < attn_bwd_workspace_bytes(B, Hq, Nq)) return ATTN_ERR_WORKSPACE;
  if (B == 0 || (Nq == 0 && Nk == 0)) return ATTN_OK;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = d_o;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.q_sb = q_stride[0]; p.q_sh = q_stride[1]; p.q_sn = q_stride[2];
  p.k_sb = k_stride[0]; p.k_sh = k_stride[1]; p.k_sn = k_stride[2];
  p.v_sb = v_stride[0]; p.v_sh = v_stride[1]; p.v_sn = v_stride[2];
  p.o_sb = o_stride[0]; p.o_sh = o_stride[1]; p.o_sn = o_stride[2];
  p.do_sb = do_stride[0]; p.do_sh = do_stride[1]; p.do_sn = do_stride[2];
  p.dq_sb = dq_stride[0]; p.dq_sh = dq_stride[1]; p.dq_sn = dq_stride[2];
  p.dk_sb = dk_stride[0]; p.dk_sh = dk_stride[1]; p.dk_sn = dk_stride[2];
  p.dv_sb = dv_stride[0]; p.dv_sh = dv_stride[1]; p.dv_sn = dv_stride[2];
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = Hq / Hkv; p.Nq = Nq; p.Nk = Nk;
  p.nq_pad = (Nq + 63) / 64 * 64;
  p.c2 = scale * 1.4426950408889634f;
  p.scale = scale;
  p.ws_l2 = workspace;
  p.ws_delta = workspace + (size_t)B * Hq * p.nq_pad;
  // Causal-like masks give later query tiles more keys and earlier key tiles
  // more rows: pair tile i with n-1-i in both kernels.
  // BlockMask lists are paired like the forward BlockMask kernel's.
  const bool pair = (bm != nullptr || causal_like(p.mask)) && !(p.sched & ATTN_SCHED_NO_PAIRING);
  const bool remap = !(p.sched & ATTN_SCHED_NO_XCD_REMAP);
  p.n_kt = (Nk + 127) / 128;
  p.kv_paired = pair && p.n_kt > 1;
  p.kv_slots = p.kv_paired ? (p.n_kt + 1) / 2 : p.n_kt;
  p.kv_xcd_remap = remap && ((long)B * Hkv * p.kv_slots) % 8 == 0;
  p.n_qt = (Nq + 127) / 128;
  p.q_paired = pair && p.n_qt > 1;
  p.q_slots = p.q_paired ? (p.n_qt + 1) / 2 : p.n_qt;
  p.q_xcd_remap = remap && ((long)B * Hq * p.q_slots) % 8 == 0;
  // dQ groups B Hq n_qt, dK/dV groups B Hkv n_kt, Delta threads 8 per padded row
  if (!grid_fits((int64_t)B * Hq * p.n_qt) || !grid_fits((int64_t)B * Hkv * p.n_kt) ||
      !grid_fits(((int64_t)B * Hq * p.nq_pad * 8 + 255) / 256))
    return ATTN_ERR_SHAPE;
  p.bm_B = bm ? bm->Bm : 1;
  p.bm_H = bm ? bm->Hm : 1;
  p.part_num = bm ? bm->part_num : nullptr;
  p.part_idx = bm ? bm->part_idx : nullptr;
  p.full_num = bm ? bm->full_num : nullptr;
  p.full_idx = bm ? bm->full_idx : nullptr;
  p.tpart_num = bm ? bm_t->part_num : nullptr;
  p.tpart_idx = bm ? bm_t->part_idx : nullptr;
  p.tfull_num = bm ? bm_t->full_num : nullptr;
  p.tfull_idx = bm ? bm_t->full_idx : nullptr;
  return launch_bwd(p, D, dtype, bm != nullptr, stream);
}

}  // namespace

extern "C" {

int attn_abi_version(void) { return 8; }

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "a size is negative or over its limit";
    case ATTN_ERR_HEAD_DIM: return "head dim D must be 64 or 128";
    case ATTN_ERR_GQA: return "Hq must be a positive multiple of Hkv";
    case ATTN_ERR_STRIDE: return "strides must be non-negative multiples of 8 elements";
    case ATTN_ERR_ALIGN: return "tensor base pointers must be 16-byte aligned";
    case ATTN_ERR_MASK: return "unknown mask flag or bad mask parameter";
    case ATTN_ERR_WORKSPACE: return "workspace or split arguments inconsistent";
    case ATTN_ERR_LAUNCH: return "the HIP runtime reported a launch error";
    case ATTN_ERR_BLOCKMASK: return "BlockMask descriptor inconsistent with the shapes";
    case ATTN_ERR_SCALE: return "scale must be finite and > 0";
    case ATTN_ERR_DTYPE: return "dtype must be ATTN_DTYPE_BF16 or ATTN_DTYPE_F16";
    case ATTN_ERR_SCORE_MOD: return "bad score_mod flags or parameters, or a score_mod this entry point does not take";
    default: return "unknown status";
  }
}

int attn_fwd(const void* q, const int64_t q_stride[3], const void* k, const int64_t k_stride[3],
             const void* v, const int64_t v_stride[3], void* o, const int64_t o_stride[3],
             float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int D, int dtype, float scale,
             const attn_mask_desc* mask, const attn_score_mod* smod, hipStream_t stream) {
  int st = check_common(q, q_stride, k, k_stride, v, v_stride, o, o_stride, B, Hq, Hkv, Nq, Nk,
                        D, dtype, scale);
  if (st) return st;
  FwdParams p;
  if ((st = make_mask(mask, Nq, Nk, true, p.mask, &p.sched))) return st;
  if ((st = make_smod(smod, scale, 0, p.smod))) return st;
  if (B == 0 || Nq == 0) return ATTN_OK;
  if (!grid_fits((int64_t)B * Hq * ((Nq + 127) / 128))) return ATTN_ERR_SHAPE;
  fill_fwd(p, q, q_stride, k, k_stride, v, v_stride, o, o_stride, lse, B, Hq, Hkv, Nq, Nk, scale);
  // Causal-like masks give later query tiles more keys: pair tile i with n-1-i.
  set_slots(p, causal_like(p.mask));
  return launch_fwd(p, D, false, dtype, stream);
}

size_t attn_blockmask_bytes(int Bm, int Hm, int nQt, int nKt) {
  if (Bm <= 0 || Hm <= 0 || nQt < 0 || nKt < 0) return 0;
  const size_t counts = checked_product({(size_t)Bm, (size_t)Hm, (size_t)nQt, 2 * sizeof(int32_t)});
  const size_t lists = checked_product({counts, (size_t)nKt});
  size_t total = 0;
  if ((nQt > 0 && counts == 0) || (nKt > 0 && counts != 0 && lists == 0) ||
      __builtin_add_overflow(counts, lists, &total))
    return 0;
  return total;
}

int attn_build_blockmask(const attn_mask_desc* mask, const uint8_t* tile_map, int B, int Nq,
                         int Nk, attn_blockmask* out, hipStream_t stream) {
  if (out == nullptr) return ATTN_ERR_NULL;
  if (!out->part_num || !out->part_idx || !out->full_num || !out->full_idx) return ATTN_ERR_NULL;
  if (Nq < 0 || Nk < 0 || Nq > kMaxLen || Nk > kMaxLen) return ATTN_ERR_SHAPE;
  if (out->Bm < 1 || out->Hm < 1 || out->Bm > 65535 || out->Hm > 65535) return ATTN_ERR_BLOCKMASK;
  if (out->nQt != (Nq + 127) / 128 || out->nKt != (Nk + 127) / 128) return ATTN_ERR_BLOCKMASK;
  BmBuildParams p;
  int st = make_mask(mask, Nq, Nk, true, p.mask);
  if (st) return st;
  if (tile_map == nullptr) {
    if (mask == nullptr) return ATTN_ERR_NULL;
    if ((p.mask.flags & ATTN_MASK_DOCUMENT) && out->Bm != B) return ATTN_ERR_BLOCKMASK;
  }
  if (out->nQt == 0) return ATTN_OK;
  p.tile_map = tile_map;
  p.Nq = Nq;
  p.Nk = Nk;
  p.shift = (int64_t)Nk - Nq;
  p.Bm = out->Bm; p.Hm = out->Hm; p.nQt = out->nQt; p.nKt = out->nKt;
  p.part_num = out->part_num; p.part_idx = out->part_idx;
  p.full_num = out->full_num; p.full_idx = out->full_idx;
  return launch_blockmask(p, stream);
}

int attn_fwd_blockmask(const void* q, const int64_t q_stride[3], const void* k,
                       const int64_t k_stride[3], const void* v, const int64_t v_stride[3],
                       void* o, const int64_t o_stride[3], float* lse, int B, int Hq, int Hkv,
                       int Nq, int Nk, int D, int dtype, float scale, const attn_mask_desc* mask,
                       const attn_score_mod* smod, const attn_blockmask* bm, hipStream_t stream) {
  int st = check_common(q, q_stride, k, k_stride, v, v_stride, o, o_stride, B, Hq, Hkv, Nq, Nk,
                        D, dtype, scale);
  if (st) return st;
  if (bm == nullptr) return ATTN_ERR_NULL;
  if (!bm->part_num || !bm->part_idx || !bm->full_num || !bm->full_idx) return ATTN_ERR_NULL;
  if (bm->nQt != (Nq + 127) / 128 || bm->nKt != (Nk + 127) / 128) return ATTN_ERR_BLOCKMASK;
  if (!(bm->Bm == 1 || bm->Bm == B) || !(bm->Hm == 1 || bm->Hm == Hq)) return ATTN_ERR_BLOCKMASK;
  FwdParams p;
  if ((st = make_mask(mask, Nq, Nk, true, p.mask, &p.sched))) return st;
  if ((st = make_smod(smod, scale, 0, p.smod))) return st;
  if (B == 0 || Nq == 0) return ATTN_OK;
  if (!grid_fits((int64_t)B * Hq * ((Nq + 127) / 128))) return ATTN_ERR_SHAPE;
  fill_fwd(p, q, q_stride, k, k_stride, v, v_stride, o, o_stride, lse, B, Hq, Hkv, Nq, Nk, scale);
  p.part_num = bm->part_num; p.part_idx = bm->part_idx;
  p.full_num = bm->full_num; p.full_idx = bm->full_idx;
  p.bm_B = bm->Bm; p.bm_H = bm->Hm;
  set_slots(p, true);
  return launch_fwd(p, D, true, dtype, stream);
}

size_t attn_decode_ws_o_bytes(int B, int Hq, int Lq, int D, int num_splits) {
  if (B < 0 || Hq < 0 || Lq < 0 || D <= 0 || num_splits <= 0) return 0;
  return checked_product({(size_t)B, (size_t)Hq, (size_t)Lq, (size_t)num_splits, (size_t)D,
                          sizeof(float)});
}

size_t attn_decode_ws_lse_bytes(int B, int Hq, int Lq, int num_splits) {
  if (B < 0 || Hq < 0 || Lq < 0 || num_splits <= 0) return 0;
  return checked_product({(size_t)B, (size_t)Hq, (size_t)Lq, (size_t)num_splits, sizeof(float)});
}

int attn_decode_num_splits(int B, int Hkv, int max_pages, int num_cus) {
  if (B <= 0 || Hkv <= 0 || max_pages <= 0) return 1;
  if (num_cus <= 0) num_cus = 256;
  // Two resident work groups per compute unit (72 KB of LDS each): enough
  // splits for two per CU, no more splits than pages, and at most 2048 pages
  // per split.
  const long units = (long)B * Hkv;
  const long target = 2L * num_cus;
  long s = (target + units - 1) / units;
  if (s < 1) s = 1;
  const long min_s = ((long)max_pages + 2047) / 2048;
  if (s < min_s) s = min_s;
  if (s > max_pages) s = max_pages;
  return (int)s;
}

int attn_decode_splitkv(const void* q, const int64_t q_stride[3], const void* k_cache,
                        const void* v_cache, int64_t num_pages, const int32_t* block_table,
                        int64_t bt_stride, const int32_t* seq_lens, int max_pages, int B, int Hq,
                        int Hkv, int Lq, int D, int dtype, int page_size, int num_splits, float scale,
                        const attn_mask_desc* mask, const attn_score_mod* smod, float* ws_o,
                        float* ws_lse, hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !ws_o || !ws_lse)
    return ATTN_ERR_NULL;
  int st = check_strides(q_stride);
  if (st) return st;
  if (B < 0 || Hq < 0 || Hkv < 0 || Lq < 0 || num_pages < 1 || page_size < 1 || max_pages < 1)
    return ATTN_ERR_SHAPE;
  if (B > 65535 || Hq > 65535 || Hkv > 65535 || Lq > 65536) return ATTN_ERR_SHAPE;
  // rows = G * Lq query rows per KV head stay well inside int
  if ((int64_t)(Hkv > 0 ? Hq / Hkv : 0) * Lq > kMaxLen) return ATTN_ERR_SHAPE;
  if ((int64_t)max_pages * page_size > kMaxLen) return ATTN_ERR_SHAPE;
  if (bt_stride < max_pages) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if ((st = check_dtype(dtype))) return st;
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(ws_o))
    return ATTN_ERR_ALIGN;
  if ((st = check_scale(scale))) return st;
  if (num_splits < 1 || num_splits > 65536) return ATTN_ERR_WORKSPACE;
  // A split's block-table entries are staged in LDS: at most 2048 pages each.
  if ((max_pages + num_splits - 1) / num_splits > 2048) return ATTN_ERR_WORKSPACE;
  DecParams p;
  attn_mask_desc causal = {ATTN_MASK_CAUSAL, -1, -1, 0, nullptr, 0, 0};
  if ((st = make_mask(mask ? mask : &causal, 0, 0, false, p.mask, &p.sched))) return st;
  if ((st = make_smod(smod, scale, 0, p.smod))) return st;
  if (B == 0 || Lq == 0) return ATTN_OK;
  const int G = Hq / Hkv;
  p.q = q;
  p.q_sb = q_stride[0]; p.q_sh = q_stride[1]; p.q_sn = q_stride[2];
  p.kc = k_cache;
  p.vc = v_cache;
  p.k_sb = p.v_sb = 0;
  p.k_sh = p.v_sh = D;
  p.k_sn = p.v_sn = (int64_t)Hkv * D;
  p.bt = block_table;
  p.bt_stride = bt_stride;
  p.seq_lens = seq_lens;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = G; p.Lq = Lq; p.ps = page_size; p.S = num_splits;
  p.chunk = page_size * ((max_pages + num_splits - 1) / num_splits);
  p.max_keys = max_pages * page_size;
  p.num_pages = num_pages;
  p.rows = G * Lq;
  p.n_rg = (p.rows + 63) / 64;
  if ((long)p.S * p.n_rg > 0x7fffffffL) return ATTN_ERR_SHAPE;
  // partials of more bytes than a size_t holds: no workspace can be that large
  if (attn_decode_ws_o_bytes(B, Hq, Lq, D, num_splits) == 0) return ATTN_ERR_SHAPE;
  p.c2 = scale * 1.4426950408889634f;
  p.ws_o = ws_o;
  p.ws_lse = ws_lse;
  return launch_decode(p, D, dtype, stream);
}

int attn_decode_combine(const float* ws_o, const float* ws_lse, int B, int Hq, int Lq, int S,
                        int D, int dtype, void* o, const int64_t o_stride[3], float* lse,
                        hipStream_t stream) {
  if (!ws_o || !ws_lse || !o) return ATTN_ERR_NULL;
  int st = check_strides(o_stride);
  if (st) return st;
  if (B < 0 || Hq < 0 || Lq < 0) return ATTN_ERR_SHAPE;
  // B * Hq < 2^62; the product with Lq may not fit.  The combine kernel numbers
  // rows 4 * group + wave in int, so its last group must stay below 2^31.
  int64_t rows = 0;
  if (__builtin_mul_overflow((int64_t)B * Hq, (int64_t)Lq, &rows) || rows > 0x7fffffffL - 3)
    return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if ((st = check_dtype(dtype))) return st;
  if (S < 1 || S > 65536) return ATTN_ERR_WORKSPACE;
  if (!aligned16(o) || !aligned16(ws_o)) return ATTN_ERR_ALIGN;
  if (B == 0 || Hq == 0 || Lq == 0) return ATTN_OK;
  return launch_combine(ws_o, ws_lse, B, Hq, Lq, S, D, dtype, o, o_stride[0], o_stride[1],
                        o_stride[2], lse, stream);
}

int attn_fwd_auto_plan(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                       const attn_score_mod* smod, attn_auto_plan* out) {
  if (out == nullptr) return ATTN_ERR_NULL;
  *out = attn_auto_plan{ATTN_PATH_PREFILL, 0, 0};
  if (B < 0 || Hq < 0 || Hkv < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SHAPE;
  if (Nq > kMaxLen || Nk > kMaxLen || B > 65535 || Hq > 65535) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (Hkv == 0 || Hq == 0 || Hq % Hkv != 0) return ATTN_ERR_GQA;
  AutoPlan pl = auto_plan(B, Hq, Hkv, Nq, Nk, D, smod);
  out->path = pl.path;
  out->num_splits = pl.S;
  out->workspace_bytes = pl.ws_bytes;
  return ATTN_OK;
}

int attn_fwd_auto(const void* q, const int64_t q_stride[3], const void* k,
                  const int64_t k_stride[3], const void* v, const int64_t v_stride[3], void* o,
                  const int64_t o_stride[3], float* lse, int B, int Hq, int Hkv, int Nq, int Nk,
                  int D, int dtype, float scale, const attn_mask_desc* mask,
                  const attn_score_mod* smod, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  int st = check_common(q, q_stride, k, k_stride, v, v_stride, o, o_stride, B, Hq, Hkv, Nq, Nk,
                        D, dtype, scale);
  if (st) return st;
  const AutoPlan pl = auto_plan(B, Hq, Hkv, Nq, Nk, D, smod);
  if (pl.path == ATTN_PATH_PREFILL)
    return attn_fwd(q, q_stride, k, k_stride, v, v_stride, o, o_stride, lse, B, Hq, Hkv, Nq, Nk,
                    D, dtype, scale, mask, smod, stream);
  DecParams p;
  if ((st = make_mask(mask, Nq, Nk, true, p.mask, &p.sched))) return st;
  if ((st = make_smod(smod, scale, 0, p.smod))) return st;
  if (B == 0 || Nq == 0) return ATTN_OK;
  if (workspace == nullptr) return ATTN_ERR_NULL;
  if (workspace_bytes < pl.ws_bytes) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  const int G = Hq / Hkv;
  p.q = q;
  p.q_sb = q_stride[0]; p.q_sh = q_stride[1]; p.q_sn = q_stride[2];
  p.kc = k;
  p.vc = v;
  p.k_sb = k_stride[0]; p.k_sh = k_stride[1]; p.k_sn = k_stride[2];
  p.v_sb = v_stride[0]; p.v_sh = v_stride[1]; p.v_sn = v_stride[2];
  p.bt = nullptr;
  p.bt_stride = 0;
  p.seq_lens = nullptr;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.G = G; p.Lq = Nq; p.ps = 1; p.S = pl.S;
  p.chunk = pl.chunk;
  p.max_keys = Nk;
  p.num_pages = 1;
  p.rows = G * Nq;
  p.n_rg = (p.rows + 63) / 64;
  p.c2 = scale * 1.4426950408889634f;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ws_o_bytes);
  if ((st = launch_decode(p, D, dtype, stream))) return st;
  return launch_combine(p.ws_o, p.ws_lse, B, Hq, Nq, pl.S, D, dtype, o, o_stride[0], o_stride[1],
                        o_stride[2], lse, stream);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq) {
  if (B < 0 || Hq < 0 || Nq < 0) return 0;
  const size_t pad = ((size_t)Nq + 63) / 64 * 64;
  return checked_product({2, (size_t)B, (size_t)Hq, pad, sizeof(float)});
}

int attn_bwd(const void* q, const int64_t q_stride[3], const void* k, const int64_t k_stride[3],
             const void* v, const int64_t v_stride[3], const void* o, const int64_t o_stride[3],
             const void* d_o, const int64_t do_stride[3], const float* lse, void* dq,
             const int64_t dq_stride[3], void* dk, const int64_t dk_stride[3], void* dv,
             const int64_t dv_stride[3], int B, int Hq, int Hkv, int Nq, int Nk, int D,
             int dtype, float scale, const attn_mask_desc* mask, const attn_score_mod* smod,
             float* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_impl(q, q_stride, k, k_stride, v, v_stride, o, o_stride, d_o, do_stride, lse, dq,
                  dq_stride, dk, dk_stride, dv, dv_stride, B, Hq, Hkv, Nq, Nk, D, dtype, scale,
                  mask, smod, workspace, workspace_bytes, nullptr, nullptr, stream);
}

int attn_bwd_blockmask(const void* q, const int64_t q_stride[3], const void* k,
                       const int64_t k_stride[3], const void* v, const int64_t v_stride[3],
                       const void* o, const int64_t o_stride[3], const void* d_o,
                       const int64_t do_stride[3], const float* lse, void* dq,
                       const int64_t dq_stride[3], void* dk, const int64_t dk_stride[3], void* dv,
                       const int64_t dv_stride[3], int B, int Hq, int Hkv, int Nq, int Nk, int D,
                       int dtype, float scale, const attn_mask_desc* mask,
                       const attn_score_mod* smod, const attn_blockmask* bm,
                       const attn_blockmask* bm_t, float* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (bm == nullptr || bm_t == nullptr) return ATTN_ERR_NULL;
  return bwd_impl(q, q_stride, k, k_stride, v, v_stride, o, o_stride, d_o, do_stride, lse, dq,
                  dq_stride, dk, dk_stride, dv, dv_stride, B, Hq, Hkv, Nq, Nk, D, dtype, scale,
                  mask, smod, workspace, workspace_bytes, bm, bm_t, stream);
}

int attn_blockmask_transpose(const attn_blockmask* bm, attn_blockmask* out, uint8_t* map_tmp,
                             size_t map_tmp_bytes, hipStream_t stream) {
  if (bm == nullptr || out == nullptr) return ATTN_ERR_NULL;
  if (!bm->part_num || !bm->part_idx || !bm->full_num || !bm->full_idx || !out->part_num ||
      !out->part_idx || !out->full_num || !out->full_idx)
    return ATTN_ERR_NULL;
  if (bm->Bm < 1 || bm->Hm < 1 || bm->Bm > 65535 || bm->Hm > 65535) return ATTN_ERR_BLOCKMASK;
  if (bm->nQt < 0 || bm->nKt < 0 || bm->nQt > (kMaxLen + 127) / 128 ||
      bm->nKt > (kMaxLen + 127) / 128)
    return ATTN_ERR_BLOCKMASK;
  if (out->Bm != bm->Bm || out->Hm != bm->Hm || out->nQt != bm->nKt || out->nKt != bm->nQt)
    return ATTN_ERR_BLOCKMASK;
  if (bm->nQt == 0 || bm->nKt == 0) return ATTN_OK;
  const size_t need = checked_product({(size_t)bm->Bm, (size_t)bm->Hm, (size_t)bm->nQt,
                                       (size_t)bm->nKt});
  if (need == 0) return ATTN_ERR_BLOCKMASK;  // more map bytes than a size_t holds
  if (map_tmp == nullptr) return ATTN_ERR_NULL;
  if (map_tmp_bytes < need) return ATTN_ERR_WORKSPACE;
  BmTransposeParams tp{bm->part_num, bm->part_idx, bm->full_num, bm->full_idx,
                       bm->Bm, bm->Hm, bm->nQt, bm->nKt, map_tmp};
  int st = launch_blockmask_transpose(tp, stream);
  if (st) return st;
  // the key-tile-major map compacted into lists by the builder (its map path)
  BmBuildParams p;
  p.mask = MaskParams{0u, -1, -1, 1, nullptr, 1, 2};
  p.tile_map = map_tmp;
  p.Nq = bm->nKt * 128;
  p.Nk = bm->nQt * 128;
  p.shift = 0;
  p.Bm = bm->Bm; p.Hm = bm->Hm; p.nQt = bm->nKt; p.nKt = bm->nQt;
  p.part_num = out->part_num; p.part_idx = out->part_idx;
  p.full_num = out->full_num; p.full_idx = out->full_idx;
  return launch_blockmask(p, stream);
}

}  // extern "C"
