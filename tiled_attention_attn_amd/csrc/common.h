// Device helpers shared by the gfx950 attention kernels: vector types, MFMA
// and LDS-transpose wrappers, cross-half exchanges, bf16 / fp16 packing and
// the per-row mask interval.  Q, K, V and O are 16-bit floats of one type T,
// bf16 or fp16; both have the same layouts, so every kernel is a template on
// T and only the MFMA opcode and the conversions differ.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tiled_attn.h"

namespace tattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define TATTN_LDS __attribute__((address_space(3)))

// Vectors of the element type T (bf16 or f16).
template <typename T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x8 x8; typedef bf16x4 x4; typedef bf16x2 x2; };
template <> struct Vec<f16> { typedef f16x8 x8; typedef f16x4 x4; typedef f16x2 x2; };
template <typename T> using vec8 = typename Vec<T>::x8;
template <typename T> using vec4 = typename Vec<T>::x4;
template <typename T> using vec2 = typename Vec<T>::x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---- MFMA ------------------------------------------------------------------
// 32x32x16 bf16: lane l holds A[m=l%32][k=8(l/32)+i], B[k=8(l/32)+i][n=l%32],
// C[m=8(r/4)+4(l/32)+r%4][n=l%32].  16x16x32 bf16: A[m=l%16][k=8(l/16)+i],
// B[k=8(l/16)+i][n=l%16], C[m=4(l/16)+r][n=l%16].  (Checked on gfx950 with an
// in-bounds probe of every lane and slot.)  The fp16 opcodes of the same
// shapes use the same register layouts.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---- LDS access --------------------------------------------------------------
template <typename T>
__device__ __forceinline__ vec8<T> lds_read_b128(const TATTN_LDS char* base, uint32_t byte_off) {
  return *reinterpret_cast<const TATTN_LDS vec8<T>*>(base + byte_off);
}

// ds_read_b64_tr_b16.  Within each 16-lane group, lane j reads 4 halfwords
// (row j of a 16x4 matrix M); lane i receives (M[i/4][i%4], M[4+i/4][i%4],
// M[8+i/4][i%4], M[12+i/4][i%4]).  So when lane j reads 8 bytes at
// row (base + j/4), columns (c0 + 4(j%4)) .. +3 of a row-major matrix, lane i
// receives column c0 + i of rows base .. base+3: a transposed 4-element load.
__device__ __forceinline__ i16x4 lds_read_tr16(const TATTN_LDS char* base, uint32_t byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<TATTN_LDS i16x4*>(const_cast<TATTN_LDS char*>(base) + byte_off));
}

template <typename T>
__device__ __forceinline__ vec8<T> join_tr(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(vec8<T>, v);
}

// Asynchronous 16-byte global -> LDS copy (global_load_lds_dwordx4): lane l's
// 16 bytes land at LDS address lds_wave_base + 16 * l; lds_wave_base must be
// wave-uniform.  Issued from inline assembly on purpose: the compiler then
// does not track these copies, so it adds no blanket vmcnt(0) wait in front
// of LDS reads it cannot prove disjoint (it does so for ds_read_b64_tr_b16),
// which would serialise the pipeline.  Completion is ordered explicitly by
// the callers: wait_vmem_le<N>() in each wave, then lds_barrier().  The
// instruction writes no VGPR, reads its address registers at issue, and the
// memory clobber keeps the compiler from moving other memory accesses across.
// The compiler writes M0 (the LDS address) right before the block; GFX9-family
// hardware needs one wait state between an SALU write of M0 and an LDS-DMA
// instruction that reads it (the compiler's hazard recognizer cannot see into
// the block), hence the s_nop.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_wave_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "{m0}"(lds_wave_base)
               : "memory");
}

// The same copy addressed as a uniform 64-bit base (SGPR pair) plus a 32-bit
// per-lane byte offset: no per-lane 64-bit address arithmetic is needed.
__device__ __forceinline__ void dma16_sv(const void* sbase, uint32_t voff_bytes,
                                         uint32_t lds_wave_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff_bytes), "s"(sbase), "{m0}"(lds_wave_base)
               : "memory");
}

// 32-bit LDS address of an LDS pointer.
__device__ __forceinline__ uint32_t lds_addr(const TATTN_LDS void* p) {
  return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ void wait_vmem() {  // vmcnt(0)
  __builtin_amdgcn_s_waitcnt(0x3f70);
  asm volatile("" ::: "memory");
}

// Work-group barrier for LDS hand-off only.  __syncthreads() adds a
// work-group release fence, which waits for every outstanding vector-memory
// operation (vmcnt(0)) -- including the asynchronous LDS copies of later
// pipeline stages.  Here each wave waits for its own copies explicitly
// (wait_vmem_le), finishes its LDS reads (lgkmcnt(0)) and then meets the
// others; the memory clobber keeps the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(N): wait until at most N vector-memory operations of this
// wave are outstanding (gfx9 encoding: vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x3f70 | (N & 15) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// ---- LDS limits ----------------------------------------------------------------
// Every kernel keeps two limits, checked at compile time beside its LDS
// declaration: its asynchronous global -> LDS copies land only in the first
// 64 KB of the work group's LDS (the copy ring is the work group's first,
// 1024-byte aligned LDS object), and its whole LDS footprint stays at or under
// 72 KB.  A build that broke both (a 136 KB decode footprint with copies at
// 64-128 KB) faulted the GPU; which of the two properties mattered was not
// isolated, so both are kept.
constexpr int kLdsCopyLimit = 64 * 1024;
constexpr int kLdsFootprintLimit = 72 * 1024;

// ---- cross-lane ----------------------------------------------------------------
// Value of the lane 32 positions away (lanes l and l^32 exchange).
__device__ __forceinline__ float other_half(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t lane = __lane_id();
  return __builtin_bit_cast(float, lane < 32 ? (uint32_t)r[1] : (uint32_t)r[0]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// fp32 -> T, round to nearest even (v_cvt_pk_bf16_f32 for bf16).
template <typename T>
__device__ __forceinline__ vec2<T> pack2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_convertvector(v, vec2<T>);
}
template <typename T>
__device__ __forceinline__ vec8<T> pack8(float a0, float a1, float a2, float a3, float a4,
                                         float a5, float a6, float a7) {
  vec2<T> p0 = pack2<T>(a0, a1), p1 = pack2<T>(a2, a3), p2 = pack2<T>(a4, a5), p3 = pack2<T>(a6, a7);
  vec8<T> r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}
template <typename T>
__device__ __forceinline__ vec4<T> pack4(float a0, float a1, float a2, float a3) {
  vec2<T> p0 = pack2<T>(a0, a1), p1 = pack2<T>(a2, a3);
  vec4<T> r = {p0[0], p0[1], p1[0], p1[1]};
  return r;
}

// ---- K/V tiles in LDS --------------------------------------------------------
// A tile is `rows` key rows of D 16-bit elements (2D bytes each).  The 16-byte chunks of
// row r are XOR-swizzled by Swz<D>::f(r), which keeps both the ds_read_b128
// K-operand reads (one chunk of 32 consecutive rows per half-wave) and the
// ds_read_b64_tr_b16 V-operand reads free of bank conflicts.  The pattern
// repeats every 32 rows at D=64 and every 16 rows at D=128.
template <int D> struct Swz;
template <> struct Swz<64> {
  static __device__ __forceinline__ uint32_t f(uint32_t r) { return ((r >> 2) ^ (r << 1)) & 7u; }
};
template <> struct Swz<128> {
  static __device__ __forceinline__ uint32_t f(uint32_t r) { return (r ^ (r << 2)) & 15u; }
};

// Byte offset of 16-byte chunk `chunk` of key row `row` in a tile.
template <int D>
__device__ __forceinline__ uint32_t tile_off(uint32_t row, uint32_t chunk) {
  return row * (2 * D) + 16u * (chunk ^ Swz<D>::f(row));
}

// ---- mask ----------------------------------------------------------------------
struct MaskParams {
  uint32_t flags;
  int32_t wl, wr, bs;
  const int32_t* doc;
  int32_t num_docs, doc_stride;
};

__device__ __forceinline__ int64_t floordiv(int64_t a, int64_t b) {
  return a >= 0 ? a / b : -((-a + b - 1) / b);
}

// Visible keys of the row at absolute position p: [lo, hi] (empty when lo > hi).
// Every flag gives an interval whose ends never decrease with p, and the
// clamping to [0, Nk-1] keeps that property, so over a block of consecutive
// rows the first row has the smallest lo and the last row the largest hi.
__device__ __forceinline__ void row_interval(const MaskParams& m, int b, int64_t p, int Nk,
                                             int& lo_out, int& hi_out) {
  int64_t lo = 0, hi = (int64_t)Nk - 1;
  if (m.flags & ATTN_MASK_CAUSAL) hi = hi < p ? hi : p;
  if (m.flags & ATTN_MASK_WINDOW) {
    if (m.wl >= 0) { int64_t a = p - m.wl; lo = lo > a ? lo : a; }
    if (m.wr >= 0) { int64_t a = p + m.wr; hi = hi < a ? hi : a; }
  }
  if (m.flags & ATTN_MASK_BLOCK_CAUSAL) {
    int64_t a = (floordiv(p, m.bs) + 1) * m.bs - 1;
    hi = hi < a ? hi : a;
  }
  if ((m.flags & ATTN_MASK_DOCUMENT) && Nk > 0) {
    const int32_t* off = m.doc + (int64_t)b * m.doc_stride;
    int64_t pc = p < 0 ? 0 : (p >= Nk ? Nk - 1 : p);
    // largest d in [0, num_docs) with off[d] <= pc
    int lo_d = 0, hi_d = m.num_docs - 1;
    while (lo_d < hi_d) {
      int mid = (lo_d + hi_d + 1) >> 1;
      if (off[mid] <= pc) lo_d = mid; else hi_d = mid - 1;
    }
    int64_t s = off[lo_d], e = (int64_t)off[lo_d + 1] - 1;
    lo = lo > s ? lo : s;
    hi = hi < e ? hi : e;
  }
  if (lo < 0) lo = 0;
  if (hi > (int64_t)Nk - 1) hi = (int64_t)Nk - 1;
  lo_out = (int)lo;
  hi_out = (int)hi;
}

// ---- score_mod ---------------------------------------------------------------
// Changes of the scaled score before the softmax (flags of attn_score_mod):
// tanh capping, then the additive ALiBi, symmetric ALiBi and relative-position
// bias table.  The kernels work in base-2 units, so a raw dot product x
// becomes x c2 + log2(e) bias(d), or with the cap
// cap log2(e) tanh(x scale / cap) + log2(e) bias(d), with d = key - query
// position.
struct ScoreParams {
  uint32_t flags;
  const float* slopes;  // [Hq]
  const float* rel;     // [Hq][2R+1]
  int32_t R;
  float cap_in;   // scale / cap
  float cap_out;  // cap * log2(e)
};

// Largest relative-bias table a kernel stages in LDS for one head (floats).
constexpr int kMaxRelTable = 2048;

// The query head's score state: its ALiBi slope in base-2 units and its bias
// table in LDS (already scaled by log2(e)).
struct ScoreHead {
  float slope2;
  const TATTN_LDS float* tab;
};

// Copies head h's bias table, times log2(e), into LDS (all threads of the
// work group take part; the caller's next barrier publishes it).
__device__ __forceinline__ void stage_rel_table(const ScoreParams& sp, int h, TATTN_LDS float* dst,
                                                int tid, int nthreads) {
  const int n = 2 * sp.R + 1;
  const float* src = sp.rel + (int64_t)h * n;
  for (int i = tid; i < n; i += nthreads) dst[i] = src[i] * kLog2e;
}

__device__ __forceinline__ float alibi_slope2(const ScoreParams& sp, int h) {
  return (sp.flags & (ATTN_SCORE_ALIBI | ATTN_SCORE_ALIBI_SYM)) ? sp.slopes[h] * kLog2e : 0.f;
}

// tanh(u) = sign(u) (1 - 2 / (e^{2|u|} + 1)): one exp2 and one reciprocal;
// +-1 exactly once e^{2|u|} overflows, absolute error a few 2^-24 near 0.
__device__ __forceinline__ float cap_tanh(float u) {
  const float e = fast_exp2((2.f * kLog2e) * __builtin_fabsf(u));
  return __builtin_copysignf(1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f), u);
}

// acc[i][r] = acc[i][r] * c2 + log2(e) bias(dist(i, r)) over NB accumulators of
// NE elements, the first term capped as cap log2(e) tanh(acc scale / cap) with
// SOFTCAP (the tanh goes to th[i][r] when KEEP_T, for the backward pass's
// factor 1 - tanh^2); -inf (masked) stays -inf.  One loop per term behind
// uniform branches, so no per-element branching.
template <int NB, int NE, bool KEEP_T = false, typename V, typename DistFn>
__device__ __forceinline__ void add_score_bias(V* acc, float c2, const ScoreParams& sp,
                                               const ScoreHead& hd, DistFn dist,
                                               V* th = nullptr) {
  if (sp.flags & ATTN_SCORE_SOFTCAP) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int r = 0; r < NE; ++r) {
        const float x = acc[i][r];
        const float t = cap_tanh(sp.cap_in * x);
        if constexpr (KEEP_T) th[i][r] = t;
        acc[i][r] = x == kNegInf ? kNegInf : sp.cap_out * t;
      }
  } else {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int r = 0; r < NE; ++r) acc[i][r] *= c2;
  }
  if (sp.flags & ATTN_SCORE_ALIBI) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int r = 0; r < NE; ++r) acc[i][r] = __builtin_fmaf(hd.slope2, (float)dist(i, r), acc[i][r]);
  } else if (sp.flags & ATTN_SCORE_ALIBI_SYM) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int r = 0; r < NE; ++r)
        acc[i][r] = __builtin_fmaf(-hd.slope2, __builtin_fabsf((float)dist(i, r)), acc[i][r]);
  }
  if (sp.flags & ATTN_SCORE_REL_BIAS) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int r = 0; r < NE; ++r) {
        const int d = dist(i, r);
        acc[i][r] += hd.tab[(d < -sp.R ? -sp.R : (d > sp.R ? sp.R : d)) + sp.R];
      }
  }
}

}  // namespace tattn
