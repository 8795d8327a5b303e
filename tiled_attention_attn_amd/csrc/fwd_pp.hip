// Dense-mask prefill with two wave groups in ping-pong, for gfx950 (used at
// D=128; the template also covers D=64).
//
// The same fused, IO-aware exact attention as fwd.hip (the tiled method of
// "FlashAttention 2 principles and PyTorch practice", sections 1 and 3:
// Q block on chip, K/V blocks streamed, online softmax with a running max and
// exp-sum), with a schedule built for the CDNA execution model:
//
//  * A work group of 8 waves owns a 256-row query tile, 32 rows per wave.
//    Waves w and w+4 share a SIMD.  Waves 0-3 (group A) and 4-7 (group B)
//    run the same per-step program -- an MFMA phase M(j) = O += V(j-1) P(j-1)
//    and S(j) = K(j) Q^T, then a VALU phase V(j) = softmax of S(j) -- but
//    group B runs one phase behind group A.  Work-group barriers separate the
//    phases, so in every phase each SIMD holds one wave issuing MFMAs and one
//    issuing the softmax VALU work, and the matrix cores and the VALU work
//    at the same time.
//  * K/V stream through a 2-stage LDS ring.  Stage j holds K(j) and V(j-1):
//    exactly what M(j) reads, in phase 2j (group A) and 2j+1 (group B).  All
//    512 threads copy their 16-byte chunks of each tile with
//    global_load_lds_dwordx4 one stage (two phases) ahead of use; the 256
//    query rows share every K/V byte copied.
//  * MFMA layouts, the chunk swizzle and the deferred-rescale online softmax
//    are those of fwd.hip: S^T on 32x32x16 bf16/fp16 MFMAs, P^T taken from the
//    S^T accumulators, V^T read with ds_read_b64_tr_b16.
//  * Each wave decides per step, from its own 32 rows' mask intervals,
//    whether the step is invisible (skipped), fully visible, or needs the
//    per-element mask.
#include <type_traits>

#include "params.h"

namespace tattn {
namespace {

constexpr int kPPThreads = 512;  // 8 waves: groups A (0-3) and B (4-7)
constexpr int kPPRows = 256;     // query rows per tile
constexpr int kPPStages = 2;     // LDS ring depth
// Keys per step: a K or V tile is 16 KB (two 16-byte chunks per thread).
template <int D> struct PPKBlk { static constexpr int value = D == 64 ? 128 : 64; };
// A lane's partial row sum of P above 2^12 moves the reference max.
constexpr float kPPSumCap = 4096.0f;

template <int D, typename T, bool SM>
__device__ __forceinline__ void pp_tile(const FwdParams& p, TATTN_LDS char* smem, int qt, int b,
                                        int h, int kvh) {
  constexpr int KB = PPKBlk<D>::value;
  constexpr int TILE_BYTES = KB * D * 2;
  constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K(j), then V(j-1)
  constexpr int NC = D / 16;                   // d-chunks of the QK MFMA
  constexpr int NDB = D / 32;                  // d-blocks of the PV MFMA
  constexpr int NKB = KB / 32;                 // 32-key blocks of S^T per step
  constexpr int NKC = KB / 16;                 // 16-key chunks of the PV MFMA per step
  constexpr int CPR = D / 8;                   // 16-byte chunks per key row
  constexpr int KC_PERIOD = D == 64 ? 2 : 1;   // swizzle period in 16-row chunks
  constexpr int CPT = TILE_BYTES / (16 * kPPThreads);  // copies per thread per tile
  static_assert(CPT * 16 * kPPThreads == TILE_BYTES, "whole copies per thread");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int half = lane >> 5;

  const T* __restrict__ Qbh = static_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* __restrict__ Kbh = static_cast<const T*>(p.k) + b * p.k_sb + kvh * p.k_sh;
  const T* __restrict__ Vbh = static_cast<const T*>(p.v) + b * p.v_sb + kvh * p.v_sh;

  const int q0 = qt * kPPRows;
  const int wq0 = q0 + wave * 32;  // this wave's first row
  const bool wave_valid = wq0 < p.Nq;
  const int qrow = wq0 + (lane & 31);
  const bool row_ok = qrow < p.Nq;
  const int64_t shift = (int64_t)p.Nk - p.Nq;

  vec8<T> qf[NC];
  {
    const int r = row_ok ? qrow : p.Nq - 1;
    const T* src = Qbh + (int64_t)r * p.q_sn + 8 * half;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const vec8<T>*>(src + 16 * c);
    wait_vmem();  // the loop's waits then only concern the K/V copies
  }
  int lo, hi;
  row_interval(p.mask, b, qrow + shift, p.Nk, lo, hi);

  // Score change (SM): slope and LDS bias table of the head, staged after
  // the ring before the first copy; scores then carry c2 and the bias.
  ScoreHead hd{0.f, nullptr};
  if constexpr (SM) {
    hd.slope2 = alibi_slope2(p.smod, h);
    TATTN_LDS float* tab = reinterpret_cast<TATTN_LDS float*>(smem + kPPStages * STAGE_BYTES);
    hd.tab = tab;
    if (p.smod.flags & ATTN_SCORE_REL_BIAS) stage_rel_table(p.smod, h, tab, tid, kPPThreads);
  }
  const float c2e = SM ? 1.f : p.c2;

  // Steps of the tile: the keys any of its rows sees (interval ends never
  // decrease with the row, so the first and last rows bound them).
  int n_steps = 0, kb_begin = 0;
  {
    int lo_first, hi_first, lo_last, hi_last;
    row_interval(p.mask, b, q0 + shift, p.Nk, lo_first, hi_first);
    row_interval(p.mask, b, min(q0 + kPPRows, p.Nq) - 1 + shift, p.Nk, lo_last, hi_last);
    if (hi_last >= lo_first) {
      kb_begin = (lo_first / KB) * KB;
      n_steps = (hi_last + 1 - kb_begin + KB - 1) / KB;
    }
  }
  // This wave's rows: union [wlo_first, whi_last], intersection [wlo_last, whi_first].
  int wlo_first = 0, whi_first = -1, wlo_last = 0, whi_last = -1;
  if (wave_valid) {
    row_interval(p.mask, b, wq0 + shift, p.Nk, wlo_first, whi_first);
    row_interval(p.mask, b, min(wq0 + 32, p.Nq) - 1 + shift, p.Nk, wlo_last, whi_last);
  }
  auto step_skip = [&](int j) {
    const int kb = kb_begin + j * KB;
    return !wave_valid || kb > whi_last || kb + KB - 1 < wlo_first;
  };

  // ---- copies: thread t moves 16-byte chunks t + 512 i of the K and V tiles ----
  uint32_t crow[CPT], kvoff[CPT], vvoff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const uint32_t slot = (uint32_t)(tid + kPPThreads * i);
    crow[i] = slot / CPR;
    const uint32_t cchunk = (slot % CPR) ^ Swz<D>::f(crow[i]);
    kvoff[i] = (uint32_t)(crow[i] * p.k_sn + cchunk * 8) * 2u;
    vvoff[i] = (uint32_t)(crow[i] * p.v_sn + cchunk * 8) * 2u;
  }
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(wave * 1024);
  // Rows of a step past the last key repeat the last key row, and a step
  // outside [0, Nk) reads the nearest in-range rows: every stage issues the
  // same copies per thread, so the vmcnt bookkeeping below is exact.
  auto copy_tile = [&](const T* base_bh, int64_t sn, const uint32_t (&voff)[CPT], int j,
                       uint32_t lds) {
    int kb = kb_begin + j * KB;
    kb = kb < 0 ? 0 : (kb > p.Nk - 1 ? p.Nk - 1 : kb);
    const T* src = base_bh + (int64_t)kb * sn;
    const uint32_t last = (uint32_t)(p.Nk - 1 - kb);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const uint32_t over = crow[i] > last ? crow[i] - last : 0u;
      dma16_sv(src, voff[i] - over * (uint32_t)sn * 2u, lds + lds_wave + i * 16 * kPPThreads);
    }
  };
  auto issue_stage = [&](int j) {
    const uint32_t base = lds_addr(smem) + (uint32_t)(j % kPPStages) * STAGE_BYTES;
    copy_tile(Kbh, p.k_sn, kvoff, j, base);
    copy_tile(Vbh, p.v_sn, vvoff, j - 1, base + TILE_BYTES);
  };

  // ---- operand addresses (as in fwd.hip) ----
  uint32_t k_addr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) k_addr[c] = tile_off<D>(lane & 31, 2 * c + half);
  uint32_t v_addr[KC_PERIOD][NDB][2];
  {
    const int g = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int kc = 0; kc < KC_PERIOD; ++kc)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t row = 16 * kc + 4 * (g >> 1) + (jj >> 2) + 8 * e;
          const uint32_t dcol = 32 * db + 16 * (g & 1) + 4 * (jj & 3);
          v_addr[kc][db][e] = tile_off<D>(row, dcol >> 3) + 8 * (jj & 1);
        }
  }

  float m_ref = kNegInf, l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) oacc[d] = f32x16{};
  f32x16 sacc[NKB];  // S(j): written in M(j), read in V(j)
  vec8<T> pf[NKC];    // P(j): written in V(j), read in M(j+1)

  // ---- MFMA phase M(j): O += V(j-1) P(j-1), then S(j) = K(j) Q^T ----
  auto mfma_phase = [&](int j) {
    const TATTN_LDS char* tK = smem + (j % kPPStages) * STAGE_BYTES;
    const TATTN_LDS char* tV = tK + TILE_BYTES;
    if (j >= 1 && !step_skip(j - 1)) {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const uint32_t kc_off = (kc / KC_PERIOD) * (16 * KC_PERIOD) * (2 * D);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const i16x4 v0 = lds_read_tr16(tV, v_addr[kc % KC_PERIOD][db][0] + kc_off);
          const i16x4 v1 = lds_read_tr16(tV, v_addr[kc % KC_PERIOD][db][1] + kc_off);
          oacc[db] = mfma32(join_tr<T>(v0, v1), pf[kc], oacc[db]);
        }
      }
      // Keep the transposing reads about four MFMAs ahead of their use.
      constexpr int NPV = NKC * NDB;
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < NPV - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    if (j < n_steps && !step_skip(j)) {
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk) {
        sacc[kbk] = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c)
          sacc[kbk] = mfma32(lds_read_b128<T>(tK, k_addr[c] + kbk * 32 * 2 * D), qf[c], sacc[kbk]);
      }
      // Keep the K reads about four MFMAs ahead of their use.
      constexpr int NQK = NKB * NC;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < NQK - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
  };

  // ---- VALU phase V(j): mask, deferred-rescale online softmax, P(j) ----
  auto probs = [&](float m_use) -> float {
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[i] = fast_exp2(__builtin_fmaf(sacc[kc >> 1][8 * (kc & 1) + i], c2e, -m_use));
        if (i & 1) ps1 += e[i]; else ps0 += e[i];
      }
      pf[kc] = pack8<T>(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    }
    return ps0 + ps1;
  };
  auto valu_phase = [&](int j) {
    if (step_skip(j)) return;
    const int kb = kb_begin + j * KB;
    bool sees = true;
    const bool full = kb >= wlo_last && kb + KB - 1 <= whi_first && kb + KB <= p.Nk;
    if (!full) {
      // Element (kbk, r) holds key kb + 32 kbk + 8 (r/4) + 4 half + r%4,
      // visible iff lo <= key <= hi (one unsigned compare).
      sees = max(lo, kb) <= min(hi, min(kb + KB, p.Nk) - 1);
      const uint32_t width = hi >= lo ? (uint32_t)(hi - lo) : 0u;
      const uint32_t base_ok = hi >= lo ? (uint32_t)(kb + 4 * half - lo) : 0x80000000u;
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t off = 32 * kbk + 8 * (r >> 2) + (r & 3);
          if (base_ok + off > width) sacc[kbk][r] = kNegInf;
        }
    }
    if constexpr (SM) {
      const int d0 = kb + 4 * half - (int)(qrow + shift);
      add_score_bias<NKB, 16>(sacc, p.c2, p.smod, hd,
                              [&](int kbk, int r) { return d0 + 32 * kbk + 8 * (r >> 2) + (r & 3); });
    }
    // P against the row's reference; the reference moves (O and l rescaled)
    // only when a partial sum shows it stale or the row's first key arrives.
    // A row that sees its first key needs the row max anyway: go straight to it.
    float psum = 0.f;
    bool fix = __any(m_ref == kNegInf && sees);
    if (!fix) {
      psum = probs(m_ref == kNegInf ? 0.f : m_ref);
      fix = __any(!(psum <= kPPSumCap));
    }
    if (fix) {
      float mx = sacc[0][0];
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kbk][r]);
      mx = fmaxf(mx, other_half(mx)) * c2e;
      const float m_new = fmaxf(m_ref, mx);
      // A row that has seen no key yet has O = 0 and l = 0: alpha is 0 there.
      const float alpha = m_ref == kNegInf ? 0.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d) oacc[d] *= alpha;
      psum = probs(m_ref == kNegInf ? 0.f : m_ref);
    }
    l_run += psum;
  };

  // ---- phases: group A runs M(0) V(0) M(1) ... M(n); group B one phase later ----
  // Iteration j covers phases 2j and 2j+1: A does M(j) then V(j), B does
  // V(j-1) then M(j).  The group is a compile-time parameter so that each
  // group's loop body is straight-line code (S and P stay in place).
  auto run = [&](auto grpc) {
    constexpr int GRP = decltype(grpc)::value;
    for (int j = 0; j <= n_steps; ++j) {
      // Stage j (issued one iteration earlier) must have landed: this wave's
      // copies, then everyone's via the barrier.
      wait_vmem();
      lds_barrier();
      // Stage j+1 reuses the slot of stage j-1, whose last reader was group
      // B's M(j-1) in the phase before this barrier.
      if (j + 1 <= n_steps) issue_stage(j + 1);
      // The MFMA phase runs at raised wave priority, so its MFMAs issue as
      // soon as the matrix pipe frees up and the other wave's VALU stream
      // fills the remaining issue cycles.
      if constexpr (GRP == 0) {
        __builtin_amdgcn_s_setprio(1);
        mfma_phase(j);
        __builtin_amdgcn_s_setprio(0);
      } else if (j >= 1) {
        valu_phase(j - 1);
      }
      lds_barrier();
      if constexpr (GRP == 0) {
        if (j < n_steps) valu_phase(j);
      } else {
        __builtin_amdgcn_s_setprio(1);
        mfma_phase(j);
        __builtin_amdgcn_s_setprio(0);
      }
    }
  };
  if (n_steps > 0) {
    issue_stage(0);
    if (grp == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
  }

  // ---- epilogue: O = O_acc / l, LSE = m ln2 + ln l ----
  const float l_tot = l_run + other_half(l_run);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T* Orow = static_cast<T*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)qrow * p.o_sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        *reinterpret_cast<vec4<T>*>(Orow + 32 * db + 8 * r4 + 4 * half) =
            pack4<T>(oacc[db][4 * r4 + 0] * inv, oacc[db][4 * r4 + 1] * inv,
                     oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
      }
    if (p.lse != nullptr && half == 0)
      p.lse[((int64_t)b * p.Hq + h) * p.Nq + qrow] =
          l_tot > 0.f ? m_ref * kLn2 + logf(l_tot) : kNegInf;
  }
}

template <int D, typename T, bool SM>
__global__ void __launch_bounds__(kPPThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
fwd_pp_kernel(const FwdParams p) {
  // the ring (64 KB), then the score-change table (8 KB) when SM
  constexpr int RING = kPPStages * 2 * PPKBlk<D>::value * D * 2;
  constexpr int LDS_BYTES = RING + (SM ? kMaxRelTable * 4 : 0);
  static_assert(RING <= kLdsCopyLimit && LDS_BYTES <= kLdsFootprintLimit, "LDS limits");
  __shared__ __attribute__((aligned(1024))) char smem_raw[LDS_BYTES];
  TATTN_LDS char* smem = (TATTN_LDS char*)smem_raw;
  const int id = (p.sched & ATTN_SCHED_REVERSE) ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  int unit = id;
  if (p.xcd_remap) {
    // work groups are dealt round-robin to the 8 XCDs: give each XCD a
    // contiguous range of units (whole KV heads) so K/V stay in one L2.
    const int per = gridDim.x >> 3;
    unit = (id & 7) * per + (id >> 3);
  }
  // unit = ((b * Hkv + kvh) * n_slots + slot) * G + g (query heads of one KV
  // head adjacent).
  const int g = unit % p.G;
  int r = unit / p.G;
  const int slot = r % p.n_slots;
  r /= p.n_slots;
  const int kvh = r % p.Hkv, b = r / p.Hkv;
  const int h = kvh * p.G + g;
  pp_tile<D, T, SM>(p, smem, slot, b, h, kvh);
  if (p.paired) {
    const int qt2 = p.n_qt - 1 - slot;
    if (qt2 != slot) {
      __syncthreads();
      pp_tile<D, T, SM>(p, smem, qt2, b, h, kvh);
    }
  }
}

}  // namespace

// Dense-mask prefill on 256-row tiles.  `p` describes 128-row tiles; the
// tile count, pairing and XCD mapping are recomputed here.
int launch_fwd_pp(const FwdParams& p_in, int D, int dtype, hipStream_t stream) {
  FwdParams p = p_in;
  p.n_qt = (p.Nq + kPPRows - 1) / kPPRows;
  p.paired = p_in.paired && p.n_qt > 1;
  p.n_slots = p.paired ? (p.n_qt + 1) / 2 : p.n_qt;
  const long units = (long)p.B * p.Hq * p.n_slots;
  p.xcd_remap = (units % 8) == 0 && !(p.sched & ATTN_SCHED_NO_XCD_REMAP);
  dim3 grid((unsigned)units), block(kPPThreads);
  if (D != 128) return ATTN_ERR_HEAD_DIM;  // D=64 prefill runs on fwd_kernel
  const bool sm = p.smod.flags != 0;
  if (dtype == ATTN_DTYPE_F16) {
    if (sm) hipLaunchKernelGGL((fwd_pp_kernel<128, f16, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fwd_pp_kernel<128, f16, false>), grid, block, 0, stream, p);
  } else {
    if (sm) hipLaunchKernelGGL((fwd_pp_kernel<128, bf16, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fwd_pp_kernel<128, bf16, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace tattn
