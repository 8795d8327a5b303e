// Prefill: fused, IO-aware exact attention for gfx950.
//
// One work group of 4 waves owns a 128-row query tile (32 rows per wave) and
// streams the visible keys through LDS in steps of 128 keys (D=64) or 64 keys
// (D=128), as the tiled method
// of "FlashAttention 2 principles and PyTorch practice" (sections 1 and 3.1)
// describes: the Q block stays on chip, K/V blocks are loaded once per step,
// and an online softmax (section 3.2: running max M and exp-sum L, the
// accumulator rescaled whenever M moves) means scores and probabilities
// never reach HBM.  Mask variants follow the FlexAttention / DFlash article:
// per-row intervals for the dense masks (section 1 mask_mod, section 3's
// symmetric window) and explicit FULL / PARTIAL tile lists for BlockMask.
//
// gfx950 mapping:
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (_f16 for fp16 inputs; keys
//    are the M dimension, queries the N dimension), so each lane owns one
//    query column and the row max / row sum are in-lane except for one
//    exchange with lane l^32 (v_permlane32_swap).
//  * The S^T accumulator registers, converted to bf16 / fp16, are directly the
//    B operand of O^T += V^T P^T: the order of the 16 keys inside each PV
//    MFMA is permuted the same way on the V side, which needs no shuffle.
//  * V^T operands come from LDS with ds_read_b64_tr_b16 (transposing loads);
//    K operands with ds_read_b128.  Both tiles use an XOR swizzle of 16-byte
//    chunks that keeps these reads free of bank conflicts.
//  * K/V tiles are copied global -> LDS by global_load_lds_dwordx4 (no
//    registers), double-buffered: step j+1 is in flight while step j computes.
//  * Causal-like masks pair query tile i with tile n-1-i in one work group so
//    every group does the same amount of work; the group -> (batch, head)
//    mapping keeps all tiles of a head (and of a GQA group) on one XCD so its
//    K/V stay in that XCD's L2.
#include <type_traits>

#include "params.h"

namespace tattn {

constexpr int kQTile = 128;
// Keys per step: 128 at D=64, 64 at D=128 (a K or V tile is 16 KB either
// way).  Longer steps halve the per-step barrier, wait and copy-issue cost
// per key; at D=128 the 128-key stage (64 KB) would not leave room for two.
template <int D> struct KBlk { static constexpr int value = D == 64 ? 128 : 64; };
constexpr int kThreads = 256;
// A lane's partial row sum of P (64 values at D=64, 32 at D=128) above
// kSumCap = 2^12 moves the reference max.
constexpr float kSumCap = 4096.0f;

// Pipeline depth: two 32 KB stages (K tile + V tile), so two work groups fit
// in one CU's LDS.
template <int D> struct Stages { static constexpr int value = 2; };

struct Step {
  int kb;      // first key of the step
  int masked;  // apply [lo_m, hi_m] per element
  int use_row_interval;  // 1: the row's own mask interval; 0: only k < Nk
};

template <int D, bool BM, int NST, typename T, bool SM>
__device__ __forceinline__ void process_tile(const FwdParams& p, TATTN_LDS char* smem, int qt,
                                             int b, int h, int kvh) {
  constexpr int kKBlk = KBlk<D>::value;
  constexpr int NKB = kKBlk / 32;              // 32-key blocks of S^T per step
  constexpr int NKC = kKBlk / 16;              // 16-key chunks of the PV MFMA per step
  constexpr int SPT = 128 / kKBlk;             // steps per 128-key BlockMask tile
  constexpr int TILE_BYTES = kKBlk * D * 2;
  constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K tile then V tile
  constexpr int NC = D / 16;                   // d-chunks of the QK MFMA
  constexpr int NDB = D / 32;                  // d-blocks of the PV MFMA
  constexpr int CPR = D / 8;                   // 16-byte chunks per key row
  constexpr int PER_WAVE = kKBlk * CPR / 64 / (kThreads / 64);  // copies per wave per tile
  // The swizzle repeats every KC_PERIOD 16-row key chunks: 32 rows at D=64,
  // 16 rows at D=128, so those row offsets fold into immediate LDS offsets.
  constexpr int KC_PERIOD = D == 64 ? 2 : 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5;

  const T* __restrict__ Qbh = static_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh;
  const T* __restrict__ Kbh = static_cast<const T*>(p.k) + b * p.k_sb + kvh * p.k_sh;
  const T* __restrict__ Vbh = static_cast<const T*>(p.v) + b * p.v_sb + kvh * p.v_sh;

  const int q0 = qt * kQTile;
  const int qrow = q0 + wave * 32 + (lane & 31);
  const bool row_ok = qrow < p.Nq;
  const int64_t shift = (int64_t)p.Nk - p.Nq;

  // Q^T fragments: B operand of S^T = K Q^T (k = head dim, n = query).
  vec8<T> qf[NC];
  {
    const int r = row_ok ? qrow : p.Nq - 1;
    const T* src = Qbh + (int64_t)r * p.q_sn + 8 * half;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const vec8<T>*>(src + 16 * c);
    // No wait here: these loads stay in flight with the first K/V copies, and
    // the first step's full vmcnt wait (or the compiler's own wait before a
    // use) completes them.
  }

  int lo, hi;
  row_interval(p.mask, b, qrow + shift, p.Nk, lo, hi);

  // Score change (SM): the head's ALiBi slope and bias table, staged in LDS
  // after the ring before the first copy (the first step's barrier
  // publishes it).  Scores then carry c2 and the bias, so the softmax below
  // runs with unit scale.
  ScoreHead hd{0.f, nullptr};
  if constexpr (SM) {
    hd.slope2 = alibi_slope2(p.smod, h);
    TATTN_LDS float* tab = reinterpret_cast<TATTN_LDS float*>(smem + NST * STAGE_BYTES);
    hd.tab = tab;
    if (p.smod.flags & ATTN_SCORE_REL_BIAS) stage_rel_table(p.smod, h, tab, tid, kThreads);
  }
  const float c2e = SM ? 1.f : p.c2;

  // Step list.
  int n_steps = 0, kb_begin = 0, lo_last = 0, hi_first = 0;
  int bm_row = 0, nf = 0;
  if constexpr (!BM) {
    int lo_first, hi_last, t0, t1;
    const int last_row = min(q0 + kQTile, p.Nq) - 1;
    row_interval(p.mask, b, q0 + shift, p.Nk, lo_first, hi_first);
    row_interval(p.mask, b, last_row + shift, p.Nk, t0, t1);
    lo_last = t0;
    hi_last = t1;
    if (hi_last >= lo_first) {
      kb_begin = (lo_first / kKBlk) * kKBlk;
      n_steps = (hi_last + 1 - kb_begin + kKBlk - 1) / kKBlk;
    }
  } else {
    const int bb = p.bm_B > 1 ? b : 0, hh = p.bm_H > 1 ? h : 0;
    bm_row = (bb * p.bm_H + hh) * p.n_qt + qt;
    nf = p.full_num[bm_row];
    n_steps = SPT * (nf + p.part_num[bm_row]);
  }
  auto step_at = [&](int s) -> Step {
    Step st;
    if constexpr (!BM) {
      st.kb = kb_begin + s * kKBlk;
      const bool full = st.kb >= lo_last && st.kb + kKBlk - 1 <= hi_first && st.kb + kKBlk <= p.Nk;
      st.masked = !full;
      st.use_row_interval = 1;
    } else {
      const int t = s / SPT;
      const int64_t base = (int64_t)bm_row * p.nKt;
      const int kt = t < nf ? p.full_idx[base + t] : p.part_idx[base + t - nf];
      st.kb = kt * 128 + (s % SPT) * kKBlk;
      const bool partial = t >= nf;
      st.use_row_interval = partial;
      st.masked = partial || st.kb + kKBlk > p.Nk;
    }
    return st;
  };

  // ---- per-lane addresses, fixed for the whole tile ----
  // Copies: lane slot (inst*64 + lane) of a tile is key row r, 16-byte chunk
  // ch ^ swz(r); its global byte offset from the step's first key row is
  // r * stride + 16 * chunk.
  uint32_t dma_row[PER_WAVE], kvoff[PER_WAVE], vvoff[PER_WAVE], dma_lds[PER_WAVE];
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int inst = wave * PER_WAVE + i;
    const uint32_t slot = inst * 64 + lane;
    const uint32_t row = slot / CPR;
    const uint32_t chunk = (slot % CPR) ^ Swz<D>::f(row);
    dma_row[i] = row;
    kvoff[i] = (uint32_t)(row * p.k_sn + chunk * 8) * 2u;
    vvoff[i] = (uint32_t)(row * p.v_sn + chunk * 8) * 2u;
    dma_lds[i] = __builtin_amdgcn_readfirstlane(inst * 1024);
    (void)chunk;
  }
  // S^T operand reads of K: row 32*kbk + lane%32, chunk 2c + lane/32.
  uint32_t k_addr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) k_addr[c] = tile_off<D>(lane & 31, 2 * c + half);
  // V^T operand reads (transposing): per 16-key chunk kc, d-block db and half e.
  uint32_t v_addr[KC_PERIOD][NDB][2];
  {
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int kc = 0; kc < KC_PERIOD; ++kc)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t row = 16 * kc + 4 * (g >> 1) + (j >> 2) + 8 * e;
          const uint32_t dcol = 32 * db + 16 * (g & 1) + 4 * (j & 3);
          v_addr[kc][db][e] = tile_off<D>(row, dcol >> 3) + 8 * (j & 1);
        }
  }

  // Loads of step s into ring stage `stage`.  Every step issues the same
  // number of copies (a ragged tail clamps its rows to the last key), so the
  // vmcnt bookkeeping in the loop is exact.
  auto load_step = [&](int s, int stage) {
    int kb = step_at(s).kb;
    kb = kb < 0 ? 0 : (kb > p.Nk - 1 ? p.Nk - 1 : kb);
    const uint32_t lk = lds_addr(smem) + stage * STAGE_BYTES;
    const T* kbase = Kbh + (int64_t)kb * p.k_sn;
    const T* vbase = Vbh + (int64_t)kb * p.v_sn;
    if (kb + kKBlk <= p.Nk) {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        dma16_sv(kbase, kvoff[i], lk + dma_lds[i]);
        dma16_sv(vbase, vvoff[i], lk + TILE_BYTES + dma_lds[i]);
      }
    } else {
      const uint32_t last = (uint32_t)(p.Nk - 1 - kb);
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const uint32_t over = dma_row[i] > last ? dma_row[i] - last : 0u;
        dma16_sv(kbase, kvoff[i] - over * (uint32_t)p.k_sn * 2u, lk + dma_lds[i]);
        dma16_sv(vbase, vvoff[i] - over * (uint32_t)p.v_sn * 2u, lk + TILE_BYTES + dma_lds[i]);
      }
    }
  };

  float m_ref = kNegInf, l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) oacc[d] = f32x16{};

  // One step of the ring at compile-time stage ST (so every LDS offset below
  // is an immediate).
  auto step = [&](auto stc, int s) {
    constexpr int ST = decltype(stc)::value;
    // Step s's copies are the only ones in flight (two-stage ring).
    static_assert(NST == 2, "ring depth");
    wait_vmem();
    lds_barrier();
    if (s + NST - 1 < n_steps) load_step(s + NST - 1, (ST + NST - 1) % NST);
    const Step st = step_at(s);
    if (st.kb < 0 || st.kb >= p.Nk) return;  // second half of a ragged last tile
    const TATTN_LDS char* tK = smem + ST * STAGE_BYTES;
    const TATTN_LDS char* tV = tK + TILE_BYTES;

    // ---- S^T = K Q^T for the step's keys, in 32-key blocks ----
    f32x16 sacc[NKB];
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk) sacc[kbk] = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk) {
        const vec8<T> kf = lds_read_b128<T>(tK, k_addr[c] + kbk * 32 * 2 * D);
        sacc[kbk] = mfma32(kf, qf[c], sacc[kbk]);
      }
    }
    // Keep the K operand reads about four MFMAs ahead of their use.
    {
      constexpr int NS = NKB * NC;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < NS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // ---- mask (partial steps only) ----
    // Element (kbk, r) holds key kb + 32 kbk + 8 (r/4) + 4 half + r%4; it is
    // visible iff lo_m <= key <= hi_m, one unsigned compare of key - lo_m
    // against hi_m - lo_m.  `sees`: the row has a visible key in this step.
    bool sees = true;
    if (st.masked) {
      const int lo_m = st.use_row_interval ? lo : 0;
      const int hi_m = st.use_row_interval ? hi : p.Nk - 1;
      sees = max(lo_m, st.kb) <= min(hi_m, min(st.kb + kKBlk, p.Nk) - 1);
      const uint32_t base = (uint32_t)(st.kb + 4 * half - lo_m);
      const uint32_t width = hi_m >= lo_m ? (uint32_t)(hi_m - lo_m) : 0u;
      const uint32_t base_ok = hi_m >= lo_m ? base : 0x80000000u;
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t off = 32 * kbk + 8 * (r >> 2) + (r & 3);
          if (base_ok + off > width) sacc[kbk][r] = kNegInf;
        }
    }
    if constexpr (SM) {
      const int d0 = st.kb + 4 * half - (int)(qrow + shift);
      add_score_bias<NKB, 16>(sacc, p.c2, p.smod, hd,
                              [&](int kbk, int r) { return d0 + 32 * kbk + 8 * (r >> 2) + (r & 3); });
    }
    // ---- online softmax against a lazily moved reference max ----
    // P = exp2(c2 s - m_ref) is taken against the row's reference m_ref
    // without a row max on the common path.  Every P value of a lane is at
    // most that lane's partial row sum, so a partial sum <= kSumCap = 2^12
    // proves them all in range.  Otherwise (a row max rose by about
    // log2(kSumCap) = 12 in base-2 units, a non-finite score, or the first
    // visible key of a row) the reference moves to the true row max, O and l
    // are rescaled by exp2(m_old - m_new), and P is taken again.  Each row is
    // thus normalised against a reference at most 12 + log2(64) below its
    // running max: the online softmax of section 3.2 with the rescale
    // deferred until it is needed.
    vec8<T> pf[NKC];
    auto probs = [&](float m_use) -> float {
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = fast_exp2(__builtin_fmaf(sacc[kc >> 1][8 * (kc & 1) + i], c2e, -m_use));
          // l sums the fp32 values: summing the rounded P instead would
          // put up to 2^-9 of relative error into LSE.
          if (i & 1) ps1 += e[i]; else ps0 += e[i];
        }
        pf[kc] = pack8<T>(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      }
      return ps0 + ps1;
    };
    // A row that sees its first key needs the row max anyway: go straight to it.
    float psum = 0.f;
    bool fix = __any(m_ref == kNegInf && sees);
    if (!fix) {
      psum = probs(m_ref == kNegInf ? 0.f : m_ref);
      fix = __any(!(psum <= kSumCap));
    }
    if (fix) {
      float mx = sacc[0][0];
#pragma unroll
      for (int kbk = 0; kbk < NKB; ++kbk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kbk][r]);
      mx = fmaxf(mx, other_half(mx)) * c2e;
      const float m_new = fmaxf(m_ref, mx);
      // A row that has seen no key yet has O = 0 and l = 0: alpha must be 0
      // there, also when its m_new is still -inf (exp2(-inf - -inf) is NaN).
      const float alpha = m_ref == kNegInf ? 0.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < NDB; ++d) oacc[d] *= alpha;
      psum = probs(m_ref == kNegInf ? 0.f : m_ref);
    }
    l_run += psum;
    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      constexpr int ROW_BYTES = 2 * D;
      const uint32_t kc_off = (kc / KC_PERIOD) * (16 * KC_PERIOD) * ROW_BYTES;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const i16x4 v0 = lds_read_tr16(tV, v_addr[kc % KC_PERIOD][db][0] + kc_off);
        const i16x4 v1 = lds_read_tr16(tV, v_addr[kc % KC_PERIOD][db][1] + kc_off);
        oacc[db] = mfma32(join_tr<T>(v0, v1), pf[kc], oacc[db]);
      }
    }
  };

  if (p.Nk > 0) {
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
      if (s < n_steps) load_step(s, s);
  }
  for (int s0 = 0; s0 < n_steps; s0 += NST) {
    step(std::integral_constant<int, 0>{}, s0);
    if (s0 + 1 < n_steps) step(std::integral_constant<int, 1>{}, s0 + 1);
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

// Waves per SIMD: two work groups per CU (64 KB of LDS and up to 256 VGPRs
// per wave each).
template <int D> struct Occ { static constexpr int value = 2; };

template <int D, bool BM, typename T, bool SM>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Occ<D>::value, Occ<D>::value)))
fwd_kernel(const FwdParams p) {
  constexpr int NST = Stages<D>::value;
  // the ring (64 KB), then the score-change table (8 KB) when SM
  constexpr int RING = NST * 2 * KBlk<D>::value * D * 2;
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
  // unit = ((b * Hkv + kvh) * n_slots + slot) * G + g: the G query heads that
  // share a KV head are adjacent, so the work groups of one query tile for
  // all of them run together and read the same K/V tiles through L2.
  const int g = unit % p.G;
  int r = unit / p.G;
  const int slot = r % p.n_slots;
  r /= p.n_slots;
  const int kvh = r % p.Hkv, b = r / p.Hkv;
  const int h = kvh * p.G + g;
  process_tile<D, BM, NST, T, SM>(p, smem, slot, b, h, kvh);
  if (p.paired) {
    const int qt2 = p.n_qt - 1 - slot;
    if (qt2 != slot) {
      __syncthreads();
      process_tile<D, BM, NST, T, SM>(p, smem, qt2, b, h, kvh);
    }
  }
}

int launch_fwd_pp(const FwdParams& p, int D, int dtype, hipStream_t stream);

template <typename T, bool SM>
void launch_fwd_t(const FwdParams& p, int D, bool blockmask, dim3 grid, dim3 block,
                  hipStream_t stream) {
  if (D == 64) {
    if (blockmask) hipLaunchKernelGGL((fwd_kernel<64, true, T, SM>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fwd_kernel<64, false, T, SM>), grid, block, 0, stream, p);
  } else {
    if (blockmask) hipLaunchKernelGGL((fwd_kernel<128, true, T, SM>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((fwd_kernel<128, false, T, SM>), grid, block, 0, stream, p);
  }
}

// Dense masks at D=128 run on the two-group ping-pong kernel of fwd_pp.hip
// (measured 5% faster there); D=64 and BlockMask lists run on fwd_kernel.
int launch_fwd(const FwdParams& p, int D, bool blockmask, int dtype, hipStream_t stream) {
  if (!blockmask && D == 128) return launch_fwd_pp(p, D, dtype, stream);
  const long units = (long)p.B * p.Hq * p.n_slots;
  dim3 grid((unsigned)units), block(kThreads);
  const bool sm = p.smod.flags != 0;
  if (dtype == ATTN_DTYPE_F16) {
    if (sm) launch_fwd_t<f16, true>(p, D, blockmask, grid, block, stream);
    else launch_fwd_t<f16, false>(p, D, blockmask, grid, block, stream);
  } else {
    if (sm) launch_fwd_t<bf16, true>(p, D, blockmask, grid, block, stream);
    else launch_fwd_t<bf16, false>(p, D, blockmask, grid, block, stream);
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace tattn
