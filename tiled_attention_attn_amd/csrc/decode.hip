// Split-KV paged decode and the log-sum-exp combine for gfx950.
//
// "Short query + long KV": the FlexAttention / DFlash article (section 1)
// names FlashDecoding-style split-KV decoding with GQA over a paged KV cache
// addressed through a block table.  Each work group here owns one
// (sequence, KV head, key split) and all the query rows that read that KV
// head -- G query heads x Lq draft tokens, packed 16 rows per wave -- so
// every K/V byte of the split is read from HBM exactly once.  Within the
// split the keys stream through LDS in steps of 64 keys (D=64) or 32 keys
// (D=128) with an online softmax (running max, exp-sum, rescaled
// accumulator), and the split's normalised partial O_s and LSE_s go to an
// fp32 workspace.  The combine kernel then merges the splits by their LSE.
// The same kernel also takes contiguous, strided K/V [B, Hkv, Nk, D] (no
// block table): the split-KV half of the shape-based choice that the same
// article describes, where a decode-shaped call switches from the prefill
// kernel to split-KV.
//
// gfx950 mapping:
//  * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 / _f16 (16 keys x
//    16 query rows per block); the S^T registers are the P^T operand
//    directly, and V^T comes from LDS through ds_read_b64_tr_b16.
//  * Page rows (256 bytes at D=128) are copied global -> LDS with
//    global_load_lds_dwordx4, double-buffered; block-table entries for the
//    next step are loaded a step ahead so no load waits on another.
#include "params.h"

namespace tattn {

constexpr int kDecThreads = 256;
constexpr int kDecStages = 4;            // LDS pipeline depth
constexpr int kDecMaxSplitPages = 2048;  // block-table entries of one split, kept in LDS
// Keys per step: the K + V ring (kDecStages stages) is 64 KB at both head
// dims.  Asynchronous LDS copies only ever target the first 64 KB of a work
// group's LDS (no copy into LDS at 64 KB or above is relied on), and 64 KB of
// ring plus the 8 KB page table lets two work groups share a CU.
template <int D> struct DecKBlk { static constexpr int value = D == 64 ? 64 : 32; };

// Chunk swizzle of the decode K/V tiles.  At D=128 the PV operand reads take
// key rows 8m..8m+7 at chunk pairs {2d, 2d+1} across 32 lanes, so row r gets
// ((r & 7) << 1) | (r >> 3 & 1): the 8 rows of a pair-of-groups then hit
// distinct chunk pairs (free of bank conflicts), and rows 0..15 still take 16
// distinct chunks for the K reads.  D=64 uses the prefill's swizzle.
template <int D> struct DecSwz;
template <> struct DecSwz<64> {
  static __device__ __forceinline__ uint32_t f(uint32_t r) { return Swz<64>::f(r); }
};
template <> struct DecSwz<128> {
  static __device__ __forceinline__ uint32_t f(uint32_t r) { return ((r & 7u) << 1) | ((r >> 3) & 1u); }
};
template <int D>
__device__ __forceinline__ uint32_t dec_tile_off(uint32_t row, uint32_t chunk) {
  return row * (2 * D) + 16u * (chunk ^ DecSwz<D>::f(row));
}

__device__ __forceinline__ float xor_lane(float x, int m) { return __shfl_xor(x, m, 64); }

template <int D, typename T, bool SM, bool PAGED>
__global__ void __launch_bounds__(kDecThreads)
decode_kernel(const DecParams p) {
  constexpr int kDecKBlk = DecKBlk<D>::value;
  constexpr int NKB = kDecKBlk / 16;               // 16-key blocks per step
  constexpr int NKC = kDecKBlk / 32;               // 32-key PV chunks per step
  constexpr int CPR = D / 8;                       // 16-byte chunks per key row
  constexpr int INSTS = kDecKBlk * CPR / 64;       // wave instructions per tile
  constexpr int PER_WAVE = INSTS / (kDecThreads / 64);
  constexpr int TILE_BYTES = kDecKBlk * D * 2;
  constexpr int NC = D / 32;   // d-chunks of the QK MFMA (K = 32)
  constexpr int NDB = D / 16;  // d-blocks of the PV MFMA (M = 16)
  constexpr int NST = kDecStages;
  static_assert(NST * 2 * TILE_BYTES <= kLdsCopyLimit &&
                    NST * 2 * TILE_BYTES + kDecMaxSplitPages * 4 <= kLdsFootprintLimit,
                "LDS limits");
  __shared__ __attribute__((aligned(1024))) char smem_raw[NST * 2 * TILE_BYTES];
  __shared__ int s_pages[kDecMaxSplitPages];
  TATTN_LDS char* smem = (TATTN_LDS char*)smem_raw;
  auto bufK = [&](int st) -> TATTN_LDS char* { return smem + (st % NST) * 2 * TILE_BYTES; };
  auto bufV = [&](int st) -> TATTN_LDS char* {
    return smem + (st % NST) * 2 * TILE_BYTES + TILE_BYTES;
  };

  const bool rev = (p.sched & ATTN_SCHED_REVERSE) != 0;
  const int bx = rev ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  const int s = bx % p.S, rg = bx / p.S;
  const int kvh = rev ? (int)(gridDim.y - 1 - blockIdx.y) : (int)blockIdx.y;
  const int b = rev ? (int)(gridDim.z - 1 - blockIdx.z) : (int)blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane >> 4, col = lane & 15;

  // Sequence length as given, clamped to what the block table can address;
  // contiguous K/V have max_keys keys in every sequence.
  const int seq_len = PAGED ? min(max(p.seq_lens[b], 0), p.max_keys) : p.max_keys;
  const int k_begin = s * p.chunk;
  const int k_end = min(seq_len, k_begin + p.chunk);

  // This lane's query row (the N index of its MFMA column).
  const int rr = rg * 64 + wave * 16 + col;
  const bool row_ok = rr < p.rows;
  const int rrc = row_ok ? rr : p.rows - 1;
  const int g = rrc / p.Lq, t = rrc % p.Lq;
  const int hq = kvh * p.G + g;
  const int64_t pos = (int64_t)seq_len - p.Lq + t;
  int lo = 1, hi = 0;
  if (seq_len > 0) row_interval(p.mask, b, pos, seq_len, lo, hi);
  lo = max(lo, k_begin);
  hi = min(hi, k_end - 1);
  if (!row_ok) { lo = 1; hi = 0; }

  // Keys any row of this group can see: rows differ only in t, and the
  // interval ends never decrease with t, so t = 0 and t = Lq-1 bound them.
  // A split that starts at or past the end of the sequence has no steps.
  int n_steps = 0, kb0 = k_begin;
  if (seq_len > 0 && k_end > k_begin) {
    int a0, a1, c0, c1;
    row_interval(p.mask, b, (int64_t)seq_len - p.Lq, seq_len, a0, a1);
    row_interval(p.mask, b, (int64_t)seq_len - 1, seq_len, c0, c1);
    const int klo = max(a0, k_begin);  // >= k_begin
    const int khi = min(c1, k_end - 1);
    if (khi >= klo) {
      kb0 = k_begin + ((klo - k_begin) / kDecKBlk) * kDecKBlk;
      n_steps = (khi + 1 - kb0 + kDecKBlk - 1) / kDecKBlk;
    }
  }
  // Rows of this wave that are unmasked on a whole step: bounds over the wave.
  int wlo = row_ok ? lo : -0x3fffffff, whi = row_ok ? hi : 0x3fffffff;
  for (int m = 32; m >= 1; m >>= 1) {
    wlo = max(wlo, __shfl_xor(wlo, m, 64));
    whi = min(whi, __shfl_xor(whi, m, 64));
  }

  // Score change (SM): the lane's query head hq sets its ALiBi slope and bias
  // table row.  Scores then carry c2 (or the cap) and the bias.  The G bias
  // tables of a work group do not fit beside the LDS ring, so the table term
  // is added here from global memory: a step whose keys all lie more than R
  // before every row's position adds the row's clamped end value rel_far
  // (loaded once); only the steps within R of the query positions look the
  // table up per element.
  ScoreParams sp = p.smod;
  sp.flags &= ATTN_SCORE_ALIBI | ATTN_SCORE_ALIBI_SYM | ATTN_SCORE_SOFTCAP;
  ScoreHead hd{0.f, nullptr};
  if constexpr (SM) hd.slope2 = alibi_slope2(sp, hq);
  const float c2e = SM ? 1.f : p.c2;
  const bool rel = SM && (p.smod.flags & ATTN_SCORE_REL_BIAS) != 0;
  const float* rel_row = p.smod.rel + (rel ? (int64_t)hq * (2 * p.smod.R + 1) : 0);
  float rel_far = 0.f;
  if (rel) rel_far = rel_row[0] * kLog2e;
  // steps with kb + kDecKBlk - 1 < rel_near are far: every row sits at >= seq_len - Lq
  const int64_t rel_near = (int64_t)seq_len - p.Lq - p.smod.R;

  // Q^T fragments (B operand, k = head dim, n = row).
  vec8<T> qf[NC];
  {
    const T* src = static_cast<const T*>(p.q) + b * p.q_sb + hq * p.q_sh + (int64_t)t * p.q_sn + 8 * grp;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const vec8<T>*>(src + 32 * c);
  }
  // The split's block-table entries go to LDS once, so the pipelined loop
  // below issues no vector-memory loads other than the K/V copies -- except
  // with a relative-position bias table: a step within R of the query
  // positions reads its table entries from global memory, and the compiler's
  // wait for those values (vmcnt counts in issue order) also drains the K/V
  // copies just issued for later stages.  Only the last ceil((Lq + R) / 32)
  // steps or so of the sequence are such steps.
  int page0 = 0, n_split_pages = 0;
  if constexpr (PAGED) {
    const int32_t* bt_row = p.bt + b * p.bt_stride;
    page0 = k_begin / p.ps;
    n_split_pages = k_end > k_begin ? (k_end - 1) / p.ps - page0 + 1 : 0;
    for (int i = tid; i < n_split_pages; i += kDecThreads) {
      const int page = bt_row[page0 + i];
      s_pages[i] = page < 0 ? 0 : (page >= p.num_pages ? (int)p.num_pages - 1 : page);
    }
  }
  wait_vmem();  // Q fragments and page entries
  __syncthreads();

  const T* kbh = static_cast<const T*>(p.kc) + kvh * p.k_sh + (PAGED ? 0 : b * p.k_sb);
  const T* vbh = static_cast<const T*>(p.vc) + kvh * p.v_sh + (PAGED ? 0 : b * p.v_sb);
  auto issue = [&](int kb, int st) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int inst = wave * PER_WAVE + i;
      const int slot = inst * 64 + lane;
      const uint32_t row = slot / CPR;
      const uint32_t chunk = (slot % CPR) ^ DecSwz<D>::f(row);
      int key = kb + (int)row;
      key = key < k_end ? key : k_end - 1;
      // the key's pool slot (paged) or its row (contiguous)
      int64_t slot_k = key;
      if constexpr (PAGED) {
        int pidx = key / p.ps - page0;  // in [0, n_split_pages) for every issued step
        pidx = pidx < 0 ? 0 : (pidx >= n_split_pages ? n_split_pages - 1 : pidx);
        slot_k = (int64_t)s_pages[pidx] * p.ps + key % p.ps;
      }
      const uint32_t loff = __builtin_amdgcn_readfirstlane(inst * 1024);
      dma16(kbh + slot_k * p.k_sn + chunk * 8, lds_addr(bufK(st)) + loff);
      dma16(vbh + slot_k * p.v_sn + chunk * 8, lds_addr(bufV(st)) + loff);
    }
  };
  constexpr int LOADS = 2 * PER_WAVE;  // copies per wave per step

  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) oacc[d] = f32x4{};

#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < n_steps) issue(kb0 + st * kDecKBlk, st);
  for (int st = 0; st < n_steps; ++st) {
    const int kb = kb0 + st * kDecKBlk;
    // Copies issued after step st's: those of steps st+1 .. min(st+NST-2, n-1).
    const int later = min(NST - 2, n_steps - 1 - st);
    if (later >= 2) wait_vmem_le<2 * LOADS>();
    else if (later == 1) wait_vmem_le<LOADS>();
    else wait_vmem();
    lds_barrier();
    if (st + NST - 1 < n_steps) issue(kb + (NST - 1) * kDecKBlk, st + NST - 1);
    const TATTN_LDS char* tK = bufK(st);
    const TATTN_LDS char* tV = bufV(st);

    f32x4 sacc[NKB];
#pragma unroll
    for (int kb16 = 0; kb16 < NKB; ++kb16) {
      sacc[kb16] = f32x4{};
      const uint32_t row = 16 * kb16 + col;
#pragma unroll
      for (int c = 0; c < NC; ++c)
        sacc[kb16] = mfma16(lds_read_b128<T>(tK, dec_tile_off<D>(row, 4 * c + grp)), qf[c], sacc[kb16]);
    }
    const bool full = kb >= wlo && kb + kDecKBlk - 1 <= whi;
    if (!full) {
#pragma unroll
      for (int kb16 = 0; kb16 < NKB; ++kb16)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb + 16 * kb16 + 4 * grp + r;
          if (key < lo || key > hi) sacc[kb16][r] = kNegInf;
        }
    }
    if constexpr (SM) {
      // element (kb16, r) holds key kb + 16 kb16 + 4 grp + r
      const int d0 = kb + 4 * grp - (int)pos;
      add_score_bias<NKB, 4>(sacc, p.c2, sp, hd, [&](int kb16, int r) { return d0 + 16 * kb16 + r; });
      if (rel) {
        if ((int64_t)kb + kDecKBlk - 1 < rel_near) {
#pragma unroll
          for (int kb16 = 0; kb16 < NKB; ++kb16)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[kb16][r] += rel_far;
        } else {
          const int R = p.smod.R;
#pragma unroll
          for (int kb16 = 0; kb16 < NKB; ++kb16)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int d = d0 + 16 * kb16 + r;
              sacc[kb16][r] += rel_row[(d < -R ? -R : (d > R ? R : d)) + R] * kLog2e;
            }
        }
      }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int kb16 = 0; kb16 < NKB; ++kb16)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kb16][r]);
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float m_new = fmaxf(m_run, mx * c2e);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int d = 0; d < NDB; ++d) oacc[d] *= alpha;
    vec8<T> pf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[i] = fast_exp2(__builtin_fmaf(sacc[2 * kc + (i >> 2)][i & 3], c2e, -m_use));
        l_run += e[i];
      }
      pf[kc] = pack8<T>(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
    }
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const uint32_t r1 = 32 * kc + 4 * grp + (col >> 2);
      const uint32_t r2 = r1 + 16;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint32_t dcol = 16 * db + 4 * (col & 3);
        const uint32_t sub = 8 * (col & 1);
        const i16x4 v0 = lds_read_tr16(tV, dec_tile_off<D>(r1, dcol >> 3) + sub);
        const i16x4 v1 = lds_read_tr16(tV, dec_tile_off<D>(r2, dcol >> 3) + sub);
        oacc[db] = mfma16(join_tr<T>(v0, v1), pf[kc], oacc[db]);
      }
    }
  }

  // Partial result of this split: normalised O_s and LSE_s.
  float l_tot = l_run + xor_lane(l_run, 16);
  l_tot += xor_lane(l_tot, 32);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int64_t orow = (((int64_t)b * p.Hq + hq) * p.Lq + t) * p.S + s;
    float* dst = p.ws_o + orow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      f32x4 w = oacc[db] * inv;
      *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * grp) = w;
    }
    if (grp == 0) p.ws_lse[orow] = l_tot > 0.f ? m_run * kLn2 + logf(l_tot) : kNegInf;
  }
}

// One wave per (sequence, head, query) row: LSE = log sum_s exp(LSE_s),
// O = sum_s exp(LSE_s - LSE) O_s.  The row's S x D partial outputs are read
// as float4s spread over the 64 lanes (lane i takes float4s i, i + 64, ...),
// so all of a row's loads are in flight together; a lane's float4s share one
// d-slice because D/4 divides 64, and the lanes holding the same d-slice are
// summed with cross-lane adds at the end.
template <int D, typename T>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ ws_o,
                                                      const float* __restrict__ ws_lse,
                                                      int n_rows, int Hq, int Lq, int S,
                                                      void* o_, int64_t o_sb, int64_t o_sh,
                                                      int64_t o_sn, float* lse) {
  T* o = static_cast<T*>(o_);
  constexpr int Q4 = D / 4;  // float4s per split row
  static_assert(64 % Q4 == 0, "a lane's float4s must share one d-slice");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= n_rows) return;
  const float* L = ws_lse + (int64_t)row * S;
  float m = kNegInf;
  for (int s = lane; s < S; s += 64) m = fmaxf(m, L[s]);
  for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
  const float m_use = m == kNegInf ? 0.f : m;
  float tot = 0.f;
  for (int s = lane; s < S; s += 64) tot += __expf(L[s] - m_use);
  for (int k = 32; k >= 1; k >>= 1) tot += __shfl_xor(tot, k, 64);
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  const f32x4* O = reinterpret_cast<const f32x4*>(ws_o + (int64_t)row * S * D);
  const int n4 = S * Q4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int i = lane; i < n4; i += 64) {
    const float w = __expf(L[i / Q4] - m_use) * inv;  // L = -inf gives 0
    acc += w * O[i];
  }
#pragma unroll
  for (int k = Q4; k < 64; k <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], k, 64);
  }
  const int t = row % Lq, bh = row / Lq, h = bh % Hq, b = bh / Hq;
  if (lane < Q4) {
    T* dst = o + b * o_sb + h * o_sh + (int64_t)t * o_sn + 4 * lane;
    *reinterpret_cast<vec4<T>*>(dst) = pack4<T>(acc[0], acc[1], acc[2], acc[3]);
  }
  if (lse != nullptr && lane == 0) lse[row] = tot > 0.f ? m_use + logf(tot) : kNegInf;
}

template <typename T, bool SM, bool PAGED>
void launch_decode_t(const DecParams& p, int D, dim3 grid, dim3 block, hipStream_t stream) {
  if (D == 64) hipLaunchKernelGGL((decode_kernel<64, T, SM, PAGED>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((decode_kernel<128, T, SM, PAGED>), grid, block, 0, stream, p);
}

template <typename T, bool PAGED>
void launch_decode_sm(const DecParams& p, int D, dim3 grid, dim3 block, hipStream_t stream) {
  if (p.smod.flags != 0) launch_decode_t<T, true, PAGED>(p, D, grid, block, stream);
  else launch_decode_t<T, false, PAGED>(p, D, grid, block, stream);
}

// p.bt == nullptr selects contiguous K/V.
int launch_decode(const DecParams& p, int D, int dtype, hipStream_t stream) {
  dim3 grid(p.S * p.n_rg, p.Hkv, p.B), block(kDecThreads);
  const bool paged = p.bt != nullptr;
  if (dtype == ATTN_DTYPE_F16) {
    if (paged) launch_decode_sm<f16, true>(p, D, grid, block, stream);
    else launch_decode_sm<f16, false>(p, D, grid, block, stream);
  } else {
    if (paged) launch_decode_sm<bf16, true>(p, D, grid, block, stream);
    else launch_decode_sm<bf16, false>(p, D, grid, block, stream);
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

template <typename T>
void launch_combine_t(const float* ws_o, const float* ws_lse, int n_rows, int Hq, int Lq, int S,
                      int D, void* o, int64_t o_sb, int64_t o_sh, int64_t o_sn, float* lse,
                      dim3 grid, dim3 block, hipStream_t stream) {
  if (D == 64)
    hipLaunchKernelGGL((combine_kernel<64, T>), grid, block, 0, stream, ws_o, ws_lse, n_rows, Hq,
                       Lq, S, o, o_sb, o_sh, o_sn, lse);
  else
    hipLaunchKernelGGL((combine_kernel<128, T>), grid, block, 0, stream, ws_o, ws_lse, n_rows, Hq,
                       Lq, S, o, o_sb, o_sh, o_sn, lse);
}

int launch_combine(const float* ws_o, const float* ws_lse, int B, int Hq, int Lq, int S, int D,
                   int dtype, void* o, int64_t o_sb, int64_t o_sh, int64_t o_sn, float* lse,
                   hipStream_t stream) {
  const int n_rows = B * Hq * Lq;
  dim3 grid((unsigned)(((int64_t)n_rows + 3) / 4)), block(256);
  if (dtype == ATTN_DTYPE_F16)
    launch_combine_t<f16>(ws_o, ws_lse, n_rows, Hq, Lq, S, D, o, o_sb, o_sh, o_sn, lse, grid, block, stream);
  else
    launch_combine_t<bf16>(ws_o, ws_lse, n_rows, Hq, Lq, S, D, o, o_sb, o_sh, o_sn, lse, grid, block, stream);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace tattn
