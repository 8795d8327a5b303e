// Backward pass: dQ, dK, dV of fused exact attention, by recomputation, for
// gfx950.
//
// Only the inputs, O and the per-row LSE are kept from the forward pass; P is
// rebuilt tile by tile from Q, K and the saved LSE whenever a gradient needs
// it (the segmented recomputation of the DeepSeek v2->v4 attention article,
// section 2; the N x N matrices never reach HBM, as in the forward tiling of
// "FlashAttention 2 principles and PyTorch practice", sections 1 and 3.1).
// With P = exp(scale QK^T + mask - LSE) and Delta = rowsum(dO * O):
//
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - Delta),
//     dQ = scale dS K,   dK = scale dS^T Q
//
// (rowsum(P * dP) = rowsum(dO * O) because O = P V, so Delta needs no pass
// over the keys).  Three launches on the caller's stream:
//
//  * bwd_pre_kernel: Delta and L2 = LSE log2(e) per query row, into the
//    caller's workspace (L2 = +inf for rows that see no key and for padding,
//    so their P is 0).
//  * bwd_kv_kernel: one work group per 128-key tile of one KV head; each wave
//    keeps its 32 keys' K and V in registers and the G query heads' Q / dO
//    tiles stream through LDS.  dK and dV of the KV head are summed over all
//    G query heads in registers and written once: no atomics, deterministic.
//  * bwd_q_kernel: one work group per 128-row query tile, shaped like the
//    forward kernel (Q and dO in registers, K / V tiles through LDS); dQ is
//    written once.
//
// gfx950 mapping (the operand layouts of the forward kernel):
//  * kv kernel: S = Q K^T and dP = dO V^T on v_mfma_f32_32x32x16_bf16 (_f16) with
//    queries as M and the wave's keys as N, so each lane owns one key column.
//    Those accumulators, converted to bf16 / fp16, are directly the B operands of
//    dV^T += dO^T P and dK^T += Q^T dS; the A operands dO^T and Q^T come from
//    LDS with ds_read_b64_tr_b16, with the 16 queries of each MFMA permuted
//    the same way as the accumulator rows.
//  * q kernel: S^T = K Q^T and dP^T = V dO^T with keys as M, so each lane owns
//    one query column and its L2 and Delta are scalars; dQ^T += K^T dS^T reads
//    K^T with transposing LDS loads, as the forward reads V^T.
//  * Masks: a query row's visible keys form an interval [lo, hi] whose ends
//    never decrease with the row, so the rows that see a given key also form
//    an interval [qa, qb]; the kv kernel finds it per lane by binary search
//    over rows and tests each element with one unsigned compare.
#include <type_traits>

#include "params.h"

namespace tattn {

constexpr int kBwdThreads = 256;

// ---- Delta and L2 per query row ----------------------------------------------
// Eight lanes per row, 16-byte loads; rows of a (batch, head) padded to
// nq_pad get Delta = 0 and L2 = +inf.
template <int D, typename T>
__global__ void __launch_bounds__(kBwdThreads) bwd_pre_kernel(const BwdParams p) {
  const int64_t row = ((int64_t)blockIdx.x * kBwdThreads + threadIdx.x) >> 3;
  const int j = threadIdx.x & 7;
  const int64_t rows = (int64_t)p.B * p.Hq * p.nq_pad;
  if (row >= rows) return;  // whole 8-lane groups leave together
  const int bh = (int)(row / p.nq_pad), qi = (int)(row % p.nq_pad);
  const int b = bh / p.Hq, h = bh % p.Hq;
  float acc = 0.f;
  if (qi < p.Nq) {
    const T* orow = static_cast<const T*>(p.o) + b * p.o_sb + h * p.o_sh + (int64_t)qi * p.o_sn;
    const T* drow = static_cast<const T*>(p.dout) + b * p.do_sb + h * p.do_sh + (int64_t)qi * p.do_sn;
#pragma unroll
    for (int c = j; c < D / 8; c += 8) {
      const vec8<T> a = *reinterpret_cast<const vec8<T>*>(orow + 8 * c);
      const vec8<T> d = *reinterpret_cast<const vec8<T>*>(drow + 8 * c);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = __builtin_fmaf((float)a[i], (float)d[i], acc);
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  if (j == 0) {
    const float l = qi < p.Nq ? p.lse[(int64_t)bh * p.Nq + qi] : kNegInf;
    p.ws_delta[row] = acc;
    p.ws_l2[row] = l == kNegInf ? __builtin_huge_valf() : l * kLog2e;
  }
}

// The searches below run in every lane with the lane's own key.  Written as
// while-loops they leave the loop lane by lane, and the compiled dK / dV
// kernel then evaluated a mask-flag test of the inlined row_interval as a lane
// mask under one loop's shrinking EXEC and branched on that mask in the next
// loop, where it could hold no active lane: the document search then ran for
// a mask without documents and read through its null offsets pointer.  So
// every loop here runs a wave-uniform number of steps and moves its bounds
// with selects; no branch depends on a lane mask made under another EXEC.

// Steps that shrink a search over n + 1 candidates to one: the bit length of n.
__device__ __forceinline__ int search_steps(int n) {
  return n > 0 ? 32 - __builtin_clz((unsigned)n) : 0;
}

// row_interval with its document search run for doc_steps = search_steps(num_docs - 1)
// steps (each step keeps at least half of the range minus one candidate).
__device__ __forceinline__ void row_interval_fixed(const MaskParams& m, int b, int64_t p, int Nk,
                                                   int doc_steps, int& lo_out, int& hi_out) {
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
    // largest d in [0, num_docs) with off[d] <= pc; mid stays inside [lo_d, hi_d]
    int lo_d = 0, hi_d = m.num_docs - 1;
    for (int it = 0; it < doc_steps; ++it) {
      const int mid = (lo_d + hi_d + 1) >> 1;
      const bool go = lo_d < hi_d;
      const bool le = off[mid] <= pc;
      lo_d = go && le ? mid : lo_d;
      hi_d = go && !le ? mid - 1 : hi_d;
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

// Rows that see key `key`: [qa, qb] (empty when qa > qb).  hi(row) never
// decreases, so {row : hi >= key} is a suffix of the rows; lo(row) never
// decreases, so {row : lo <= key} is a prefix; the rows seeing the key are
// their intersection.  Each search takes search_steps(Nq) steps: a step
// leaves at most half of the z - a remaining candidates beyond the first.
__device__ __forceinline__ void key_rows(const MaskParams& m, int b, int key, int Nq, int Nk,
                                         int64_t shift, int& qa, int& qb) {
  const int steps = search_steps(Nq);
  const int doc_steps = (m.flags & ATTN_MASK_DOCUMENT) ? search_steps(m.num_docs - 1) : 0;
  int a = 0, z = Nq;  // first row with hi >= key (Nq if none)
  for (int it = 0; it < steps; ++it) {
    const int mid = (a + z) >> 1;
    int l, h;
    row_interval_fixed(m, b, mid + shift, Nk, doc_steps, l, h);
    const bool go = a < z, right = h >= key;
    z = go && right ? mid : z;
    a = go && !right ? mid + 1 : a;
  }
  qa = a;
  a = -1;
  z = Nq - 1;  // last row with lo <= key (-1 if none)
  for (int it = 0; it < steps; ++it) {
    const int mid = (a + z + 1) >> 1;
    int l, h;
    row_interval_fixed(m, b, mid + shift, Nk, doc_steps, l, h);
    const bool go = a < z, left = l <= key;
    a = go && left ? mid : a;
    z = go && !left ? mid - 1 : z;
  }
  qb = a;
}

// Query rows per kv-kernel step: 64 at D=64, 32 at D=128 (a Q or dO tile is
// 8 KB either way; a stage adds 1 KB for L2 and Delta).
template <int D> struct BwdQRows { static constexpr int value = D == 64 ? 64 : 32; };
// Bias-table floats the kv kernel stages for the G query heads of a KV head:
// G (2R + 1) <= 8192 (the host checks it).
constexpr int kMaxRelTables = 8192;

// BlockMask (BM): the dK / dV kernel walks the key tile's column of the
// BlockMask -- for each query head of the KV head, its FULL then PARTIAL query
// tiles from the key-tile-major (transposed) lists -- in QB-row steps; a FULL
// tile applies no predicate, a PARTIAL tile the mask intervals.
template <int D, typename T, bool SM, bool BM>
__device__ __forceinline__ void kv_tile(const BwdParams& p, TATTN_LDS char* smem, int kt, int b,
                                        int kvh) {
  constexpr int QB = BwdQRows<D>::value;
  constexpr int NQB = QB / 32;                  // 32-row blocks per step
  constexpr int NC = D / 16;                    // d-chunks of the S / dP MFMAs
  constexpr int NDB = D / 32;                   // d-blocks of the dK / dV MFMAs
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int TILE_BYTES = QB * D * 2;
  constexpr int LD_OFF = 2 * TILE_BYTES;        // L2 then Delta, QB floats each
  constexpr int STAGE_BYTES = LD_OFF + 1024;
  constexpr int PER_WAVE = QB * CPR / 64 / (kBwdThreads / 64);
  constexpr int ROW_BYTES = 2 * D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5;
  const int64_t shift = (int64_t)p.Nk - p.Nq;

  const int k0 = kt * 128;
  const int key = k0 + wave * 32 + (lane & 31);
  const bool key_ok = key < p.Nk;

  // K and V of the lane's key: B operands of S = Q K^T and dP = dO V^T
  // (k = head dim, n = key).
  vec8<T> kf[NC], vf[NC];
  {
    const int r = key_ok ? key : p.Nk - 1;
    const T* ks = static_cast<const T*>(p.k) + b * p.k_sb + kvh * p.k_sh + (int64_t)r * p.k_sn + 8 * half;
    const T* vs = static_cast<const T*>(p.v) + b * p.v_sb + kvh * p.v_sh + (int64_t)r * p.v_sn + 8 * half;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[c] = *reinterpret_cast<const vec8<T>*>(ks + 16 * c);
      vf[c] = *reinterpret_cast<const vec8<T>*>(vs + 16 * c);
    }
    wait_vmem();
  }

  // Score change (SM): the G query heads' bias tables in LDS after the ring
  // (staged before the first copy; the first step's barrier publishes them).
  TATTN_LDS float* tabs = reinterpret_cast<TATTN_LDS float*>(smem + 2 * STAGE_BYTES);
  if constexpr (SM) {
    if (p.smod.flags & ATTN_SCORE_REL_BIAS)
      for (int g = 0; g < p.G; ++g)
        stage_rel_table(p.smod, kvh * p.G + g, tabs + g * (2 * p.smod.R + 1), tid, kBwdThreads);
  }

  // Every lane searches (a key past Nk searches for key Nk - 1), so the
  // search runs outside any lane-dependent branch.
  int qa, qb;
  key_rows(p.mask, b, key_ok ? key : p.Nk - 1, p.Nq, p.Nk, shift, qa, qb);
  if (!key_ok || qa > qb) { qa = 0x3fffffff; qb = -1; }
  // Wave bounds, wave-uniform (scalar registers): rows any lane sees
  // [w_lo, w_hi]; rows every lane sees [w_lo_max, w_hi_min].
  int w_lo = qa, w_hi = qb, w_lo_max = qa, w_hi_min = qb;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    w_lo = min(w_lo, __shfl_xor(w_lo, m, 64));
    w_hi = max(w_hi, __shfl_xor(w_hi, m, 64));
    w_lo_max = max(w_lo_max, __shfl_xor(w_lo_max, m, 64));
    w_hi_min = min(w_hi_min, __shfl_xor(w_hi_min, m, 64));
  }
  w_lo = __builtin_amdgcn_readfirstlane(w_lo);
  w_hi = __builtin_amdgcn_readfirstlane(w_hi);
  w_lo_max = __builtin_amdgcn_readfirstlane(w_lo_max);
  w_hi_min = __builtin_amdgcn_readfirstlane(w_hi_min);

  // Rows the tile's keys see: from the first key's first row to the last
  // key's last row (both ends never decrease with the key).
  // ---- step sequence ----
  // Dense masks: for g < G, query blocks qs0 + qi QB (qi < n_qs), from the
  // first key's first row to the last key's last row.  BlockMask: for g < G,
  // the FULL then PARTIAL query tiles of head kvh G + g, SPQ blocks each.
  constexpr int SPQ = 128 / QB;  // steps per 128-row BlockMask tile
  int n_qs = 0, qs0 = 0, n_steps = 0;
  if constexpr (!BM) {
    if (p.Nk > k0) {
      int a0, b0, a1, b1;
      key_rows(p.mask, b, k0, p.Nq, p.Nk, shift, a0, b0);
      key_rows(p.mask, b, min(k0 + 127, p.Nk - 1), p.Nq, p.Nk, shift, a1, b1);
      if (b1 >= a0) {
        qs0 = (a0 / QB) * QB;
        n_qs = (b1 + 1 - qs0 + QB - 1) / QB;
      }
    }
    n_qs = __builtin_amdgcn_readfirstlane(n_qs);
    qs0 = __builtin_amdgcn_readfirstlane(qs0);
    n_steps = p.G * n_qs;
  }
  // Transposed-list row of head kvh G + g for this key tile.
  auto bm_row = [&](int g) -> int64_t {
    const int hh = p.bm_H > 1 ? kvh * p.G + g : 0, bb = p.bm_B > 1 ? b : 0;
    return ((int64_t)bb * p.bm_H + hh) * p.n_kt + kt;
  };
  if constexpr (BM) {
    for (int g = 0; g < p.G; ++g) {
      const int64_t r = bm_row(g);
      n_steps += SPQ * (p.tfull_num[r] + p.tpart_num[r]);
    }
  }
  // A cursor over the step sequence: head g, block or tile index i, sub-step
  // sub, and (BlockMask) the head's tile count nt and FULL count nf.
  struct Cur { int g, i, sub, nt, nf; };
  auto cur_head = [&](Cur& c) {  // BlockMask: first head at or after c.g with a tile
    for (; c.g < p.G; ++c.g) {
      const int64_t r = bm_row(c.g);
      c.nf = p.tfull_num[r];
      c.nt = c.nf + p.tpart_num[r];
      if (c.nt > 0) break;
    }
  };
  auto cur_init = [&](Cur& c) {
    c = Cur{0, 0, 0, 0, 0};
    if constexpr (BM) cur_head(c);
  };
  // First row of the cursor's step; `partial`: apply the mask intervals.
  auto cur_q0 = [&](const Cur& c, bool& partial) -> int {
    if constexpr (!BM) {
      partial = true;
      return qs0 + c.i * QB;
    } else {
      const int64_t base = bm_row(c.g) * p.n_qt;
      partial = c.i >= c.nf;
      const int qt = partial ? p.tpart_idx[base + c.i - c.nf] : p.tfull_idx[base + c.i];
      return qt * 128 + c.sub * QB;
    }
  };
  auto cur_next = [&](Cur& c) {
    if constexpr (!BM) {
      if (++c.i == n_qs) { c.i = 0; ++c.g; }
    } else {
      if (++c.sub == SPQ) {
        c.sub = 0;
        if (++c.i == c.nt) {
          c.i = 0;
          ++c.g;
          cur_head(c);
        }
      }
    }
  };

  // Copies: lane slot (inst*64 + lane) of a tile is row r, 16-byte chunk
  // ch ^ swz(r), as for the forward kernel's K/V tiles.
  uint32_t dma_row[PER_WAVE], qoff[PER_WAVE], dooff[PER_WAVE], dma_lds[PER_WAVE];
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int inst = wave * PER_WAVE + i;
    const uint32_t slot = inst * 64 + lane;
    const uint32_t row = slot / CPR;
    const uint32_t chunk = (slot % CPR) ^ Swz<D>::f(row);
    dma_row[i] = row;
    qoff[i] = (uint32_t)(row * p.q_sn + chunk * 8) * 2u;
    dooff[i] = (uint32_t)(row * p.do_sn + chunk * 8) * 2u;
    dma_lds[i] = __builtin_amdgcn_readfirstlane(inst * 1024);
  }
  // A-operand reads of Q and dO (row lane%32, chunk 2c + half) and the
  // transposing reads of Q^T / dO^T per 16-row chunk kc, d-block db, half e.
  uint32_t a_addr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) a_addr[c] = tile_off<D>(lane & 31, 2 * c + half);
  uint32_t t_addr[2][NDB][2];
  {
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t row = 16 * kc + 4 * (g >> 1) + (j >> 2) + 8 * e;
          const uint32_t dcol = 32 * db + 16 * (g & 1) + 4 * (j & 3);
          t_addr[kc][db][e] = tile_off<D>(row, dcol >> 3) + 8 * (j & 1);
        }
  }

  // Steps run head-major; a cursor per direction (copies issued, steps
  // computed) advances without divisions.
  const T* q_head = static_cast<const T*>(p.q) + b * p.q_sb + (int64_t)kvh * p.G * p.q_sh;
  const T* do_head = static_cast<const T*>(p.dout) + b * p.do_sb + (int64_t)kvh * p.G * p.do_sh;
  const float* ws_head = p.ws_l2 + (int64_t)(b * p.Hq + kvh * p.G) * p.nq_pad;
  const int64_t ws_delta_off = p.ws_delta - p.ws_l2;
  Cur ld;
  cur_init(ld);
  // The last QB-row block that holds a row: a BlockMask step past the last
  // row (the tail of a ragged last tile) copies that block instead and
  // computes nothing.
  const int last_q0 = p.Nq > 0 ? ((p.Nq - 1) / QB) * QB : 0;
  auto load_next = [&](int stage) {
    bool partial_unused;
    const int q0 = min(cur_q0(ld, partial_unused), last_q0);
    const int ld_g = ld.g;
    const uint32_t lb = lds_addr(smem) + stage * STAGE_BYTES;
    const T* qbase = q_head + ld_g * p.q_sh + (int64_t)q0 * p.q_sn;
    const T* dbase = do_head + ld_g * p.do_sh + (int64_t)q0 * p.do_sn;
    if (q0 + QB <= p.Nq) {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        dma16_sv(qbase, qoff[i], lb + dma_lds[i]);
        dma16_sv(dbase, dooff[i], lb + TILE_BYTES + dma_lds[i]);
      }
    } else {
      // Rows past the end repeat the last row (their P is masked to 0).
      const uint32_t last = (uint32_t)(p.Nq - 1 - q0);
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const uint32_t over = dma_row[i] > last ? dma_row[i] - last : 0u;
        dma16_sv(qbase, qoff[i] - over * (uint32_t)p.q_sn * 2u, lb + dma_lds[i]);
        dma16_sv(dbase, dooff[i] - over * (uint32_t)p.do_sn * 2u, lb + TILE_BYTES + dma_lds[i]);
      }
    }
    if (wave == 0) {
      // L2 (lanes 0 .. QB/4-1) then Delta (QB/4 .. QB/2-1), 16 bytes a lane;
      // the other lanes repeat them into the stage's padding.  Rows up to
      // q0 + QB lie inside the padded workspace row.
      const int li = lane % (QB / 2);
      const float* src = ws_head + (int64_t)ld_g * p.nq_pad + (li < QB / 4 ? 0 : ws_delta_off) + q0 +
                         4 * (li % (QB / 4));
      dma16(src, lb + LD_OFF);
    }
    cur_next(ld);
  };

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) dk[d] = dv[d] = f32x16{};

  Cur cc;
  cur_init(cc);
  auto step = [&](auto stc, int s) {
    constexpr int ST = decltype(stc)::value;
    wait_vmem();
    lds_barrier();
    if (s + 1 < n_steps) load_next(ST ^ 1);
    bool partial;
    const int q0 = cur_q0(cc, partial);
    const int g = cc.g;
    cur_next(cc);
    if (q0 >= p.Nq) return;  // tail of a ragged last BlockMask tile
    // rows outside the wave's keys' rows (only where the mask intervals apply)
    if (partial && (q0 > w_hi || q0 + QB - 1 < w_lo)) return;
    const bool full = !partial || (w_lo_max <= q0 && w_hi_min >= q0 + QB - 1);
    const TATTN_LDS char* tQ = smem + ST * STAGE_BYTES;
    const TATTN_LDS char* tD = tQ + TILE_BYTES;
    const TATTN_LDS float* tL = reinterpret_cast<const TATTN_LDS float*>(tQ + LD_OFF);
    // ---- S = Q K^T and dP = dO V^T for every 32-row block of the step ----
    f32x16 sacc[NQB], dpacc[NQB];
#pragma unroll
    for (int blk = 0; blk < NQB; ++blk) {
      const uint32_t roff = blk * 32 * ROW_BYTES;
      sacc[blk] = dpacc[blk] = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        sacc[blk] = mfma32(lds_read_b128<T>(tQ, a_addr[c] + roff), kf[c], sacc[blk]);
        dpacc[blk] = mfma32(lds_read_b128<T>(tD, a_addr[c] + roff), vf[c], dpacc[blk]);
      }
    }
    // Keep the operand reads about four MFMAs ahead of their use.
    constexpr int NSD = 2 * NQB * NC;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < NSD - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (!full) {
      // element r of block blk is row q0 + 32 blk + 8 (r/4) + 4 half + r%4
      const uint32_t width = qb >= qa ? (uint32_t)(qb - qa) : 0u;
      const uint32_t base = qb >= qa ? (uint32_t)(q0 + 4 * half - qa) : 0x80000000u;
#pragma unroll
      for (int blk = 0; blk < NQB; ++blk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t off = 32 * blk + 8 * (r >> 2) + (r & 3);
          if (base + off > width) sacc[blk][r] = kNegInf;
        }
    }
    // tanh of the capped scores (SOFTCAP only): dS takes the factor 1 - tanh^2
    f32x16 th[NQB];
    if constexpr (SM) {
      // scores now carry c2 (or the cap) and the bias of query head kvh G + g
      const ScoreHead hd{alibi_slope2(p.smod, kvh * p.G + g), tabs + g * (2 * p.smod.R + 1)};
      const int d0 = key - (int)(q0 + 4 * half + shift);
      add_score_bias<NQB, 16, true>(
          sacc, p.c2, p.smod, hd,
          [&](int blk, int r) { return d0 - (32 * blk + 8 * (r >> 2) + (r & 3)); }, th);
    }
#pragma unroll
    for (int blk = 0; blk < NQB; ++blk) {
      const uint32_t roff = blk * 32 * ROW_BYTES;
      // Its L2 and Delta: four float4 broadcast reads each.
      f32x4 l2[4], dl[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        l2[j] = *reinterpret_cast<const TATTN_LDS f32x4*>(tL + 32 * blk + 8 * j + 4 * half);
        dl[j] = *reinterpret_cast<const TATTN_LDS f32x4*>(tL + QB + 32 * blk + 8 * j + 4 * half);
      }
      float pr[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        pr[r] = fast_exp2(__builtin_fmaf(sacc[blk][r], SM ? 1.f : p.c2, -l2[r >> 2][r & 3]));
        ds[r] = pr[r] * (dpacc[blk][r] - dl[r >> 2][r & 3]);
      }
      if constexpr (SM) {
        if (p.smod.flags & ATTN_SCORE_SOFTCAP) {
#pragma unroll
          for (int r = 0; r < 16; ++r) ds[r] *= __builtin_fmaf(-th[blk][r], th[blk][r], 1.f);
        }
      }
      vec8<T> pp[2], pd[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        pp[c] = pack8<T>(pr[8 * c], pr[8 * c + 1], pr[8 * c + 2], pr[8 * c + 3], pr[8 * c + 4],
                      pr[8 * c + 5], pr[8 * c + 6], pr[8 * c + 7]);
        pd[c] = pack8<T>(ds[8 * c], ds[8 * c + 1], ds[8 * c + 2], ds[8 * c + 3], ds[8 * c + 4],
                      ds[8 * c + 5], ds[8 * c + 6], ds[8 * c + 7]);
      }
      // ---- dV^T += dO^T P and dK^T += Q^T dS over these 32 rows ----
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const i16x4 a0 = lds_read_tr16(tD, t_addr[c][db][0] + roff);
          const i16x4 a1 = lds_read_tr16(tD, t_addr[c][db][1] + roff);
          dv[db] = mfma32(join_tr<T>(a0, a1), pp[c], dv[db]);
          const i16x4 b0 = lds_read_tr16(tQ, t_addr[c][db][0] + roff);
          const i16x4 b1 = lds_read_tr16(tQ, t_addr[c][db][1] + roff);
          dk[db] = mfma32(join_tr<T>(b0, b1), pd[c], dk[db]);
        }
    }
  };

  if (n_steps > 0) load_next(0);
  for (int s0 = 0; s0 < n_steps; s0 += 2) {
    step(std::integral_constant<int, 0>{}, s0);
    if (s0 + 1 < n_steps) step(std::integral_constant<int, 1>{}, s0 + 1);
  }

  // ---- epilogue: lane owns key `key`, d = 32 db + 8 (r/4) + 4 half + r%4 ----
  if (key_ok) {
    T* dkrow = static_cast<T*>(p.dk) + b * p.dk_sb + kvh * p.dk_sh + (int64_t)key * p.dk_sn;
    T* dvrow = static_cast<T*>(p.dv) + b * p.dv_sb + kvh * p.dv_sh + (int64_t)key * p.dv_sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        *reinterpret_cast<vec4<T>*>(dkrow + 32 * db + 8 * r4 + 4 * half) =
            pack4<T>(dk[db][4 * r4] * p.scale, dk[db][4 * r4 + 1] * p.scale,
                     dk[db][4 * r4 + 2] * p.scale, dk[db][4 * r4 + 3] * p.scale);
        *reinterpret_cast<vec4<T>*>(dvrow + 32 * db + 8 * r4 + 4 * half) =
            pack4<T>(dv[db][4 * r4], dv[db][4 * r4 + 1], dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]);
      }
  }
}

// Waves per SIMD of the dK / dV kernel: at D=128 a wave holds 32 keys' K, V,
// dK and dV (256 registers before any temporary), so it takes the whole
// 512-entry register file of one SIMD lane.
template <int D> struct BwdKvOcc { static constexpr int value = D == 64 ? 2 : 1; };

template <int D, typename T, bool SM, bool BM>
__global__ void __launch_bounds__(kBwdThreads)
__attribute__((amdgpu_waves_per_eu(BwdKvOcc<D>::value, BwdKvOcc<D>::value)))
bwd_kv_kernel(const BwdParams p) {
  constexpr int STAGE_BYTES = 2 * BwdQRows<D>::value * D * 2 + 1024;
  // the ring (34 KB), then the G bias tables (up to 32 KB) when SM
  constexpr int LDS_BYTES = 2 * STAGE_BYTES + (SM ? kMaxRelTables * 4 : 0);
  static_assert(2 * STAGE_BYTES <= kLdsCopyLimit && LDS_BYTES <= kLdsFootprintLimit, "LDS limits");
  __shared__ __attribute__((aligned(1024))) char smem_raw[LDS_BYTES];
  TATTN_LDS char* smem = (TATTN_LDS char*)smem_raw;
  const int id = (p.sched & ATTN_SCHED_REVERSE) ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  int unit = id;
  if (p.kv_xcd_remap) {
    // whole KV heads per XCD, so their Q / dO tiles stay in one L2
    const int per = gridDim.x >> 3;
    unit = (id & 7) * per + (id >> 3);
  }
  const int slot = unit % p.kv_slots;
  const int r = unit / p.kv_slots;
  const int kvh = r % p.Hkv, b = r / p.Hkv;
  kv_tile<D, T, SM, BM>(p, smem, slot, b, kvh);
  if (p.kv_paired) {
    const int kt2 = p.n_kt - 1 - slot;
    if (kt2 != slot) {
      __syncthreads();
      kv_tile<D, T, SM, BM>(p, smem, kt2, b, kvh);
    }
  }
}

// ---- dQ -----------------------------------------------------------------------
// Keys per step as in the forward kernel: 128 at D=64, 64 at D=128.
template <int D> struct BwdKBlk { static constexpr int value = D == 64 ? 128 : 64; };

// BlockMask (BM): the query tile's FULL then PARTIAL key tiles of the
// forward lists, kKBlk keys a step, as in the forward kernel.
template <int D, typename T, bool SM, bool BM>
__device__ __forceinline__ void q_tile(const BwdParams& p, TATTN_LDS char* smem, int qt, int b,
                                       int h, int kvh) {
  constexpr int kKBlk = BwdKBlk<D>::value;
  constexpr int NKB = kKBlk / 32;
  constexpr int NC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CPR = D / 8;
  constexpr int TILE_BYTES = kKBlk * D * 2;
  constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  constexpr int PER_WAVE = kKBlk * CPR / 64 / (kBwdThreads / 64);
  constexpr int KC_PERIOD = D == 64 ? 2 : 1;  // 16-row chunks per swizzle period
  constexpr int ROW_BYTES = 2 * D;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5;
  const int64_t shift = (int64_t)p.Nk - p.Nq;

  const int q0 = qt * 128;
  const int qrow = q0 + wave * 32 + (lane & 31);
  const bool row_ok = qrow < p.Nq;
  const int rr = row_ok ? qrow : p.Nq - 1;

  // Q^T and dO^T: B operands of S^T = K Q^T and dP^T = V dO^T.
  vec8<T> qf[NC], df[NC];
  float l2, dl;
  {
    const T* qs = static_cast<const T*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)rr * p.q_sn + 8 * half;
    const T* ds = static_cast<const T*>(p.dout) + b * p.do_sb + h * p.do_sh + (int64_t)rr * p.do_sn + 8 * half;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qf[c] = *reinterpret_cast<const vec8<T>*>(qs + 16 * c);
      df[c] = *reinterpret_cast<const vec8<T>*>(ds + 16 * c);
    }
    const int64_t w = (int64_t)(b * p.Hq + h) * p.nq_pad + rr;
    l2 = p.ws_l2[w];
    dl = p.ws_delta[w];
    wait_vmem();
  }

  int lo, hi;
  row_interval(p.mask, b, qrow + shift, p.Nk, lo, hi);
  // Score change (SM): slope and LDS bias table of the head, after the ring.
  ScoreHead hd{0.f, nullptr};
  if constexpr (SM) {
    hd.slope2 = alibi_slope2(p.smod, h);
    TATTN_LDS float* tab = reinterpret_cast<TATTN_LDS float*>(smem + 2 * STAGE_BYTES);
    hd.tab = tab;
    if (p.smod.flags & ATTN_SCORE_REL_BIAS) stage_rel_table(p.smod, h, tab, tid, kBwdThreads);
  }
  constexpr int SPT = 128 / kKBlk;  // steps per 128-key BlockMask tile
  int n_steps = 0, kb_begin = 0, lo_last = 0, hi_first = 0;
  int64_t bm_base = 0;
  int bm_nf = 0;
  if constexpr (!BM) {
    int lo_first, hi_last, t0;
    const int last_row = min(q0 + 128, p.Nq) - 1;
    row_interval(p.mask, b, q0 + shift, p.Nk, lo_first, hi_first);
    row_interval(p.mask, b, last_row + shift, p.Nk, t0, hi_last);
    lo_last = t0;
    if (hi_last >= lo_first) {
      kb_begin = (lo_first / kKBlk) * kKBlk;
      n_steps = (hi_last + 1 - kb_begin + kKBlk - 1) / kKBlk;
    }
  } else {
    const int bb = p.bm_B > 1 ? b : 0, hh = p.bm_H > 1 ? h : 0;
    const int64_t row = ((int64_t)bb * p.bm_H + hh) * p.n_qt + qt;
    bm_nf = p.full_num[row];
    n_steps = SPT * (bm_nf + p.part_num[row]);
    bm_base = row * p.n_kt;
  }
  // First key of step s and whether it applies the row's mask interval
  // (dense masks: wherever a step is not inside every row's interval;
  // BlockMask: on PARTIAL tiles, and [0, Nk) on a ragged last tile).
  auto step_kb = [&](int s, bool& masked, bool& use_row) -> int {
    if constexpr (!BM) {
      const int kb = kb_begin + s * kKBlk;
      masked = !(kb >= lo_last && kb + kKBlk - 1 <= hi_first && kb + kKBlk <= p.Nk);
      use_row = true;
      return kb;
    } else {
      const int t = s / SPT;
      const bool partial = t >= bm_nf;
      const int kt = partial ? p.part_idx[bm_base + t - bm_nf] : p.full_idx[bm_base + t];
      const int kb = kt * 128 + (s % SPT) * kKBlk;
      use_row = partial;
      masked = partial || kb + kKBlk > p.Nk;
      return kb;
    }
  };

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
  }
  uint32_t k_addr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) k_addr[c] = tile_off<D>(lane & 31, 2 * c + half);
  uint32_t t_addr[KC_PERIOD][NDB][2];
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
          t_addr[kc][db][e] = tile_off<D>(row, dcol >> 3) + 8 * (j & 1);
        }
  }

  const T* Kbh = static_cast<const T*>(p.k) + b * p.k_sb + kvh * p.k_sh;
  const T* Vbh = static_cast<const T*>(p.v) + b * p.v_sb + kvh * p.v_sh;
  auto load_step = [&](int s, int stage) {
    bool m_unused, u_unused;
    int kb = step_kb(s, m_unused, u_unused);
    kb = kb > p.Nk - 1 ? p.Nk - 1 : kb;  // the tail of a ragged last BlockMask tile
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

  f32x16 dq[NDB];
#pragma unroll
  for (int d = 0; d < NDB; ++d) dq[d] = f32x16{};

  auto step = [&](auto stc, int s) {
    constexpr int ST = decltype(stc)::value;
    wait_vmem();
    lds_barrier();
    if (s + 1 < n_steps) load_step(s + 1, ST ^ 1);
    bool masked, use_row;
    const int kb = step_kb(s, masked, use_row);
    if (kb >= p.Nk) return;  // tail of a ragged last BlockMask tile
    const TATTN_LDS char* tK = smem + ST * STAGE_BYTES;
    const TATTN_LDS char* tV = tK + TILE_BYTES;
    const int lo_m = use_row ? lo : 0, hi_m = use_row ? hi : p.Nk - 1;
    const uint32_t base = (uint32_t)(kb + 4 * half - lo_m);
    const uint32_t width = hi_m >= lo_m ? (uint32_t)(hi_m - lo_m) : 0u;
    const uint32_t base_ok = hi_m >= lo_m ? base : 0x80000000u;
#pragma unroll
    for (int kbk = 0; kbk < NKB; ++kbk) {
      // ---- S^T = K Q^T and dP^T = V dO^T for 32 keys ----
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        sacc = mfma32(lds_read_b128<T>(tK, k_addr[c] + kbk * 32 * ROW_BYTES), qf[c], sacc);
        dpacc = mfma32(lds_read_b128<T>(tV, k_addr[c] + kbk * 32 * ROW_BYTES), df[c], dpacc);
      }
      // Keep the operand reads about four MFMAs ahead of their use.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * NC - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      // element r holds key kb + 32 kbk + 8 (r/4) + 4 half + r%4
      if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t off = 32 * kbk + 8 * (r >> 2) + (r & 3);
          if (base_ok + off > width) sacc[r] = kNegInf;
        }
      }
      f32x16 th;  // tanh of the capped scores (SOFTCAP only)
      if constexpr (SM) {
        const int d0 = kb + 32 * kbk + 4 * half - (int)(qrow + shift);
        add_score_bias<1, 16, true>(
            &sacc, p.c2, p.smod, hd, [&](int, int r) { return d0 + 8 * (r >> 2) + (r & 3); }, &th);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ds[r] = fast_exp2(__builtin_fmaf(sacc[r], SM ? 1.f : p.c2, -l2)) * (dpacc[r] - dl);
      if constexpr (SM) {
        if (p.smod.flags & ATTN_SCORE_SOFTCAP) {
#pragma unroll
          for (int r = 0; r < 16; ++r) ds[r] *= __builtin_fmaf(-th[r], th[r], 1.f);
        }
      }
      // ---- dQ^T += K^T dS^T over these 32 keys (two 16-key chunks) ----
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const vec8<T> pd = pack8<T>(ds[8 * c], ds[8 * c + 1], ds[8 * c + 2], ds[8 * c + 3],
                                ds[8 * c + 4], ds[8 * c + 5], ds[8 * c + 6], ds[8 * c + 7]);
        const int kc = 2 * kbk + c;
        const uint32_t kc_off = (kc / KC_PERIOD) * (16 * KC_PERIOD) * ROW_BYTES;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const i16x4 a0 = lds_read_tr16(tK, t_addr[kc % KC_PERIOD][db][0] + kc_off);
          const i16x4 a1 = lds_read_tr16(tK, t_addr[kc % KC_PERIOD][db][1] + kc_off);
          dq[db] = mfma32(join_tr<T>(a0, a1), pd, dq[db]);
        }
      }
    }
  };

  if (p.Nk > 0 && n_steps > 0) load_step(0, 0);
  for (int s0 = 0; s0 < n_steps; s0 += 2) {
    step(std::integral_constant<int, 0>{}, s0);
    if (s0 + 1 < n_steps) step(std::integral_constant<int, 1>{}, s0 + 1);
  }

  if (row_ok) {
    T* drow = static_cast<T*>(p.dq) + b * p.dq_sb + h * p.dq_sh + (int64_t)qrow * p.dq_sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        *reinterpret_cast<vec4<T>*>(drow + 32 * db + 8 * r4 + 4 * half) =
            pack4<T>(dq[db][4 * r4] * p.scale, dq[db][4 * r4 + 1] * p.scale,
                     dq[db][4 * r4 + 2] * p.scale, dq[db][4 * r4 + 3] * p.scale);
      }
  }
}

template <int D, typename T, bool SM, bool BM>
__global__ void __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_q_kernel(const BwdParams p) {
  // the ring (64 KB), then the head's bias table (8 KB) when SM
  constexpr int RING = 2 * 2 * BwdKBlk<D>::value * D * 2;
  constexpr int LDS_BYTES = RING + (SM ? kMaxRelTable * 4 : 0);
  static_assert(RING <= kLdsCopyLimit && LDS_BYTES <= kLdsFootprintLimit, "LDS limits");
  __shared__ __attribute__((aligned(1024))) char smem_raw[LDS_BYTES];
  TATTN_LDS char* smem = (TATTN_LDS char*)smem_raw;
  const int id = (p.sched & ATTN_SCHED_REVERSE) ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  int unit = id;
  if (p.q_xcd_remap) {
    const int per = gridDim.x >> 3;
    unit = (id & 7) * per + (id >> 3);
  }
  // unit = ((b * Hkv + kvh) * q_slots + slot) * G + g, as in the forward pass
  const int g = unit % p.G;
  int r = unit / p.G;
  const int slot = r % p.q_slots;
  r /= p.q_slots;
  const int kvh = r % p.Hkv, b = r / p.Hkv;
  const int h = kvh * p.G + g;
  q_tile<D, T, SM, BM>(p, smem, slot, b, h, kvh);
  if (p.q_paired) {
    const int qt2 = p.n_qt - 1 - slot;
    if (qt2 != slot) {
      __syncthreads();
      q_tile<D, T, SM, BM>(p, smem, qt2, b, h, kvh);
    }
  }
}

template <int D, typename T, bool BM>
void launch_bwd_t(const BwdParams& p, dim3 gpre, dim3 gkv, dim3 gq, dim3 block, hipStream_t stream) {
  if (gpre.x) hipLaunchKernelGGL((bwd_pre_kernel<D, T>), gpre, block, 0, stream, p);
  if constexpr (BM) {  // no score change over a BlockMask (the host rejects it)
    if (gkv.x) hipLaunchKernelGGL((bwd_kv_kernel<D, T, false, true>), gkv, block, 0, stream, p);
    if (gq.x) hipLaunchKernelGGL((bwd_q_kernel<D, T, false, true>), gq, block, 0, stream, p);
  } else if (p.smod.flags) {
    if (gkv.x) hipLaunchKernelGGL((bwd_kv_kernel<D, T, true, BM>), gkv, block, 0, stream, p);
    if (gq.x) hipLaunchKernelGGL((bwd_q_kernel<D, T, true, BM>), gq, block, 0, stream, p);
  } else {
    if (gkv.x) hipLaunchKernelGGL((bwd_kv_kernel<D, T, false, BM>), gkv, block, 0, stream, p);
    if (gq.x) hipLaunchKernelGGL((bwd_q_kernel<D, T, false, BM>), gq, block, 0, stream, p);
  }
}

int launch_bwd(const BwdParams& p, int D, int dtype, bool blockmask, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.Hq * p.nq_pad;
  const dim3 block(kBwdThreads);
  const dim3 gpre((unsigned)((rows * 8 + kBwdThreads - 1) / kBwdThreads));
  const dim3 gkv((unsigned)((int64_t)p.B * p.Hkv * p.kv_slots));
  const dim3 gq((unsigned)((int64_t)p.B * p.Hq * p.q_slots));
  const bool f16in = dtype == ATTN_DTYPE_F16;
  if (blockmask) {
    if (D == 64) {
      if (f16in) launch_bwd_t<64, f16, true>(p, gpre, gkv, gq, block, stream);
      else launch_bwd_t<64, bf16, true>(p, gpre, gkv, gq, block, stream);
    } else {
      if (f16in) launch_bwd_t<128, f16, true>(p, gpre, gkv, gq, block, stream);
      else launch_bwd_t<128, bf16, true>(p, gpre, gkv, gq, block, stream);
    }
  } else if (D == 64) {
    if (f16in) launch_bwd_t<64, f16, false>(p, gpre, gkv, gq, block, stream);
    else launch_bwd_t<64, bf16, false>(p, gpre, gkv, gq, block, stream);
  } else {
    if (f16in) launch_bwd_t<128, f16, false>(p, gpre, gkv, gq, block, stream);
    else launch_bwd_t<128, bf16, false>(p, gpre, gkv, gq, block, stream);
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace tattn
