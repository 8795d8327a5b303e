// BlockMask builder for gfx950: classifies 128 x 128 (query tile, key tile)
// pairs as EMPTY / PARTIAL / FULL and compacts each query-tile row into
// ascending lists of PARTIAL and FULL key tiles -- the block sparsity of the
// FlexAttention / DFlash article (section 1), where fully masked blocks are
// skipped and only partial blocks evaluate the mask predicate.
//
// One work group (4 waves) per (batch row, head, query tile).  The 128 row
// intervals of the tile are evaluated once into LDS; each thread then
// classifies one key tile against them; a ballot-based block scan assigns
// list positions so the lists come out in ascending order with no atomics.
#include "params.h"

namespace tattn {

__global__ void __launch_bounds__(256) blockmask_kernel(const BmBuildParams p) {
  __shared__ int s_lo[ATTN_BLOCKMASK_TILE];
  __shared__ int s_hi[ATTN_BLOCKMASK_TILE];
  __shared__ int s_cnt[2][4];
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int q0 = qt * ATTN_BLOCKMASK_TILE;
  const int n_rows = min(ATTN_BLOCKMASK_TILE, p.Nq - q0);
  if (p.tile_map == nullptr && tid < ATTN_BLOCKMASK_TILE) {
    int lo = 1, hi = 0;
    if (tid < n_rows) row_interval(p.mask, b, q0 + tid + p.shift, p.Nk, lo, hi);
    s_lo[tid] = lo;
    s_hi[tid] = hi;
  }
  __syncthreads();
  const int64_t row = ((int64_t)b * p.Hm + h) * p.nQt + qt;
  const int64_t lbase = row * p.nKt;
  int np = 0, nf = 0;
  for (int base = 0; base < p.nKt; base += 256) {
    const int kt = base + tid;
    int cls = ATTN_TILE_EMPTY;
    if (kt < p.nKt) {
      if (p.tile_map != nullptr) {
        const int c = p.tile_map[lbase + kt];
        cls = (c == ATTN_TILE_PARTIAL || c == ATTN_TILE_FULL) ? c : ATTN_TILE_EMPTY;
      } else {
        const int k0 = kt * ATTN_BLOCKMASK_TILE;
        const int k1 = min(p.Nk, k0 + ATTN_BLOCKMASK_TILE) - 1;
        bool any = false, all = true;
        for (int r = 0; r < n_rows; ++r) {
          const int lo = s_lo[r], hi = s_hi[r];
          if (max(lo, k0) <= min(hi, k1)) any = true;
          if (!(lo <= k0 && hi >= k1)) all = false;
        }
        cls = !any ? ATTN_TILE_EMPTY : (all ? ATTN_TILE_FULL : ATTN_TILE_PARTIAL);
      }
    }
    const uint64_t bp = __ballot(cls == ATTN_TILE_PARTIAL);
    const uint64_t bf = __ballot(cls == ATTN_TILE_FULL);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (lane == 0) {
      s_cnt[0][wave] = __popcll(bp);
      s_cnt[1][wave] = __popcll(bf);
    }
    __syncthreads();
    int offp = np + __popcll(bp & below), offf = nf + __popcll(bf & below);
    int totp = 0, totf = 0;
    for (int w = 0; w < 4; ++w) {
      if (w < wave) { offp += s_cnt[0][w]; offf += s_cnt[1][w]; }
      totp += s_cnt[0][w];
      totf += s_cnt[1][w];
    }
    if (cls == ATTN_TILE_PARTIAL) p.part_idx[lbase + offp] = kt;
    if (cls == ATTN_TILE_FULL) p.full_idx[lbase + offf] = kt;
    np += totp;
    nf += totf;
    __syncthreads();
  }
  for (int i = np + tid; i < p.nKt; i += 256) p.part_idx[lbase + i] = 0;
  for (int i = nf + tid; i < p.nKt; i += 256) p.full_idx[lbase + i] = 0;
  if (tid == 0) {
    p.part_num[row] = np;
    p.full_num[row] = nf;
  }
}

// Key-tile-major class map of a BlockMask: map_t[b][h][kt][qt] = the class of
// tile (qt, kt) in the lists (binary search in the ascending FULL and PARTIAL
// lists of row qt).  Every entry is written, so the map needs no clearing.
// One work group per (batch row, head, query tile); a thread per key tile.
__global__ void __launch_bounds__(256) blockmask_transpose_kernel(const BmTransposeParams p) {
  const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int64_t row = ((int64_t)b * p.Hm + h) * p.nQt + qt;
  const int nf = p.full_num[row], np = p.part_num[row];
  const int32_t* fi = p.full_idx + row * p.nKt;
  const int32_t* pi = p.part_idx + row * p.nKt;
  auto in_list = [](const int32_t* a, int n, int key) {
    int lo = 0, hi = n - 1;
    while (lo <= hi) {
      const int mid = (lo + hi) >> 1;
      const int v = a[mid];
      if (v == key) return true;
      if (v < key) lo = mid + 1; else hi = mid - 1;
    }
    return false;
  };
  uint8_t* dst = p.map_t + ((int64_t)b * p.Hm + h) * p.nKt * p.nQt + qt;
  for (int kt = threadIdx.x; kt < p.nKt; kt += 256) {
    const int c = in_list(fi, nf, kt) ? ATTN_TILE_FULL
                                      : (in_list(pi, np, kt) ? ATTN_TILE_PARTIAL : ATTN_TILE_EMPTY);
    dst[(int64_t)kt * p.nQt] = (uint8_t)c;
  }
}

int launch_blockmask_transpose(const BmTransposeParams& p, hipStream_t stream) {
  dim3 grid(p.nQt, p.Hm, p.Bm), block(256);
  hipLaunchKernelGGL(blockmask_transpose_kernel, grid, block, 0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int launch_blockmask(const BmBuildParams& p, hipStream_t stream) {
  dim3 grid(p.nQt, p.Hm, p.Bm), block(256);
  hipLaunchKernelGGL(blockmask_kernel, grid, block, 0, stream, p);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace tattn
