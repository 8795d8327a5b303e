// Paged split-KV decode that allocates nothing: attn_decode_splitkv followed by
// attn_decode_combine, with the split partials in a library-owned static
// device buffer instead of a caller workspace.  For callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid it).
//
// The buffer is one file-scope __device__ array per GPU, held until the
// process ends.  In host code the array's name is only a host-side stand-in,
// so its device address is looked up once per device (hipGetSymbolAddress,
// with that device current) and that address is what the kernels receive.
// The split kernel writes every (row, split) partial it owns -- O_s and
// LSE_s, also for splits with no visible key -- before the combine reads
// them, so nothing in the buffer has to start at zero.  Every call on a GPU
// shares that GPU's buffer: calls that overlap on one GPU (two streams, two
// host threads) race.
#include <mutex>

#include "params.h"

namespace {

constexpr size_t kNoAllocBytes = size_t(32) << 20;
constexpr size_t kLseAlign = 256;
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) char scratch[kNoAllocBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's buffer (looked up on its first use).
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ATTN_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

size_t attn_decode_noalloc_max_bytes(void) { return kNoAllocBytes; }

int attn_decode_noalloc(const void* q, const int64_t q_stride[3], const void* k_cache,
                        const void* v_cache, int64_t num_pages, const int32_t* block_table,
                        int64_t bt_stride, const int32_t* seq_lens, int max_pages, int B, int Hq,
                        int Hkv, int Lq, int D, int dtype, int page_size, int num_splits,
                        float scale, const attn_mask_desc* mask, const attn_score_mod* smod,
                        void* o, const int64_t o_stride[3], float* lse, hipStream_t stream) {
  // The combine's own checks first: with an error nothing may be launched.
  if (!o || !o_stride) return ATTN_ERR_NULL;
  for (int i = 0; i < 3; ++i)
    if (o_stride[i] < 0 || (o_stride[i] & 7) != 0) return ATTN_ERR_STRIDE;
  if (!aligned16(o)) return ATTN_ERR_ALIGN;
  if (B < 0 || Hq < 0 || Lq < 0) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return ATTN_ERR_HEAD_DIM;
  if (num_splits < 1 || num_splits > 65536) return ATTN_ERR_WORKSPACE;
  if (B > 65535 || Hq > 65535 || Lq > 65536) return ATTN_ERR_SHAPE;
  // Partials: ws_o [B][Hq][Lq][S][D] floats, then (256-byte aligned) ws_lse [B][Hq][Lq][S].
  const uint64_t parts = (uint64_t)B * Hq * Lq;  // < 2^48
  const uint64_t per_row = (uint64_t)num_splits * (uint64_t)(D + 1) * sizeof(float);
  if (parts != 0 && parts > kNoAllocBytes / per_row) return ATTN_ERR_WORKSPACE;
  const size_t o_bytes = (size_t)parts * num_splits * D * sizeof(float);
  const size_t lse_off = (o_bytes + kLseAlign - 1) / kLseAlign * kLseAlign;
  const size_t lse_bytes = (size_t)parts * num_splits * sizeof(float);
  if (lse_off + lse_bytes > kNoAllocBytes) return ATTN_ERR_WORKSPACE;
  if (B == 0 || Hq == 0 || Lq == 0) {
    // An empty problem launches nothing.  The split entry point still reports
    // its argument errors; it gets placeholder workspace pointers, which it
    // never dereferences when there is nothing to compute.
    return attn_decode_splitkv(q, q_stride, k_cache, v_cache, num_pages, block_table, bt_stride,
                               seq_lens, max_pages, B, Hq, Hkv, Lq, D, dtype, page_size,
                               num_splits, scale, mask, smod, reinterpret_cast<float*>(16),
                               reinterpret_cast<float*>(16), stream);
  }
  void* base = nullptr;
  int st = scratch_ptr(&base);
  if (st) return st;
  float* ws_o = static_cast<float*>(base);
  float* ws_lse = reinterpret_cast<float*>(static_cast<char*>(base) + lse_off);
  // attn_decode_splitkv validates everything else before it launches.
  st = attn_decode_splitkv(q, q_stride, k_cache, v_cache, num_pages, block_table, bt_stride,
                           seq_lens, max_pages, B, Hq, Hkv, Lq, D, dtype, page_size, num_splits,
                           scale, mask, smod, ws_o, ws_lse, stream);
  if (st) return st;
  return attn_decode_combine(ws_o, ws_lse, B, Hq, Lq, num_splits, D, dtype, o, o_stride, lse,
                             stream);
}

}  // extern "C"
