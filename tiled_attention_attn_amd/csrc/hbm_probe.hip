// Read-only HBM streaming kernel: the measured read ceiling the decode
// kernel's bandwidth is compared against.
//
// Every lane reads 16-byte vectors of the buffer (grid-stride, UNROLL loads
// in flight per lane before any is consumed) and folds them into one word
// with XOR; a work group writes one word.  The bytes read are the buffer's
// size; the bytes written (one word per group) are negligible.  Nothing of
// the attention arithmetic is here: the kernel exists so a benchmark can
// state the rate a plain read stream reaches on the same device, in the same
// process, next to the decode kernel's rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tiled_attn.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kProbeThreads)
stream_read_kernel(const u32x4* __restrict__ src, uint64_t n16, uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
  uint64_t i = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // whole rounds of kUnroll vectors per lane
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  // One word per lane reduced over the group through LDS would cost more
  // than it shows; a group writes its first lane's fold (the loads above
  // cannot be removed: every value reaches acc).
  __shared__ uint32_t s_fold[kProbeThreads];
  s_fold[threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t f = 0;
    for (int t = 0; t < kProbeThreads; ++t) f ^= s_fold[t];
    sink[blockIdx.x] = f;
  }
}

}  // namespace

extern "C" int attn_probe_stream_read(const void* src, size_t bytes, int blocks, uint32_t* sink,
                                      hipStream_t stream) {
  if (src == nullptr || sink == nullptr) return ATTN_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (bytes & 15u) != 0) return ATTN_ERR_ALIGN;
  if (blocks < 1 || blocks > (1 << 20)) return ATTN_ERR_SHAPE;
  if (bytes == 0) return ATTN_OK;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), (uint64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
