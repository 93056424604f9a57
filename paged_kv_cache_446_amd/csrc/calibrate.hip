// Measurement only, not part of the attention path: a read-only stream over one
// device buffer, the practical HBM read rate that the decode kernel's traffic is
// compared with beside the 8 TB/s peak.
//
// Each thread keeps four 16-byte non-temporal loads in flight per round
// (grid-stride over the buffer) and folds them with XOR so the loads cannot be
// dropped; the fold reaches memory only in the (data-dependent, practically never
// taken) case that all its bits are set.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"
#include "pkv_device.h"

namespace pkv {

typedef uint32_t stream_v4 __attribute__((ext_vector_type(4)));

constexpr int kStreamDepth = 4;
constexpr int kStreamThreads = 256;
constexpr int64_t kStreamMaxGrid = 65536;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                                    int64_t n, u32x4* sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  for (; i + (kStreamDepth - 1) * stride < n; i += kStreamDepth * stride) {
    u32x4 b[kStreamDepth];
#pragma unroll
    for (int u = 0; u < kStreamDepth; ++u)
      b[u] = __builtin_bit_cast(u32x4, __builtin_nontemporal_load((const stream_v4*)(p + i + u * stride)));
#pragma unroll
    for (int u = 0; u < kStreamDepth; ++u) {
      a0 ^= b[u].x;
      a1 ^= b[u].y;
      a2 ^= b[u].z;
      a3 ^= b[u].w;
    }
  }
  for (; i < n; i += stride) {
    const u32x4 b = p[i];
    a0 ^= b.x;
    a1 ^= b.y;
    a2 ^= b.z;
    a3 ^= b.w;
  }
  if ((a0 & a1 & a2 & a3) == 0xFFFFFFFFu) {
    u32x4 r;
    r.x = a0;
    r.y = a1;
    r.z = a2;
    r.w = a3;
    sink[0] = r;
  }
}

}  // namespace pkv

extern "C" int pkv_calib_stream_read(const void* buf, size_t bytes, void* sink, void* stream) {
  using namespace pkv;
  if (bytes == 0) return PKV_OK;
  if (!buf || !sink || bytes % 16 != 0 || (uintptr_t)buf % 16 != 0 || (uintptr_t)sink % 16 != 0)
    return PKV_ERR_INVALID_ARGUMENT;
  const int64_t n = (int64_t)(bytes / 16);
  int64_t grid = (n + (int64_t)kStreamThreads * kStreamDepth - 1) / ((int64_t)kStreamThreads * kStreamDepth);
  if (grid > kStreamMaxGrid) grid = kStreamMaxGrid;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kStreamThreads), 0,
                     (hipStream_t)stream, (const u32x4*)buf, n, (u32x4*)sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
