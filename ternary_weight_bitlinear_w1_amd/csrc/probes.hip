// Measurement probes: what this GPU achieves on the two resources the BitLinear
// kernels are bound by, measured in the same process as the kernels. They are
// denominators for the roofline fractions, not steps of the method.
//
// probe_read_kernel: a coalesced stream of 16-byte loads over a buffer, every
// load of a thread issued before any is consumed, folded into one value that is
// stored only if it equals a key passed at run time (so the compiler keeps the
// loads; a chance match writes one dword to the sink, which nothing reads). One launch over a buffer of a decode projection's
// size gives that size's per-launch floor; over a buffer larger than the
// last-level cache, the HBM read rate.
//
// probe_mfma_kernel: independent chains of v_mfma_i32_32x32x32_i8 per wave,
// no memory traffic: the int8 matrix-core issue rate.
#include "common.h"

namespace bl {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const v4i *__restrict__ src, int64_t n16,
                                                                   uint32_t key, uint32_t *__restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  v4i acc = v4i{0, 0, 0, 0};
  for (; i < n16; i += kProbeUnroll * stride) {
    v4i v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + u * stride;
      v[u] = j < n16 ? src[j] : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  const uint32_t f = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  if (f == key) sink[0] = f;
}

__global__ __launch_bounds__(256, 2) void probe_mfma_kernel(int iters, int32_t key, int32_t *__restrict__ sink) {
  v16i acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[c][q] = 0;
  const v4i a = v4i{(int)threadIdx.x, 1, 2, 3}, b = v4i{3, 2, 1, (int)blockIdx.x};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
  int s = 0;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int q = 0; q < 16; ++q) s ^= acc[c][q];
  if (s == key) sink[0] = s;
}

}  // namespace

hipError_t launch_probe_read(const void *src, int64_t bytes, uint32_t *sink, int64_t grid, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  if (grid <= 0) grid = (n16 + kProbeThreads * kProbeUnroll - 1) / (kProbeThreads * kProbeUnroll);
  if (grid > 65536) grid = 65536;
  probe_read_kernel<<<dim3((unsigned)grid), dim3(kProbeThreads), 0, stream>>>(static_cast<const v4i *>(src), n16,
                                                                             0x9e3779b9u, sink);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int iters, int64_t workgroups, int32_t *sink, hipStream_t stream) {
  probe_mfma_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, stream>>>(iters, 0x7f4a7c15, sink);
  return hipGetLastError();
}

}  // namespace bl
