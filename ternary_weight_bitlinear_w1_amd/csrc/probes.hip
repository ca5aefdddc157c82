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
// no memory traffic: the int8 matrix-core issue rate. With fixed operands
// (every MFMA of a lane multiplies the same small values) it shows the issue
// rate at the clock such light work allows; with varied operands (VARIED:
// four operand sets per lane, consecutive MFMAs of a wave taking different
// ones, A values in {0, 1, 2} like the unpacked ternary codes and B any int8
// like the activation codes) the matrix cores switch as in the GEMMs, draw
// more power, and the clock the GPU then holds sets the rate a contraction
// over such data can reach.
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

// xorshift32 (Marsaglia, "Xorshift RNGs", 2003): operand bytes for the
// varied-operand probe
__device__ __forceinline__ uint32_t xorshift32(uint32_t &h) {
  h ^= h << 13;
  h ^= h >> 17;
  h ^= h << 5;
  return h;
}

template <bool VARIED>
__global__ __launch_bounds__(256, 2) void probe_mfma_kernel(int iters, int32_t key, int32_t *__restrict__ sink) {
  v16i acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[c][q] = 0;
  if constexpr (VARIED) {
    v4i a[4], b[4];
    uint32_t h = threadIdx.x * 0x9E3779B9u + blockIdx.x * 0x85EBCA6Bu + 0x2545F491u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t u = xorshift32(h) & 0x03030303u;
        u -= (u & (u >> 1)) & 0x01010101u;  // byte value 3 -> 2
        a[i][q] = (int)u;
        b[i][q] = (int)xorshift32(h);
      }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[c & 3], b[(c + 1 + (c >> 2)) & 3], acc[c], 0, 0, 0);
  } else {
    const v4i a = v4i{(int)threadIdx.x, 1, 2, 3}, b = v4i{3, 2, 1, (int)blockIdx.x};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[c], 0, 0, 0);
  }
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

hipError_t launch_probe_mfma(int iters, int64_t workgroups, bool varied, int32_t *sink, hipStream_t stream) {
  if (varied)
    probe_mfma_kernel<true><<<dim3((unsigned)workgroups), dim3(256), 0, stream>>>(iters, 0x7f4a7c15, sink);
  else
    probe_mfma_kernel<false><<<dim3((unsigned)workgroups), dim3(256), 0, stream>>>(iters, 0x7f4a7c15, sink);
  return hipGetLastError();
}

}  // namespace bl
