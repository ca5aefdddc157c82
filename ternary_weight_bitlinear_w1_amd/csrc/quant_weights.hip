// Absmean ternarization of fp32 master weights and four-to-a-byte packing
// (gfx950). Offline step of the packed checkpoint mode: the nnterp "BitNet
// b1.58" page, "The projections quantize their inputs and weights" (weights
// rounded to {-1, 0, 1} * mean|W|, stored four to a byte with a weight_scale)
// and "The two checkpoints"; the model card's "Model Details" (absmean).
//
// gamma = mean|W| is reduced in fp64 in a fixed order: each of G workgroups
// (G depends only on the element count) sums a fixed contiguous slice, thread
// by thread and then by a fixed wave/block tree; one workgroup then adds the G
// partials in a fixed tree. Results are bit-identical run to run.
// Codes compare |W| with gamma / 2 in fp64, which is exact; a tie gives 0.
// Packing: word g of a row holds codes 16g..16g+15; code 16g + 4t + b is the
// field u = c + 1 at bits 8b + 2t (see the layout note in bitlinear.h).
#include "common.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPartials = 2048;
constexpr int64_t kPerBlock = 1 << 14;  // elements per partial, at least
constexpr int kUnroll = 8;              // float4 loads in flight per thread

__device__ __forceinline__ double block_sum(double v, double *red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) t += red[w];
  return t;
}

// partials[b] = sum |w| over elements [b * per, min((b+1) * per, count)), per % 4 == 0
__global__ __launch_bounds__(kThreads) void absmean_partial_kernel(const float *__restrict__ w, int64_t count,
                                                                   int64_t per, double *__restrict__ partials) {
  __shared__ double red[kThreads / 64];
  const int64_t lo = blockIdx.x * per;
  const int64_t hi = lo + per < count ? lo + per : count;
  // thread t adds elements t, t + 256, ... (in float4 units) of the slice in
  // order; kUnroll loads are issued before their sums
  double s = 0.0;
  for (int64_t i0 = lo + 4 * (int64_t)threadIdx.x; i0 < hi; i0 += 4 * kThreads * kUnroll) {
    float4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t i = i0 + 4 * (int64_t)kThreads * j;
      v[j] = i < hi ? *reinterpret_cast<const float4 *>(w + i) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      s += fabs((double)v[j].x);
      s += fabs((double)v[j].y);
      s += fabs((double)v[j].z);
      s += fabs((double)v[j].w);
    }
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void absmean_final_kernel(const double *__restrict__ partials, int np,
                                                                 int64_t count, double *__restrict__ gamma) {
  __shared__ double red[kThreads / 64];
  double s = 0.0;
  for (int i = threadIdx.x; i < np; i += kThreads) s += partials[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) gamma[0] = count > 0 ? s / (double)count : 0.0;
}

// one thread per packed 32-bit word (16 codes)
__global__ __launch_bounds__(kThreads) void ternarize_pack_kernel(const float *__restrict__ w, int64_t words,
                                                                  const double *__restrict__ gamma,
                                                                  uint32_t *__restrict__ packed) {
  const double half = 0.5 * gamma[0];
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < words; i += (int64_t)gridDim.x * kThreads) {
    const float4 *src = reinterpret_cast<const float4 *>(w + 16 * i);
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 f = src[j];
      v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
    }
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const uint32_t u = fabs((double)v[t]) > half ? (v[t] > 0.0f ? 2u : 0u) : 1u;
      word |= u << (8 * (t & 3) + 2 * (t >> 2));
    }
    packed[i] = word;
  }
}

__global__ void copy_gamma_kernel(const double *__restrict__ src, double *__restrict__ dst) {
  if (threadIdx.x == 0 && blockIdx.x == 0) dst[0] = src[0];
}

__global__ void zero_i64_kernel(int64_t *p) {
  if (threadIdx.x == 0 && blockIdx.x == 0) p[0] = 0;
}

// fields equal to 3 have both bits set: popcount(w & (w >> 1) & 0x55555555)
__global__ __launch_bounds__(kThreads) void validate_kernel(const uint32_t *__restrict__ packed, int64_t words,
                                                            int64_t *__restrict__ n_bad) {
  __shared__ int red[kThreads / 64];
  int c = 0;
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < words; i += (int64_t)gridDim.x * kThreads) {
    const uint32_t v = packed[i];
    c += __popc(v & (v >> 1) & 0x55555555u);
  }
  c = wave_sum(c);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t += red[w];
    if (t) atomicAdd(reinterpret_cast<unsigned long long *>(n_bad), (unsigned long long)t);
  }
}

int64_t partial_span(int64_t count) {
  int64_t per = kPerBlock;
  while ((count + per - 1) / per > kMaxPartials) per *= 2;
  return per;
}

unsigned grid_for(int64_t items) {
  int64_t b = (items + kThreads - 1) / kThreads;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

}  // namespace

size_t absmean_partials(int64_t count) {
  if (count <= 0) return 1;
  const int64_t per = partial_span(count);
  return (size_t)((count + per - 1) / per);
}

hipError_t launch_absmean(const float *w, int64_t count, double *partials, double *gamma_out, hipStream_t stream) {
  if (count <= 0) {
    zero_i64_kernel<<<1, 64, 0, stream>>>(reinterpret_cast<int64_t *>(gamma_out));  // 0.0 is all-zero bits
    return hipGetLastError();
  }
  const int64_t per = partial_span(count);
  const int np = (int)((count + per - 1) / per);
  absmean_partial_kernel<<<dim3(np), dim3(kThreads), 0, stream>>>(w, count, per, partials);
  absmean_final_kernel<<<dim3(1), dim3(kThreads), 0, stream>>>(partials, np, count, gamma_out);
  return hipGetLastError();
}

hipError_t launch_ternarize_pack(const float *w, int64_t n, int64_t k, const double *gamma, uint8_t *packed,
                                 hipStream_t stream) {
  const int64_t words = n * (k / 16);
  if (words == 0) return hipSuccess;
  ternarize_pack_kernel<<<dim3(grid_for(words)), dim3(kThreads), 0, stream>>>(w, words, gamma,
                                                                               reinterpret_cast<uint32_t *>(packed));
  return hipGetLastError();
}

hipError_t launch_copy_gamma(const double *src, double *dst, hipStream_t stream) {
  copy_gamma_kernel<<<1, 64, 0, stream>>>(src, dst);
  return hipGetLastError();
}

hipError_t launch_validate_packed(const uint8_t *packed, int64_t n, int64_t k, int64_t *n_bad, hipStream_t stream) {
  zero_i64_kernel<<<1, 64, 0, stream>>>(n_bad);
  const int64_t words = n * (k / 16);
  if (words > 0)
    validate_kernel<<<dim3(grid_for(words)), dim3(kThreads), 0, stream>>>(reinterpret_cast<const uint32_t *>(packed),
                                                                          words, n_bad);
  return hipGetLastError();
}

}  // namespace bl
