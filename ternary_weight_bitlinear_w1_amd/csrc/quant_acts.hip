// Per-token int8 quantization of fp32 activations, with the fused prologues
// of a BitNet b1.58 block (gfx950): one workgroup per token row, 256 threads,
// or 512 for 17 to 128 rows (each thread then walks a quarter as many
// elements); the arithmetic is quant_row (act_prologue.h).
// HBM-bound: 4 (or 8 for gate|up, 8 for the residual pair) bytes read and
// 1 byte written per element.
#include "act_prologue.h"

namespace bl {
namespace {

constexpr int kThreads = kQuantThreads;

template <int MODE, int NV, bool PART, int TH>
__global__ __launch_bounds__(TH) void quant_acts_kernel(Src s, int8_t *__restrict__ codes,
                                                        float *__restrict__ deq, int32_t *__restrict__ rowsum,
                                                        float eps) {
  __shared__ float red_f[TH / 64];
  __shared__ double red_d[TH / 64];
  __shared__ int red_i[TH / 64];
  const int64_t r = blockIdx.x;
  int *crow = reinterpret_cast<int *>(codes + r * (int64_t)s.k);
  const RowQuant q = quant_row<MODE, NV, PART, TH>(s, r, eps, crow, red_f, red_d, red_i);
  if (threadIdx.x == 0) {
    if (rowsum) rowsum[r] = q.rowsum;
    deq[r] = q.deq;
  }
}

template <int MODE, bool PART, int TH>
hipError_t launch_threads(const Src &s, int64_t m, int8_t *codes, float *deq, int32_t *rowsum, float eps,
                          hipStream_t stream) {
  const int per_thread = (s.k / 4 + TH - 1) / TH;
  dim3 grid((unsigned)m), block(TH);
  if (per_thread <= 1)
    quant_acts_kernel<MODE, 1, PART, TH><<<grid, block, 0, stream>>>(s, codes, deq, rowsum, eps);
  else if (per_thread <= 2)
    quant_acts_kernel<MODE, 2, PART, TH><<<grid, block, 0, stream>>>(s, codes, deq, rowsum, eps);
  else if (per_thread <= 4)
    quant_acts_kernel<MODE, 4, PART, TH><<<grid, block, 0, stream>>>(s, codes, deq, rowsum, eps);
  else if (per_thread <= 8)
    quant_acts_kernel<MODE, 8, PART, TH><<<grid, block, 0, stream>>>(s, codes, deq, rowsum, eps);
  else
    quant_acts_kernel<MODE, 0, PART, TH><<<grid, block, 0, stream>>>(s, codes, deq, rowsum, eps);
  return hipGetLastError();
}

// 17 to 128 rows (too few to fill the CUs) take 512-thread workgroups:
// measured on the 30-layer stack at 64 tokens, 1.510-1.518 ms against 1.528
// with 320 threads, 1.515-1.518 with 448 or 640 and 1.550-1.556 with 1024
// (and, in an earlier form of the step, 1.673 ms with 256); at 3 and 4 tokens
// a wide form was 1-2% slower than 256 threads.
template <int MODE, bool PART = false>
hipError_t launch_mode(const Src &s, int64_t m, int8_t *codes, float *deq, int32_t *rowsum, float eps,
                       hipStream_t stream) {
  if (m > 16 && m <= 128) return launch_threads<MODE, PART, 512>(s, m, codes, deq, rowsum, eps, stream);
  return launch_threads<MODE, PART, kThreads>(s, m, codes, deq, rowsum, eps, stream);
}

// ---------------------------------------------------------------- helpers
__global__ __launch_bounds__(kThreads) void code_rowsum_kernel(const int8_t *__restrict__ codes, int k,
                                                               int32_t *__restrict__ rowsum) {
  __shared__ int red[kThreads / 64];
  const int64_t r = blockIdx.x;
  const int8_t *row = codes + r * (int64_t)k;
  int t = 0;
  for (int f = threadIdx.x; f < k / 4; f += kThreads) {
    const int w = *reinterpret_cast<const int *>(row + 4 * f);
    t += (int)(int8_t)(w & 0xff) + (int)(int8_t)((w >> 8) & 0xff) + (int)(int8_t)((w >> 16) & 0xff) + (w >> 24);
  }
  t = wave_sum(t);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    int s = 0;
    for (int w = 0; w < kThreads / 64; ++w) s += red[w];
    rowsum[r] = s;
  }
}

__global__ __launch_bounds__(kThreads) void add_kernel(const float4 *__restrict__ a, const float4 *__restrict__ b,
                                                       float4 *__restrict__ out, int64_t n4) {
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
    const float4 x = a[i], y = b[i];
    float4 o;
    o.x = __fadd_rn(x.x, y.x); o.y = __fadd_rn(x.y, y.y);
    o.z = __fadd_rn(x.z, y.z); o.w = __fadd_rn(x.w, y.w);
    out[i] = o;
  }
}

// y[m][j] = fl32(fl32(max(g, 0)^2) * u) from gu = [m][g (inter) | u (inter)]
__global__ __launch_bounds__(kThreads) void relu2_glu_kernel(const float *__restrict__ gu, int64_t m, int inter,
                                                             float *__restrict__ y) {
  const int q4 = inter / 4;
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < m * q4; i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / q4;
    const int c = (int)(i - r * q4);
    const float4 g = *reinterpret_cast<const float4 *>(gu + r * 2 * inter + 4 * c);
    const float4 u = *reinterpret_cast<const float4 *>(gu + r * 2 * inter + inter + 4 * c);
    float4 o;
    float t;
    t = g.x > 0.0f ? g.x : 0.0f; o.x = __fmul_rn(__fmul_rn(t, t), u.x);
    t = g.y > 0.0f ? g.y : 0.0f; o.y = __fmul_rn(__fmul_rn(t, t), u.y);
    t = g.z > 0.0f ? g.z : 0.0f; o.z = __fmul_rn(__fmul_rn(t, t), u.z);
    t = g.w > 0.0f ? g.w : 0.0f; o.w = __fmul_rn(__fmul_rn(t, t), u.w);
    *reinterpret_cast<float4 *>(y + r * inter + 4 * c) = o;
  }
}

}  // namespace

hipError_t launch_relu2_glu(const float *gu, int64_t m, int64_t inter, float *y, hipStream_t stream) {
  const int64_t n4 = m * (inter / 4);
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  relu2_glu_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(gu, m, (int)inter, y);
  return hipGetLastError();
}

hipError_t launch_quant_acts(int mode, const float *x, const float *x2, int64_t ld_x, int64_t m, int64_t k,
                             const float *gain, float eps, int gqa_offset, int head_dim, int group,
                             float *h_out, int8_t *codes, float *deq, int32_t *rowsum, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  Src s{x, x2, ld_x, (int)k, gain, gqa_offset, head_dim, group, h_out};
  switch (mode) {
    case BITLINEAR_ACT_ABSMAX: return launch_mode<BITLINEAR_ACT_ABSMAX>(s, m, codes, deq, rowsum, eps, stream);
    case BITLINEAR_ACT_RMSNORM: return launch_mode<BITLINEAR_ACT_RMSNORM>(s, m, codes, deq, rowsum, eps, stream);
    case BITLINEAR_ACT_RELU2_RMSNORM:
      return launch_mode<BITLINEAR_ACT_RELU2_RMSNORM>(s, m, codes, deq, rowsum, eps, stream);
    case ACT_RESID_RMSNORM: return launch_mode<ACT_RESID_RMSNORM>(s, m, codes, deq, rowsum, eps, stream);
    case ACT_GQA_RMSNORM: return launch_mode<ACT_GQA_RMSNORM>(s, m, codes, deq, rowsum, eps, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quant_acts_src(int mode, const ActSrc &src, int64_t m, float eps, int8_t *codes, float *deq,
                                 int32_t *rowsum, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  if (!src.part)
    return launch_quant_acts(mode, src.x, src.x2, src.ld, m, src.k, src.gain, eps, src.gqa_offset, src.head_dim,
                             src.group, src.h_out, codes, deq, rowsum, stream);
  switch (mode) {
    case BITLINEAR_ACT_RELU2_RMSNORM:
      return launch_mode<BITLINEAR_ACT_RELU2_RMSNORM, true>(src, m, codes, deq, rowsum, eps, stream);
    case ACT_RESID_RMSNORM: return launch_mode<ACT_RESID_RMSNORM, true>(src, m, codes, deq, rowsum, eps, stream);
    case ACT_GQA_RMSNORM: return launch_mode<ACT_GQA_RMSNORM, true>(src, m, codes, deq, rowsum, eps, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_code_rowsum(const int8_t *codes, int64_t m, int64_t k, int32_t *rowsum, hipStream_t stream) {
  if (m == 0) return hipSuccess;
  code_rowsum_kernel<<<dim3((unsigned)m), dim3(kThreads), 0, stream>>>(codes, (int)k, rowsum);
  return hipGetLastError();
}

hipError_t launch_add(const float *a, const float *b, float *out, int64_t count, hipStream_t stream) {
  const int64_t n4 = count / 4;
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  add_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(
      reinterpret_cast<const float4 *>(a), reinterpret_cast<const float4 *>(b), reinterpret_cast<float4 *>(out), n4);
  return hipGetLastError();
}

}  // namespace bl
