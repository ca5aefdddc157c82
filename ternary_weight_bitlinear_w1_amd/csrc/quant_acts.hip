// Per-token int8 quantization of fp32 activations, with the fused prologues
// of a BitNet b1.58 block (gfx950).
//
// Codes: round(v * 127 / max|v|), half to even, in [-127, 127]; deq = max|v| / 127
// (nnterp "BitNet b1.58" page, "The projections quantize their inputs and
// weights"; model card "Model Details": 8-bit absmax per token).
// RMSNorm prologues ("The block, in order"; eps from "Config") keep the codes
// of v = g * pre and move 1 / sqrt(mean(pre^2) + eps) into deq, since a positive
// per-token factor cancels inside the rounding ("Scaling inside a sublayer is
// undone by the sub-norm"). The squared-ReLU prologue forms
// (max(gate, 0)^2) * up ("The MLP gates with a squared ReLU").
//
// One workgroup of 256 threads per token row. Pass 1 forms the normed input
// v (kept in registers when the row fits, NV float4 per thread), the fp32 max
// |v| and the fp64 sum of squares; both are reduced wave-wise then across the
// four waves in a fixed order. Pass 2 writes the codes (one 32-bit store per
// four codes) and their row sum, which the contraction kernels use to undo the
// offset of the stored weight fields (u = c + 1).
// HBM-bound: 4 (or 8 for gate|up, 8 for the residual pair) bytes read and
// 1 byte written per element.
#include "common.h"

namespace bl {
namespace {

constexpr int kThreads = 256;

struct Src {
  const float *x;   // row-major source, row stride ld
  const float *x2;  // second operand (residual mode)
  int64_t ld;
  int k;
  const float *gain;
  int gqa_offset, head_dim, group;
  float *h_out;     // residual mode: the sum is also written here ([m][k])
};

// pre-norm input for elements 4f .. 4f+3 of row r
template <int MODE>
__device__ __forceinline__ float4 load_pre(const Src &s, int64_t r, int f, bool write_h) {
  if constexpr (MODE == BITLINEAR_ACT_RELU2_RMSNORM) {
    const float4 g = *reinterpret_cast<const float4 *>(s.x + r * s.ld + 4 * f);
    const float4 u = *reinterpret_cast<const float4 *>(s.x + r * s.ld + s.k + 4 * f);
    float4 o;
    float t;
    t = g.x > 0.0f ? g.x : 0.0f; o.x = __fmul_rn(__fmul_rn(t, t), u.x);
    t = g.y > 0.0f ? g.y : 0.0f; o.y = __fmul_rn(__fmul_rn(t, t), u.y);
    t = g.z > 0.0f ? g.z : 0.0f; o.z = __fmul_rn(__fmul_rn(t, t), u.z);
    t = g.w > 0.0f ? g.w : 0.0f; o.w = __fmul_rn(__fmul_rn(t, t), u.w);
    return o;
  } else if constexpr (MODE == ACT_RESID_RMSNORM) {
    const float4 a = *reinterpret_cast<const float4 *>(s.x + r * s.ld + 4 * f);
    const float4 b = *reinterpret_cast<const float4 *>(s.x2 + r * s.ld + 4 * f);
    float4 o;
    o.x = __fadd_rn(a.x, b.x); o.y = __fadd_rn(a.y, b.y);
    o.z = __fadd_rn(a.z, b.z); o.w = __fadd_rn(a.w, b.w);
    if (write_h) *reinterpret_cast<float4 *>(s.h_out + r * (int64_t)s.k + 4 * f) = o;
    return o;
  } else if constexpr (MODE == ACT_GQA_RMSNORM) {
    // element e of the attention output reads value head (e / head_dim) / group
    const int e = 4 * f;
    const int head = e / s.head_dim, d = e - head * s.head_dim;
    return *reinterpret_cast<const float4 *>(s.x + r * s.ld + s.gqa_offset + (head / s.group) * s.head_dim + d);
  } else {
    return *reinterpret_cast<const float4 *>(s.x + r * s.ld + 4 * f);
  }
}

template <int MODE>
__device__ __forceinline__ float4 apply_gain(const Src &s, int f, float4 p) {
  if (MODE != BITLINEAR_ACT_ABSMAX && s.gain != nullptr) {
    const float4 g = *reinterpret_cast<const float4 *>(s.gain + 4 * f);
    p.x = __fmul_rn(g.x, p.x); p.y = __fmul_rn(g.y, p.y);
    p.z = __fmul_rn(g.z, p.z); p.w = __fmul_rn(g.w, p.w);
  }
  return p;
}

__device__ __forceinline__ int code_of(float v, float pre, float s) {
  float p = __fmul_rn(__fmul_rn(v, pre), s);
  float r = __builtin_rintf(p);
  r = r > 127.0f ? 127.0f : r;
  r = r < -127.0f ? -127.0f : r;
  return (int)r;
}

template <int MODE, int NV>
__global__ __launch_bounds__(kThreads) void quant_acts_kernel(Src s, int8_t *__restrict__ codes,
                                                              float *__restrict__ deq, int32_t *__restrict__ rowsum,
                                                              float eps) {
  constexpr bool kRms = MODE != BITLINEAR_ACT_ABSMAX;
  __shared__ float red_f[kThreads / 64];
  __shared__ double red_d[kThreads / 64];
  __shared__ int red_i[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r = blockIdx.x;
  const int nf = s.k >> 2;  // float4 per row

  float4 cache[NV > 0 ? NV : 1];
  float amax = 0.0f;
  double ss = 0.0;
  // ---- pass 1: normed input, max |v|, sum of squares of the pre-gain input
  auto visit1 = [&](int f) -> float4 {
    const float4 p = load_pre<MODE>(s, r, f, true);
    if (kRms) {
      ss += (double)p.x * (double)p.x;
      ss += (double)p.y * (double)p.y;
      ss += (double)p.z * (double)p.z;
      ss += (double)p.w * (double)p.w;
    }
    const float4 v = apply_gain<MODE>(s, f, p);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    return v;
  };
  if constexpr (NV > 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int f = tid + j * kThreads;
      if (f < nf) cache[j] = visit1(f);
    }
  } else {
    for (int f = tid; f < nf; f += kThreads) (void)visit1(f);
  }
  amax = wave_max(amax);
  if (kRms) ss = wave_sum(ss);
  if (lane == 0) {
    red_f[wave] = amax;
    red_d[wave] = ss;
  }
  __syncthreads();
  float a = red_f[0];
  double sum_sq = red_d[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) {
    a = fmaxf(a, red_f[w]);
    sum_sq += red_d[w];
  }

  // ---- pass 2: codes
  int rs = 0;
  int8_t *crow = codes + r * (int64_t)s.k;
  if (a == 0.0f) {
    for (int f = tid; f < nf; f += kThreads) *reinterpret_cast<int *>(crow + 4 * f) = 0;
  } else {
    // rows whose max is below 2^-64 are scaled by 2^64 first (exact), which
    // keeps 127 / a finite and changes no code the unscaled steps reach
    const float pre = a < 0x1p-64f ? 0x1p64f : 1.0f;
    const float sc = 127.0f / __fmul_rn(a, pre);
    auto emit = [&](int f, float4 v) {
      const int q0 = code_of(v.x, pre, sc), q1 = code_of(v.y, pre, sc);
      const int q2 = code_of(v.z, pre, sc), q3 = code_of(v.w, pre, sc);
      rs += q0 + q1 + q2 + q3;
      *reinterpret_cast<int *>(crow + 4 * f) =
          (q0 & 0xff) | ((q1 & 0xff) << 8) | ((q2 & 0xff) << 16) | ((int)((unsigned)(q3 & 0xff) << 24));
    };
    if constexpr (NV > 0) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int f = tid + j * kThreads;
        if (f < nf) emit(f, cache[j]);
      }
    } else {
      for (int f = tid; f < nf; f += kThreads) emit(f, apply_gain<MODE>(s, f, load_pre<MODE>(s, r, f, false)));
    }
  }
  rs = wave_sum(rs);
  if (lane == 0) red_i[wave] = rs;
  __syncthreads();
  if (tid == 0) {
    int t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t += red_i[w];
    if (rowsum) rowsum[r] = t;
    float d = 0.0f;
    if (a != 0.0f) {
      if (kRms) {
        const double ms = sum_sq / (double)s.k;
        const double rr = sqrt(ms + (double)eps);
        d = (float)(((double)a / 127.0) / rr);
      } else {
        d = a / 127.0f;
      }
    }
    deq[r] = d;
  }
}

template <int MODE>
hipError_t launch_mode(const Src &s, int64_t m, int8_t *codes, float *deq, int32_t *rowsum, float eps,
                       hipStream_t stream) {
  const int per_thread = (s.k / 4 + kThreads - 1) / kThreads;
  dim3 grid((unsigned)m), block(kThreads);
  if (per_thread <= 1)
    quant_acts_kernel<MODE, 1><<<grid, block, 0, stream>>>(s, codes, deq, rowsum, eps);
  else if (per_thread <= 2)
    quant_acts_kernel<MODE, 2><<<grid, block, 0, stream>>>(s, codes, deq, rowsum, eps);
  else if (per_thread <= 4)
    quant_acts_kernel<MODE, 4><<<grid, block, 0, stream>>>(s, codes, deq, rowsum, eps);
  else if (per_thread <= 8)
    quant_acts_kernel<MODE, 8><<<grid, block, 0, stream>>>(s, codes, deq, rowsum, eps);
  else
    quant_acts_kernel<MODE, 0><<<grid, block, 0, stream>>>(s, codes, deq, rowsum, eps);
  return hipGetLastError();
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

}  // namespace

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
