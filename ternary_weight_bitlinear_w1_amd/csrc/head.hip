// The model's head: the final RMSNorm, rounded to bfloat16, then the bfloat16
// lm_head (2560 -> 128256, no bias), for 1 to 4 tokens per launch.
//
// What is computed ([nnterp] "Printout": (norm) RMSNorm over the hidden size,
// eps 1e-5, then lm_head = Linear(2560, 128256, bias=False); "Config": dtype
// bfloat16, the head tied to the embedding table; the order of the norm's
// steps in an fp32 stream is reading R20):
//   ms = sum_k x_k^2 / K (fp64);  r = fl32(1 / sqrt(ms + eps));
//   o_k = bf16(fl32(g_k * fl32(x_k * r)));   logits[n] = sum_k o_k w[n][k] (fp32).
//
// final_norm_kernel: one workgroup per token; the fp64 sum of squares is
// reduced in a fixed order, so o repeats run to run.
//
// lm_head_kernel: bound by HBM on the head (656.7 MB at 128256 x 2560). A wave
// owns R rows (2, 2, 4, 8 for one to four tokens, measured); for each it issues C
// loads of 1 KB (64 lanes x 16 bytes, 8
// bfloat16 each), so lane l always reads the same columns 512 c + 8 l .. + 7 and
// keeps the tokens' o for exactly those columns in registers for the whole
// kernel. Products use v_dot2_f32_bf16 (exact bfloat16 products, fp32 sums);
// the 64 lane partials of a row are added with DPP adds within rows of 16
// lanes and permlane swaps across them.
#include "common.h"

namespace bl {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kNormThreads = 256;
constexpr int kHeadMaxChunks = 8;  // K <= 8 * 512

// nearest bfloat16 of a finite float, ties to an even last kept bit
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t kept = u >> 16, dropped = u & 0xFFFFu;
  return kept + ((dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) ? 1u : 0u);
}

constexpr int kNormPer = 512 * kHeadMaxChunks / kNormThreads;  // values per thread at the largest K

// (every load of the row and the gain is issued before the sum)
__global__ __launch_bounds__(kNormThreads) void final_norm_kernel(const float *__restrict__ x, int K,
                                                                  const float *__restrict__ gain, float eps,
                                                                  uint16_t *__restrict__ o) {
  __shared__ double red[kNormThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *xr = x + (int64_t)blockIdx.x * K;
  float xv[kNormPer], gv[kNormPer];
#pragma unroll
  for (int i = 0; i < kNormPer; ++i) {
    const int k = tid + kNormThreads * i;
    xv[i] = k < K ? xr[k] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < kNormPer; ++i) {
    const int k = tid + kNormThreads * i;
    gv[i] = gain && k < K ? gain[k] : 1.0f;
  }
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < kNormPer; ++i)
    if (tid + kNormThreads * i < K) ss += (double)xv[i] * (double)xv[i];
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) ss += __shfl_xor(ss, s, 64);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  double tot = red[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / 64; ++w) tot += red[w];
  const float r = (float)(1.0 / sqrt(tot / (double)K + (double)eps));
  uint16_t *orow = o + (int64_t)blockIdx.x * K;
#pragma unroll
  for (int i = 0; i < kNormPer; ++i) {
    const int k = tid + kNormThreads * i;
    if (k < K) {
      const float v = __fmul_rn(xv[i], r);
      const float g = gain ? __fmul_rn(gv[i], v) : v;
      orow[k] = (uint16_t)bf16_bits(g);
    }
  }
}

// rows per wave, by tokens: the fastest of 2, 4 and 8 on the 2B4T head
// (one and two tokens 107.0 and 107.5 us with 2 rows; three 108.7 us with 4;
// four 113.3 us with 8, against 117.3 with 4)
template <int MT>
constexpr int head_rows_per_wave() {
  return MT <= 2 ? 2 : (MT == 3 ? 4 : 8);
}

template <int MT, int C>
__global__ __launch_bounds__(256) void lm_head_kernel(const uint16_t *__restrict__ o, const uint16_t *__restrict__ W,
                                                      int N, int K, float *__restrict__ Y) {
  constexpr int kHeadRowsPerWave = head_rows_per_wave<MT>();
  static_assert(kHeadRowsPerWave * MT <= 64, "one lane per output of the wave");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 4 + wave) * kHeadRowsPerWave;
  // the weights first (HBM), then the tokens' o (a few KB from L2)
  v4i w[kHeadRowsPerWave][C];
#pragma unroll
  for (int r = 0; r < kHeadRowsPerWave; ++r)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int k0 = 512 * c + 8 * lane;
      const bool use = n0 + r < N && k0 < K;
      // past the end, reload finite values (the first o), which meet a zero o
      w[r][c] = *reinterpret_cast<const v4i *>(use ? W + (int64_t)(n0 + r) * K + k0 : o);
    }
  v4i xo[MT][C];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int k0 = 512 * c + 8 * lane;
      xo[t][c] = k0 < K ? *reinterpret_cast<const v4i *>(o + (int64_t)t * K + k0) : v4i{0, 0, 0, 0};
    }
  float acc[kHeadRowsPerWave][MT];
#pragma unroll
  for (int r = 0; r < kHeadRowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      float a = 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // (bit casts take values: a vector element lvalue is copied out first)
          const int wv = w[r][c][q], xv = xo[t][c][q];
          a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wv), __builtin_bit_cast(bf16x2, xv), a,
                                              false);
        }
      }
      acc[r][t] = a;
    }
#pragma unroll
  for (int r = 0; r < kHeadRowsPerWave; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      acc[r][t] = rows_sum(row16_sum(acc[r][t]));
    }
  if (lane < kHeadRowsPerWave * MT) {
    const int r = lane / MT, t = lane - r * MT;
    float v = 0.0f;
#pragma unroll
    for (int rr = 0; rr < kHeadRowsPerWave; ++rr)
#pragma unroll
      for (int tt = 0; tt < MT; ++tt)
        if (rr == r && tt == t) v = acc[rr][tt];
    if (n0 + r < N) Y[(int64_t)t * N + n0 + r] = v;
  }
}

// x[t] = the table row of token ids[t], widened to fp32 (exact); an id outside
// [0, vocab) gives a zero row. Each thread moves 8 values (16 bytes) per piece,
// all pieces loaded before any is stored.
constexpr int kEmbedPieces = 512 * kHeadMaxChunks / (256 * 8);
__global__ __launch_bounds__(256) void embed_kernel(const int64_t *__restrict__ ids, const uint16_t *__restrict__ table,
                                                    int64_t vocab, int K, float *__restrict__ x) {
  const int64_t id = ids[blockIdx.x];
  const bool ok = id >= 0 && id < vocab;
  float *xr = x + (int64_t)blockIdx.x * K;
  v4i w[kEmbedPieces];
#pragma unroll
  for (int i = 0; i < kEmbedPieces; ++i) {
    const int k = 8 * (threadIdx.x + 256 * i);
    w[i] = ok && k < K ? *reinterpret_cast<const v4i *>(table + id * K + k) : v4i{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < kEmbedPieces; ++i) {
    const int k = 8 * (threadIdx.x + 256 * i);
    if (k < K) {
      const uint32_t w0 = (uint32_t)w[i][0], w1 = (uint32_t)w[i][1];
      const uint32_t w2 = (uint32_t)w[i][2], w3 = (uint32_t)w[i][3];
      *reinterpret_cast<float4 *>(xr + k) =
          make_float4(__uint_as_float(w0 << 16), __uint_as_float(w0 & 0xFFFF0000u), __uint_as_float(w1 << 16),
                      __uint_as_float(w1 & 0xFFFF0000u));
      *reinterpret_cast<float4 *>(xr + k + 4) =
          make_float4(__uint_as_float(w2 << 16), __uint_as_float(w2 & 0xFFFF0000u), __uint_as_float(w3 << 16),
                      __uint_as_float(w3 & 0xFFFF0000u));
    }
  }
}

template <int MT>
hipError_t launch_head_mt(const uint16_t *o, const uint16_t *w, int n, int k, float *y, hipStream_t stream) {
  constexpr int kHeadRowsPerWave = head_rows_per_wave<MT>();
  const int chunks = (k + 511) / 512;
  const dim3 grid((unsigned)((n + 4 * kHeadRowsPerWave - 1) / (4 * kHeadRowsPerWave))), block(256);
#define BL_HEAD(C_) \
  lm_head_kernel<MT, C_><<<grid, block, 0, stream>>>(o, w, n, k, y); \
  return hipGetLastError()
  if (chunks <= 2) { BL_HEAD(2); }
  if (chunks <= 4) { BL_HEAD(4); }
  if (chunks <= 5) { BL_HEAD(5); }
  BL_HEAD(8);
#undef BL_HEAD
}

}  // namespace

bool lm_head_supported(int64_t k) { return k > 0 && k % 8 == 0 && k <= 512 * kHeadMaxChunks; }

hipError_t launch_final_norm(const float *x, int64_t m, int64_t k, const float *gain, float eps, uint16_t *o,
                             hipStream_t stream) {
  if (m == 0) return hipSuccess;
  final_norm_kernel<<<dim3((unsigned)m), dim3(kNormThreads), 0, stream>>>(x, (int)k, gain, eps, o);
  return hipGetLastError();
}

hipError_t launch_embed(const int64_t *ids, int64_t m, const uint16_t *table, int64_t vocab, int64_t k, float *x,
                        hipStream_t stream) {
  if (m == 0) return hipSuccess;
  embed_kernel<<<dim3((unsigned)m), dim3(256), 0, stream>>>(ids, table, vocab, (int)k, x);
  return hipGetLastError();
}

// logits [m][n] of o [m][k]; tokens go four to a launch
hipError_t launch_lm_head(const uint16_t *o, int64_t m, int64_t k, const uint16_t *w, int64_t n, float *y,
                          hipStream_t stream) {
  if (!lm_head_supported(k)) return hipErrorInvalidValue;
  for (int64_t t0 = 0; t0 < m; t0 += 4) {
    const int mt = (int)(m - t0 < 4 ? m - t0 : 4);
    const uint16_t *ot = o + t0 * k;
    float *yt = y + t0 * n;
    hipError_t e;
    switch (mt) {
      case 1: e = launch_head_mt<1>(ot, w, (int)n, (int)k, yt, stream); break;
      case 2: e = launch_head_mt<2>(ot, w, (int)n, (int)k, yt, stream); break;
      case 3: e = launch_head_mt<3>(ot, w, (int)n, (int)k, yt, stream); break;
      default: e = launch_head_mt<4>(ot, w, (int)n, (int)k, yt, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bl
