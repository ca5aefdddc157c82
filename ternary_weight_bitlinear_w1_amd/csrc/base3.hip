// Five ternary codes per byte (base 3): the repacking kernel and the
// few-token contraction that reads that storage.
//
// Storage ([tiny] "O que é" and "Arquivos": the ternary checkpoint also ships
// in a format denser than two bits per weight; the pages give no layout, so
// this one is the library's own): row n of K codes takes RB = 16 ceil(K / 80)
// bytes, 1.6 bits per weight. Code k is digit k % 5 of byte k / 5, stored as
// u = c + 1: byte j = sum_i u(5j + i) 3^i. Codes past K are 0 (digit 1), so a
// valid byte is at most 242; bytes 243 .. 255 read as five zero codes.
//
// Contraction (gemv_b3_kernel, m <= 4 tokens, K % 16 == 0, K <= 8192): the
// shape of the one-token dot-product kernel (8 lanes per weight row, 16 bytes
// = 80 codes per lane and load, 128 contiguous bytes per row and wave load,
// K split over up to four waves), with the decode of a byte by table lookup.
// Table j (j = 0 .. 3, the byte's place in its dword) maps a byte to 8 bytes:
// its digits 0..3 as signed codes in the low dword, and digit 4 as a signed
// code in byte j of the high dword (zeros elsewhere), so the four high dwords
// of a weight dword OR together into one dword of codes. The token's codes are
// stored in LDS in the matching order: per 20 codes (one weight dword),
// [q0..q3][q5..q8][q10..q13][q15..q18][q4 q9 q14 q19]. A weight dword (20
// weights) then takes four table reads, two ORs and five v_dot4 per token.
// The codes are signed, so acc = sum q c directly (no row-sum correction).
#include "common.h"

namespace bl {
namespace {

constexpr int kB3MaxK = 8192;
constexpr int kB3MaxKP = 80 * ((kB3MaxK + 79) / 80);  // padded codes per token in LDS

__device__ __forceinline__ int b3_row_bytes(int k) { return 16 * ((k + 79) / 80); }


// One output dword (four base-3 bytes) per thread, from the two-bit layout
// (code k of a row: field u = c + 1 in byte 4 (k / 16) + k % 4, bits
// 2 ((k % 16) / 4)). A field of 3 (not a code) is taken as code 0.
__global__ __launch_bounds__(256) void pack_base3_kernel(const uint8_t *__restrict__ P, int N, int K,
                                                         uint8_t *__restrict__ Q) {
  const int rb = b3_row_bytes(K), words = rb / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)N * words) return;
  const int r = (int)(i / words), w = (int)(i - (int64_t)r * words);
  const uint8_t *row = P + (int64_t)r * (K / 4);
  uint32_t out = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    int byte = 0, pw = 1;
#pragma unroll
    for (int d = 0; d < 5; ++d) {
      const int k = 5 * (4 * w + b) + d;
      int u = 1;
      if (k < K) {
        u = (row[4 * (k >> 4) + (k & 3)] >> (2 * ((k & 15) >> 2))) & 3;
        if (u == 3) u = 1;
      }
      byte += u * pw;
      pw *= 3;
    }
    out |= (uint32_t)byte << (8 * b);
  }
  reinterpret_cast<uint32_t *>(Q + (int64_t)r * rb)[w] = out;
}

// Five code dwords of one group of 20 codes (i0..i4 = codes 0..3, 4..7, ...,
// 16..19) in the order the tables expect.
__device__ __forceinline__ void permute20(const uint32_t *i, uint32_t *o) {
  o[0] = i[0];                                    // q0  q1  q2  q3
  o[1] = (i[1] >> 8) | (i[2] << 24);              // q5  q6  q7  q8
  o[2] = (i[2] >> 16) | (i[3] << 16);             // q10 q11 q12 q13
  o[3] = (i[3] >> 24) | (i[4] << 8);              // q15 q16 q17 q18
  o[4] = (i[1] & 0xFFu) | (i[2] & 0xFF00u) | (i[3] & 0xFF0000u) | (i[4] & 0xFF000000u);  // q4 q9 q14 q19
}

template <int MT, int KS, int LPW>
__global__ __launch_bounds__(256) void gemv_b3_kernel(const int8_t *__restrict__ A, const uint8_t *__restrict__ B,
                                                      const float *__restrict__ deq, int N, int K, Epilogue ep_in,
                                                      float *__restrict__ Y, int32_t *__restrict__ acc_out) {
  const Epilogue ep = resolve_gamma(ep_in);
  constexpr int RG = 4 / KS;  // row groups of 8 rows per workgroup
  __shared__ __attribute__((aligned(16))) int8_t sc[MT * kB3MaxKP];
  __shared__ __attribute__((aligned(16))) uint2 lut[4 * 256];
  __shared__ int red[KS][RG][8][MT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = wave % KS, rg = wave / KS;
  const int n = blockIdx.x * 8 * RG + rg * 8 + (lane >> 3);
  const int p = lane & 7;
  const int rb = b3_row_bytes(K);  // bytes per weight row (multiple of 16)
  const int blk = rb / 16;         // 80-code blocks per token
  const int L = (rb + 127) >> 7;   // 128-byte lines per row, the last may be partial
  const int l_lo = L * ks / KS, l_hi = L * (ks + 1) / KS;

  // Loads in issue order: the token codes (a few KB from L2), then the
  // weights (from HBM). Loads complete in issue order, so the codes are ready
  // first. Every lane issues the same number of loads (out-of-range pieces
  // reload a valid address and are replaced by zeros).
  constexpr int kBlocks = (MT * (kB3MaxKP / 80) + 255) / 256;  // 80-code blocks per thread
  const int nblk = MT * blk;
  v4i cw[kBlocks][5];
#pragma unroll
  for (int j = 0; j < kBlocks; ++j) {
    const int i = tid + 256 * j;
    const int t = i / blk, c = i - t * blk;
#pragma unroll
    for (int e = 0; e < 5; ++e) {
      const int k0 = 80 * c + 16 * e;
      cw[j][e] = *reinterpret_cast<const v4i *>(i < nblk && k0 < K ? A + (int64_t)t * K + k0 : A);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  v4i w[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int off = 128 * (l_lo + i) + 16 * p;
    const bool use = l_lo + i < l_hi && off < rb && n < N;
    w[i] = *reinterpret_cast<const v4i *>(use ? B + (int64_t)n * rb + off : B);
  }
  __builtin_amdgcn_sched_barrier(0);

  // the decode tables (ALU work while the loads are in flight; loading a
  // precomputed 8 KB table instead measured slower)
  for (int e = tid; e < 4 * 256; e += 256) {
    const int j = e >> 8, v = e & 255;
    uint32_t lo = 0, hi = 0;
    if (v < 243) {
      int x = v;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        lo |= (uint32_t)((x % 3 - 1) & 0xFF) << (8 * d);
        x /= 3;
      }
      hi = (uint32_t)((x % 3 - 1) & 0xFF) << (8 * j);
    }
    lut[e] = make_uint2(lo, hi);
  }
  // the token codes, permuted per 20 codes
#pragma unroll
  for (int j = 0; j < kBlocks; ++j) {
    const int i = tid + 256 * j;
    if (i < nblk) {
      const int t = i / blk, c = i - t * blk;
      uint32_t in[20], out[20];
#pragma unroll
      for (int e = 0; e < 5; ++e) {
        const bool valid = 80 * c + 16 * e < K;
#pragma unroll
        for (int q = 0; q < 4; ++q) in[4 * e + q] = valid ? (uint32_t)cw[j][e][q] : 0u;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) permute20(in + 5 * g, out + 5 * g);
      v4i *dst = reinterpret_cast<v4i *>(sc + t * kB3MaxKP + 80 * c);
#pragma unroll
      for (int e = 0; e < 5; ++e)
        dst[e] = v4i{(int)out[4 * e], (int)out[4 * e + 1], (int)out[4 * e + 2], (int)out[4 * e + 3]};
    }
  }
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS stores are done
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  float dq[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) dq[t] = deq[t];

  int acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = 0;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int piece = 8 * (l_lo + i) + p;  // 16-byte piece of the row: codes 80 piece ..
    if (l_lo + i < l_hi && 16 * piece < rb) {
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t wd = (uint32_t)w[i][d];
        uint32_t lo[4], hi = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint2 e = lut[(j << 8) | ((wd >> (8 * j)) & 0xFFu)];
          lo[j] = e.x;
          hi |= e.y;
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          const int *cp = reinterpret_cast<const int *>(sc + t * kB3MaxKP + 80 * piece + 20 * d);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[t] = __builtin_amdgcn_sdot4((int)lo[j], cp[j], acc[t], false);
          acc[t] = __builtin_amdgcn_sdot4((int)hi, cp[4], acc[t], false);
        }
      }
    }
  }
  // 8 lanes per row
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    acc[t] = lanes8_sum(acc[t]);
  }
  if (p == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) red[ks][rg][lane >> 3][t] = acc[t];
  }
  __syncthreads();
  if (ks == 0 && p == 0 && n < N) {
    const float g = epi_gamma(ep, n);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      int sum = 0;
#pragma unroll
      for (int q = 0; q < KS; ++q) sum += red[q][rg][lane >> 3][t];
      const int64_t o = (int64_t)t * N + n;
      if (acc_out) acc_out[o] = sum;
      Y[o] = rescale(sum, dq[t], g);
    }
  }
}

template <int MT>
hipError_t launch_b3_mt(const int8_t *codes, const uint8_t *w, const float *deq, int n, int k, const Epilogue &ep,
                        float *y, int32_t *acc_out, hipStream_t stream) {
  const int lines = (16 * ((k + 79) / 80) + 127) >> 7;
  // split K over the waves of a workgroup until the workgroups cover the CUs
  const int ks = n / 32 >= 256 ? 1 : (n / 16 >= 256 ? 2 : 4);
  const int lpw = (lines + ks - 1) / ks;
  const int rows_per_wg = 8 * (4 / ks);
  const dim3 grid((unsigned)((n + rows_per_wg - 1) / rows_per_wg)), block(256);
#define BL_B3(KS_, LPW_)                                                                              \
  gemv_b3_kernel<MT, KS_, LPW_><<<grid, block, 0, stream>>>(codes, w, deq, n, k, ep, y, acc_out); \
  return hipGetLastError()
  if (ks == 1) {
    if (lpw <= 4) { BL_B3(1, 4); }
    if (lpw <= 8) { BL_B3(1, 8); }
    BL_B3(1, 16);
  }
  if (ks == 2) {
    if (lpw <= 4) { BL_B3(2, 4); }
    if (lpw <= 8) { BL_B3(2, 8); }
    BL_B3(2, 16);
  }
  if (lpw <= 4) { BL_B3(4, 4); }
  if (lpw <= 8) { BL_B3(4, 8); }
  BL_B3(4, 16);
#undef BL_B3
}

}  // namespace

bool gemv_b3_supported(int64_t m, int64_t k) { return m >= 1 && m <= 4 && k % 16 == 0 && k > 0 && k <= kB3MaxK; }

hipError_t launch_pack_base3(const uint8_t *packed, int64_t n, int64_t k, uint8_t *out, hipStream_t stream) {
  const int64_t words = n * (16 * ((k + 79) / 80) / 4);
  if (words == 0) return hipSuccess;
  pack_base3_kernel<<<dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream>>>(packed, (int)n, (int)k, out);
  return hipGetLastError();
}

hipError_t launch_gemv_b3(const int8_t *codes, const uint8_t *w, const float *deq, int64_t m, int64_t n, int64_t k,
                          const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (!gemv_b3_supported(m, k)) return hipErrorInvalidValue;
  switch (m) {
    case 1: return launch_b3_mt<1>(codes, w, deq, (int)n, (int)k, ep, y, acc_out, stream);
    case 2: return launch_b3_mt<2>(codes, w, deq, (int)n, (int)k, ep, y, acc_out, stream);
    case 3: return launch_b3_mt<3>(codes, w, deq, (int)n, (int)k, ep, y, acc_out, stream);
    default: return launch_b3_mt<4>(codes, w, deq, (int)n, (int)k, ep, y, acc_out, stream);
  }
}

}  // namespace bl
