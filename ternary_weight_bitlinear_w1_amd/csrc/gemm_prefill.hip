// Prefill contraction: int8 activation codes x packed ternary weights -> fp32,
// on gfx950 int8 MFMA (v_mfma_i32_32x32x32_i8).
//
// What is computed (nnterp "BitNet b1.58" page, "The projections quantize
// their inputs and weights"; "The two checkpoints"; model card "Model
// Details": no bias):  y[m][n] = fl32(fl32((float)acc * deq[m]) * gamma(n)),
// acc = sum_k q[m][k] * c[n][k], exact in int32.
//
// Weights arrive as fields u = c + 1 (0..2); the kernel multiplies q by u and
// subtracts the code row sum sum_k q[m][k], which is exact integer arithmetic,
// so a 2-bit field becomes an MFMA byte with one shift and one AND.
//
// Tiling: a workgroup of WM x WN waves owns a BM x BN output tile
// (BM = 32 WM TM, BN = 32 WN TN); each wave owns TM x TN MFMA tiles of 32 x 32.
// Per K chunk of 128:
//   A (codes, BM x 128 bytes) is loaded global -> registers (prefetched one
//     chunk ahead) -> LDS (rows padded by 16 bytes against bank conflicts);
//     it is reused by the WN waves that share those rows.
//   B (packed, 32 bytes per output row per chunk) is loaded global ->
//     registers one chunk ahead and unpacked in registers: each lane's one
//     dword (16 weights) expands to exactly its 16-byte MFMA operand.
// MFMA operand convention (checked on gfx950): lane l supplies row l % 32 of
// A (column l % 32 of B) and the 16 k values of k-block l / 32; any k order is
// fine as long as A and B use the same one. Here lane l in k-step s (0..3) of
// a chunk takes k-block 4 (l / 32) + s, so its four B blocks are one 16-byte
// load and its four A blocks one 64-byte LDS row segment.
// Output: lane l, accumulator q holds row 8 (q / 4) + 4 (l / 32) + q % 4,
// column l % 32 of the 32 x 32 tile.
#include "common.h"

namespace bl {
namespace {

typedef int v4i_u __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kBK = 128;
constexpr int kLda = kBK + 16;
constexpr uint32_t kFieldMask = 0x03030303u;

__device__ __forceinline__ v4i unpack16(uint32_t p) {
  v4i b;
  b[0] = (int)(p & kFieldMask);
  b[1] = (int)((p >> 2) & kFieldMask);
  b[2] = (int)((p >> 4) & kFieldMask);
  b[3] = (int)((p >> 6) & kFieldMask);
  return b;
}

template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(WM *WN * 64) void gemm_prefill_kernel(const int8_t *__restrict__ A,
                                                                   const uint8_t *__restrict__ B,
                                                                   const float *__restrict__ deq,
                                                                   const int32_t *__restrict__ rowsum, int M, int N,
                                                                   int K, Epilogue ep, float *__restrict__ Y,
                                                                   int32_t *__restrict__ acc_out) {
  constexpr int kThreads = WM * WN * 64;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int kChunks = BM * (kBK / 16);  // 16-byte pieces of one A tile
  static_assert(kChunks % kThreads == 0, "A tile must split evenly");
  constexpr int kAPer = kChunks / kThreads;
  __shared__ __attribute__((aligned(16))) int8_t sA[BM * kLda];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_n = (N + BN - 1) / BN;
  const int bm = blockIdx.x / tiles_n, bn = blockIdx.x % tiles_n;
  const int m0 = bm * BM, n0 = bn * BN;
  const int G = K >> 4;            // 16-code groups per row
  const int64_t ldb = K >> 2;      // packed bytes per weight row
  const int nk = (K + kBK - 1) / kBK;
  const int half = lane >> 5, l32 = lane & 31;

  v4i areg[kAPer];
  v4i breg[TN];

  auto load_a = [&](int kc) {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int c = tid + i * kThreads;
      const int row = c >> 3, col = (c & 7) << 4;
      const int gm = m0 + row, gk = kc * kBK + col;
      if (gm < M && gk < K)
        areg[i] = *reinterpret_cast<const v4i *>(A + (int64_t)gm * K + gk);
      else
        areg[i] = v4i{0, 0, 0, 0};
    }
  };
  auto store_a = [&]() {
#pragma unroll
    for (int i = 0; i < kAPer; ++i) {
      const int c = tid + i * kThreads;
      const int row = c >> 3, col = (c & 7) << 4;
      *reinterpret_cast<v4i *>(sA + row * kLda + col) = areg[i];
    }
  };
  auto load_b = [&](int kc) {
    const int g0 = kc * 8 + 4 * half;  // first of this lane's four groups
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int n = n0 + (wn * TN + tn) * 32 + l32;
      v4i b = v4i{0, 0, 0, 0};
      if (n < N) {
        const uint8_t *p = B + (int64_t)n * ldb + 4 * (int64_t)g0;
        if (g0 + 4 <= G) {
          const v4i_u t = *reinterpret_cast<const v4i_u *>(p);
          b = v4i{t[0], t[1], t[2], t[3]};
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (g0 + t < G) b[t] = reinterpret_cast<const int *>(p)[t];
        }
      }
      breg[tn] = b;
    }
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0;

  load_a(0);
  load_b(0);
  for (int kc = 0; kc < nk; ++kc) {
    store_a();
    v4i bcur[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) bcur[tn] = breg[tn];
    __syncthreads();
    if (kc + 1 < nk) {
      load_a(kc + 1);
      load_b(kc + 1);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i bop[TN];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) bop[tn] = unpack16((uint32_t)bcur[tn][s]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int row = (wm * TM + tm) * 32 + l32;
        const v4i a = *reinterpret_cast<const v4i *>(sA + row * kLda + 64 * half + 16 * s);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bop[tn], acc[tm][tn], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- epilogue: undo the field offset, rescale, store
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int n = n0 + (wn * TN + tn) * 32 + l32;
    if (n >= N) continue;
    const float g = epi_gamma(ep, n);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = m0 + (wm * TM + tm) * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
        if (m < M) {
          const int a = acc[tm][tn][q] - rowsum[m];
          const int64_t o = (int64_t)m * N + n;
          if (acc_out) acc_out[o] = a;
          Y[o] = rescale(a, deq[m], g);
        }
      }
    }
  }
}

template <int WM, int WN, int TM, int TN>
hipError_t launch_cfg(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum, int m,
                      int n, int k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const int64_t tiles = (int64_t)((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  gemm_prefill_kernel<WM, WN, TM, TN>
      <<<dim3((unsigned)tiles), dim3(WM * WN * 64), 0, stream>>>(codes, packed, deq, rowsum, m, n, k, ep, y, acc_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_prefill(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum,
                               int64_t m, int64_t n, int64_t k, const Epilogue &ep, float *y, int32_t *acc_out,
                               hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (m >= 256)
    return launch_cfg<2, 2, 4, 2>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
  if (m > 64)
    return launch_cfg<2, 2, 2, 2>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
  return launch_cfg<1, 4, 2, 1>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
}

}  // namespace bl
