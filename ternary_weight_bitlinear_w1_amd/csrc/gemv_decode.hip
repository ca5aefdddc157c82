// Decode contraction (m <= 16 tokens): stream the packed ternary weights once
// from HBM and contract them with the int8 codes on gfx950 int8 MFMA
// (v_mfma_i32_16x16x64_i8). Same result as the prefill kernel:
// y[m][n] = fl32(fl32((float)acc * deq[m]) * gamma(n)), acc exact in int32
// (nnterp "BitNet b1.58" page, "The projections quantize their inputs and
// weights" and "The two checkpoints"; no bias: model card "Model Details").
//
// This path is bound by HBM bandwidth on the packed weights (n * k / 4 bytes);
// the codes (m * k bytes) stay in L2.
//
// A workgroup of NW waves owns RT tiles of 16 output rows and splits K into NW
// contiguous slices, one per wave. A "superstep" is 256 k: lane l loads one
// 16-byte piece of row (l % 16) of the tile, covering k-blocks 4 (l / 16) .. +3,
// so the 4 lanes of a row read 64 contiguous bytes and a wave-wide load moves
// 16 rows x 64 bytes. Each packed dword (16 weights) unpacks with one shift and
// one AND per 4 weights into exactly the lane's 16-byte MFMA operand; MFMA t of
// the superstep uses dword t. MFMA operand convention (checked on gfx950):
// lane l supplies row l % 16 of A and column l % 16 of B, both for k-block
// l / 16; output lane l, register r holds row 4 (l / 16) + r, column l % 16.
// Here A rows are tokens (rows >= m are zero) and B columns are output rows.
// The NW partial tiles are added in LDS (exact integer sums), then the field
// offset is removed (acc = sum q u - sum q) and the rescale is fused.
#include "common.h"

namespace bl {
namespace {

typedef int v4i_u __attribute__((ext_vector_type(4), aligned(4)));
constexpr uint32_t kFieldMask = 0x03030303u;

// Launch shape (tuned on MI355X; overridable when building variants to sweep).
#ifndef BL_GEMV_MIN_WAVES
#define BL_GEMV_MIN_WAVES 4
#endif
#ifndef BL_GEMV_RT1_MAX_M
#define BL_GEMV_RT1_MAX_M 4
#endif

__device__ __forceinline__ v4i unpack16(uint32_t p) {
  v4i b;
  b[0] = (int)(p & kFieldMask);
  b[1] = (int)((p >> 2) & kFieldMask);
  b[2] = (int)((p >> 4) & kFieldMask);
  b[3] = (int)((p >> 6) & kFieldMask);
  return b;
}

// Weight-streaming kernel: wave w of the workgroup takes supersteps
// [S w / NW, S (w + 1) / NW) (at most SPW of them) and issues every load of its
// slice before its first MFMA, so a wave waits for memory once, not once per
// superstep.
template <int RT, int NW, int SPW>
__global__ __launch_bounds__(NW * 64) void gemv_decode_kernel(const int8_t *__restrict__ A,
                                                              const uint8_t *__restrict__ B,
                                                              const float *__restrict__ deq,
                                                              const int32_t *__restrict__ rowsum, int M, int N, int K,
                                                              Epilogue ep, float *__restrict__ Y,
                                                              int32_t *__restrict__ acc_out) {
  __shared__ int red[NW][RT][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16 * RT;
  const int G = K >> 4;
  const int S = (G + 15) >> 4;
  const int s_lo = S * wave / NW, cnt = S * (wave + 1) / NW - s_lo;
  const int row = lane & 15, kb = lane >> 4;
  const bool has_a = row < M;
  const int64_t ldb = K >> 2;

  v4i b[SPW][RT];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int g0 = (s_lo + i) * 16 + 4 * kb;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int n = n0 + rt * 16 + row;
      b[i][rt] = v4i{0, 0, 0, 0};
      if (i < cnt && n < N) {
        const uint8_t *p = B + (int64_t)n * ldb + 4 * (int64_t)g0;
        if (g0 + 4 <= G) {
          const v4i_u t = *reinterpret_cast<const v4i_u *>(p);
          b[i][rt] = v4i{t[0], t[1], t[2], t[3]};
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (g0 + t < G) b[i][rt][t] = reinterpret_cast<const int *>(p)[t];
        }
      }
    }
  }
  v4i a[SPW][4];
#pragma unroll
  for (int i = 0; i < SPW; ++i) {
    const int g0 = (s_lo + i) * 16 + 4 * kb;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[i][t] = v4i{0, 0, 0, 0};
      if (i < cnt && has_a && g0 + t < G)
        a[i][t] = *reinterpret_cast<const v4i *>(A + (int64_t)row * K + 16 * (g0 + t));
    }
  }
  v4i acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < SPW; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i][t], unpack16((uint32_t)b[i][rt][t]), acc[rt], 0, 0, 0);

#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][rt][lane][r] = acc[rt][r];
  __syncthreads();
  for (int e = threadIdx.x; e < RT * 256; e += NW * 64) {
    const int rt = e >> 8, l = (e >> 2) & 63, r = e & 3;
    int sum = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += red[w][rt][l][r];
    const int m = 4 * (l >> 4) + r, n = n0 + rt * 16 + (l & 15);
    if (m < M && n < N) {
      const int acc_v = sum - rowsum[m];
      const int64_t o = (int64_t)m * N + n;
      if (acc_out) acc_out[o] = acc_v;
      Y[o] = rescale(acc_v, deq[m], epi_gamma(ep, n));
    }
  }
}

// Fallback for very long rows (more than 16 waves x 8 supersteps): loops over
// its supersteps.
template <int RT, int NW>
__global__ __launch_bounds__(NW * 64) void gemv_loop_kernel(const int8_t *__restrict__ A,
                                                            const uint8_t *__restrict__ B,
                                                            const float *__restrict__ deq,
                                                            const int32_t *__restrict__ rowsum, int M, int N, int K,
                                                            Epilogue ep, float *__restrict__ Y,
                                                            int32_t *__restrict__ acc_out) {
  __shared__ int red[NW][RT][64][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16 * RT;
  const int G = K >> 4;
  const int S = (G + 15) >> 4;
  const int s_lo = S * wave / NW, s_hi = S * (wave + 1) / NW;
  const int row = lane & 15, kb = lane >> 4;
  const bool has_a = row < M;
  const int64_t ldb = K >> 2;

  v4i acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = v4i{0, 0, 0, 0};

  for (int ss = s_lo; ss < s_hi; ++ss) {
    const int g0 = ss * 16 + 4 * kb;
    v4i b[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int n = n0 + rt * 16 + row;
      b[rt] = v4i{0, 0, 0, 0};
      if (n < N) {
        const uint8_t *p = B + (int64_t)n * ldb + 4 * (int64_t)g0;
        if (g0 + 4 <= G) {
          const v4i_u t = *reinterpret_cast<const v4i_u *>(p);
          b[rt] = v4i{t[0], t[1], t[2], t[3]};
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (g0 + t < G) b[rt][t] = reinterpret_cast<const int *>(p)[t];
        }
      }
    }
    v4i a[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[t] = v4i{0, 0, 0, 0};
      if (has_a && g0 + t < G) a[t] = *reinterpret_cast<const v4i *>(A + (int64_t)row * K + 16 * (g0 + t));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        acc[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], unpack16((uint32_t)b[rt][t]), acc[rt], 0, 0, 0);
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][rt][lane][r] = acc[rt][r];
  __syncthreads();
  for (int e = threadIdx.x; e < RT * 256; e += NW * 64) {
    const int rt = e >> 8, l = (e >> 2) & 63, r = e & 3;
    int sum = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += red[w][rt][l][r];
    const int m = 4 * (l >> 4) + r, n = n0 + rt * 16 + (l & 15);
    if (m < M && n < N) {
      const int acc_v = sum - rowsum[m];
      const int64_t o = (int64_t)m * N + n;
      if (acc_out) acc_out[o] = acc_v;
      Y[o] = rescale(acc_v, deq[m], epi_gamma(ep, n));
    }
  }
}

template <int RT, int NW, int SPW>
hipError_t launch_cfg(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum, int m,
                      int n, int k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream) {
  const int blocks = (n + 16 * RT - 1) / (16 * RT);
  gemv_decode_kernel<RT, NW, SPW>
      <<<dim3((unsigned)blocks), dim3(NW * 64), 0, stream>>>(codes, packed, deq, rowsum, m, n, k, ep, y, acc_out);
  return hipGetLastError();
}

template <int RT>
hipError_t launch_rt(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum, int m,
                     int n, int k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream) {
  const int S = ((k >> 4) + 15) >> 4;  // supersteps of 256 k
  // fewest waves per workgroup whose slices fit in the unrolled register budget
  if (S <= 4 * BL_GEMV_MIN_WAVES) {
    return launch_cfg<RT, BL_GEMV_MIN_WAVES, (4 * BL_GEMV_MIN_WAVES + BL_GEMV_MIN_WAVES - 1) / BL_GEMV_MIN_WAVES>(
        codes, packed, deq, rowsum, m, n, k, ep, y, acc_out, stream);
  }
  if (S <= 4 * 8) return launch_cfg<RT, 8, 4>(codes, packed, deq, rowsum, m, n, k, ep, y, acc_out, stream);
  if (S <= 4 * 16) return launch_cfg<RT, 16, 4>(codes, packed, deq, rowsum, m, n, k, ep, y, acc_out, stream);
  const int blocks = (n + 16 * RT - 1) / (16 * RT);
  gemv_loop_kernel<RT, 16><<<dim3((unsigned)blocks), dim3(1024), 0, stream>>>(codes, packed, deq, rowsum, m, n, k, ep,
                                                                              y, acc_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_decode(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum,
                              int64_t m, int64_t n, int64_t k, const Epilogue &ep, float *y, int32_t *acc_out,
                              hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (m > BL_GEMV_RT1_MAX_M)
    return launch_rt<2>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
  return launch_rt<1>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
}

}  // namespace bl
