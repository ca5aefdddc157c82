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
__global__ __launch_bounds__(WM *WN * 64) void gemm_generic_kernel(const int8_t *__restrict__ A,
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

// ---------------------------------------------------------------------------
// Pipelined kernel for N % BN == 0 and K % 128 == 0 (every 2B4T projection).
//
// Per K chunk of 128 a stage holds the activation tile (BM rows x 128 bytes)
// and the packed weight tile (BN rows x 32 bytes). Both are copied straight
// from global memory into LDS with the 16-byte global->LDS load (lane l's 16
// bytes land at the wave's LDS base + 16 l), two chunks ahead, into a ring of
// three stages; one barrier per chunk separates reuse of a stage. Rows are
// XOR-swizzled in 16-byte units so that each group of 16 lanes reading one
// 16-byte piece of 16 consecutive rows touches 16 distinct bank groups:
//   activation row r, piece c (of 8) is stored at piece c ^ ((r >> 1) & 7),
//   weight row r, half h (of 2) at half h ^ ((r >> 3) & 1).
// Rows past M are clamped to M - 1 for loading; their outputs are not stored.
// Workgroups are numbered so that each XCD (workgroup id mod 8) receives a
// contiguous range of tiles, walked in groups of kGroupM tile rows, which keeps
// an XCD's activation rows and the weight columns it is streaming in its L2.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

constexpr int kStages = 3;
constexpr int kGroupM = 4;

// 16-byte global -> LDS copy: lane l's 16 bytes go to LDS byte address
// lds_base + 16 l (lds_base must be the same on every lane). Issued as a plain
// instruction so that the compiler adds no waits of its own for it: it has no
// output register, and its completion is awaited explicitly with wait_vm.
__device__ __forceinline__ void copy16_to_lds(const void *src, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(lds_base)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int WM, int WN, int TM, int TN>
__global__ __launch_bounds__(WM *WN * 64, 2) void gemm_prefill_kernel(const int8_t *__restrict__ A,
                                                                      const uint8_t *__restrict__ B,
                                                                      const float *__restrict__ deq,
                                                                      const int32_t *__restrict__ rowsum, int M,
                                                                      int N, int K, Epilogue ep,
                                                                      float *__restrict__ Y,
                                                                      int32_t *__restrict__ acc_out) {
  constexpr int NW = WM * WN;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int kAStage = BM * 128, kBStage = BN * 32, kStage = kAStage + kBStage;
  constexpr int LA = BM / 8 / NW;   // 1 KB activation loads per wave per chunk
  constexpr int LB = BN / 32 / NW;  // 1 KB weight loads per wave per chunk
  static_assert(LA * NW * 8 == BM && LB * NW * 32 == BN, "tile must split into 1 KB wave loads");
  // one array per stage, so that the compiler can tell a stage being read from
  // the stages whose loads are still in flight
  __shared__ __attribute__((aligned(1024))) int8_t st0[kStage];
  __shared__ __attribute__((aligned(1024))) int8_t st1[kStage];
  __shared__ __attribute__((aligned(1024))) int8_t st2[kStage];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;

  // ---- tile index: XCD-contiguous ranges, grouped along M
  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;
  const int T = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((T & 7) == 0) bid = (bid & 7) * (T >> 3) + (bid >> 3);
  const int per_group = kGroupM * tiles_n;
  const int group = bid / per_group, first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = bid - group * per_group;
  const int m0 = (first_m + in_group % gsize) * BM;
  const int n0 = (in_group / gsize) * BN;
  const int64_t ldb = K >> 2;
  const int nk = K >> 7;

  // ---- per-lane load sources (chunk 0); chunk kc adds 128 kc (A) / 32 kc (B)
  const int8_t *a_src[LA];
#pragma unroll
  for (int j = 0; j < LA; ++j) {
    const int r = 8 * (wave * LA + j) + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    const int row = min(m0 + r, M - 1);
    a_src[j] = A + (int64_t)row * K + 16 * c;
  }
  const uint8_t *b_src[LB];
#pragma unroll
  for (int j = 0; j < LB; ++j) {
    const int r = 32 * (wave * LB + j) + (lane >> 1);
    const int h = (lane & 1) ^ ((r >> 3) & 1);
    b_src[j] = B + (int64_t)(n0 + r) * ldb + 16 * h;
  }
  auto issue = [&](int8_t *st, int kc) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(st) + wave * 1024 * (LA + 0));
#pragma unroll
    for (int j = 0; j < LA; ++j) copy16_to_lds(a_src[j] + 128 * kc, base + j * 1024);
    const uint32_t bbase = __builtin_amdgcn_readfirstlane(lds_addr(st + kAStage) + wave * 1024 * LB);
#pragma unroll
    for (int j = 0; j < LB; ++j) copy16_to_lds(b_src[j] + 32 * kc, bbase + j * 1024);
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0;

  auto compute = [&](const int8_t *sa) {
    const int8_t *sb = sa + kAStage;
    v4i bp[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int r = (wn * TN + tn) * 32 + l32;
      bp[tn] = *reinterpret_cast<const v4i *>(sb + r * 32 + 16 * (half ^ ((r >> 3) & 1)));
    }
    v4i af[4][TM];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int r = (wm * TM + tm) * 32 + l32;
        af[s][tm] = *reinterpret_cast<const v4i *>(sa + r * 128 + 16 * ((4 * half + s) ^ ((r >> 1) & 7)));
      }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const v4i bo = unpack16((uint32_t)bp[tn][s]);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tm][tn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[s][tm], bo, acc[tm][tn], 0, 0, 0);
      }
    }
  };
  // One K chunk: wait for this thread's loads of chunk kc (those of kc + 1 may
  // stay in flight), meet the other waves (their loads of kc have landed and
  // they are done reading chunk kc - 1's stage), refill that stage with chunk
  // kc + 2, then compute. The barrier carries no memory fence: the loads are
  // ordered by the explicit vmcnt wait, and each wave's LDS reads have been
  // consumed by its MFMAs before it reaches the next barrier.
  auto step = [&](int8_t *cur, int8_t *refill, int kc) {
    if (kc + 1 < nk)
      wait_vm<LA + LB>();
    else
      wait_vm<0>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kc + 2 < nk) issue(refill, kc + 2);
    compute(cur);
  };

  issue(st0, 0);
  if (nk > 1) issue(st1, 1);
  int kc = 0;
  for (; kc + 3 <= nk; kc += 3) {
    step(st0, st2, kc);
    step(st1, st0, kc + 1);
    step(st2, st1, kc + 2);
  }
  if (kc < nk) step(st0, st2, kc);
  if (kc + 1 < nk) step(st1, st0, kc + 1);

  // ---- epilogue: row data through LDS, then undo the field offset, rescale, store
  __syncthreads();
  float *s_deq = reinterpret_cast<float *>(st0);
  int *s_rs = reinterpret_cast<int *>(st0 + BM * 4);
  for (int i = threadIdx.x; i < BM; i += NW * 64) {
    const int m = min(m0 + i, M - 1);
    s_deq[i] = deq[m];
    s_rs[i] = rowsum[m];
  }
  __syncthreads();
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) {
    const int n = n0 + (wn * TN + tn) * 32 + l32;
    const float g = epi_gamma(ep, n);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int rl = (wm * TM + tm) * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
        const int m = m0 + rl;
        if (m < M) {
          const int a = acc[tm][tn][q] - s_rs[rl];
          const int64_t o = (int64_t)m * N + n;
          if (acc_out) acc_out[o] = a;
          __builtin_nontemporal_store(rescale(a, s_deq[rl], g), Y + o);
        }
      }
    }
  }
}

template <int WM, int WN, int TM, int TN>
hipError_t launch_generic(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum, int m,
                          int n, int k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const int64_t tiles = (int64_t)((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  gemm_generic_kernel<WM, WN, TM, TN>
      <<<dim3((unsigned)tiles), dim3(WM * WN * 64), 0, stream>>>(codes, packed, deq, rowsum, m, n, k, ep, y, acc_out);
  return hipGetLastError();
}

template <int WM, int WN, int TM, int TN>
hipError_t launch_pipelined(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum, int m,
                            int n, int k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const int64_t tiles = (int64_t)((m + BM - 1) / BM) * (n / BN);
  gemm_prefill_kernel<WM, WN, TM, TN>
      <<<dim3((unsigned)tiles), dim3(WM * WN * 64), 0, stream>>>(codes, packed, deq, rowsum, m, n, k, ep, y, acc_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_prefill(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum,
                               int64_t m, int64_t n, int64_t k, const Epilogue &ep, float *y, int32_t *acc_out,
                               hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  const int M = (int)m, N = (int)n, K = (int)k;
  if (K % 128 == 0) {
    if (N % 256 == 0 && M > 64)
      return launch_pipelined<2, 2, 2, 4>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, stream);
    if (N % 128 == 0 && M > 64)
      return launch_pipelined<2, 2, 2, 2>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, stream);
    if (N % 256 == 0)
      return launch_pipelined<1, 4, 2, 2>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, stream);
  }
  if (m >= 256)
    return launch_generic<2, 2, 4, 2>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, stream);
  if (m > 64)
    return launch_generic<2, 2, 2, 2>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, stream);
  return launch_generic<1, 4, 2, 1>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, stream);
}

}  // namespace bl
