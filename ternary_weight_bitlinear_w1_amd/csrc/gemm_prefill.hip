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
#include <atomic>
#include <type_traits>

#include "common.h"

namespace bl {
namespace {

typedef int v4i_u __attribute__((ext_vector_type(4), aligned(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

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
                                                                   int K, Epilogue ep_in, float *__restrict__ Y,
                                                                   int32_t *__restrict__ acc_out) {
  const Epilogue ep = resolve_gamma(ep_in);
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


// Tile of the large-M kernel: waves in M, waves in N, 32x32 tiles per wave in M
// and N (tuned on MI355X; overridable when building variants to sweep).
#ifndef BL_GEMM_BIG_CFG
#define BL_GEMM_BIG_CFG 2, 2, 2, 4
#define BL_GEMM_BIG_BN 256
#endif
// tile of the few-token kernel (m <= 64): 64 rows x BL_GEMM_SMALL_BN columns,
// with a deeper ring: its chunks are small, so more of them are kept in flight.
// Four waves of 32 x 32 each: these shapes have about one workgroup per CU, and
// two waves of 64 x 32 left half of each CU's SIMDs idle (the 30-layer stack at
// 64 tokens: 1.605 against 1.660 ms per step on MI355X)
#ifndef BL_GEMM_SMALL_CFG
#define BL_GEMM_SMALL_CFG 2, 2, 1, 1
#define BL_GEMM_SMALL_BN 64
#endif
#ifndef BL_GEMM_SMALL_STAGES
#define BL_GEMM_SMALL_STAGES 4
#endif
// tile of the 8-wave kernel for shapes whose 128 x 256 tiles fill the chip
// unevenly (the down projection: 4096 x 2560 has 320 of them for 512 slots):
// 128 x 320 with waves 4 x 2, one workgroup per CU
#ifndef BL_GEMM_WIDE_CFG
#define BL_GEMM_WIDE_CFG 4, 2, 1, 5
#define BL_GEMM_WIDE_BN 320
#endif
#ifndef BL_GEMM_WIDE_STAGES
#define BL_GEMM_WIDE_STAGES 4
#endif
constexpr int kGroupM = 4;
// 1: a persistent grid (workgroups per CU x CUs) walks the tiles; 0: one
// workgroup per tile
#ifndef BL_GEMM_PERSIST
#define BL_GEMM_PERSIST 1
#endif

// Workgroups per CU of the persistent kernel: 8-wave workgroups run one per CU,
// smaller ones two (both give two waves per SIMD).
constexpr int wgs_per_cu(int waves) { return waves >= 8 ? 1 : 2; }

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

// 4-byte global -> LDS copy (lane l's dword lands at lds_base + 4 l).
__device__ __forceinline__ void copy4_to_lds(const void *src, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, off"
      :
      : "v"(src), "s"(lds_base)
      : "memory", "m0");
}

// Persistent form: gridDim.x workgroups (two per CU) walk the tiles
// t = blockIdx.x, blockIdx.x + gridDim.x, ... and the ring of P stages (P - 1
// chunks in flight) runs on across tile boundaries, so the next tile's loads
// and MFMAs overlap the previous tile's stores.
//
// The MFMA takes the unpacked weights as its A operand and the activation
// codes as its B operand, so a lane's accumulators hold 4 consecutive output
// features of one token and the epilogue stores them as one 16-byte store.
// Rows past M are clamped to M - 1 for loading and storing: every lane then
// computes and stores row M - 1's own value, which keeps the number of store
// instructions the same on every wave.
//
// Waiting: vector memory operations of a wave complete in issue order, so
// "at most X outstanding" waits exactly for everything older than the X most
// recent. Per wave and step c the operations younger than chunk c are the
// loads of chunks c + 1 .. c + P - 2, and, in the first P - 1 steps of a tile,
// the previous tile's row-data load (one per wave) and its kStores output
// stores; X is set to that count (or 0 when an acc_out copy doubles the stores
// past the counter, near the end of the stream, and for tiles of at most
// P - 1 chunks).
// Per-token deq / row sums go through a small double-buffered LDS area loaded
// with the same global->LDS copy, one instruction per wave per tile.
//
// Gated form (GLU): the weights are [gate; up] (N = 2 I rows) and a tile
// covers BN / 2 features j0 .. of both: its 32-column block cb holds gate
// (cb even) or up (cb odd) rows of features j0 + 32 (cb / 2) .. + 31, so a
// wave's accumulator tiles 2f and 2f + 1 are the gate and up sums of the same
// elements and the epilogue stores fl32(fl32(max(g, 0)^2) * u) ([M][I])
// instead of both (nnterp "BitNet b1.58" page, "The MLP gates with a squared
// ReLU"; gamma[0] scales the gate rows, gamma[1] the up rows).
//
// Split K (S > 1, for shapes with few tiles): work item t covers output tile
// t mod (tiles) over the K range [s K / S, (s + 1) K / S) with s = t / tiles,
// and stores its exact int32 sum of q * u over that range to
// part[s][m][n]; the row sums, rescale and sum over s are left to the
// consumer (integer sums: the total is the same in any order).
//
// K groups (KG > 1, for few-token shapes with at most one work item per CU):
// the workgroup holds KG groups of WM x WN waves, each with a ring of its own;
// group g takes chunks g, g + KG, g + 2 KG, ... of the work item, so each wave
// walks 1 / KG of the chunk chain and two or more waves share each SIMD. At
// the end the groups' exact int32 sums are added in group 0 through LDS and
// group 0 runs the epilogue. Every group steps through the same number of
// chunks, so all waves meet at every barrier. KG > 1 needs one work item per
// workgroup (the host launches one workgroup per item), since a group's ring
// serves as the area its sums are handed over in.
template <int WM, int WN, int TM, int TN, int P, bool GLU, int KG = 1>
__global__ __launch_bounds__(KG *WM *WN * 64, wgs_per_cu(KG *WM *WN)) void gemm_prefill_kernel(const int8_t *__restrict__ A,
                                                                      const uint8_t *__restrict__ B,
                                                                      const float *__restrict__ deq,
                                                                      const int32_t *__restrict__ rowsum, int M,
                                                                      int N, int K, Epilogue ep_in,
                                                                      float *__restrict__ Y,
                                                                      int32_t *__restrict__ acc_out, int S,
                                                                      int32_t *__restrict__ part) {
  const Epilogue ep = resolve_gamma(ep_in);
  constexpr int NW = WM * WN;
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  constexpr int kAStage = BM * 128, kBStage = BN * 32, kStage = kAStage + kBStage;
  constexpr int LA = BM / 8 / NW;   // 1 KB activation loads per wave per chunk
  constexpr int LBT = BN / 32;      // 1 KB weight loads per chunk
  // per wave: load j of wave w is weight load j NW + w; where LBT is not a
  // multiple of NW the waves past the end issue a 256-byte dummy copy instead,
  // so every wave has the same number of loads in flight
  constexpr int LB = (LBT + NW - 1) / NW;
  static_assert(!GLU || TN % 2 == 0, "gate and up tiles come in pairs");
  constexpr int kStores = TM * (GLU ? TN / 2 : TN) * 4;  // 16-byte output stores per wave per tile
  constexpr int kRowOps = BM / 32;      // 64-dword row-data loads per tile (deq, then row sums)
  static_assert(LA * NW * 8 == BM && LBT * 32 == BN, "tile must split into 1 KB wave loads");
  static_assert(kRowOps <= NW && kRowOps >= 2, "one row-data load per wave");
  constexpr int D = P - 1;  // chunks issued ahead of the one being computed
  constexpr int kWaitSteady = (D - 1) * (LA + LB);
  constexpr int kWaitAfterTile = kWaitSteady + 1 + kStores;
  static_assert(P >= 3, "ring of at least three stages");
  static_assert(kWaitAfterTile < 64, "vmcnt range");
  // the epilogue transposes through the stage just consumed, or through an
  // area of its own when the waves' 4 KB blocks do not fit in one stage
  constexpr bool kOwnScratch = NW * 32 * 32 * 4 > kStage;
  __shared__ __attribute__((aligned(1024))) int8_t ring[KG * P * kStage];
  __shared__ __attribute__((aligned(1024))) float own_scratch[kOwnScratch ? NW * 32 * 32 : 1];
  __shared__ __attribute__((aligned(256))) int s_dummy[64];
  __shared__ __attribute__((aligned(256))) float s_deq[2][BM];
  __shared__ __attribute__((aligned(256))) int s_rs[2][BM];

  const int lane = threadIdx.x & 63;
  const int kg = KG == 1 ? 0 : (int)(threadIdx.x >> 6) / NW;  // K group
  const int wave = KG == 1 ? (int)(threadIdx.x >> 6) : (int)(threadIdx.x >> 6) % NW;  // wave in the group
  const int wm = wave / WN, wn = wave % WN;
  int8_t *const my_ring = ring + kg * (P * kStage);  // this K group's stages
  const int half = lane >> 5, l32 = lane & 31;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = N / BN;  // GLU: (N / 2) / (BN / 2)
  const int I = N / 2;                                       // GLU: features
  const int Tmn = tiles_m * tiles_n;
  const int T = Tmn * S;
  const int G = gridDim.x, b = blockIdx.x;
  const int my_tiles = (T - b + G - 1) / G;
  const int64_t ldb = K >> 2;
  const int nk = (K >> 7) / S;  // chunks per work item
  const int nkg = nk / KG;      // of them, this K group's
  const int total = my_tiles * nkg;
  const bool two_stores = acc_out != nullptr;

  // work item i of this workgroup -> (m0, n0, split): XCD-contiguous ranges,
  // grouped along M; items of one split (one K range) are contiguous
  auto coords = [&](int i, int &m0, int &n0, int &sp) {
    int t = b + i * G;
    if ((T & 7) == 0 && (G & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
    sp = t / Tmn;
    t -= sp * Tmn;
    const int per_group = kGroupM * tiles_n;
    const int group = t / per_group, first_m = group * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int in_group = t - group * per_group;
    m0 = (first_m + in_group % gsize) * BM;
    n0 = (in_group / gsize) * (GLU ? BN / 2 : BN);
  };

  // ---- issue side: the chunk stream (tile is_i, chunk is_kc)
  int is_i = 0, is_kc = 0, is_m0, is_n0, is_s;
  coords(0, is_m0, is_n0, is_s);
  // per-lane source offsets of the current issue tile (32-bit: pick_cfg sends
  // only shapes with M K and N K / 4 below 2^31 here)
  uint32_t a_off[LA], b_off[LB];
  auto set_src = [&]() {
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int r = 8 * (wave * LA + j) + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int row = min(is_m0 + r, M - 1);
      a_off[j] = (uint32_t)row * (uint32_t)K + 16u * c + 128u * (uint32_t)(is_s * nk + kg);
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int jj = j * NW + wave < LBT ? j * NW + wave : 0;  // (dummy loads: any valid row)
      const int r = 32 * jj + (lane >> 1);
      const int h = (lane & 1) ^ ((r >> 3) & 1);
      const int wrow = GLU ? ((r >> 5) & 1) * I + is_n0 + 32 * (r >> 6) + (r & 31) : is_n0 + r;
      b_off[j] = (uint32_t)wrow * (uint32_t)ldb + 16u * h + 32u * (uint32_t)(is_s * nk + kg);
    }
  };
  set_src();
  auto issue_chunk = [&](int8_t *st) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(st) + wave * 1024 * LA);
#pragma unroll
    for (int j = 0; j < LA; ++j) copy16_to_lds(A + a_off[j] + 128 * KG * is_kc, base + j * 1024);
    const uint32_t bbase = __builtin_amdgcn_readfirstlane(lds_addr(st + kAStage) + wave * 1024);
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      if (LBT % NW == 0 || j * NW + wave < LBT)  // wave-uniform
        copy16_to_lds(B + b_off[j] + 32 * KG * is_kc, bbase + j * NW * 1024);
      else
        copy4_to_lds(B + 4 * lane, __builtin_amdgcn_readfirstlane(lds_addr(s_dummy)));
    }
    if (++is_kc == nkg) {
      is_kc = 0;
      if (++is_i < my_tiles) {
        coords(is_i, is_m0, is_n0, is_s);
        set_src();
      }
    }
  };
  // per-token deq and row sums of tile i into buffer i & 1: wave w loads part
  // (w % kRowOps) of [deq (BM/64 parts) | row sums (BM/64 parts)]
  auto issue_rows = [&](int i) {
    int m0, n0, sp;
    coords(i, m0, n0, sp);
    const int op = wave % kRowOps, part = op % (kRowOps / 2);
    const int row = min(m0 + part * 64 + lane, M - 1);
    if (op < kRowOps / 2)
      copy4_to_lds(deq + row, __builtin_amdgcn_readfirstlane(lds_addr(&s_deq[i & 1][part * 64])));
    else
      copy4_to_lds(rowsum + row, __builtin_amdgcn_readfirstlane(lds_addr(&s_rs[i & 1][part * 64])));
  };

  v16i acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0;

  // One chunk: the packed weights of the chunk and the codes of k-step 0 are
  // read first; the codes of k-step s + 1 are read while k-step s's MFMAs run.
  auto compute = [&](const int8_t *sa) {
    const int8_t *sb = sa + kAStage;
    auto read_codes = [&](int s, v4i *af) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int r = (wm * TM + tm) * 32 + l32;
        af[tm] = *reinterpret_cast<const v4i *>(sa + r * 128 + 16 * ((4 * half + s) ^ ((r >> 1) & 7)));
      }
    };
    v4i bp[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int r = (wn * TN + tn) * 32 + l32;
      bp[tn] = *reinterpret_cast<const v4i *>(sb + r * 32 + 16 * (half ^ ((r >> 3) & 1)));
    }
    v4i af[2][TM];
    read_codes(0, af[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) read_codes(s + 1, af[(s + 1) & 1]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const v4i wo = unpack16((uint32_t)bp[tn][s]);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tn][tm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(wo, af[s & 1][tm], acc[tn][tm], 0, 0, 0);
      }
    }
  };

  // ---- compute side
  int c_i = 0, c_m0, c_n0, c_s;
  coords(0, c_m0, c_n0, c_s);
  // Output of one tile. The stage just consumed serves as scratch: after a
  // barrier (every wave is done reading it) each wave writes one 32 x 32 fp32
  // block at a time in its accumulator layout and reads it back so that one
  // store instruction covers 8 rows x 128 contiguous bytes. Row r's 16-byte
  // piece c sits at piece c ^ ((r >> 1) & 7), so both the writes (16 rows, one
  // piece) and the reads (2 rows, all pieces) of 16 lanes hit distinct banks.
  auto epilogue = [&](int8_t *scratch_stage) {
    float *sc;
    if constexpr (kOwnScratch) {
      sc = own_scratch + wave * (32 * 32);
    } else {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      sc = reinterpret_cast<float *>(scratch_stage) + wave * (32 * 32);
    }
    const float *sd = s_deq[c_i & 1];
    const int *sr = s_rs[c_i & 1];
    if constexpr (GLU) {
      const float g_gate = ep.gamma[0], g_up = ep.gamma[1];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int mb = (wm * TM + tm) * 32;
        const int ml = mb + l32;
        const int rs = sr[ml];
        const float dq = sd[ml];
#pragma unroll
        for (int f = 0; f < TN / 2; ++f) {
          const int nb = c_n0 + 32 * ((wn * TN) / 2 + f);  // first feature of this block
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int nl = 8 * j + 4 * half;
            v4f v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float g = rescale(acc[2 * f][tm][4 * j + e] - rs, dq, g_gate);
              const float u = rescale(acc[2 * f + 1][tm][4 * j + e] - rs, dq, g_up);
              const float t = g > 0.0f ? g : 0.0f;
              v[e] = __fmul_rn(__fmul_rn(t, t), u);
            }
            *reinterpret_cast<v4f *>(sc + l32 * 32 + 4 * ((nl >> 2) ^ ((l32 >> 1) & 7))) = v;
          }
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            acc[2 * f][tm][q] = 0;
            acc[2 * f + 1][tm][q] = 0;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 8 * i + (lane >> 3);
            const v4f v = *reinterpret_cast<const v4f *>(sc + r * 32 + 4 * ((lane & 7) ^ ((r >> 1) & 7)));
            const int m = min(c_m0 + mb + r, M - 1);
            __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(Y + (int64_t)m * I + nb + 4 * (lane & 7)));
          }
        }
      }
      return;
    }
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const int mb = (wm * TM + tm) * 32;
      const int ml = mb + l32;
      const int rs = sr[ml];
      const float dq = sd[ml];
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const int nb = c_n0 + (wn * TN + tn) * 32;
        const float gb = epi_gamma(ep, nb);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int nl = 8 * j + 4 * half;
          if (part) {  // split K: the raw partial sums, bit for bit through the fp32 scratch
            const v4i raw = v4i{acc[tn][tm][4 * j], acc[tn][tm][4 * j + 1], acc[tn][tm][4 * j + 2],
                                acc[tn][tm][4 * j + 3]};
            *reinterpret_cast<v4f *>(sc + l32 * 32 + 4 * ((nl >> 2) ^ ((l32 >> 1) & 7))) =
                __builtin_bit_cast(v4f, raw);
            continue;
          }
          const int a0 = acc[tn][tm][4 * j] - rs, a1 = acc[tn][tm][4 * j + 1] - rs;
          const int a2 = acc[tn][tm][4 * j + 2] - rs, a3 = acc[tn][tm][4 * j + 3] - rs;
          if (two_stores) {
            const int m = min(c_m0 + ml, M - 1);
            *reinterpret_cast<v4i *>(acc_out + (int64_t)m * N + nb + nl) = v4i{a0, a1, a2, a3};
          }
          const int n = nb + nl;
          v4f v;
          if (ep.blocks32) {
            v = v4f{rescale(a0, dq, gb), rescale(a1, dq, gb), rescale(a2, dq, gb), rescale(a3, dq, gb)};
          } else {
            v = v4f{rescale(a0, dq, epi_gamma(ep, n)), rescale(a1, dq, epi_gamma(ep, n + 1)),
                    rescale(a2, dq, epi_gamma(ep, n + 2)), rescale(a3, dq, epi_gamma(ep, n + 3))};
          }
          *reinterpret_cast<v4f *>(sc + l32 * 32 + 4 * ((nl >> 2) ^ ((l32 >> 1) & 7))) = v;
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[tn][tm][q] = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * i + (lane >> 3);
          const v4f v = *reinterpret_cast<const v4f *>(sc + r * 32 + 4 * ((lane & 7) ^ ((r >> 1) & 7)));
          const int m = min(c_m0 + mb + r, M - 1);
          float *dst = part ? reinterpret_cast<float *>(part + ((int64_t)c_s * M + m) * N) : Y + (int64_t)m * N;
          __builtin_nontemporal_store(v, reinterpret_cast<v4f *>(dst + nb + 4 * (lane & 7)));
        }
      }
    }
  };

  auto meet = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // the row data of a tile is group 0's: only its epilogue reads it (in the
  // other groups every wait then covers one operation fewer, which waits for
  // no less)
  if (kg == 0) issue_rows(0);
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < total) issue_chunk(my_ring + j * kStage);
  int stage = 0;  // ring slot of chunk c
  int c = 0;
  for (; c_i < my_tiles;) {
    for (int kc = 0; kc < nkg; ++kc, ++c) {
      // wait for this wave's loads of chunk c: everything but the operations
      // issued after them (see the note above the kernel)
      if (c + D - 1 >= total || nkg <= D)
        wait_vm<0>();
      else if (c_i > 0 && kc < D)
        two_stores ? wait_vm<0>() : wait_vm<kWaitAfterTile>();
      else
        wait_vm<kWaitSteady>();
      meet();
      const int prev = stage == 0 ? P - 1 : stage - 1;  // the slot computed in the last step
      if (c + D < total) issue_chunk(my_ring + prev * kStage);
      compute(my_ring + stage * kStage);
      stage = stage == P - 1 ? 0 : stage + 1;
    }
    if (kg == 0 && c_i + 1 < my_tiles) issue_rows(c_i + 1);
    if (nkg <= D) {
      // with so few chunks the row data may still be in flight
      wait_vm<0>();
      meet();
    }
    if constexpr (KG > 1) {
      // Hand the sums to group 0. Every wave is past its last chunk and, with
      // one work item per workgroup, no chunk is in flight: each group's ring
      // is free. Lane l's accumulator q of tile t goes to int (t 16 + q) 64 + l
      // of its wave's block (one wave's stores cover 64 consecutive ints).
      constexpr int kAccInts = TN * TM * 16 * 64;
      static_assert(NW * kAccInts * 4 <= P * kStage, "a group's sums fit in its ring");
      wait_vm<0>();
      meet();
      if (kg != 0) {
        int *dst = reinterpret_cast<int *>(my_ring) + wave * kAccInts;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int q = 0; q < 16; ++q) dst[((tn * TM + tm) * 16 + q) * 64 + lane] = acc[tn][tm][q];
      }
      meet();
      if (kg == 0) {
#pragma unroll
        for (int g = 1; g < KG; ++g) {
          const int *src = reinterpret_cast<const int *>(ring + g * (P * kStage)) + wave * kAccInts;
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
              for (int q = 0; q < 16; ++q) acc[tn][tm][q] += src[((tn * TM + tm) * 16 + q) * 64 + lane];
        }
      }
    }
    if (kg == 0)
      epilogue(my_ring + (stage == 0 ? P - 1 : stage - 1) * kStage);
    else if constexpr (!kOwnScratch)
      meet();  // the epilogue's one barrier
    if (++c_i < my_tiles) coords(c_i, c_m0, c_n0, c_s);
  }
}

template <int WM, int WN, int TM, int TN>
hipError_t launch_generic(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum, int m,
                          int n, int k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const int64_t tiles = (int64_t)((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  if (tiles > 0x7fffffff) return hipErrorInvalidValue;  // one workgroup per tile
  gemm_generic_kernel<WM, WN, TM, TN>
      <<<dim3((unsigned)tiles), dim3(WM * WN * 64), 0, stream>>>(codes, packed, deq, rowsum, m, n, k, ep, y, acc_out);
  return hipGetLastError();
}

// CUs of the current device, asked once per device (threads that race on the
// first call store the same value)
int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int WM, int WN, int TM, int TN, int P, bool GLU = false, int KG = 1>
hipError_t launch_pipelined(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum, int m,
                            int n, int k, const Epilogue &ep, float *y, int32_t *acc_out, int splits, int32_t *part,
                            hipStream_t stream) {
  constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  const int64_t tiles = (int64_t)((m + BM - 1) / BM) * (n / BN) * splits;
  // K groups: each group takes an equal share of a work item's chunks
  if (KG > 1 && ((k / 128) / splits) % KG != 0) return hipErrorInvalidValue;
#if BL_GEMM_PERSIST
  int64_t grid = wgs_per_cu(KG * WM * WN) * (int64_t)cu_count();
  if (grid > tiles || KG > 1) grid = tiles;  // K groups: one work item per workgroup
#else
  const int64_t grid = tiles;
#endif
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  gemm_prefill_kernel<WM, WN, TM, TN, P, GLU, KG><<<dim3((unsigned)grid), dim3(KG * WM * WN * 64), 0, stream>>>(
      codes, packed, deq, rowsum, m, n, k, ep, y, part ? nullptr : acc_out, splits, part);
  return hipGetLastError();
}

// y = rescale(sum_s part[s] - rowsum, deq, gamma): the end of a split-K
// contraction, four outputs per thread
// (res: NULL, or [M][N] added to y: y = fl32(res + y))
__global__ __launch_bounds__(256) void splitk_finish_kernel(const int32_t *__restrict__ part, int S,
                                                            const float *__restrict__ deq,
                                                            const int32_t *__restrict__ rowsum, int M, int N,
                                                            Epilogue ep_in, float *__restrict__ Y,
                                                            int32_t *__restrict__ acc_out,
                                                            const float *__restrict__ res) {
  const Epilogue ep = resolve_gamma(ep_in);
  const int64_t plane = (int64_t)M * N;
  const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (4 * i4 >= plane) return;
  const int m = (int)(4 * i4 / N), n = (int)(4 * i4 - (int64_t)m * N);
  // every plane's load issued before the first add (straight-line code per
  // plane count: a loop over a run-time count waits for each load in turn)
  const int32_t *p0 = part + 4 * i4;
  v4i t;
  auto planes = [&](auto sc) {
    constexpr int SP = decltype(sc)::value;
    v4i u[SP];
#pragma unroll
    for (int j = 0; j < SP; ++j) u[j] = *reinterpret_cast<const v4i *>(p0 + j * plane);
    t = u[0];
#pragma unroll
    for (int j = 1; j < SP; ++j) t += u[j];
  };
  switch (S) {
    case 1: planes(std::integral_constant<int, 1>{}); break;
    case 2: planes(std::integral_constant<int, 2>{}); break;
    case 3: planes(std::integral_constant<int, 3>{}); break;
    case 4: planes(std::integral_constant<int, 4>{}); break;
    case 5: planes(std::integral_constant<int, 5>{}); break;
    case 6: planes(std::integral_constant<int, 6>{}); break;
    case 7: planes(std::integral_constant<int, 7>{}); break;
    case 8: planes(std::integral_constant<int, 8>{}); break;
    case 9: planes(std::integral_constant<int, 9>{}); break;
    default:
      t = *reinterpret_cast<const v4i *>(p0);
      for (int j = 1; j < S; ++j) t += *reinterpret_cast<const v4i *>(p0 + j * plane);
  }
  const int rs = rowsum[m];
  const float dq = deq[m];
  t -= v4i{rs, rs, rs, rs};
  if (acc_out) *reinterpret_cast<v4i *>(acc_out + 4 * i4) = t;
  v4f v = v4f{rescale(t[0], dq, epi_gamma(ep, n)), rescale(t[1], dq, epi_gamma(ep, n + 1)),
              rescale(t[2], dq, epi_gamma(ep, n + 2)), rescale(t[3], dq, epi_gamma(ep, n + 3))};
  if (res) {
    const v4f r = *reinterpret_cast<const v4f *>(res + 4 * i4);
    v = v4f{__fadd_rn(r[0], v[0]), __fadd_rn(r[1], v[1]), __fadd_rn(r[2], v[2]), __fadd_rn(r[3], v[3])};
  }
  *reinterpret_cast<v4f *>(Y + 4 * i4) = v;
}

}  // namespace

namespace {

// Tile shape of the pipelined kernel for (m, n, k), or 0 for the generic one.
enum { CFG_GENERIC = 0, CFG_BIG = 1, CFG_2224 = 2, CFG_2222 = 3, CFG_1422 = 4, CFG_SMALL = 5, CFG_WIDE = 6 };

// The 8-wave 128 x 320 tile where it fills the chip better than 128 x 256:
// with two 128 x 256 workgroups or one 128 x 320 workgroup per CU, a CU's share
// of the time is (rounds of workgroups) x (tile work), the tile work being
// 2 x 128 x 256 per round for the former and 128 x 320 for the latter.
bool wide_pays(int64_t m, int64_t n) {
  if (m <= 64 || n % BL_GEMM_WIDE_BN != 0) return false;
  const int64_t cus = cu_count(), tm = (m + 127) / 128;
  const int64_t t_wide = tm * (n / BL_GEMM_WIDE_BN);
  if (t_wide < cus) return false;
  const int64_t r_wide = (t_wide + cus - 1) / cus;
  if (n % BL_GEMM_BIG_BN != 0) return true;
  const int64_t t_big = tm * (n / BL_GEMM_BIG_BN), r_big = (t_big + 2 * cus - 1) / (2 * cus);
  return r_wide * BL_GEMM_WIDE_BN < r_big * 2 * BL_GEMM_BIG_BN;
}

// The pipelined kernel keeps its per-lane source offsets in 32 bits, so it
// takes only shapes whose codes (m k bytes) and packed weights (n k / 4 bytes)
// stay below 2^31; larger ones go to the generic kernel's 64-bit indexing.
constexpr int64_t kPipelinedMaxBytes = (int64_t)1 << 31;

// Where 128-row tiles leave at least half of the CUs without one, the 64 x 64
// tile of the few-token shapes spreads the same work over 4 to 8 times as many
// workgroups (on MI355X the FFN block at 1024 tokens, hidden 512: its down
// projection, 16 tiles of 128 x 256, took 21 us).
bool few_big_tiles(int64_t m, int64_t n, int64_t bm, int64_t bn) {
  return n % BL_GEMM_SMALL_BN == 0 && 2 * ((m + bm - 1) / bm) * (n / bn) <= cu_count();
}

int pick_cfg(int64_t m, int64_t n, int64_t k, int64_t *bm, int64_t *bn) {
  *bm = 0;
  *bn = 0;
  if (k % 128 != 0) return CFG_GENERIC;
  if (m * k >= kPipelinedMaxBytes || n * (k / 4) >= kPipelinedMaxBytes) return CFG_GENERIC;
  int cfg = CFG_GENERIC;
  if (wide_pays(m, n)) { *bm = 128; *bn = BL_GEMM_WIDE_BN; cfg = CFG_WIDE; }
  else if (n % BL_GEMM_BIG_BN == 0 && m > 64) { *bm = 128; *bn = BL_GEMM_BIG_BN; cfg = CFG_BIG; }
  else if (n % 256 == 0 && m > 64) { *bm = 128; *bn = 256; cfg = CFG_2224; }
  else if (n % 128 == 0 && m > 64) { *bm = 128; *bn = 128; cfg = CFG_2222; }
  if (cfg != CFG_GENERIC && !few_big_tiles(m, n, *bm, *bn)) return cfg;
  if ((m <= 64 || cfg != CFG_GENERIC) && n % BL_GEMM_SMALL_BN == 0) {
    *bm = 64; *bn = BL_GEMM_SMALL_BN; return CFG_SMALL;
  }
  *bm = 0;
  *bn = 0;
  if (n % 256 == 0) { *bm = 64; *bn = 256; return CFG_1422; }
  return CFG_GENERIC;
}

}  // namespace

int gemm_prefill_splits(int64_t m, int64_t n, int64_t k) {
  int64_t bm, bn;
  if (m <= 0 || n <= 0 || pick_cfg(m, n, k, &bm, &bn) == CFG_GENERIC) return 1;
  const int64_t tiles = ((m + bm - 1) / bm) * (n / bn);
  if (tiles >= kSplitMinTiles) return 1;
  // the divisor of the chunk count (K / 128) that brings the work items
  // closest to kSplitTarget, keeping at least two chunks per item and the
  // partial sums (d m n int32) within kSplitBytesPerWeightByte x the packed
  // weights (n k / 4 bytes): they are written and read back once more
  const int64_t chunks = k / 128;
  int best = 1;
  int64_t best_gap = kSplitTarget > tiles ? kSplitTarget - tiles : tiles - kSplitTarget;
  for (int64_t d = 2; 2 * d <= chunks; ++d) {
    if (chunks % d) continue;
    if (d * m * n * 4 > kSplitBytesPerWeightByte * (n * k / 4)) break;
    const int64_t items = tiles * d, gap = items > kSplitTarget ? items - kSplitTarget : kSplitTarget - items;
    if (gap < best_gap) {
      best = (int)d;
      best_gap = gap;
    }
  }
  return best;
}

// Two K groups for the few-token tile of (m, n, k) split S ways: where every
// work item gets a CU of its own and its chunk count is even. On MI355X the
// 30-layer stack at 64 tokens took 1.458 ms per step with up to two groups,
// 1.490 with none, 1.461 with up to three and 1.492 with up to four (the
// 64-token gate|up contraction: 10.3 against 12.1 us).
static bool small_k_groups(int64_t m, int64_t n, int64_t k, int S) {
  const int64_t items = ((m + 63) / 64) * (n / BL_GEMM_SMALL_BN) * S, nk = (k / 128) / S;
  return items <= cu_count() && nk % 2 == 0;
}

bool gemm_glu_supported(int64_t m, int64_t inter, int64_t k) {
  return m > 64 && k % 128 == 0 && inter % (BL_GEMM_BIG_BN / 2) == 0 && inter > 0 && m * k < kPipelinedMaxBytes &&
         2 * inter * (k / 4) < kPipelinedMaxBytes;
}

hipError_t launch_gemm_glu(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum,
                           int64_t m, int64_t inter, int64_t k, const Epilogue &ep, float *y, hipStream_t stream) {
  if (!gemm_glu_supported(m, inter, k) || ep.n_seg != 2) return hipErrorInvalidValue;
  // few 128 x 256 tiles: 64 x 128 ones (64 features of gate and up, four waves
  // of 32 x 64), 8 times as many (the FFN block at 1024 tokens, intermediate
  // 2048: 128 tiles of 128 x 256 took 12 us on MI355X)
  if (few_big_tiles(m, 2 * inter, 128, BL_GEMM_BIG_BN))
    return launch_pipelined<2, 2, 1, 2, 4, true>(codes, packed, deq, rowsum, (int)m, (int)(2 * inter), (int)k, ep, y,
                                                 nullptr, 1, nullptr, stream);
  return launch_pipelined<BL_GEMM_BIG_CFG, 3, true>(codes, packed, deq, rowsum, (int)m, (int)(2 * inter), (int)k, ep,
                                                    y, nullptr, 1, nullptr, stream);
}

size_t gemm_prefill_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  const int s = gemm_prefill_splits(m, n, k);
  return s > 1 ? (size_t)s * (size_t)m * (size_t)n * sizeof(int32_t) : 0;
}

hipError_t launch_gemm_prefill(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum,
                               int64_t m, int64_t n, int64_t k, const Epilogue &ep, float *y, int32_t *acc_out,
                               int32_t *split_ws, hipStream_t stream, int *splits_left, const float *res) {
  if (m == 0 || n == 0) return hipSuccess;
  const int M = (int)m, N = (int)n, K = (int)k;
  int64_t bm, bn;
  const int cfg = pick_cfg(m, n, k, &bm, &bn);
  const int S = split_ws ? gemm_prefill_splits(m, n, k) : 1;
  int32_t *part = S > 1 ? split_ws : nullptr;
  hipError_t e = hipSuccess;
  switch (cfg) {
    case CFG_BIG:
      e = launch_pipelined<BL_GEMM_BIG_CFG, 3>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, S, part, stream);
      break;
    case CFG_WIDE:
      e = launch_pipelined<BL_GEMM_WIDE_CFG, BL_GEMM_WIDE_STAGES>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, S,
                                                                  part, stream);
      break;
    case CFG_2224:
      e = launch_pipelined<2, 2, 2, 4, 3>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, S, part, stream);
      break;
    case CFG_2222:
      e = launch_pipelined<2, 2, 2, 2, 3>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, S, part, stream);
      break;
    case CFG_1422:
      e = launch_pipelined<1, 4, 2, 2, 3>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, S, part, stream);
      break;
    case CFG_SMALL:
      if (small_k_groups(m, n, k, S))
        e = launch_pipelined<BL_GEMM_SMALL_CFG, BL_GEMM_SMALL_STAGES, false, 2>(codes, packed, deq, rowsum, M, N, K, ep,
                                                                                y, acc_out, S, part, stream);
      else
        e = launch_pipelined<BL_GEMM_SMALL_CFG, BL_GEMM_SMALL_STAGES>(codes, packed, deq, rowsum, M, N, K, ep, y,
                                                                      acc_out, S, part, stream);
      break;
    default:
      if (m >= 256) return launch_generic<2, 2, 4, 2>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, stream);
      if (m > 64) return launch_generic<2, 2, 2, 2>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, stream);
      return launch_generic<1, 4, 2, 1>(codes, packed, deq, rowsum, M, N, K, ep, y, acc_out, stream);
  }
  if (splits_left) *splits_left = part ? S : 1;
  if (e != hipSuccess || !part || splits_left) return e;
  const int64_t quads = m * n / 4;
  splitk_finish_kernel<<<dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream>>>(part, S, deq, rowsum, M, N,
                                                                                        ep, y, acc_out, res);
  return hipGetLastError();
}

hipError_t launch_splitk_finish(const int32_t *part, int splits, const float *deq, const int32_t *rowsum, int64_t m,
                                int64_t n, const Epilogue &ep, float *y, int32_t *acc_out, const float *res,
                                hipStream_t stream) {
  const int64_t quads = m * n / 4;
  if (quads == 0) return hipSuccess;
  splitk_finish_kernel<<<dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, stream>>>(
      part, splits, deq, rowsum, (int)m, (int)n, ep, y, acc_out, res);
  return hipGetLastError();
}

}  // namespace bl
