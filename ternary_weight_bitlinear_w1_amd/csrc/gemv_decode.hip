// Decode contraction (m <= 16 tokens): stream the packed ternary weights once
// from HBM and contract them with the int8 codes. Same result as the prefill
// kernel: y[m][n] = fl32(fl32((float)acc * deq[m]) * gamma(n)), acc exact in
// int32 (nnterp "BitNet b1.58" page, "The projections quantize their inputs and
// weights" and "The two checkpoints"; no bias: model card "Model Details").
//
// This path is bound by HBM bandwidth on the packed weights (n * k / 4 bytes);
// the codes (m * k bytes) stay in L2. Two kernels:
//
// * one token (gemv_dot4_kernel): coalesced lines, v_dot4, cross-lane sums;
//   described above the kernel.
// * several tokens (gemv_decode_kernel, int8 MFMA v_mfma_i32_16x16x64_i8): a
//   workgroup of NW waves owns RT tiles of 16 output rows and splits K into NW
//   contiguous slices, one per wave. A "superstep" is 256 k: lane l loads one
//   16-byte piece of row (l % 16) of the tile, covering k-blocks 4 (l / 16) ..
//   +3, so the 4 lanes of a row read 64 contiguous bytes and a wave-wide load
//   moves 16 rows x 64 bytes. Each packed dword (16 weights) unpacks with one
//   shift and one AND per 4 weights into exactly the lane's 16-byte MFMA
//   operand; MFMA t of the superstep uses dword t. MFMA operand convention
//   (checked on gfx950): lane l supplies row l % 16 of A and column l % 16 of
//   B, both for k-block l / 16; output lane l, register r holds row
//   4 (l / 16) + r, column l % 16. Here A rows are tokens (rows >= m repeat
//   row m - 1 and give outputs that are not stored) and B columns are output
//   rows. The NW partial tiles are added in LDS
//   (exact integer sums), then the field offset is removed
//   (acc = sum q u - sum q) and the rescale is fused.
#include <type_traits>

#include "common.h"

namespace bl {
namespace {

typedef int v4i_u __attribute__((ext_vector_type(4), aligned(4)));
constexpr uint32_t kFieldMask = 0x03030303u;

// Launch shape (tuned on MI355X; overridable when building variants to sweep).
#ifndef BL_GEMV_MIN_WAVES
#define BL_GEMV_MIN_WAVES 4
#endif
#ifndef BL_GEMV_DOT4_MAX_M  // measured at 2 tokens: down 3.65 us with MFMA, 4.21 with v_dot4
#define BL_GEMV_DOT4_MAX_M 1
#endif
#ifndef BL_GEMV_MIN_WGS
#define BL_GEMV_MIN_WGS 512
#endif
#ifndef BL_GEMV_RT1_MAX_M
#define BL_GEMV_RT1_MAX_M 4
#endif
#ifndef BL_GEMV_MC_5_8
#define BL_GEMV_MC_5_8 8
#endif
#ifndef BL_GEMV_FEW_WG_NW16
#define BL_GEMV_FEW_WG_NW16 1
#endif
#ifndef BL_GEMV_LDS_CODES
#define BL_GEMV_LDS_CODES 1
#endif
#ifndef BL_DOT4_EXACT_LPW
#define BL_DOT4_EXACT_LPW 1
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
//
// ROPE form (RT = 2, the cached decoder's q|k|v projection): a workgroup of the
// q and k heads owns rows e (tile 0) and e + hd/2 (tile 1) of one head for 16
// consecutive e, so it rotates each pair itself, with the cosine and sine read
// from the step's rows of the rotary table (rope_gather_kernel) while the weights load, and writes the
// keys to the bfloat16 cache; workgroups of the value heads append the values.
template <int RT, int NW, int SPW, bool ROPE = false, int MC = 0, bool K64 = false>
__global__ __launch_bounds__(NW * 64) void gemv_decode_kernel(const int8_t *__restrict__ A,
                                                              const uint8_t *__restrict__ B,
                                                              const float *__restrict__ deq,
                                                              const int32_t *__restrict__ rowsum, int M, int N, int K,
                                                              Epilogue ep_in, float *__restrict__ Y,
                                                              int32_t *__restrict__ acc_out, DecodeRope rope) {
  static_assert(!ROPE || RT == 2, "rotated pairs take the two row tiles");
  static_assert(SPW >= 1 && SPW <= 4, "at most four supersteps per wave");
  const Epilogue ep = resolve_gamma(ep_in);
  __shared__ int red[NW][RT][64][4];
  __shared__ __attribute__((aligned(16))) int8_t scodes[MC > 0 ? NW : 1][MC > 0 ? MC * SPW * 256 : 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16 * RT;
  // ROPE form: workgroups [0, rot_wgs) hold rotated pairs, hd / 32 per head
  const int rot_wgs = ROPE ? (rope.n_heads + rope.n_kv) * (rope.hd / 32) : 0;
  const bool rotated = ROPE && (int)blockIdx.x < rot_wgs;
  const int rh = rotated ? (int)blockIdx.x / (rope.hd / 32) : 0;
  const int rj = rotated ? (int)blockIdx.x - rh * (rope.hd / 32) : 0;
  // output row of row tile rt, tile row rr
  auto row_of = [&](int rt, int rr) -> int {
    if (rotated) return rh * rope.hd + rt * (rope.hd / 2) + 16 * rj + rr;
    return n0 + rt * 16 + rr;
  };
  const int G = K >> 4;
  const int S = (G + 15) >> 4;
  const int s_lo = S * wave / NW, cnt = S * (wave + 1) / NW - s_lo;
  const int row = lane & 15, kb = lane >> 4;
  const int64_t ldb = K >> 2;
  const int ta = row < M ? row : M - 1;  // token row of this lane's operand loads

  // Every load below is unconditional, with rows and pieces clamped into
  // range: a token row past M, a weight row past N or a piece past the row's
  // end loads in-range data that only meets zero weights or feeds outputs that
  // are never stored. Loads guarded by conditions made the compiler merge the
  // guarded values through register copies, each preceded by a wait for every
  // load in flight, which serialized the code loads (one L2 round trip each).

  // row data of this thread's epilogue elements, fetched first
  constexpr int kEpi = (RT * 256 + NW * 64 - 1) / (NW * 64);
  int e_rs[kEpi];
  float e_dq[kEpi];
#pragma unroll
  for (int j = 0; j < kEpi; ++j) {
    const int e = threadIdx.x + j * NW * 64;
    int m = 4 * ((e >> 6) & 3) + (e & 3);
    m = m < M ? m : M - 1;
    e_rs[j] = rowsum[m];
    e_dq[j] = deq[m];
  }
  // ROPE form: the cosine and sine of each of this thread's pairs (epilogue entries in
  // tile 0: token m, pair e = 16 rj + l % 16)
  float rc[kEpi], rsn[kEpi];
#pragma unroll
  for (int j = 0; j < kEpi; ++j) {
    rc[j] = 0.0f;
    rsn[j] = 0.0f;
    if constexpr (ROPE) {
      const int e = threadIdx.x + j * NW * 64;
      const int l = (e >> 2) & 63;
      int m = 4 * (l >> 4) + (e & 3);
      m = m < M ? m : M - 1;
      const float2 cs = rope.cs[m * (rope.hd / 2) + 16 * rj + (l & 15)];
      rc[j] = cs.x;
      rsn[j] = cs.y;
    }
  }

  // four independent accumulators per row tile (one per 64-k block of a
  // superstep), so the MFMAs do not wait on one another's results
  v4i acc4[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc4[rt][t] = v4i{0, 0, 0, 0};
  // The loads and MFMAs of a wave with C supersteps, straight-line code. With
  // K % 64 == 0 (K64) a 16-byte weight piece lies wholly inside or wholly past
  // the row: pieces past it load the row's last piece, and the codes they meet
  // are zero.
  auto contract = [&](auto cc) {
    constexpr int C = decltype(cc)::value;
    v4i b[C][RT];
    v4i a[C][4];
    auto load_weights = [&]() {
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const int g0 = (s_lo + i) * 16 + 4 * kb;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const int n = row_of(rt, row);
          if constexpr (K64) {
            const int gc = g0 < G ? g0 : G - 4;
            const v4i_u t = *reinterpret_cast<const v4i_u *>(B + (int64_t)(n < N ? n : N - 1) * ldb + 4 * (int64_t)gc);
            b[i][rt] = v4i{t[0], t[1], t[2], t[3]};
            continue;
          }
          const uint8_t *p = B + (int64_t)(n < N ? n : N - 1) * ldb + 4 * (int64_t)g0;
          if (g0 + 4 <= G) {
            const v4i_u t = *reinterpret_cast<const v4i_u *>(p);
            b[i][rt] = v4i{t[0], t[1], t[2], t[3]};
          } else {  // the row's last, partial superstep
            b[i][rt] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int t = 0; t < 4; ++t)
              if (g0 + t < G) b[i][rt][t] = reinterpret_cast<const int *>(p)[t];
          }
        }
      }
    };
    if constexpr (MC > 0) {
      // The wave's code slice goes through LDS: slot (i, t) of its area holds the
      // 256 codes of token t in its superstep i, its 16-byte piece c at piece
      // c ^ t, so that the 16 lanes reading one piece of 16 tokens hit 16
      // distinct bank groups. Every code load is a full 64-lane load of 16
      // bytes (lane l covers slot 4 j + l / 16, piece l % 16), so a few loads
      // carry what per-lane operand loads would take 4 C partly masked loads for.
      v4i cs[MC * C / 4];
#pragma unroll
      for (int j = 0; j < MC * C / 4; ++j) {
        const int slot = 4 * j + (lane >> 4);
        const int i = slot / MC, t = slot - i * MC;
        int off = (s_lo + i) * 256 + 16 * (lane & 15);
        off = off < K - 16 ? off : K - 16;
        cs[j] = *reinterpret_cast<const v4i *>(A + (int64_t)(t < M ? t : M - 1) * K + off);
      }
      load_weights();
#pragma unroll
      for (int j = 0; j < MC * C / 4; ++j) {
        const int slot = 4 * j + (lane >> 4);
        const int t = slot % MC;
        v4i v = cs[j];
        if constexpr (K64) {  // codes past the row's end are zero
          const bool in = (s_lo + slot / MC) * 256 + 16 * (lane & 15) < K;
          v = in ? v : v4i{0, 0, 0, 0};
        }
        *reinterpret_cast<v4i *>(scodes[wave] + 1024 * j + 256 * (lane >> 4) + 16 * ((lane & 15) ^ t)) = v;
      }
      __asm__ volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave's own stores are in LDS
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < C; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          a[i][t] = row < MC ? *reinterpret_cast<const v4i *>(scodes[wave] + (i * MC + row) * 256 +
                                                              16 * ((4 * kb + t) ^ row))
                             : v4i{0, 0, 0, 0};
    } else {
      // the codes (a few KB, from L2) first: a wave's loads return in issue
      // order, so they are in registers by the time the first weights arrive
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const int g0 = (s_lo + i) * 16 + 4 * kb;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          a[i][t] = *reinterpret_cast<const v4i *>(A + (int64_t)ta * K + 16 * (g0 + t < G ? g0 + t : G - 1));
      }
      load_weights();
    }
#pragma unroll
    for (int i = 0; i < C; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v4i ai = a[i][t];
        if constexpr (K64 && MC == 0) {  // codes past the row's end are zero
          const int g = (s_lo + i) * 16 + 4 * kb + t;
          ai = g < G ? ai : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          acc4[rt][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ai, unpack16((uint32_t)b[i][rt][t]), acc4[rt][t], 0, 0, 0);
      }
  };
  // cnt <= SPW (wave-uniform)
  switch (cnt) {
    case 1: contract(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (SPW >= 2) contract(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (SPW >= 3) contract(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr (SPW >= 4) contract(std::integral_constant<int, 4>{}); break;
    default: break;
  }
  v4i acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = (acc4[rt][0] + acc4[rt][1]) + (acc4[rt][2] + acc4[rt][3]);

#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][rt][lane][r] = acc[rt][r];
  __syncthreads();
  if constexpr (ROPE) {
    // entries of tile 0 take their tile-1 partner: (rows e, e + hd/2) rotated,
    // or two value rows appended
#pragma unroll
    for (int j = 0; j < kEpi; ++j) {
      const int e = threadIdx.x + j * NW * 64;
      if (e >= 256) break;
      const int l = (e >> 2) & 63, r = e & 3;
      int s0 = 0, s1 = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        s0 += red[w][0][l][r];
        s1 += red[w][1][l][r];
      }
      const int m = 4 * (l >> 4) + r, na = row_of(0, l & 15), nb = row_of(1, l & 15);
      if (m >= M) continue;
      const int a0 = s0 - e_rs[j], a1 = s1 - e_rs[j];
      float y0 = rescale(a0, e_dq[j], epi_gamma(ep, na)), y1 = rescale(a1, e_dq[j], epi_gamma(ep, nb));
      if (acc_out) {
        acc_out[(int64_t)m * N + na] = a0;
        acc_out[(int64_t)m * N + nb] = a1;
      }
      const int64_t sl = rope.slot[m], p = rope.pos[m];
      const bool put = sl >= 0 && sl < rope.n_slots && p >= 0 && p < rope.tmax;
      if (rotated) {
        const float ra = __fsub_rn(__fmul_rn(y0, rc[j]), __fmul_rn(y1, rsn[j]));
        const float rb = __fadd_rn(__fmul_rn(y1, rc[j]), __fmul_rn(y0, rsn[j]));
        y0 = ra;
        y1 = rb;
        if (rh >= rope.n_heads && put) {  // a key head
          const int pe = 16 * rj + (l & 15);
          const int64_t dst = ((sl * rope.n_kv + (rh - rope.n_heads)) * rope.tmax + p) * rope.hd;
          rope.kc[dst + pe] = (uint16_t)bf16_rne(ra);
          rope.kc[dst + pe + rope.hd / 2] = (uint16_t)bf16_rne(rb);
        }
      } else if (put) {  // value rows
        const int v0 = na - (rope.n_heads + rope.n_kv) * rope.hd, v1 = nb - (rope.n_heads + rope.n_kv) * rope.hd;
        const int g0 = v0 / rope.hd, g1 = v1 / rope.hd;
        rope.vc[((sl * rope.n_kv + g0) * rope.tmax + p) * rope.hd + (v0 - g0 * rope.hd)] = (uint16_t)bf16_rne(y0);
        rope.vc[((sl * rope.n_kv + g1) * rope.tmax + p) * rope.hd + (v1 - g1 * rope.hd)] = (uint16_t)bf16_rne(y1);
      }
      Y[(int64_t)m * N + na] = y0;
      Y[(int64_t)m * N + nb] = y1;
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < kEpi; ++j) {
    const int e = threadIdx.x + j * NW * 64;
    if (e >= RT * 256) break;
    const int rt = e >> 8, l = (e >> 2) & 63, r = e & 3;
    int sum = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += red[w][rt][l][r];
    const int m = 4 * (l >> 4) + r, n = n0 + rt * 16 + (l & 15);
    if (m < M && n < N) {
      const int acc_v = sum - e_rs[j];
      const int64_t o = (int64_t)m * N + n;
      if (acc_out) acc_out[o] = acc_v;
      Y[o] = rescale(acc_v, e_dq[j], epi_gamma(ep, n));
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
                                                            Epilogue ep_in, float *__restrict__ Y,
                                                            int32_t *__restrict__ acc_out) {
  const Epilogue ep = resolve_gamma(ep_in);
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

// ---------------------------------------------------------------------------
// One-token kernel (K % 64 == 0, K <= kDot4MaxK; written for up to four tokens,
// but from two tokens on the MFMA kernel is faster): dot-product form.
//
// Lane l of a wave reads 16 bytes (64 weights) of row l / 8 at piece l % 8 of
// each 128-byte line, so every wave-wide load moves 8 full lines. The token
// codes of the workgroup's K range sit in LDS, where the 8 lanes that share a
// piece read the same bytes (broadcast). Each packed dword d gives, with one
// shift and one AND, the four weight bytes (d >> 2j) & 0x03030303 of codes
// 16g + 4j .. +3, contracted against the matching code dword by v_dot4_i32_i8.
// The 8 partial sums of a row are added with DPP adds, the KS
// waves that split a row's K range through LDS, all in exact integers.
constexpr int kDot4MaxK = 8192;

template <int MT, int KS, int LPW>
__global__ __launch_bounds__(256) void gemv_dot4_kernel(const int8_t *__restrict__ A, const uint8_t *__restrict__ B,
                                                        const float *__restrict__ deq,
                                                        const int32_t *__restrict__ rowsum, int N, int K, Epilogue ep_in,
                                                        float *__restrict__ Y, int32_t *__restrict__ acc_out) {
  const Epilogue ep = resolve_gamma(ep_in);
  constexpr int RG = 4 / KS;  // row groups of 8 rows per workgroup
  constexpr int NT = 256;
  __shared__ __attribute__((aligned(16))) int8_t sc[MT * kDot4MaxK];
  __shared__ int red[KS][RG][8][MT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ks = wave % KS, rg = wave / KS;
  const int n = blockIdx.x * 8 * RG + rg * 8 + (lane >> 3);
  const int p = lane & 7;
  const int ldb = K >> 2;                 // bytes per weight row (multiple of 16)
  const int L = (ldb + 127) >> 7;         // 128-byte lines per row, the last may be partial
  const int l_lo = L * ks / KS, l_hi = L * (ks + 1) / KS;

  // Loads in issue order: this workgroup's token codes (a few KB from L2; the
  // waves of a row group share them through LDS), then the weights (from
  // HBM). Loads complete in issue order, so the codes are in LDS while the
  // weights stream, and each weight piece is used as soon as it arrives: the
  // barrier below waits for LDS traffic only. Every lane issues the same
  // number of loads (out-of-range pieces reload a valid address, unused).
  constexpr int kCodeLoads = (MT * kDot4MaxK / 16 + NT - 1) / NT;
  const int n_pieces = MT * (K >> 4);
  v4i cw[kCodeLoads];
#pragma unroll
  for (int j = 0; j < kCodeLoads; ++j) {
    const int i = threadIdx.x + NT * j;
    const int t = i / (K >> 4), c = i - t * (K >> 4);
    cw[j] = *reinterpret_cast<const v4i *>(i < n_pieces ? A + (int64_t)t * K + 16 * c : A);
  }
  __builtin_amdgcn_sched_barrier(0);
  v4i w[LPW];
  // (a piece past the row's end reloads the first piece of the lane's own row,
  // so such reloads spread over many lines instead of meeting on one)
  const uint8_t *own = B + (int64_t)(n < N ? n : N - 1) * ldb + 16 * p;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int off = 128 * (l_lo + i) + 16 * p;
    const bool use = l_lo + i < l_hi && off < ldb && n < N;
    w[i] = *reinterpret_cast<const v4i *>(use ? B + (int64_t)n * ldb + off : own);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kCodeLoads; ++j) {
    const int i = threadIdx.x + NT * j;
    if (i < n_pieces) {
      const int t = i / (K >> 4), c = i - t * (K >> 4);
      *reinterpret_cast<v4i *>(sc + t * kDot4MaxK + 16 * c) = cw[j];
    }
  }
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's code stores are in LDS
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  int rs[MT];
  float dq[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    rs[t] = rowsum[t];
    dq[t] = deq[t];
  }

  int acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = 0;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int k0 = 4 * (128 * (l_lo + i) + 16 * p);  // first code of this piece
    if (l_lo + i < l_hi && k0 < K) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const v4i *cp = reinterpret_cast<const v4i *>(sc + t * kDot4MaxK + k0);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const v4i c = cp[d];  // codes k0 + 16 d .. + 15
          const uint32_t wd = (uint32_t)w[i][d];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[t] = __builtin_amdgcn_sdot4((int)((wd >> (2 * j)) & kFieldMask), c[j], acc[t], false);
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
      const int a = sum - rs[t];
      const int64_t o = (int64_t)t * N + n;
      if (acc_out) acc_out[o] = a;
      Y[o] = rescale(a, dq[t], g);
    }
  }
}

template <int MT>
hipError_t launch_dot4_mt(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum, int n,
                          int k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream) {
  const int lines = ((k >> 2) + 127) >> 7;
  // split K over the waves of a workgroup until the workgroups cover the CUs
  const int ks = n / 32 >= BL_GEMV_MIN_WGS ? 1 : (n / 16 >= BL_GEMV_MIN_WGS ? 2 : 4);
  const int lpw = (lines + ks - 1) / ks;
  const int rows_per_wg = 8 * (4 / ks);
  const dim3 grid((unsigned)((n + rows_per_wg - 1) / rows_per_wg)), block(256);
#define BL_DOT4(KS_, LPW_)                                                                                          \
  gemv_dot4_kernel<MT, KS_, LPW_><<<grid, block, 0, stream>>>(codes, packed, deq, rowsum, n, k, ep, y, acc_out); \
  return hipGetLastError()
  // loads per wave: exactly the lines of its K range where an instantiation
  // has that count (a longer list would issue loads that carry nothing)
#if BL_DOT4_EXACT_LPW
#define BL_DOT4_KS(KS_)                       \
  switch (lpw) {                              \
    case 1: BL_DOT4(KS_, 1);                  \
    case 2: BL_DOT4(KS_, 2);                  \
    case 3: BL_DOT4(KS_, 3);                  \
    case 4: BL_DOT4(KS_, 4);                  \
    case 5: BL_DOT4(KS_, 5);                  \
    case 6: BL_DOT4(KS_, 6);                  \
    case 7: BL_DOT4(KS_, 7);                  \
    case 8: BL_DOT4(KS_, 8);                  \
    default: BL_DOT4(KS_, 16);                \
  }
#else
#define BL_DOT4_KS(KS_)                       \
  if (lpw <= 4) { BL_DOT4(KS_, 4); }          \
  if (lpw <= 8) { BL_DOT4(KS_, 8); }          \
  BL_DOT4(KS_, 16);
#endif
  if (ks == 1) { BL_DOT4_KS(1) }
  if (ks == 2) { BL_DOT4_KS(2) }
  BL_DOT4_KS(4)
#undef BL_DOT4_KS
#undef BL_DOT4
}

// (codes through LDS: 4 token rows for m <= 4, 8 for 5 <= m <= 8, 16 for
// 9 <= m <= 16, where the wave areas fit: NW x MC x SPW x 256 bytes; measured
// on MI355X at 8 tokens, gate|up 5.05 us and down 4.16 us against 5.94 and 5.25
// with per-lane operand loads)
template <int RT, int NW, int SPW, bool ROPE = false>
hipError_t launch_cfg(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum, int m,
                      int n, int k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream,
                      const DecodeRope &rope = DecodeRope{}) {
  const int blocks = (n + 16 * RT - 1) / (16 * RT);
#define BL_DECODE_LAUNCH(MC_)                                                                          \
  do {                                                                                                       \
    if (k % 64 == 0)                                                                                         \
      gemv_decode_kernel<RT, NW, SPW, ROPE, MC_, true><<<dim3((unsigned)blocks), dim3(NW * 64), 0, stream>>>( \
          codes, packed, deq, rowsum, m, n, k, ep, y, acc_out, rope);                                        \
    else                                                                                                     \
      gemv_decode_kernel<RT, NW, SPW, ROPE, MC_, false><<<dim3((unsigned)blocks), dim3(NW * 64), 0,          \
                                                          stream>>>(codes, packed, deq, rowsum, m, n, k, ep, y, \
                                                                    acc_out, rope);                           \
  } while (0)
  if constexpr (BL_GEMV_LDS_CODES && NW * 16 * SPW * 256 + NW * RT * 1024 <= 160 * 1024) {
    if (m <= 4)
      BL_DECODE_LAUNCH(4);
    else if (m <= 8)
      BL_DECODE_LAUNCH(BL_GEMV_MC_5_8);
    else
      BL_DECODE_LAUNCH(16);
  } else {
    BL_DECODE_LAUNCH(0);
  }
#undef BL_DECODE_LAUNCH
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
#if BL_GEMV_FEW_WG_NW16
  // fewer row tiles than CUs: sixteen waves of at most two supersteps each,
  // so each CU keeps more loads in flight (measured on MI355X, down 2560 rows
  // at 4 tokens: 3.86 us against 4.12 with eight waves of four)
  if constexpr (RT == 1) {
    if (n / 16 < 256 && S > 4 * BL_GEMV_MIN_WAVES && S <= 2 * 16)
      return launch_cfg<RT, 16, 2>(codes, packed, deq, rowsum, m, n, k, ep, y, acc_out, stream);
  }
#endif
  if (S <= 4 * 8) return launch_cfg<RT, 8, 4>(codes, packed, deq, rowsum, m, n, k, ep, y, acc_out, stream);
  if (S <= 4 * 16) return launch_cfg<RT, 16, 4>(codes, packed, deq, rowsum, m, n, k, ep, y, acc_out, stream);
  const int blocks = (n + 16 * RT - 1) / (16 * RT);
  gemv_loop_kernel<RT, 16><<<dim3((unsigned)blocks), dim3(1024), 0, stream>>>(codes, packed, deq, rowsum, m, n, k, ep,
                                                                              y, acc_out);
  return hipGetLastError();
}

}  // namespace

bool gemv_decode_rope_supported(int64_t m, int64_t k, int n_heads, int n_kv, int hd) {
  const int64_t S = ((k >> 4) + 15) >> 4;
  return m >= 2 && m <= 16 && k % 16 == 0 && S <= 4 * 16 && hd > 0 && hd % 32 == 0 && n_heads > 0 && n_kv > 0;
}

// The cached decoder's q|k|v projection with RoPE and the cache append in its
// epilogue (2 to 16 tokens, n = (n_heads + 2 n_kv) hd rows)
hipError_t launch_gemv_decode_rope(const int8_t *codes, const uint8_t *packed, const float *deq,
                                   const int32_t *rowsum, int64_t m, int64_t k, const Epilogue &ep, float *y,
                                   int32_t *acc_out, const DecodeRope &rope, hipStream_t stream) {
  const int64_t n = (int64_t)(rope.n_heads + 2 * rope.n_kv) * rope.hd;
  if (!gemv_decode_rope_supported(m, k, rope.n_heads, rope.n_kv, rope.hd)) return hipErrorInvalidValue;
  const int S = ((int)(k >> 4) + 15) >> 4;
  if (S <= 4 * BL_GEMV_MIN_WAVES)
    return launch_cfg<2, BL_GEMV_MIN_WAVES, (4 * BL_GEMV_MIN_WAVES + BL_GEMV_MIN_WAVES - 1) / BL_GEMV_MIN_WAVES, true>(
        codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream, rope);
  if (S <= 4 * 8)
    return launch_cfg<2, 8, 4, true>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream, rope);
  return launch_cfg<2, 16, 4, true>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream, rope);
}

hipError_t launch_gemv_decode(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum,
                              int64_t m, int64_t n, int64_t k, const Epilogue &ep, float *y, int32_t *acc_out,
                              hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (m <= BL_GEMV_DOT4_MAX_M && k % 64 == 0 && k <= kDot4MaxK) {
    switch (m) {
      case 1: return launch_dot4_mt<1>(codes, packed, deq, rowsum, (int)n, (int)k, ep, y, acc_out, stream);
#if BL_GEMV_DOT4_MAX_M >= 2
      case 2: return launch_dot4_mt<2>(codes, packed, deq, rowsum, (int)n, (int)k, ep, y, acc_out, stream);
      case 3: return launch_dot4_mt<3>(codes, packed, deq, rowsum, (int)n, (int)k, ep, y, acc_out, stream);
      default: return launch_dot4_mt<4>(codes, packed, deq, rowsum, (int)n, (int)k, ep, y, acc_out, stream);
#else
      default: break;
#endif
    }
  }
  // two row tiles per workgroup above BL_GEMV_RT1_MAX_M tokens halve the code
  // bytes each weight byte needs, where that still leaves a workgroup per CU
  // (measured on MI355X at 8 and 16 tokens: gate|up 13824 rows 5.9 / 6.4 us
  // against 6.6 / 8.0 with one tile and 5.9 / 6.9 with four; down 2560 rows
  // 4.9 / 5.0 us with one tile against 6.2 / 6.2 with two)
  // 5 to 16 tokens on a tall matrix whose rows hold at most 16 supersteps of
  // 256 k: four row tiles per workgroup, one wave per superstep (measured on
  // MI355X, gate|up 13824 x 2560 at 16 tokens: 5.19 us with ten waves of one
  // superstep, against 5.61 with two row tiles of four waves, 5.80 with two of
  // eight waves, 5.82 with four tiles of eight waves and 5.37-5.40 with four
  // tiles of sixteen waves; at 8 tokens 4.89 against 5.03 us; at 2 and 4
  // tokens no faster than one tile of four waves)
  const int S = ((int)(k >> 4) + 15) >> 4;
  if (m > 4 && n / 64 >= 200 && S <= 16) {
    if (S <= 4) return launch_cfg<4, 4, 1>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
    if (S <= 6) return launch_cfg<4, 6, 1>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
    if (S <= 8) return launch_cfg<4, 8, 1>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
    if (S <= 10)
      return launch_cfg<4, 10, 1>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
    if (S <= 12)
      return launch_cfg<4, 12, 1>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
    return launch_cfg<4, 16, 1>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
  }
  if (m > BL_GEMV_RT1_MAX_M && n / 32 >= 256)
    return launch_rt<2>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
  return launch_rt<1>(codes, packed, deq, rowsum, (int)m, (int)n, (int)k, ep, y, acc_out, stream);
}

}  // namespace bl
