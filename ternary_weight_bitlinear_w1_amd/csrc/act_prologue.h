// Per-token activation quantization of one row by a workgroup of TH threads
// (256 unless stated): the prologue transforms of a BitNet b1.58 block, the
// max |v|, the fp64 sum of squares, the int8 codes and their row sum. Shared
// by the standalone quantization kernel and by the decode contraction that
// quantizes its own input. Codes and row sums do not depend on TH; deq does
// only through the order of the fp64 sum of squares, and at equal TH both
// produce the same deq bit for bit.
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
// Thread t visits float4 f = t, t + 256, ... of the row: pass 1 forms the
// normed input v (kept in registers when NV > 0), the fp32 max |v| and the fp64
// sum of squares of the pre-gain input; both are reduced wave-wise, then across
// the four waves in a fixed order. Pass 2 writes the codes (one 32-bit word per
// four codes) and their row sum.
//
// With NV > 0 the row's loads can be issued on their own (row_load) and used
// later (row_finish): vector memory operations of a wave complete in issue
// order, so a caller that also streams other data (the weights of a
// contraction) issues the row's loads first and waits for them alone. The
// workgroup barriers here wait for LDS operations only, never for loads still
// in flight.
#pragma once

#include <type_traits>

#include "common.h"

namespace bl {

constexpr int kQuantThreads = 256;

typedef ActSrc Src;


// The raw operands of elements 4f .. 4f+3 of one row, as loaded.
struct RawIn {
  float4 a;  // x (or the gate half, or the value head read)
  float4 b;  // up half (ReLU^2) or second summand (residual)
  float4 g;  // RMSNorm gain (1 when the gain is absent: multiplying by 1 is exact)
};

// rescale of four exact sums (less the code row sum), as the contraction does
__device__ __forceinline__ float4 part_rescale(const Src &s, v4i t, int rs, float dq, int c) {
  float4 y;
  y.x = rescale(t[0] - rs, dq, epi_gamma(s.part_ep, c));
  y.y = rescale(t[1] - rs, dq, epi_gamma(s.part_ep, c + 1));
  y.z = rescale(t[2] - rs, dq, epi_gamma(s.part_ep, c + 2));
  y.w = rescale(t[3] - rs, dq, epi_gamma(s.part_ep, c + 3));
  return y;
}

// Elements c .. c+3 of row r of a projection output given as split-K partial
// sums: the exact sums over the splits, less the row sum of the codes,
// rescaled as the contraction's own epilogue does.
__device__ __forceinline__ float4 part_load(const Src &s, int64_t r, int c) {
  const int32_t *p = s.part + r * s.ld + c;
  v4i t = *reinterpret_cast<const v4i *>(p);
  for (int j = 1; j < s.part_splits; ++j) t += *reinterpret_cast<const v4i *>(p + j * s.part_plane);
  return part_rescale(s, t, s.part_rowsum[r], s.part_deq[r], c);
}

// PART: the projection-output operand comes from split-K partial sums.
template <int MODE, bool PART = false>
__device__ __forceinline__ RawIn raw_load(const Src &s, int64_t r, int f) {
  RawIn v;
  const float *row = s.x + r * s.ld;
  constexpr bool kPartA = PART && MODE != ACT_RESID_RMSNORM;  // the residual form's projection operand is b
  if constexpr (MODE == ACT_GQA_RMSNORM) {
    // element e of the attention output reads value head (e / head_dim) / group
    const int e = 4 * f;
    const int head = e / s.head_dim, d = e - head * s.head_dim;
    const int col = s.gqa_offset + (head / s.group) * s.head_dim + d;
    if constexpr (kPartA) v.a = part_load(s, r, col);
    else v.a = *reinterpret_cast<const float4 *>(row + col);
  } else {
    if constexpr (kPartA) v.a = part_load(s, r, 4 * f);
    else v.a = *reinterpret_cast<const float4 *>(row + 4 * f);
  }
  if constexpr (MODE == BITLINEAR_ACT_RELU2_RMSNORM) {
    if constexpr (PART) v.b = part_load(s, r, s.k + 4 * f);
    else v.b = *reinterpret_cast<const float4 *>(row + s.k + 4 * f);
  }
  if constexpr (MODE == ACT_RESID_RMSNORM) {
    if constexpr (PART) v.b = part_load(s, r, 4 * f);
    else v.b = *reinterpret_cast<const float4 *>(s.x2 + r * s.ld + 4 * f);
  }
  if constexpr (MODE != BITLINEAR_ACT_ABSMAX) {
    // branch-free: without a gain, load a row of the input again and use 1
    // (from the partial sums when those replace x, which is then NULL)
    const bool has_gain = s.gain != nullptr;
    const float *again = kPartA ? reinterpret_cast<const float *>(s.part + r * s.ld) : row;
    const float4 g = *reinterpret_cast<const float4 *>((has_gain ? s.gain : again) + 4 * f);
    v.g = has_gain ? g : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
  }
  return v;
}

// pre-norm input from the raw operands (the residual form also stores it)
template <int MODE>
__device__ __forceinline__ float4 pre_of(const Src &s, int64_t r, int f, const RawIn &v, bool write_h) {
  if constexpr (MODE == BITLINEAR_ACT_RELU2_RMSNORM) {
    float4 o;
    float t;
    t = v.a.x > 0.0f ? v.a.x : 0.0f; o.x = __fmul_rn(__fmul_rn(t, t), v.b.x);
    t = v.a.y > 0.0f ? v.a.y : 0.0f; o.y = __fmul_rn(__fmul_rn(t, t), v.b.y);
    t = v.a.z > 0.0f ? v.a.z : 0.0f; o.z = __fmul_rn(__fmul_rn(t, t), v.b.z);
    t = v.a.w > 0.0f ? v.a.w : 0.0f; o.w = __fmul_rn(__fmul_rn(t, t), v.b.w);
    return o;
  } else if constexpr (MODE == ACT_RESID_RMSNORM) {
    float4 o;
    o.x = __fadd_rn(v.a.x, v.b.x); o.y = __fadd_rn(v.a.y, v.b.y);
    o.z = __fadd_rn(v.a.z, v.b.z); o.w = __fadd_rn(v.a.w, v.b.w);
    if (write_h) *reinterpret_cast<float4 *>(s.h_out + r * (int64_t)s.k + 4 * f) = o;
    return o;
  } else {
    return v.a;
  }
}

template <int MODE>
__device__ __forceinline__ float4 gain_of(const RawIn &v, float4 p) {
  if constexpr (MODE != BITLINEAR_ACT_ABSMAX) {
    p.x = __fmul_rn(v.g.x, p.x); p.y = __fmul_rn(v.g.y, p.y);
    p.z = __fmul_rn(v.g.z, p.z); p.w = __fmul_rn(v.g.w, p.w);
  }
  return p;
}

// round(v pre s) half to even. With s = fl(127 / fl(a pre)) and |v| <= a, the
// product y stays within 127.5 in magnitude (two roundings of relative size
// 2^-24), so the code lies in [-127, 127] without a clamp. pre is 1 except on
// rows whose max is below 2^-64.
//
// The rounding is one fp32 add: for |y| < 2^22, y + 1.5 * 2^23 lies in
// [2^23, 2^24), where the spacing of floats is 1, so the round-to-nearest-even
// add rounds y to the nearest integer, ties to even, and the result's bit
// pattern is 0x4B400000 + round(y) (two's complement, borrowing from the upper
// bits when round(y) < 0). Its low byte is therefore the int8 code, and a sum
// of such patterns modulo 2^32, less count * 0x4B400000, is the sum of the
// codes. (Non-finite inputs are outside the contract.)
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23
constexpr uint32_t kRoundBits = 0x4B400000u;
__device__ __forceinline__ uint32_t code_bits(float y) { return __float_as_uint(__fadd_rn(y, kRoundMagic)); }
// four code patterns -> the word of their low bytes (first code lowest)
__device__ __forceinline__ int pack_codes(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
  const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u), hi = __builtin_amdgcn_perm(b3, b2, 0x0c0c0400u);
  return (int)(lo | (hi << 16));
}

struct RowQuant {
  float deq;   // dequantization factor of the row's codes
  int rowsum;  // sum of the row's codes
};

// The loads of one row held in registers (NV float4 per thread).
template <int NV>
struct RowStage {
  RawIn in[NV];
};

// Column of the projection output that operand p (0: a, 1: the ReLU^2 form's
// up half) of elements 4f .. 4f+3 reads.
template <int MODE>
__device__ __forceinline__ int part_col(const Src &s, int f, int p) {
  if constexpr (MODE == ACT_GQA_RMSNORM) {
    const int e = 4 * f;
    const int head = e / s.head_dim, d = e - head * s.head_dim;
    return s.gqa_offset + (head / s.group) * s.head_dim + d;
  } else {
    return p ? s.k + 4 * f : 4 * f;
  }
}

// A row whose projection operand is given as split-K partial sums. The plain
// operands (residual summand, gain) are issued first; then the partial sums of
// every plane for every slot of the thread, so a row takes one memory round
// trip (beyond eight planes: two planes per round trip). Integer sums are
// exact, so the order of the planes does not matter.
template <int MODE, int NV, int TH>
__device__ __forceinline__ void row_load_part(const Src &s, int64_t r, RowStage<NV> &st) {
  constexpr int NP = MODE == BITLINEAR_ACT_RELU2_RMSNORM ? 2 : 1;
  const int nf = s.k >> 2;
  int col[NV][NP];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    int f = threadIdx.x + j * TH;
    f = f < nf ? f : 0;
#pragma unroll
    for (int p = 0; p < NP; ++p) col[j][p] = part_col<MODE>(s, f, p);
    if constexpr (MODE == ACT_RESID_RMSNORM)
      st.in[j].a = *reinterpret_cast<const float4 *>(s.x + r * s.ld + 4 * f);
    const bool has_gain = s.gain != nullptr;
    const float *again = reinterpret_cast<const float *>(s.part + r * s.ld);
    const float4 g = *reinterpret_cast<const float4 *>((has_gain ? s.gain : again) + 4 * f);
    st.in[j].g = has_gain ? g : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
  }
  const int32_t *base = s.part + r * s.ld;
  const int S = s.part_splits;
  v4i t[NV][NP];
  // Up to kPartStraight planes: every plane's loads issued before the first
  // sum, in straight-line code per plane count (a loop over a run-time count
  // waits for each round trip in turn). More planes: two per round trip.
  auto planes = [&](auto sc) {
    constexpr int SP = decltype(sc)::value;
    v4i u[SP][NV][NP];
#pragma unroll
    for (int sp = 0; sp < SP; ++sp)
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int p = 0; p < NP; ++p)
          u[sp][j][p] = *reinterpret_cast<const v4i *>(base + sp * s.part_plane + col[j][p]);
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        v4i a = u[0][j][p];
#pragma unroll
        for (int sp = 1; sp < SP; ++sp) a += u[sp][j][p];
        t[j][p] = a;
      }
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
    default: {
#pragma unroll
      for (int j = 0; j < NV; ++j)
#pragma unroll
        for (int p = 0; p < NP; ++p) t[j][p] = *reinterpret_cast<const v4i *>(base + col[j][p]);
      for (int sp = 1; sp < S; sp += 2) {
        // past the last plane the second load repeats plane sp and is not added
        const bool two = sp + 1 < S;
        const int64_t o0 = sp * s.part_plane, o1 = (two ? sp + 1 : sp) * s.part_plane;
        v4i u0[NV][NP], u1[NV][NP];
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            u0[j][p] = *reinterpret_cast<const v4i *>(base + o0 + col[j][p]);
            u1[j][p] = *reinterpret_cast<const v4i *>(base + o1 + col[j][p]);
          }
        const v4i zero = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
          for (int p = 0; p < NP; ++p) t[j][p] += u0[j][p] + (two ? u1[j][p] : zero);
      }
    }
  }
  const int rs = s.part_rowsum[r];
  const float dq = s.part_deq[r];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    if constexpr (MODE == ACT_RESID_RMSNORM) {
      st.in[j].b = part_rescale(s, t[j][0], rs, dq, col[j][0]);
    } else {
      st.in[j].a = part_rescale(s, t[j][0], rs, dq, col[j][0]);
      if constexpr (NP == 2) st.in[j].b = part_rescale(s, t[j][1], rs, dq, col[j][1]);
    }
  }
}

template <int MODE, int NV, bool PART = false, int TH = kQuantThreads>
__device__ __forceinline__ void row_load(const Src &s, int64_t r, RowStage<NV> &st) {
  static_assert(NV > 0, "register-resident rows only");
  if constexpr (PART) {
    row_load_part<MODE, NV, TH>(s, r, st);
  } else {
    const int nf = s.k >> 2;
    // every lane issues the same NV loads (past the row end it reloads element
    // 0, unused), so the number of loads in flight is known where they are used
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int f = threadIdx.x + j * TH;
      st.in[j] = raw_load<MODE, PART>(s, r, f < nf ? f : 0);
    }
  }
}

// All 256 threads of the workgroup call this for row r; `words` receives the
// codes (word f = codes 4f .. 4f + 3, low byte first) and may point to LDS or
// to global memory. The LDS arrays hold the cross-wave partials. Every thread
// returns the same deq and row sum; words in LDS are visible to the whole
// workgroup on return. NV = 0 streams the row twice instead of holding it.
template <int MODE, int NV, bool PART = false, int TH = kQuantThreads>
__device__ __forceinline__ RowQuant row_finish(const Src &s, int64_t r, float eps, const RowStage<(NV > 0 ? NV : 1)> &st,
                                               int *words, float *red_f, double *red_d, int *red_i) {
  constexpr bool kRms = MODE != BITLINEAR_ACT_ABSMAX;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nf = s.k >> 2;  // float4 per row

  float4 cache[NV > 0 ? NV : 1];
  float amax = 0.0f;
  double ss = 0.0;
  // ---- pass 1: normed input, max |v|, sum of squares of the pre-gain input
  auto visit1 = [&](int f, const RawIn &raw) -> float4 {
    const float4 p = pre_of<MODE>(s, r, f, raw, true);
    if (kRms) {
      // the square of an fp32 value is exact in fp64, so the fused form adds
      // the same product as a multiply then an add would
      ss = __fma_rn((double)p.x, (double)p.x, ss);
      ss = __fma_rn((double)p.y, (double)p.y, ss);
      ss = __fma_rn((double)p.z, (double)p.z, ss);
      ss = __fma_rn((double)p.w, (double)p.w, ss);
    }
    const float4 v = gain_of<MODE>(raw, p);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    return v;
  };
  if constexpr (NV > 0) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int f = tid + j * TH;
      if (f < nf) cache[j] = visit1(f, st.in[j]);
    }
  } else {
    for (int f = tid; f < nf; f += TH) (void)visit1(f, raw_load<MODE, PART>(s, r, f));
  }
  amax = wave_max(amax);
  if (kRms) ss = wave_sum(ss);
  if (lane == 0) {
    red_f[wave] = amax;
    red_d[wave] = ss;
  }
  lds_barrier();
  float a = red_f[0];
  double sum_sq = red_d[0];
#pragma unroll
  for (int w = 1; w < TH / 64; ++w) {
    a = fmaxf(a, red_f[w]);
    sum_sq += red_d[w];
  }

  // ---- pass 2: codes
  int rs = 0;
  if (a == 0.0f) {
    for (int f = tid; f < nf; f += TH) words[f] = 0;
  } else {
    // rows whose max is below 2^-64 are scaled by 2^64 first (exact), which
    // keeps 127 / a finite and changes no code the unscaled steps reach
    const float pre = a < 0x1p-64f ? 0x1p64f : 1.0f;
    const float sc = 127.0f / __fmul_rn(a, pre);
    uint32_t rb = 0;  // sum of code patterns (mod 2^32)
    int nq = 0;       // codes in rb
    auto emit = [&](int f, float4 v) {
      const uint32_t b0 = code_bits(__fmul_rn(__fmul_rn(v.x, pre), sc));
      const uint32_t b1 = code_bits(__fmul_rn(__fmul_rn(v.y, pre), sc));
      const uint32_t b2 = code_bits(__fmul_rn(__fmul_rn(v.z, pre), sc));
      const uint32_t b3 = code_bits(__fmul_rn(__fmul_rn(v.w, pre), sc));
      rb += b0 + b1 + b2 + b3;
      nq += 4;
      words[f] = pack_codes(b0, b1, b2, b3);
    };
    if constexpr (NV > 0) {
      if (pre == 1.0f) {  // (v 1 = v exactly: one multiply per element)
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int f = tid + j * TH;
          if (f < nf) {
            const float4 v = cache[j];
            const uint32_t b0 = code_bits(__fmul_rn(v.x, sc)), b1 = code_bits(__fmul_rn(v.y, sc));
            const uint32_t b2 = code_bits(__fmul_rn(v.z, sc)), b3 = code_bits(__fmul_rn(v.w, sc));
            rb += b0 + b1 + b2 + b3;
            nq += 4;
            words[f] = pack_codes(b0, b1, b2, b3);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int f = tid + j * TH;
          if (f < nf) emit(f, cache[j]);
        }
      }
    } else {
      for (int f = tid; f < nf; f += TH) {
        const RawIn raw = raw_load<MODE, PART>(s, r, f);
        emit(f, gain_of<MODE>(raw, pre_of<MODE>(s, r, f, raw, false)));
      }
    }
    rs = (int)(rb - (uint32_t)nq * kRoundBits);
  }
  rs = wave_sum(rs);
  if (lane == 0) red_i[wave] = rs;
  lds_barrier();
  RowQuant out;
  out.rowsum = 0;
#pragma unroll
  for (int w = 0; w < TH / 64; ++w) out.rowsum += red_i[w];
  out.deq = 0.0f;
  if (a != 0.0f) {
    if (kRms) {
      const double ms = sum_sq / (double)s.k;
      const double rr = sqrt(ms + (double)eps);
      out.deq = (float)(((double)a / 127.0) / rr);
    } else {
      out.deq = a / 127.0f;
    }
  }
  return out;
}

template <int MODE, int NV, bool PART = false, int TH = kQuantThreads>
__device__ __forceinline__ RowQuant quant_row(const Src &s, int64_t r, float eps, int *words, float *red_f,
                                              double *red_d, int *red_i) {
  RowStage<(NV > 0 ? NV : 1)> st;
  if constexpr (NV > 0) row_load<MODE, NV, PART, TH>(s, r, st);
  return row_finish<MODE, NV, PART, TH>(s, r, eps, st, words, red_f, red_d, red_i);
}

}  // namespace bl
