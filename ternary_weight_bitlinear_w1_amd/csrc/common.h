// Internal declarations shared by the gfx950 kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bitlinear.h"

namespace bl {

// Sets the reason bitlinear_last_error() reports on this thread; returns s.
bitlinear_status report_error(bitlinear_status s, const char *reason);

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- epilogue
// Per-column weight scales of a (possibly fused) projection: column j uses
// gamma[s] for seg_end[s-1] <= j < seg_end[s]; n_seg <= BITLINEAR_MAX_SEGMENTS.
struct Epilogue {
  float gamma[BITLINEAR_MAX_SEGMENTS];
  int32_t seg_end[BITLINEAR_MAX_SEGMENTS];
  int32_t n_seg;
  int32_t blocks32;  // every segment end is a multiple of 32: gamma is constant per 32 columns
  // NULL, or the segments' fp64 gammas in device memory (as the weight pass
  // writes them); they replace gamma[], rounded to fp32
  const double *gamma_dev;
};

// A kernel's view of its epilogue: device-side gammas read and rounded once.
__device__ __forceinline__ Epilogue resolve_gamma(const Epilogue &in) {
  Epilogue e = in;
  if (e.gamma_dev) {
#pragma unroll
    for (int s = 0; s < BITLINEAR_MAX_SEGMENTS; ++s)
      if (s < e.n_seg) e.gamma[s] = (float)e.gamma_dev[s];
  }
  return e;
}

__device__ __forceinline__ float epi_gamma(const Epilogue &ep, int n) {
  float g = ep.gamma[0];
#pragma unroll
  for (int s = 1; s < BITLINEAR_MAX_SEGMENTS; ++s)
    if (s < ep.n_seg && n >= ep.seg_end[s - 1]) g = ep.gamma[s];
  return g;
}

// nearest bfloat16 of a finite float (its upper 16 bits), ties to an even last kept bit
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t kept = u >> 16, dropped = u & 0xFFFFu;
  return kept + ((dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) ? 1u : 0u);
}

// y = fl32(fl32((float)acc * deq) * gamma); acc is the exact int32 sum.
__device__ __forceinline__ float rescale(int acc, float deq, float gamma) {
  const float t = __fmul_rn((float)acc, deq);
  return __fmul_rn(t, gamma);
}

// ---------------------------------------------------------------- reductions
// Cross-lane sums and maxima that leave the same bits in every lane taking
// part: each step combines a value with its partner's (a + b = b + a), in a
// fixed order, so results repeat run to run. Within a row of 16 lanes, DPP:
// lane ^ 1 and lane ^ 2 (quad permutes), the partner quad of the half row
// (row_half_mirror, 7 - lane) and the partner half (row_mirror, 15 - lane).
// Across the four rows: v_permlane16_swap (rows 0|1, 2|3), then
// v_permlane32_swap (the two halves); with both operands the same value the
// two results hold a lane's value and its partner's, in the same order in
// both lanes.
template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {  // the two 32-bit halves
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)dpp<CTRL>((int)(uint32_t)u), hi = (uint32_t)dpp<CTRL>((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// Workgroup barrier that orders LDS traffic only: outstanding global loads
// keep flowing across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maximum
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <typename T>
__device__ __forceinline__ T lanes8_sum(T v) {  // lanes 8 g .. 8 g + 7
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  return v + dpp<kDppHalfMirror>(v);
}
template <typename T>
__device__ __forceinline__ T row16_sum(T v) {  // lanes 16 g .. 16 g + 15
  v = lanes8_sum(v);
  return v + dpp<kDppMirror>(v);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kDppXor1>(v));
  v = fmaxf(v, dpp<kDppXor2>(v));
  v = fmaxf(v, dpp<kDppHalfMirror>(v));
  return fmaxf(v, dpp<kDppMirror>(v));
}
__device__ __forceinline__ uint32_t bits_of(int v) { return (uint32_t)v; }
__device__ __forceinline__ uint32_t bits_of(float v) { return __float_as_uint(v); }
__device__ __forceinline__ int from_bits(uint32_t b, int) { return (int)b; }
__device__ __forceinline__ float from_bits(uint32_t b, float) { return __uint_as_float(b); }
template <typename T>
__device__ __forceinline__ T rows_sum(T v) {  // the four rows (values equal within each row)
  const auto a = __builtin_amdgcn_permlane16_swap(bits_of(v), bits_of(v), false, false);
  v = from_bits(a[0], v) + from_bits(a[1], v);
  const auto b = __builtin_amdgcn_permlane32_swap(bits_of(v), bits_of(v), false, false);
  return from_bits(b[0], v) + from_bits(b[1], v);
}
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Wave64 results in every lane.
__device__ __forceinline__ float wave_max(float v) { return rows_max(row16_max(v)); }
__device__ __forceinline__ int wave_sum(int v) { return rows_sum(row16_sum(v)); }
// fp64: the same steps, moving the two 32-bit halves
__device__ __forceinline__ double rows_sum(double v) {
  auto join = [](uint32_t lo, uint32_t hi) { return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo)); };
  uint64_t u = (uint64_t)__double_as_longlong(v);
  const auto al = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto ah = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  v = join(al[0], ah[0]) + join(al[1], ah[1]);
  u = (uint64_t)__double_as_longlong(v);
  const auto bl_ = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto bh = __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  return join(bl_[0], bh[0]) + join(bl_[1], bh[1]);
}
__device__ __forceinline__ double wave_sum(double v) { return rows_sum(row16_sum(v)); }

// ---------------------------------------------------------------- launchers
// Implemented next to their kernels; all enqueue on `stream` and return the
// hipGetLastError() of the launch.
hipError_t launch_quant_acts(int mode, const float *x, const float *x2, int64_t ld_x, int64_t m, int64_t k,
                             const float *gain, float eps, int gqa_offset, int head_dim, int group,
                             float *h_out, int8_t *codes, float *deq, int32_t *rowsum, hipStream_t stream);
struct ActSrc;
// The same, with every source field given (partial-sum operands included).
hipError_t launch_quant_acts_src(int mode, const ActSrc &src, int64_t m, float eps, int8_t *codes, float *deq,
                                 int32_t *rowsum, hipStream_t stream);
hipError_t launch_code_rowsum(const int8_t *codes, int64_t m, int64_t k, int32_t *rowsum, hipStream_t stream);
hipError_t launch_add(const float *a, const float *b, float *out, int64_t count, hipStream_t stream);
// y[m][inter] = fl32(fl32(max(g, 0)^2) * u), gu = [m][g | u], inter % 4 == 0
hipError_t launch_relu2_glu(const float *gu, int64_t m, int64_t inter, float *y, hipStream_t stream);

// Absmean ternarization of a master matrix [n][k] whose rows form n_seg
// consecutive segments (row_end[j] exclusive, ascending, row_end[n_seg - 1] =
// n, 1 <= n_seg <= BITLINEAR_MAX_SEGMENTS), one gamma per segment: one launch
// reduces every segment's partial sums, one forms the gammas, one ternarizes
// and packs the whole matrix. partials holds absmean_partials() doubles.
size_t absmean_partials(int64_t k, const int64_t *row_end, int n_seg);
hipError_t launch_absmean(const float *w, int64_t k, const int64_t *row_end, int n_seg, double *partials,
                          double *gamma_out, hipStream_t stream);
hipError_t launch_ternarize_pack(const float *w, int64_t k, const int64_t *row_end, int n_seg, const double *gamma,
                                 uint8_t *packed, hipStream_t stream);
// the same two passes over bfloat16 masters (bit patterns, widened exactly)
hipError_t launch_absmean_bf16(const uint16_t *w, int64_t k, const int64_t *row_end, int n_seg, double *partials,
                               double *gamma_out, hipStream_t stream);
hipError_t launch_ternarize_pack_bf16(const uint16_t *w, int64_t k, const int64_t *row_end, int n_seg,
                                      const double *gamma, uint8_t *packed, hipStream_t stream);
// One token (m = 1) of the online mode straight from the masters: the codes,
// deq and row sum of the token, the masters [n][k], and ep with gamma_dev set
// to the segments' gammas (as launch_absmean writes them). Equal bit for bit
// to ternarize + the packed forward. Supported where online_dot_supported().
bool online_dot_supported(int64_t n, int64_t k, bool bf16);
hipError_t launch_online_dot(const int8_t *codes, const float *deq, const int32_t *rowsum, const float *w, int64_t n,
                             int64_t k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream);
hipError_t launch_online_dot_bf16(const int8_t *codes, const float *deq, const int32_t *rowsum, const uint16_t *w,
                                  int64_t n, int64_t k, const Epilogue &ep, float *y, int32_t *acc_out,
                                  hipStream_t stream);
hipError_t launch_copy_gamma(const double *src, double *dst, hipStream_t stream);
hipError_t launch_validate_packed(const uint8_t *packed, int64_t n, int64_t k, int64_t *n_bad,
                                  hipStream_t stream);

// Prefill contraction. For shapes with few output tiles (small m) it splits K
// into gemm_prefill_splits() ranges when split_ws (gemm_prefill_workspace_bytes()
// bytes) is given, and adds the ranges' exact partial sums in a second kernel.
#ifndef BL_SPLIT_TARGET
#define BL_SPLIT_TARGET 256
#endif
#ifndef BL_SPLIT_BYTES_RATIO
#define BL_SPLIT_BYTES_RATIO 2
#endif
constexpr int64_t kSplitMinTiles = 256;                         // split only below this many output tiles
constexpr int64_t kSplitTarget = BL_SPLIT_TARGET;               // aim for about this many work items
constexpr int64_t kSplitBytesPerWeightByte = BL_SPLIT_BYTES_RATIO;  // partial sums vs packed weight bytes
int gemm_prefill_splits(int64_t m, int64_t n, int64_t k);
size_t gemm_prefill_workspace_bytes(int64_t m, int64_t n, int64_t k);
// splits_left: NULL, or receives the number S of K ranges whose partial sums
// were left in split_ws (part[s][m][n], int32; 1 = y was written) for the
// caller to add (the finish kernel is then not launched).
// res: NULL, or [m][n] added to y by the finish kernel.
hipError_t launch_gemm_prefill(const int8_t *codes, const uint8_t *packed, const float *deq,
                               const int32_t *rowsum, int64_t m, int64_t n, int64_t k, const Epilogue &ep,
                               float *y, int32_t *acc_out, int32_t *split_ws, hipStream_t stream,
                               int *splits_left = nullptr, const float *res = nullptr);
// y = [res +] rescale(sum_s part[s] - rowsum, deq, gamma), [m][n], n % 4 == 0
hipError_t launch_splitk_finish(const int32_t *part, int splits, const float *deq, const int32_t *rowsum, int64_t m,
                                int64_t n, const Epilogue &ep, float *y, int32_t *acc_out, const float *res,
                                hipStream_t stream);
// Gated prefill contraction: packed [gate; up] (2 inter rows), gamma[0] gate,
// gamma[1] up; y[m][j] = fl32(fl32(max(g, 0)^2) * u), [m][inter].
bool gemm_glu_supported(int64_t m, int64_t inter, int64_t k);
hipError_t launch_gemm_glu(const int8_t *codes, const uint8_t *packed, const float *deq, const int32_t *rowsum,
                           int64_t m, int64_t inter, int64_t k, const Epilogue &ep, float *y, hipStream_t stream);
// RoPE and the cache append in a decode projection's epilogue (the cached
// decoder's q|k|v rows: n_heads q heads, n_kv k heads, n_kv v heads of hd)
struct DecodeRope {
  const int64_t *slot = nullptr, *pos = nullptr;
  const float2 *cs = nullptr;  // [m][hd/2] (cosine, sine) of each token's rotated pairs (launch_rope_gather)
  uint16_t *kc = nullptr, *vc = nullptr;
  int64_t n_slots = 0, tmax = 0;
  int n_heads = 0, n_kv = 0, hd = 0;
};
bool gemv_decode_rope_supported(int64_t m, int64_t k, int n_heads, int n_kv, int hd);
hipError_t launch_gemv_decode_rope(const int8_t *codes, const uint8_t *packed, const float *deq,
                                   const int32_t *rowsum, int64_t m, int64_t k, const Epilogue &ep, float *y,
                                   int32_t *acc_out, const DecodeRope &rope, hipStream_t stream);
hipError_t launch_gemv_decode(const int8_t *codes, const uint8_t *packed, const float *deq,
                              const int32_t *rowsum, int64_t m, int64_t n, int64_t k, const Epilogue &ep,
                              float *y, int32_t *acc_out, hipStream_t stream);

// act-quant prologues beyond the public bitlinear_act_mode values
enum { ACT_RESID_RMSNORM = 16, ACT_GQA_RMSNORM = 17 };

// ---------------------------------------------------------------- fused decode
// A decode projection that quantizes its own input (decode_fused.hip).
enum { FUSED_EPI_PLAIN = 0, FUSED_EPI_RESID = 1, FUSED_EPI_RELU2 = 2, FUSED_EPI_ROPE = 3 };
// Up to two tokens: from three on, a quantization launch plus the
// contraction is faster than every workgroup quantizing all the tokens' rows
// (a decode step of the 30-layer model at 4096 positions, measured: fused
// 1.12 / 1.57 / 1.86 / 2.22 ms against 1.39 / 1.60 / 1.66 / 1.82 ms for one to
// four sequences).
constexpr int kFusedMaxM = 2;

struct ActSrc {
  const float *x;   // input rows, row stride ld
  const float *x2;  // residual prologue: second operand
  int64_t ld;
  int k;            // input features
  const float *gain;
  int gqa_offset, head_dim, group;
  float *h_out;     // residual prologue: receives x + x2 ([m][k]); the fused decode takes no residual prologue
  // The projection-output operand (x2 in the residual prologue, x otherwise)
  // given as split-K partial sums instead of fp32 rows (standalone
  // quantization kernel only): element (r, c) is
  //   fl32(fl32((float)(sum_s part[s][r][c] - part_rowsum[r]) * part_deq[r]) * gamma(c)),
  // with row stride ld and part_plane elements per split; part_ep.gamma_dev is NULL.
  const int32_t *part;
  int part_splits;
  int64_t part_plane;
  const int32_t *part_rowsum;
  const float *part_deq;
  Epilogue part_ep;
};

struct FusedDecode {
  ActSrc src;
  float eps;
  int m;               // tokens, 1 .. kFusedMaxM
  const uint8_t *w;    // packed weights [n][k/4]
  int n;
  Epilogue ep;
  float *y;            // [m][n]: required by the plain form, optional (trace) otherwise
  int32_t *acc_out;    // [m][n] exact sums, optional
  const float *res;    // residual form: [m][n] input added to y
  float *out2;         // residual form: [m][n] res + y
  float *mi;           // ReLU^2 form: [m][n/2]
  int8_t *codes_out;   // optional [m][k] codes of the input
  float *deq_out;      // optional [m]
  // RoPE form (q|k|v rows: n_heads q heads, n_kv k heads, n_kv v heads of hd):
  // y gets q and k rotated at pos[t] and v as is; k and v also go to the
  // bfloat16 caches [n_slots][n_kv][tmax][hd] at (slot[t], pos[t]) when both
  // are in range
  const int64_t *slot, *pos;
  const float2 *cs;  // [m][hd/2] (cosine, sine) of each token's rotated pairs (launch_rope_gather)
  uint16_t *kc, *vc;
  int64_t n_slots, tmax;
  int n_heads, n_kv, hd;
};

// The head (head.hip): final norm to bfloat16, the bfloat16 lm_head, and the
// embedding gather of the tied table.
bool lm_head_supported(int64_t k);
hipError_t launch_final_norm(const float *x, int64_t m, int64_t k, const float *gain, float eps, uint16_t *o,
                             hipStream_t stream);
hipError_t launch_lm_head(const uint16_t *o, int64_t m, int64_t k, const uint16_t *w, int64_t n, float *y,
                          hipStream_t stream);
hipError_t launch_embed(const int64_t *ids, int64_t m, const uint16_t *table, int64_t vocab, int64_t k, float *x,
                        hipStream_t stream);

// Measurement probes (probes.hip): a coalesced 16-byte read stream (grid <= 0:
// one thread per 8 loads) and independent int8 MFMA chains (256-thread
// workgroups, iters x 8 v_mfma_i32_32x32x32_i8 per wave).
hipError_t launch_probe_read(const void *src, int64_t bytes, uint32_t *sink, int64_t grid, hipStream_t stream);
hipError_t launch_probe_mfma(int iters, int64_t workgroups, bool varied, int32_t *sink, hipStream_t stream);

// RoPE, the bfloat16 KV cache and causal attention (attention.hip).
bool attention_supported(int n_heads, int n_kv, int hd);
int attention_splits(int64_t tmax);
size_t attention_workspace_floats(int64_t m, int n_heads, int64_t tmax);
// tab: the rotary table [n_pos][hd/2] (cosine, sine); positions outside
// [0, n_pos) take row 0
hipError_t launch_rope(float *x, int64_t m, int64_t ld, int64_t col0, int n_heads, int hd, const int64_t *pos,
                       const float2 *tab, int64_t n_pos, hipStream_t stream);
// every token's rows of the rotary table, cs [m][hd/2]
hipError_t launch_rope_gather(const int64_t *pos, int64_t m, int hd, const float2 *tab, int64_t n_pos, float2 *cs,
                              hipStream_t stream);
// RoPE and the cache append on a q|k|v row (q heads, then k heads, then v
// heads), one launch, with the rows from launch_rope_gather
hipError_t launch_rope_append(float *qkv, int64_t m, int64_t ld, int n_heads, int n_kv, int hd, const int64_t *slot,
                              const int64_t *pos, const float2 *cs, uint16_t *kc, uint16_t *vc, int64_t n_slots,
                              int64_t tmax, hipStream_t stream);
hipError_t launch_kv_append(const float *k, const float *v, int64_t m, int64_t ld, int n_kv, int hd,
                            const int64_t *slot, const int64_t *pos, uint16_t *kc, uint16_t *vc, int64_t n_slots,
                            int64_t tmax, hipStream_t stream);
hipError_t launch_attention(const float *q, int64_t m, int64_t ldq, int n_heads, int n_kv, int hd,
                            const uint16_t *kc, const uint16_t *vc, int64_t n_slots, int64_t tmax,
                            const int64_t *slot, const int64_t *pos, float *out, int64_t ldo, float *ws,
                            hipStream_t stream);

// Five codes per byte (base3.hip): repacking, and the 1..4-token contraction.
bool gemv_b3_supported(int64_t m, int64_t k);
hipError_t launch_pack_base3(const uint8_t *packed, int64_t n, int64_t k, uint8_t *out, hipStream_t stream);
hipError_t launch_gemv_b3(const int8_t *codes, const uint8_t *w, const float *deq, int64_t m, int64_t n, int64_t k,
                          const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream);

bool fused_decode_supported(int64_t m, int64_t k);
hipError_t launch_gemv_fused(int mode, int epi, const FusedDecode &a, hipStream_t stream);

}  // namespace bl
