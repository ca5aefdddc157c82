// Absmean ternarization of fp32 or bfloat16 master weights and four-to-a-byte packing
// (gfx950). Offline step of the packed checkpoint mode: the nnterp "BitNet
// b1.58" page, "The projections quantize their inputs and weights" (weights
// rounded to {-1, 0, 1} * mean|W|, stored four to a byte with a weight_scale)
// and "The two checkpoints"; the model card's "Model Details" (absmean).
//
// gamma = mean|W| is reduced in fp64 in a fixed order: each of G workgroups
// (G depends only on the element count) sums a fixed contiguous slice, thread
// by thread and then by a fixed wave/block tree; one workgroup then adds the G
// partials in a fixed tree. Results are bit-identical run to run.
// Codes compare |W| with gamma / 2 in fp64, which is exact; a tie gives 0.
// Packing: word g of a row holds codes 16g..16g+15; code 16g + 4t + b is the
// field u = c + 1 at bits 8b + 2t (see the layout note in bitlinear.h).
#include "common.h"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxPartials = 2048;
constexpr int64_t kPerBlock = 1 << 14;  // elements per partial, at least
constexpr int kUnroll = 8;              // float4 loads in flight per thread

__device__ __forceinline__ double block_sum(double v, double *red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) t += red[w];
  return t;
}

// Master weights are fp32 or bfloat16 (the bf16 checkpoint of "The two
// checkpoints"). A 16-byte load holds E of them; a bfloat16 value widens to
// fp32 exactly (its bits are the top half of the fp32's).
template <typename T>
struct Master;
template <>
struct Master<float> {
  static constexpr int E = 4;
  __device__ static float at(const v4i &r, int e) { return __int_as_float(r[e]); }
};
template <>
struct Master<uint16_t> {
  static constexpr int E = 8;
  __device__ static float at(const v4i &r, int e) {
    const uint32_t w = (uint32_t)r[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
};

// The segments of one launch: segment j is rows [row_end[j - 1], row_end[j])
// (elements [lo_j, hi_j) = rows times k), cut into partial slices of per[j]
// elements (a multiple of 16) numbered from part_lo[j]. A segment's slices
// depend only on its own element count, so its partial sums and gamma are the
// same whether it is reduced alone or beside other segments.
struct SegSpan {
  int n;
  int64_t k;
  int64_t row_end[BITLINEAR_MAX_SEGMENTS];
  int64_t per[BITLINEAR_MAX_SEGMENTS];
  int part_lo[BITLINEAR_MAX_SEGMENTS + 1];
  __device__ int64_t elem_lo(int j) const { return (j ? row_end[j - 1] : 0) * k; }
  __device__ int64_t elem_hi(int j) const { return row_end[j] * k; }
};

// partials[b] = sum |w| over the elements of slice b of its segment
template <typename T>
__global__ __launch_bounds__(kThreads) void absmean_partial_kernel(const T *__restrict__ w, SegSpan sp,
                                                                   double *__restrict__ partials) {
  constexpr int E = Master<T>::E;
  __shared__ double red[kThreads / 64];
  const int b = blockIdx.x;
  int j = 0;
  while (j + 1 < sp.n && b >= sp.part_lo[j + 1]) ++j;
  const int64_t lo = sp.elem_lo(j) + (int64_t)(b - sp.part_lo[j]) * sp.per[j];
  const int64_t hi = lo + sp.per[j] < sp.elem_hi(j) ? lo + sp.per[j] : sp.elem_hi(j);
  // thread t adds elements t, t + 256, ... (in 16-byte units) of the slice in
  // order; kUnroll loads are issued before their sums
  double s = 0.0;
  for (int64_t i0 = lo + E * (int64_t)threadIdx.x; i0 < hi; i0 += E * kThreads * kUnroll) {
    v4i v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + E * (int64_t)kThreads * u;
      v[u] = i < hi ? *reinterpret_cast<const v4i *>(w + i) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int e = 0; e < E; ++e) s += fabs((double)Master<T>::at(v[u], e));
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) partials[b] = s;
}

// gamma[j] = (sum of segment j's partials, in slice order) / its element count
// (0 for an empty segment); one workgroup per segment
__global__ __launch_bounds__(kThreads) void absmean_final_kernel(const double *__restrict__ partials, SegSpan sp,
                                                                 double *__restrict__ gamma) {
  __shared__ double red[kThreads / 64];
  const int j = blockIdx.x;
  const int p0 = sp.part_lo[j], np = sp.part_lo[j + 1] - p0;
  const int64_t count = sp.elem_hi(j) - sp.elem_lo(j);
  // thread t adds partials t, t + 256, ... in order; all its loads (clamped
  // into range, at most kMaxPartials / 256) are issued before the first sum,
  // and the ones past the end add 0
  constexpr int kLoads = kMaxPartials / kThreads;
  double s = 0.0;
  if (np > 0) {
    double v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int i = threadIdx.x + kThreads * u;
      v[u] = partials[p0 + (i < np ? i : np - 1)];
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
      if ((int)threadIdx.x + kThreads * u < np) s += v[u];
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) gamma[j] = count > 0 ? s / (double)count : 0.0;
}

// one thread per packed 32-bit word (16 codes); word i lies in segment j when
// it precedes the segment's last row's end (row_end[j] k / 16 words)
template <typename T>
__global__ __launch_bounds__(kThreads) void ternarize_pack_kernel(const T *__restrict__ w, int64_t words,
                                                                  SegSpan sp, const double *__restrict__ gamma,
                                                                  uint32_t *__restrict__ packed) {
  constexpr int E = Master<T>::E;
  const int64_t wpr = sp.k / 16;
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < words; i += (int64_t)gridDim.x * kThreads) {
    int j = 0;
    while (j + 1 < sp.n && i >= sp.row_end[j] * wpr) ++j;
    const double half = 0.5 * gamma[j];
    const v4i *src = reinterpret_cast<const v4i *>(w + 16 * i);
    v4i raw[16 / E];
#pragma unroll
    for (int u = 0; u < 16 / E; ++u) raw[u] = src[u];
    uint32_t word = 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float v = Master<T>::at(raw[t / E], t % E);
      const uint32_t c = fabs((double)v) > half ? (v > 0.0f ? 2u : 0u) : 1u;
      word |= c << (8 * (t & 3) + 2 * (t >> 2));
    }
    packed[i] = word;
  }
}

// ---------------------------------------------------------------------------
// One-token online contraction: y[n] = rescale(sum_k q_k u(w[n][k]) - sum_k q_k,
// deq, fl32(gamma_j)), u = c + 1 the field of the ternary code that the
// ternarize pass would store for w[n][k] under gamma_j of row n's segment, so
// the result is that of ternarize + the packed forward, bit for bit, without
// writing and re-reading the packed codes. The masters are read straight from
// HBM once more (the mean|W| pass read them first).
//
// The code test |w| > gamma / 2 is taken in fp32 against h = gamma / 2 rounded
// down to fp32: for an fp32 |w|, |w| > gamma / 2 exactly when |w| > h (no fp32
// lies strictly between h and gamma / 2), so it agrees with the fp64 test of
// the ternarize pass; a NaN compares false in both.
//
// Shape as the packed one-token kernel: lane l reads the 16-byte piece l % 8 of
// each 128-byte line of row l / 8 (E weights: 8 bfloat16 or 4 fp32), 8 rows per
// wave, KS waves splitting a row's lines, the token's codes in LDS; four
// fields at a time go into one v_dot4_i32_i8 against the matching code dword.
constexpr int kOnlineMaxK = 8192;
constexpr int kOnlineMaxLines = 32;  // 128-byte lines per wave

typedef short short2 __attribute__((ext_vector_type(2)));

// The fields u = c + 1 (bytes, element e in byte e) of four bfloat16 weights,
// elements 0, 1 in da (low half first) and 2, 3 in db. For a bfloat16 w and an
// fp32 h >= 0, |w| > h exactly when w's 15 magnitude bits exceed h's top 15
// (floats of one sign order as their bits, and w's low 16 bits are zero), so
// h16 - |w|16 is negative exactly where the code is nonzero; the code's sign
// is w's sign bit. With G and S the 0/1 bytes of those two tests,
// u = 1 + G - 2 (G & S), which never borrows across bytes.
__device__ __forceinline__ uint32_t bf16_fields4(uint32_t da, uint32_t db, short2 hh) {
  const short2 ta = hh - __builtin_bit_cast(short2, da & 0x7fff7fffu);
  const short2 tb = hh - __builtin_bit_cast(short2, db & 0x7fff7fffu);
  constexpr uint32_t kHighBytes = 0x07050301u;  // byte 1 and 3 of each source, da first
  const uint32_t g = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, tb), __builtin_bit_cast(uint32_t, ta),
                                           kHighBytes) & 0x80808080u;
  const uint32_t s = __builtin_amdgcn_perm(db, da, kHighBytes) & 0x80808080u;
  return 0x01010101u + (g >> 7) - ((g & s) >> 6);
}

template <typename T, int KS, int LPW>
__global__ __launch_bounds__(256) void online_dot_kernel(const int8_t *__restrict__ codes, const float *__restrict__ deq,
                                                         const int32_t *__restrict__ rowsum, const T *__restrict__ w,
                                                         int N, int K, Epilogue ep_in, float *__restrict__ Y,
                                                         int32_t *__restrict__ acc_out) {
  constexpr int E = Master<T>::E;
  constexpr int RG = 4 / KS;  // row groups of 8 rows per workgroup
  constexpr int kCodeLoads = kOnlineMaxK / 16 / kThreads;
  __shared__ __attribute__((aligned(16))) int8_t sc[kOnlineMaxK];
  __shared__ int red[KS][RG][8];
  const Epilogue ep = resolve_gamma(ep_in);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ks = wave % KS, rg = wave / KS;
  const int n = blockIdx.x * 8 * RG + rg * 8 + (lane >> 3);
  const int p = lane & 7;
  const int rowb = K * (int)sizeof(T);  // bytes per master row (a multiple of 32)
  const int L = (rowb + 127) >> 7;      // 128-byte lines per row, the last may be partial
  const int l_lo = L * ks / KS, l_hi = L * (ks + 1) / KS;
  const int nc = n < N ? n : N - 1;

  // loads in issue order: the token's codes (L2), then the masters (HBM); a
  // piece past the row's end reloads the lane's first piece, unused
  v4i cw[kCodeLoads];
#pragma unroll
  for (int j = 0; j < kCodeLoads; ++j) {
    const int i = threadIdx.x + kThreads * j;
    cw[j] = *reinterpret_cast<const v4i *>(codes + (16 * i < K ? 16 * i : 0));
  }
  __builtin_amdgcn_sched_barrier(0);
  const char *row = reinterpret_cast<const char *>(w) + (int64_t)nc * rowb;
  v4i wv[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int off = 128 * (l_lo + i) + 16 * p;
    const bool use = l_lo + i < l_hi && off < rowb;
    wv[i] = *reinterpret_cast<const v4i *>(row + (use ? off : 16 * p < rowb ? 16 * p : 0));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kCodeLoads; ++j) {
    const int i = threadIdx.x + kThreads * j;
    if (16 * i < K) *reinterpret_cast<v4i *>(sc + 16 * i) = cw[j];
  }
  lds_barrier();

  // row n's segment and its threshold
  int seg = 0;
#pragma unroll
  for (int q = 1; q < BITLINEAR_MAX_SEGMENTS; ++q)
    if (q < ep.n_seg && nc >= ep.seg_end[q - 1]) seg = q;
  const float h = __double2float_rd(0.5 * ep_in.gamma_dev[seg]);
  // bfloat16 masters: |w| > h on the 15 magnitude bits against h's top 15
  // (a NaN threshold, from NaN masters, lets nothing pass, as in fp)
  const uint32_t h16 = h != h ? 0x7fffu : (__float_as_uint(h) >> 16) & 0x7fffu;
  const short2 hh = {(short)h16, (short)h16};

  // Branch-free: a piece past the row's end (or the wave's lines) meets code
  // words of zero and adds nothing.
  int acc = 0;
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int off = 128 * (l_lo + i) + 16 * p;
    const bool use = l_lo + i < l_hi && off < rowb;
    const int k0 = use ? off / (int)sizeof(T) : 0;  // first weight of this piece
    int cv[E / 4];
    if constexpr (E == 8) {
      const int2 c2 = *reinterpret_cast<const int2 *>(sc + k0);
      cv[0] = c2.x;
      cv[1] = c2.y;
    } else {
      cv[0] = *reinterpret_cast<const int *>(sc + k0);
    }
#pragma unroll
    for (int g = 0; g < E / 4; ++g) {
      uint32_t u;
      if constexpr (E == 8) {
        u = bf16_fields4((uint32_t)wv[i][2 * g], (uint32_t)wv[i][2 * g + 1], hh);
      } else {
        u = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = Master<T>::at(wv[i], 4 * g + e);
          const uint32_t f = fabsf(v) > h ? (v > 0.0f ? 2u : 0u) : 1u;
          u |= f << (8 * e);
        }
      }
      acc = __builtin_amdgcn_sdot4((int)u, use ? cv[g] : 0, acc, false);
    }
  }
  acc = lanes8_sum(acc);  // the 8 lanes of a row
  if (p == 0) red[ks][rg][lane >> 3] = acc;
  __syncthreads();
  if (ks == 0 && p == 0 && n < N) {
    int sum = 0;
#pragma unroll
    for (int q = 0; q < KS; ++q) sum += red[q][rg][lane >> 3];
    const int a = sum - rowsum[0];
    if (acc_out) acc_out[n] = a;
    Y[n] = rescale(a, deq[0], epi_gamma(ep, n));
  }
}

template <typename T, int KS>
hipError_t launch_online_dot_ks(const int8_t *codes, const float *deq, const int32_t *rowsum, const T *w, int n, int k,
                                const Epilogue &ep, float *y, int32_t *acc_out, int lpw, hipStream_t stream) {
  const dim3 grid((unsigned)((n + 32 / KS - 1) / (32 / KS))), block(kThreads);
#define BL_ONLINE(LPW_)                                                                                    \
  online_dot_kernel<T, KS, LPW_><<<grid, block, 0, stream>>>(codes, deq, rowsum, w, n, k, ep, y, acc_out); \
  return hipGetLastError()
  if (lpw <= 8) { BL_ONLINE(8); }
  if (lpw <= 16) { BL_ONLINE(16); }
  if (lpw <= 20) { BL_ONLINE(20); }
  if (lpw <= 24) { BL_ONLINE(24); }
  BL_ONLINE(32);
#undef BL_ONLINE
}

// K split over the fewest waves (1, 2 or 4) that give at least 512
// workgroups and at most kOnlineMaxLines lines per wave; 0 if none does
int online_dot_splits(int64_t n, int64_t k, int esize) {
  if (n <= 0 || k <= 0 || k > kOnlineMaxK || k % 16 != 0) return 0;
  const int64_t lines = (k * esize + 127) / 128;
  for (int ks = 1; ks <= 4; ks *= 2) {
    const int64_t wgs = (n + 32 / ks - 1) / (32 / ks);
    if ((wgs >= 512 || ks == 4) && (lines + ks - 1) / ks <= kOnlineMaxLines) return ks;
  }
  return 0;
}

template <typename T>
hipError_t launch_online_dot_impl(const int8_t *codes, const float *deq, const int32_t *rowsum, const T *w, int64_t n,
                                  int64_t k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream) {
  const int ks = online_dot_splits(n, k, (int)sizeof(T));
  if (ks == 0 || !ep.gamma_dev) return hipErrorInvalidValue;
  const int lines = (int)((k * (int64_t)sizeof(T) + 127) / 128);
  const int lpw = (lines + ks - 1) / ks;
  if (ks == 1) return launch_online_dot_ks<T, 1>(codes, deq, rowsum, w, (int)n, (int)k, ep, y, acc_out, lpw, stream);
  if (ks == 2) return launch_online_dot_ks<T, 2>(codes, deq, rowsum, w, (int)n, (int)k, ep, y, acc_out, lpw, stream);
  return launch_online_dot_ks<T, 4>(codes, deq, rowsum, w, (int)n, (int)k, ep, y, acc_out, lpw, stream);
}

__global__ void copy_gamma_kernel(const double *__restrict__ src, double *__restrict__ dst) {
  if (threadIdx.x == 0 && blockIdx.x == 0) dst[0] = src[0];
}

__global__ void zero_i64_kernel(int64_t *p) {
  if (threadIdx.x == 0 && blockIdx.x == 0) p[0] = 0;
}

// fields equal to 3 have both bits set: popcount(w & (w >> 1) & 0x55555555)
__global__ __launch_bounds__(kThreads) void validate_kernel(const uint32_t *__restrict__ packed, int64_t words,
                                                            int64_t *__restrict__ n_bad) {
  __shared__ int red[kThreads / 64];
  int c = 0;
  for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < words; i += (int64_t)gridDim.x * kThreads) {
    const uint32_t v = packed[i];
    c += __popc(v & (v >> 1) & 0x55555555u);
  }
  c = wave_sum(c);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < kThreads / 64; ++w) t += red[w];
    if (t) atomicAdd(reinterpret_cast<unsigned long long *>(n_bad), (unsigned long long)t);
  }
}

int64_t partial_span(int64_t count) {
  int64_t per = kPerBlock;
  while ((count + per - 1) / per > kMaxPartials) per *= 2;
  return per;
}

unsigned grid_for(int64_t items) {
  int64_t b = (items + kThreads - 1) / kThreads;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

SegSpan make_span(int64_t k, const int64_t *row_end, int n_seg) {
  SegSpan sp{};
  sp.n = n_seg;
  sp.k = k;
  sp.part_lo[0] = 0;
  int64_t lo = 0;
  for (int j = 0; j < n_seg; ++j) {
    const int64_t count = (row_end[j] - lo) * k;
    sp.row_end[j] = row_end[j];
    sp.per[j] = partial_span(count);
    sp.part_lo[j + 1] = sp.part_lo[j] + (int)((count + sp.per[j] - 1) / sp.per[j]);
    lo = row_end[j];
  }
  return sp;
}

}  // namespace

size_t absmean_partials(int64_t k, const int64_t *row_end, int n_seg) {
  const int np = make_span(k, row_end, n_seg).part_lo[n_seg];
  return np > 0 ? (size_t)np : 1;
}

template <typename T>
hipError_t absmean_impl(const T *w, int64_t k, const int64_t *row_end, int n_seg, double *partials,
                        double *gamma_out, hipStream_t stream) {
  const SegSpan sp = make_span(k, row_end, n_seg);
  if (sp.part_lo[n_seg] > 0)
    absmean_partial_kernel<T><<<dim3((unsigned)sp.part_lo[n_seg]), dim3(kThreads), 0, stream>>>(w, sp, partials);
  absmean_final_kernel<<<dim3((unsigned)n_seg), dim3(kThreads), 0, stream>>>(partials, sp, gamma_out);
  return hipGetLastError();
}

template <typename T>
hipError_t ternarize_impl(const T *w, int64_t k, const int64_t *row_end, int n_seg, const double *gamma,
                          uint8_t *packed, hipStream_t stream) {
  const int64_t words = row_end[n_seg - 1] * (k / 16);
  if (words == 0) return hipSuccess;
  ternarize_pack_kernel<T><<<dim3(grid_for(words)), dim3(kThreads), 0, stream>>>(
      w, words, make_span(k, row_end, n_seg), gamma, reinterpret_cast<uint32_t *>(packed));
  return hipGetLastError();
}

hipError_t launch_absmean(const float *w, int64_t k, const int64_t *row_end, int n_seg, double *partials,
                          double *gamma_out, hipStream_t stream) {
  return absmean_impl(w, k, row_end, n_seg, partials, gamma_out, stream);
}

hipError_t launch_absmean_bf16(const uint16_t *w, int64_t k, const int64_t *row_end, int n_seg, double *partials,
                               double *gamma_out, hipStream_t stream) {
  return absmean_impl(w, k, row_end, n_seg, partials, gamma_out, stream);
}

hipError_t launch_ternarize_pack(const float *w, int64_t k, const int64_t *row_end, int n_seg, const double *gamma,
                                 uint8_t *packed, hipStream_t stream) {
  return ternarize_impl(w, k, row_end, n_seg, gamma, packed, stream);
}

hipError_t launch_ternarize_pack_bf16(const uint16_t *w, int64_t k, const int64_t *row_end, int n_seg,
                                      const double *gamma, uint8_t *packed, hipStream_t stream) {
  return ternarize_impl(w, k, row_end, n_seg, gamma, packed, stream);
}


hipError_t launch_copy_gamma(const double *src, double *dst, hipStream_t stream) {
  copy_gamma_kernel<<<1, 64, 0, stream>>>(src, dst);
  return hipGetLastError();
}

hipError_t launch_validate_packed(const uint8_t *packed, int64_t n, int64_t k, int64_t *n_bad, hipStream_t stream) {
  zero_i64_kernel<<<1, 64, 0, stream>>>(n_bad);
  const int64_t words = n * (k / 16);
  if (words > 0)
    validate_kernel<<<dim3(grid_for(words)), dim3(kThreads), 0, stream>>>(reinterpret_cast<const uint32_t *>(packed),
                                                                          words, n_bad);
  return hipGetLastError();
}

bool online_dot_supported(int64_t n, int64_t k, bool bf16) { return online_dot_splits(n, k, bf16 ? 2 : 4) > 0; }

hipError_t launch_online_dot(const int8_t *codes, const float *deq, const int32_t *rowsum, const float *w, int64_t n,
                             int64_t k, const Epilogue &ep, float *y, int32_t *acc_out, hipStream_t stream) {
  return launch_online_dot_impl(codes, deq, rowsum, w, n, k, ep, y, acc_out, stream);
}

hipError_t launch_online_dot_bf16(const int8_t *codes, const float *deq, const int32_t *rowsum, const uint16_t *w,
                                  int64_t n, int64_t k, const Epilogue &ep, float *y, int32_t *acc_out,
                                  hipStream_t stream) {
  return launch_online_dot_impl(codes, deq, rowsum, w, n, k, ep, y, acc_out, stream);
}

}  // namespace bl
