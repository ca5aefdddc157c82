// Decode projection that quantizes its own input (one or two tokens).
//
// One launch computes, for the tokens of a decode step, the per-token int8
// codes of the projection's input (with the block's prologue: RMSNorm gain,
// the self-only attention read of the value heads, or none) and the ternary
// contraction with its rescale, and applies the block's elementwise epilogue:
//   plain     y = fl32(fl32((float)acc * deq) * gamma(n))
//   residual  out2 = fl32(res + y)                 (h = x + o, x' = h + down)
//   ReLU^2    mi = fl32(fl32(max(g, 0)^2) * u)     (gate and up rows paired)
//   RoPE      q and k rotated at the token's position, k and v into the
//             bfloat16 KV cache (rows i and i + hd/2 of a head paired)
// (nnterp "BitNet b1.58" page: "The projections quantize their inputs and
// weights", "The block, in order", "The MLP gates with a squared ReLU").
//
// Each workgroup re-derives the codes of the whole input row with quant_row
// (act_prologue.h), the same arithmetic as the standalone quantization kernel
// at 256 threads, so codes and deq equal that kernel's bit for bit; the input
// is a few KB read from L2, while the weights, issued first, stream from HBM.
//
// Contraction as the one-token kernel of gemv_decode.hip: 8 lanes share one
// weight row and read 16-byte pieces of its 128-byte lines (a wave reads 8
// rows x 128 contiguous bytes), the fields are expanded with
// (w >> 2j) & 0x03030303 and fed to v_dot4_i32_i8 against the codes in LDS,
// and the 8 lanes of a row are summed with DPP adds. KS waves split the
// lines of a row; their partial sums are added in LDS in a fixed order.
// In the ReLU^2 form, workgroup b owns gate rows [b R/2, (b + 1) R/2) and the
// up rows I + the same range, so it can form its slice of mi itself. In the
// RoPE form a workgroup of the q and k heads owns R/2 rotated pairs of one
// head (rows e and e + hd/2), so it rotates them itself, with the cosine and
// sine of each pair read from the step's rows of the rotary table (rope_gather_kernel) while the
// weights load.
#include "act_prologue.h"

namespace bl {
namespace {

constexpr uint32_t kFieldMask = 0x03030303u;
constexpr int kFusedMaxK = 8192;

#ifndef BL_FUSED_TH
#define BL_FUSED_TH 256
#endif

// TH threads per workgroup; NV: float4 of one input row per thread
// (K <= 4 TH NV). A row has at most TH NV / 128 lines of 128 bytes, so each of
// the KS waves of a row loads LPW lines.
template <int MODE, int EPI, int MT, int KS, int NV, int TH>
__global__ __launch_bounds__(TH) void gemv_fused_kernel(FusedDecode a) {
  constexpr int NW = TH / 64;
  constexpr int RG = NW / KS;  // row groups of 8 rows
  constexpr int R = 8 * RG;    // weight rows per workgroup
  constexpr int LPW = (TH * NV / 128 + KS - 1) / KS;
  __shared__ __attribute__((aligned(16))) int8_t sc[MT * kFusedMaxK];
  __shared__ int red[KS][RG][8][MT];
  __shared__ float red_f[NW];
  __shared__ double red_d[NW];
  __shared__ int red_i[NW];
  __shared__ float ybuf[EPI == FUSED_EPI_RELU2 || EPI == FUSED_EPI_ROPE ? MT * R : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ks = wave % KS, rg = wave / KS;
  const int r = rg * 8 + (lane >> 3);  // local row
  const int p = lane & 7;
  const int N = a.n, K = a.src.k;
  const Epilogue ep = resolve_gamma(a.ep);
  int n;
  // RoPE form: workgroups [0, rot_wgs) hold rotated pairs, hd / R per head
  const int rot_wgs = EPI == FUSED_EPI_ROPE ? (a.n_heads + a.n_kv) * (a.hd / R) : 0;
  const int rh = EPI == FUSED_EPI_ROPE && (int)blockIdx.x < rot_wgs ? blockIdx.x / (a.hd / R) : 0;
  const int rj = EPI == FUSED_EPI_ROPE && (int)blockIdx.x < rot_wgs ? blockIdx.x - rh * (a.hd / R) : 0;
  if constexpr (EPI == FUSED_EPI_RELU2) {
    const int half = R / 2, inter = N / 2;
    n = r < half ? blockIdx.x * half + r : inter + blockIdx.x * half + (r - half);
  } else if constexpr (EPI == FUSED_EPI_ROPE) {
    const int half = R / 2;
    n = (int)blockIdx.x < rot_wgs ? rh * a.hd + (r < half ? rj * half + r : a.hd / 2 + rj * half + (r - half))
                                  : blockIdx.x * R + r;
  } else {
    n = blockIdx.x * R + r;
  }
  const bool valid = n < N;
  const int ldb = K >> 2;          // bytes per weight row
  const int L = (ldb + 127) >> 7;  // 128-byte lines per row, the last may be partial
  const int l_lo = L * ks / KS, l_hi = L * (ks + 1) / KS;

  // Loads in issue order: the first token's input row (a few KB, from L2),
  // then the weights (from HBM). Loads complete in issue order, so the
  // quantization of the first token waits for its own row only and runs while
  // the weights are in flight.
  RowStage<NV> st;
  row_load<MODE, NV, false, TH>(a.src, 0, st);
  __builtin_amdgcn_sched_barrier(0);
  // every lane issues LPW loads; pieces past its range reload the first piece
  // of the matrix and are not used
  v4i w[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int off = 128 * (l_lo + i) + 16 * p;
    const bool use = l_lo + i < l_hi && off < ldb && valid;
    w[i] = *reinterpret_cast<const v4i *>(use ? a.w + (int64_t)n * ldb + off : a.w);
  }
  __builtin_amdgcn_sched_barrier(0);

  // RoPE form: thread t (R/2) + i < MT (R/2) takes pair i of token t (its
  // cosine and sine from the step's table)
  float rc = 0.0f, rsn = 0.0f;
  if constexpr (EPI == FUSED_EPI_ROPE) {
    const int t = threadIdx.x / (R / 2), e = rj * (R / 2) + (int)threadIdx.x % (R / 2);
    if ((int)blockIdx.x < rot_wgs && t < a.m && threadIdx.x < MT * (R / 2)) {
      const float2 cs = a.cs[t * (a.hd / 2) + e];
      rc = cs.x;
      rsn = cs.y;
    }
  }

  // the codes of every token of the step, into LDS
  RowQuant q[MT];
  q[0] = row_finish<MODE, NV, false, TH>(a.src, 0, a.eps, st, reinterpret_cast<int *>(sc), red_f, red_d, red_i);
#pragma unroll
  for (int t = 1; t < MT; ++t) {
    q[t].deq = 0.0f;
    q[t].rowsum = 0;
    if (t < a.m)
      q[t] = quant_row<MODE, NV, false, TH>(a.src, t, a.eps, reinterpret_cast<int *>(sc + t * kFusedMaxK), red_f,
                                            red_d, red_i);
  }
  if (blockIdx.x == 0 && a.codes_out) {
    for (int i = threadIdx.x; i < a.m * (K >> 4); i += TH) {
      const int t = i / (K >> 4), c = i - t * (K >> 4);
      *reinterpret_cast<v4i *>(a.codes_out + (int64_t)t * K + 16 * c) =
          *reinterpret_cast<const v4i *>(sc + t * kFusedMaxK + 16 * c);
    }
    if (threadIdx.x == 0 && a.deq_out) {
#pragma unroll
      for (int t = 0; t < MT; ++t)
        if (t < a.m) a.deq_out[t] = q[t].deq;
    }
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
        if (t < a.m) {
          const v4i *cp = reinterpret_cast<const v4i *>(sc + t * kFusedMaxK + k0);
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
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    acc[t] = lanes8_sum(acc[t]);
  }
  if (p == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) red[ks][rg][lane >> 3][t] = acc[t];
  }
  __syncthreads();
  if (ks == 0 && p == 0 && valid) {
    const float g = epi_gamma(ep, n);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < a.m) {
        int sum = 0;
#pragma unroll
        for (int s = 0; s < KS; ++s) sum += red[s][rg][lane >> 3][t];
        const int av = sum - q[t].rowsum;
        const float yv = rescale(av, q[t].deq, g);
        const int64_t o = (int64_t)t * N + n;
        if (a.acc_out) a.acc_out[o] = av;
        if (EPI == FUSED_EPI_PLAIN || (EPI != FUSED_EPI_ROPE && a.y)) a.y[o] = yv;
        if constexpr (EPI == FUSED_EPI_RESID) a.out2[o] = __fadd_rn(a.res[o], yv);
        if constexpr (EPI == FUSED_EPI_RELU2 || EPI == FUSED_EPI_ROPE) ybuf[t * R + r] = yv;
      }
    }
  }
  if constexpr (EPI == FUSED_EPI_RELU2) {
    constexpr int half = R / 2;
    __syncthreads();
    const int inter = N / 2;
    for (int i = threadIdx.x; i < MT * half; i += TH) {
      const int t = i / half, j = i - t * half;
      if (t < a.m) {
        const float gt = ybuf[t * R + j], up = ybuf[t * R + half + j];
        const float tt = gt > 0.0f ? gt : 0.0f;
        a.mi[(int64_t)t * inter + blockIdx.x * half + j] = __fmul_rn(__fmul_rn(tt, tt), up);
      }
    }
  }
  if constexpr (EPI == FUSED_EPI_ROPE) {
    constexpr int half = R / 2;
    __syncthreads();
    const int hd = a.hd, tid = threadIdx.x;
    if ((int)blockIdx.x < rot_wgs) {
      const int t = tid / half, i = tid - t * half;
      if (tid < MT * half && t < a.m) {
        const float x0 = ybuf[t * R + i], x1 = ybuf[t * R + half + i];
        const float ra = __fsub_rn(__fmul_rn(x0, rc), __fmul_rn(x1, rsn));
        const float rb = __fadd_rn(__fmul_rn(x1, rc), __fmul_rn(x0, rsn));
        const int e = rj * half + i;
        const int64_t row = (int64_t)t * N + (int64_t)rh * hd + e;
        a.y[row] = ra;
        a.y[row + hd / 2] = rb;
        const int64_t sl = a.slot[t], p = a.pos[t];
        if (rh >= a.n_heads && sl >= 0 && sl < a.n_slots && p >= 0 && p < a.tmax) {  // a key head
          const int64_t dst = ((sl * a.n_kv + (rh - a.n_heads)) * a.tmax + p) * hd;
          a.kc[dst + e] = (uint16_t)bf16_rne(ra);
          a.kc[dst + e + hd / 2] = (uint16_t)bf16_rne(rb);
        }
      }
    } else {
      const int t = tid / R, i = tid - t * R;
      if (tid < MT * R && t < a.m) {
        const int nn = blockIdx.x * R + i;
        const float yv = ybuf[t * R + i];
        a.y[(int64_t)t * N + nn] = yv;
        const int64_t sl = a.slot[t], p = a.pos[t];
        if (sl >= 0 && sl < a.n_slots && p >= 0 && p < a.tmax) {
          const int vr = nn - (a.n_heads + a.n_kv) * hd, g = vr / hd;
          a.vc[((sl * a.n_kv + g) * a.tmax + p) * hd + (vr - g * hd)] = (uint16_t)bf16_rne(yv);
        }
      }
    }
  }
}

template <int MODE, int EPI, int MT>
hipError_t launch_mt(const FusedDecode &a, hipStream_t stream) {
  // split K over the waves of a workgroup until the workgroups cover the CUs
  const int rows = EPI == FUSED_EPI_RELU2 ? a.n / 2 : a.n;  // output rows that set the grid
  const int per32 = EPI == FUSED_EPI_RELU2 ? rows / 16 : rows / 32;
  // (one token: at most about one workgroup per CU, since every workgroup
  // quantizes the whole input row; more tokens: at least 256 workgroups)
  const int min_wgs = MT == 1 ? 128 : 256;
  const int ks = per32 >= min_wgs ? 1 : (2 * per32 >= min_wgs ? 2 : 4);
  const int R = 32 / ks;
  constexpr int TH = BL_FUSED_TH, F = TH / 256;  // F: waves per row group per wave of the 256-thread form
  const int lines = ((a.src.k >> 2) + 127) >> 7;
  const int nv = a.src.k <= 4096 / F ? 4 / F : 8 / F;
  if (lines > TH * nv / 128) return hipErrorInvalidValue;
  int grid;
  if (EPI == FUSED_EPI_ROPE) {
    // whole heads of hd rows, hd a multiple of R; every row in a workgroup
    if (a.hd <= 0 || a.hd % R != 0 || a.n != (a.n_heads + 2 * a.n_kv) * a.hd || a.n_kv <= 0) return hipErrorInvalidValue;
    grid = a.n / R;
  } else if (EPI == FUSED_EPI_RELU2) {
    if (a.n % 2 != 0 || (a.n / 2) % (R / 2) != 0) return hipErrorInvalidValue;
    grid = (a.n / 2) / (R / 2);
  } else {
    grid = (a.n + R - 1) / R;
  }
  // R rows per workgroup as R / 8 row groups, each split over F ks waves
  const dim3 g((unsigned)grid), b(TH);
  if (nv == 4 / F) {
    if (ks == 1) gemv_fused_kernel<MODE, EPI, MT, F, 4 / F, TH><<<g, b, 0, stream>>>(a);
    else if (ks == 2) gemv_fused_kernel<MODE, EPI, MT, 2 * F, 4 / F, TH><<<g, b, 0, stream>>>(a);
    else gemv_fused_kernel<MODE, EPI, MT, 4 * F, 4 / F, TH><<<g, b, 0, stream>>>(a);
  } else {
    if (ks == 1) gemv_fused_kernel<MODE, EPI, MT, F, 8 / F, TH><<<g, b, 0, stream>>>(a);
    else if (ks == 2) gemv_fused_kernel<MODE, EPI, MT, 2 * F, 8 / F, TH><<<g, b, 0, stream>>>(a);
    else gemv_fused_kernel<MODE, EPI, MT, 4 * F, 8 / F, TH><<<g, b, 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <int MODE, int EPI>
hipError_t launch_pair(const FusedDecode &a, hipStream_t stream) {
  return a.m == 1 ? launch_mt<MODE, EPI, 1>(a, stream) : launch_mt<MODE, EPI, kFusedMaxM>(a, stream);
}

}  // namespace

bool fused_decode_supported(int64_t m, int64_t k) {
  return m >= 1 && m <= kFusedMaxM && k % 64 == 0 && k <= kFusedMaxK;
}

hipError_t launch_gemv_fused(int mode, int epi, const FusedDecode &a, hipStream_t stream) {
  if (!fused_decode_supported(a.m, a.src.k) || a.n <= 0) return hipErrorInvalidValue;
  if (mode == BITLINEAR_ACT_RMSNORM && epi == FUSED_EPI_PLAIN)
    return launch_pair<BITLINEAR_ACT_RMSNORM, FUSED_EPI_PLAIN>(a, stream);
  if (mode == BITLINEAR_ACT_RMSNORM && epi == FUSED_EPI_RESID)
    return launch_pair<BITLINEAR_ACT_RMSNORM, FUSED_EPI_RESID>(a, stream);
  if (mode == BITLINEAR_ACT_RMSNORM && epi == FUSED_EPI_RELU2)
    return launch_pair<BITLINEAR_ACT_RMSNORM, FUSED_EPI_RELU2>(a, stream);
  if (mode == BITLINEAR_ACT_RMSNORM && epi == FUSED_EPI_ROPE)
    return launch_pair<BITLINEAR_ACT_RMSNORM, FUSED_EPI_ROPE>(a, stream);
  if (mode == ACT_GQA_RMSNORM && epi == FUSED_EPI_RESID) return launch_pair<ACT_GQA_RMSNORM, FUSED_EPI_RESID>(a, stream);
  if (mode == BITLINEAR_ACT_ABSMAX && epi == FUSED_EPI_RELU2)
    return launch_pair<BITLINEAR_ACT_ABSMAX, FUSED_EPI_RELU2>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace bl
