// Rotary position embedding, the bfloat16 KV cache, and each token's causal
// attention over its own sequence's cache.
//
// What is computed ([card] "Model Details": RoPE; [nnterp] "Loading": eager
// attention without softcap, window or sink; "Config": 20 query and 5
// key/value heads of 128, bfloat16; readings R19 and R21):
//   RoPE, per head vector v, i < hd/2: (c, s) = the rotary table's row for the
//     position (fl32 of cos and sin of p theta^(-2i/hd), formed on the host in
//     fp64); v[i], v[i + hd/2] <- v[i] c - v[i + hd/2] s, v[i + hd/2] c + v[i] s
//   cache[slot][g][p][:] = bf16(k after RoPE), bf16(v)
//   out_h = sum_{t <= p} softmax_t(q_h . k_t / sqrt(hd)) v_t, kv head g = h / (heads / kv heads)
//
// Attention runs as flash-decoding in two kernels. attn_partial_kernel: a
// workgroup takes one token, one key/value head and a chunk of positions, a
// wave a quarter of them. Lanes split each row into 16 pieces of 8 dims, so a
// wave load moves four whole 256-byte key (or value) rows, the query stays in
// registers, and a score is summed over its row's 16 lanes with DPP adds;
// the lanes that scored a position then weight its value row. It stores the
// chunk's max, sum of exponentials and unnormalized output.
// attn_combine_kernel rescales and adds the chunks, one exponential per chunk
// and head, one wave per head and token. Tokens whose slot or position is out of range get zeros and write
// nothing to the cache.
#include "common.h"

namespace bl {
namespace {

#ifndef BL_ATTN_CHUNK
#define BL_ATTN_CHUNK 128
#endif
constexpr int kAttnChunk = BL_ATTN_CHUNK;  // positions per workgroup (a multiple of 16)
#ifndef BL_ATTN_SPLIT_MAX_M
#define BL_ATTN_SPLIT_MAX_M 2
#endif
static_assert(kAttnChunk % 16 == 0 && kAttnChunk <= 256, "four waves, four positions per wave load");

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t kept = u >> 16, dropped = u & 0xFFFFu;
  return kept + ((dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) ? 1u : 0u);
}

// one thread per rotated pair; the (cosine, sine) come from the rotary table
// tab [n_pos][hd/2] (bitlinear_rope_table); a position outside [0, n_pos)
// takes row 0, angle 0
__global__ __launch_bounds__(256) void rope_kernel(float *__restrict__ x, int64_t m, int64_t ld, int64_t col0,
                                                   int n_heads, int hd, const int64_t *__restrict__ pos,
                                                   const float2 *__restrict__ tab, int64_t n_pos) {
  const int half = hd / 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m * n_heads * half) return;
  const int64_t r = i / (n_heads * half);
  const int rem = (int)(i - r * n_heads * half);
  const int h = rem / half, e = rem - h * half;
  const int64_t p = pos[r];
  const float2 csv = tab[(p >= 0 && p < n_pos ? p : 0) * half + e];
  const float c = csv.x, s = csv.y;
  float *v = x + r * ld + col0 + (int64_t)h * hd;
  const float a = v[e], b = v[e + half];
  v[e] = __fsub_rn(__fmul_rn(a, c), __fmul_rn(b, s));
  v[e + half] = __fadd_rn(__fmul_rn(b, c), __fmul_rn(a, s));
}

// The (cosine, sine) of every rotated pair of every token, cs[r][e] for
// e < hd/2, gathered from the rotary table at the token's position (row 0
// outside [0, n_pos)). All layers of a decode step rotate at the same
// positions, so a step gathers these rows once and the RoPE epilogues read
// them next to the token's other per-token data.
__global__ __launch_bounds__(256) void rope_gather_kernel(const int64_t *__restrict__ pos, int64_t m, int hd,
                                                          const float2 *__restrict__ tab, int64_t n_pos,
                                                          float2 *__restrict__ cs) {
  const int half = hd / 2;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m * half) return;
  const int64_t r = i / half;
  const int e = (int)(i - r * half);
  const int64_t p = pos[r];
  cs[i] = tab[(p >= 0 && p < n_pos ? p : 0) * half + e];
}

// RoPE on the q and k heads of a q|k|v row and the keys and values into the
// caches, one thread per rotated pair of q or k (plus the matching value pair);
// the (cosine, sine) come from rope_gather_kernel's rows
__global__ __launch_bounds__(256) void rope_append_kernel(float *__restrict__ qkv, int64_t m, int64_t ld,
                                                          int n_heads, int n_kv, int hd,
                                                          const int64_t *__restrict__ slot,
                                                          const int64_t *__restrict__ pos,
                                                          const float2 *__restrict__ cs,
                                                          uint16_t *__restrict__ kc, uint16_t *__restrict__ vc,
                                                          int64_t n_slots, int64_t tmax) {
  const int half = hd / 2, heads = n_heads + n_kv;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m * heads * half) return;
  const int64_t r = i / (heads * half);
  const int rem = (int)(i - r * heads * half);
  const int h = rem / half, e = rem - h * half;
  const int64_t p = pos[r];
  const float2 csv = cs[r * half + e];
  const float c = csv.x, s = csv.y;
  float *v = qkv + r * ld + (int64_t)h * hd;
  const float a = v[e], b = v[e + half];
  const float ra = __fsub_rn(__fmul_rn(a, c), __fmul_rn(b, s));
  const float rb = __fadd_rn(__fmul_rn(b, c), __fmul_rn(a, s));
  v[e] = ra;
  v[e + half] = rb;
  if (h < n_heads) return;  // a query head
  const int64_t sl = slot[r];
  if (sl < 0 || sl >= n_slots || p < 0 || p >= tmax) return;
  const int g = h - n_heads;
  const int64_t dst = ((sl * n_kv + g) * tmax + p) * hd;
  kc[dst + e] = (uint16_t)f32_to_bf16(ra);
  kc[dst + e + half] = (uint16_t)f32_to_bf16(rb);
  const float *vrow = qkv + r * ld + (int64_t)(n_heads + n_kv) * hd + (int64_t)g * hd;
  vc[dst + e] = (uint16_t)f32_to_bf16(vrow[e]);
  vc[dst + e + half] = (uint16_t)f32_to_bf16(vrow[e + half]);
}

// one thread per element of a token's keys (and values)
__global__ __launch_bounds__(256) void kv_append_kernel(const float *__restrict__ k, const float *__restrict__ v,
                                                        int64_t m, int64_t ld, int n_kv, int hd,
                                                        const int64_t *__restrict__ slot,
                                                        const int64_t *__restrict__ pos, uint16_t *__restrict__ kc,
                                                        uint16_t *__restrict__ vc, int64_t n_slots, int64_t tmax) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int row = n_kv * hd;
  if (i >= m * row) return;
  const int64_t r = i / row;
  const int e = (int)(i - r * row);
  const int64_t sl = slot[r], p = pos[r];
  if (sl < 0 || sl >= n_slots || p < 0 || p >= tmax) return;
  const int g = e / hd, d = e - g * hd;
  const int64_t dst = ((sl * n_kv + g) * tmax + p) * hd + d;
  kc[dst] = (uint16_t)f32_to_bf16(k[r * ld + e]);
  vc[dst] = (uint16_t)f32_to_bf16(v[r * ld + e]);
}

// Partials of token r, kv head g, chunk s (kAttnChunk positions): po
// [r][g][s][group][HD] (sum of exp(score - max) v), pml [r][g][s][group][2]
// (max, sum of exp); chunks past the token's position are not written. Wave w
// takes positions kAttnChunk/4 w .. + kAttnChunk/4 - 1 of the chunk; lane l
// takes dims 8 (l % 16) .. + 7 of positions kAttnChunk/4 w + 4 i + l / 16
// (i < PW), for keys and values alike, so every wave load moves four whole
// 256-byte rows, the query's 8 dims of each head stay in registers, and a
// position's score (summed over its 16 lanes with DPP adds) is already in
// the lanes that weight its value row.
template <int HD, int G>
__global__ __launch_bounds__(256) void attn_partial_kernel(const float *__restrict__ q, int64_t ldq, int n_kv, int grp,
                                                           const uint16_t *__restrict__ kc,
                                                           const uint16_t *__restrict__ vc, int64_t n_slots,
                                                           int64_t tmax, const int64_t *__restrict__ slot,
                                                           const int64_t *__restrict__ pos, float *__restrict__ po,
                                                           float *__restrict__ pml) {
  static_assert(HD == 128, "16 lanes of 8 dims cover a row");
  constexpr int PW = kAttnChunk / 16;  // positions per lane
  constexpr int kWavePos = kAttnChunk / 4;
  __shared__ float red[G][4];
  __shared__ __attribute__((aligned(16))) float accs[4][G][HD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // G of the kv head's grp query heads per workgroup: head part hs of kv head g
  const int s = blockIdx.x, S = gridDim.x, hsn = grp / G;
  const int g = blockIdx.y / hsn, hs = blockIdx.y - g * hsn;
  const int64_t r = blockIdx.z;
  const int64_t sl = slot[r], p = pos[r];
  const bool ok = sl >= 0 && sl < n_slots && p >= 0 && p < tmax;
  const int64_t T = ok ? p + 1 : 0;
  const int64_t t0 = (int64_t)s * kAttnChunk;
  const int64_t pb = (r * n_kv + g) * S;  // first chunk of (r, g)
  if (t0 >= T) return;  // nothing to attend in this chunk
  const int cnt_pos = (int)(T - t0 < kAttnChunk ? T - t0 : kAttnChunk);
  const int64_t base = (sl * n_kv + g) * tmax + t0;
  const int sub = lane >> 4, d0 = 8 * (lane & 15);
  // loads in issue order: keys, values (past the chunk end: the chunk's first
  // row, weight 0 below), the query's 8 dims of each head
  v4i kr[PW], vr[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int j = kWavePos * wave + 4 * i + sub;
    kr[i] = *reinterpret_cast<const v4i *>(kc + (base + (j < cnt_pos ? j : 0)) * HD + d0);
  }
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int j = kWavePos * wave + 4 * i + sub;
    vr[i] = *reinterpret_cast<const v4i *>(vc + (base + (j < cnt_pos ? j : 0)) * HD + d0);
  }
  float qv[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float4 a = *reinterpret_cast<const float4 *>(q + r * ldq + (int64_t)(g * grp + hs * G + hh) * HD + d0);
    const float4 b = *reinterpret_cast<const float4 *>(q + r * ldq + (int64_t)(g * grp + hs * G + hh) * HD + d0 + 4);
    qv[hh][0] = a.x; qv[hh][1] = a.y; qv[hh][2] = a.z; qv[hh][3] = a.w;
    qv[hh][4] = b.x; qv[hh][5] = b.y; qv[hh][6] = b.z; qv[hh][7] = b.w;
  }
  // keep every load above the arithmetic: left to itself the compiler sinks the
  // value loads below the scores, a second memory round trip after the first
  __builtin_amdgcn_sched_barrier(0);
  const float scale = (float)(1.0 / sqrt((double)HD));
  // ---- scores, and this lane's max over its positions
  float sc[PW][G], mx[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) mx[hh] = -INFINITY;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    float kf[8];
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) {
      kf[2 * q2] = bf16_to_f32((uint32_t)kr[i][q2] & 0xFFFFu);
      kf[2 * q2 + 1] = bf16_to_f32((uint32_t)kr[i][q2] >> 16);
    }
    const bool valid = kWavePos * wave + 4 * i + sub < cnt_pos;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = __fmaf_rn(qv[hh][e], kf[e], d);
      d = row16_sum(d);  // the 16 lanes of the row
      sc[i][hh] = valid ? __fmul_rn(d, scale) : -INFINITY;
      mx[hh] = fmaxf(mx[hh], sc[i][hh]);
    }
  }
  // ---- chunk max per head: the wave's four position groups, then the four waves
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    const float m = rows_max(mx[hh]);
    if (lane == 0) red[hh][wave] = m;
  }
  __syncthreads();
  float cmax[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) cmax[hh] = fmaxf(fmaxf(red[hh][0], red[hh][1]), fmaxf(red[hh][2], red[hh][3]));
  __syncthreads();
  // ---- exp(score - max), the sums (fixed order), and the values
  float acc[G][8];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.0f;
  float lsum[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) lsum[hh] = 0.0f;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    float vf[8];
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) {
      vf[2 * q2] = bf16_to_f32((uint32_t)vr[i][q2] & 0xFFFFu);
      vf[2 * q2 + 1] = bf16_to_f32((uint32_t)vr[i][q2] >> 16);
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float w = sc[i][hh] == -INFINITY ? 0.0f : expf(sc[i][hh] - cmax[hh]);
      lsum[hh] += w;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = __fmaf_rn(w, vf[e], acc[hh][e]);
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    // (each position's weight sits in the 16 lanes of its group: add one lane per group)
    const float l = rows_sum(lsum[hh]);
    if (lane == 0) red[hh][wave] = l;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = rows_sum(acc[hh][e]);
    if (sub == 0) {
      *reinterpret_cast<float4 *>(&accs[wave][hh][d0]) =
          make_float4(acc[hh][0], acc[hh][1], acc[hh][2], acc[hh][3]);
      *reinterpret_cast<float4 *>(&accs[wave][hh][d0 + 4]) =
          make_float4(acc[hh][4], acc[hh][5], acc[hh][6], acc[hh][7]);
    }
  }
  __syncthreads();
  const int64_t part = (pb + s) * grp + hs * G;
  if (tid < G) {
    pml[(part + tid) * 2] = cmax[tid];
    pml[(part + tid) * 2 + 1] = ((red[tid][0] + red[tid][1]) + red[tid][2]) + red[tid][3];
  }
  for (int e = tid; e < G * HD; e += 256) {
    const int hh = e / HD, d = e - hh * HD;
    po[part * HD + e] = ((accs[0][hh][d] + accs[1][hh][d]) + accs[2][hh][d]) + accs[3][hh][d];
  }
}

// out[r][h HD + d] from the chunks of token r's query head h (kv head h / G):
// one single-wave workgroup per head and token, 32 chunks per round. Every load
// of a round (each lane's two dims of the 32 chunk outputs; lane j's chunk j
// max and sum) is issued before any arithmetic, the first round's before the
// max over all chunks is formed. Lane j then forms exp(max_j - max) and its
// share of the sum of exponentials, and every lane adds its two dims of the
// chunk outputs, weighted by those factors, in chunk order.
template <int HD, int G>
__global__ __launch_bounds__(64) void attn_combine_kernel(
    const float *__restrict__ po, const float *__restrict__ pml, int n_kv, int S, int64_t n_slots, int64_t tmax,
    const int64_t *__restrict__ slot, const int64_t *__restrict__ pos, float *__restrict__ out, int64_t ldo) {
  constexpr int kR = 32;
  const int lane = threadIdx.x;
  const int g = blockIdx.x / G, hh = blockIdx.x - g * G;
  const int64_t r = blockIdx.y;
  const int64_t sl = slot[r], p = pos[r];
  const bool ok = sl >= 0 && sl < n_slots && p >= 0 && p < tmax;
  const int nch = ok ? (int)(p / kAttnChunk) + 1 : 0;  // chunks that hold positions
  const int64_t pb = (r * n_kv + g) * S;
  {
    float2 o[kR];
    float mc = -INFINITY, lc = 0.0f;
    // the loads of the round that starts at chunk c0 (past the last chunk:
    // the last chunk's finite values, weighted 0)
    auto issue = [&](int c0) {
      const int n_here = nch - c0 < kR ? nch - c0 : kR;
#pragma unroll
      for (int j = 0; j < kR; ++j) {
        const int cj = c0 + (j < n_here ? j : n_here - 1);
        o[j] = *reinterpret_cast<const float2 *>(po + ((pb + cj) * G + hh) * HD + 2 * lane);
      }
      mc = -INFINITY;
      lc = 0.0f;
      if (lane < n_here) {
        mc = pml[((pb + c0 + lane) * G + hh) * 2];
        lc = pml[((pb + c0 + lane) * G + hh) * 2 + 1];
      }
    };
    float M = -INFINITY, L = 0.0f, a0 = 0.0f, a1 = 0.0f;
    if (nch > 0) {
      issue(0);
      M = mc;
      for (int c = kR + lane; c < nch; c += 64) M = fmaxf(M, pml[((pb + c) * G + hh) * 2]);
      M = rows_max(row16_max(M));
      for (int c0 = 0; c0 < nch; c0 += kR) {
        if (c0 > 0) issue(c0);
        const float f = mc == -INFINITY ? 0.0f : expf(mc - M);
        L += rows_sum(row16_sum(__fmul_rn(f, lc)));
#pragma unroll
        for (int j = 0; j < kR; ++j) {
          const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j));
          a0 = __fmaf_rn(fj, o[j].x, a0);
          a1 = __fmaf_rn(fj, o[j].y, a1);
        }
      }
    }
    const float2 res = nch > 0 ? make_float2(__fdiv_rn(a0, L), __fdiv_rn(a1, L)) : make_float2(0.0f, 0.0f);
    *reinterpret_cast<float2 *>(out + r * ldo + (int64_t)(g * G + hh) * HD + 2 * lane) = res;
  }
}

}  // namespace

int attention_splits(int64_t tmax) { return (int)((tmax + kAttnChunk - 1) / kAttnChunk); }

bool attention_supported(int n_heads, int n_kv, int hd) {
  if (hd != 128 || n_kv <= 0 || n_heads % n_kv != 0) return false;
  const int g = n_heads / n_kv;
  return g == 1 || g == 2 || g == 4 || g == 8;
}

hipError_t launch_rope(float *x, int64_t m, int64_t ld, int64_t col0, int n_heads, int hd, const int64_t *pos,
                       const float2 *tab, int64_t n_pos, hipStream_t stream) {
  const int64_t n = m * n_heads * (hd / 2);
  if (n == 0) return hipSuccess;
  rope_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(x, m, ld, col0, n_heads, hd, pos, tab,
                                                                          n_pos);
  return hipGetLastError();
}

hipError_t launch_rope_gather(const int64_t *pos, int64_t m, int hd, const float2 *tab, int64_t n_pos, float2 *cs,
                              hipStream_t stream) {
  const int64_t n = m * (hd / 2);
  if (n == 0) return hipSuccess;
  rope_gather_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(pos, m, hd, tab, n_pos, cs);
  return hipGetLastError();
}

hipError_t launch_rope_append(float *qkv, int64_t m, int64_t ld, int n_heads, int n_kv, int hd, const int64_t *slot,
                              const int64_t *pos, const float2 *cs, uint16_t *kc, uint16_t *vc, int64_t n_slots,
                              int64_t tmax, hipStream_t stream) {
  const int64_t n = m * (n_heads + n_kv) * (hd / 2);
  if (n == 0) return hipSuccess;
  rope_append_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(qkv, m, ld, n_heads, n_kv, hd, slot,
                                                                                 pos, cs, kc, vc, n_slots, tmax);
  return hipGetLastError();
}

hipError_t launch_kv_append(const float *k, const float *v, int64_t m, int64_t ld, int n_kv, int hd,
                            const int64_t *slot, const int64_t *pos, uint16_t *kc, uint16_t *vc, int64_t n_slots,
                            int64_t tmax, hipStream_t stream) {
  const int64_t n = m * n_kv * hd;
  if (n == 0) return hipSuccess;
  kv_append_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(k, v, m, ld, n_kv, hd, slot, pos, kc,
                                                                              vc, n_slots, tmax);
  return hipGetLastError();
}

// workspace: attention_workspace_floats(m, n_heads, tmax) floats: the chunks'
// outputs [m][n_heads][S][HD], then their (max, sum) [m][n_heads][S][2]
size_t attention_workspace_floats(int64_t m, int n_heads, int64_t tmax) {
  const int64_t S = attention_splits(tmax);
  return (size_t)(m * n_heads * S) * (128 + 2);
}

hipError_t launch_attention(const float *q, int64_t m, int64_t ldq, int n_heads, int n_kv, int hd,
                            const uint16_t *kc, const uint16_t *vc, int64_t n_slots, int64_t tmax,
                            const int64_t *slot, const int64_t *pos, float *out, int64_t ldo, float *ws,
                            hipStream_t stream) {
  if (m == 0) return hipSuccess;
  if (!attention_supported(n_heads, n_kv, hd)) return hipErrorInvalidValue;
  const int S = attention_splits(tmax);
  float *po = ws;
  float *pml = ws + (size_t)(m * n_heads * S) * 128;
  // few tokens fill few CUs: several workgroups per (chunk, kv head), each
  // with a share of the kv head's query heads (all read the same keys and
  // values): up to four at one or two tokens, two at three or four (measured:
  // at four tokens four were slower than two, and two faster than one)
  const int grp = n_heads / n_kv;
  const int hsn = m <= BL_ATTN_SPLIT_MAX_M ? (grp >= 4 ? 4 : grp) : (m <= 4 && grp >= 2 ? 2 : 1);
  const dim3 grid((unsigned)S, (unsigned)(n_kv * hsn), (unsigned)m), block(256), cgrid((unsigned)n_heads, (unsigned)m);
#define BL_PART(GW_) \
  attn_partial_kernel<128, GW_><<<grid, block, 0, stream>>>(q, ldq, n_kv, grp, kc, vc, n_slots, tmax, slot, pos, po, pml)
#define BL_ATTN(G_)                                                                                                  \
  switch (G_ / hsn) {                                                                                                \
    case 1: BL_PART(1); break;                                                                                       \
    case 2: BL_PART(2); break;                                                                                       \
    case 4: BL_PART(4); break;                                                                                       \
    default: BL_PART(8); break;                                                                                      \
  }                                                                                                                  \
  e = hipGetLastError();                                                                                             \
  if (e != hipSuccess) return e;                                                                                     \
  attn_combine_kernel<128, G_><<<cgrid, dim3(64), 0, stream>>>(po, pml, n_kv, S, n_slots, tmax, slot, pos, out, ldo)
  hipError_t e;
  switch (grp) {
    case 1: BL_ATTN(1); break;
    case 2: BL_ATTN(2); break;
    case 4: BL_ATTN(4); break;
    default: BL_ATTN(8); break;
  }
#undef BL_PART
#undef BL_ATTN
  return hipGetLastError();
}

}  // namespace bl
