/* CPU oracle for the BitNet b1.58 BitLinear hot path — TEST INFRASTRUCTURE.
 *
 * Plain, slow, single-threaded C11. It is the reference the HIP path is
 * checked against, and nothing else: only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it. It shares no code, header or
 * table with the HIP library, and never reads a value the HIP path produced.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off (no fast-math; x86-64 SSE2, so
 * every float operation is one correctly rounded binary32 operation and every
 * double operation one binary64 operation; rintf rounds half to even).
 *
 * Sources ("pages"):
 *  [card]   "BitNet b1.58 2B4T - Scaling Native 1-bit LLM" (Azure AI model card),
 *           section "Model Details".
 *  [nnterp] "nnterp encyclopedia: BitNet b1.58" (family bitnet), sections
 *           "The block, in order", "Scaling inside a sublayer is undone by the
 *           sub-norm", "The projections quantize their inputs and weights",
 *           "The MLP gates with a squared ReLU", "The two checkpoints", "Config",
 *           "Printout", "Loading", "From the family module".
 *  [tiny]   "BitNet TinyDialogues 1.58b" README, sections "O que é", "Arquivos".
 *
 * Where the pages leave a step open, the reading taken is stated at the step
 * (R-numbers match the list of readings kept with the design notes).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ---- O1: weight scale gamma = mean |W| over the whole matrix ------------------
 * [card] "Model Details": weights are quantized with absmean quantization;
 * [nnterp] "The projections quantize their inputs and weights": rounded to
 * {-1, 0, 1} * mean|W|, stored with one weight_scale.
 * R4: one gamma per matrix. Sum in fp64, sequentially in row-major order. */
double orc_absmean(const float *w, int64_t count) {
  if (count <= 0) return 0.0;
  double s = 0.0;
  for (int64_t i = 0; i < count; ++i) s += fabs((double)w[i]);
  return s / (double)count;
}

/* ---- O2: ternary code of each weight ----------------------------------------
 * c = round(W / gamma) clipped to [-1, 1] (same passages as O1). In exact
 * arithmetic that is sign(W) when |W| > gamma / 2, and 0 otherwise; a tie
 * |W| == gamma / 2 rounds half to even, to 0 (R5, R1). The comparison below
 * is exact: (double)|W| is exact and 0.5 * gamma is an exact halving. */
void orc_ternarize(const float *w, int64_t count, double gamma, int8_t *c) {
  const double half = 0.5 * gamma;
  for (int64_t i = 0; i < count; ++i) {
    double a = fabs((double)w[i]);
    c[i] = (int8_t)(a > half ? (w[i] > 0.0f ? 1 : -1) : 0);
  }
}

/* ---- O3: "four to a byte" storage ([nnterp] "The projections quantize their
 * inputs and weights"; "The two checkpoints") ----------------------------------
 * The pages fix only the density. Our layout (R6): row n of K codes takes K/4
 * bytes. Code k sits in group g = k / 16, slot t = k % 16; it is stored as the
 * field u = c + 1 (0, 1 or 2) in byte 4g + (t % 4) of the row, at bits
 * 2 * (t / 4) and 2 * (t / 4) + 1. Field value 3 is invalid. */
static int64_t pack_byte(int64_t row, int64_t k, int64_t kdim) {
  return row * (kdim / 4) + 4 * (k / 16) + (k % 16) % 4;
}
static int pack_shift(int64_t k) { return 2 * ((k % 16) / 4); }

/* returns 0, or -1 when k is not a multiple of 16 or a code is outside {-1,0,1} */
int orc_pack(const int8_t *c, int64_t n, int64_t k, uint8_t *p) {
  if (k % 16 != 0) return -1;
  memset(p, 0, (size_t)(n * (k / 4)));
  for (int64_t r = 0; r < n; ++r)
    for (int64_t j = 0; j < k; ++j) {
      int v = c[r * k + j];
      if (v < -1 || v > 1) return -1;
      p[pack_byte(r, j, k)] |= (uint8_t)((v + 1) << pack_shift(j));
    }
  return 0;
}

/* decodes; returns the number of invalid fields (value 3), which decode as 0;
 * -1 when k is not a multiple of 16 */
int64_t orc_unpack(const uint8_t *p, int64_t n, int64_t k, int8_t *c) {
  if (k % 16 != 0) return -1;
  int64_t bad = 0;
  for (int64_t r = 0; r < n; ++r)
    for (int64_t j = 0; j < k; ++j) {
      int u = (p[pack_byte(r, j, k)] >> pack_shift(j)) & 3;
      if (u == 3) { ++bad; u = 1; }
      c[r * k + j] = (int8_t)(u - 1);
    }
  return bad;
}

/* ---- Five codes to a byte (base 3) -------------------------------------------
 * [tiny] "O que é" and "Arquivos": the same ternary checkpoint ships in a denser
 * ternary format (TQ1_0, the smaller file) beside a two-bit one (TQ2_0). The
 * pages give no layout for it; this one is our own (reading R18): a ternary
 * code has three values, and 3^5 = 243 <= 256, so a byte holds five codes as
 * base-3 digits. Row n of K codes takes 16 * ceil(K / 80) bytes (a whole number
 * of 16-byte pieces of 80 codes). Code k is digit k % 5 of byte k / 5, stored
 * as u = c + 1: byte j = sum_i u(5j + i) * 3^i. Codes past K are 0 (digit 1),
 * so every pad byte is 121 and a full byte is at most 242; 243 .. 255 are
 * invalid. */
int64_t orc_base3_row_bytes(int64_t k) { return 16 * ((k + 79) / 80); }

/* returns 0, or -1 when a code is outside {-1, 0, 1} */
int orc_pack_base3(const int8_t *c, int64_t n, int64_t k, uint8_t *p) {
  const int64_t rb = orc_base3_row_bytes(k);
  for (int64_t r = 0; r < n; ++r)
    for (int64_t j = 0; j < rb; ++j) {
      int byte = 0, w = 1;
      for (int i = 0; i < 5; ++i) {
        const int64_t kk = 5 * j + i;
        int u = 1;
        if (kk < k) {
          const int v = c[r * k + kk];
          if (v < -1 || v > 1) return -1;
          u = v + 1;
        }
        byte += u * w;
        w *= 3;
      }
      p[r * rb + j] = (uint8_t)byte;
    }
  return 0;
}

/* decodes the first k codes of each row; returns the number of invalid bytes
 * (243 .. 255) among those that hold them; such a byte decodes as all zeros */
int64_t orc_unpack_base3(const uint8_t *p, int64_t n, int64_t k, int8_t *c) {
  const int64_t rb = orc_base3_row_bytes(k);
  int64_t bad = 0;
  for (int64_t r = 0; r < n; ++r)
    for (int64_t j = 0; 5 * j < k; ++j) {
      int byte = p[r * rb + j];
      if (byte > 242) { ++bad; byte = 121; }
      for (int i = 0; i < 5; ++i) {
        const int64_t kk = 5 * j + i;
        if (kk < k) c[r * k + kk] = (int8_t)(byte % 3 - 1);
        byte /= 3;
      }
    }
  return bad;
}

/* ---- codes of one row: round(v * 127 / max|v|) to 255 levels ---------------
 * [nnterp] "The projections quantize their inputs and weights": each input is
 * rounded per token to 255 levels as round(x * 127 / max|x|); [card] "Model
 * Details": 8-bit absmax per token.
 * R1: round half to even. R2: the scale s = 127 / a is one correctly rounded
 * fp32 division per row, then one fp32 product per element, as written.
 * Clamp to [-127, 127] (255 levels; it never binds, see the pins).
 * R3: a == 0 gives all-zero codes. When a < 2^-64 the row is first scaled by
 * 2^64 (exact), which keeps 127 / a finite and changes no code that the
 * unscaled steps could compute. Returns a (unscaled). */
static float codes_of_row(const float *v, int64_t k, int8_t *q) {
  float a = 0.0f;
  for (int64_t i = 0; i < k; ++i) {
    float t = fabsf(v[i]);
    if (t > a) a = t;
  }
  if (a == 0.0f) {
    memset(q, 0, (size_t)k);
    return a;
  }
  const int tiny = a < 0x1p-64f;
  const float pre = tiny ? 0x1p64f : 1.0f;
  const float s = 127.0f / (a * pre);
  for (int64_t i = 0; i < k; ++i) {
    float p = (v[i] * pre) * s;
    float r = rintf(p);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    q[i] = (int8_t)r;
  }
  return a;
}

/* ---- O4: per-token absmax quantization ----------------------------------------
 * codes as above; dequantization factor deq = a / 127 (fp32 division), 0 for
 * an all-zero row. */
void orc_quant_absmax(const float *x, int64_t m, int64_t k, int8_t *q, float *deq) {
  for (int64_t r = 0; r < m; ++r) {
    float a = codes_of_row(x + r * k, k, q + r * k);
    deq[r] = a == 0.0f ? 0.0f : a / 127.0f;
  }
}

/* ---- O5: RMSNorm followed by the per-token quantization -----------------------
 * [nnterp] "The block, in order" and "Config": RMSNorms with eps 1e-5 sit
 * before the projections (pre-norms, and attn_sub_norm / ffn_sub_norm right
 * before o_proj / down_proj). R7: RMSNorm(x) = g * x / sqrt(mean(x^2) + eps).
 * R8: "Scaling inside a sublayer is undone by the sub-norm": the positive
 * per-token 1 / r cancels inside round(u * 127 / max|u|), so the codes are
 * taken from v = g * x (fp32 product) and 1 / r goes into deq only:
 *   ms  = (sum_k x_k^2) / K              fp64, sequential
 *   r   = sqrt(ms + eps)                 fp64
 *   deq = fl32((a_v / 127) / r)          fp64, rounded once
 * gain == NULL means g = 1. */
void orc_quant_rms(const float *x, int64_t m, int64_t k, const float *gain, float eps,
                   int8_t *q, float *deq, float *scratch_v) {
  for (int64_t r = 0; r < m; ++r) {
    const float *xr = x + r * k;
    double ss = 0.0;
    for (int64_t i = 0; i < k; ++i) ss += (double)xr[i] * (double)xr[i];
    const double ms = ss / (double)k;
    const double rr = sqrt(ms + (double)eps);
    for (int64_t i = 0; i < k; ++i) scratch_v[i] = gain ? gain[i] * xr[i] : xr[i];
    float a = codes_of_row(scratch_v, k, q + r * k);
    deq[r] = a == 0.0f ? 0.0f : (float)(((double)a / 127.0) / rr);
  }
}

/* ---- O6: squared-ReLU gating ---------------------------------------------------
 * [nnterp] "The block, in order": m = relu(gate)^2 * up; "The MLP gates with a
 * squared ReLU": exactly zero where the gate is not positive.
 * R9: left to right in fp32: t = max(G, 0); m = (t * t) * U.
 * gu rows hold [gate (inter) | up (inter)]; out is [m][inter]. */
void orc_relu2_mul(const float *gu, int64_t m, int64_t inter, float *out) {
  for (int64_t r = 0; r < m; ++r)
    for (int64_t i = 0; i < inter; ++i) {
      float g = gu[r * 2 * inter + i], u = gu[r * 2 * inter + inter + i];
      float t = g > 0.0f ? g : 0.0f;
      float tt = t * t;
      out[r * inter + i] = tt * u;
    }
}

/* ---- O7: the ternary x int8 contraction ---------------------------------------
 * [nnterp] "The projections quantize their inputs and weights": a projection's
 * output is exactly the product of its per-token quantized input with its
 * ternary codes (then rescaled, O8).
 * acc[r][n] = sum_k q[r][k] * c[n][k], exact in int64. R15: stored as int32;
 * returns -1 if a sum does not fit (it cannot for |q| <= 127, K < 2^24). */
int orc_contract(const int8_t *q, int64_t m, int64_t k, const int8_t *c, int64_t n, int32_t *acc) {
  int rc = 0;
  for (int64_t r = 0; r < m; ++r)
    for (int64_t j = 0; j < n; ++j) {
      int64_t s = 0;
      const int8_t *qr = q + r * k, *cj = c + j * k;
      for (int64_t i = 0; i < k; ++i) s += (int64_t)qr[i] * (int64_t)cj[i];
      if (s > INT32_MAX || s < INT32_MIN) rc = -1;
      acc[r * n + j] = (int32_t)s;
    }
  return rc;
}

/* ---- O8: rescale (no bias) ------------------------------------------------------
 * [nnterp] "The two checkpoints": the packed checkpoint multiplies by its stored
 * ternary weights and weight_scale; [card] "Model Details": no bias terms.
 * R10: y = fl32(fl32((float)acc * deq) * gamma_f), gamma_f = fl32(gamma).
 * R11: a fused projection (gate|up, q|k|v) is its matrices stacked along N with
 * one gamma each: output column j uses gamma[s] for seg_end[s-1] <= j < seg_end[s]. */
void orc_rescale(const int32_t *acc, int64_t m, int64_t n, const float *deq, const double *gamma,
                 const int64_t *seg_end, int n_seg, float *y) {
  for (int64_t r = 0; r < m; ++r) {
    int s = 0;
    for (int64_t j = 0; j < n; ++j) {
      while (s < n_seg - 1 && j >= seg_end[s]) ++s;
      const float g = (float)gamma[s];
      const float t = (float)acc[r * n + j] * deq[r];
      y[r * n + j] = t * g;
    }
  }
}

/* ---- O11: bfloat16 ------------------------------------------------------------
 * [nnterp] "Config": the checkpoint's dtype is bfloat16. A bfloat16 value is
 * the top 16 bits of a binary32 one; rounding keeps the nearest such value,
 * ties to the one whose last kept bit is 0 (R1's rule). Inputs are finite
 * (R17). */
static uint16_t bf16_of(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint32_t dropped = u & 0xFFFFu, kept = u >> 16;
  uint32_t r = kept;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) r += 1u;
  return (uint16_t)r;
}

static float f32_of_bf16(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

void orc_round_bf16(const float *x, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_of(x[i]);
}

void orc_bf16_to_f32(const uint16_t *b, int64_t n, float *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_of_bf16(b[i]);
}

/* ---- O12: the final norm, as the head's bfloat16 input --------------------------
 * [nnterp] "Printout": (norm) BitNetRMSNorm((2560,), eps=1e-05) after the last
 * block, then lm_head; "From the family module": Llama's tree (model.norm, then
 * lm_head). R7's norm; R20 fixes the order in our fp32 stream:
 *   ms = sum_k x_k^2 / K in fp64, in order;  r = fl32(1 / sqrt(ms + eps));
 *   o_k = bf16(fl32(g_k * fl32(x_k * r))).
 * gain NULL means 1. */
void orc_final_norm(const float *x, int64_t m, int64_t k, const float *gain, float eps, uint16_t *out) {
  for (int64_t r = 0; r < m; ++r) {
    const float *xr = x + r * k;
    double ss = 0.0;
    for (int64_t i = 0; i < k; ++i) ss += (double)xr[i] * (double)xr[i];
    const double ms = ss / (double)k;
    const float rf = (float)(1.0 / sqrt(ms + (double)eps));
    for (int64_t i = 0; i < k; ++i) {
      const float v = xr[i] * rf;
      const float o = gain ? gain[i] * v : v;
      out[r * k + i] = bf16_of(o);
    }
  }
}

/* ---- O13: the head ----------------------------------------------------------------
 * [nnterp] "Printout": lm_head = Linear(2560 -> 128256, bias=False); "Config":
 * bfloat16, tie_word_embeddings (the head's matrix is the embedding table).
 * logits[r][n] = sum_k o[r][k] * w[n][k] over bfloat16 o and w: every product
 * is exact in binary64 and the fp64 sum of K of them is within K 2^-53 of the
 * exact one, far inside the fp32 rounding; stored rounded to fp32. absdot gets
 * sum_k |o w| (fp64), the scale of the rounding error any fp32 summation order
 * may make. */
void orc_lm_head(const uint16_t *o, int64_t m, int64_t k, const uint16_t *w, int64_t n, float *y, double *absdot) {
  for (int64_t r = 0; r < m; ++r)
    for (int64_t j = 0; j < n; ++j) {
      double s = 0.0, a = 0.0;
      for (int64_t i = 0; i < k; ++i) {
        const double p = (double)f32_of_bf16(o[r * k + i]) * (double)f32_of_bf16(w[j * k + i]);
        s += p;
        a += fabs(p);
      }
      y[r * n + j] = (float)s;
      if (absdot) absdot[r * n + j] = a;
    }
}

/* ---- O14: rotary position embedding ----------------------------------------------
 * [card] "Model Details": the model uses RoPE; [nnterp] "Loading": Llama's
 * rotate_half with rope_theta 500,000, over 4096 positions; "Config": head_dim
 * 128, max_position_embeddings 4096. rotate_half pairs element i of a head with
 * element i + hd/2. R19 (the pages leave the precision open): for token r at
 * position p and each head vector v of hd values (heads start at column col0
 * of a row of ld floats), for i < hd/2:
 *   a = p * theta^(-2i/hd) (fp64), c = fl32(cos a), s = fl32(sin a),
 *   v[i] <- fl32(fl32(v[i] c) - fl32(v[i + hd/2] s)),
 *   v[i + hd/2] <- fl32(fl32(v[i + hd/2] c) + fl32(v[i] s))  (old values).
 * The rotary covers positions 0 .. n_pos - 1; a position outside that range
 * is turned by angle 0 (as position 0 is). */
void orc_rope(float *x, int64_t m, int64_t ld, int64_t col0, int n_heads, int hd, const int64_t *pos,
              double theta, int64_t n_pos) {
  const int half = hd / 2;
  for (int64_t r = 0; r < m; ++r) {
    const int64_t p = (pos[r] >= 0 && pos[r] < n_pos) ? pos[r] : 0;
    for (int h = 0; h < n_heads; ++h) {
      float *v = x + r * ld + col0 + (int64_t)h * hd;
      for (int i = 0; i < half; ++i) {
        const double ang = (double)p * pow(theta, -(2.0 * i) / (double)hd);
        const float c = (float)cos(ang), s = (float)sin(ang);
        const float a = v[i], b = v[i + half];
        const float ac = a * c, bs = b * s, bc = b * c, as = a * s;
        v[i] = ac - bs;
        v[i + half] = bc + as;
      }
    }
  }
}

/* ---- O15: one token's attention over its sequence's cache -------------------------
 * [nnterp] "Loading": the eager attention (no softcap, window or sink);
 * "Printout"/"Config": 20 query heads, 5 key/value heads of 128; query head h
 * reads key/value head h / (n_heads / n_kv). R21: the cache holds the keys
 * (after RoPE) and values rounded to bfloat16, [slot][kv head][position][hd];
 * token r of sequence slot[r] sits at position pos[r] and attends to positions
 * 0 .. pos[r] of that slot (causal). In fp64:
 *   s_t = (1/sqrt(hd)) sum_d q_d k_td;  w_t = exp(s_t - max s) / sum exp(. - max s);
 *   out_d = fl32(sum_t w_t v_td).
 * vmag gets sum_t w_t |v_td| and smag max_t (1/sqrt(hd)) sum_d |q_d k_td|, the
 * scales of the fp32 rounding a kernel makes. Returns the number of tokens whose
 * slot or position is out of range (their outputs are zero). */
int64_t orc_attention(const float *q, int64_t m, int64_t ldq, int n_heads, int n_kv, int hd, const uint16_t *kc,
                      const uint16_t *vc, int64_t n_slots, int64_t tmax, const int64_t *slot, const int64_t *pos,
                      float *out, double *vmag, double *smag, double *scratch) {
  const int group = n_heads / n_kv;
  const double scale = 1.0 / sqrt((double)hd);
  int64_t bad = 0;
  for (int64_t r = 0; r < m; ++r) {
    const int ok = slot[r] >= 0 && slot[r] < n_slots && pos[r] >= 0 && pos[r] < tmax;
    if (!ok) ++bad;
    for (int h = 0; h < n_heads; ++h) {
      float *o = out + r * (int64_t)n_heads * hd + (int64_t)h * hd;
      double *vm = vmag + r * (int64_t)n_heads * hd + (int64_t)h * hd;
      if (!ok) {
        for (int d = 0; d < hd; ++d) { o[d] = 0.0f; vm[d] = 0.0; }
        smag[r * n_heads + h] = 0.0;
        continue;
      }
      const int g = h / group;
      const uint16_t *kb = kc + ((slot[r] * n_kv + g) * tmax) * (int64_t)hd;
      const uint16_t *vb = vc + ((slot[r] * n_kv + g) * tmax) * (int64_t)hd;
      const float *qh = q + r * ldq + (int64_t)h * hd;
      const int64_t T = pos[r] + 1;
      double mx = -INFINITY, sm = 0.0;
      for (int64_t t = 0; t < T; ++t) {
        double dot = 0.0, ad = 0.0;
        for (int d = 0; d < hd; ++d) {
          const double p = (double)qh[d] * (double)f32_of_bf16(kb[t * hd + d]);
          dot += p;
          ad += fabs(p);
        }
        scratch[t] = scale * dot;
        if (scratch[t] > mx) mx = scratch[t];
        if (scale * ad > sm) sm = scale * ad;
      }
      double L = 0.0;
      for (int64_t t = 0; t < T; ++t) {
        scratch[t] = exp(scratch[t] - mx);
        L += scratch[t];
      }
      for (int d = 0; d < hd; ++d) {
        double acc = 0.0, mag = 0.0;
        for (int64_t t = 0; t < T; ++t) {
          const double v = (double)f32_of_bf16(vb[t * hd + d]);
          acc += scratch[t] * v;
          mag += scratch[t] * fabs(v);
        }
        o[d] = (float)(acc / L);
        vm[d] = mag / L;
      }
      smag[r * n_heads + h] = sm;
    }
  }
  return bad;
}
