/* bitlinear.h — C ABI of the BitNet b1.58 BitLinear hot path for AMD gfx950 (MI355X).
 *
 * The operation (sources: the "BitNet b1.58 2B4T" model card, section "Model
 * Details"; the nnterp encyclopedia page "BitNet b1.58", sections "The
 * projections quantize their inputs and weights", "The two checkpoints", "The
 * block, in order", "The MLP gates with a squared ReLU", "Scaling inside a
 * sublayer is undone by the sub-norm"):
 *
 *   weights  W [n][k] fp32 -> gamma = mean|W|, codes c = round(W / gamma) in {-1,0,1},
 *            stored four to a byte;
 *   inputs   x [m][k] fp32 -> per token: a = max|x|, codes q = round(x * 127 / a)
 *            in [-127, 127], deq = a / 127;
 *   output   y [m][n] = (sum_k q[m][k] * c[n][k]) * deq[m] * gamma, no bias.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers (memory of the current HIP device),
 *    row-major, owned by the caller. The library never allocates, frees or
 *    keeps tensors; scratch memory comes from a caller `workspace` whose size
 *    the *_workspace_bytes functions give.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work is
 *    enqueued on it and the call returns without synchronizing; device-side
 *    faults surface at the caller's next synchronization.
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check returns a status and enqueues nothing. bitlinear_last_error() then
 *    gives a one-line reason (per thread).
 *  - A call over m == 0 tokens is a no-op that returns BITLINEAR_OK after the
 *    shape and argument checks; its per-token buffers (activations, codes,
 *    scales, outputs, workspace) may then be NULL.
 *  - Inputs must be finite; NaN and Inf are outside the contract.
 *  - The library is stateless between calls and reentrant on distinct buffers.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BITLINEAR_OK = 0,
  BITLINEAR_ERR_NULL = 1,      /* a required pointer is NULL */
  BITLINEAR_ERR_SHAPE = 2,     /* a size is negative, k % 16 != 0, bad segments, ... */
  BITLINEAR_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  BITLINEAR_ERR_WORKSPACE = 4, /* workspace NULL or smaller than required */
  BITLINEAR_ERR_DEVICE = 5,    /* no gfx950 device current, or a HIP launch failed */
  BITLINEAR_ERR_ARG = 6        /* an enum or flag argument is out of range */
} bitlinear_status;

#define BITLINEAR_ABI_VERSION 3
#define BITLINEAR_MAX_SEGMENTS 4

/* ---------------------------------------------------------------------------
 * Packed weight layout ("four to a byte": the nnterp page, sections "The
 * projections quantize their inputs and weights" and "The two checkpoints").
 * The pages fix only the density; the layout is this library's own:
 * row r of k codes occupies bytes [r * k/4, (r+1) * k/4). Code j of the row is
 * stored as u = c + 1 (0, 1, 2; 3 is invalid) in byte 4*(j/16) + (j%16)%4 of
 * the row, at bits 2*((j%16)/4) .. +1. Read as little-endian 32-bit words, word
 * g holds codes 16g .. 16g+15 and (word >> 2t) & 0x03030303 gives codes
 * 16g+4t .. 16g+4t+3 as bytes. k must be a multiple of 16.
 * ------------------------------------------------------------------------- */

/* bitlinear_quantize_weights — absmean ternarization and packing (offline
 * checkpoint mode: "The two checkpoints"; absmean: "Model Details").
 *   w          [n][k] fp32 master weights.
 *   gamma_in   NULL, or a device pointer to one double: use this gamma and skip
 *              the mean (e.g. a stored weight_scale).
 *   w_packed   [n][k/4] bytes, layout above, 16-byte aligned.
 *   gamma_out  device pointer to one double: the gamma used, mean|W| computed
 *              in fp64 by a fixed-order (deterministic) reduction unless
 *              gamma_in was given.
 *   Codes: c = sign(W) where |W| > gamma/2 (compared exactly in fp64), else 0;
 *   a tie |W| == gamma/2 gives 0 (round half to even).
 *   workspace  >= bitlinear_quantize_weights_workspace_bytes(n, k) bytes.
 * Errors: NULL w/w_packed/gamma_out/workspace -> ERR_NULL; n < 0, k <= 0 or
 * k % 16 != 0 -> ERR_SHAPE; misaligned w or w_packed -> ERR_ALIGN. n == 0 is a
 * no-op that still writes gamma_out (0). */
bitlinear_status bitlinear_quantize_weights(const float *w, int64_t n, int64_t k, const double *gamma_in,
                                            uint8_t *w_packed, double *gamma_out, void *workspace,
                                            size_t workspace_bytes, void *stream);
size_t bitlinear_quantize_weights_workspace_bytes(int64_t n, int64_t k);

/* bitlinear_validate_packed — counts fields equal to 3 (not a ternary code).
 *   n_bad  device pointer to one int64, overwritten with the count. */
bitlinear_status bitlinear_validate_packed(const uint8_t *w_packed, int64_t n, int64_t k, int64_t *n_bad,
                                           void *stream);

/* Prologue of the per-token activation quantization. */
typedef enum {
  /* q = round(x * 127 / max|x|), deq = max|x| / 127 ("The projections quantize
     their inputs and weights"). x is [m][k]. */
  BITLINEAR_ACT_ABSMAX = 0,
  /* RMSNorm (gain g, eps) then the same rounding ("The block, in order": the
     pre-norms and attn_sub_norm / ffn_sub_norm; eps 1e-5 in "Config"). Because
     a positive per-token factor cancels inside the rounding ("Scaling inside a
     sublayer is undone by the sub-norm"), the codes are those of v = g*x and
     deq = (max|v| / 127) / sqrt(mean(x^2) + eps), mean taken in fp64. */
  BITLINEAR_ACT_RMSNORM = 1,
  /* ReLU^2 gating then RMSNorm ("The MLP gates with a squared ReLU"): x is
     [m][2k], each row [gate (k) | up (k)]; the normed tensor is
     (max(gate, 0) * max(gate, 0)) * up in fp32, left to right. */
  BITLINEAR_ACT_RELU2_RMSNORM = 2
} bitlinear_act_mode;

/* bitlinear_quantize_acts — per-token int8 quantization of an fp32 activation.
 *   x          [m][k] fp32 ([m][2k] for RELU2_RMSNORM), 16-byte aligned.
 *   mode       bitlinear_act_mode.
 *   norm_gain  NULL (gain 1) or [k] fp32; used by the RMSNORM modes.
 *   eps        RMSNorm epsilon (RMSNORM modes).
 *   codes      [m][k] int8, 16-byte aligned.
 *   deq        [m] fp32.
 *   code_rowsum NULL or [m] int32: sum_k codes[m][k].
 * Rounding is half to even; an all-zero token gives codes 0 and deq 0.
 * Errors: NULL x/codes/deq (m > 0) -> ERR_NULL; m < 0, k <= 0, k % 16 != 0 ->
 * ERR_SHAPE; bad mode -> ERR_ARG. m == 0 is a no-op. */
bitlinear_status bitlinear_quantize_acts(const float *x, int64_t m, int64_t k, int32_t mode,
                                         const float *norm_gain, float eps, int8_t *codes, float *deq,
                                         int32_t *code_rowsum, void *stream);

/* Kernel choice for bitlinear_forward. AUTO takes DECODE for m <= 16. */
typedef enum {
  BITLINEAR_PATH_AUTO = 0,
  BITLINEAR_PATH_DECODE = 1,  /* weight-streaming GEMV, m <= 16 only */
  BITLINEAR_PATH_PREFILL = 2  /* LDS-tiled int8 MFMA GEMM, any m */
} bitlinear_path;

/* bitlinear_forward — one BitLinear projection (AutoBitLinear's forward: "The
 * projections quantize their inputs and weights"; packed checkpoint: "The two
 * checkpoints"; no bias: "Model Details").
 *   x          [m][k] fp32, quantized inside (ACT_ABSMAX); or NULL, and then
 *   codes_in   [m][k] int8 and deq_in [m] fp32 are used as given, with
 *   rowsum_in  NULL or [m] int32 = sum_k codes_in (computed when NULL).
 *   w_packed   [n][k/4] packed codes (layout above).
 *   gamma      HOST array of n_seg fp32 weight scales; seg_end HOST array of
 *              n_seg ascending int64 ends, seg_end[n_seg-1] == n. Output column
 *              j uses gamma[s] for seg_end[s-1] <= j < seg_end[s]: a fused
 *              projection (q|k|v, gate|up) is its matrices stacked along n with
 *              one gamma each. 1 <= n_seg <= BITLINEAR_MAX_SEGMENTS.
 *   y          [m][n] fp32: y = fl32(fl32((float)acc * deq[m]) * gamma_seg),
 *              acc = sum_k q[m][k] * c[n][k] computed exactly in int32.
 *   acc_out    NULL or [m][n] int32: acc.
 *   path       bitlinear_path.
 *   workspace  >= bitlinear_forward_workspace_bytes(m, n, k, x != NULL) bytes
 *              (may be NULL when that is 0).
 * Errors: NULL w_packed/y/gamma/seg_end, or (m > 0 and) x and codes_in/deq_in
 * both missing -> ERR_NULL; m < 0, n <= 0, k <= 0, k % 16 != 0, bad segments, DECODE with
 * m > 16 -> ERR_SHAPE; misaligned tensors -> ERR_ALIGN; small workspace ->
 * ERR_WORKSPACE; bad path -> ERR_ARG. m == 0 is a no-op. */
bitlinear_status bitlinear_forward(const float *x, const int8_t *codes_in, const float *deq_in,
                                   const int32_t *rowsum_in, int64_t m, int64_t k, const uint8_t *w_packed,
                                   int64_t n, const float *gamma, const int64_t *seg_end, int32_t n_seg,
                                   float *y, int32_t *acc_out, int32_t path, void *workspace,
                                   size_t workspace_bytes, void *stream);
size_t bitlinear_forward_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t quantize_inside);

/* bitlinear_forward_noalloc — bitlinear_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Arguments and result as bitlinear_forward,
 * without the workspace: the scratch is a device array inside the library of
 * bitlinear_forward_noalloc_max_scratch_bytes() = 32 MiB, one per GPU, held
 * from the first call on that GPU until the process ends. The call allocates
 * nothing (no hipMalloc, no allocating library routine). A shape whose
 * workspace (bitlinear_forward_workspace_bytes) exceeds the limit returns
 * ERR_WORKSPACE. Nothing in the scratch needs to start at zero; it keeps the
 * last call's contents. All calls on one GPU share the array: calls that may
 * overlap on one GPU (concurrent streams, threads) race and must be
 * serialized by the caller. Errors otherwise as bitlinear_forward. */
bitlinear_status bitlinear_forward_noalloc(const float *x, const int8_t *codes_in, const float *deq_in,
                                           const int32_t *rowsum_in, int64_t m, int64_t k, const uint8_t *w_packed,
                                           int64_t n, const float *gamma, const int64_t *seg_end, int32_t n_seg,
                                           float *y, int32_t *acc_out, int32_t path, void *stream);
size_t bitlinear_forward_noalloc_max_scratch_bytes(void);

/* Storage of master weights for the online mode ("The two checkpoints": the
 * bf16 checkpoint keeps its weights in bfloat16). */
typedef enum {
  BITLINEAR_MASTER_F32 = 0,  /* fp32 */
  BITLINEAR_MASTER_BF16 = 1  /* bfloat16 bit patterns (uint16), widened to fp32 exactly */
} bitlinear_master_dtype;

/* bitlinear_forward_online — the projection in the checkpoint mode that keeps
 * the full-precision weights and ternarizes them in every forward ("The two
 * checkpoints": the online mode; "The projections quantize their inputs and
 * weights"): per segment, gamma = mean|W| (fp64), codes = sign(W) [|W| >
 * gamma / 2], packed into the workspace, then bitlinear_forward with the
 * segments' gammas rounded to fp32. For one token (m == 1, path AUTO or
 * DECODE, k <= 8192 and each row within 32 128-byte lines per wave: k <= 8192
 * for bfloat16 masters, k <= 4096 for fp32 ones) the contraction forms the
 * codes from the masters as it reads them and no packed copy is written; the
 * result is the same.
 *   w_master   [n][k] master weights in master_dtype (bitlinear_master_dtype),
 *              16-byte aligned; segment j is rows [seg_end[j-1], seg_end[j])
 *              and gets its own gamma. bfloat16 masters are read as their
 *              exact fp32 values: half the bytes of fp32 masters.
 *   seg_end    HOST array of n_seg ascending int64 ends, seg_end[n_seg-1] == n.
 *   gamma_out  NULL or device [n_seg] fp64: the gammas used.
 * Other arguments as bitlinear_forward. The result equals
 * bitlinear_quantize_weights on each segment (of the widened masters) followed
 * by bitlinear_forward with those gammas, bit for bit.
 *   workspace  >= bitlinear_forward_online_workspace_bytes(m, n, k, x != NULL,
 *              seg_end, n_seg) bytes.
 * Errors as bitlinear_forward, plus ERR_ARG for an unknown master_dtype; m == 0
 * still computes the gammas. */
bitlinear_status bitlinear_forward_online(const float *x, const int8_t *codes_in, const float *deq_in,
                                          const int32_t *rowsum_in, int64_t m, int64_t k, const void *w_master,
                                          int32_t master_dtype, int64_t n, const int64_t *seg_end, int32_t n_seg,
                                          double *gamma_out, float *y, int32_t *acc_out, int32_t path,
                                          void *workspace, size_t workspace_bytes, void *stream);
size_t bitlinear_forward_online_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t quantize_inside,
                                                const int64_t *seg_end, int32_t n_seg);

/* bitlinear_forward_relu2_glu — the MLP's gate and up projections with the
 * squared-ReLU gating applied in the same pass ("The MLP gates with a squared
 * ReLU"; "The block, in order"): with g and u the outputs of bitlinear_forward
 * on the stacked matrix [gate; up] (segments [0, inter) and [inter, 2 inter)),
 *   y[m][j] = fl32(fl32(max(g[m][j], 0) * max(g[m][j], 0)) * u[m][j]).
 * Arguments as bitlinear_forward, except:
 *   w_packed   [2 inter][k/4]: the inter gate rows, then the inter up rows.
 *   inter      features of each matrix (> 0).
 *   gamma      HOST array of 2 fp32 scales {gate, up}.
 *   y          [m][inter] fp32 (half the columns of g|u).
 *   workspace  >= bitlinear_forward_relu2_glu_workspace_bytes(m, inter, k,
 *              x != NULL, path) bytes. When the tile shape allows (m > 64,
 *              k % 128 == 0, inter % 128 == 0, not DECODE) g and u never
 *              leave the chip; otherwise they pass through the workspace.
 * The result equals bitlinear_forward followed by the same gating, bit for
 * bit. Errors as bitlinear_forward. */
bitlinear_status bitlinear_forward_relu2_glu(const float *x, const int8_t *codes_in, const float *deq_in,
                                             const int32_t *rowsum_in, int64_t m, int64_t k,
                                             const uint8_t *w_packed, int64_t inter, const float *gamma, float *y,
                                             int32_t path, void *workspace, size_t workspace_bytes, void *stream);
size_t bitlinear_forward_relu2_glu_workspace_bytes(int64_t m, int64_t inter, int64_t k, int32_t quantize_inside,
                                                   int32_t path);

/* ---------------------------------------------------------------------------
 * The model's ends ([nnterp] "Printout": embed_tokens = Embedding(128256, 2560),
 * the final norm, lm_head = Linear(2560, 128256, bias=False); "Config": dtype
 * bfloat16, tie_word_embeddings: the head's matrix is the embedding table).
 * Tables are bfloat16 bit patterns (uint16), row-major [vocab][k].
 * ------------------------------------------------------------------------- */

/* bitlinear_embed — x[t][:] = the table row of ids[t], widened to fp32 (exact).
 *   ids    device [m] int64; an id outside [0, vocab) gives a zero row.
 *   table  device [vocab][k] bfloat16.   x  device [m][k] fp32, written.
 *   k % 8 == 0, 0 < k <= 4096; table and x 16-byte aligned.
 * Errors: NULL pointers -> ERR_NULL; m < 0, vocab <= 0, bad k -> ERR_SHAPE;
 * misaligned table or x -> ERR_ALIGN. m == 0 is a no-op. */
bitlinear_status bitlinear_embed(const int64_t *ids, int64_t m, const uint16_t *table, int64_t vocab, int64_t k,
                                 float *x, void *stream);

/* bitlinear_lm_head — the final RMSNorm and the head, per token (reading R20):
 *   ms = sum_k x_k^2 / k (fp64);  r = fl32(1 / sqrt(ms + eps));
 *   o_k = bf16(fl32(g_k * fl32(x_k * r)));  logits[n] = sum_k o_k w[n][k],
 * the bfloat16 products exact and the sum in fp32 (its rounding is within
 * k 2^-24 sum_k |o_k w[n][k]|).
 *   x          device [m][k] fp32 (the last block's output).
 *   norm_gain  NULL (gain 1) or device [k] fp32.
 *   w_head     device [n_vocab][k] bfloat16, 16-byte aligned; k % 8 == 0, k <= 4096.
 *   logits     device [m][n_vocab] fp32, written.
 *   normed_out NULL or device [m][k] bfloat16: o.
 *   workspace  >= bitlinear_lm_head_workspace_bytes(m, k) bytes when normed_out
 *              is NULL (0 otherwise).
 * Tokens are taken four per pass over the head.
 * Errors: NULL x/w_head/logits -> ERR_NULL; bad shapes -> ERR_SHAPE;
 * misaligned -> ERR_ALIGN; small workspace -> ERR_WORKSPACE. m == 0 is a no-op. */
bitlinear_status bitlinear_lm_head(const float *x, int64_t m, int64_t k, const float *norm_gain, float eps,
                                   const uint16_t *w_head, int64_t n_vocab, float *logits, uint16_t *normed_out,
                                   void *workspace, size_t workspace_bytes, void *stream);
size_t bitlinear_lm_head_workspace_bytes(int64_t m, int64_t k);

/* ---------------------------------------------------------------------------
 * Attention with a KV cache ([card] "Model Details": RoPE; [nnterp] "Loading":
 * eager attention, no softcap, window or sink; "Config": 20 heads, 5 kv heads,
 * head_dim 128, bfloat16). Caches are bfloat16 bit patterns laid out
 * [n_slots][n_kv][t_max][head_dim] (reading R21): one slot per sequence. Token r
 * belongs to sequence slot[r] at position pos[r] (device int64 arrays); a token
 * whose slot or position is out of range writes nothing and gets zeros.
 * ------------------------------------------------------------------------- */

/* bitlinear_rope_table — the rotary table, formed on the HOST ([nnterp]
 * "Loading": Llama's rotate_half with rope_theta 500,000, over 4096 positions;
 * reading R19): for position p < n_pos and pair e < head_dim/2,
 *   a = p theta^(-2e/head_dim) in fp64 (the host's libm pow),
 *   table[p][e] = { fl32(cos a), fl32(sin a) }   (the host's libm cos, sin),
 * written to the HOST array table of n_pos * head_dim floats. The caller
 * copies it to the device once (4096 x 64 pairs: 2 MB) and passes it to
 * bitlinear_rope and to the cached decoder block; forming it once on the host
 * keeps every RoPE path on identical angles.
 * Errors: NULL table -> ERR_NULL; head_dim odd or <= 0, n_pos <= 0 ->
 * ERR_SHAPE; theta not finite and > 0 -> ERR_ARG. Enqueues nothing. */
bitlinear_status bitlinear_rope_table(double theta, int32_t head_dim, int64_t n_pos, float *table);

/* bitlinear_rope — rotate, in place, the n_heads head vectors of each row of x
 * that start at column col0 (row stride ld floats), token r at position pos[r]
 * (reading R19: pairs (i, i + head_dim/2); v[i], v[i + head_dim/2] <-
 * v[i] c - v[i + head_dim/2] s, v[i + head_dim/2] c + v[i] s in fp32, with
 * (c, s) = rope_table[pos[r]][i]).
 *   rope_table  device [n_pos][head_dim/2][2] fp32 from bitlinear_rope_table,
 *               8-byte aligned. A position outside [0, n_pos) takes row 0
 *               (angle 0: the vector is unchanged).
 * Errors: NULL -> ERR_NULL; m < 0, head_dim odd or <= 0, n_heads <= 0,
 * col0 + n_heads head_dim > ld, n_pos <= 0 -> ERR_SHAPE; misaligned table ->
 * ERR_ALIGN. m == 0 is a no-op. */
bitlinear_status bitlinear_rope(float *x, int64_t m, int64_t ld, int64_t col0, int32_t n_heads, int32_t head_dim,
                                const int64_t *pos, const float *rope_table, int64_t n_pos, void *stream);

/* bitlinear_kv_append — write each token's keys and values (rows of k and v,
 * stride ld floats, n_kv head_dim values each) rounded to bfloat16 into the
 * caches at [slot[r]][g][pos[r]][:].
 * Errors: NULL -> ERR_NULL; bad sizes -> ERR_SHAPE. */
bitlinear_status bitlinear_kv_append(const float *k, const float *v, int64_t m, int64_t ld, int32_t n_kv,
                                     int32_t head_dim, const int64_t *slot, const int64_t *pos, uint16_t *k_cache,
                                     uint16_t *v_cache, int64_t n_slots, int64_t t_max, void *stream);

/* bitlinear_attention_decode — out[r][h head_dim + d] = sum over t <= pos[r] of
 * softmax_t(q_h . k_t / sqrt(head_dim)) v_t[d], with q head h (columns
 * h head_dim .. of row r of q, stride ldq) reading kv head h / (n_heads / n_kv)
 * of sequence slot[r]; fp32 arithmetic, causal. out has row stride ldo.
 * Supported: head_dim == 128, n_heads % n_kv == 0, n_heads / n_kv <= 8.
 *   workspace  >= bitlinear_attention_workspace_bytes(m, n_heads, t_max) bytes.
 * Errors: NULL -> ERR_NULL; unsupported or bad sizes -> ERR_SHAPE; small
 * workspace -> ERR_WORKSPACE. m == 0 is a no-op. */
bitlinear_status bitlinear_attention_decode(const float *q, int64_t m, int64_t ldq, int32_t n_heads, int32_t n_kv,
                                            int32_t head_dim, const uint16_t *k_cache, const uint16_t *v_cache,
                                            int64_t n_slots, int64_t t_max, const int64_t *slot, const int64_t *pos,
                                            float *out, int64_t ldo, void *workspace, size_t workspace_bytes,
                                            void *stream);
size_t bitlinear_attention_workspace_bytes(int64_t m, int32_t n_heads, int64_t t_max);

/* ---------------------------------------------------------------------------
 * Five codes per byte ([tiny] "O que é" and "Arquivos": the ternary checkpoint
 * also ships in a storage denser than two bits per weight; the pages give no
 * layout, so this one is the library's own). Row n of k codes takes
 * bitlinear_base3_row_bytes(k) = 16 ceil(k / 80) bytes; code j is base-3 digit
 * j % 5 of byte j / 5, stored as u = c + 1 (byte = sum_i u(5 b + i) 3^i);
 * codes past k are 0; bytes 243..255 are invalid and read as five zero codes.
 * ------------------------------------------------------------------------- */
size_t bitlinear_base3_row_bytes(int64_t k);

/* bitlinear_pack_base3 — rewrite two-bit packed weights in the base-3 storage.
 *   w_packed  [n][k/4] bytes (layout of bitlinear_quantize_weights), 16-byte
 *             aligned, k % 16 == 0. A field of 3 (not a code) becomes code 0.
 *   w_base3   [n][bitlinear_base3_row_bytes(k)] bytes, 16-byte aligned, written.
 * Errors: NULL pointers -> ERR_NULL; n <= 0, k <= 0, k % 16 != 0 -> ERR_SHAPE;
 * misaligned -> ERR_ALIGN. */
bitlinear_status bitlinear_pack_base3(const uint8_t *w_packed, int64_t n, int64_t k, uint8_t *w_base3,
                                      void *stream);

/* bitlinear_forward_base3 — bitlinear_forward for 1 to 4 tokens, reading the
 * weights in the base-3 storage: y = fl32(fl32((float)acc deq[m]) gamma(n)),
 * acc = sum_k q[m][k] c[n][k] exactly (the same result as bitlinear_forward on
 * the two-bit weights, bit for bit).
 *   x, codes_in, deq_in, m, k, n, gamma, seg_end, n_seg, y, acc_out: as
 *              bitlinear_forward (no row sums are needed: the decoded codes
 *              are signed).
 *   w_base3    [n][bitlinear_base3_row_bytes(k)] bytes, 16-byte aligned.
 *   workspace  >= bitlinear_forward_base3_workspace_bytes(m, k, x != NULL)
 *              bytes (may be NULL when that is 0).
 * Errors: as bitlinear_forward; m > 4 or k > 8192 -> ERR_SHAPE. m == 0 is a
 * no-op. */
bitlinear_status bitlinear_forward_base3(const float *x, const int8_t *codes_in, const float *deq_in, int64_t m,
                                         int64_t k, const uint8_t *w_base3, int64_t n, const float *gamma,
                                         const int64_t *seg_end, int32_t n_seg, float *y, int32_t *acc_out,
                                         void *workspace, size_t workspace_bytes, void *stream);
size_t bitlinear_forward_base3_workspace_bytes(int64_t m, int64_t k, int32_t quantize_inside);

/* ---------------------------------------------------------------------------
 * Block-level chains ("The block, in order").
 * ------------------------------------------------------------------------- */
typedef enum {
  /* The MLP alone: q1 = ACT_ABSMAX(x); [gate|up] = forward; ReLU^2 + ffn_sub_norm
     (ACT_RELU2_RMSNORM); y = down. No pre-norm and no residual. */
  BITLINEAR_BLOCK_FFN = 0,
  /* The projection stack of n_layers decoder blocks. Per layer:
       x -> input_layernorm -> q|k|v -> attention -> attn_sub_norm -> o_proj,
       h = x + o;  h -> post_attention_layernorm -> gate|up -> ReLU^2 ->
       ffn_sub_norm -> down;  x' = h + down.
     The attention is taken for a token that attends only to itself (a
     one-token sequence at position 0): the output of query head i is the
     value of key/value head i / (n_heads / n_kv_heads) ("Loading": 20 query
     heads share 5 key/value heads). q and k are computed but not consumed. */
  BITLINEAR_BLOCK_DECODER = 1,
  /* The same stack with the attention of a decode step: after q|k|v, RoPE on
     q and k (bitlinear_rope with the block's rope_table), the token's keys and values
     appended to its layer's caches at (slot[r], pos[r]) (bitlinear_kv_append),
     and each token's causal attention over its sequence's cache
     (bitlinear_attention_decode) feeds attn_sub_norm. Needs head_dim 128 and at
     most 8 query heads per key/value head. */
  BITLINEAR_BLOCK_DECODER_CACHED = 2
} bitlinear_block_kind;

typedef struct {
  const uint8_t *qkv;        /* DECODER: packed [(H + 2*KV)][H/4]: q rows, k rows, v rows */
  float qkv_gamma[3];
  const uint8_t *o;          /* DECODER: packed [H][H/4] */
  float o_gamma;
  const uint8_t *gate_up;    /* packed [2I][H/4]: gate rows then up rows */
  float gate_up_gamma[2];
  const uint8_t *down;       /* packed [H][I/4] */
  float down_gamma;
  const float *input_norm_gain;     /* DECODER: [H] or NULL (gain 1) */
  const float *attn_sub_norm_gain;  /* DECODER: [H] or NULL */
  const float *post_attn_norm_gain; /* DECODER: [H] or NULL */
  const float *ffn_sub_norm_gain;   /* [I] or NULL */
  uint16_t *k_cache, *v_cache;      /* DECODER_CACHED: [n_slots][n_kv_heads][t_max][head_dim] bfloat16 */
} bitlinear_layer;

typedef struct {
  int32_t kind;          /* bitlinear_block_kind */
  int32_t n_layers;      /* FFN: 1 */
  int64_t hidden;        /* H (multiple of 16) */
  int64_t intermediate;  /* I (multiple of 16) */
  int32_t n_heads, n_kv_heads, head_dim; /* DECODER: H == n_heads * head_dim, KV = n_kv_heads * head_dim */
  float eps;             /* RMSNorm epsilon */
  const bitlinear_layer *layers; /* HOST array of n_layers (device pointers inside) */
  /* DECODER_CACHED: token r of the call belongs to sequence slot[r] at position
     pos[r] (device [m] int64); caches hold n_slots sequences of t_max positions. */
  const int64_t *slot, *pos;
  int64_t n_slots, t_max;
  /* DECODER_CACHED: the rotary table (bitlinear_rope_table), device
     [rope_n_pos][head_dim/2][2] fp32, 8-byte aligned */
  const float *rope_table;
  int64_t rope_n_pos;
} bitlinear_block;

/* Optional per-stage outputs for checking a chain stage by stage. Every pointer
 * may be NULL. Layer l writes at element offset l * m * width. Widths: H, KV,
 * I as in bitlinear_block; Q = H + 2*KV. FFN blocks use codes_in, gate_up,
 * codes_ffn, deq (and acc_gate_up, acc_down). */
typedef struct {
  int8_t *codes_in;     /* [L][m][H]  codes of the block input (after input_layernorm) */
  int8_t *codes_attn;   /* [L][m][H]  codes after attn_sub_norm */
  int8_t *codes_post;   /* [L][m][H]  codes after post_attention_layernorm */
  int8_t *codes_ffn;    /* [L][m][I]  codes after ReLU^2 and ffn_sub_norm */
  float *deq;           /* [L][4][m]  deq of the four stages above, in that order */
  float *qkv;           /* [L][m][Q] */
  float *h;             /* [L][m][H]  residual after the attention add */
  float *gate_up;       /* [L][m][2I] */
  float *x_out;         /* [L][m][H]  layer outputs */
  int32_t *acc_qkv;     /* [L][m][Q] */
  int32_t *acc_o;       /* [L][m][H] */
  int32_t *acc_gate_up; /* [L][m][2I] */
  int32_t *acc_down;    /* [L][m][H] */
  float *attn;          /* [L][m][H]  DECODER_CACHED: the attention output (attn_sub_norm's input) */
} bitlinear_block_trace;

/* bitlinear_block_forward — run a block chain on x [m][H] fp32 into y [m][H].
 *   trace      NULL or per-stage outputs (above).
 *   workspace  >= bitlinear_block_workspace_bytes(blk, m) bytes.
 * Errors as bitlinear_forward, plus ERR_SHAPE for inconsistent head counts and
 * ERR_ARG for an unknown kind. */
bitlinear_status bitlinear_block_forward(const bitlinear_block *blk, const float *x, int64_t m, float *y,
                                         const bitlinear_block_trace *trace, void *workspace,
                                         size_t workspace_bytes, void *stream);
size_t bitlinear_block_workspace_bytes(const bitlinear_block *blk, int64_t m);

/* ---------------------------------------------------------------------------
 * Measurement probes: the denominators of the roofline fractions, measured on
 * the running GPU (not steps of the method; they compute nothing a caller
 * uses). The kernels above are bound by HBM reads (decode, quantization) and by
 * the int8 matrix cores (prefill).
 * ------------------------------------------------------------------------- */

/* bitlinear_probe_read — read bytes of device memory at src once, as coalesced
 * 16-byte loads, eight per thread in flight, and write nothing (sink, one
 * device uint32, is never written in practice). grid <= 0 takes one 256-thread
 * workgroup per 32 KB (at most 65536).
 * Errors: NULL -> ERR_NULL; bytes < 0 or bytes % 16 -> ERR_SHAPE; misaligned
 * src -> ERR_ALIGN. bytes == 0 is a no-op. */
bitlinear_status bitlinear_probe_read(const void *src, int64_t bytes, int64_t grid, uint32_t *sink, void *stream);

/* bitlinear_probe_mfma — workgroups of 4 waves, each wave issuing iters x 8
 * independent v_mfma_i32_32x32x32_i8 (65,536 int8 ops each) with no memory
 * traffic; sink as above.
 * Errors: NULL sink -> ERR_NULL; iters <= 0 or workgroups outside 1..65536 ->
 * ERR_SHAPE. */
bitlinear_status bitlinear_probe_mfma(int32_t iters, int64_t workgroups, int32_t *sink, void *stream);

/* bitlinear_probe_mfma_varied — as bitlinear_probe_mfma, but the operands vary
 * from one MFMA to the next (four pseudo-random operand sets per lane: A bytes
 * in {0, 1, 2} like the unpacked ternary codes, B bytes any int8 like the
 * activation codes). The matrix cores then draw about the power they draw in
 * the GEMMs, and the clock the GPU holds under that power sets the int8 rate a
 * contraction over such data can reach. Same arguments and errors. */
bitlinear_status bitlinear_probe_mfma_varied(int32_t iters, int64_t workgroups, int32_t *sink, void *stream);

/* ---------------------------------------------------------------------------
 * Misc.
 * ------------------------------------------------------------------------- */
const char *bitlinear_status_str(bitlinear_status s);
/* Reason for the last non-OK status returned on this thread ("" if none). */
const char *bitlinear_last_error(void);
int32_t bitlinear_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BITLINEAR_H */
