// C-ABI entry points of the BitLinear library (declared in include/bitlinear.h).
//
// Every entry point validates its arguments on the host first, and returns a
// status without touching the HIP runtime when they are wrong; then it checks
// that the current device is gfx950, and enqueues kernels on the caller's
// stream without synchronizing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "common.h"

namespace {

thread_local std::string g_err;

bitlinear_status fail(bitlinear_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

}  // namespace

bitlinear_status bl::report_error(bitlinear_status s, const char *reason) { return fail(s, "%s", reason); }

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

bitlinear_status check_device() {
  static std::mutex mu;
  static int state[256];  // 0 unknown, 1 gfx950, 2 other
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BITLINEAR_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 256) return fail(BITLINEAR_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (state[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(BITLINEAR_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (state[dev] == 2) return fail(BITLINEAR_ERR_DEVICE, "device %d is %s, this library targets gfx950", dev,
                                     prop.gcnArchName);
  }
  if (state[dev] != 1) return fail(BITLINEAR_ERR_DEVICE, "device %d is not gfx950", dev);
  return BITLINEAR_OK;
}

bitlinear_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(BITLINEAR_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return BITLINEAR_OK;
}

#define BL_TRY(expr)                              \
  do {                                            \
    bitlinear_status st_ = (expr);                \
    if (st_ != BITLINEAR_OK) return st_;          \
  } while (0)

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// ---------------------------------------------------------------- forward core
bitlinear_status make_segments(const float *gamma, const int64_t *seg_end, int32_t n_seg, int64_t n,
                               bl::Epilogue *ep);

bitlinear_status check_segments(const float *gamma, const int64_t *seg_end, int32_t n_seg, int64_t n,
                                bl::Epilogue *ep) {
  if (!gamma || !seg_end) return fail(BITLINEAR_ERR_NULL, "gamma and seg_end are required");
  return make_segments(gamma, seg_end, n_seg, n, ep);
}

// gamma: host scales, or NULL when they live on the device (set gamma_dev after)
bitlinear_status make_segments(const float *gamma, const int64_t *seg_end, int32_t n_seg, int64_t n,
                               bl::Epilogue *ep) {
  if (!seg_end) return fail(BITLINEAR_ERR_NULL, "seg_end is required");
  if (n_seg < 1 || n_seg > BITLINEAR_MAX_SEGMENTS)
    return fail(BITLINEAR_ERR_SHAPE, "n_seg = %d, must be 1..%d", n_seg, BITLINEAR_MAX_SEGMENTS);
  int64_t prev = 0;
  for (int s = 0; s < n_seg; ++s) {
    if (seg_end[s] <= prev) return fail(BITLINEAR_ERR_SHAPE, "seg_end must be strictly ascending and positive");
    prev = seg_end[s];
  }
  if (prev != n) return fail(BITLINEAR_ERR_SHAPE, "seg_end[n_seg-1] = %lld, must equal n = %lld", (long long)prev,
                             (long long)n);
  for (int s = 0; s < BITLINEAR_MAX_SEGMENTS; ++s) {
    ep->gamma[s] = s < n_seg && gamma ? gamma[s] : 0.0f;
    ep->seg_end[s] = s < n_seg ? (int32_t)seg_end[s] : (int32_t)n;
  }
  ep->gamma_dev = nullptr;
  ep->n_seg = n_seg;
  ep->blocks32 = 1;
  for (int s = 0; s < n_seg; ++s)
    if (seg_end[s] % 32) ep->blocks32 = 0;
  return BITLINEAR_OK;
}

// int32 indexing inside the kernels
constexpr int64_t kMaxDim = (int64_t)1 << 30;

// split_ws: gemm_prefill_workspace_bytes(m, n, k) bytes, or NULL (no split K)
bitlinear_status contract(const int8_t *codes, const float *deq, const int32_t *rowsum, int64_t m, int64_t k,
                          const uint8_t *w, int64_t n, const bl::Epilogue &ep, float *y, int32_t *acc_out,
                          int32_t path, int32_t *split_ws, hipStream_t stream) {
  const bool decode = path == BITLINEAR_PATH_DECODE || (path == BITLINEAR_PATH_AUTO && m <= 16);
  if (decode) return launched(bl::launch_gemv_decode(codes, w, deq, rowsum, m, n, k, ep, y, acc_out, stream),
                              "decode kernel");
  return launched(bl::launch_gemm_prefill(codes, w, deq, rowsum, m, n, k, ep, y, acc_out, split_ws, stream),
                  "prefill kernel");
}

}  // namespace

extern "C" {

const char *bitlinear_status_str(bitlinear_status s) {
  switch (s) {
    case BITLINEAR_OK: return "ok";
    case BITLINEAR_ERR_NULL: return "null pointer";
    case BITLINEAR_ERR_SHAPE: return "bad shape";
    case BITLINEAR_ERR_ALIGN: return "misaligned pointer";
    case BITLINEAR_ERR_WORKSPACE: return "workspace too small";
    case BITLINEAR_ERR_DEVICE: return "device error";
    case BITLINEAR_ERR_ARG: return "bad argument";
  }
  return "unknown status";
}

const char *bitlinear_last_error(void) { return g_err.c_str(); }

bitlinear_status bitlinear_probe_read(const void *src, int64_t bytes, int64_t grid, uint32_t *sink, void *stream) {
  g_err.clear();
  if (bytes != 0 && (!src || !sink)) return fail(BITLINEAR_ERR_NULL, "src and sink are required");
  if (bytes < 0 || bytes % 16 != 0) return fail(BITLINEAR_ERR_SHAPE, "bytes must be a non-negative multiple of 16");
  if (bytes != 0 && !aligned16(src)) return fail(BITLINEAR_ERR_ALIGN, "src must be 16-byte aligned");
  if (bytes == 0) return BITLINEAR_OK;
  BL_TRY(check_device());
  return launched(bl::launch_probe_read(src, bytes, sink, grid, as_stream(stream)), "probe read");
}

static bitlinear_status probe_mfma(int32_t iters, int64_t workgroups, bool varied, int32_t *sink, void *stream) {
  g_err.clear();
  if (!sink) return fail(BITLINEAR_ERR_NULL, "sink is required");
  if (iters <= 0 || workgroups <= 0 || workgroups > 65536)
    return fail(BITLINEAR_ERR_SHAPE, "iters > 0 and 0 < workgroups <= 65536");
  BL_TRY(check_device());
  return launched(bl::launch_probe_mfma(iters, workgroups, varied, sink, as_stream(stream)), "probe mfma");
}

bitlinear_status bitlinear_probe_mfma(int32_t iters, int64_t workgroups, int32_t *sink, void *stream) {
  return probe_mfma(iters, workgroups, false, sink, stream);
}

bitlinear_status bitlinear_probe_mfma_varied(int32_t iters, int64_t workgroups, int32_t *sink, void *stream) {
  return probe_mfma(iters, workgroups, true, sink, stream);
}

int32_t bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

// ---------------------------------------------------------------- weights
size_t bitlinear_quantize_weights_workspace_bytes(int64_t n, int64_t k) {
  if (n < 0 || k <= 0) return 0;
  return align256(bl::absmean_partials(k, &n, 1) * sizeof(double));
}

bitlinear_status bitlinear_quantize_weights(const float *w, int64_t n, int64_t k, const double *gamma_in,
                                            uint8_t *w_packed, double *gamma_out, void *workspace,
                                            size_t workspace_bytes, void *stream) {
  g_err.clear();
  if (!w || !w_packed || !gamma_out) return fail(BITLINEAR_ERR_NULL, "w, w_packed and gamma_out are required");
  if (n < 0 || k <= 0 || k % 16 != 0 || n > kMaxDim || k > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "n = %lld, k = %lld: need n >= 0, k > 0, k %% 16 == 0", (long long)n,
                (long long)k);
  if (!aligned16(w) || !aligned16(w_packed)) return fail(BITLINEAR_ERR_ALIGN, "w and w_packed must be 16-byte aligned");
  const size_t need = bitlinear_quantize_weights_workspace_bytes(n, k);
  if (!gamma_in && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  BL_TRY(check_device());
  hipStream_t s = as_stream(stream);
  if (gamma_in) {
    BL_TRY(launched(bl::launch_copy_gamma(gamma_in, gamma_out, s), "copy gamma"));
  } else {
    BL_TRY(launched(bl::launch_absmean(w, k, &n, 1, static_cast<double *>(workspace), gamma_out, s), "absmean"));
  }
  return launched(bl::launch_ternarize_pack(w, k, &n, 1, gamma_out, w_packed, s), "ternarize");
}

bitlinear_status bitlinear_validate_packed(const uint8_t *w_packed, int64_t n, int64_t k, int64_t *n_bad,
                                           void *stream) {
  g_err.clear();
  if (!w_packed || !n_bad) return fail(BITLINEAR_ERR_NULL, "w_packed and n_bad are required");
  if (n < 0 || k <= 0 || k % 16 != 0) return fail(BITLINEAR_ERR_SHAPE, "need n >= 0, k > 0, k %% 16 == 0");
  if (!aligned16(w_packed)) return fail(BITLINEAR_ERR_ALIGN, "w_packed must be 16-byte aligned");
  BL_TRY(check_device());
  return launched(bl::launch_validate_packed(w_packed, n, k, n_bad, as_stream(stream)), "validate");
}

// ---------------------------------------------------------------- activations
bitlinear_status bitlinear_quantize_acts(const float *x, int64_t m, int64_t k, int32_t mode, const float *norm_gain,
                                         float eps, int8_t *codes, float *deq, int32_t *code_rowsum, void *stream) {
  g_err.clear();
  if (m != 0 && (!x || !codes || !deq)) return fail(BITLINEAR_ERR_NULL, "x, codes and deq are required");
  if (m < 0 || k <= 0 || k % 16 != 0 || m > kMaxDim || k > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "m = %lld, k = %lld: need m >= 0, k > 0, k %% 16 == 0", (long long)m,
                (long long)k);
  if (mode != BITLINEAR_ACT_ABSMAX && mode != BITLINEAR_ACT_RMSNORM && mode != BITLINEAR_ACT_RELU2_RMSNORM)
    return fail(BITLINEAR_ERR_ARG, "unknown mode %d", mode);
  if (!aligned16(x) || !aligned16(codes) || (norm_gain && !aligned16(norm_gain)))
    return fail(BITLINEAR_ERR_ALIGN, "x, codes and norm_gain must be 16-byte aligned");
  if (m == 0) return BITLINEAR_OK;
  BL_TRY(check_device());
  const int64_t ld = mode == BITLINEAR_ACT_RELU2_RMSNORM ? 2 * k : k;
  return launched(bl::launch_quant_acts(mode, x, nullptr, ld, m, k, norm_gain, eps, 0, 1, 1, nullptr, codes, deq,
                                        code_rowsum, as_stream(stream)),
                  "quantize_acts");
}

// ---------------------------------------------------------------- forward
size_t bitlinear_forward_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t quantize_inside) {
  if (m < 0 || k < 0 || n < 0) return 0;
  size_t b = align256((size_t)m * sizeof(int32_t));  // row sums
  if (quantize_inside) b += align256((size_t)(m * k)) + align256((size_t)m * sizeof(float));
  b += align256(bl::gemm_prefill_workspace_bytes(m, n, k));  // split-K partial sums
  return b;
}

}  // extern "C"

namespace {

// Argument checks shared by the packed and the online forward.
bitlinear_status check_forward_args(const float *x, const int8_t *codes_in, const float *deq_in, int64_t m,
                                    int64_t k, const void *w, int64_t n, float *y, int32_t path) {
  if (!w || (m != 0 && !y)) return fail(BITLINEAR_ERR_NULL, "the weights and y are required");
  if (m != 0 && !x && (!codes_in || !deq_in)) return fail(BITLINEAR_ERR_NULL, "give x, or codes_in and deq_in");
  if (m < 0 || n <= 0 || k <= 0 || k % 16 != 0 || m > kMaxDim || n > kMaxDim || k > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "m = %lld, n = %lld, k = %lld: need m >= 0, n > 0, k > 0, k %% 16 == 0",
                (long long)m, (long long)n, (long long)k);
  if (path != BITLINEAR_PATH_AUTO && path != BITLINEAR_PATH_DECODE && path != BITLINEAR_PATH_PREFILL)
    return fail(BITLINEAR_ERR_ARG, "unknown path %d", path);
  if (path == BITLINEAR_PATH_DECODE && m > 16) return fail(BITLINEAR_ERR_SHAPE, "the decode path takes m <= 16");
  if ((x && !aligned16(x)) || (codes_in && !x && !aligned16(codes_in)) || !aligned16(w) || !aligned16(y))
    return fail(BITLINEAR_ERR_ALIGN, "x, codes_in, the weights and y must be 16-byte aligned");
  return BITLINEAR_OK;
}

// The projection once the arguments are checked: quantize x (or take the
// given codes), then contract with the packed weights. ws holds
// bitlinear_forward_workspace_bytes(m, n, k, x != NULL) bytes.
bitlinear_status forward_impl(const float *x, const int8_t *codes_in, const float *deq_in, const int32_t *rowsum_in,
                              int64_t m, int64_t k, const uint8_t *w_packed, int64_t n, const bl::Epilogue &ep,
                              float *y, int32_t *acc_out, int32_t path, char *ws, hipStream_t s) {
  int32_t *rowsum = reinterpret_cast<int32_t *>(ws);
  ws += align256((size_t)m * sizeof(int32_t));
  const size_t split_bytes = bl::gemm_prefill_workspace_bytes(m, n, k);
  int32_t *split_ws = split_bytes ? reinterpret_cast<int32_t *>(ws) : nullptr;
  ws += align256(split_bytes);
  const int8_t *codes = codes_in;
  const float *deq = deq_in;
  if (x) {
    int8_t *c = reinterpret_cast<int8_t *>(ws);
    ws += align256((size_t)(m * k));
    float *d = reinterpret_cast<float *>(ws);
    BL_TRY(launched(bl::launch_quant_acts(BITLINEAR_ACT_ABSMAX, x, nullptr, k, m, k, nullptr, 0.0f, 0, 1, 1, nullptr,
                                          c, d, rowsum, s),
                    "quantize_acts"));
    codes = c;
    deq = d;
  } else if (rowsum_in) {
    rowsum = const_cast<int32_t *>(rowsum_in);
  } else {
    BL_TRY(launched(bl::launch_code_rowsum(codes, m, k, rowsum, s), "code row sums"));
  }
  return contract(codes, deq, rowsum, m, k, w_packed, n, ep, y, acc_out, path, split_ws, s);
}

}  // namespace

extern "C" {

bitlinear_status bitlinear_forward(const float *x, const int8_t *codes_in, const float *deq_in,
                                   const int32_t *rowsum_in, int64_t m, int64_t k, const uint8_t *w_packed, int64_t n,
                                   const float *gamma, const int64_t *seg_end, int32_t n_seg, float *y,
                                   int32_t *acc_out, int32_t path, void *workspace, size_t workspace_bytes,
                                   void *stream) {
  g_err.clear();
  BL_TRY(check_forward_args(x, codes_in, deq_in, m, k, w_packed, n, y, path));
  bl::Epilogue ep;
  BL_TRY(check_segments(gamma, seg_end, n_seg, n, &ep));
  const size_t need = bitlinear_forward_workspace_bytes(m, n, k, x != nullptr);
  if (m > 0 && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  if (m == 0) return BITLINEAR_OK;
  BL_TRY(check_device());
  return forward_impl(x, codes_in, deq_in, rowsum_in, m, k, w_packed, n, ep, y, acc_out, path,
                      static_cast<char *>(workspace), as_stream(stream));
}

// ---------------------------------------------------------------- online mode
size_t bitlinear_forward_online_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t quantize_inside,
                                                const int64_t *seg_end, int32_t n_seg) {
  if (m < 0 || n < 0 || k < 0 || !seg_end || n_seg < 1 || n_seg > BITLINEAR_MAX_SEGMENTS) return 0;
  const size_t partials = bl::absmean_partials(k, seg_end, n_seg);  // every segment's, side by side
  return bitlinear_forward_workspace_bytes(m, n, k, quantize_inside) + align256((size_t)(n * (k / 4))) +
         align256(sizeof(double) * BITLINEAR_MAX_SEGMENTS) + align256(partials * sizeof(double));
}

bitlinear_status bitlinear_forward_online(const float *x, const int8_t *codes_in, const float *deq_in,
                                          const int32_t *rowsum_in, int64_t m, int64_t k, const void *w_master,
                                          int32_t master_dtype, int64_t n, const int64_t *seg_end, int32_t n_seg,
                                          double *gamma_out, float *y, int32_t *acc_out, int32_t path,
                                          void *workspace, size_t workspace_bytes, void *stream) {
  g_err.clear();
  BL_TRY(check_forward_args(x, codes_in, deq_in, m, k, w_master, n, y, path));
  if (master_dtype != BITLINEAR_MASTER_F32 && master_dtype != BITLINEAR_MASTER_BF16)
    return fail(BITLINEAR_ERR_ARG, "unknown master dtype %d", master_dtype);
  bl::Epilogue ep;
  BL_TRY(make_segments(nullptr, seg_end, n_seg, n, &ep));
  const size_t need = bitlinear_forward_online_workspace_bytes(m, n, k, x != nullptr, seg_end, n_seg);
  if (!workspace || workspace_bytes < need) return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  BL_TRY(check_device());
  hipStream_t s = as_stream(stream);
  // layout: [forward workspace][packed weights][gammas][absmean partials]
  char *ws_fwd = static_cast<char *>(workspace);
  char *ws = ws_fwd + bitlinear_forward_workspace_bytes(m, n, k, x != nullptr);
  uint8_t *packed = reinterpret_cast<uint8_t *>(ws);
  ws += align256((size_t)(n * (k / 4)));
  double *gam = gamma_out ? gamma_out : reinterpret_cast<double *>(ws);
  ws += align256(sizeof(double) * BITLINEAR_MAX_SEGMENTS);
  double *partials = reinterpret_cast<double *>(ws);
  const bool bf16 = master_dtype == BITLINEAR_MASTER_BF16;
  const bool decode = path == BITLINEAR_PATH_DECODE || path == BITLINEAR_PATH_AUTO;
  if (m == 1 && decode && bl::online_dot_supported(n, k, bf16)) {
    // one token: the gammas, then the codes formed from the masters inside the
    // contraction (no packed copy written)
    if (bf16)
      BL_TRY(launched(bl::launch_absmean_bf16(static_cast<const uint16_t *>(w_master), k, seg_end, n_seg, partials,
                                              gam, s),
                      "absmean"));
    else
      BL_TRY(launched(bl::launch_absmean(static_cast<const float *>(w_master), k, seg_end, n_seg, partials, gam, s),
                      "absmean"));
    // the token's codes, deq and row sum: given, or quantized into the
    // forward's workspace (row sums first, as the packed forward lays it out)
    int32_t *rowsum = reinterpret_cast<int32_t *>(ws_fwd);
    const int8_t *codes = codes_in;
    const float *deq = deq_in;
    if (x) {
      int8_t *c = reinterpret_cast<int8_t *>(ws_fwd + align256(sizeof(int32_t)));
      float *d = reinterpret_cast<float *>(ws_fwd + align256(sizeof(int32_t)) + align256((size_t)k));
      BL_TRY(launched(bl::launch_quant_acts(BITLINEAR_ACT_ABSMAX, x, nullptr, k, 1, k, nullptr, 0.0f, 0, 1, 1,
                                            nullptr, c, d, rowsum, s),
                      "quantize_acts"));
      codes = c;
      deq = d;
    } else if (rowsum_in) {
      rowsum = const_cast<int32_t *>(rowsum_in);
    } else {
      BL_TRY(launched(bl::launch_code_rowsum(codes, 1, k, rowsum, s), "code row sums"));
    }
    ep.gamma_dev = gam;
    if (bf16)
      return launched(bl::launch_online_dot_bf16(codes, deq, rowsum, static_cast<const uint16_t *>(w_master), n, k, ep,
                                                 y, acc_out, s),
                      "online contraction");
    return launched(bl::launch_online_dot(codes, deq, rowsum, static_cast<const float *>(w_master), n, k, ep, y,
                                          acc_out, s),
                    "online contraction");
  }
  // every segment in one launch per pass: partial sums, gammas, ternary codes
  if (master_dtype == BITLINEAR_MASTER_BF16) {
    const uint16_t *w = static_cast<const uint16_t *>(w_master);
    BL_TRY(launched(bl::launch_absmean_bf16(w, k, seg_end, n_seg, partials, gam, s), "absmean"));
    BL_TRY(launched(bl::launch_ternarize_pack_bf16(w, k, seg_end, n_seg, gam, packed, s), "ternarize"));
  } else {
    const float *w = static_cast<const float *>(w_master);
    BL_TRY(launched(bl::launch_absmean(w, k, seg_end, n_seg, partials, gam, s), "absmean"));
    BL_TRY(launched(bl::launch_ternarize_pack(w, k, seg_end, n_seg, gam, packed, s), "ternarize"));
  }
  if (m == 0) return BITLINEAR_OK;
  ep.gamma_dev = gam;
  return forward_impl(x, codes_in, deq_in, rowsum_in, m, k, packed, n, ep, y, acc_out, path, ws_fwd, s);
}

// ---------------------------------------------------------------- gated up-projection
namespace {
bool glu_fused(int64_t m, int64_t inter, int64_t k, int32_t path) {
  const bool decode = path == BITLINEAR_PATH_DECODE || (path == BITLINEAR_PATH_AUTO && m <= 16);
  return !decode && bl::gemm_glu_supported(m, inter, k);
}
}  // namespace

size_t bitlinear_forward_relu2_glu_workspace_bytes(int64_t m, int64_t inter, int64_t k, int32_t quantize_inside,
                                                   int32_t path) {
  if (m < 0 || k < 0 || inter < 0) return 0;
  size_t b = align256((size_t)m * sizeof(int32_t));  // row sums
  if (quantize_inside) b += align256((size_t)(m * k)) + align256((size_t)m * sizeof(float));
  if (!glu_fused(m, inter, k, path))
    b += align256((size_t)(m * 2 * inter) * sizeof(float)) + align256(bl::gemm_prefill_workspace_bytes(m, 2 * inter, k));
  return b;
}

bitlinear_status bitlinear_forward_relu2_glu(const float *x, const int8_t *codes_in, const float *deq_in,
                                             const int32_t *rowsum_in, int64_t m, int64_t k,
                                             const uint8_t *w_packed, int64_t inter, const float *gamma, float *y,
                                             int32_t path, void *workspace, size_t workspace_bytes, void *stream) {
  g_err.clear();
  if (!w_packed || !gamma || (m != 0 && !y)) return fail(BITLINEAR_ERR_NULL, "w_packed, gamma and y are required");
  if (m != 0 && !x && (!codes_in || !deq_in)) return fail(BITLINEAR_ERR_NULL, "give x, or codes_in and deq_in");
  if (m < 0 || inter <= 0 || inter % 4 != 0 || k <= 0 || k % 16 != 0 || m > kMaxDim || 2 * inter > kMaxDim ||
      k > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "m = %lld, inter = %lld, k = %lld: need m >= 0, inter > 0, inter %% 4 == 0, "
                "k > 0, k %% 16 == 0", (long long)m, (long long)inter, (long long)k);
  if (path != BITLINEAR_PATH_AUTO && path != BITLINEAR_PATH_DECODE && path != BITLINEAR_PATH_PREFILL)
    return fail(BITLINEAR_ERR_ARG, "unknown path %d", path);
  if (path == BITLINEAR_PATH_DECODE && m > 16) return fail(BITLINEAR_ERR_SHAPE, "the decode path takes m <= 16");
  if ((x && !aligned16(x)) || (codes_in && !x && !aligned16(codes_in)) || !aligned16(w_packed) || !aligned16(y))
    return fail(BITLINEAR_ERR_ALIGN, "x, codes_in, w_packed and y must be 16-byte aligned");
  const int64_t seg[2] = {inter, 2 * inter};
  bl::Epilogue ep;
  BL_TRY(check_segments(gamma, seg, 2, 2 * inter, &ep));
  const size_t need = bitlinear_forward_relu2_glu_workspace_bytes(m, inter, k, x != nullptr, path);
  if (m > 0 && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  if (m == 0) return BITLINEAR_OK;
  BL_TRY(check_device());
  hipStream_t s = as_stream(stream);
  char *ws = static_cast<char *>(workspace);
  int32_t *rowsum = reinterpret_cast<int32_t *>(ws);
  ws += align256((size_t)m * sizeof(int32_t));
  const int8_t *codes = codes_in;
  const float *deq = deq_in;
  if (x) {
    int8_t *c = reinterpret_cast<int8_t *>(ws);
    ws += align256((size_t)(m * k));
    float *d = reinterpret_cast<float *>(ws);
    ws += align256((size_t)m * sizeof(float));
    BL_TRY(launched(bl::launch_quant_acts(BITLINEAR_ACT_ABSMAX, x, nullptr, k, m, k, nullptr, 0.0f, 0, 1, 1, nullptr,
                                          c, d, rowsum, s),
                    "quantize_acts"));
    codes = c;
    deq = d;
  } else if (rowsum_in) {
    rowsum = const_cast<int32_t *>(rowsum_in);
  } else {
    BL_TRY(launched(bl::launch_code_rowsum(codes, m, k, rowsum, s), "code row sums"));
  }
  if (glu_fused(m, inter, k, path))
    return launched(bl::launch_gemm_glu(codes, w_packed, deq, rowsum, m, inter, k, ep, y, s), "gated prefill kernel");
  float *gu = reinterpret_cast<float *>(ws);
  ws += align256((size_t)(m * 2 * inter) * sizeof(float));
  int32_t *split_ws = bl::gemm_prefill_workspace_bytes(m, 2 * inter, k) ? reinterpret_cast<int32_t *>(ws) : nullptr;
  BL_TRY(contract(codes, deq, rowsum, m, k, w_packed, 2 * inter, ep, gu, nullptr, path, split_ws, s));
  return launched(bl::launch_relu2_glu(gu, m, inter, y, s), "relu2 gating");
}

// ---------------------------------------------------------------- the model's ends
bitlinear_status bitlinear_embed(const int64_t *ids, int64_t m, const uint16_t *table, int64_t vocab, int64_t k,
                                 float *x, void *stream) {
  g_err.clear();
  if (m != 0 && (!ids || !table || !x)) return fail(BITLINEAR_ERR_NULL, "ids, table and x are required");
  if (m < 0 || vocab <= 0 || !bl::lm_head_supported(k) || m > kMaxDim || vocab > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "m = %lld, vocab = %lld, k = %lld: need k %% 8 == 0, 0 < k <= 4096",
                (long long)m, (long long)vocab, (long long)k);
  if (m == 0) return BITLINEAR_OK;
  if (!aligned16(table) || !aligned16(x)) return fail(BITLINEAR_ERR_ALIGN, "table and x must be 16-byte aligned");
  BL_TRY(check_device());
  return launched(bl::launch_embed(ids, m, table, vocab, k, x, as_stream(stream)), "embedding gather");
}

size_t bitlinear_lm_head_workspace_bytes(int64_t m, int64_t k) {
  return m > 0 && k > 0 ? align256((size_t)(m * k) * sizeof(uint16_t)) : 0;
}

bitlinear_status bitlinear_lm_head(const float *x, int64_t m, int64_t k, const float *norm_gain, float eps,
                                   const uint16_t *w_head, int64_t n_vocab, float *logits, uint16_t *normed_out,
                                   void *workspace, size_t workspace_bytes, void *stream) {
  g_err.clear();
  if (m != 0 && (!x || !w_head || !logits)) return fail(BITLINEAR_ERR_NULL, "x, w_head and logits are required");
  if (m < 0 || n_vocab <= 0 || !bl::lm_head_supported(k) || m > kMaxDim || n_vocab > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "m = %lld, k = %lld, n_vocab = %lld: need k %% 8 == 0, 0 < k <= 4096",
                (long long)m, (long long)k, (long long)n_vocab);
  if (!(eps >= 0.0f)) return fail(BITLINEAR_ERR_ARG, "eps must be >= 0");
  if (m != 0 && (!aligned16(x) || !aligned16(w_head) || (normed_out && !aligned16(normed_out))))
    return fail(BITLINEAR_ERR_ALIGN, "x, w_head and normed_out must be 16-byte aligned");
  const size_t need = normed_out ? 0 : bitlinear_lm_head_workspace_bytes(m, k);
  if (m > 0 && need > 0 && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  if (m == 0) return BITLINEAR_OK;
  BL_TRY(check_device());
  hipStream_t s = as_stream(stream);
  uint16_t *o = normed_out ? normed_out : static_cast<uint16_t *>(workspace);
  BL_TRY(launched(bl::launch_final_norm(x, m, k, norm_gain, eps, o, s), "final norm"));
  return launched(bl::launch_lm_head(o, m, k, w_head, n_vocab, logits, s), "lm_head");
}

// ---------------------------------------------------------------- attention with a KV cache
bitlinear_status bitlinear_rope_table(double theta, int32_t head_dim, int64_t n_pos, float *table) {
  g_err.clear();
  if (!table) return fail(BITLINEAR_ERR_NULL, "table is required");
  if (head_dim <= 0 || head_dim % 2 != 0 || n_pos <= 0 || n_pos > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "head_dim = %d, n_pos = %lld", head_dim, (long long)n_pos);
  if (!(theta > 0.0) || !std::isfinite(theta)) return fail(BITLINEAR_ERR_ARG, "theta must be finite and > 0");
  const int half = head_dim / 2;
  for (int64_t p = 0; p < n_pos; ++p)
    for (int e = 0; e < half; ++e) {
      const double ang = (double)p * std::pow(theta, -(2.0 * e) / (double)head_dim);
      table[2 * (p * half + e)] = (float)std::cos(ang);
      table[2 * (p * half + e) + 1] = (float)std::sin(ang);
    }
  return BITLINEAR_OK;
}

bitlinear_status bitlinear_rope(float *x, int64_t m, int64_t ld, int64_t col0, int32_t n_heads, int32_t head_dim,
                                const int64_t *pos, const float *rope_table, int64_t n_pos, void *stream) {
  g_err.clear();
  if (m != 0 && (!x || !pos || !rope_table)) return fail(BITLINEAR_ERR_NULL, "x, pos and rope_table are required");
  if (m < 0 || n_heads <= 0 || head_dim <= 0 || head_dim % 2 != 0 || col0 < 0 ||
      col0 + (int64_t)n_heads * head_dim > ld || m > kMaxDim || ld > kMaxDim || n_pos <= 0 || n_pos > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "m = %lld, ld = %lld, col0 = %lld, %d heads of %d, n_pos = %lld", (long long)m,
                (long long)ld, (long long)col0, n_heads, head_dim, (long long)n_pos);
  if (m != 0 && reinterpret_cast<uintptr_t>(rope_table) % 8 != 0)
    return fail(BITLINEAR_ERR_ALIGN, "rope_table must be 8-byte aligned");
  if (m == 0) return BITLINEAR_OK;
  BL_TRY(check_device());
  return launched(bl::launch_rope(x, m, ld, col0, n_heads, head_dim, pos,
                                  reinterpret_cast<const float2 *>(rope_table), n_pos, as_stream(stream)),
                  "rope");
}

bitlinear_status bitlinear_kv_append(const float *k, const float *v, int64_t m, int64_t ld, int32_t n_kv,
                                     int32_t head_dim, const int64_t *slot, const int64_t *pos, uint16_t *k_cache,
                                     uint16_t *v_cache, int64_t n_slots, int64_t t_max, void *stream) {
  g_err.clear();
  if (m != 0 && (!k || !v || !slot || !pos || !k_cache || !v_cache))
    return fail(BITLINEAR_ERR_NULL, "k, v, slot, pos and both caches are required");
  if (m < 0 || n_kv <= 0 || head_dim <= 0 || (int64_t)n_kv * head_dim > ld || n_slots <= 0 || t_max <= 0 ||
      m > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "m = %lld, ld = %lld, %d kv heads of %d, %lld slots of %lld", (long long)m,
                (long long)ld, n_kv, head_dim, (long long)n_slots, (long long)t_max);
  if (m == 0) return BITLINEAR_OK;
  BL_TRY(check_device());
  return launched(bl::launch_kv_append(k, v, m, ld, n_kv, head_dim, slot, pos, k_cache, v_cache, n_slots, t_max,
                                       as_stream(stream)),
                  "kv append");
}

size_t bitlinear_attention_workspace_bytes(int64_t m, int32_t n_heads, int64_t t_max) {
  if (m <= 0 || n_heads <= 0 || t_max <= 0) return 0;
  return align256(bl::attention_workspace_floats(m, n_heads, t_max) * sizeof(float));
}

bitlinear_status bitlinear_attention_decode(const float *q, int64_t m, int64_t ldq, int32_t n_heads, int32_t n_kv,
                                            int32_t head_dim, const uint16_t *k_cache, const uint16_t *v_cache,
                                            int64_t n_slots, int64_t t_max, const int64_t *slot, const int64_t *pos,
                                            float *out, int64_t ldo, void *workspace, size_t workspace_bytes,
                                            void *stream) {
  g_err.clear();
  if (m != 0 && (!q || !k_cache || !v_cache || !slot || !pos || !out))
    return fail(BITLINEAR_ERR_NULL, "q, the caches, slot, pos and out are required");
  if (m < 0 || !bl::attention_supported(n_heads, n_kv, head_dim) || (int64_t)n_heads * head_dim > ldq ||
      (int64_t)n_heads * head_dim > ldo || n_slots <= 0 || t_max <= 0 || m > kMaxDim || t_max > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "m = %lld, %d heads / %d kv heads of %d (need 128, at most 8 per kv head), "
                "ldq = %lld, ldo = %lld", (long long)m, n_heads, n_kv, head_dim, (long long)ldq, (long long)ldo);
  const size_t need = bitlinear_attention_workspace_bytes(m, n_heads, t_max);
  if (m > 0 && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  if (m == 0) return BITLINEAR_OK;
  BL_TRY(check_device());
  return launched(bl::launch_attention(q, m, ldq, n_heads, n_kv, head_dim, k_cache, v_cache, n_slots, t_max, slot, pos,
                                       out, ldo, static_cast<float *>(workspace), as_stream(stream)),
                  "attention");
}

// ---------------------------------------------------------------- five codes per byte
size_t bitlinear_base3_row_bytes(int64_t k) { return k > 0 ? (size_t)(16 * ((k + 79) / 80)) : 0; }

bitlinear_status bitlinear_pack_base3(const uint8_t *w_packed, int64_t n, int64_t k, uint8_t *w_base3,
                                      void *stream) {
  g_err.clear();
  if (!w_packed || !w_base3) return fail(BITLINEAR_ERR_NULL, "w_packed and w_base3 are required");
  if (n <= 0 || k <= 0 || k % 16 != 0 || n > kMaxDim || k > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "n = %lld, k = %lld: need n > 0, k > 0, k %% 16 == 0", (long long)n,
                (long long)k);
  if (!aligned16(w_packed) || !aligned16(w_base3))
    return fail(BITLINEAR_ERR_ALIGN, "w_packed and w_base3 must be 16-byte aligned");
  BL_TRY(check_device());
  return launched(bl::launch_pack_base3(w_packed, n, k, w_base3, as_stream(stream)), "pack_base3");
}

size_t bitlinear_forward_base3_workspace_bytes(int64_t m, int64_t k, int32_t quantize_inside) {
  if (m <= 0 || k <= 0 || !quantize_inside) return 0;
  // codes, deq and the row sums the quantization kernel also writes
  return align256((size_t)(m * k)) + align256((size_t)m * sizeof(float)) + align256((size_t)m * sizeof(int32_t));
}

bitlinear_status bitlinear_forward_base3(const float *x, const int8_t *codes_in, const float *deq_in, int64_t m,
                                         int64_t k, const uint8_t *w_base3, int64_t n, const float *gamma,
                                         const int64_t *seg_end, int32_t n_seg, float *y, int32_t *acc_out,
                                         void *workspace, size_t workspace_bytes, void *stream) {
  g_err.clear();
  BL_TRY(check_forward_args(x, codes_in, deq_in, m, k, w_base3, n, y, BITLINEAR_PATH_DECODE));
  if (m > 4 || k > 8192)
    return fail(BITLINEAR_ERR_SHAPE, "m = %lld, k = %lld: the base-3 path takes m <= 4 and k <= 8192", (long long)m,
                (long long)k);
  bl::Epilogue ep;
  BL_TRY(check_segments(gamma, seg_end, n_seg, n, &ep));
  const size_t need = bitlinear_forward_base3_workspace_bytes(m, k, x != nullptr);
  if (m > 0 && need > 0 && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  if (m == 0) return BITLINEAR_OK;
  BL_TRY(check_device());
  hipStream_t s = as_stream(stream);
  const int8_t *codes = codes_in;
  const float *deq = deq_in;
  if (x) {
    char *ws = static_cast<char *>(workspace);
    int8_t *c = reinterpret_cast<int8_t *>(ws);
    ws += align256((size_t)(m * k));
    float *d = reinterpret_cast<float *>(ws);
    ws += align256((size_t)m * sizeof(float));
    int32_t *rs = reinterpret_cast<int32_t *>(ws);
    BL_TRY(launched(bl::launch_quant_acts(BITLINEAR_ACT_ABSMAX, x, nullptr, k, m, k, nullptr, 0.0f, 0, 1, 1, nullptr,
                                          c, d, rs, s),
                    "quantize_acts"));
    codes = c;
    deq = d;
  }
  return launched(bl::launch_gemv_b3(codes, w_base3, deq, m, n, k, ep, y, acc_out, s), "base-3 decode kernel");
}

}  // extern "C"

// ---------------------------------------------------------------- blocks
namespace {

struct BlockBufs {
  int8_t *codes;
  float *deq;
  int32_t *rowsum;
  float *deq2;      // second set, so that a quantization can read the previous
  int32_t *rowsum2; // stage's deq and row sums while it writes its own
  float *qkv, *o, *h, *x, *gu, *d;
  int32_t *split;  // split-K partial sums of the widest projection, or NULL
  float *att;      // cached decoder: attention output [m][H]
  float *attn_ws;  // cached decoder: attention chunk partials
  float2 *rope_cs; // cached decoder: [m][head_dim/2] (cosine, sine) of each token's rotated pairs
};

bool is_decoder(int32_t kind) { return kind == BITLINEAR_BLOCK_DECODER || kind == BITLINEAR_BLOCK_DECODER_CACHED; }

size_t block_layout(const bitlinear_block *blk, int64_t m, BlockBufs *b, char *base) {
  const int64_t H = blk->hidden, I = blk->intermediate;
  const bool dec = is_decoder(blk->kind), cached = blk->kind == BITLINEAR_BLOCK_DECODER_CACHED;
  const int64_t Q = dec ? H + 2 * (int64_t)blk->n_kv_heads * blk->head_dim : 0;
  const int64_t widest = H > I ? H : I;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *p = base ? base + off : nullptr;
    off += align256(bytes);
    return p;
  };
  BlockBufs t;
  t.codes = reinterpret_cast<int8_t *>(take((size_t)(m * widest)));
  t.deq = reinterpret_cast<float *>(take((size_t)m * 4));
  t.rowsum = reinterpret_cast<int32_t *>(take((size_t)m * 4));
  t.deq2 = reinterpret_cast<float *>(take((size_t)m * 4));
  t.rowsum2 = reinterpret_cast<int32_t *>(take((size_t)m * 4));
  t.gu = reinterpret_cast<float *>(take((size_t)(m * 2 * I) * 4));
  t.qkv = reinterpret_cast<float *>(take(dec ? (size_t)(m * Q) * 4 : 0));
  t.o = reinterpret_cast<float *>(take(dec ? (size_t)(m * H) * 4 : 0));
  t.h = reinterpret_cast<float *>(take(dec ? (size_t)(m * H) * 4 : 0));
  t.x = reinterpret_cast<float *>(take(dec ? (size_t)(m * H) * 4 : 0));
  t.d = reinterpret_cast<float *>(take(dec ? (size_t)(m * H) * 4 : 0));
  size_t split = bl::gemm_prefill_workspace_bytes(m, 2 * I, H);
  const size_t sd = bl::gemm_prefill_workspace_bytes(m, H, I);
  if (sd > split) split = sd;
  if (dec) {
    const size_t sq = bl::gemm_prefill_workspace_bytes(m, Q, H), so = bl::gemm_prefill_workspace_bytes(m, H, H);
    if (sq > split) split = sq;
    if (so > split) split = so;
  }
  t.split = reinterpret_cast<int32_t *>(split ? take(split) : nullptr);
  t.att = reinterpret_cast<float *>(take(cached ? (size_t)(m * H) * 4 : 0));
  t.attn_ws = reinterpret_cast<float *>(
      take(cached ? bl::attention_workspace_floats(m, blk->n_heads, blk->t_max) * sizeof(float) : 0));
  t.rope_cs = reinterpret_cast<float2 *>(take(cached ? (size_t)(m * (blk->head_dim / 2)) * sizeof(float2) : 0));
  if (b) *b = t;
  return off;
}

bitlinear_status check_block(const bitlinear_block *blk) {
  if (!blk || !blk->layers) return fail(BITLINEAR_ERR_NULL, "blk and blk->layers are required");
  if (blk->kind != BITLINEAR_BLOCK_FFN && !is_decoder(blk->kind))
    return fail(BITLINEAR_ERR_ARG, "unknown block kind %d", blk->kind);
  const int64_t H = blk->hidden, I = blk->intermediate;
  if (blk->n_layers < 1 || H <= 0 || I <= 0 || H % 16 || I % 16 || H > kMaxDim || I > kMaxDim)
    return fail(BITLINEAR_ERR_SHAPE, "need n_layers >= 1 and hidden, intermediate positive multiples of 16");
  if (blk->kind == BITLINEAR_BLOCK_FFN && blk->n_layers != 1) return fail(BITLINEAR_ERR_SHAPE, "an FFN block has 1 layer");
  if (is_decoder(blk->kind)) {
    if (blk->n_heads <= 0 || blk->n_kv_heads <= 0 || blk->head_dim <= 0 || blk->head_dim % 4 ||
        blk->n_heads % blk->n_kv_heads || (int64_t)blk->n_heads * blk->head_dim != H)
      return fail(BITLINEAR_ERR_SHAPE, "need n_heads * head_dim == hidden, n_kv_heads | n_heads, head_dim %% 4 == 0");
    if (((int64_t)blk->n_kv_heads * blk->head_dim) % 16)
      return fail(BITLINEAR_ERR_SHAPE, "n_kv_heads * head_dim must be a multiple of 16");
  }
  if (blk->kind == BITLINEAR_BLOCK_DECODER_CACHED) {
    if (!bl::attention_supported(blk->n_heads, blk->n_kv_heads, blk->head_dim))
      return fail(BITLINEAR_ERR_SHAPE, "the cached decoder needs head_dim 128 and at most 8 heads per kv head");
    if (!blk->slot || !blk->pos) return fail(BITLINEAR_ERR_NULL, "slot and pos are required");
    if (blk->n_slots <= 0 || blk->t_max <= 0 || blk->n_slots > kMaxDim || blk->t_max > kMaxDim)
      return fail(BITLINEAR_ERR_SHAPE, "n_slots = %lld, t_max = %lld", (long long)blk->n_slots,
                  (long long)blk->t_max);
    if (!blk->rope_table) return fail(BITLINEAR_ERR_NULL, "rope_table is required");
    if (reinterpret_cast<uintptr_t>(blk->rope_table) % 8 != 0)
      return fail(BITLINEAR_ERR_ALIGN, "rope_table must be 8-byte aligned");
    if (blk->rope_n_pos <= 0 || blk->rope_n_pos > kMaxDim)
      return fail(BITLINEAR_ERR_SHAPE, "rope_n_pos = %lld", (long long)blk->rope_n_pos);
  }
  for (int l = 0; l < blk->n_layers; ++l) {
    const bitlinear_layer &L = blk->layers[l];
    if (!L.gate_up || !L.down) return fail(BITLINEAR_ERR_NULL, "layer %d: gate_up and down are required", l);
    if (!aligned16(L.gate_up) || !aligned16(L.down)) return fail(BITLINEAR_ERR_ALIGN, "layer %d: misaligned weights", l);
    if (L.ffn_sub_norm_gain && !aligned16(L.ffn_sub_norm_gain)) return fail(BITLINEAR_ERR_ALIGN, "layer %d: gain", l);
    if (blk->kind == BITLINEAR_BLOCK_DECODER_CACHED) {
      if (!L.k_cache || !L.v_cache) return fail(BITLINEAR_ERR_NULL, "layer %d: k_cache and v_cache are required", l);
      if (!aligned16(L.k_cache) || !aligned16(L.v_cache)) return fail(BITLINEAR_ERR_ALIGN, "layer %d: caches", l);
    }
    if (is_decoder(blk->kind)) {
      if (!L.qkv || !L.o) return fail(BITLINEAR_ERR_NULL, "layer %d: qkv and o are required", l);
      if (!aligned16(L.qkv) || !aligned16(L.o)) return fail(BITLINEAR_ERR_ALIGN, "layer %d: misaligned weights", l);
      const float *g[3] = {L.input_norm_gain, L.attn_sub_norm_gain, L.post_attn_norm_gain};
      for (const float *p : g)
        if (p && !aligned16(p)) return fail(BITLINEAR_ERR_ALIGN, "layer %d: misaligned gain", l);
    }
  }
  return BITLINEAR_OK;
}

bitlinear_status copy_to(void *dst, const void *src, size_t bytes, hipStream_t s) {
  if (!dst) return BITLINEAR_OK;
  return launched(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s), "trace copy");
}

template <typename T>
T *at(T *p, int64_t off) {
  return p ? p + off : nullptr;
}

bl::ActSrc act_src(const float *x, int64_t ld, int64_t k, const float *gain) {
  bl::ActSrc a{};
  a.x = x;
  a.x2 = nullptr;
  a.ld = ld;
  a.k = (int)k;
  a.gain = gain;
  a.gqa_offset = 0;
  a.head_dim = 1;
  a.group = 1;
  a.h_out = nullptr;
  return a;
}

// One fused decode projection: quantize the input rows in the prologue,
// contract, then the plain / residual / ReLU^2 epilogue.
bitlinear_status fused(int mode, int epi, const bl::ActSrc &src, float eps, int64_t m, const uint8_t *w, int64_t n,
                       const float *gam, const int64_t *seg, int n_seg, float *y, int32_t *acc, const float *res,
                       float *out2, float *mi, int8_t *codes_out, float *deq_out, hipStream_t s,
                       const bitlinear_block *rope_blk = nullptr, const bitlinear_layer *rope_layer = nullptr,
                       const float2 *rope_cs = nullptr) {
  bl::FusedDecode a{};
  a.src = src;
  a.eps = eps;
  a.m = (int)m;
  a.w = w;
  a.n = (int)n;
  BL_TRY(check_segments(gam, seg, n_seg, n, &a.ep));
  a.y = y;
  a.acc_out = acc;
  a.res = res;
  a.out2 = out2;
  a.mi = mi;
  a.codes_out = codes_out;
  a.deq_out = deq_out;
  if (rope_blk) {  // the RoPE form: positions, caches and head layout of the cached decoder
    a.slot = rope_blk->slot;
    a.pos = rope_blk->pos;
    a.cs = rope_cs;
    a.kc = rope_layer->k_cache;
    a.vc = rope_layer->v_cache;
    a.n_slots = rope_blk->n_slots;
    a.tmax = rope_blk->t_max;
    a.n_heads = rope_blk->n_heads;
    a.n_kv = rope_blk->n_kv_heads;
    a.hd = rope_blk->head_dim;
  }
  return launched(bl::launch_gemv_fused(mode, epi, a, s), "fused decode projection");
}

// The attention of the cached decoder on the q|k|v rows in qkv ([m][Q]): RoPE
// on q and k (adjacent heads from column 0), the keys and values into layer
// L's caches, each token's causal attention into b.att ([m][H]).
bitlinear_status cached_attention(const bitlinear_block *blk, const bitlinear_layer &L, int64_t m, float *qkv,
                                  const BlockBufs &b, float *tr_attn, hipStream_t s) {
  const int hd = blk->head_dim, nh = blk->n_heads, nkv = blk->n_kv_heads;
  const int64_t H = blk->hidden, KV = (int64_t)nkv * hd, Q = H + 2 * KV;
  BL_TRY(launched(bl::launch_rope_append(qkv, m, Q, nh, nkv, hd, blk->slot, blk->pos, b.rope_cs, L.k_cache,
                                         L.v_cache, blk->n_slots, blk->t_max, s),
                  "rope and kv append"));
  BL_TRY(launched(bl::launch_attention(qkv, m, Q, nh, nkv, hd, L.k_cache, L.v_cache, blk->n_slots, blk->t_max,
                                       blk->slot, blk->pos, b.att, H, b.attn_ws, s),
                  "attention"));
  return copy_to(tr_attn, b.att, (size_t)(m * H) * 4, s);
}

// The block chains for a decode step of at most bl::kFusedMaxM tokens: four
// launches per decoder layer (two for the FFN block), each projection
// quantizing its own input and applying the block's elementwise step.
bitlinear_status block_forward_fused(const bitlinear_block *blk, const float *x, int64_t m, float *y,
                                     const bitlinear_block_trace &tr, const BlockBufs &b, hipStream_t s) {
  const int64_t H = blk->hidden, I = blk->intermediate;
  const float eps = blk->eps;
  const int64_t gu_seg[2] = {I, 2 * I};
  const int64_t h_seg[1] = {H};
  float *mi = b.gu;  // [m][I]: ReLU^2(gate) * up
  if (blk->kind == BITLINEAR_BLOCK_FFN) {
    const bitlinear_layer &L = blk->layers[0];
    BL_TRY(fused(BITLINEAR_ACT_ABSMAX, bl::FUSED_EPI_RELU2, act_src(x, H, H, nullptr), eps, m, L.gate_up, 2 * I,
                 L.gate_up_gamma, gu_seg, 2, tr.gate_up, tr.acc_gate_up, nullptr, nullptr, mi, tr.codes_in, tr.deq,
                 s));
    return fused(BITLINEAR_ACT_RMSNORM, bl::FUSED_EPI_PLAIN, act_src(mi, I, I, L.ffn_sub_norm_gain), eps, m, L.down,
                 H, &L.down_gamma, h_seg, 1, y, tr.acc_down, nullptr, nullptr, nullptr, tr.codes_ffn,
                 at(tr.deq, 3 * m), s);
  }
  const int hd = blk->head_dim, group = blk->n_heads / blk->n_kv_heads;
  const int64_t KV = (int64_t)blk->n_kv_heads * hd, Q = H + 2 * KV;
  const int64_t qkv_seg[3] = {H, H + KV, Q};
  const bool cached = blk->kind == BITLINEAR_BLOCK_DECODER_CACHED;
  const float *xin = x;
  for (int l = 0; l < blk->n_layers; ++l) {
    const bitlinear_layer &L = blk->layers[l];
    const int64_t oH = (int64_t)l * m * H, oI = (int64_t)l * m * I, oQ = (int64_t)l * m * Q;
    float *dq = at(tr.deq, 4 * m * l);
    // (the cached decoder rotates q and k in place: its trace copy is taken first)
    float *qkv = tr.qkv && !cached ? tr.qkv + oQ : b.qkv;
    float *h = tr.h ? tr.h + oH : b.h;
    float *xnext = tr.x_out ? tr.x_out + oH : (l + 1 == blk->n_layers ? y : b.x);
    // input_layernorm -> q|k|v; the cached decoder without a q|k|v trace takes
    // RoPE and the cache append in the same launch
    const bool rope_fused = cached && !tr.qkv;
    BL_TRY(fused(BITLINEAR_ACT_RMSNORM, rope_fused ? bl::FUSED_EPI_ROPE : bl::FUSED_EPI_PLAIN,
                 act_src(xin, H, H, L.input_norm_gain), eps, m, L.qkv, Q, L.qkv_gamma, qkv_seg, 3, qkv,
                 at(tr.acc_qkv, oQ), nullptr, nullptr, nullptr, at(tr.codes_in, oH), dq, s,
                 rope_fused ? blk : nullptr, rope_fused ? &L : nullptr, b.rope_cs));
    if (cached) {
      // RoPE, cache append, attention -> attn_sub_norm -> o_proj; h = x + o
      if (rope_fused) {
        BL_TRY(launched(bl::launch_attention(qkv, m, Q, blk->n_heads, blk->n_kv_heads, hd, L.k_cache, L.v_cache,
                                             blk->n_slots, blk->t_max, blk->slot, blk->pos, b.att, H, b.attn_ws, s),
                        "attention"));
        BL_TRY(copy_to(at(tr.attn, oH), b.att, (size_t)(m * H) * 4, s));
      } else {
        BL_TRY(copy_to(at(tr.qkv, oQ), qkv, (size_t)(m * Q) * 4, s));
        BL_TRY(cached_attention(blk, L, m, qkv, b, at(tr.attn, oH), s));
      }
      BL_TRY(fused(BITLINEAR_ACT_RMSNORM, bl::FUSED_EPI_RESID, act_src(b.att, H, H, L.attn_sub_norm_gain), eps, m,
                   L.o, H, &L.o_gamma, h_seg, 1, nullptr, at(tr.acc_o, oH), xin, h, nullptr, at(tr.codes_attn, oH),
                   at(dq, m), s));
    } else {
      // self-only attention -> attn_sub_norm -> o_proj; h = x + o
      bl::ActSrc att = act_src(qkv, Q, H, L.attn_sub_norm_gain);
      att.gqa_offset = (int)(H + KV);
      att.head_dim = hd;
      att.group = group;
      BL_TRY(fused(bl::ACT_GQA_RMSNORM, bl::FUSED_EPI_RESID, att, eps, m, L.o, H, &L.o_gamma, h_seg, 1, nullptr,
                   at(tr.acc_o, oH), xin, h, nullptr, at(tr.codes_attn, oH), at(dq, m), s));
    }
    // post_attention_layernorm -> gate|up -> ReLU^2(gate) * up
    BL_TRY(fused(BITLINEAR_ACT_RMSNORM, bl::FUSED_EPI_RELU2, act_src(h, H, H, L.post_attn_norm_gain), eps, m,
                 L.gate_up, 2 * I, L.gate_up_gamma, gu_seg, 2, at(tr.gate_up, 2 * oI), at(tr.acc_gate_up, 2 * oI),
                 nullptr, nullptr, mi, at(tr.codes_post, oH), at(dq, 2 * m), s));
    // ffn_sub_norm -> down; x' = h + down
    BL_TRY(fused(BITLINEAR_ACT_RMSNORM, bl::FUSED_EPI_RESID, act_src(mi, I, I, L.ffn_sub_norm_gain), eps, m, L.down,
                 H, &L.down_gamma, h_seg, 1, nullptr, at(tr.acc_down, oH), h, xnext, nullptr, at(tr.codes_ffn, oI),
                 at(dq, 3 * m), s));
    xin = xnext;
  }
  if (tr.x_out) return copy_to(y, xin, (size_t)(m * H) * 4, s);
  return BITLINEAR_OK;
}


// A projection's output as the next stage reads it: fp32 rows, or the split-K
// partial sums the next quantization adds itself (with the deq and row sums
// of the codes that were contracted).
struct ProjOut {
  const float *y = nullptr;
  const int32_t *part = nullptr;
  int splits = 1;
  int64_t plane = 0;
  const int32_t *rowsum = nullptr;
  const float *deq = nullptr;
  bl::Epilogue ep{};
};

void attach(bl::ActSrc &a, const ProjOut &o) {
  if (!o.part) return;
  a.part = o.part;
  a.part_splits = o.splits;
  a.part_plane = o.plane;
  a.part_rowsum = o.rowsum;
  a.part_deq = o.deq;
  a.part_ep = o.ep;
}

// The quantize -> contract chain for m > 4 tokens (and whenever the one-launch
// decode form does not apply). Each quantization writes the deq / row-sum set
// the previous one did not, so it can read a split-K projection's partial sums
// with the previous set.
struct Chain {
  BlockBufs b;
  int64_t m;
  float eps;
  hipStream_t s;
  int set = 0;  // 0: (deq, rowsum), 1: (deq2, rowsum2) hold the current codes' scales
  float *deq() const { return set ? b.deq2 : b.deq; }
  int32_t *rowsum() const { return set ? b.rowsum2 : b.rowsum; }

  bitlinear_status quant(int mode, const bl::ActSrc &src) {
    set ^= 1;
    return launched(bl::launch_quant_acts_src(mode, src, m, eps, b.codes, deq(), rowsum(), s), "quantize stage");
  }
  // keep: the caller takes split-K partial sums (no trace of this projection)
  bitlinear_status proj(int64_t k, const uint8_t *w, int64_t n, const float *gam, const int64_t *seg, int n_seg,
                        float *y, int32_t *acc, bool keep, ProjOut *out) {
    ProjOut o;
    BL_TRY(check_segments(gam, seg, n_seg, n, &o.ep));
    o.y = y;
    if (!keep || m <= 16) {
      BL_TRY(contract(b.codes, deq(), rowsum(), m, k, w, n, o.ep, y, acc, BITLINEAR_PATH_AUTO, b.split, s));
    } else {
      int splits = 1;
      BL_TRY(launched(bl::launch_gemm_prefill(b.codes, w, deq(), rowsum(), m, n, k, o.ep, y, nullptr, b.split, s,
                                              &splits),
                      "prefill kernel"));
      if (splits > 1) {
        o.y = nullptr;
        o.part = b.split;
        o.splits = splits;
        o.plane = m * n;
        o.rowsum = rowsum();
        o.deq = deq();
      }
    }
    *out = o;
    return BITLINEAR_OK;
  }
  // the cached decoder's q|k|v projection (2 to 16 tokens) with RoPE on q and
  // k and the keys and values appended to layer L's caches in its epilogue
  bitlinear_status proj_rope(const bitlinear_block *blk, const bitlinear_layer &L, int64_t k, int64_t n,
                             const int64_t *seg, float *y, int32_t *acc) {
    bl::Epilogue ep;
    BL_TRY(check_segments(L.qkv_gamma, seg, 3, n, &ep));
    bl::DecodeRope r;
    r.slot = blk->slot;
    r.pos = blk->pos;
    r.cs = b.rope_cs;
    r.kc = L.k_cache;
    r.vc = L.v_cache;
    r.n_slots = blk->n_slots;
    r.tmax = blk->t_max;
    r.n_heads = blk->n_heads;
    r.n_kv = blk->n_kv_heads;
    r.hd = blk->head_dim;
    return launched(bl::launch_gemv_decode_rope(b.codes, L.qkv, deq(), rowsum(), m, k, ep, y, acc, r, s),
                    "q|k|v projection with RoPE");
  }
  // gate|up -> ReLU^2 -> ffn_sub_norm quantization (codes of the down input)
  bitlinear_status ffn_input(int64_t H, int64_t I, const bitlinear_layer &L, float *tr_gate_up,
                             int32_t *tr_acc_gate_up) {
    const int64_t gu_seg[2] = {I, 2 * I};
    const bool traced = tr_gate_up || tr_acc_gate_up;
    if (!traced && bl::gemm_glu_supported(m, I, H)) {
      // the gated kernel writes fl32(max(g, 0)^2 * u) ([m][I]) and gate, up never leave the chip
      bl::Epilogue ep;
      BL_TRY(check_segments(L.gate_up_gamma, gu_seg, 2, 2 * I, &ep));
      BL_TRY(launched(bl::launch_gemm_glu(b.codes, L.gate_up, deq(), rowsum(), m, I, H, ep, b.gu, s),
                      "gated prefill kernel"));
      return quant(BITLINEAR_ACT_RMSNORM, act_src(b.gu, I, I, L.ffn_sub_norm_gain));
    }
    ProjOut gu;
    BL_TRY(proj(H, L.gate_up, 2 * I, L.gate_up_gamma, gu_seg, 2, b.gu, tr_acc_gate_up, !traced, &gu));
    BL_TRY(copy_to(tr_gate_up, b.gu, (size_t)(m * 2 * I) * 4, s));
    bl::ActSrc src = act_src(gu.y, 2 * I, I, L.ffn_sub_norm_gain);
    attach(src, gu);
    return quant(BITLINEAR_ACT_RELU2_RMSNORM, src);
  }
};

bitlinear_status block_forward_chain(const bitlinear_block *blk, const float *x, int64_t m, float *y,
                                     const bitlinear_block_trace &tr, const BlockBufs &bufs, hipStream_t s) {
  const int64_t H = blk->hidden, I = blk->intermediate;
  const int64_t h_seg[1] = {H};
  Chain c{bufs, m, blk->eps, s};
  const BlockBufs &b = bufs;

  if (blk->kind == BITLINEAR_BLOCK_FFN) {
    const bitlinear_layer &L = blk->layers[0];
    BL_TRY(c.quant(BITLINEAR_ACT_ABSMAX, act_src(x, H, H, nullptr)));
    BL_TRY(copy_to(tr.codes_in, b.codes, (size_t)(m * H), s));
    BL_TRY(copy_to(tr.deq, c.deq(), (size_t)m * 4, s));
    BL_TRY(c.ffn_input(H, I, L, tr.gate_up, tr.acc_gate_up));
    BL_TRY(copy_to(tr.codes_ffn, b.codes, (size_t)(m * I), s));
    BL_TRY(copy_to(at(tr.deq, 3 * m), c.deq(), (size_t)m * 4, s));
    ProjOut d;
    return c.proj(I, L.down, H, &L.down_gamma, h_seg, 1, y, tr.acc_down, false, &d);
  }

  const int hd = blk->head_dim, group = blk->n_heads / blk->n_kv_heads;
  const int64_t KV = (int64_t)blk->n_kv_heads * hd, Q = H + 2 * KV;
  const int64_t qkv_seg[3] = {H, H + KV, Q};
  const bool cached = blk->kind == BITLINEAR_BLOCK_DECODER_CACHED;
  ProjOut d;  // the previous layer's down projection
  for (int l = 0; l < blk->n_layers; ++l) {
    const bitlinear_layer &L = blk->layers[l];
    const int64_t oH = (int64_t)l * m * H, oI = (int64_t)l * m * I, oQ = (int64_t)l * m * Q;
    // input_layernorm; for l > 0 the layer input is h + down of the previous layer
    const float *xin = x;
    if (l == 0) {
      BL_TRY(c.quant(BITLINEAR_ACT_RMSNORM, act_src(x, H, H, L.input_norm_gain)));
    } else {
      bl::ActSrc src = act_src(b.h, H, H, L.input_norm_gain);
      src.x2 = d.y;
      src.h_out = b.x;
      attach(src, d);
      BL_TRY(c.quant(bl::ACT_RESID_RMSNORM, src));
      xin = b.x;
    }
    BL_TRY(copy_to(at(tr.codes_in, oH), b.codes, (size_t)(m * H), s));
    BL_TRY(copy_to(at(tr.deq, 4 * m * l), c.deq(), (size_t)m * 4, s));
    ProjOut qkv;
    // the cached decoder at 2 to 16 tokens without a q|k|v trace takes RoPE and
    // the cache append in the projection's epilogue
    const bool rope_fused =
        cached && !tr.qkv && bl::gemv_decode_rope_supported(m, H, blk->n_heads, blk->n_kv_heads, hd);
    if (rope_fused) {
      BL_TRY(c.proj_rope(blk, L, H, Q, qkv_seg, b.qkv, at(tr.acc_qkv, oQ)));
    } else {
      BL_TRY(c.proj(H, L.qkv, Q, L.qkv_gamma, qkv_seg, 3, b.qkv, at(tr.acc_qkv, oQ),
                    !tr.qkv && !tr.acc_qkv && !cached, &qkv));
      BL_TRY(copy_to(at(tr.qkv, oQ), b.qkv, (size_t)(m * Q) * 4, s));
    }
    if (cached) {
      // RoPE, cache append, attention -> attn_sub_norm -> o_proj
      if (rope_fused) {
        BL_TRY(launched(bl::launch_attention(b.qkv, m, Q, blk->n_heads, blk->n_kv_heads, hd, L.k_cache, L.v_cache,
                                             blk->n_slots, blk->t_max, blk->slot, blk->pos, b.att, H, b.attn_ws, s),
                        "attention"));
        BL_TRY(copy_to(at(tr.attn, oH), b.att, (size_t)(m * H) * 4, s));
      } else {
        BL_TRY(cached_attention(blk, L, m, b.qkv, b, at(tr.attn, oH), s));
      }
      BL_TRY(c.quant(BITLINEAR_ACT_RMSNORM, act_src(b.att, H, H, L.attn_sub_norm_gain)));
    } else {
      // self-only attention output -> attn_sub_norm -> o_proj
      bl::ActSrc src = act_src(qkv.y, Q, H, L.attn_sub_norm_gain);
      src.gqa_offset = (int)(H + KV);
      src.head_dim = hd;
      src.group = group;
      attach(src, qkv);
      BL_TRY(c.quant(bl::ACT_GQA_RMSNORM, src));
    }
    BL_TRY(copy_to(at(tr.codes_attn, oH), b.codes, (size_t)(m * H), s));
    BL_TRY(copy_to(at(tr.deq, 4 * m * l + m), c.deq(), (size_t)m * 4, s));
    ProjOut o;
    BL_TRY(c.proj(H, L.o, H, &L.o_gamma, h_seg, 1, b.o, at(tr.acc_o, oH), !tr.acc_o, &o));
    // h = x + o -> post_attention_layernorm
    {
      bl::ActSrc src = act_src(xin, H, H, L.post_attn_norm_gain);
      src.x2 = o.y;
      src.h_out = b.h;
      attach(src, o);
      BL_TRY(c.quant(bl::ACT_RESID_RMSNORM, src));
    }
    BL_TRY(copy_to(at(tr.h, oH), b.h, (size_t)(m * H) * 4, s));
    BL_TRY(copy_to(at(tr.codes_post, oH), b.codes, (size_t)(m * H), s));
    BL_TRY(copy_to(at(tr.deq, 4 * m * l + 2 * m), c.deq(), (size_t)m * 4, s));
    // relu^2 gating -> ffn_sub_norm -> down
    BL_TRY(c.ffn_input(H, I, L, at(tr.gate_up, 2 * oI), at(tr.acc_gate_up, 2 * oI)));
    BL_TRY(copy_to(at(tr.codes_ffn, oI), b.codes, (size_t)(m * I), s));
    BL_TRY(copy_to(at(tr.deq, 4 * m * l + 3 * m), c.deq(), (size_t)m * 4, s));
    BL_TRY(c.proj(I, L.down, H, &L.down_gamma, h_seg, 1, b.d, at(tr.acc_down, oH), !tr.acc_down && !tr.x_out, &d));
    if (tr.x_out) BL_TRY(launched(bl::launch_add(b.h, b.d, tr.x_out + oH, m * H, s), "trace add"));
  }
  if (d.part)
    return launched(bl::launch_splitk_finish(d.part, d.splits, d.deq, d.rowsum, m, H, d.ep, y, nullptr, b.h, s),
                    "residual add");
  return launched(bl::launch_add(b.h, b.d, y, m * H, s), "residual add");
}
}  // namespace

extern "C" {

size_t bitlinear_block_workspace_bytes(const bitlinear_block *blk, int64_t m) {
  if (!blk || m < 0 || blk->hidden <= 0 || blk->intermediate <= 0) return 0;
  return block_layout(blk, m, nullptr, nullptr);
}

bitlinear_status bitlinear_block_forward(const bitlinear_block *blk, const float *x, int64_t m, float *y,
                                         const bitlinear_block_trace *trace, void *workspace, size_t workspace_bytes,
                                         void *stream) {
  g_err.clear();
  BL_TRY(check_block(blk));
  if (m != 0 && (!x || !y)) return fail(BITLINEAR_ERR_NULL, "x and y are required");
  if (m < 0 || m > kMaxDim) return fail(BITLINEAR_ERR_SHAPE, "m = %lld", (long long)m);
  if (!aligned16(x) || !aligned16(y)) return fail(BITLINEAR_ERR_ALIGN, "x and y must be 16-byte aligned");
  const size_t need = bitlinear_block_workspace_bytes(blk, m);
  if (m > 0 && (!workspace || workspace_bytes < need))
    return fail(BITLINEAR_ERR_WORKSPACE, "workspace of %zu bytes needed", need);
  if (m == 0) return BITLINEAR_OK;
  BL_TRY(check_device());
  hipStream_t s = as_stream(stream);
  BlockBufs b;
  block_layout(blk, m, &b, static_cast<char *>(workspace));
  const int64_t H = blk->hidden, I = blk->intermediate;
  bitlinear_block_trace tr;
  memset(&tr, 0, sizeof tr);
  if (trace) tr = *trace;
  // every layer rotates q and k at the same positions: their rows of the rotary table once per call
  if (blk->kind == BITLINEAR_BLOCK_DECODER_CACHED)
    BL_TRY(launched(bl::launch_rope_gather(blk->pos, m, blk->head_dim,
                                           reinterpret_cast<const float2 *>(blk->rope_table), blk->rope_n_pos,
                                           b.rope_cs, s),
                    "rope rows"));

  if (bl::fused_decode_supported(m, H) && bl::fused_decode_supported(m, I) && I % 16 == 0)
    return block_forward_fused(blk, x, m, y, tr, b, s);
  return block_forward_chain(blk, x, m, y, tr, b, s);
}

}  // extern "C"
