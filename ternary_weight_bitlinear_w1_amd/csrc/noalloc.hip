// bitlinear_forward_noalloc: bitlinear_forward for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc). Its scratch is one file-scope device
// array, `scratch`, of kNoallocScratchBytes: each GPU the library runs on
// holds its own copy until the process ends. Host code never passes the
// array's name to a kernel or a copy (on the host it is only a stand-in
// symbol, not a device address); it resolves the device address once per
// device with hipGetSymbolAddress and passes that pointer on, exactly as
// bitlinear_forward passes a caller's workspace.
#include <mutex>

#include "common.h"

namespace {

constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;  // 32 MiB per device

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // per device: the device address of scratch (NULL until resolved)

// The device address of this device's scratch, resolved on the first call on
// the device (with the device current) and kept.
bitlinear_status scratch_of_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return bl::report_error(BITLINEAR_ERR_DEVICE, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return bl::report_error(BITLINEAR_ERR_DEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return bl::report_error(BITLINEAR_ERR_DEVICE, "hipGetSymbolAddress of the scratch array failed");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return BITLINEAR_OK;
}

}  // namespace

extern "C" {

size_t bitlinear_forward_noalloc_max_scratch_bytes(void) { return kNoallocScratchBytes; }

bitlinear_status bitlinear_forward_noalloc(const float *x, const int8_t *codes_in, const float *deq_in,
                                           const int32_t *rowsum_in, int64_t m, int64_t k, const uint8_t *w_packed,
                                           int64_t n, const float *gamma, const int64_t *seg_end, int32_t n_seg,
                                           float *y, int32_t *acc_out, int32_t path, void *stream) {
  // m == 0, or arguments bitlinear_forward rejects: its checks and status,
  // without touching the device
  if (m <= 0 || n <= 0 || k <= 0 || k % 16 != 0)
    return bitlinear_forward(x, codes_in, deq_in, rowsum_in, m, k, w_packed, n, gamma, seg_end, n_seg, y, acc_out,
                             path, nullptr, 0, stream);
  const size_t need = bitlinear_forward_workspace_bytes(m, n, k, x != nullptr);
  if (need > kNoallocScratchBytes)
    return bl::report_error(BITLINEAR_ERR_WORKSPACE,
                            "this shape needs more scratch than the no-allocation entry point holds (32 MiB)");
  void *ws = nullptr;
  const bitlinear_status st = scratch_of_current_device(&ws);
  if (st != BITLINEAR_OK) return st;
  return bitlinear_forward(x, codes_in, deq_in, rowsum_in, m, k, w_packed, n, gamma, seg_end, n_seg, y, acc_out, path,
                           ws, kNoallocScratchBytes, stream);
}

}  // extern "C"
