// w12_gemm_noalloc: w12_gemm for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation).  The
// workspace of a K-split launch (tickets, FP32 partials, row sums of x^2) lives in
// `scratch`, a fixed array of W12_NOALLOC_SCRATCH_BYTES of device memory in this
// library: each GPU the library runs on holds its own copy, from the first call on that
// GPU until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: the device
// address of the current GPU's copy comes from hipGetSymbolAddress, taken once per GPU on
// its first call (with that GPU current) and kept; kernels get that address only.
#include "w12.h"
#include "w12_internal.h"

#include <mutex>

namespace {

constexpr size_t kScratchBytes = (size_t)W12_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// Zero at load (device globals are zero-initialised); the first call on each GPU clears
// the split-K tickets at its start again, on the caller's stream, and every call leaves
// them at zero.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];        // device address of each GPU's copy
hipError_t g_status[kMaxDevices];

// The current GPU's copy of `scratch`; *first is set on the call that looked it up.
hipError_t device_scratch(void** out, bool* first) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev, first] {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = r == hipSuccess ? p : nullptr;
    g_status[dev] = r;
    *first = true;
  });
  *out = g_scratch[dev];
  return g_status[dev];
}

}  // namespace

extern "C" w12_status w12_gemm_noalloc(const uint16_t* x, uint32_t m, const w12_desc* d,
                                       uint16_t* y, void* stream) {
  size_t need = 0;
  const w12_status st = w12::gemm_check(x, m, d, y, &need);
  if (st != W12_OK) return st;
  if (need > kScratchBytes) return W12_ERR_WORKSPACE;
  void* ws = nullptr;
  bool first = false;
  if (device_scratch(&ws, &first) != hipSuccess || !ws) return W12_ERR_HIP;
  // the tickets (the first 4096 bytes) start at zero: clear them once per GPU, with a fill
  // kernel on the caller's stream ahead of the first launch that uses them
  if (first && w12::launch_fill_zero(ws, 4096, (hipStream_t)stream) != hipSuccess)
    return W12_ERR_HIP;
  return w12::gemm_launch(x, m, d, y, ws, stream, false);
}
