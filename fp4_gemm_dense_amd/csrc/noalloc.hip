// dg_fp8_gemm_nt_noalloc: the dense NT GEMM for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses that
// forbid allocation).  It runs exactly the kernels of dg_fp8_gemm_nt; the one
// difference is where the split-K partial tiles live: in a file-scope device
// array of this library instead of a caller workspace.
//
// The array belongs to the loaded code object, so every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Host code
// never uses the array's name as a device address (in host code it only names a
// host-side stand-in): the first call on each device looks the device address up
// with hipGetSymbolAddress, with that device current, and keeps it; kernels get
// that pointer as their workspace argument.
//
// Nothing in the array has to start at zero: every split slice writes its whole
// fp32 partial tile before the reduce kernel reads it.  Calls on one GPU share
// the array, so calls that may overlap in time on one GPU (different streams
// without ordering) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/dg.h"
#include "dg_internal.hpp"

namespace dg {

// Largest split-K workspace the static buffer serves (24 MiB per GPU): every
// skinny plan on 256 CUs (one 64x128 partial per slot, 8 MiB) and split tails of
// up to 192 partial 128x256 tiles.
constexpr size_t kScratchBytes = size_t(24) << 20;

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static float* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device (null: not looked up)

// Device address of the scratch array on the current device, looked up once per
// device.  Returns null (and sets *err) if the lookup fails.
static float* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  return g_scratch_ptr[dev];
}

}  // namespace dg

extern "C" int dg_fp8_gemm_nt_noalloc(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                                      const uint16_t* c, uint16_t* d, int m, int n, int k, void* stream) {
  try {
    // the plan's workspace need (0 for invalid sizes: dense_entry reports those)
    const size_t need = dg_fp8_gemm_workspace_bytes(DG_FORM_NT, m, n, k, 1, 0, 0);
    if (need > dg::kScratchBytes) return DG_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0) {
      hipError_t err = hipSuccess;
      ws = dg::scratch_on_current_device(&err);
      if (!ws) {
        (void)hipGetLastError();
        return DG_ERR_HIP;
      }
    }
    return dg::dense_entry(a, sfa, b, sfb, c, d, m, n, k, ws, need > 0 ? dg::kScratchBytes : 0, stream, 0);
  } catch (...) {
    return DG_ERR_HIP;
  }
}
