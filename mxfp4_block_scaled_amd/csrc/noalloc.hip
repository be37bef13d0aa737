// mxfp4_gemm_noalloc: the dense MXFP4 GEMM with its workspace in a file-scope
// device array instead of caller memory, for callers that cannot allocate.
//
// `scratch` below is a device symbol. In host code its name is only a host-side
// stand-in, never a device address: the device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept in
// g_scratch, and only that pointer is handed to the kernels.
#include <mutex>

#include <hip/hip_runtime.h>

#include "mxfp4_moe.h"

namespace {

constexpr size_t kScratchBytes = MXF_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

// every GPU the library runs on holds its own copy until the process ends
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// device address of this device's scratch array, looked up on first use
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXF_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MXF_ERR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MXF_OK;
}

}  // namespace

extern "C" {

size_t mxfp4_noalloc_scratch_bytes(void) { return kScratchBytes; }

int mxfp4_gemm_noalloc(const uint16_t* a, int64_t M, int64_t N, int64_t K, int act_fmt, const uint8_t* w,
                       const uint8_t* w_scale, float* c, mxf_stream stream) {
  // the checks that need no device come first: an oversized call fails before any HIP call
  if (act_fmt != MXF_E4M3 && act_fmt != MXF_E2M1) return MXF_ERR_FORMAT;
  if (M < 0 || N <= 0 || N % 16 != 0 || K <= 0 || K % 512 != 0) return MXF_ERR_SHAPE;
  if (M == 0) return MXF_OK;
  if (mxfp4_gemm_workspace_bytes(M, N, K, act_fmt) > kScratchBytes) return MXF_ERR_WORKSPACE;
  if (!a || !w || !w_scale || !c) return MXF_ERR_NULL;
  void* ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc != MXF_OK) return rc;
  return mxfp4_gemm(a, M, N, K, act_fmt, w, w_scale, c, ws, kScratchBytes, stream);
}

}  // extern "C"
