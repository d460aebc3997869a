// ckv_decode_step_static: the single-call decode step with its workspace in a
// device array of this library instead of a caller-supplied buffer, for
// callers that cannot allocate (code under stream capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array lives in device memory of every GPU the library is loaded on
// for the life of the process.  Host code never passes the array's name to a
// kernel or a copy (in host code that name is a host-side stand-in, not a
// device address): on the first call on a device, with that device current,
// hipGetSymbolAddress gives that device's copy's address, which is kept per
// device and used from then on.  Calls on one GPU share its array, so calls
// that overlap on one GPU race; the histogram and counter region the kernels
// accumulate into is cleared by a fill kernel at the start of every call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ckv_internal.h"

namespace {

constexpr size_t kStaticScratchBytes = CKV_STATIC_WORKSPACE_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Address of the current device's copy of `scratch` (looked up once per device).
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CKV_E_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return CKV_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CKV_OK;
}

// Zeros n bytes (n a multiple of 16) with vector stores: a kernel, not a
// runtime memset, so that the call records no memset node under capture.
__global__ __launch_bounds__(256) void k_zero16(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" int ckv_decode_step_static(const ckv_layer_desc* desc, const ckv_layer_weights* w,
                                      const ckv_layer_cache* cache, const void* x, const void* u, const void* q,
                                      const void* qI, const float* iw, const int32_t* pos, int32_t B,
                                      int32_t* topk, void* out, void* stream) {
  // every check first (a placeholder aligned address stands for the
  // workspace, whose size is checked against the array's), nothing enqueued
  // on an error
  ckv::LayerParams P;
  ckv::WsLayout L;
  int rc = ckv::decode_step_checks(desc, w, cache, x, u, q, qI, iw, pos, B, topk, out, (void*)uintptr_t(256),
                                   kStaticScratchBytes, &P, &L);
  if (rc) return rc;
  void* ws = nullptr;
  if ((rc = scratch_of_current_device(&ws))) return rc;
  const size_t sync = L.sync_bytes;
  if (sync) {
    (void)hipGetLastError();
    const size_t n16 = (sync + 15) / 16;
    const unsigned blocks = (unsigned)((n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024);
    hipLaunchKernelGGL(k_zero16, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (uint4*)ws, n16);
    if (hipGetLastError() != hipSuccess) return CKV_E_HIP;
  }
  return ckv_decode_step(desc, w, cache, x, u, q, qI, iw, pos, B, topk, out, ws, kStaticScratchBytes, stream);
}
