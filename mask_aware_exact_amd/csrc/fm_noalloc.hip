// fm_bwd for callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation): the backward's workspace, the float32 row term D of
// [B, H, N], lives in a fixed array in this library's device memory instead of a caller buffer.
//
// The array is a file-scope __device__ variable: each GPU the library runs on holds its own copy, at its
// own address, from the code object's load until the process ends. Host code never uses the array's
// name as an address (on the host it is only a stand-in); the device address of the current device's
// copy is looked up once per device with hipGetSymbolAddress and kept. Calls on one GPU share its copy:
// calls that overlap on one GPU (on different streams) race. The D values are written in full by every
// call before they are read, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fm.h"

constexpr size_t kScratchBytes = FM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "the scratch array holds whole 256-byte units");

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up on the first call on that device.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

fm_status fm_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const void* dout,
                         const float* lse, fm_dtype dtype, int B, int H, int N, int d, const int32_t* lts,
                         const int32_t* lte, const int32_t* uts, const int32_t* ute, int Hm, const int32_t* bounds,
                         const int32_t* sched, int causal, float scale, void* dq, void* dk, void* dv,
                         hipStream_t stream) {
  const size_t need = fm_bwd_workspace_bytes(dtype, B, H, N, d);
  if (need > kScratchBytes) return FM_ERR_WORKSPACE;  // B * H * N * 4 bytes past the fixed array
  void* ws = nullptr;
  if (need != 0) {
    if (scratch_ptr(&ws) != hipSuccess) return FM_ERR_LAUNCH;
  }
  // need == 0 means bad sizes or dtype: fm_bwd reports them (a null workspace is never reached then)
  return fm_bwd(q, k, v, out, dout, lse, dtype, B, H, N, d, lts, lte, uts, ute, Hm, bounds, sched, causal, scale,
                dq, dk, dv, ws, kScratchBytes, stream);
}

}  // extern "C"
