// Allocation-free emulated DGEMV: ozk_dgemv with its scratch memory in a fixed-size
// device array of this library instead of a caller-provided workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never passes
// the variable's name to a kernel or a copy (on the host it is only a stand-in); the
// device address comes from hipGetSymbolAddress, taken once per device with that device
// current, and is kept per device.  All calls on one GPU share that GPU's array, so
// calls that overlap in time on one GPU (different streams or threads) race; calls
// ordered on one stream do not.  Every kernel of the GEMV path either overwrites the
// scratch it reads or clears it first with a fill kernel (no memset nodes), so the
// contents a previous call left behind never reach a result.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ozk_internal.h"

namespace {

constexpr size_t kScratchBytes = OZK_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Device address of the current device's scratch array (looked up on the first call on
// that device).
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return OZK_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return OZK_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return OZK_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return OZK_OK;
}

}  // namespace

extern "C" {

int ozk_dgemv_noalloc(int64_t m, int64_t k, int64_t nrhs, const double* A, int64_t lda,
                      const int8_t* A_planes, int64_t ldp, int64_t plane_stride,
                      const int32_t* A_exps, const double* X, int64_t ldx, double* Y,
                      int64_t ldy, int r, int mode, void* stream) {
  int st = ozk::dgemv_validate(m, k, nrhs, A, lda, A_planes, ldp, plane_stride, A_exps, X, ldx,
                               Y, ldy, r, mode);
  if (st != OZK_OK || m == 0) return st;
  size_t need = 0;
  if ((st = ozk_dgemv_workspace_size(m, k, nrhs, r, mode, &need)) != OZK_OK) return st;
  if (need > kScratchBytes) return OZK_ENOSCRATCH;
  void* ws = nullptr;
  if ((st = current_scratch(&ws)) != OZK_OK) return st;
  return ozk_dgemv(m, k, nrhs, A, lda, A_planes, ldp, plane_stride, A_exps, X, ldx, Y, ldy, r,
                   mode, ws, kScratchBytes, stream);
}

}  // extern "C"
