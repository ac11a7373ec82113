// Measurement support: the sustained matrix-core rate of this GPU on the instruction
// shapes the products use, with operand data like theirs.  On MI355X the matrix cores
// draw data-dependent power: random int8 or e2m1 operands drive the board to its power
// cap well below the datasheet clock, so the rate this kernel reaches is the practical
// ceiling against which the product kernels are judged (next to the datasheet peak).
//
// 512 threads per workgroup (two waves per SIMD) run a register-only loop of 32 MFMAs
// per iteration over 8 accumulators; the 16 operand registers of each wave hold 256 bytes
// of the caller's data per lane and every MFMA pairs a different two of them, so the
// operand bits change from one instruction to the next as they do in a GEMM.  Nothing is
// stored until the end (one word per thread into `sink`, so the work is not elided).
#include "ozk_internal.h"

namespace ozk {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 512;

template <int kFp4>
__global__ __launch_bounds__(kProbeThreads, 1) void mfma_probe_kernel(
    const v4i* __restrict__ src, int64_t src_vectors, int64_t iters, int32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6);
  v4i f[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) f[q] = src[(wave * 1024 + q * 64 + lane) % src_vectors];
  int32_t s = 0;
  if (kFp4) {
    v16f acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < 32; ++m) {
        const v4i& a = f[m & 15];
        const v4i& b = f[(m * 5 + 3) & 15];
        const v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
        const v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
        acc[m & 7] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[m & 7], 4, 4,
                                                                     0, 0x80, 0, 0x80);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s ^= __float_as_int(acc[i][0]) ^ __float_as_int(acc[i][15]);
  } else {
    v16i acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][v] = 0;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
      for (int m = 0; m < 32; ++m)
        acc[m & 7] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[m & 15], f[(m * 5 + 3) & 15],
                                                            acc[m & 7], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s ^= acc[i][0] ^ acc[i][15];
  }
  sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace ozk

extern "C" {

int ozk_probe_mfma(int kind, const void* operands, int64_t operand_bytes, int64_t iters,
                   int workgroups, int32_t* sink, double* ops, void* stream) {
  using namespace ozk;
  if (kind != 0 && kind != 1) return OZK_EINVAL;
  if (!operands || !sink || operand_bytes < 16 || iters < 1 || workgroups < 1) return OZK_EINVAL;
  if (reinterpret_cast<uintptr_t>(operands) % 16 != 0) return OZK_EINVAL;
  if (ops) *ops = (double)workgroups * (kProbeThreads / 64) * 32.0 * 65536.0 * (kind ? 2 : 1) *
                  (double)iters;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const v4i* src = static_cast<const v4i*>(operands);
  const int64_t nvec = operand_bytes / 16;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s,
                       src, nvec, iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s,
                       src, nvec, iters, sink);
  return hipGetLastError() == hipSuccess ? OZK_OK : OZK_EHIP;
}

}  // extern "C"
