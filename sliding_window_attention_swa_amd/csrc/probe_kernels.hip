// Measurement probes: the practical HBM read and copy ceilings and the
// practical bf16 MFMA ceiling of the GPU the benchmark runs on (declared in
// swa_probe.h).
#include "common.hpp"
#include "swa_probe.h"

namespace {

// Grid-stride read with 16-byte loads; the per-thread sum keeps the loads.
__global__ void __launch_bounds__(256) probe_read_kernel(const uint4 *__restrict__ x, size_t n16, float *out) {
  float s = 0.f;
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = x[i];
    s += (__uint_as_float(v.x) + __uint_as_float(v.y)) + (__uint_as_float(v.z) + __uint_as_float(v.w));
  }
  out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// Grid-stride copy with 16-byte loads and stores.
__global__ void __launch_bounds__(256) probe_copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                         size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

// Eight independent accumulator chains per wavefront keep the matrix core
// busy; the operands depend on the lane so nothing is folded.
__global__ void __launch_bounds__(256) probe_mfma_kernel(float *out, int32_t iters) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
  typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
  const int32_t lane = threadIdx.x & 63;
  const short av = static_cast<short>(0x3C00 + (lane & 7));   // about 2^-7
  const short bv = static_cast<short>(0x3C00 + (lane >> 3));
  const bf16x8 a = {av, av, av, av, av, av, av, av};
  const bf16x8 b = {bv, bv, bv, bv, bv, bv, bv, bv};
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0, c4 = c0, c5 = c0, c6 = c0, c7 = c0;
  for (int32_t it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c3, 0, 0, 0);
    c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c4, 0, 0, 0);
    c5 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c5, 0, 0, 0);
    c6 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c6, 0, 0, 0);
    c7 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c7, 0, 0, 0);
  }
  const f32x4 s4 = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
}

swa_status_t from_launch() { return hipGetLastError() == hipSuccess ? SWA_OK : SWA_E_HIP; }

}  // namespace

extern "C" swa_status_t swa_probe_read(const void *buf, size_t bytes, float *out, int32_t grid, hipStream_t stream) {
  if (!buf || !out || bytes == 0 || (bytes & 15u) || (reinterpret_cast<uintptr_t>(buf) & 15u) || grid < 1 ||
      grid > 65535)
    return SWA_E_ARG;
  hipLaunchKernelGGL(probe_read_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                     static_cast<const uint4 *>(buf), bytes / 16, out);
  return from_launch();
}

extern "C" swa_status_t swa_probe_copy(const void *src, void *dst, size_t bytes, int32_t grid, hipStream_t stream) {
  const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
  if (!src || !dst || bytes == 0 || (bytes & 15u) || (s & 15u) || (d & 15u) || grid < 1 || grid > 65535 ||
      (s < d + bytes && d < s + bytes))
    return SWA_E_ARG;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream,
                     static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), bytes / 16);
  return from_launch();
}

extern "C" swa_status_t swa_probe_mfma(float *out, int32_t grid, int32_t iters, hipStream_t stream) {
  if (!out || grid < 1 || grid > 65535 || iters < 1) return SWA_E_ARG;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, stream, out, iters);
  return from_launch();
}
