// MFMA throughput probe for gfx950: how many dense bf16 flops per second this GPU's matrix
// cores sustain on v_mfma_f32_32x32x16_bf16, the instruction the attention kernel uses. It is
// measurement context for the attention kernel's MFMA figures, not part of the attention path,
// and it is built as its own library (libsfa_probe.so).
//
// Each wave keeps kChains independent accumulator chains in flight, so that back-to-back MFMAs
// never wait on each other's results; two workgroups of four waves per CU give every SIMD two
// waves. Operands are register-resident and never change, so no memory traffic competes.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;

__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = floatx16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;  // keeps the chains live
}

}  // namespace

// Launches `workgroups` workgroups of 256 threads, each wave issuing iters * 4 MFMAs of
// 32 x 32 x 16 (32,768 flops each). out must hold workgroups * 256 floats (device memory).
// Returns 0 or the hipError_t of the launch.
extern "C" int sfa_probe_mfma(int workgroups, int iters, float* out, hipStream_t stream) {
  if (workgroups < 1 || iters < 1 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(256), 0, stream, iters, out);
  return (int)hipGetLastError();
}
