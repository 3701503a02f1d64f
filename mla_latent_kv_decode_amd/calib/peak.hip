// Achievable-peak calibration for the benchmark (not part of the MLA ABI):
// a dense bf16 matrix-core loop, timed by the caller, gives the MFMA rate the
// chip sustains (its clock under load included) beside the nominal peak.
//
//   int mla_calib_mfma_loop(int iters, int workgroups, void* sink, void* stream)
//     launches `workgroups` workgroups of 512 threads (two waves per SIMD);
//     every wave issues iters x 32 v_mfma_f32_32x32x16_bf16 into four
//     independent accumulators (32768 flop each) and writes one float per
//     thread to sink (workgroups * 512 floats, device memory) so nothing is
//     optimised away.  Flop count: workgroups * 8 * iters * 32 * 32768.
//     Returns 0, or the HIP error code of the launch.
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) void mfma_loop(float* sink, int iters) {
  const int lane = threadIdx.x % 64;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (i + 1));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * 512 + threadIdx.x] = s;
}

extern "C" int mla_calib_mfma_loop(int iters, int workgroups, void* sink, void* stream) {
  hipLaunchKernelGGL(mfma_loop, dim3(workgroups), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<float*>(sink), iters);
  return int(hipGetLastError());
}
