// Per-head value up-projection o[r, i, :] = W^UV_i u[r, i, :]
// ([MLA-93] decoding section).  Generic VALU path: one workgroup per
// (head, 16-row tile, 128-wide d_v tile), reduction chunks staged in LDS.
#include "mla_internal.h"

namespace mla {

constexpr int kOpNT = 256;
constexpr int kOpRT = 16;   // rows per workgroup
constexpr int kOpVT = 128;  // d_v columns per workgroup
constexpr int kOpKT = 32;

template <int ADT>
MLA_DEV float ldo(const void* p, int64_t i) {
  if constexpr (ADT == MLA_FP32)
    return static_cast<const float*>(p)[i];
  else
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int ADT>
__global__ __launch_bounds__(kOpNT) void out_proj_generic_kernel(OutProjArgs a) {
  __shared__ float us[kOpRT][kOpKT + 1];
  __shared__ float wsh[kOpVT][kOpKT + 1];
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * kOpRT;
  const int v0 = blockIdx.z * kOpVT;
  const int tid = threadIdx.x;
  const int H = a.H, dc = a.d_latent, dv = a.d_v;
  const int vc = tid % kOpVT, rg = tid / kOpVT;  // 2 row groups of 8
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < dc; k0 += kOpKT) {
    for (int e = tid; e < kOpRT * kOpKT; e += kOpNT) {
      const int rr = e / kOpKT, kk = e % kOpKT, r = r0 + rr, k = k0 + kk;
      us[rr][kk] = (r < a.rows && k < dc) ? ldo<ADT>(a.u, (int64_t(r) * H + h) * dc + k) : 0.f;
    }
    for (int e = tid; e < kOpVT * kOpKT; e += kOpNT) {
      const int vv = e / kOpKT, kk = e % kOpKT, v = v0 + vv, k = k0 + kk;
      wsh[vv][kk] = (v < dv && k < dc) ? ldo<ADT>(a.w, (int64_t(h) * dv + v) * dc + k) : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kOpKT; ++kk) {
      const float wv = wsh[vc][kk];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = fmaf(us[rg * 8 + q][kk], wv, acc[q]);
    }
    __syncthreads();
  }
  const int v = v0 + vc;
  if (v >= dv) return;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = r0 + rg * 8 + q;
    if (r >= a.rows) break;
    const int64_t o = (int64_t(r) * H + h) * dv + v;
    if constexpr (ADT == MLA_FP32)
      static_cast<float*>(a.out)[o] = acc[q];
    else
      static_cast<uint16_t*>(a.out)[o] = f32_to_bf16(acc[q]);
  }
}

hipError_t launch_out_proj_generic(const OutProjArgs& a, hipStream_t st) {
  dim3 grid(unsigned(a.H), unsigned((a.rows + kOpRT - 1) / kOpRT),
            unsigned((a.d_v + kOpVT - 1) / kOpVT));
  if (a.act_dtype == MLA_FP32)
    hipLaunchKernelGGL(out_proj_generic_kernel<MLA_FP32>, grid, dim3(kOpNT), 0, st, a);
  else
    hipLaunchKernelGGL(out_proj_generic_kernel<MLA_BF16>, grid, dim3(kOpNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
