// Weight-streaming GEMMs of the decode step on gfx950 matrix cores (bf16 in,
// fp32 accumulate):
//  * append: [c ; k^R] rows = h . [W^DKV ; W^KR]^T as split-K partials, then a
//    per-token finalize (sum of partials, RoPE on k^R, cast, paged write,
//    optional e4m3 tile quantisation)  ([MLA-93] Core Mechanics 1 and 3;
//    decoding section);
//  * out_proj: o[r, i, :] = W^UV_i u[r, i, :]  ([MLA-93] decoding section).
// Both are bound by streaming the weights once.  Operands go straight from
// global memory into the MFMA lane layout (16 contiguous bytes per lane along
// the reduction), so no LDS staging is needed.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kNT = 256;

MLA_DEV bf16x8 ld16(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// --------------------------------------------------------------------------
// out_proj: one workgroup per (head, 64 d_v columns, 64 rows); wave w covers
// rows (w/2)*32.., columns (w%2)*32..  A = u rows, B = W^UV_i rows (both K-contiguous).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kNT) void out_proj_mfma_kernel(OutProjArgs a) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int h = blockIdx.x;
  const int v0 = blockIdx.y * 64 + (w % 2) * 32;
  const int r0 = blockIdx.z * 64 + (w / 2) * 32;
  if (v0 >= a.d_v || r0 >= a.rows) return;
  const int m = lane % 32, g = lane / 32;
  const int H = a.H, dc = a.d_latent, dv = a.d_v;
  const int row = min(r0 + m, a.rows - 1);  // clamped rows are computed, never stored
  const __bf16* arow = static_cast<const __bf16*>(a.u) + (int64_t(row) * H + h) * dc + 8 * g;
  const __bf16* brow = static_cast<const __bf16*>(a.w) + (int64_t(h) * dv + v0 + m) * dc + 8 * g;
  f32x16 acc = {};
  for (int k0 = 0; k0 < dc; k0 += 128) {
    bf16x8 af[8], bf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      af[s] = ld16(arow + k0 + 16 * s);
      bf[s] = ld16(brow + k0 + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s], bf[s], acc, 0, 0, 0);
  }
  __bf16* out = static_cast<__bf16*>(a.out);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = r0 + 8 * (r / 4) + 4 * g + (r % 4);
    if (rr < a.rows) out[(int64_t(rr) * H + h) * dv + v0 + m] = (__bf16)acc[r];
  }
}

// --------------------------------------------------------------------------
// append, step 1: partial[kc][t][n] = sum over the kc-th slice of the model
// dimension of h[t][k] * Wcat[n][k], Wcat = [W^DKV ; W^KR] (n < D).
// One workgroup per (32 tokens, 128 columns, k slice); wave w owns 32 columns.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kNT) void append_partial_kernel(AppendArgs a, float* ws, int kchunk) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int t0 = blockIdx.x * 32;
  const int n0 = blockIdx.y * 128 + w * 32;
  const int kc = blockIdx.z;
  const int D = a.D, dm = a.d_model, dc = a.d_latent;
  if (n0 >= D) return;
  const int m = lane % 32, g = lane / 32;
  const int k_lo = kc * kchunk, k_hi = min(dm, k_lo + kchunk);
  const int tok = min(t0 + m, a.n_tokens - 1);
  const int n = min(n0 + m, D - 1);
  const __bf16* arow = static_cast<const __bf16*>(a.h) + int64_t(tok) * dm + 8 * g;
  const __bf16* brow = n < dc ? static_cast<const __bf16*>(a.w_dkv) + int64_t(n) * dm + 8 * g
                              : static_cast<const __bf16*>(a.w_kr) + int64_t(n - dc) * dm + 8 * g;
  f32x16 acc = {};
  int k0 = k_lo;
  for (; k0 + 128 <= k_hi; k0 += 128) {
    bf16x8 af[8], bf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      af[s] = ld16(arow + k0 + 16 * s);
      bf[s] = ld16(brow + k0 + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s], bf[s], acc, 0, 0, 0);
  }
  for (; k0 < k_hi; k0 += 16)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld16(arow + k0), ld16(brow + k0), acc, 0, 0, 0);
  const int col = n0 + m;
  if (col >= D) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = t0 + 8 * (r / 4) + 4 * g + (r % 4);
    if (t < a.n_tokens) ws[(int64_t(kc) * a.n_tokens + t) * D + col] = acc[r];
  }
}

// --------------------------------------------------------------------------
// append, step 2: one workgroup per token: sum the k-slice partials, rotate
// k^R (rotate-half pairs (j, j + d_R/2), angle pos * base^(-j/(d_R/2)) in
// fp64, cos/sin rounded to fp32), then store in the cache format.
// --------------------------------------------------------------------------
template <int CDT>
__global__ __launch_bounds__(kNT) void append_finalize_kernel(AppendArgs a, const float* ws, int nk) {
  __shared__ float y[1024];
  __shared__ float4 part[4][256];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int D = a.D, dc = a.d_latent, D4 = D / 4;
  // sum of the k-slice partials: 4 groups of 64 threads split the slices,
  // each thread owns float4 column quads q, q+64, ...; loads are independent
  {
    const int q = tid % 64, grp = tid / 64;
    const float4* w4 = reinterpret_cast<const float4*>(ws);
    for (int cq = q; cq < D4; cq += 64) {
      float4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
      int kc = grp;
      for (; kc + 4 < nk; kc += 8) {
        const float4 x0 = w4[(int64_t(kc) * a.n_tokens + t) * D4 + cq];
        const float4 x1 = w4[(int64_t(kc + 4) * a.n_tokens + t) * D4 + cq];
        s0.x += x0.x; s0.y += x0.y; s0.z += x0.z; s0.w += x0.w;
        s1.x += x1.x; s1.y += x1.y; s1.z += x1.z; s1.w += x1.w;
      }
      if (kc < nk) {
        const float4 x0 = w4[(int64_t(kc) * a.n_tokens + t) * D4 + cq];
        s0.x += x0.x; s0.y += x0.y; s0.z += x0.z; s0.w += x0.w;
      }
      part[grp][cq] = float4{s0.x + s1.x, s0.y + s1.y, s0.z + s1.z, s0.w + s1.w};
    }
  }
  __syncthreads();
  for (int cq = tid; cq < D4; cq += kNT) {
    const float4 a0 = part[0][cq], a1 = part[1][cq], a2 = part[2][cq], a3 = part[3][cq];
    y[4 * cq + 0] = (a0.x + a1.x) + (a2.x + a3.x);
    y[4 * cq + 1] = (a0.y + a1.y) + (a2.y + a3.y);
    y[4 * cq + 2] = (a0.z + a1.z) + (a2.z + a3.z);
    y[4 * cq + 3] = (a0.w + a1.w) + (a2.w + a3.w);
  }
  __syncthreads();
  const int pos = a.positions[t];
  const int half = a.d_rope / 2;
  for (int jr = tid; jr < half; jr += kNT) {
    const double theta = double(pos) * pow(double(a.rope_base), -double(jr) / double(half));
    const float cs = float(cos(theta)), sn = float(sin(theta));
    const float x = y[dc + jr], z = y[dc + jr + half];
    y[dc + jr] = x * cs - z * sn;
    y[dc + jr + half] = z * cs + x * sn;
  }
  __syncthreads();
  const int blk = a.page_table[int64_t(a.seq_ids[t]) * a.max_blocks + pos / a.block_size];
  const int64_t row = int64_t(blk) * a.block_size + pos % a.block_size;
  if constexpr (CDT == MLA_BF16) {
    uint16_t* dst = static_cast<uint16_t*>(a.cache) + row * D;
    for (int c = tid; c < D; c += kNT) dst[c] = f32_to_bf16(y[c]);
  } else if constexpr (CDT == MLA_FP32) {
    float* dst = static_cast<float*>(a.cache) + row * D;
    for (int c = tid; c < D; c += kNT) dst[c] = y[c];
  } else {
    // one 128-channel tile per wave-pass: amax, scale = amax/448, codes
    const int ntiles = (D + 127) / 128;
    const int lane = tid % kWave, w = tid / kWave;
    uint8_t* dst = static_cast<uint8_t*>(a.cache) + row * D;
    for (int k = w; k < ntiles; k += kNT / kWave) {
      const int lo = 128 * k, hi = min(D, lo + 128);
      float amax = 0.f;
      for (int c = lo + lane; c < hi; c += kWave) amax = fmaxf(amax, fabsf(y[c]));
      amax = wave_max(amax);
      const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
      for (int c = lo + lane; c < hi; c += kWave) dst[c] = uint8_t(f32_to_e4m3(__fmul_rn(y[c], inv)));
      if (lane == 0) a.scales[row * ntiles + k] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    }
  }
}

}  // namespace

bool out_proj_mfma_supported(const OutProjArgs& a) {
  return a.act_dtype == MLA_BF16 && a.d_latent % 128 == 0 && a.d_v % 32 == 0 &&
         (reinterpret_cast<uintptr_t>(a.u) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.w) % 16) == 0;
}

hipError_t launch_out_proj_mfma(const OutProjArgs& a, hipStream_t st) {
  dim3 grid(unsigned(a.H), unsigned((a.d_v + 63) / 64), unsigned((a.rows + 63) / 64));
  hipLaunchKernelGGL(out_proj_mfma_kernel, grid, dim3(kNT), 0, st, a);
  return hipGetLastError();
}

// Split of the model dimension: enough (tokens x columns x slices) workgroups
// to cover the chip, slices a multiple of 16 wide.
static void append_split(const AppendArgs& a, int* nk, int* kchunk) {
  const int tiles = ((a.n_tokens + 31) / 32) * ((a.D + 127) / 128);
  int want = (512 + tiles - 1) / tiles;
  want = max(1, min(want, a.d_model / 128));
  int chunk = (a.d_model + want - 1) / want;
  chunk = (chunk + 15) / 16 * 16;
  *kchunk = chunk;
  *nk = (a.d_model + chunk - 1) / chunk;
}

bool append_mfma_supported(const AppendArgs& a) {
  return a.act_dtype == MLA_BF16 && a.d_model % 16 == 0 && a.D <= 1024 && a.D % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(a.h) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.w_dkv) % 16) == 0 &&
         (a.d_rope == 0 || (reinterpret_cast<uintptr_t>(a.w_kr) % 16) == 0);
}

size_t append_mfma_workspace(const AppendArgs& a) {
  int nk, chunk;
  append_split(a, &nk, &chunk);
  return size_t(nk) * size_t(a.n_tokens) * size_t(a.D) * sizeof(float);
}

hipError_t launch_append_mfma(const AppendArgs& a, void* ws, hipStream_t st) {
  int nk, chunk;
  append_split(a, &nk, &chunk);
  dim3 g1(unsigned((a.n_tokens + 31) / 32), unsigned((a.D + 127) / 128), unsigned(nk));
  hipLaunchKernelGGL(append_partial_kernel, g1, dim3(kNT), 0, st, a, static_cast<float*>(ws), chunk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(unsigned(a.n_tokens));
  if (a.cache_dtype == MLA_BF16)
    hipLaunchKernelGGL(append_finalize_kernel<MLA_BF16>, g2, dim3(kNT), 0, st, a, static_cast<const float*>(ws), nk);
  else if (a.cache_dtype == MLA_FP32)
    hipLaunchKernelGGL(append_finalize_kernel<MLA_FP32>, g2, dim3(kNT), 0, st, a, static_cast<const float*>(ws), nk);
  else
    hipLaunchKernelGGL(append_finalize_kernel<MLA_FP8_E4M3>, g2, dim3(kNT), 0, st, a, static_cast<const float*>(ws), nk);
  return hipGetLastError();
}

}  // namespace mla
