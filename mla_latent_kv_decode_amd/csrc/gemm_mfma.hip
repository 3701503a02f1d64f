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
// out_proj: one workgroup per (head, 32 d_v columns, 32 rows); the four waves
// split the d_latent reduction (each issues all its loads at once) and meet in
// LDS.  A = u rows, B = W^UV_i rows, both contiguous along the reduction.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kNT) void out_proj_mfma_kernel(OutProjArgs a) {
  __shared__ float red[kNT / kWave][32 * 32];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int h = blockIdx.x, v0 = blockIdx.y * 32, r0 = blockIdx.z * 32;
  const int m = lane % 32, g = lane / 32;
  const int H = a.H, dc = a.d_latent, dv = a.d_v;
  const int row = min(r0 + m, a.rows - 1);  // clamped rows are computed, never stored
  const int col = min(v0 + m, dv - 1);
  const int kq = dc / (kNT / kWave);        // this wave's share of the reduction
  const __bf16* arow = static_cast<const __bf16*>(a.u) + (int64_t(row) * H + h) * dc + w * kq + 8 * g;
  const __bf16* brow = static_cast<const __bf16*>(a.w) + (int64_t(h) * dv + col) * dc + w * kq + 8 * g;
  f32x16 acc = {};
  int k = 0;
  for (; k + 128 <= kq; k += 128) {
    bf16x8 af[8], bf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      af[s] = ld16(arow + k + 16 * s);
      bf[s] = ld16(brow + k + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s], bf[s], acc, 0, 0, 0);
  }
  for (; k < kq; k += 16)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld16(arow + k), ld16(brow + k), acc, 0, 0, 0);
  // lane (g, m) holds rows 8*(r/4) + 4*g + r%4 of column m
#pragma unroll
  for (int r = 0; r < 16; ++r) red[w][(8 * (r / 4) + 4 * g + (r % 4)) * 32 + m] = acc[r];
  __syncthreads();
  __bf16* out = static_cast<__bf16*>(a.out);
  for (int i = threadIdx.x; i < 32 * 32; i += kNT) {
    const int rr = r0 + i / 32, cc = v0 + i % 32;
    const float v = (red[0][i] + red[1][i]) + (red[2][i] + red[3][i]);
    if (rr < a.rows && cc < dv) out[(int64_t(rr) * H + h) * dv + cc] = (__bf16)v;
  }
}

// --------------------------------------------------------------------------
// append, step 1: partial[kc][t][n] = sum over the kc-th slice of the model
// dimension of h[t][k] * Wcat[n][k], Wcat = [W^DKV ; W^KR] (n < D).
// One workgroup per (32 columns, k slice, 64 tokens): the four waves split the
// slice, each accumulating 64 tokens x 32 columns (two MFMA tiles sharing the
// weight fragment), and reduce through LDS, so each weight byte is read once
// per 64 tokens and one fp32 tile per workgroup reaches memory.
// --------------------------------------------------------------------------
constexpr int kAppTok = 64, kAppCol = 32;

__global__ __launch_bounds__(kNT) void append_partial_kernel(AppendArgs a, float* ws, int kslice) {
  __shared__ float red[kNT / kWave][kAppTok * kAppCol];
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const int n0 = blockIdx.x * kAppCol, kc = blockIdx.y, t0 = blockIdx.z * kAppTok;
  const int D = a.D, dm = a.d_model, dc = a.d_latent, T = a.n_tokens;
  const int m = lane % 32, g = lane / 32;
  const int sub = kslice / (kNT / kWave);
  const int k_lo = min(dm, kc * kslice + w * sub), k_hi = min(dm, k_lo + sub);
  const int n = min(n0 + m, D - 1);  // clamped columns are computed, never stored
  const __bf16* brow = (n < dc ? static_cast<const __bf16*>(a.w_dkv) + int64_t(n) * dm
                               : static_cast<const __bf16*>(a.w_kr) + int64_t(n - dc) * dm) + 8 * g;
  const __bf16* h = static_cast<const __bf16*>(a.h);
  const __bf16* arow0 = h + int64_t(min(t0 + m, T - 1)) * dm + 8 * g;
  const __bf16* arow1 = h + int64_t(min(t0 + 32 + m, T - 1)) * dm + 8 * g;
  f32x16 acc0 = {}, acc1 = {};
  int k = k_lo;
  for (; k + 128 <= k_hi; k += 128) {
    bf16x8 a0[8], a1[8], b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      b[s] = ld16(brow + k + 16 * s);
      a0[s] = ld16(arow0 + k + 16 * s);
      a1[s] = ld16(arow1 + k + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[s], b[s], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[s], b[s], acc1, 0, 0, 0);
    }
  }
  for (; k < k_hi; k += 16) {
    const bf16x8 b = ld16(brow + k);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld16(arow0 + k), b, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld16(arow1 + k), b, acc1, 0, 0, 0);
  }
  // lane (g, m) holds tokens 8*(r/4) + 4*g + r%4 (+32 for acc1) of column m
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = 8 * (r / 4) + 4 * g + (r % 4);
    red[w][t * kAppCol + m] = acc0[r];
    red[w][(t + 32) * kAppCol + m] = acc1[r];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kAppTok * kAppCol; i += kNT) {
    const int t = t0 + i / kAppCol, col = n0 + i % kAppCol;
    const float v = (red[0][i] + red[1][i]) + (red[2][i] + red[3][i]);
    if (t < T && col < D) ws[(int64_t(kc) * T + t) * D + col] = v;
  }
}

// --------------------------------------------------------------------------
// append, step 2: one 128-thread workgroup per (token, 128-channel tile): sum
// the k-slice partials of its columns, rotate k^R (rotate-half pairs
// (j, j + d_R/2), angle pos * base^(-j/(d_R/2)) in fp64, cos/sin rounded to
// fp32; the host keeps the RoPE part inside one tile), then store in the
// cache format (e4m3: the tile's amax sets the scale).
// --------------------------------------------------------------------------
constexpr int kFinNT = 128;

template <int CDT>
__global__ __launch_bounds__(kFinNT) void append_finalize_kernel(AppendArgs a, const float* ws, int nk) {
  __shared__ float y[kFinNT];
  __shared__ float wmax[kFinNT / kWave];
  const int t = blockIdx.x, tile = blockIdx.y, tid = threadIdx.x;
  const int D = a.D, dc = a.d_latent, T = a.n_tokens;
  const int c = tile * kFinNT + tid;
  float v = 0.f;
  if (c < D) {
    const float* p = ws + int64_t(t) * D + c;
    const int64_t stride = int64_t(T) * D;
    float s0 = 0.f, s1 = 0.f;  // two chains, fixed order: deterministic
    int kc = 0;
    for (; kc + 1 < nk; kc += 2) {
      s0 += p[int64_t(kc) * stride];
      s1 += p[int64_t(kc + 1) * stride];
    }
    if (kc < nk) s0 += p[int64_t(kc) * stride];
    v = s0 + s1;
  }
  y[tid] = v;
  __syncthreads();
  const int pos = a.positions[t];
  const int half = a.d_rope / 2;
  const int jr = c - dc;
  if (jr >= 0 && jr < half) {  // this thread owns the pair (jr, jr + half)
    const double theta = double(pos) * pow(double(a.rope_base), -double(jr) / double(half));
    const float cs = float(cos(theta)), sn = float(sin(theta));
    const float x = y[tid], z = y[tid + half];
    y[tid] = x * cs - z * sn;
    y[tid + half] = z * cs + x * sn;
  }
  __syncthreads();
  v = y[tid];
  const int blk = a.page_table[int64_t(a.seq_ids[t]) * a.max_blocks + pos / a.block_size];
  const int64_t row = int64_t(blk) * a.block_size + pos % a.block_size;
  if constexpr (CDT == MLA_BF16) {
    if (c < D) static_cast<uint16_t*>(a.cache)[row * D + c] = f32_to_bf16(v);
  } else if constexpr (CDT == MLA_FP32) {
    if (c < D) static_cast<float*>(a.cache)[row * D + c] = v;
  } else {
    const float am = wave_max(c < D ? fabsf(v) : 0.f);
    if (tid % kWave == 0) wmax[tid / kWave] = am;
    __syncthreads();
    const float amax = fmaxf(wmax[0], wmax[1]);
    const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
    if (c < D) static_cast<uint8_t*>(a.cache)[row * D + c] = uint8_t(f32_to_e4m3(__fmul_rn(v, inv)));
    if (tid == 0) a.scales[row * ((D + 127) / 128) + tile] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  }
}

}  // namespace

bool out_proj_mfma_supported(const OutProjArgs& a) {
  return a.act_dtype == MLA_BF16 && a.d_latent % 64 == 0 &&
         (reinterpret_cast<uintptr_t>(a.u) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.w) % 16) == 0;
}

hipError_t launch_out_proj_mfma(const OutProjArgs& a, hipStream_t st) {
  dim3 grid(unsigned(a.H), unsigned((a.d_v + 31) / 32), unsigned((a.rows + 31) / 32));
  hipLaunchKernelGGL(out_proj_mfma_kernel, grid, dim3(kNT), 0, st, a);
  return hipGetLastError();
}

// Split of the model dimension: about 256 workgroups over (column tiles x
// token tiles x slices); slices are a multiple of 64 wide (16 per wave).
static void append_split(const AppendArgs& a, int* nk, int* kslice) {
  const int tiles = ((a.D + kAppCol - 1) / kAppCol) * ((a.n_tokens + kAppTok - 1) / kAppTok);
  int want = (256 + tiles - 1) / tiles;
  want = max(1, min(want, a.d_model / 64));
  int ks = (a.d_model + want - 1) / want;
  ks = (ks + 63) / 64 * 64;
  *kslice = ks;
  *nk = (a.d_model + ks - 1) / ks;
}

bool append_mfma_supported(const AppendArgs& a) {
  return a.act_dtype == MLA_BF16 && a.d_model % 16 == 0 && a.D <= 1024 && a.D % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(a.h) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.w_dkv) % 16) == 0 &&
         (a.d_rope == 0 || (reinterpret_cast<uintptr_t>(a.w_kr) % 16) == 0);
}

size_t append_mfma_workspace(const AppendArgs& a) {
  int nk, ks;
  append_split(a, &nk, &ks);
  return size_t(nk) * size_t(a.n_tokens) * size_t(a.D) * sizeof(float);
}

hipError_t launch_append_mfma(const AppendArgs& a, void* ws, hipStream_t st) {
  int nk, ks;
  append_split(a, &nk, &ks);
  dim3 g1(unsigned((a.D + kAppCol - 1) / kAppCol), unsigned(nk), unsigned((a.n_tokens + kAppTok - 1) / kAppTok));
  hipLaunchKernelGGL(append_partial_kernel, g1, dim3(kNT), 0, st, a, static_cast<float*>(ws), ks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g2(unsigned(a.n_tokens), unsigned((a.D + kFinNT - 1) / kFinNT));
  const float* w = static_cast<const float*>(ws);
  if (a.cache_dtype == MLA_BF16)
    hipLaunchKernelGGL(append_finalize_kernel<MLA_BF16>, g2, dim3(kFinNT), 0, st, a, w, nk);
  else if (a.cache_dtype == MLA_FP32)
    hipLaunchKernelGGL(append_finalize_kernel<MLA_FP32>, g2, dim3(kFinNT), 0, st, a, w, nk);
  else
    hipLaunchKernelGGL(append_finalize_kernel<MLA_FP8_E4M3>, g2, dim3(kFinNT), 0, st, a, w, nk);
  return hipGetLastError();
}

}  // namespace mla
