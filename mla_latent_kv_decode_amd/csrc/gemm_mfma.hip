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
#include "append_finalize.h"

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
// append, step 1 (tiled form, used when d_latent and d_rope are multiples of
// 64 and d_model of 256 -- DeepSeek-V3's 512 / 64 / 7168): one workgroup per
// (64 columns, 256-wide k slice, 64 tokens).  Both operand tiles (64 rows x
// 512 bytes) are copied into LDS with direct 1 KB loads -- two rows per
// instruction, 16-byte chunks XOR-swizzled by row -- so every request is a
// whole contiguous KB.  Wave w then computes the 32 x 32 block (token half
// w & 1, column half w >> 1) over the whole slice: 16 MFMAs, no cross-wave
// reduction, and stores its fp32 partial straight from the accumulator.
// --------------------------------------------------------------------------
constexpr int kTT = 64, kTC = 64, kTK = 256;   // tokens x columns x k slice
constexpr int kTRow = kTK * 2;                 // 512-byte tile rows
struct AppTileSmem {
  alignas(128) unsigned char h[kTT * kTRow];
  alignas(128) unsigned char w[kTC * kTRow];
};
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8_c;
MLA_DEV uint32_t lds_addr_u8(const unsigned char* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) unsigned char*)p));
}

// rows [0, nrows) of a 64-row tile, row r at src + r * row_stride bytes,
// kTRow bytes each, into dst; rows >= nrows read zeros (descriptor range)
MLA_DEV void tile_to_lds(unsigned char* dst, const unsigned char* src, int nrows, int row_stride, int wave,
                         int lane) {
  const uint32_t range = uint32_t((nrows - 1) * row_stride + kTRow);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, range, 0x00020000);
  for (int i = wave; i < kTT / 2; i += kNT / kWave) {
    const int row = 2 * i + (lane >> 5);
    // lane fills LDS chunk slot lane & 31 of its row with source chunk (lane & 31) ^ (row & 31)
    const uint32_t voff = uint32_t(row * row_stride + (((lane & 31) ^ (row & 31)) << 4));
    asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(r), "{m0}"(lds_addr_u8(dst + i * 1024))
                 : "memory");
  }
}

__global__ __launch_bounds__(kNT) void append_partial_tiled_kernel(AppendArgs a, float* ws) {
  extern __shared__ __attribute__((aligned(128))) unsigned char smem_raw[];
  AppTileSmem& sm = *reinterpret_cast<AppTileSmem*>(smem_raw);
  const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int T = a.n_tokens, D = a.D, dm = a.d_model, dc = a.d_latent;
  // Slice-major and XCD-aware: workgroups are dealt round-robin to the 8
  // XCDs, so consecutive logical ids share one, and all column and token
  // tiles of a k slice (which share its h and W tiles) land on the same
  // XCD and read those tiles from HBM once between them.
  const int nct = D / kTC, ntt = (T + kTT - 1) / kTT;
  const int NB = gridDim.x, xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int logical = xcd * (NB / 8) + min(xcd, NB % 8) + idx;
  const int kc = logical / (nct * ntt), rem = logical % (nct * ntt);
  const int t0 = (rem / nct) * kTT, c0 = (rem % nct) * kTC;
  const int64_t k0 = int64_t(kc) * kTK;
  const unsigned char* hsrc = static_cast<const unsigned char*>(a.h) + (int64_t(t0) * dm + k0) * 2;
  const unsigned char* wsrc =
      c0 < dc ? static_cast<const unsigned char*>(a.w_dkv) + (int64_t(c0) * dm + k0) * 2
              : static_cast<const unsigned char*>(a.w_kr) + (int64_t(c0 - dc) * dm + k0) * 2;
  tile_to_lds(sm.h, hsrc, min(kTT, T - t0), dm * 2, wave, lane);
  tile_to_lds(sm.w, wsrc, kTC, dm * 2, wave, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  const int m = lane % 32, g = lane / 32, th = wave & 1, ch = wave >> 1;
  const uint32_t ha = lds_addr_u8(sm.h) + uint32_t((32 * th + m) * kTRow);
  const uint32_t wa = lds_addr_u8(sm.w) + uint32_t((32 * ch + m) * kTRow);
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < kTK / 16; ++s) {
    const uint32_t slot = uint32_t(((2 * s + g) ^ m) << 4);  // row & 31 == m
    const bf16x8 av = *(lds_bf16x8_c*)(uintptr_t)(ha + slot);
    const bf16x8 bv = *(lds_bf16x8_c*)(uintptr_t)(wa + slot);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
  }
  // lane (g, m) holds tokens 8*(r/4) + 4*g + r%4 (of this half) of column m
  const int col = c0 + 32 * ch + m;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = t0 + 32 * th + 8 * (r / 4) + 4 * g + (r % 4);
    if (t < T) ws[(int64_t(kc) * T + t) * D + col] = acc[r];
  }
}

// append, step 2 (append_finalize.h): two (token, 128-channel tile) units
// per workgroup.
template <int CDT>
__global__ __launch_bounds__(kNT) void append_finalize_kernel(AppendArgs a, const float* ws, int nk) {
  append_finalize_pair<CDT>(a, ws, nk, blockIdx.x);
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

// The tiled partial kernel needs column tiles that do not straddle W^DKV /
// W^KR and k slices that divide the model dimension.
static bool append_tiled(const AppendArgs& a) {
  return a.d_latent % kTC == 0 && a.d_rope % kTC == 0 && a.d_model % kTK == 0;
}

bool append_mfma_supported(const AppendArgs& a) {
  return a.act_dtype == MLA_BF16 && a.d_model % 16 == 0 && a.D <= 1024 && a.D % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(a.h) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.w_dkv) % 16) == 0 &&
         (a.d_rope == 0 || (reinterpret_cast<uintptr_t>(a.w_kr) % 16) == 0);
}

int append_mfma_slices(const AppendArgs& a) {
  int nk, ks;
  append_split(a, &nk, &ks);
  return append_tiled(a) ? a.d_model / kTK : nk;
}

size_t append_mfma_workspace(const AppendArgs& a) {
  return size_t(append_mfma_slices(a)) * size_t(a.n_tokens) * size_t(a.D) * sizeof(float);
}

hipError_t launch_append_partial_mfma(const AppendArgs& a, void* ws, hipStream_t st) {
  const int nk = append_mfma_slices(a);
  if (append_tiled(a)) {
    if (hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(append_partial_tiled_kernel),
                                          int(sizeof(AppTileSmem)));
        e != hipSuccess)
      return e;
    const dim3 g1(unsigned(a.D / kTC) * unsigned(nk) * unsigned((a.n_tokens + kTT - 1) / kTT));
    hipLaunchKernelGGL(append_partial_tiled_kernel, g1, dim3(kNT), sizeof(AppTileSmem), st, a,
                       static_cast<float*>(ws));
  } else {
    int nk_split, ks;  // nk_split == nk for this form
    append_split(a, &nk_split, &ks);
    dim3 g1(unsigned((a.D + kAppCol - 1) / kAppCol), unsigned(nk), unsigned((a.n_tokens + kAppTok - 1) / kAppTok));
    hipLaunchKernelGGL(append_partial_kernel, g1, dim3(kNT), 0, st, a, static_cast<float*>(ws), ks);
  }
  return hipGetLastError();
}

hipError_t launch_append_mfma(const AppendArgs& a, void* ws, hipStream_t st) {
  if (hipError_t e = launch_append_partial_mfma(a, ws, st); e != hipSuccess) return e;
  const int nk = append_mfma_slices(a);
  const dim3 g2(unsigned((append_finalize_units(a) + 1) / 2));
  const float* w = static_cast<const float*>(ws);
  if (a.cache_dtype == MLA_BF16)
    hipLaunchKernelGGL(append_finalize_kernel<MLA_BF16>, g2, dim3(kNT), 0, st, a, w, nk);
  else if (a.cache_dtype == MLA_FP32)
    hipLaunchKernelGGL(append_finalize_kernel<MLA_FP32>, g2, dim3(kNT), 0, st, a, w, nk);
  else if (a.cache_dtype == MLA_FP8_E4M3_PO2)
    hipLaunchKernelGGL(append_finalize_kernel<MLA_FP8_E4M3_PO2>, g2, dim3(kNT), 0, st, a, w, nk);
  else
    hipLaunchKernelGGL(append_finalize_kernel<MLA_FP8_E4M3>, g2, dim3(kNT), 0, st, a, w, nk);
  return hipGetLastError();
}

}  // namespace mla
