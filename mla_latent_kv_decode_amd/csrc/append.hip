// Cache append: c = W^DKV h, k^R = RoPE(W^KR h, pos), row [c ; k^R] written to
// the token's paged slot ([MLA-93] Core Mechanics 1 and 3; decoding
// section), optionally quantised to e4m3 with one fp32 scale per 128-channel
// tile of the row.
//
// One workgroup per (16-token tile, 128-column tile).  Column tiles coincide
// with the fp8 quantisation tiles, so the tile's amax is workgroup-local, and
// the RoPE part (d_rope columns) lies inside one tile, so both members of a
// rotated pair (j, j + d_rope/2) are too.
#include "mla_internal.h"

namespace mla {

constexpr int kApNT = 256;
constexpr int kApTT = 16;   // tokens per workgroup
constexpr int kApTN = 128;  // columns per workgroup (= quantisation tile)
constexpr int kApTK = 32;   // reduction chunk

template <int ADT>
MLA_DEV float ld(const void* p, int64_t i) {
  if constexpr (ADT == MLA_FP32)
    return static_cast<const float*>(p)[i];
  else
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int ADT, int CDT>
__global__ __launch_bounds__(kApNT) void append_kernel(AppendArgs a) {
  __shared__ float hs[kApTT][kApTK + 1];
  __shared__ float ws[kApTN][kApTK + 1];
  __shared__ float ys[kApTT][kApTN + 1];

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kApTT;
  const int n0 = blockIdx.y * kApTN;
  const int D = a.D, dc = a.d_latent, dm = a.d_model;
  const int col = tid % kApTN, tg = tid / kApTN;  // 2 token groups of 8
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < dm; k0 += kApTK) {
    for (int e = tid; e < kApTT * kApTK; e += kApNT) {
      const int tt = e / kApTK, kk = e % kApTK, tok = t0 + tt, k = k0 + kk;
      hs[tt][kk] = (tok < a.n_tokens && k < dm) ? ld<ADT>(a.h, int64_t(tok) * dm + k) : 0.f;
    }
    for (int e = tid; e < kApTN * kApTK; e += kApNT) {
      const int nn = e / kApTK, kk = e % kApTK, n = n0 + nn, k = k0 + kk;
      float w = 0.f;
      if (n < D && k < dm)
        w = n < dc ? ld<ADT>(a.w_dkv, int64_t(n) * dm + k) : ld<ADT>(a.w_kr, int64_t(n - dc) * dm + k);
      ws[nn][kk] = w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kApTK; ++kk) {
      const float wv = ws[col][kk];
#pragma unroll
      for (int r = 0; r < 8; ++r) acc[r] = fmaf(hs[tg * 8 + r][kk], wv, acc[r]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) ys[tg * 8 + r][col] = acc[r];
  __syncthreads();

  // RoPE (rotate-half) on the k^R columns of this tile.
  const int half = a.d_rope / 2;
  if (dc < n0 + kApTN && D > n0) {
    for (int e = tid; e < kApTT * half; e += kApNT) {
      const int tt = e / half, jr = e % half, tok = t0 + tt;
      if (tok >= a.n_tokens) continue;
      const double theta =
          double(a.positions[tok]) * pow(double(a.rope_base), -double(jr) / double(half));
      const float cs = float(cos(theta)), sn = float(sin(theta));
      const int ca = dc + jr - n0, cb = dc + jr + half - n0;
      const float x = ys[tt][ca], y = ys[tt][cb];
      ys[tt][ca] = x * cs - y * sn;
      ys[tt][cb] = y * cs + x * sn;
    }
    __syncthreads();
  }

  // Store: 16 threads per token row, 8 columns each.
  const int tt = tid / 16, sub = tid % 16;
  const int tok = t0 + tt;
  const int ncols = min(kApTN, D - n0);
  int64_t row = 0;
  if (tok < a.n_tokens) {
    const int pos = a.positions[tok];
    const int blk = a.page_table[int64_t(a.seq_ids[tok]) * a.max_blocks + pos / a.block_size];
    row = int64_t(blk) * a.block_size + pos % a.block_size;
  }
  if constexpr (CDT == MLA_FP8_E4M3) {
    float amax = 0.f;
    for (int c = sub; c < ncols; c += 16) amax = fmaxf(amax, fabsf(ys[tt][c]));
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
    const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (tok < a.n_tokens) {
      uint8_t* dst = static_cast<uint8_t*>(a.cache) + row * D + n0;
      for (int c = sub; c < ncols; c += 16) dst[c] = uint8_t(f32_to_e4m3(__fmul_rn(ys[tt][c], inv)));
      if (sub == 0) a.scales[row * ((D + 127) / 128) + blockIdx.y] = scale;
    }
  } else if constexpr (CDT == MLA_FP8_E4M3_PO2) {
    float amax = 0.f;
    for (int c = sub; c < ncols; c += 16) amax = fmaxf(amax, fabsf(ys[tt][c]));
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    const int e = amax > 0.f ? pow2_scale_exp(amax) : 0;
    if (tok < a.n_tokens) {
      uint8_t* dst = static_cast<uint8_t*>(a.cache) + row * D + n0;
      for (int c = sub; c < ncols; c += 16) dst[c] = uint8_t(f32_to_e4m3(__builtin_ldexpf(ys[tt][c], -e)));
      if (sub == 0) a.scales[row * ((D + 127) / 128) + blockIdx.y] = __builtin_ldexpf(1.0f, e);
    }
  } else if constexpr (CDT == MLA_BF16) {
    if (tok < a.n_tokens) {
      uint16_t* dst = static_cast<uint16_t*>(a.cache) + row * D + n0;
      for (int c = sub; c < ncols; c += 16) dst[c] = f32_to_bf16(ys[tt][c]);
    }
  } else {
    if (tok < a.n_tokens) {
      float* dst = static_cast<float*>(a.cache) + row * D + n0;
      for (int c = sub; c < ncols; c += 16) dst[c] = ys[tt][c];
    }
  }
}

bool append_supported(const AppendArgs& a) {
  // the RoPE part must sit inside one 128-column tile
  return a.d_rope % 2 == 0 && a.d_latent / kApTN == (a.D - 1) / kApTN;
}

template <int ADT, int CDT>
static hipError_t launch_t(const AppendArgs& a, hipStream_t st) {
  dim3 grid(unsigned((a.n_tokens + kApTT - 1) / kApTT), unsigned((a.D + kApTN - 1) / kApTN));
  hipLaunchKernelGGL((append_kernel<ADT, CDT>), grid, dim3(kApNT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  if (a.act_dtype == MLA_FP32) {
    if (a.cache_dtype == MLA_FP32) return launch_t<MLA_FP32, MLA_FP32>(a, st);
    if (a.cache_dtype == MLA_BF16) return launch_t<MLA_FP32, MLA_BF16>(a, st);
    if (a.cache_dtype == MLA_FP8_E4M3_PO2) return launch_t<MLA_FP32, MLA_FP8_E4M3_PO2>(a, st);
    return launch_t<MLA_FP32, MLA_FP8_E4M3>(a, st);
  }
  if (a.cache_dtype == MLA_FP32) return launch_t<MLA_BF16, MLA_FP32>(a, st);
  if (a.cache_dtype == MLA_BF16) return launch_t<MLA_BF16, MLA_BF16>(a, st);
  if (a.cache_dtype == MLA_FP8_E4M3_PO2) return launch_t<MLA_BF16, MLA_FP8_E4M3_PO2>(a, st);
  return launch_t<MLA_BF16, MLA_FP8_E4M3>(a, st);
}

}  // namespace mla
