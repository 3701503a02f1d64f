// Generic split-KV decode over the paged latent cache (VALU, any dims/dtypes).
//
// One workgroup per (partition g, query token j, head i).  For every piece of
// its partition it runs an online softmax over 64-token tiles:
//   s_t = scale * (q~ . c_t + q^R . k^R_t)       ([MLA-93] Core Mechanics 3)
//   u   = sum_t softmax(s)_t c_t                 ([MLA-93] decoding section)
// and writes the piece's normalised output and log-sum-exp to the workspace.
// This path serves small or unusual dims (and fp32), and is an independent
// second GPU implementation for cross-checking the MFMA kernel.
#include "mla_internal.h"

namespace mla {

constexpr int kGenNT = 256;
constexpr int kGenTile = 64;  // tokens per tile (4 threads per token for scores)
constexpr int kGenMaxD = 1024;

template <int CDT>
MLA_DEV float load_cache(const void* cache, const float* scales, int64_t row, int ch, int D,
                         int ntiles) {
  if constexpr (CDT == MLA_FP32) {
    return static_cast<const float*>(cache)[row * D + ch];
  } else if constexpr (CDT == MLA_BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(cache)[row * D + ch]);
  } else {
    const uint8_t* c8 = static_cast<const uint8_t*>(cache);
    return e4m3_to_f32(c8[row * D + ch]) * scales[row * ntiles + (ch >> 7)];
  }
}

template <int ADT>
MLA_DEV float load_act(const void* p, int64_t i) {
  if constexpr (ADT == MLA_FP32)
    return static_cast<const float*>(p)[i];
  else
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

template <int CDT, int ADT>
__global__ __launch_bounds__(kGenNT) void decode_generic_kernel(DecodeArgs a) {
  __shared__ PlanScratch<kGenNT> plan;
  __shared__ float qs[kGenMaxD];
  __shared__ float ps[kGenTile];
  __shared__ float red[kGenNT / kWave];

  const int H = a.H, D = a.D, dc = a.d_latent, bs = a.block_size;
  const int ntiles = (D + 127) / 128;
  // blockIdx.x = (g * n_q + j) * H + i
  const int i = blockIdx.x % H;
  const int j = (blockIdx.x / H) % a.n_q;
  const int g = blockIdx.x / (H * a.n_q);
  const int tid = threadIdx.x;

  plan_for_each_piece<kGenNT>(a.seq_lens, a.batch, bs, a.G, g, plan,
                              [&](int b, int ulo, int uhi, int slot, int L) {
    const int nvis = L - a.n_q + j + 1;  // positions 0 .. L - n_q + j
    const int t_begin = ulo * bs;
    const int t_end = min(uhi * bs, nvis);
    const int64_t qoff = ((int64_t(b) * a.n_q + j) * H + i) * D;
    __syncthreads();
    for (int c = tid; c < D; c += kGenNT) qs[c] = load_act<ADT>(a.q, qoff + c);
    __syncthreads();

    float m = -INFINITY, l = 0.f;
    float acc[kGenMaxD / kGenNT];
#pragma unroll
    for (int r = 0; r < kGenMaxD / kGenNT; ++r) acc[r] = 0.f;

    for (int t0 = t_begin; t0 < t_end; t0 += kGenTile) {
      // scores: 4 threads per token
      const int tk = t0 + tid / 4, part = tid % 4;
      float s = 0.f;
      int64_t row = 0;
      if (tk < t_end) {
        row = int64_t(a.page_table[int64_t(b) * a.max_blocks + tk / bs]) * bs + tk % bs;
        for (int c = part; c < D; c += 4) s += qs[c] * load_cache<CDT>(a.cache, a.scales, row, c, D, ntiles);
      }
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s = tk < t_end ? s * a.scale : -INFINITY;
      const float tmax = block_max<kGenNT>(s, red);
      const float m_new = fmaxf(m, tmax);
      const float p = tk < t_end ? expf(s - m_new) : 0.f;
      const float alpha = expf(m - m_new);  // 0 on the first tile (m = -inf)
      if (part == 0) ps[tid / 4] = p;
      const float psum = block_sum<kGenNT>(part == 0 ? p : 0.f, red);
      l = l * alpha + psum;
      m = m_new;
      __syncthreads();
      const int nt = min(kGenTile, t_end - t0);
#pragma unroll
      for (int r = 0; r < kGenMaxD / kGenNT; ++r) {
        const int c = tid + r * kGenNT;
        if (c < dc) {
          float v = acc[r] * alpha;
          for (int t = 0; t < nt; ++t) {
            const int tt = t0 + t;
            const int64_t rr = int64_t(a.page_table[int64_t(b) * a.max_blocks + tt / bs]) * bs + tt % bs;
            v += ps[t] * load_cache<CDT>(a.cache, a.scales, rr, c, D, ntiles);
          }
          acc[r] = v;
        }
      }
      __syncthreads();
    }
    const size_t obase = ((size_t(slot) * a.n_q + j) * H + i);
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int r = 0; r < kGenMaxD / kGenNT; ++r) {
      const int c = tid + r * kGenNT;
      if (c < dc) {
        if constexpr (ADT == MLA_FP32)
          static_cast<float*>(a.ws_o)[obase * dc + c] = acc[r] * inv;
        else
          static_cast<uint16_t*>(a.ws_o)[obase * dc + c] = f32_to_bf16(acc[r] * inv);
      }
    }
    if (tid == 0) a.ws_lse[obase] = l > 0.f ? m + logf(l) : -INFINITY;
  });
}

template <int CDT, int ADT>
static hipError_t launch_generic(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(unsigned(a.G) * a.n_q * a.H);
  hipLaunchKernelGGL((decode_generic_kernel<CDT, ADT>), grid, dim3(kGenNT), 0, st, a);
  return hipGetLastError();
}

bool decode_generic_supported(const DecodeArgs& a) { return a.D <= kGenMaxD; }

hipError_t launch_decode_generic(const DecodeArgs& a, hipStream_t st) {
  if (a.act_dtype == MLA_FP32) {
    if (a.cache_dtype == MLA_FP32) return launch_generic<MLA_FP32, MLA_FP32>(a, st);
    if (a.cache_dtype == MLA_BF16) return launch_generic<MLA_BF16, MLA_FP32>(a, st);
    return launch_generic<MLA_FP8_E4M3, MLA_FP32>(a, st);
  }
  if (a.cache_dtype == MLA_FP32) return launch_generic<MLA_FP32, MLA_BF16>(a, st);
  if (a.cache_dtype == MLA_BF16) return launch_generic<MLA_BF16, MLA_BF16>(a, st);
  return launch_generic<MLA_FP8_E4M3, MLA_BF16>(a, st);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the pieces of each (sequence, query token, head):
// M = max_s lse_s, w_s = exp(lse_s - M), u = sum_s w_s o_s / sum_s w_s,
// lse = M + ln sum_s w_s.  One workgroup per (b, j) and group of 4 heads;
// 64 threads per head, each owning 8 consecutive channels (two float4).
// ---------------------------------------------------------------------------
constexpr int kCombNT = 256;
constexpr int kCombHeads = kCombNT / 64;
constexpr int kCombChunk = 64;  // pieces weighed per pass

template <int ADT>
__global__ __launch_bounds__(kCombNT) void combine_kernel(CombineArgs a) {
  __shared__ PlanScratch<kCombNT> plan;
  __shared__ float wts[kCombHeads][kCombChunk];
  const int bj = blockIdx.x;
  const int b = bj / a.n_q, j = bj % a.n_q;
  const int hh = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int h = blockIdx.y * kCombHeads + hh;
  int slot0, np;
  plan_lookup<kCombNT>(a.seq_lens, a.batch, a.block_size, a.G, b, plan, &slot0, &np);
  const int H = a.H, dc = a.d_latent;
  const bool live = h < H;
  const size_t orow = (size_t(b) * a.n_q + j) * H + (live ? h : 0);
  auto lse_of = [&](int s) { return a.ws_lse[(size_t(slot0 + s) * a.n_q + j) * H + h]; };
  // global max over the pieces (one wave per head)
  float M = -INFINITY;
  if (live)
    for (int s = lane; s < np; s += 64) M = fmaxf(M, lse_of(s));
  M = wave_max(M);
  float wsum = 0.f;
  // channels of this thread: 8 per chunk of 512
  const int nvec = dc / 8;  // threads needed per head
  float acc[2][8];
  for (int r = 0; r < 2; ++r)
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
  for (int s0 = 0; s0 < np; s0 += kCombChunk) {
    const int cnt = min(kCombChunk, np - s0);
    float w = 0.f;
    if (live && lane < cnt) {
      const float ls = lse_of(s0 + lane);
      w = ls == -INFINITY ? 0.f : expf(ls - M);
    }
    wsum += wave_sum(w);
    __syncthreads();
    wts[hh][lane] = w;
    __syncthreads();
    if (live) {
      for (int r = 0; r < 2; ++r) {
        const int v = lane + 64 * r;  // float8 index within the row
        if (v >= nvec) break;
#pragma unroll 4
        for (int s = 0; s < cnt; ++s) {
          const float ws_ = wts[hh][s];
          const size_t off = ((size_t(slot0 + s0 + s) * a.n_q + j) * H + h) * dc + 8 * v;
          float x[8];
          if constexpr (ADT == MLA_FP32) {
            const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.ws_o) + off);
            const float4 x0 = src[0], x1 = src[1];
            x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
            x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
          } else {
            const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.ws_o) + off);
            const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[2 * e] = __uint_as_float(wv[e] << 16);
              x[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[r][e] += ws_ * x[e];
        }
      }
    }
  }
  if (!live) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  for (int r = 0; r < 2; ++r) {
    const int v = lane + 64 * r;
    if (v >= nvec) break;
    if constexpr (ADT == MLA_FP32) {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.u) + orow * dc + 8 * v);
      dst[0] = float4{acc[r][0] * inv, acc[r][1] * inv, acc[r][2] * inv, acc[r][3] * inv};
      dst[1] = float4{acc[r][4] * inv, acc[r][5] * inv, acc[r][6] * inv, acc[r][7] * inv};
    } else {
      uint32_t pk[4];
      for (int e = 0; e < 4; ++e)
        pk[e] = uint32_t(f32_to_bf16(acc[r][2 * e] * inv)) | (uint32_t(f32_to_bf16(acc[r][2 * e + 1] * inv)) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.u) + orow * dc + 8 * v) = uint4{pk[0], pk[1], pk[2], pk[3]};
    }
  }
  if (lane == 0 && a.lse_out) a.lse_out[orow] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
}

bool combine_vector_ok(const CombineArgs& a) { return a.d_latent % 8 == 0 && a.d_latent <= 1024; }

// Scalar fallback (any d_latent): one thread per channel.
template <int ADT>
__global__ __launch_bounds__(kCombNT) void combine_scalar_kernel(CombineArgs a) {
  __shared__ PlanScratch<kCombNT> plan;
  const int bj = blockIdx.x;
  const int b = bj / a.n_q, j = bj % a.n_q;
  const int h = blockIdx.y;
  int slot0, np;
  plan_lookup<kCombNT>(a.seq_lens, a.batch, a.block_size, a.G, b, plan, &slot0, &np);
  const int H = a.H, dc = a.d_latent;
  float M = -INFINITY;
  for (int s = 0; s < np; ++s) M = fmaxf(M, a.ws_lse[(size_t(slot0 + s) * a.n_q + j) * H + h]);
  float wsum = 0.f;
  for (int s = 0; s < np; ++s) {
    const float ls = a.ws_lse[(size_t(slot0 + s) * a.n_q + j) * H + h];
    wsum += ls == -INFINITY ? 0.f : expf(ls - M);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const size_t orow = (size_t(b) * a.n_q + j) * H + h;
  for (int c = threadIdx.x; c < dc; c += kCombNT) {
    float acc = 0.f;
    for (int s = 0; s < np; ++s) {
      const size_t r = (size_t(slot0 + s) * a.n_q + j) * H + h;
      const float ls = a.ws_lse[r];
      if (ls != -INFINITY) {
        const float o = ADT == MLA_FP32 ? static_cast<const float*>(a.ws_o)[r * dc + c]
                                        : bf16_to_f32(static_cast<const uint16_t*>(a.ws_o)[r * dc + c]);
        acc += expf(ls - M) * o;
      }
    }
    if constexpr (ADT == MLA_FP32)
      static_cast<float*>(a.u)[orow * dc + c] = acc * inv;
    else
      static_cast<uint16_t*>(a.u)[orow * dc + c] = f32_to_bf16(acc * inv);
  }
  if (threadIdx.x == 0 && a.lse_out) a.lse_out[orow] = wsum > 0.f ? M + logf(wsum) : -INFINITY;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  if (combine_vector_ok(a)) {
    dim3 grid(unsigned(a.batch) * a.n_q, unsigned((a.H + kCombHeads - 1) / kCombHeads));
    if (a.act_dtype == MLA_FP32)
      hipLaunchKernelGGL(combine_kernel<MLA_FP32>, grid, dim3(kCombNT), 0, st, a);
    else
      hipLaunchKernelGGL(combine_kernel<MLA_BF16>, grid, dim3(kCombNT), 0, st, a);
  } else {
    dim3 grid(unsigned(a.batch) * a.n_q, unsigned(a.H));
    if (a.act_dtype == MLA_FP32)
      hipLaunchKernelGGL(combine_scalar_kernel<MLA_FP32>, grid, dim3(kCombNT), 0, st, a);
    else
      hipLaunchKernelGGL(combine_scalar_kernel<MLA_BF16>, grid, dim3(kCombNT), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace mla
