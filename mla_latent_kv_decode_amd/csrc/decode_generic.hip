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

  // the (j = 0, head 0) workgroup of each partition records the slot table
  int32_t* const tab = (i == 0 && j == 0) ? a.ws_tab : nullptr;
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
  }, tab);
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
    return launch_generic<MLA_FP8_E4M3, MLA_FP32>(a, st);  // either e4m3 format: code * fp32 scale
  }
  if (a.cache_dtype == MLA_FP32) return launch_generic<MLA_FP32, MLA_BF16>(a, st);
  if (a.cache_dtype == MLA_BF16) return launch_generic<MLA_BF16, MLA_BF16>(a, st);
  return launch_generic<MLA_FP8_E4M3, MLA_BF16>(a, st);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the pieces of each (sequence, query token, head):
// M = max_s lse_s, w_s = exp(lse_s - M), u = sum_s w_s o_s / sum_s w_s,
// lse = M + ln sum_s w_s.  One workgroup per (b, j) and 16 heads; a wave owns
// 4 heads, a lane 8 consecutive channels of each (16 bytes of bf16 / 32 of
// fp32).  Pieces are merged in chunks of 4 with a running maximum; a chunk's
// lse values and partial rows are all loaded before any of them is used, so
// the wave waits for memory once per chunk.
// ---------------------------------------------------------------------------
constexpr int kCombNT = 256;
constexpr int kCHW = 4;                        // heads per wave
constexpr int kCPC = 4;                        // pieces per chunk
constexpr int kCombHeads = kCombNT / kWave * kCHW;  // heads per workgroup

// 8 consecutive channels of a partial row, kept as loaded (bf16 pairs or fp32)
template <int ADT>
struct Raw8 {
  uint4 w[ADT == MLA_FP32 ? 2 : 1];
  __device__ __forceinline__ void load(const void* base, size_t off) {
    if constexpr (ADT == MLA_FP32) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + off);
      w[0] = src[0];
      w[1] = src[1];
    } else {
      w[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    }
  }
  __device__ __forceinline__ float get(int e) const {
    if constexpr (ADT == MLA_FP32) {
      const uint4& q = w[e / 4];
      const uint32_t v = (e % 4) == 0 ? q.x : (e % 4) == 1 ? q.y : (e % 4) == 2 ? q.z : q.w;
      return __uint_as_float(v);
    } else {
      const uint32_t v = (e / 2) == 0 ? w[0].x : (e / 2) == 1 ? w[0].y : (e / 2) == 2 ? w[0].z : w[0].w;
      return __uint_as_float((e % 2) == 0 ? v << 16 : v & 0xffff0000u);
    }
  }
};

// NV = 8-channel vectors per lane (d_latent <= 512 * NV)
template <int ADT, int NV>
__global__ __launch_bounds__(kCombNT) void combine_kernel(CombineArgs a) {
  const int bj = blockIdx.x;
  const int b = bj / a.n_q, j = bj % a.n_q;
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int slot0 = a.ws_tab[2 * b], np = a.ws_tab[2 * b + 1];
  const int H = a.H, dc = a.d_latent, nvec = dc / 8;
  const int h0 = blockIdx.y * kCombHeads + w * kCHW;
  float M[kCHW], wsum[kCHW], acc[kCHW][NV][8];
#pragma unroll
  for (int k = 0; k < kCHW; ++k) {
    M[k] = -INFINITY;
    wsum[k] = 0.f;
#pragma unroll
    for (int r = 0; r < NV; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[k][r][e] = 0.f;
  }
  for (int s0 = 0; s0 < np; s0 += kCPC) {
    const int cnt = min(kCPC, np - s0);
    float ls[kCHW][kCPC];
    Raw8<ADT> x[kCHW][kCPC][NV];
#pragma unroll
    for (int k = 0; k < kCHW; ++k)
#pragma unroll
      for (int s = 0; s < kCPC; ++s) {
        // unconditional loads from clamped (valid) rows, masked by lse = -inf:
        // a branch around each load would serialise them
        const bool live = s < cnt && h0 + k < H;
        const size_t r = (size_t(slot0 + s0 + min(s, cnt - 1)) * a.n_q + j) * H + min(h0 + k, H - 1);
        (void)live;
        ls[k][s] = a.ws_lse[r];
#pragma unroll
        for (int rr = 0; rr < NV; ++rr)
          x[k][s][rr].load(a.ws_o, r * dc + 8 * min(lane + 64 * rr, nvec - 1));
      }
    __builtin_amdgcn_sched_barrier(0);  // every load of the chunk is issued before the first use
#pragma unroll
    for (int k = 0; k < kCHW; ++k)
#pragma unroll
      for (int s = 0; s < kCPC; ++s)
        if (!(s < cnt && h0 + k < H)) ls[k][s] = -INFINITY;  // mask clamped loads
#pragma unroll
    for (int k = 0; k < kCHW; ++k) {
      float mc = ls[k][0];
#pragma unroll
      for (int s = 1; s < kCPC; ++s) mc = fmaxf(mc, ls[k][s]);
      const float Mn = fmaxf(M[k], mc);
      const float sc = M[k] == -INFINITY ? 0.f : expf(M[k] - Mn);  // rescale earlier chunks
      M[k] = Mn;
      wsum[k] *= sc;
#pragma unroll
      for (int rr = 0; rr < NV; ++rr)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][rr][e] *= sc;
#pragma unroll
      for (int s = 0; s < kCPC; ++s) {
        const float ws_ = ls[k][s] == -INFINITY ? 0.f : expf(ls[k][s] - Mn);
        wsum[k] += ws_;
        if (ws_ != 0.f) {
#pragma unroll
          for (int rr = 0; rr < NV; ++rr)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[k][rr][e] += ws_ * x[k][s][rr].get(e);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kCHW; ++k) {
    const int h = h0 + k;
    if (h >= H) break;
    const size_t orow = (size_t(b) * a.n_q + j) * H + h;
    const float inv = wsum[k] > 0.f ? 1.f / wsum[k] : 0.f;
#pragma unroll
    for (int rr = 0; rr < NV; ++rr) {
      const int v = lane + 64 * rr;
      if (v >= nvec) break;
      if constexpr (ADT == MLA_FP32) {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.u) + orow * dc + 8 * v);
        dst[0] = float4{acc[k][rr][0] * inv, acc[k][rr][1] * inv, acc[k][rr][2] * inv, acc[k][rr][3] * inv};
        dst[1] = float4{acc[k][rr][4] * inv, acc[k][rr][5] * inv, acc[k][rr][6] * inv, acc[k][rr][7] * inv};
      } else {
        uint32_t pk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(acc[k][rr][2 * e] * inv, acc[k][rr][2 * e + 1] * inv);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.u) + orow * dc + 8 * v) = uint4{pk[0], pk[1], pk[2], pk[3]};
      }
    }
    if (lane == 0 && a.lse_out) a.lse_out[orow] = wsum[k] > 0.f ? M[k] + logf(wsum[k]) : -INFINITY;
  }
}

bool combine_vector_ok(const CombineArgs& a) { return a.d_latent % 8 == 0 && a.d_latent <= 1024; }

// Scalar fallback (any d_latent): one thread per channel.
template <int ADT>
__global__ __launch_bounds__(kCombNT) void combine_scalar_kernel(CombineArgs a) {
  const int bj = blockIdx.x;
  const int b = bj / a.n_q, j = bj % a.n_q;
  const int h = blockIdx.y;
  const int slot0 = a.ws_tab[2 * b], np = a.ws_tab[2 * b + 1];
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
    const bool two = a.d_latent > 512;
    if (a.act_dtype == MLA_FP32) {
      if (two) hipLaunchKernelGGL((combine_kernel<MLA_FP32, 2>), grid, dim3(kCombNT), 0, st, a);
      else hipLaunchKernelGGL((combine_kernel<MLA_FP32, 1>), grid, dim3(kCombNT), 0, st, a);
    } else {
      if (two) hipLaunchKernelGGL((combine_kernel<MLA_BF16, 2>), grid, dim3(kCombNT), 0, st, a);
      else hipLaunchKernelGGL((combine_kernel<MLA_BF16, 1>), grid, dim3(kCombNT), 0, st, a);
    }
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
