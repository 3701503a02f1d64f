// Cache append, second step ([MLA-93] Core Mechanics 1 and 3; decoding
// section): per (token, 128-channel tile) unit, sum the k-slice partials of
// [c ; k^R] = h . [W^DKV ; W^KR]^T, rotate k^R (rotate-half pairs
// (j, j + d_R/2), angle pos * base^(-j/(d_R/2)) in fp64, cos/sin rounded to
// fp32; the host keeps the RoPE part inside one tile), then store the row in
// the cache format (e4m3: the tile's amax sets the scale, amax / 448 or the
// smallest power of two that maps amax into (224, 448]).
//
// A 256-thread workgroup finalises two units, one per 128-thread half, so
// the body can share a launch with other 256-thread work.
#pragma once
#include "mla_internal.h"

namespace mla {

constexpr int kFinNT = 128;  // threads per unit (one per channel of the tile)

// (token, 128-channel tile) units of a call
static __host__ __device__ inline int append_finalize_units(const AppendArgs& a) {
  return a.n_tokens * ((a.D + kFinNT - 1) / kFinNT);
}

// Units 2 * pair and 2 * pair + 1 (unit u = token u / tiles, tile u % tiles).
// A half past the last unit recomputes the last one and stores nothing.
template <int CDT>
MLA_DEV void append_finalize_pair(const AppendArgs& a, const float* ws, int nk, int pair) {
  __shared__ float y_s[2][kFinNT];
  __shared__ float wmax_s[2][kFinNT / kWave];
  const int hw = threadIdx.x / kFinNT, tid = threadIdx.x % kFinNT;
  const int ntiles = (a.D + kFinNT - 1) / kFinNT, units = a.n_tokens * ntiles;
  const int u0 = 2 * pair + hw;
  const bool live = u0 < units;
  const int u = min(u0, units - 1);
  const int t = u / ntiles, tile = u % ntiles;
  float* y = y_s[hw];
  float* wmax = wmax_s[hw];
  const int D = a.D, dc = a.d_latent, T = a.n_tokens;
  const int c = tile * kFinNT + tid;
  float v = 0.f;
  int pos = 0;
  int64_t row = 0;
  {
    // All partials of a chunk are loaded before any is added (unconditional
    // loads of clamped indices, masked after): one memory round trip per 32
    // slices; the sum order is fixed (deterministic).  The token's position
    // and cache row (two dependent scalar lookups) are fetched while the
    // first chunk is in flight.
    const float* p = ws + int64_t(t) * D + min(c, D - 1);
    const int64_t stride = int64_t(T) * D;
    constexpr int kChunk = 32;
    for (int kc0 = 0; kc0 < nk; kc0 += kChunk) {
      float x[kChunk];
#pragma unroll
      for (int i = 0; i < kChunk; ++i) x[i] = p[int64_t(min(kc0 + i, nk - 1)) * stride];
      __builtin_amdgcn_sched_barrier(0);
      if (kc0 == 0) {
        pos = a.positions[t];
        const int blk = a.page_table[int64_t(a.seq_ids[t]) * a.max_blocks + pos / a.block_size];
        row = int64_t(blk) * a.block_size + pos % a.block_size;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < kChunk; ++i)
        if (kc0 + i >= nk) x[i] = 0.f;
#pragma unroll
      for (int w = kChunk / 2; w > 0; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) x[i] += x[i + w];
      v += x[0];
    }
    if (c >= D) v = 0.f;
  }
  y[tid] = v;
  __syncthreads();
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
  const bool st = live && c < D;
  if constexpr (CDT == MLA_BF16) {
    if (st) static_cast<uint16_t*>(a.cache)[row * D + c] = f32_to_bf16(v);
  } else if constexpr (CDT == MLA_FP32) {
    if (st) static_cast<float*>(a.cache)[row * D + c] = v;
  } else {
    const float am = wave_max(c < D ? fabsf(v) : 0.f);
    if (tid % kWave == 0) wmax[tid / kWave] = am;
    __syncthreads();
    const float amax = fmaxf(wmax[0], wmax[1]);
    if constexpr (CDT == MLA_FP8_E4M3_PO2) {  // scale 2^E, codes of v * 2^-E (exact scaling)
      const int e = amax > 0.f ? pow2_scale_exp(amax) : 0;
      if (st) static_cast<uint8_t*>(a.cache)[row * D + c] = uint8_t(f32_to_e4m3(__builtin_ldexpf(v, -e)));
      if (live && tid == 0) a.scales[row * ((D + 127) / 128) + tile] = __builtin_ldexpf(1.0f, e);
    } else {
      const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
      if (st) static_cast<uint8_t*>(a.cache)[row * D + c] = uint8_t(f32_to_e4m3(__fmul_rn(v, inv)));
      if (live && tid == 0) a.scales[row * ((D + 127) / 128) + tile] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    }
  }
}

}  // namespace mla
