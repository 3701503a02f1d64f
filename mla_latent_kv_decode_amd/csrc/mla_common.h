// Internal device helpers of the MLA decode library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

#define MLA_DEV static __device__ __forceinline__

namespace mla {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// storage formats
// ---------------------------------------------------------------------------
MLA_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even fp32 -> bf16 (NaN stays NaN).
MLA_DEV uint16_t f32_to_bf16(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// OCP E4M3: 1 sign, 4 exponent (bias 7), 3 mantissa bits; S.1111.111 = NaN;
// no infinities; largest finite 448.
MLA_DEV float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if (e == 0)
    v = float(m) * 0.001953125f;  // m * 2^-9
  else if (e == 15 && m == 7)
    v = __uint_as_float(0x7fc00000u);
  else
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  return (c & 0x80u) ? -v : v;
}

// fp32 -> E4M3, round to nearest even, magnitudes >= 448 saturate to 448.
MLA_DEV uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;     // NaN
  float ax = __uint_as_float(a);
  if (ax >= 448.0f) return sign | 0x7eu;
  if (ax < 0.015625f) {                          // below 2^-6: subnormal grid m * 2^-9
    float m = __builtin_rintf(ax * 512.0f);      // exact scaling, RNE
    return sign | uint32_t(m);                   // m == 8 is the smallest normal, code 0x08
  }
  uint32_t e = (a >> 23) - 120u;                 // biased e4m3 exponent (>= 1)
  uint32_t code = (e << 3) | ((a >> 20) & 7u);
  uint32_t rest = a & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) code += 1u;
  return sign | (code > 0x7eu ? 0x7eu : code);
}

// ---------------------------------------------------------------------------
// workgroup reductions (NT threads, NT a multiple of 64)
// ---------------------------------------------------------------------------
MLA_DEV float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
MLA_DEV float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
MLA_DEV int wave_sum_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <int NT>
MLA_DEV float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < NT / kWave; ++i) r = fmaxf(r, red[i]);
  return r;
}
template <int NT>
MLA_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < NT / kWave; ++i) r += red[i];
  return r;
}

// Exclusive scan of one int per thread across the workgroup; returns the
// thread's exclusive prefix and writes the total to *total.
template <int NT>
MLA_DEV int block_excl_scan(int v, int* red, int* total) {
  const int l = threadIdx.x % kWave, w = threadIdx.x / kWave;
  int incl = v;
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(incl, o, 64);
    if (l >= o) incl += t;
  }
  __syncthreads();
  if (l == kWave - 1) red[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < NT / kWave; ++i) {
    if (i < w) base += red[i];
    tot += red[i];
  }
  *total = tot;
  return base + incl - v;
}

// ---------------------------------------------------------------------------
// Partition plan.
//
// The cache blocks ("units") of all sequences are laid end to end: sequence b
// owns units [S_b, S_b + n_b), n_b = ceil(seq_lens[b] / block_size), T = sum n_b.
// Partition g of G owns units [floor(gT/G), floor((g+1)T/G)).  A sequence is
// cut into one piece per partition it touches; piece slots are numbered
// sequence by sequence (P_b = slots before sequence b), so there are at most
// B + G - 1 of them.  G is first clamped to T so that no partition is empty
// (an empty partition inside a sequence's span would own a slot it never
// writes).  Every kernel recomputes this from seq_lens, so no planning launch
// or stored plan is needed.
// ---------------------------------------------------------------------------
MLA_DEV int64_t part_lo(int g, int64_t T, int G) { return (int64_t(g) * T) / G; }
MLA_DEV int part_of_unit(int64_t u, int64_t T, int G) {
  return int(((u + 1) * int64_t(G) - 1) / T);
}
MLA_DEV int units_of(int len, int bs) { return len <= 0 ? 0 : (len + bs - 1) / bs; }

template <int NT>
struct PlanScratch {
  int S[NT], P[NT], n[NT], first[NT];
  int red[NT / kWave];
};

template <int NT>
MLA_DEV int plan_total_units(const int32_t* seq_lens, int B, int bs, PlanScratch<NT>& sc) {
  int T = 0;
  for (int c = 0; c < B; c += NT) {
    const int b = c + threadIdx.x;
    int n = b < B ? units_of(seq_lens[b], bs) : 0;
    int tot;
    block_excl_scan<NT>(n, sc.red, &tot);
    T += tot;
  }
  return T;
}

// Calls f(b, unit_lo, unit_hi, slot) (units relative to the sequence start)
// for every piece of partition g, in sequence order.  All threads call it
// with identical arguments; f may use __syncthreads.
template <int NT, class F>
MLA_DEV void plan_for_each_piece(const int32_t* seq_lens, int B, int bs, int G, int g,
                                 PlanScratch<NT>& sc, F&& f) {
  const int T = plan_total_units<NT>(seq_lens, B, bs, sc);
  if (T == 0) return;
  G = min(G, T);
  if (g >= G) return;
  const int64_t lo = part_lo(g, T, G), hi = part_lo(g + 1, T, G);
  if (lo >= hi) return;
  int carryS = 0, carryP = 0;
  for (int c = 0; c < B; c += NT) {
    const int b = c + threadIdx.x;
    const int n = b < B ? units_of(seq_lens[b], bs) : 0;
    int totN, totP;
    const int S = carryS + block_excl_scan<NT>(n, sc.red, &totN);
    const int first = n > 0 ? part_of_unit(S, T, G) : 0;
    const int pieces = n > 0 ? part_of_unit(int64_t(S) + n - 1, T, G) - first + 1 : 0;
    const int P = carryP + block_excl_scan<NT>(pieces, sc.red, &totP);
    sc.S[threadIdx.x] = S;
    sc.P[threadIdx.x] = P;
    sc.n[threadIdx.x] = n;
    sc.first[threadIdx.x] = first;
    __syncthreads();
    const int cnt = min(NT, B - c);
    bool done = false;
    for (int k = 0; k < cnt; ++k) {
      const int Sk = sc.S[k], nk = sc.n[k];
      if (Sk >= hi) { done = true; break; }
      if (int64_t(Sk) + nk <= lo || nk == 0) continue;
      const int ulo = int(max(lo, int64_t(Sk)) - Sk);
      const int uhi = int(min(hi, int64_t(Sk) + nk) - Sk);
      f(c + k, ulo, uhi, sc.P[k] + (g - sc.first[k]));
    }
    __syncthreads();
    if (done) return;
    carryS += totN;
    carryP += totP;
  }
}

// Slot of the first piece of sequence b and its number of pieces.
template <int NT>
MLA_DEV void plan_lookup(const int32_t* seq_lens, int B, int bs, int G, int b,
                         PlanScratch<NT>& sc, int* slot0, int* npieces) {
  const int T = plan_total_units<NT>(seq_lens, B, bs, sc);
  *slot0 = 0;
  *npieces = 0;
  if (T == 0) return;
  G = min(G, T);
  int carryS = 0, carryP = 0;
  for (int c = 0; c <= b; c += NT) {
    const int bb = c + threadIdx.x;
    const int n = bb < B ? units_of(seq_lens[bb], bs) : 0;
    int totN, totP;
    const int S = carryS + block_excl_scan<NT>(n, sc.red, &totN);
    const int first = n > 0 ? part_of_unit(S, T, G) : 0;
    const int pieces = n > 0 ? part_of_unit(int64_t(S) + n - 1, T, G) - first + 1 : 0;
    const int P = carryP + block_excl_scan<NT>(pieces, sc.red, &totP);
    __syncthreads();
    if (bb == b) {
      sc.S[0] = P;
      sc.n[0] = pieces;
    }
    __syncthreads();
    if (b < c + NT) {
      *slot0 = sc.S[0];
      *npieces = sc.n[0];
      __syncthreads();
      return;
    }
    __syncthreads();
    carryS += totN;
    carryP += totP;
  }
}

// Workspace layout: [o: n_slots][n_q][H][d_latent] in the activation dtype |
// [lse: n_slots][n_q][H] fp32.
struct Workspace {
  float* o;
  float* lse;
};
static inline __host__ __device__ size_t ws_slots(int B, int G) { return size_t(B) + size_t(G); }

}  // namespace mla
