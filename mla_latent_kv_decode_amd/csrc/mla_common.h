// Internal device helpers of the MLA decode library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

#define MLA_DEV static __device__ __forceinline__
#define MLA_HD __host__ __device__ __forceinline__

// Wait states in front of every buffer load issued from inline asm.  The
// compiler resolves hardware hazards only for instructions it can see, so
// an asm load must cover the ones its operands can meet: an SGPR operand
// (soffset, descriptor) written by a VALU instruction -- v_readfirstlane, or
// a reload of a spilled SGPR with v_readlane -- needs 5 wait states before
// a VMEM instruction reads it, and a write of M0 needs 1 before an LDS DMA
// uses it.
#define MLA_ASM_VMEM_WAIT "s_nop 4\n\t"

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

// Two floats to packed bf16 (round to nearest even) with the gfx950
// conversion instruction.
MLA_DEV uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
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
// Either e4m3 cache format (tile scales of any value, or powers of two).
MLA_HD bool is_fp8_cache(int dt) { return dt == MLA_FP8_E4M3 || dt == MLA_FP8_E4M3_PO2; }

// Exponent E of a power-of-two tile scale: the smallest integer with
// amax <= 448 * 2^E (amax > 0 and finite).  With amax = 1.m * 2^e and
// 448 = 1.75 * 2^8 that is e - 8, or e - 7 when 1.m > 1.75.
MLA_DEV int pow2_scale_exp(float amax) {
  int bias = 0;
  if (amax < 1.17549435e-38f) {  // subnormal: normalise first (exact)
    amax *= 18446744073709551616.0f;  // 2^64
    bias = 64;
  }
  const uint32_t u = __float_as_uint(amax);
  const int e = int((u >> 23) & 0xffu) - 127;
  return (e - 8 + ((u & 0x7fffffu) > 0x600000u ? 1 : 0)) - bias;
}

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

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, then s_barrier.  Unlike __syncthreads() it carries no fence, so
// the compiler does not wait for outstanding global loads first -- loads
// issued earlier (e.g. weights streamed into LDS by direct loads) stay in
// flight across it.  Every barrier of the partition plan is of this kind.
MLA_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Values every lane holds identically, moved to scalar registers: the
// compiler cannot prove that a value read back from LDS or computed with
// vector (e.g. double) arithmetic is wave-uniform, and would otherwise keep
// it in a vector register for as long as it lives.
MLA_DEV int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// threadIdx.x behind an empty asm: what is derived from it is recomputed
// where it is used instead of being hoisted out of loops and kept live (or
// spilled) across long loop bodies that need every register.
MLA_DEV int tid_fresh() {
  int t = int(threadIdx.x);
  asm volatile("" : "+v"(t));
  // (the asm hides the range too: restate it, so that % and / by powers of
  // two stay single masks and shifts instead of signed sequences)
  __builtin_assume(t >= 0 && t < 1024);
  return t;
}
MLA_DEV int64_t uniform64(int64_t v) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(uint64_t(v) >> 32))));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// Inclusive prefix sum across the 64 lanes of a wave with DPP moves (six
// VALU adds, no LDS round trips): shifts by 1, 2, 4 and 8 lanes within each
// row of 16 (lanes without a source add 0), then lane 15 of rows 0 and 2 is
// added to rows 1 and 3, and lane 31 to rows 2 and 3.
MLA_DEV int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// Exclusive scan of one int per thread across the workgroup; returns the
// thread's exclusive prefix and writes the total (wave-uniform) to *total.
template <int NT>
MLA_DEV int block_excl_scan(int v, int* red, int* total) {
  const int t = tid_fresh(), l = t % kWave, w = t / kWave;
  const int incl = wave_incl_scan(v);
  lds_barrier();
  if (l == kWave - 1) red[w] = incl;
  lds_barrier();
  int base = 0, tot = 0;
  for (int i = 0; i < NT / kWave; ++i) {
    if (i < w) base += red[i];
    tot += red[i];
  }
  *total = uniform(tot);
  return base + incl - v;
}

// Two independent exclusive scans for the price of one pair of barriers;
// red holds 2 * NT / 64 ints.
template <int NT>
MLA_DEV int2 block_excl_scan2(int va, int vb, int* red, int* tota, int* totb) {
  const int t = tid_fresh(), l = t % kWave, w = t / kWave;
  const int ia = wave_incl_scan(va), ib = wave_incl_scan(vb);
  lds_barrier();
  if (l == kWave - 1) { red[w] = ia; red[NT / kWave + w] = ib; }
  lds_barrier();
  int ba = 0, bb = 0, sa = 0, sb = 0;
  for (int i = 0; i < NT / kWave; ++i) {
    const int ra = red[i], rb = red[NT / kWave + i];
    if (i < w) { ba += ra; bb += rb; }
    sa += ra;
    sb += rb;
  }
  *tota = uniform(sa);
  *totb = uniform(sb);
  return int2{ba + ia - va, bb + ib - vb};
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
// or stored plan is needed; with B <= NT it costs one load of seq_lens and two
// workgroup scans.
// ---------------------------------------------------------------------------
// floor(num / den) for 0 <= num < 2^52, den > 0: a double division (exact
// enough at these magnitudes that the quotient is off by at most one) and an
// integer correction.  Far shorter code than a 64-bit integer division.
MLA_HD int64_t floor_div(int64_t num, int64_t den) {
  int64_t q = int64_t(double(num) / double(den));
  if (q * den > num) --q;
  else if ((q + 1) * den <= num) ++q;
  return q;
}
// Partitions of T units into G ranges (T < 2^31 and G <= 2^20, which the
// host enforces, keep every product below 2^52).
struct PartGrid {
  int64_t T;
  int G;
  MLA_HD PartGrid(int64_t T_, int G_) : T(T_), G(G_) {}
  MLA_HD int64_t lo(int g) const { return floor_div(int64_t(g) * T, G); }
  MLA_HD int part_of(int64_t u) const {  // partition that owns unit u
    return int(floor_div((u + 1) * int64_t(G) - 1, T));
  }
};
MLA_DEV int units_of(int len, int bs) { return len <= 0 ? 0 : (len + bs - 1) / bs; }

template <int NT>
struct PlanScratch {
  // pieces of this partition in the current chunk of sequences
  int b[NT], ulo[NT], uhi[NT], slot[NT], len[NT];
  int red[2 * NT / kWave];
};

// Where the plan reads the sequence lengths from: a global pointer, or an LDS
// window of one chunk of NT sequences that is filled by a direct load when the
// plan moves to that chunk (lens_stage(src, c) is called by every thread at
// each chunk start).
typedef __attribute__((address_space(3))) const int32_t lds_len_t;
MLA_DEV void lens_stage(const int32_t*, int) {}
MLA_DEV int lens_get(const int32_t* p, int b) { return p[b]; }
struct LdsLensWindow {
  uint32_t lds;          // LDS byte address of a 1 KB window (256 lengths)
  const int32_t* g;      // the lengths in global memory
  int B;
  int cur;               // first sequence of the staged chunk, -1 if none
};
// Wave 0 issues the four direct dword loads (64 lengths each; only 4-byte
// alignment needed) of the window starting at sequence c; lengths past B read
// as 0.  The caller waits for them.
MLA_DEV void lens_window_issue(const LdsLensWindow& w, int c) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(w.g + c), (short)0, min(w.B - c, 256) * 4, 0x00020000);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dword %0, %1, %2 offen lds"
                 :
                 : "v"(int(threadIdx.x) * 4), "s"(r), "s"(i * 256), "{m0}"(w.lds + i * 256)
                 : "memory");
}
MLA_DEV void lens_stage(LdsLensWindow& w, int c) {
  if (c == w.cur) return;  // uniform
  lds_barrier();           // nobody reads the previous window any more
  if (threadIdx.x < kWave) {
    lens_window_issue(w, c);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  lds_barrier();
  w.cur = c;
}
MLA_DEV int lens_get(const LdsLensWindow& w, int b) { return ((lds_len_t*)(uintptr_t)w.lds)[b - w.cur]; }

// T = total units.  Also returns the first chunk's per-thread length,
// exclusive unit prefix and unit total, which the callers reuse (the whole
// plan when B <= NT).
template <int NT, class LenP>
MLA_DEV int plan_total_units(LenP&& seq_lens, int B, int bs, PlanScratch<NT>& sc, int* len0,
                             int* S0, int* tot0) {
  static_assert(NT <= 256, "one length window holds 256 sequences");
  int T = 0;
  *len0 = *S0 = *tot0 = 0;
  for (int c = 0; c < B; c += NT) {
    const int b = c + threadIdx.x;
    lens_stage(seq_lens, c);
    const int len = b < B ? lens_get(seq_lens, b) : 0;
    int tot;
    const int S = block_excl_scan<NT>(units_of(len, bs), sc.red, &tot);
    if (c == 0) { *len0 = len; *S0 = S; *tot0 = tot; }
    T += tot;
  }
  return T;
}

// One chunk of sequences [c, c + NT): writes the pieces of partition g that
// fall in it to sc (in sequence order) and returns their number.  len/S are
// this thread's sequence length and global unit prefix; totP receives the
// chunk's piece total.  With tab non-null, the partition that owns a
// sequence's first unit (for an empty sequence: the one that owns unit S_b,
// or the last) also records the sequence's first slot and piece count in
// tab[2b], tab[2b + 1] -- exactly one partition per sequence, so the combine
// kernels need not plan.
template <int NT>
MLA_DEV int plan_chunk(int c, int len, int S, int bs, const PartGrid& pg, int g, int64_t lo,
                       int64_t hi, int carryP, PlanScratch<NT>& sc, int* totP, int B, int32_t* tab) {
  const int n = units_of(len, bs);
  const int first = n > 0 ? pg.part_of(S) : 0;
  const int pieces = n > 0 ? pg.part_of(int64_t(S) + n - 1) - first + 1 : 0;
  const bool mine = n > 0 && S < hi && int64_t(S) + n > lo;  // sequence meets [lo, hi)
  int cnt;
  const int2 r = block_excl_scan2<NT>(pieces, mine ? 1 : 0, sc.red, totP, &cnt);
  if (mine) {
    sc.b[r.y] = c + int(threadIdx.x);
    sc.ulo[r.y] = int(max(lo, int64_t(S)) - S);
    sc.uhi[r.y] = int(min(hi, int64_t(S) + n) - S);
    sc.slot[r.y] = carryP + r.x + (g - first);
    sc.len[r.y] = len;
  }
  const int b = c + int(threadIdx.x);
  if (tab && b < B) {
    const int owner = n > 0 ? first : min(pg.part_of(S), pg.G - 1);
    if (owner == g) {
      tab[2 * b] = carryP + r.x;
      tab[2 * b + 1] = pieces;
    }
  }
  lds_barrier();
  return cnt;
}

// Calls f(b, unit_lo, unit_hi, slot, seq_len) (units relative to the
// sequence start) for every piece of partition g, in sequence order.  All
// threads call it with identical arguments; f may use barriers.  Only
// workgroup-uniform values stay live across f (the chunk-0 list is built
// before the loop), so f gets the whole register file.
template <int NT, class LenP, class F>
MLA_DEV void plan_for_each_piece(LenP&& seq_lens, int B, int bs, int G, int g,
                                 PlanScratch<NT>& sc, F&& f, int32_t* tab = nullptr) {
  int len0, S0, tot0;
  const int T = plan_total_units<NT>(seq_lens, B, bs, sc, &len0, &S0, &tot0);
  if (T == 0) {  // nothing to attend: every sequence has no pieces
    if (tab && g == 0)
      for (int b = threadIdx.x; b < B; b += NT) tab[2 * b] = tab[2 * b + 1] = 0;
    return;
  }
  G = min(G, T);
  if (g >= G) return;
  const PartGrid pg(T, G);
  const int64_t lo = uniform64(pg.lo(g)), hi = uniform64(pg.lo(g + 1));
  if (lo >= hi) return;
  int totP;
  int cnt = plan_chunk<NT>(0, len0, S0, bs, pg, g, lo, hi, 0, sc, &totP, B, tab);
  int c = 0, carryS = 0, carryP = 0, totN = tot0;
  for (;;) {
    cnt = __builtin_amdgcn_readfirstlane(cnt);
    for (int k = 0; k < cnt; ++k)
      f(sc.b[k], sc.ulo[k], sc.uhi[k], sc.slot[k], sc.len[k]);
    // (the last partition goes on to the end: trailing empty sequences are
    // recorded by it)
    if (c + NT >= B || (carryS + totN >= hi && !(tab && g == G - 1))) return;
    carryS = __builtin_amdgcn_readfirstlane(carryS + totN);
    carryP = __builtin_amdgcn_readfirstlane(carryP + totP);
    c += NT;
    lds_barrier();  // the next chunk rewrites the piece list
    const int b = c + int(threadIdx.x);
    lens_stage(seq_lens, c);
    const int len = b < B ? lens_get(seq_lens, b) : 0;
    const int S = carryS + block_excl_scan<NT>(units_of(len, bs), sc.red, &totN);
    totN = __builtin_amdgcn_readfirstlane(totN);
    cnt = plan_chunk<NT>(c, len, S, bs, pg, g, lo, hi, carryP, sc, &totP, B, tab);
  }
}

// Partial slots a decode over B sequences and G partitions can fill: each
// partition starts at most one piece that is not some sequence's first.
static inline __host__ __device__ size_t ws_slots(int B, int G) { return size_t(B) + size_t(G); }

}  // namespace mla
