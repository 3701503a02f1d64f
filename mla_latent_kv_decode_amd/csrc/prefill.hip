// Chunked prefill over the latent cache in the un-absorbed form, gfx950.
//
// What it computes ("DeepSeek MLA Architecture: How Multi-Head Latent
// Attention Cuts KV Cache by 93%": the prefill/decode contrast at its start,
// and Core Mechanics 1-3): the C tokens of a prompt chunk attend, causally, to
// the T cached tokens of their sequence, the chunk's own rows last.  For a
// long chunk the per-head keys and values are expanded from the cached
// latents once per chunk,
//   k_{t,i} = [W^UK_i c_t ; k^R_t]  (192 wide),   v_{t,i} = W^UV_i c_t  (128),
// and head i of chunk token j (position T - C + j) gets
//   o = sum_t softmax_t(scale * [q^C ; RoPE(q^R)] . k_t) v_t   over t <= T - C + j.
//
// Steps (launched by mla_prefill):
//  1. prefill_gather_kernel: the sequence's rows from the paged cache into
//     contiguous c [T][512] and k^R [T][64]; prefill_rope_kernel: the chunk's
//     queries with q^R rotated at each token's position;
//  2. the expansion, two matrix-core linear layers (mla_linear's kernel):
//     K^C = c W^UK^T [T][H*128] and V = c W^UV^T [T][H*128];
//  3. prefill_attn_kernel: one workgroup per (head, 128 chunk tokens), four
//     waves of 32 tokens.  Key/value steps of 32 cached tokens (12 KB of keys,
//     8 KB of values) move HBM -> LDS once with direct loads and serve the
//     four waves; scores S^T = K . Q^T and outputs O^T += V^T . P^T run on
//     v_mfma_f32_32x32x16_bf16 with the decode kernel's register layouts
//     (one query per lane of the score accumulator, which already is the P
//     operand; V^T read with ds_read_b64_tr_b16); online softmax in log2
//     units against a per-query reference, rescaled only when a step's
//     probabilities would leave the headroom.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kH = 128, kDC = 512, kDR = 64, kDN = 128, kDV = 128;
constexpr int kDK = kDN + kDR;                  // per-head key width, 192
constexpr int kNT = 256;                        // 4 waves x 32 chunk tokens
constexpr int kRowsPerWG = 128;
constexpr int kStep = 32;                       // cached tokens per step
constexpr int kKG = kDK * 2 / 128;              // 3 column groups (8 chunks of 16 B) per key row
constexpr int kVG = kDV * 2 / 128;              // 2 per value row
constexpr int kKBytes = kStep * kDK * 2;        // 12 KB
constexpr int kBufBytes = kKBytes + kStep * kDV * 2;  // + 8 KB of values
constexpr int kNBuf = 4;                        // steps h-1 (PV), h (QK), h+1 and h+2 in flight
constexpr int kQK = kDK / 16;                   // score MFMAs per step
constexpr int kPV = 2 * (kDV / 32);             // output MFMAs per step
constexpr int kLoads = (kStep / 8) * (kKG + kVG);        // 1 KB sub-block loads per step
constexpr int kLoadsPerWave = kLoads / (kNT / kWave);    // 5
constexpr float kPSumLimit = 4294967296.0f;     // 2^32: a lane's 16 probabilities of a step
static_assert(kLoads % (kNT / kWave) == 0, "loads split evenly over the waves");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

// 16-byte-chunk swizzle inside an 8-token x 8-chunk sub-block (as the decode's).
MLA_DEV int swz(int t) { return ((((t & 3) << 1) | ((t >> 2) & 1)) ^ ((t >> 2) & 2)) & 7; }
// Byte offset of chunk c of token t in a region of rows of ng column groups.
MLA_DEV int sub_off(int t, int c, int ng) {
  return (((t >> 3) * ng + (c >> 3)) * 64 + (t & 7) * 8 + ((c & 7) ^ swz(t))) * 16;
}
MLA_DEV uint32_t lds_addr(const unsigned char* p) { return uint32_t(reinterpret_cast<uintptr_t>((const lds_u8*)p)); }
MLA_DEV bf16x8 lds_b128_at(uint32_t addr) { return *(lds_bf16x8*)(uintptr_t)addr; }
MLA_DEV bf16x8 lds_tr_pair_at(uint32_t p0, uint32_t p1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p0);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p1);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}
template <int N>
MLA_DEV void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
MLA_DEV void step_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Score MFMAs with the accumulator in VGPRs, output MFMAs with it in AGPRs
// (the same constraints, and hazard handling, as the decode kernel).
MLA_DEV void mfma_qk_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
MLA_DEV void mfma_qk(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
MLA_DEV void scores_ready(f32x16& s) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s)); }
MLA_DEV void mfma_pv(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
MLA_DEV void zero_acc(f32x16& acc, const bf16x8& z) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
}
MLA_DEV void o_ready(f32x16 (&O)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]));
}

// One 1 KB direct load into LDS: 8 rows of 8 chunks of 16 bytes; lane l
// fills slot l % 8 of row l / 8 with the row's chunk (l % 8) ^ swz(t).
MLA_DEV void load_sub(__amdgpu_buffer_rsrc_t r, uint32_t lds, int voff, int soff) {
  asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(r), "s"(soff), "{m0}"(lds)
               : "memory");
}

MLA_DEV void rope_pair(float x, float z, int pos, double inv_freq, float* y0, float* y1) {
  double sd, cd;
  sincos(double(pos) * inv_freq, &sd, &cd);
  const float cs = float(cd), sn = float(sd);
  *y0 = x * cs - z * sn;
  *y1 = z * cs + x * sn;
}

// The chunk's queries with q^R rotated at each token's position (rotate-half
// pairs (j, j + 32), angle pos * base^(-j/32) in fp64, cos/sin rounded to
// fp32): one thread per (token, head, pair); q^C is copied through.
__global__ __launch_bounds__(kNT) void prefill_rope_kernel(PrefillArgs a) {
  const int64_t i = int64_t(blockIdx.x) * kNT + threadIdx.x;
  if (i >= int64_t(a.n_tokens) * kH * (kDR / 2 + kDN / 2)) return;
  const int per = kDR / 2 + kDN / 2;  // 32 RoPE pairs + 64 pairs of q^C channels per head
  const int64_t row = i / per;        // token * H + head
  const int k = int(i % per);
  const uint32_t* src = reinterpret_cast<const uint32_t*>(static_cast<const __bf16*>(a.q) + row * kDK);
  uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<__bf16*>(a.ws_q) + row * kDK);
  if (k < kDN / 2) {  // two q^C channels
    dst[k] = src[k];
    return;
  }
  const int j = k - kDN / 2;
  const __bf16* q = static_cast<const __bf16*>(a.q) + row * kDK + kDN;
  __bf16* o = static_cast<__bf16*>(a.ws_q) + row * kDK + kDN;
  const int pos = a.seq_len - a.n_tokens + int(row / kH);
  float y0, y1;
  rope_pair(float(q[j]), float(q[j + kDR / 2]), pos, pow(double(a.rope_base), -double(j) / double(kDR / 2)), &y0, &y1);
  o[j] = (__bf16)y0;
  o[j + kDR / 2] = (__bf16)y1;
}

__global__ __launch_bounds__(kNT) void prefill_gather_kernel(PrefillArgs a) {
  // one 16-byte chunk per thread: row t, chunk k of 72 (64 latent + 8 RoPE)
  const int64_t i = int64_t(blockIdx.x) * kNT + threadIdx.x;
  if (i >= int64_t(a.seq_len) * 72) return;
  const int t = int(i / 72), k = int(i % 72);
  const int blk = a.page_table[t / a.block_size];
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(a.cache) +
                                                    (int64_t(blk) * a.block_size + t % a.block_size) * (kDC + kDR) * 2);
  const uint4 v = src[k];
  if (k < 64)
    reinterpret_cast<uint4*>(a.ws_c)[int64_t(t) * 64 + k] = v;
  else
    reinterpret_cast<uint4*>(a.ws_kr)[int64_t(t) * 8 + (k - 64)] = v;
}

__global__ __launch_bounds__(kNT, 2) void prefill_attn_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(128))) unsigned char smem[];
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int hl = lane % 32, g = lane / 32;
  const int nqb = (a.n_tokens + kRowsPerWG - 1) / kRowsPerWG;
  // the query blocks of one head run one after another on one XCD
  const int NB = gridDim.x, xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int logical = xcd * (NB / 8) + min(xcd, NB % 8) + idx;
  const int h = logical / nqb, qb = logical % nqb;
  const int C = a.n_tokens, T = a.seq_len, p0 = T - C;
  const int q_row = qb * kRowsPerWG + wave * 32 + hl;       // this lane's chunk token
  const int q_lim = p0 + min(q_row, C - 1);                 // last position it sees
  // the workgroup's last token sees positions up to p0 + last row
  const int t_end = p0 + min(C, (qb + 1) * kRowsPerWG);     // positions [0, t_end)
  const int nsteps = (t_end + kStep - 1) / kStep;
  const float c_log2 = a.scale * 1.4426950408889634f;

  // ---- Q^T fragments (lane (g, hl): chunk 2n + g of row q_row; q^R rotated
  // by prefill_rope_kernel) ----
  bf16x8 qf[kQK];
  {
    const bf16x8* src = reinterpret_cast<const bf16x8*>(static_cast<const unsigned char*>(a.ws_q) +
                                                        (int64_t(min(q_row, C - 1)) * kH + h) * kDK * 2);
#pragma unroll
    for (int n = 0; n < kQK; ++n) qf[n] = src[2 * n + g];
  }

  // ---- loads of one step: 12 key sub-blocks (3 column groups: K^C, K^C, k^R)
  // and 8 value sub-blocks per step; wave w issues loads 5w .. 5w + 4 ----
  const int64_t row_bytes = int64_t(kH) * kDN * 2;  // one token's K^C (or V) row of all heads
  auto issue_step = [&](int s) __attribute__((always_inline)) {
    const int t0 = s * kStep;
    const int nvalid = min(kStep, T - t0);
    unsigned char* buf = smem + (s % kNBuf) * kBufBytes;
    const unsigned char* kc = static_cast<const unsigned char*>(a.ws_kc) + int64_t(t0) * row_bytes + h * kDN * 2;
    const unsigned char* vv = static_cast<const unsigned char*>(a.ws_v) + int64_t(t0) * row_bytes + h * kDV * 2;
    const unsigned char* kr = static_cast<const unsigned char*>(a.ws_kr) + int64_t(t0) * kDR * 2;
    // descriptors cover the live rows only: rows past T read as zeros
    const __amdgpu_buffer_rsrc_t rkc = __builtin_amdgcn_make_buffer_rsrc((void*)kc, (short)0,
        int(int64_t(nvalid - 1) * row_bytes + kDN * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vv, (short)0,
        int(int64_t(nvalid - 1) * row_bytes + kDV * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rkr = __builtin_amdgcn_make_buffer_rsrc((void*)kr, (short)0, nvalid * kDR * 2, 0x00020000);
#pragma unroll
    for (int m = 0; m < kLoadsPerWave; ++m) {
      const int k = wave * kLoadsPerWave + m;  // wave-uniform
      const int t = (k < 12 ? (k / 3) : ((k - 12) / 2)) * 8 + lane / 8;  // token inside the step
      const int slot = lane % 8, chunk = slot ^ swz(t);
      if (k < 12) {
        const int tg = k / 3, cg = k % 3;
        const uint32_t dst = lds_addr(buf) + uint32_t((tg * kKG + cg) * 1024);
        if (cg < 2)
          load_sub(rkc, dst, int((t) * row_bytes) + chunk * 16, cg * 128);
        else
          load_sub(rkr, dst, t * kDR * 2 + chunk * 16, 0);
      } else {
        const int kk = k - 12, tg = kk / 2, cg = kk % 2;
        const uint32_t dst = lds_addr(buf) + uint32_t(kKBytes + (tg * kVG + cg) * 1024);
        load_sub(rv, dst, int((t) * row_bytes) + chunk * 16, cg * 128);
      }
    }
  };

  // fragment offsets (see the decode kernel: the same layouts with 3 and 2
  // column groups per row instead of 9)
  const uint32_t koff0 = uint32_t(sub_off(hl, g, kKG));
  const int gg = lane >> 5, hh = (lane >> 4) & 1, ss = lane & 15;
  const uint32_t voff0 = uint32_t(sub_off(4 * gg + (ss >> 2), 2 * hh + ((ss & 3) >> 1), kVG) + 8 * (ss & 1));

  f32x16 O[kDV / 32];
  {
    const bf16x8 z = {};
#pragma unroll
    for (int cb = 0; cb < kDV / 32; ++cb) zero_acc(O[cb], z);
  }
  float m_ref = -INFINITY, l_run = 0.f;
  bf16x8 p_prev[2] = {};
  uint32_t p_cur[2][4];

  auto run_step = [&](auto qk_on, int h_) __attribute__((always_inline)) {
    constexpr bool kQKOn = decltype(qk_on)::value;
    const uint32_t kb = lds_addr(smem + (h_ % kNBuf) * kBufBytes) + koff0;
    const uint32_t vb = lds_addr(smem + ((h_ + kNBuf - 1) % kNBuf) * kBufBytes + kKBytes) + voff0;
    auto kfrag = [&](int n) __attribute__((always_inline)) {  // chunk pair n & 3 of column group n >> 2
      return lds_b128_at((kb ^ uint32_t((n & 3) << 5)) + uint32_t((n >> 2) * 1024));
    };
    auto vfrag = [&](int n) __attribute__((always_inline)) {  // block n >> 1, token half n & 1
      const int i = n & 1, cb = n >> 1;
      const uint32_t base = uint32_t((2 * i) * (kVG * 1024) + (cb >> 1) * 1024);
      const uint32_t v = vb ^ uint32_t((cb & 1) << 6);
      return lds_tr_pair_at(v + base, (v ^ 32u) + base + uint32_t(kVG * 1024));
    };
    f32x16 S;
    bf16x8 vr[4];
    if constexpr (kQKOn) {
      bf16x8 kr[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) kr[n] = kfrag(n);
#pragma unroll
      for (int n = 0; n < kQK; ++n) {
        if (n == 0)
          mfma_qk_first(S, kr[0], qf[0]);
        else
          mfma_qk(S, kr[n % 4], qf[n]);
        if (n + 4 < kQK)
          kr[n % 4] = kfrag(n + 4);
        else if (h_ > 0)
          vr[n + 4 - kQK] = vfrag(n + 4 - kQK);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int n = 0; n < 4; ++n) vr[n] = vfrag(n);
    }
    // softmax of step h_ (lane = one chunk token; tokens 8*(r/4) + 4*g + r%4)
    float lsum = 0.f, lsum2 = 0.f;
    auto softmax_part = [&](int k) __attribute__((always_inline)) {
      if constexpr (kQKOn) {
        if (k == 0) {
          scores_ready(S);
          const int lim = q_lim - (h_ * kStep + 4 * g);  // causal: token index <= q_lim
#pragma unroll
          for (int r = 0; r < 16; ++r) S[r] = (8 * (r / 4) + (r % 4) > lim) ? -INFINITY : S[r];
        }
        if (k >= 1 && k < 9) {
          const int i = (k - 1) >> 2, e = 2 * ((k - 1) & 3);
          const float p0 = __builtin_amdgcn_exp2f(fmaf(S[8 * i + e], c_log2, -m_ref));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(S[8 * i + e + 1], c_log2, -m_ref));
          lsum += p0;
          lsum2 += p1;
          p_cur[i][e / 2] = pack_bf16x2(p0, p1);
          asm volatile("" : "+v"(p_cur[i][e / 2]), "+v"(lsum), "+v"(lsum2));
        }
      }
    };
    if (h_ > 0) {
#pragma unroll
      for (int n = 0; n < kPV; ++n) {
        mfma_pv(O[n >> 1], vr[n % 4], p_prev[n & 1]);
        if (n + 4 < kPV) vr[n % 4] = vfrag(n + 4);
        softmax_part(n);
        softmax_part(n + kPV);  // parts 8.. run behind the last MFMAs
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 2 * kPV; ++k) softmax_part(k);
    }
    if constexpr (kQKOn) {
      if (h_ == 0 || __any(!(lsum + lsum2 <= kPSumLimit))) {
        // exact path: the step's maximum per token (both lane halves), the
        // reference moved to it, the step's p recomputed, O rescaled
        float mx = S[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c_log2;
        const float m_new = h_ == 0 ? mx : fmaxf(m_ref, mx);
        const float corr = h_ == 0 ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        lsum = lsum2 = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(S[8 * i + e], c_log2, -m_ref));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(S[8 * i + e + 1], c_log2, -m_ref));
            lsum += p0;
            lsum2 += p1;
            p_cur[i][e / 2] = pack_bf16x2(p0, p1);
          }
        if (h_ != 0) {
          o_ready(O);
#pragma unroll
          for (int cb = 0; cb < kDV / 32; ++cb) {
            O[cb] *= corr;
            asm volatile("" : "+a"(O[cb]));
          }
        }
        l_run *= corr;
      }
      l_run += lsum + lsum2;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        p_prev[i] = __builtin_bit_cast(bf16x8, u32x4{p_cur[i][0], p_cur[i][1], p_cur[i][2], p_cur[i][3]});
    }
  };

  issue_step(0);
  if (nsteps > 1) issue_step(1);
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps)
      wait_vm<kLoadsPerWave>();
    else
      wait_vm<0>();
    step_barrier();  // step s visible; buffer (s + 2) % 4 free
    if (s + 2 < nsteps) issue_step(s + 2);
    run_step(std::true_type{}, s);
  }
  run_step(std::false_type{}, nsteps);  // PV of the last step
  o_ready(O);

  // ---- epilogue: o = O / l, bf16, this lane's token hl, 64 of 128 channels ----
  if (q_row < C) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    const float inv = 1.f / (__uint_as_float(sw[0]) + __uint_as_float(sw[1]));
    __bf16* out = static_cast<__bf16*>(a.out) + (int64_t(q_row) * kH + h) * kDV;
#pragma unroll
    for (int cb = 0; cb < kDV / 32; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint32_t lo = pack_bf16x2(O[cb][4 * rg + 0] * inv, O[cb][4 * rg + 1] * inv);
        const uint32_t hi = pack_bf16x2(O[cb][4 * rg + 2] * inv, O[cb][4 * rg + 3] * inv);
        *reinterpret_cast<uint2*>(out + 32 * cb + 8 * rg + 4 * g) = uint2{lo, hi};
      }
  }
}

}  // namespace

bool prefill_supported(const PrefillArgs& a) {
  return a.H == kH && a.d_latent == kDC && a.d_rope == kDR && a.d_nope == kDN && a.d_v == kDV &&
         (reinterpret_cast<uintptr_t>(a.q) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.cache) % 16) == 0 &&
         (reinterpret_cast<uintptr_t>(a.out) % 8) == 0;
}

hipError_t launch_prefill_gather(const PrefillArgs& a, hipStream_t st) {
  const int64_t n = int64_t(a.seq_len) * 72;
  hipLaunchKernelGGL(prefill_gather_kernel, dim3(unsigned((n + kNT - 1) / kNT)), dim3(kNT), 0, st, a);
  const int64_t m = int64_t(a.n_tokens) * kH * (kDR / 2 + kDN / 2);
  hipLaunchKernelGGL(prefill_rope_kernel, dim3(unsigned((m + kNT - 1) / kNT)), dim3(kNT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t st) {
  const int smem = kNBuf * kBufBytes;
  if (hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(prefill_attn_kernel), smem); e != hipSuccess)
    return e;
  const int nqb = (a.n_tokens + kRowsPerWG - 1) / kRowsPerWG;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(unsigned(kH * nqb)), dim3(kNT), smem, st, a);
  return hipGetLastError();
}

}  // namespace mla
