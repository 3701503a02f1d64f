// Split-KV MLA decode on gfx950 matrix cores, DeepSeek-V3 dims:
// H = 128 heads, d_c = 512, d_R = 64 (row D = 576), 64-token cache blocks,
// bf16 queries and cache, fp32 accumulation.
//
// What it computes ("DeepSeek MLA Architecture: How Multi-Head Latent
// Attention Cuts KV Cache by 93%", Core Mechanics 3 and its single-token
// decoding section): for every head i,
// s_t = scale * ([q~_i ; q^R_i] . [c_t ; k^R_t]), p = softmax(s),
// u_i = sum_t p_t c_t -- here per piece of a partition of the cache blocks,
// written as (normalised u, log-sum-exp) partials.
//
// Design (one workgroup of 4 waves per (partition, query token)):
//  * All 128 heads share the cache.  The kernel walks the piece in steps of
//    32 tokens (half a cache block, 36 KB); each step moves HBM -> LDS once
//    with direct-to-LDS 16-byte buffer loads and every wave reads it for its
//    own 32 heads, so each cache byte crosses HBM once.
//  * Software pipeline over four LDS step buffers: iteration h computes the
//    scores of step h, then the output update of step h-1 with the softmax of
//    step h interleaved between those MFMAs (the VALU work runs under matrix
//    work), while steps h+1 and h+2 are in flight.
//  * Scores as S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: the K fragment (32
//    tokens x 16 channels) comes from LDS as one ds_read_b128 per lane, Q^T
//    (16 channels x 32 heads) stays in registers for the whole piece.  In the
//    S^T accumulator a lane owns one head and 16 of the 32 tokens, so the
//    softmax row max is an in-lane reduction plus one exchange with lane^32,
//    and the accumulator already has the layout of the P operand of P.V (the
//    token order inside each K=16 step is a permutation mirrored on V).
//  * O^T[channel][head] += V^T . P^T with the V^T fragment read from the same
//    token-major step by ds_read_b64_tr_b16 (each 16-lane group turns a
//    4-token x 16-channel block into per-lane columns).  O^T lives in the
//    AGPRs (256 per lane) and keeps one head per lane, so the epilogue needs
//    no cross-lane traffic.
//  * Softmax in log2 units against a per-head reference m_ref taken from the
//    head's first step: p = 2^(s' - m_ref).  While later scores stay below
//    m_ref + kHeadroom (32), p <= 2^32 and nothing can overflow in fp32 or
//    bf16, so O is only ever touched by MFMA.  A head that exceeds it moves
//    its reference to the new maximum and its wave rescales O and the running
//    sum by 2^(old - new) (the exact online-softmax update; it does not
//    happen for ordinary logits).
//  * Masked (past-length) tokens: their score is -inf, and their rows lie
//    outside the load's buffer range, which fills them with zeros, so
//    0 * (stale value / NaN) never reaches the accumulators.
//  * LDS step layout: 8-token x 8-chunk sub-blocks (one 1 KB direct load
//    each), 16-byte chunks XOR-swizzled by token so both the b128 K reads and
//    the transposed V reads spread over all banks.
//  * The partial is transposed through LDS in the epilogue and written with
//    whole-row non-temporal stores.  The partition that owns a sequence's
//    first cache block also records the sequence's first slot and piece count
//    in the workspace, where the combine kernels read them.
//  * Before the plan, the workgroup already streams the Q of the sequence its
//    first piece would belong to with equal lengths; the plan reads the
//    lengths from an LDS window loaded ahead of that Q.
//  * fp8 cache (kF8): each step's e4m3 codes and per-(token, 128-channel)
//    scales land in a staging buffer and the workgroup dequantises them (code
//    x scale in fp32, one bf16 rounding) into a bf16 step buffer one
//    iteration ahead of use; from there the step is read as above.
#include <utility>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kH = 128, kDC = 512, kDR = 64, kD = kDC + kDR, kBS = 64;
constexpr int kNT = 256;                      // 4 waves x 32 heads
constexpr int kStep = 32;                     // tokens per step
constexpr int kRowBytes = kD * 2;             // 1152
constexpr int kBlockBytes = kBS * kRowBytes;  // 73728
constexpr int kStepBytes = kStep * kRowBytes; // 36864 = 36 sub-blocks of 1 KB
constexpr int kNBuf = 4;                      // bf16 cache: LDS step buffers h-1 (PV), h (QK), h+1, h+2 in flight
// fp8 cache: three bf16 step buffers (h-1, h, h+1 being converted) and two
// staging buffers for the e4m3 codes (18 KB) and scales (640 B, one 1 KB load)
constexpr int kF8NBuf = 3;
constexpr int kF8Codes = kStep * kD;                 // 18432
constexpr int kF8ScaleBytes = kStep * 5 * 4;         // 640
constexpr int kF8Stage = kF8Codes + 1024;            // 19456
constexpr int kF8Loads = kF8Codes / 1024;            // 18 direct loads of codes per step
constexpr int kLdsBytes = (kNBuf * kStepBytes > kF8NBuf * kStepBytes + 2 * kF8Stage)
                              ? kNBuf * kStepBytes : kF8NBuf * kStepBytes + 2 * kF8Stage;
constexpr int kLoadsPerWave = 9;              // 1 KB direct loads per wave per step
constexpr float kHeadroom = 32.0f;            // log2 headroom above the reference max
constexpr int kStageRow = kDC * 2 + 16;       // epilogue transpose row (padded against bank conflicts)
constexpr int kQK = kD / 16;                  // score MFMAs per step
constexpr int kPV = 2 * (kDC / 32);           // output MFMAs per step
constexpr int kRK = 4, kRV = 4;               // LDS operand fragments read ahead of their MFMA
static_assert(4 * 32 * kStageRow <= kLdsBytes, "epilogue stage must fit the step buffers");
static_assert(kF8NBuf * kStepBytes + 2 * kF8Stage <= kLdsBytes && kF8ScaleBytes <= 1024, "fp8 staging layout");
static_assert(kNT / kWave == kNBuf && kH * kRowBytes <= kLdsBytes, "Q is staged through the step buffers");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef const __attribute__((address_space(4))) int32_t const_i32;

// 16-byte-chunk swizzle: chunk slot (c & 7) ^ swz(t) within token t's sub-row.
MLA_DEV int swz(int t) { return ((((t & 3) << 1) | ((t >> 2) & 1)) ^ ((t >> 2) & 2)) & 7; }

// Byte offset of chunk c (0..71) of token t (0..31) inside a step buffer.
MLA_DEV int step_off(int t, int c) {
  return (((t >> 3) * 9 + (c >> 3)) * 64 + (t & 7) * 8 + ((c & 7) ^ swz(t))) * 16;
}

struct Smem {
  // bf16 step buffer i at i * kStepBytes (kStepBytes is a multiple of 128);
  // for the fp8 cache, staging buffer i follows the three step buffers
  alignas(128) unsigned char lds[kLdsBytes];
  PlanScratch<kNT> plan;
  alignas(16) int32_t lens[256];  // window of sequence lengths for the plan
};

// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
MLA_DEV void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Workgroup barrier for the step loop.  __syncthreads() carries a workgroup
// fence, which makes the compiler wait for *all* outstanding vector-memory
// operations -- including the prefetches of later steps.  The step loop needs
// less: its own LDS traffic complete (lgkmcnt) and the explicit vmcnt wait for
// the current step that precedes each call.  The memory clobber keeps memory
// accesses from moving across it.
MLA_DEV void step_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Per-lane byte offset (inside its 8-token group) of the chunk it loads;
// the group parity p selects the swizzle variant.
MLA_DEV int load_lane_off(int lane, int p) {
  const int t = 8 * p + lane / 8;
  return (lane / 8) * kRowBytes + ((lane & 7) ^ swz(t)) * 16;
}

// This wave's 9 direct HBM->LDS loads of one step: token group `wave`
// (8 tokens) x 9 column groups.  The descriptor covers only the live rows, so
// lanes past `nvalid` read out of range, which writes zeros into LDS.
// The loads are issued from inline asm on purpose: the compiler cannot tell
// that the LDS reads of the current step never touch the buffers these loads
// fill, and would otherwise wait for *every* pending load (vmcnt(0)) before
// each of them.  The step loop waits for exactly the loads it needs (wait_vm).
// No register is written by these instructions (the data goes to LDS).  The
// column offset goes into soffset: an immediate offset would also shift the
// LDS destination.
template <int M>
MLA_DEV void load_one(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int wave, int loff) {
  const int k = wave * kLoadsPerWave + M;  // sub-block (token group `wave`, column group M)
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) unsigned char*)(dst + k * 1024)));
  // s_nop: one wait state between the M0 write and its use by the LDS DMA
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(loff), "s"(r), "s"(wave * 9216 + M * 128), "{m0}"(lds)
               : "memory");
}
template <int... Ms>
MLA_DEV void load_all(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int wave, int loff,
                      std::integer_sequence<int, Ms...>) {
  (load_one<Ms>(r, dst, wave, loff), ...);
}
MLA_DEV void load_step(unsigned char* dst, const unsigned char* src, int nvalid, int wave, int loff) {
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nvalid * kRowBytes, 0x00020000);
  load_all(r, dst, wave, loff, std::make_integer_sequence<int, kLoadsPerWave>{});
}

// One fp8 step into a staging buffer: the 32 rows of e4m3 codes are one
// contiguous 18 KB run (18 direct 1 KB loads, dealt round-robin to the waves)
// and their 32 x 5 fp32 scales one more load (wave 3, which has one code load
// fewer).  The codes' descriptor covers only the live rows, so the rest reads
// zeros; the scales are read whole (640 bytes, inside the block) and those of
// rows past the length are dropped by the conversion.
MLA_DEV void load_step_f8(unsigned char* dst, const unsigned char* codes, const float* scales,
                          int nvalid, int wave, int lane) {
  const __amdgpu_buffer_rsrc_t rc =
      __builtin_amdgcn_make_buffer_rsrc((void*)codes, (short)0, nvalid * kD, 0x00020000);
  for (int k = wave; k < kF8Loads; k += kNT / kWave) {
    const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)(dst + k * 1024)));
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(lane * 16), "s"(rc), "s"(k * 1024), "{m0}"(lds)
                 : "memory");
  }
  if (wave == kNT / kWave - 1) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)scales, (short)0, kF8ScaleBytes, 0x00020000);
    const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)(dst + kF8Codes)));
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(lane * 16), "s"(rs), "{m0}"(lds)
                 : "memory");
  }
}

typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
MLA_DEV uint32_t lds_addr(const unsigned char* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_u8*)p));
}
MLA_DEV bf16x8 lds_b128_at(uint32_t addr) { return *(lds_bf16x8*)(uintptr_t)addr; }

// Dequantise a staged fp8 step into a bf16 step buffer (the cache-step
// layout): value = e4m3 code (decoded exactly) * its (token, 128-channel tile)
// scale in fp32, rounded once to bf16.  Unit u = 16 codes of one token.
// Rows at or past `nvalid` have zero codes; their scale is replaced by 0 so
// whatever the cache holds there (NaN included) yields exact zeros.
MLA_DEV void convert_step_f8(unsigned char* dst, const unsigned char* stage, int nvalid) {
  typedef __attribute__((address_space(3))) const u32x4 lds_u4;
  typedef __attribute__((address_space(3))) u32x4 lds_u4w;
  typedef __attribute__((address_space(3))) const float lds_f32;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const uint32_t sb = lds_addr(stage), db = lds_addr(dst);
#pragma unroll 1
  for (int u = tid_fresh(); u < kStep * (kD / 16); u += kNT) {
    const int t = u / (kD / 16), c8 = u % (kD / 16);
    const u32x4 cw = *(lds_u4*)(uintptr_t)(sb + t * kD + c8 * 16);
    const float sc_raw = *(lds_f32*)(uintptr_t)(sb + kF8Codes + (t * 5 + c8 / 8) * 4);
    const float sc = t < nvalid ? sc_raw : 0.f;
    const uint32_t w[4] = {cw[0], cw[1], cw[2], cw[3]};
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[e]), false);  // codes 4e, 4e+1
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[e]), true);   // codes 4e+2, 4e+3
      o[2 * e] = pack_bf16x2(lo[0] * sc, lo[1] * sc);
      o[2 * e + 1] = pack_bf16x2(hi[0] * sc, hi[1] * sc);
    }
    *(lds_u4w*)(uintptr_t)(db + step_off(t, 2 * c8)) = u32x4{o[0], o[1], o[2], o[3]};
    *(lds_u4w*)(uintptr_t)(db + step_off(t, 2 * c8 + 1)) = u32x4{o[4], o[5], o[6], o[7]};
  }
}

MLA_DEV bf16x8 lds_tr_pair_at(uint32_t p0, uint32_t p1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p0);
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p1);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Score MFMAs are written as inline asm with the accumulator constrained to
// arch VGPRs: O needs the whole AGPR file, and the compiler would otherwise
// place the scores in AGPRs and shuttle O blocks through VGPRs every step.
// Hazards the compiler cannot see are handled explicitly: the chain starts
// from a literal-zero accumulator (no VALU->MFMA dependency), and
// scores_ready() puts 24 wait states (more than the longest
// MFMA-write -> VALU-read requirement) between the last write and the softmax.
MLA_DEV void mfma_qk_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
MLA_DEV void mfma_qk(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
MLA_DEV void scores_ready(f32x16& s) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s)); }
// Output MFMAs with the accumulator pinned to AGPRs: left to itself the
// register allocator keeps some O blocks in VGPRs and copies them into AGPRs
// around every MFMA, which pushes Q out of registers.  Consecutive updates of
// one accumulator are exactly overlapping (hardware forwards them); the only
// other readers and writers of O (zeroing, epilogue) sit behind o_ready().
MLA_DEV void mfma_pv(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// O = 0 straight into the AGPRs (an MFMA on zero operands with a zero
// accumulator); volatile, so it is not hoisted out of the piece loop as a
// constant that then has to be kept (or spilled) across it.  The zero
// operand is written by VALU moves just before: an MFMA reading a VGPR that
// a VALU instruction wrote needs two wait states in between, which the
// compiler does not insert for inline asm -- hence the s_nop.
MLA_DEV void zero_acc(f32x16& acc, const bf16x8& z) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
}
MLA_DEV void o_ready(f32x16 (&O)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]), "+a"(O[4]), "+a"(O[5]),
                 "+a"(O[6]), "+a"(O[7]), "+a"(O[8]), "+a"(O[9]), "+a"(O[10]), "+a"(O[11]),
                 "+a"(O[12]), "+a"(O[13]), "+a"(O[14]), "+a"(O[15]));
}

template <bool kF8>
__global__ __launch_bounds__(kNT, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(128))) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  constexpr int NB = kF8 ? kF8NBuf : kNBuf;  // bf16 step buffers in the ring
  auto bbuf = [&](int i) __attribute__((always_inline)) { return sm.lds + i * kStepBytes; };
  auto stage_buf = [&](int i) __attribute__((always_inline)) {
    return sm.lds + kF8NBuf * kStepBytes + i * kF8Stage;
  };

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int g = lane / 32;       // lane group: which 8-wide half of a 16-wide k step
  const int hl = lane % 32;      // head within the wave (S^T / O^T column)

  // XCD-aware mapping: consecutive logical ids share an XCD (workgroups are
  // dealt round-robin to the 8 XCDs), so the n_q workgroups of a partition and
  // neighbouring partitions of one sequence share that XCD's L2.
  const int P = gridDim.x, xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int per = P / 8, rem = P % 8;
  const int logical = xcd * per + min(xcd, rem) + idx;
  const int part = logical / a.n_q, j = logical % a.n_q;

  const float c_log2 = a.scale * 1.4426950408889634f;  // scores -> log2 units

  // Per-lane LDS offsets inside a step buffer, one register each; the
  // other fragments follow from the swizzle's structure:
  //  K fragment a (token hl, chunk 2a + g):   koff0 ^ (a << 5)
  //  V fragment (transposed read; token 8*sec + 4*g + s16/4, chunk
  //  4*cbo + 2*h16 + (s16%4)/2, half s16%2):   (voff0 ^ (cbo << 6) ^ (sec << 5)) + sec * 9216
  // (+8 tokens moves one 8-token group down and flips swizzle bit 1).  Step
  // buffers are 128-byte aligned, so the XORs commute with adding the base.
  auto koff0_of = [](int l) __attribute__((always_inline)) { return uint32_t(step_off(l & 31, l >> 5)); };
  auto voff0_of = [](int l) __attribute__((always_inline)) {
    const int gg = l >> 5, hh = (l >> 4) & 1, ss = l & 15;
    return uint32_t(step_off(4 * gg + (ss >> 2), 2 * hh + ((ss & 3) >> 1)) + 8 * (ss & 1));
  };
  // bf16: kept in two registers for the whole kernel.  fp8: recomputed from
  // a fresh lane id at every step -- two registers fewer across the loop,
  // which the dequantisation needs to stay spill-free.
  const uint32_t koff0 = koff0_of(lane), voff0 = voff0_of(lane);
  auto koff0_at = [&]() __attribute__((always_inline)) {
    if constexpr (kF8) return koff0_of(tid_fresh() & (kWave - 1)); else return koff0;
  };
  auto voff0_at = [&]() __attribute__((always_inline)) {
    if constexpr (kF8) return voff0_of(tid_fresh() & (kWave - 1)); else return voff0;
  };
  const int loff = load_lane_off(lane, wave & 1);

  // Speculative Q: with equal lengths, partition `part`'s first piece belongs
  // to sequence part * B / G, so that sequence's Q starts streaming into the
  // step buffers now and the plan is computed while it is in flight.  The
  // plan reads its lengths from an LDS window whose loads wave 0 issues
  // before the Q loads (so waiting for them never waits for Q).  A wrong
  // guess costs only the load: the piece then issues its own, which
  // completes later and overwrites it.
  LdsLensWindow lens{lds_addr(reinterpret_cast<const unsigned char*>(sm.lens)), a.seq_lens, a.batch, 0};
  const int b_pre = int(int64_t(part) * a.batch / a.G);
  auto load_q = [&](int b) __attribute__((always_inline)) {
    const unsigned char* qblk = static_cast<const unsigned char*>(a.q) + (size_t(b) * a.n_q + j) * kH * kRowBytes;
#pragma unroll
    for (int t = 0; t < kNT / kWave; ++t) load_step(bbuf(t), qblk + t * kStepBytes, kStep, wave, loff);
  };
  if (wave == 0) lens_window_issue(lens, 0);
  load_q(b_pre);
  if (wave == 0) wait_vm<kNBuf * kLoadsPerWave>();  // the lengths, not the Q loads behind them
  lds_barrier();
  bool q_pre = true;  // the prefetched Q may still serve the first piece

  int32_t* const tab = j == 0 ? a.ws_tab : nullptr;  // query 0's workgroups record the slot table
  plan_for_each_piece<kNT>(lens, a.batch, kBS, a.G, part, sm.plan,
                           [&](int b_, int ulo_, int uhi_, int slot_, int L_) {
    // piece bounds come from LDS: tell the compiler they are wave-uniform
    const int b = __builtin_amdgcn_readfirstlane(b_), ulo = __builtin_amdgcn_readfirstlane(ulo_);
    const int uhi = __builtin_amdgcn_readfirstlane(uhi_), slot = __builtin_amdgcn_readfirstlane(slot_);
    const int L = __builtin_amdgcn_readfirstlane(L_);
    const int nvis = L - a.n_q + j + 1;               // visible positions 0 .. nvis-1
    const int t_lo = ulo * kBS;
    const int t_hi = min(uhi * kBS, nvis);
    const int nsteps = max(0, (t_hi - t_lo + kStep - 1) / kStep);
    const size_t orow0 = (size_t(slot) * a.n_q + j) * kH + wave * 32;
    if (nsteps == 0) {  // nothing visible to this query in the piece
      const int elane = tid_fresh() % kWave;
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.ws_o) + orow0 * kDC);
      for (int e = elane; e < 32 * kDC / 8; e += kWave) dst[e] = uint4{0u, 0u, 0u, 0u};
      if (elane < 32) a.ws_lse[orow0 + elane] = -INFINITY;
      return;
    }
    // page table through the constant address space: scalar loads
    const_i32* pt = (const_i32*)(uintptr_t)(a.page_table + int64_t(b) * a.max_blocks);
    const unsigned char* cache = static_cast<const unsigned char*>(a.cache);
    auto step_at = [&](int blk, int h) {  // first byte of step h, which lies in block blk
      return cache + int64_t(blk) * kBlockBytes + (h & 1) * kStepBytes;
    };
    // fp8 cache: 1-byte codes, rows of kD bytes; scales [blk][64][5]
    auto load_f8 = [&](int i, int blk, int h, int nvalid) __attribute__((always_inline)) {
      load_step_f8(stage_buf(i), cache + int64_t(blk) * (kBS * kD) + (h & 1) * kF8Codes,
                   a.scales + (int64_t(blk) * kBS + (h & 1) * kStep) * 5, nvalid, wave, lane);
    };
    auto valid_in = [&](int h) { return min(kStep, t_hi - (t_lo + h * kStep)); };
    const int blk0 = pt[ulo];  // steps 0 and 1 lie in the piece's first block

    // Q^T fragments for this wave's 32 heads, resident for the whole piece.
    // The 32 heads' rows of a wave are one contiguous 36 KB block -- a step
    // tile -- so Q is staged through the step buffers with the cache loads'
    // own direct loads and layout (wave t's block into buffer t), and each
    // wave reads its fragments exactly like K fragments: whole-row loads
    // instead of 16-byte pieces of 32 rows per instruction.
    if (!(q_pre && b == b_pre)) load_q(b);
    q_pre = false;
    wait_vm<0>();
    step_barrier();
    bf16x8 qf[kQK];
    {
      // (addresses from a fresh lane id: not kept live across the step loop)
      const int ql = tid_fresh() % kWave;
      const uint32_t qb = lds_addr(bbuf(wave)) + uint32_t(step_off(ql % 32, ql / 32));
#pragma unroll
      for (int s = 0; s < kQK; ++s) qf[s] = lds_b128_at((qb ^ uint32_t((s & 3) << 5)) + uint32_t((s >> 2) * 1024));
    }
    step_barrier();  // every wave holds its Q: the buffers are free for the cache
    if constexpr (kF8)
      load_f8(0, blk0, 0, valid_in(0));
    else
      load_step(bbuf(0), step_at(blk0, 0), valid_in(0), wave, loff);

    f32x16 O[kDC / 32];
    {
      const bf16x8 z = {};
#pragma unroll
      for (int cb = 0; cb < kDC / 32; ++cb) zero_acc(O[cb], z);
    }
    float m_ref = -INFINITY, l_run = 0.f;
    bf16x8 p_prev[2] = {};  // P of the step before the first: zero
    uint32_t p_cur[2][4];   // P of the current step, bf16 pairs

    // One pipeline step.  QK: S^T = K . Q^T for step h (36 MFMAs).  PV: O^T +=
    // V^T . P^T for step h-1 (32 MFMAs), with the softmax of step h spread
    // between them, so the exp/max VALU work runs under matrix work.  The
    // first step has no PV yet; the drain after the last step has no QK.
    auto run_step = [&](auto qk_on, auto pv_on, int h) __attribute__((always_inline)) {
      constexpr bool kQKOn = decltype(qk_on)::value, kPVOn = decltype(pv_on)::value;
      const uint32_t kb = lds_addr(bbuf(h % NB)) + koff0_at();
      const uint32_t vb = lds_addr(bbuf(h > 0 ? (h + NB - 1) % NB : 0)) + voff0_at();
      auto kfrag = [&](int n) __attribute__((always_inline)) {  // chunk pair n&3 of sub-block column n>>2
        return lds_b128_at((kb ^ uint32_t((n & 3) << 5)) + uint32_t((n >> 2) * 1024));
      };
      // output MFMA n updates O block n/2 with token half n%2: the two updates
      // of a block run back to back, so the second takes the first's result
      // from the matrix core instead of re-reading the AGPRs (less register
      // file traffic, which shows up as a higher sustained clock)
      auto vfrag = [&](int n) __attribute__((always_inline)) {
        const int i = n & 1, cb = n >> 1;
        const uint32_t base = uint32_t((2 * i) * 9216 + (cb >> 1) * 1024);  // token rows 16i..16i+15
        const uint32_t v = vb ^ uint32_t((cb & 1) << 6);
        return lds_tr_pair_at(v + base, (v ^ 32u) + base + 9216u);
      };
      f32x16 S;
      bf16x8 vr[kRV];
      if constexpr (kQKOn) {
        bf16x8 kr[kRK];
#pragma unroll
        for (int n = 0; n < kRK; ++n) kr[n] = kfrag(n);
#pragma unroll
        for (int n = 0; n < kQK; ++n) {
          if (n == 0)
            mfma_qk_first(S, kr[0], qf[0]);
          else
            mfma_qk(S, kr[n % kRK], qf[n]);
          if (n + kRK < kQK) {
            kr[n % kRK] = kfrag(n + kRK);
          } else if constexpr (kPVOn) {  // the tail of QK prefetches the first V fragments
            const int v = n + kRK - kQK;
            if (v < kRV) vr[v] = vfrag(v);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int n = 0; n < kRV; ++n) vr[n] = vfrag(n);
      }

      // softmax of step h in pieces (lane = one head; tokens 8*(r/4) + 4*g + r%4)
      const int nv = kQKOn ? valid_in(h) : kStep;
      float mx = 0.f, lsum = 0.f, corr = 1.f;
      bool spike = false;
      auto softmax_part = [&](int k) __attribute__((always_inline)) {
        if constexpr (kQKOn) {
          if (k == 0) scores_ready(S);
          if (k == 1 && nv < kStep) {  // past-length tokens of a partial step: -inf
            const int lim = nv - 4 * ((tid_fresh() % kWave) / 32);
#pragma unroll
            for (int r = 0; r < 16; ++r) S[r] = (8 * (r / 4) + (r % 4) >= lim) ? -INFINITY : S[r];
          }
          if (k == 2) {
            mx = S[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
          }
          if (k == 3) {
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c_log2;
            // the piece's first step sets the head's reference; a later step
            // more than kHeadroom above it moves it (and rescales O below)
            spike = m_ref != -INFINITY && mx > m_ref + kHeadroom;
            const float m_new = m_ref == -INFINITY || spike ? mx : m_ref;
            corr = spike ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
            m_ref = m_new;
          }
          if (k >= 4 && k < 12) {
            const int i = (k - 4) >> 2, e = 2 * ((k - 4) & 3);
            const float p0 = __builtin_amdgcn_exp2f(fmaf(S[8 * i + e], c_log2, -m_ref));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(S[8 * i + e + 1], c_log2, -m_ref));
            lsum += p0;
            lsum += p1;
            p_cur[i][e / 2] = pack_bf16x2(p0, p1);
            // pin the work here, between the output MFMAs: left alone, the
            // compiler sinks it to the end of the step where nothing hides it
            asm volatile("" : "+v"(p_cur[i][e / 2]), "+v"(lsum));
          }
        }
      };

      if constexpr (kPVOn) {
#pragma unroll
        for (int n = 0; n < kPV; ++n) {
          mfma_pv(O[n >> 1], vr[n % kRV], p_prev[n & 1]);
          if (n + kRV < kPV) vr[n % kRV] = vfrag(n + kRV);
          softmax_part(n);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 12; ++k) softmax_part(k);
      }
      if constexpr (kQKOn) {
        if (__any(spike)) {  // rare: rescale this wave's accumulated output
          o_ready(O);
#pragma unroll
          for (int cb = 0; cb < kDC / 32; ++cb) {
            O[cb] *= corr;                        // through VGPRs ...
            asm volatile("" : "+a"(O[cb]));       // ... and back into the AGPRs
          }
        }
        l_run = l_run * corr + lsum;
#pragma unroll
        for (int i = 0; i < 2; ++i)
          p_prev[i] = __builtin_bit_cast(bf16x8, u32x4{p_cur[i][0], p_cur[i][1], p_cur[i][2], p_cur[i][3]});
      }
    };

    // block of the next step to prefetch, looked up one step early
    int blk_nx = nsteps > 2 ? pt[ulo + 1] : 0;
    if constexpr (!kF8) {
      if (nsteps > 1) load_step(bbuf(1), step_at(blk0, 1), valid_in(1), wave, loff);
      // Step h waits until its own loads are done (at most the loads of step
      // h+1, issued one iteration earlier, still pending), then a barrier makes
      // every wave's share visible and frees buffer (h+2)%4 for the next load.
      auto begin_step = [&](int h) __attribute__((always_inline)) {
        if (h + 1 < nsteps)
          wait_vm<kLoadsPerWave>();
        else
          wait_vm<0>();
        step_barrier();
        if (h + 2 < nsteps)
          load_step(bbuf((h + 2) % kNBuf), step_at(blk_nx, h + 2), valid_in(h + 2), wave, loff);
        if (h + 3 < nsteps) blk_nx = pt[ulo + ((h + 3) >> 1)];
      };
      // Step 0 runs the same code with P = 0 against its own (finite, zero-filled
      // past the length) buffer: a second specialisation without PV costs the
      // register allocator more than these 32 MFMAs cost the piece.
      for (int h = 0; h < nsteps; ++h) {
        begin_step(h);
        run_step(std::true_type{}, std::true_type{}, h);
      }
    } else {
      // fp8: step h's codes land in staging buffer h%2 and are dequantised
      // into bf16 step buffer h%3 at the end of iteration h-1, which then
      // needs one more barrier.  That leaves the load of step h+2 (issued at
      // the top of iteration h) two iterations to arrive.  A wave issues 4 or
      // 5 loads per step, so vmcnt(4) means "every earlier step has landed".
      if (nsteps > 1) load_f8(1, blk0, 1, valid_in(1));
      if (nsteps > 1)
        wait_vm<4>();
      else
        wait_vm<0>();
      step_barrier();
      convert_step_f8(bbuf(0), stage_buf(0), valid_in(0));
      for (int h = 0; h < nsteps; ++h) {
        step_barrier();  // step h converted; staging buffer h%2 free again
        if (h + 2 < nsteps) load_f8(h & 1, blk_nx, h + 2, valid_in(h + 2));
        if (h + 3 < nsteps) blk_nx = pt[ulo + ((h + 3) >> 1)];
        run_step(std::true_type{}, std::true_type{}, h);
        if (h + 1 < nsteps) {
          if (h + 2 < nsteps)
            wait_vm<4>();
          else
            wait_vm<0>();
          step_barrier();
          convert_step_f8(bbuf((h + 1) % kF8NBuf), stage_buf((h + 1) & 1), valid_in(h + 1));
        }
      }
    }
    run_step(std::false_type{}, std::true_type{}, nsteps);  // PV of the last step
    o_ready(O);
    __syncthreads();  // buffers are reused by the epilogue stage

    // ---- epilogue: normalise and write the partial (bf16) ----
    // lane (g, hl) holds O^T rows = channels 32*cb + 8*rg + 4*g + {0..3} of
    // head hl.  The wave first transposes its 32 x 512 block through the (now
    // idle) step buffers, so that each global store covers one whole 1 KB head
    // row; the stores are non-temporal.  Scattered or ordinary stores issued
    // right after a piece has streamed through L2 run at a fraction of the
    // write bandwidth, and nothing rereads the partials soon.
    // lane-derived values are recomputed here rather than kept across the loop
    const int elane = tid_fresh() % kWave, eg = elane / 32, ehl = elane % 32;
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.f / l_tot;
    if (elane < 32) a.ws_lse[orow0 + elane] = (m_ref + log2f(l_tot)) * 0.6931471805599453f;
    unsigned char* stage = sm.lds + wave * (32 * kStageRow);
#pragma unroll
    for (int cb = 0; cb < kDC / 32; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint32_t lo = pack_bf16x2(O[cb][4 * rg + 0] * inv, O[cb][4 * rg + 1] * inv);
        const uint32_t hi = pack_bf16x2(O[cb][4 * rg + 2] * inv, O[cb][4 * rg + 3] * inv);
        *reinterpret_cast<uint2*>(stage + ehl * kStageRow + (32 * cb + 8 * rg + 4 * eg) * 2) = uint2{lo, hi};
      }
    // the wave reads back only what it wrote itself: LDS order within a wave suffices
    u32x4* orow = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(a.ws_o) + orow0 * kDC) + elane;
#pragma unroll 8
    for (int r = 0; r < 32; ++r)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(stage + r * kStageRow + elane * 16),
                                  orow + r * (kDC / 8));
    step_barrier();  // every wave is done with the stage before a next piece loads into it
  }, tab);
  wait_vm<0>();  // a prefetched Q no piece used must land before the workgroup's LDS is released
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs& a) {
  const bool cache_ok =
      a.cache_dtype == MLA_BF16 ||
      (a.cache_dtype == MLA_FP8_E4M3 && a.scales != nullptr && (reinterpret_cast<uintptr_t>(a.scales) % 16) == 0);
  return a.H == kH && a.d_latent == kDC && a.D == kD && a.block_size == kBS && a.act_dtype == MLA_BF16 &&
         cache_ok && (reinterpret_cast<uintptr_t>(a.cache) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.q) % 16) == 0;
}

template <bool kF8>
hipError_t launch_decode_mfma_t(const DecodeArgs& a, hipStream_t st) {
  const size_t smem = sizeof(Smem);
  if (hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(decode_mfma_kernel<kF8>), int(smem));
      e != hipSuccess)
    return e;
  dim3 grid(unsigned(a.G) * unsigned(a.n_q));
  hipLaunchKernelGGL(decode_mfma_kernel<kF8>, grid, dim3(kNT), smem, st, a);
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  return a.cache_dtype == MLA_FP8_E4M3 ? launch_decode_mfma_t<true>(a, st) : launch_decode_mfma_t<false>(a, st);
}

}  // namespace mla
