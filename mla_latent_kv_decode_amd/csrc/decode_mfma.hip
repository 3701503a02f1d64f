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
//    head's first step: p = 2^(s' - m_ref).  While a lane's 16 values of a
//    step sum to at most 2^32, nothing can overflow in fp32 or bf16, so O is
//    only ever touched by MFMA and no per-step maximum is needed.  A step
//    whose sum exceeds that is redone against its maximum, and the wave
//    rescales O and the running sum by 2^(old - new) (the exact online-softmax
//    update; it does not happen for ordinary logits).
//  * Instruction issue, not the matrix cores or LDS, bounds the step loop (one
//    wave per SIMD issues in order and nothing hides its stalls): the loop
//    keeps per-step scalar and VALU work, branches and full waits small.
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
//  * e4m3 cache with tile scales of any value (mode 1): each step's codes
//    and per-(token, 128-channel) scales land in a staging buffer and the
//    workgroup dequantises them (code x scale in fp32, one bf16 rounding)
//    into a bf16 step buffer one iteration ahead of use; from there the step
//    is read as above.
//  * e4m3 cache with power-of-two tile scales (mode 2): the scores run on
//    v_mfma_scale_f32_32x32x64_f8f6f4 straight from the staged codes.  The
//    MFMA applies each token's tile scale (its exponent byte, per A row) and
//    Q is e4m3 under one power-of-two scale per head, folded into the
//    softmax's log2 factor; both operands are exact, so only Q's rounding to
//    e4m3 differs from the bf16 path.  V = code x 2^E is exact in bf16: the
//    workgroup converts each step's latent codes with the scaled conversion
//    instruction (two values per instruction) into a bf16 V buffer during
//    the step's own output MFMAs, and the next step's barrier publishes it;
//    the output product is the bf16 one above.  Half the score-side MFMA
//    cycles and LDS bytes of the bf16 path, and no conversion pass of its own.
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
// A lane's 16 probabilities of a step summing past this (2^32) left the
// headroom above the reference: the step is recomputed against its maximum.
constexpr float kPSumLimit = 4294967296.0f;
constexpr int kStageRow = kDC * 2 + 16;       // epilogue transpose row (padded against bank conflicts)
constexpr int kQK = kD / 16;                  // score MFMAs per step
constexpr int kPV = 2 * (kDC / 32);           // output MFMAs per step
constexpr int kRK = 4, kRV = 4;               // LDS operand fragments read ahead of their MFMA
// e4m3 with power-of-two scales: two bf16 V buffers (8 column groups of 1 KB
// per 8-token group: the latent part only) and three code staging buffers
// (steps h, h+1, h+2): codes as 9 regions of 2 KB, region n the 32 x 64-byte
// A tile of score MFMA n, then the 1 KB scale load.
constexpr int kVBytes = kStep * kDC * 2;                 // 32768
constexpr int kF8Q = kD / 64;                            // fp8 score MFMAs per step (K = 64)
constexpr int kP2Loads = kF8Loads + 1;                   // 18 code loads + 1 scale load per step
constexpr int kP2LdsEnd = 2 * kVBytes + 3 * kF8Stage;    // 123904
static_assert(4 * 32 * kStageRow <= kLdsBytes, "epilogue stage must fit the step buffers");
static_assert(kF8NBuf * kStepBytes + 2 * kF8Stage <= kLdsBytes && kF8ScaleBytes <= 1024, "fp8 staging layout");
static_assert(kNT / kWave == kNBuf && kH * kRowBytes <= kLdsBytes, "Q is staged through the step buffers");
static_assert(kP2LdsEnd <= kLdsBytes && kP2Loads <= 5 * (kNT / kWave), "power-of-two fp8 layout");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16-byte-chunk swizzle: chunk slot (c & 7) ^ swz(t) within token t's sub-row.
MLA_DEV int swz(int t) { return ((((t & 3) << 1) | ((t >> 2) & 1)) ^ ((t >> 2) & 2)) & 7; }

// Byte offset of chunk c (0..71) of token t (0..31) inside a step buffer.
MLA_DEV int step_off(int t, int c) {
  return (((t >> 3) * 9 + (c >> 3)) * 64 + (t & 7) * 8 + ((c & 7) ^ swz(t))) * 16;
}

// Byte offset of bf16 chunk c (0..63) of token t in a latent-only V buffer
// (the step layout with 8 column groups instead of 9).
MLA_DEV int v8_off(int t, int c) {
  return (((t >> 3) * 8 + (c >> 3)) * 64 + (t & 7) * 8 + ((c & 7) ^ swz(t))) * 16;
}
// Code staging of a power-of-two fp8 step: 16-byte chunk c (0..3) of token t
// in region n sits in slot c ^ cswz(t) of the token's 64-byte row, so that 16
// consecutive tokens read at one chunk index cover all banks.
MLA_DEV int cswz(int t) { return (t >> 2) & 3; }

constexpr int kPtab = 1024;  // page-table entries of a piece staged in LDS at a time

struct Smem {
  // bf16 step buffer i at i * kStepBytes (kStepBytes is a multiple of 128);
  // for the fp8 cache, staging buffer i follows the three step buffers
  alignas(128) unsigned char lds[kLdsBytes];
  PlanScratch<kNT> plan;
  alignas(16) int32_t lens[256];  // window of sequence lengths for the plan
  // The piece's physical block ids, blocks [pbase, pbase + kPtab): the step
  // loop reads them from here instead of issuing scalar loads.  A scalar load
  // in flight completes out of order, so every wait for an LDS operand behind
  // it would have to wait for it too (lgkmcnt(0)) -- once per step.
  alignas(16) int32_t ptab[kPtab];
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
// LDS destination.  Every cache-stream load (here and in the fp8 loaders
// below) is non-temporal (`nt`): a step's rows are read once, and streaming
// them through the caches leaves the partials, Q and W^UV that the step's
// other kernels re-read in place (the v3 step measured 2-3% faster).
template <int M>
MLA_DEV void load_one(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int wave, int loff) {
  const int k = wave * kLoadsPerWave + M;  // sub-block (token group `wave`, column group M)
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) unsigned char*)(dst + k * 1024)));
  // (MLA_ASM_VMEM_WAIT: the hazards an asm load must cover itself)
  asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, %2 offen nt lds"
               :
               : "v"(loff), "s"(r), "s"(wave * 9216 + M * 128), "{m0}"(lds)
               : "memory");
}
// Load m (0..8) of this wave's share of a step (runtime m, same as load_one<m>).
MLA_DEV void load_piece(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int wave, int loff, int m) {
  const int k = wave * kLoadsPerWave + m;
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) unsigned char*)(dst + k * 1024)));
  asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, %2 offen nt lds"
               :
               : "v"(loff), "s"(r), "s"(wave * 9216 + m * 128), "{m0}"(lds)
               : "memory");
}
template <int... Ms>
MLA_DEV void load_all(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int wave, int loff,
                      std::integer_sequence<int, Ms...>) {
  (load_one<Ms>(r, dst, wave, loff), ...);
}
// Descriptor of one step's rows in the cache: only the live rows are in range.
MLA_DEV __amdgpu_buffer_rsrc_t step_rsrc(const unsigned char* src, int nvalid) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nvalid * kRowBytes, 0x00020000);
}
MLA_DEV void load_step(unsigned char* dst, const unsigned char* src, int nvalid, int wave, int loff) {
  load_all(step_rsrc(src, nvalid), dst, wave, loff, std::make_integer_sequence<int, kLoadsPerWave>{});
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
    asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :
                 : "v"(lane * 16), "s"(rc), "s"(k * 1024), "{m0}"(lds)
                 : "memory");
  }
  if (wave == kNT / kWave - 1) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)scales, (short)0, kF8ScaleBytes, 0x00020000);
    const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)(dst + kF8Codes)));
    asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(lane * 16), "s"(rs), "{m0}"(lds)
                 : "memory");
  }
}

// Load m (0..4) of this wave's share of a power-of-two fp8 step: code load
// k = wave + 4m (region k / 2, token half k % 2 = wave % 2) or, for k = 18,
// the 640 bytes of scales; wave 3 has four loads.  Lane i of a code load
// fills slot i % 4 of token 16 * (k % 2) + i / 4 (voff: that token's source
// chunk, wave-fixed); the region's column offset goes into soffset.
MLA_DEV void load_piece_p2(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, unsigned char* dst,
                           int wave, int voff, int lane, int m) {
  const int k = wave + 4 * m;
  if (m < 4 || wave < 2) {  // k < 18: a code load
    const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)(dst + k * 1024)));
    asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :
                 : "v"(voff), "s"(rc), "s"((k >> 1) * 64), "{m0}"(lds)
                 : "memory");
  } else if (wave == 2) {  // k == 18: the scales
    const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) unsigned char*)(dst + kF8Codes)));
    asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, 0 offen nt lds"
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
  constexpr int kUnits = kStep * (kD / 16);  // 1152 units of 16 codes: token u / 36, chunk u % 36
  static_assert(kUnits > 4 * kNT && kUnits <= 5 * kNT && (kUnits - 4 * kNT) % kWave == 0 && kNT == 7 * 36 + 4,
                "units tid + 256 i: four for every thread, a fifth for whole waves; 256 = 7 x 36 + 4");
  const uint32_t sb = lds_addr(stage), db = lds_addr(dst);
  const int tid = tid_fresh();
  const int t0 = tid / 36, c0 = tid % 36;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    if (i == 4 && tid >= kUnits - 4 * kNT) break;  // (wave-uniform)
    // unit u = tid + 256 i: its codes are the contiguous 16 bytes at u * 16
    // of the staged step; its token and chunk follow from (t0, c0)
    const int cw = c0 + 4 * i, carry = cw >= 36;
    const int c8 = cw - 36 * carry, t = t0 + 7 * i + carry;
    const u32x4 cwv = *(lds_u4*)(uintptr_t)(sb + uint32_t(tid * 16 + i * kNT * 16));
    const float sc_raw = *(lds_f32*)(uintptr_t)(sb + uint32_t(kF8Codes + (t * 5 + c8 / 8) * 4));
    const float sc = t < nvalid ? sc_raw : 0.f;
    const uint32_t w[4] = {cwv[0], cwv[1], cwv[2], cwv[3]};
    uint32_t o[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[e]), false);  // codes 4e, 4e+1
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[e]), true);   // codes 4e+2, 4e+3
      o[2 * e] = pack_bf16x2(lo[0] * sc, lo[1] * sc);
      o[2 * e + 1] = pack_bf16x2(hi[0] * sc, hi[1] * sc);
    }
    // bf16 chunks 2 c8 and 2 c8 + 1 of token t: the same 128-byte row, slots
    // differing in their lowest bit
    const uint32_t d0 = db + uint32_t(step_off(t, 2 * c8));
    *(lds_u4w*)(uintptr_t)d0 = u32x4{o[0], o[1], o[2], o[3]};
    *(lds_u4w*)(uintptr_t)(d0 ^ 16u) = u32x4{o[4], o[5], o[6], o[7]};
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
// fp8 score MFMA with the A rows' scales taken from byte J of `sa` (E8M0:
// 2^(byte - 127)) and unit B scales (byte 127 of `sb`).  The scale registers
// are written by VALU code ahead of the chain; scales_ready() puts three wait
// states between those writes and the first MFMA that reads them.
template <int J>
MLA_DEV void mfma_qk8(f32x16& acc, const i32x8& a, const i32x8& b, uint32_t sa, uint32_t sb) {
  if constexpr (J == 0)
    asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
        : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  else if constexpr (J == 1)
    asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,0,0] op_sel_hi:[0,0,0]"
        : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  else if constexpr (J == 2)
    asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[1,0,0]"
        : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
  else
    asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "+v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
MLA_DEV void mfma_qk8_first(f32x16& acc, const i32x8& a, const i32x8& b, uint32_t sa, uint32_t sb) {
  asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
      : "=&v"(acc) : "v"(a), "v"(b), "v"(sa), "v"(sb));
}
MLA_DEV void scales_ready(uint32_t& a, uint32_t& b, uint32_t& c) {
  asm volatile("s_nop 2" : "+v"(a), "+v"(b), "+v"(c));
}
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

// kMode: 0 bf16 cache, 1 e4m3 cache with any tile scales, 2 e4m3 cache with
// power-of-two tile scales.
template <int kMode>
__global__ __launch_bounds__(kNT, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(DecodeArgs a) {
  constexpr bool kF8 = kMode == 1, kP2 = kMode == 2;
  extern __shared__ __attribute__((aligned(128))) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  constexpr int NB = kF8 ? kF8NBuf : kNBuf;  // bf16 step buffers in the ring
  constexpr int kTG = kP2 ? 8 * 1024 : 9 * 1024;  // V: bytes per 8-token group
  auto bbuf = [&](int i) __attribute__((always_inline)) { return sm.lds + i * kStepBytes; };
  auto stage_buf = [&](int i) __attribute__((always_inline)) {
    return sm.lds + kF8NBuf * kStepBytes + i * kF8Stage;
  };
  auto vbuf = [&](int i) __attribute__((always_inline)) { return sm.lds + i * kVBytes; };      // mode 2
  auto cbuf = [&](int i) __attribute__((always_inline)) { return sm.lds + 2 * kVBytes + i * kF8Stage; };

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  // Notation below: lane (g, hl) with g = lane / 32 (which 8-wide half of a
  // 16-wide k step) and hl = lane % 32 (the head within the wave: the S^T /
  // O^T column).

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
  // (mode 2's V offsets, from a 64-byte-row layout; recomputed from a fresh
  // lane id at every step: no register across the loop)
  auto voff0_of8 = [](int l) __attribute__((always_inline)) {
    const int gg = l >> 5, hh = (l >> 4) & 1, ss = l & 15;
    return uint32_t(v8_off(4 * gg + (ss >> 2), 2 * hh + ((ss & 3) >> 1)) + 8 * (ss & 1));
  };
  // mode 2: the score A fragment of lane (g, hl) is chunks 2g, 2g+1 of token
  // hl's 64-byte row of a region (the second at XOR 16).  Recomputed from a
  // fresh lane id where used, like the V offsets: no register across the loop.
  auto koff8_of = [](int l) __attribute__((always_inline)) {
    const int t = l & 31;
    return uint32_t(t * 64 + (((2 * (l >> 5)) ^ cswz(t)) << 4));
  };
  const uint32_t koff0 = koff0_of(lane), voff0 = voff0_of(lane);
  // kept in two registers across the step loop (the bf16 and the any-scale
  // loops; recomputing them from a fresh lane id each step costs the
  // instruction-bound loop more than the two registers)
  auto koff0_at = [&]() __attribute__((always_inline)) { return koff0; };
  auto voff0_at = [&]() __attribute__((always_inline)) { return voff0; };
  const int loff = load_lane_off(lane, wave & 1);
  // mode 2: this lane's source chunk in its code loads (token 16 (wave % 2) +
  // lane / 4); from the plain lane id, so the compiler keeps it across the
  // step loop instead of recomputing it for each of a step's loads
  auto loff8_at = [&]() __attribute__((always_inline)) {
    const int t = 16 * (wave & 1) + lane / 4;
    return t * kD + (((lane & 3) ^ cswz(t)) << 4);
  };

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
    // the piece's row of the page table (vector loads into sm.ptab)
    const int32_t* pt = a.page_table + int64_t(b) * a.max_blocks + ulo;
    const int nblk_need = (nsteps + 1) >> 1;  // blocks holding the piece's visible steps
    auto fill_ptab = [&](int base) __attribute__((always_inline)) {
      const int n = min(kPtab, nblk_need - base);
      for (int i = tid_fresh(); i < n; i += kNT) sm.ptab[i] = pt[base + i];
    };
    int pbase = 0;  // first block of the piece held in sm.ptab (wave-uniform)
    auto block_of = [&](int i) __attribute__((always_inline)) {  // physical block of the piece's block i
      return __builtin_amdgcn_readfirstlane(sm.ptab[i - pbase]);
    };
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

    // Q^T fragments for this wave's 32 heads, resident for the whole piece.
    // The 32 heads' rows of a wave are one contiguous 36 KB block -- a step
    // tile -- so Q is staged through the step buffers with the cache loads'
    // own direct loads and layout (wave t's block into buffer t), and each
    // wave reads its fragments exactly like K fragments: whole-row loads
    // instead of 16-byte pieces of 32 rows per instruction.
    if (!(q_pre && b == b_pre)) load_q(b);
    q_pre = false;
    fill_ptab(0);  // in flight together with Q
    wait_vm<0>();
    step_barrier();
    const int blk0 = block_of(0);  // steps 0 and 1 lie in the piece's first block
    bf16x8 qf[kP2 ? 1 : kQK];
    i32x8 qf8[kP2 ? kF8Q : 1];
    float c_l2 = c_log2;  // scores -> log2 units (mode 2: times the head's Q scale)
    if constexpr (!kP2) {
      // (addresses from a fresh lane id: not kept live across the step loop)
      const int ql = tid_fresh() % kWave;
      const uint32_t qb = lds_addr(bbuf(wave)) + uint32_t(step_off(ql % 32, ql / 32));
#pragma unroll
      for (int s = 0; s < kQK; ++s) qf[s] = lds_b128_at((qb ^ uint32_t((s & 3) << 5)) + uint32_t((s >> 2) * 1024));
    } else {
      // Q of head hl in e4m3 under one power-of-two scale 2^E (the smallest
      // with max |q| <= 448 * 2^E): lane (g, hl) holds channels 64 n + 32 g
      // .. + 31 of score MFMA n, which are bf16 chunks 8 n + 4 g + k (k < 4)
      // of the staged row.  Pass 1 takes the head's max |q| (the other half
      // of the row is in lane ^ 32), pass 2 scales and converts.
      const int ql = tid_fresh() % kWave, qg = ql / 32, qh = ql % 32;
      const uint32_t qb = lds_addr(bbuf(wave)) + uint32_t(step_off(qh, 4 * qg));  // chunk 4 qg (+ k: XOR k << 4)
      float amax = 0.f;
      for (int n = 0; n < kF8Q; ++n)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16x8 v = lds_b128_at((qb ^ uint32_t(k << 4)) + uint32_t(n * 1024));
#pragma unroll
          for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(float(v[e])));
        }
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax), false, false);
      amax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      const int qe = amax > 0.f ? pow2_scale_exp(amax) : 0;
      const float down = __builtin_ldexpf(1.0f, -qe);
      c_l2 = __builtin_ldexpf(c_log2, qe);
#pragma unroll
      for (int n = 0; n < kF8Q; ++n)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16x8 v = lds_b128_at((qb ^ uint32_t(k << 4)) + uint32_t(n * 1024));
          int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(float(v[0]) * down, float(v[1]) * down, 0, false);
          w0 = __builtin_amdgcn_cvt_pk_fp8_f32(float(v[2]) * down, float(v[3]) * down, w0, true);
          int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(float(v[4]) * down, float(v[5]) * down, 0, false);
          w1 = __builtin_amdgcn_cvt_pk_fp8_f32(float(v[6]) * down, float(v[7]) * down, w1, true);
          qf8[n][2 * k] = w0;
          qf8[n][2 * k + 1] = w1;
        }
    }
    step_barrier();  // every wave holds its Q: the buffers are free for the cache
    // mode 2: descriptors of step s's codes and scales (empty past the piece:
    // the loads then write zeros into a free buffer)
    auto rsrc_codes = [&](int blk, int s_, bool live) __attribute__((always_inline)) {
      return __builtin_amdgcn_make_buffer_rsrc(
          (void*)(cache + int64_t(blk) * (kBS * kD) + (s_ & 1) * kF8Codes), (short)0, live ? valid_in(s_) * kD : 0,
          0x00020000);
    };
    auto rsrc_scales = [&](int blk, int s_, bool live) __attribute__((always_inline)) {
      return __builtin_amdgcn_make_buffer_rsrc((void*)(a.scales + (int64_t(blk) * kBS + (s_ & 1) * kStep) * 5),
                                               (short)0, live ? kF8ScaleBytes : 0, 0x00020000);
    };
    if constexpr (kF8) {
      load_f8(0, blk0, 0, valid_in(0));
    } else if constexpr (kP2) {
      for (int s_ = 0; s_ < 2; ++s_) {
        const auto rc = rsrc_codes(blk0, s_, s_ < nsteps), rs = rsrc_scales(blk0, s_, s_ < nsteps);
#pragma unroll
        for (int m = 0; m < 5; ++m) load_piece_p2(rc, rs, cbuf(s_), wave, loff8_at(), lane, m);
      }
    } else {
      load_step(bbuf(0), step_at(blk0, 0), valid_in(0), wave, loff);
    }

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
    auto run_step = [&](auto qk_on, auto pv_on, int h, auto&& after_qk_mfma, auto&& after_pv_mfma)
                        __attribute__((always_inline)) {
      constexpr bool kQKOn = decltype(qk_on)::value, kPVOn = decltype(pv_on)::value;
      const uint32_t kb = kP2 ? lds_addr(cbuf(h % 3)) + koff8_of(tid_fresh() % kWave)
                              : lds_addr(bbuf(h % NB)) + koff0_at();
      const uint32_t vb = kP2 ? lds_addr(vbuf((h + 1) & 1)) + voff0_of8(tid_fresh() % kWave)
                              : lds_addr(bbuf(h > 0 ? (h + NB - 1) % NB : 0)) + voff0_at();
      auto kfrag = [&](int n) __attribute__((always_inline)) {  // chunk pair n&3 of sub-block column n>>2
        return lds_b128_at((kb ^ uint32_t((n & 3) << 5)) + uint32_t((n >> 2) * 1024));
      };
      // output MFMA n updates O block n/2 with token half n%2: the two updates
      // of a block run back to back, so the second takes the first's result
      // from the matrix core instead of re-reading the AGPRs (less register
      // file traffic, which shows up as a higher sustained clock)
      auto vfrag = [&](int n) __attribute__((always_inline)) {
        const int i = n & 1, cb = n >> 1;
        const uint32_t base = uint32_t((2 * i) * kTG + (cb >> 1) * 1024);  // token rows 16i..16i+15
        const uint32_t v = vb ^ uint32_t((cb & 1) << 6);
        return lds_tr_pair_at(v + base, (v ^ 32u) + base + uint32_t(kTG));
      };
      f32x16 S;
      bf16x8 vr[kRV];
      // mode 2: this lane's token hl of step h -- its five tile scales give the
      // score MFMAs' A scales (exponent bytes; 127 = 1 past the length) and the
      // V conversion's scales (tiles 0..3 of the same token)
      const int nv = kQKOn ? valid_in(h) : kStep;
      float vsc[4];
      if constexpr (kP2 && kQKOn) {
        typedef __attribute__((address_space(3))) const float lds_f32;
        const int sl = tid_fresh() % 32;
        const uint32_t sbase = lds_addr(cbuf(h % 3)) + uint32_t(kF8Codes + sl * 20);
        const bool live = sl < nv;
        uint32_t sa0 = 0, sa1, sb = 127u;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          const float sc = *(lds_f32*)(uintptr_t)(sbase + 4 * j);
          const uint32_t e = live ? (__float_as_uint(sc) >> 23) & 0xffu : 127u;
          if (j < 4) {
            sa0 |= e << (8 * j);
            vsc[j] = live ? sc : 1.0f;
          } else {
            sa1 = e;
          }
        }
        scales_ready(sa0, sa1, sb);
        auto kfrag8 = [&](int n) __attribute__((always_inline)) {  // A tile of score MFMA n
          const bf16x8 lo = lds_b128_at(kb + uint32_t(n * 2048));
          const bf16x8 hi = lds_b128_at((kb ^ 16u) + uint32_t(n * 2048));
          const u32x4 l4 = __builtin_bit_cast(u32x4, lo), h4 = __builtin_bit_cast(u32x4, hi);
          return i32x8{int(l4[0]), int(l4[1]), int(l4[2]), int(l4[3]), int(h4[0]), int(h4[1]), int(h4[2]), int(h4[3])};
        };
        constexpr int kR8 = 3;
        i32x8 kr[kR8];
#pragma unroll
        for (int n = 0; n < kR8; ++n) {
          kr[n] = kfrag8(n);
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int n = 0; n < kF8Q; ++n) {
          if (n == 0) mfma_qk8_first(S, kr[0], qf8[0], sa0, sb);
          else if (n == 8) mfma_qk8<0>(S, kr[n % kR8], qf8[n], sa1, sb);
          else if (n >> 1 == 0) mfma_qk8<0>(S, kr[n % kR8], qf8[n], sa0, sb);
          else if (n >> 1 == 1) mfma_qk8<1>(S, kr[n % kR8], qf8[n], sa0, sb);
          else if (n >> 1 == 2) mfma_qk8<2>(S, kr[n % kR8], qf8[n], sa0, sb);
          else mfma_qk8<3>(S, kr[n % kR8], qf8[n], sa0, sb);
          if (n + kR8 < kF8Q) {
            kr[n % kR8] = kfrag8(n + kR8);
          } else if constexpr (kPVOn) {
            const int v = n + kR8 - kF8Q;
            if (v < kRV) vr[v] = vfrag(v);
          }
          after_qk_mfma(n);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kPVOn) {
#pragma unroll
          for (int v = kR8; v < kRV; ++v) vr[v] = vfrag(v);
        }
      } else if constexpr (kQKOn) {
        bf16x8 kr[kRK];
#pragma unroll
        for (int n = 0; n < kRK; ++n) {  // in order: the first MFMA waits only for the first read
          kr[n] = kfrag(n);
          __builtin_amdgcn_sched_barrier(0);
        }
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
          after_qk_mfma(n);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int n = 0; n < kRV; ++n) vr[n] = vfrag(n);
      }

      // mode 2: step h's latent codes -> bf16 V buffer h % 2, four 16-code
      // chunks per lane (token hl, chunk 2 wave + g + 8 i of tile i),
      // interleaved with the output MFMAs below
      u32x4 cq;
      // this lane's conversion offsets, once per step (not kept across steps)
      uint32_t cv_rd = 0, cv_wr = 0;
      if constexpr (kP2 && kQKOn) {  // (the step's own codes are converted whenever its scores run)
        const int dl = tid_fresh() % kWave, dg = (2 * wave + dl / 32), dt = dl % 32;
        cv_rd = lds_addr(cbuf(h % 3)) + uint32_t((dg >> 2) * 2048 + dt * 64 + (((dg & 3) ^ cswz(dt)) << 4));
        cv_wr = lds_addr(vbuf(h & 1)) + uint32_t(v8_off(dt, 2 * dg));
      }
      auto v_read = [&](int i) __attribute__((always_inline)) {
        typedef __attribute__((address_space(3))) const u32x4 lds_u4;
        cq = *(lds_u4*)(uintptr_t)(cv_rd + uint32_t(i * 4096));
      };
      auto v_write = [&](int i) __attribute__((always_inline)) {
        typedef __attribute__((address_space(3))) u32x4 lds_u4w;
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        uint32_t o[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(cq[e]), vsc[i], false);
          const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(cq[e]), vsc[i], true);
          o[2 * e] = __builtin_bit_cast(uint32_t, lo);
          o[2 * e + 1] = __builtin_bit_cast(uint32_t, hi);
        }
        const uint32_t addr = cv_wr + uint32_t(i * 2048);
        *(lds_u4w*)(uintptr_t)addr = u32x4{o[0], o[1], o[2], o[3]};
        *(lds_u4w*)(uintptr_t)(addr ^ 16u) = u32x4{o[4], o[5], o[6], o[7]};
      };

      // softmax of step h in pieces (lane = one head; tokens 8*(r/4) + 4*g + r%4):
      // p = 2^(s' - m_ref) against the head's current reference, without
      // first taking the step's maximum.  Whether a p left the headroom is
      // read off the lane's sum of its 16 values afterwards (> 2^32, inf or
      // NaN); that -- and the piece's first step, whose reference is still
      // -inf -- takes the exact path below, which recomputes the step against
      // its maximum.
      float lsum = 0.f, lsum2 = 0.f;
      auto softmax_part = [&](int k) __attribute__((always_inline)) {
        if constexpr (kQKOn) {
          if (k == 0) scores_ready(S);
          if (k == 1 && nv < kStep) {  // past-length tokens of a partial step: -inf
            const int lim = nv - 4 * ((tid_fresh() % kWave) / 32);
#pragma unroll
            for (int r = 0; r < 16; ++r) S[r] = (8 * (r / 4) + (r % 4) >= lim) ? -INFINITY : S[r];
          }
          if (k >= 2 && k < 10) {
            const int i = (k - 2) >> 2, e = 2 * ((k - 2) & 3);
            const float p0 = __builtin_amdgcn_exp2f(fmaf(S[8 * i + e], c_l2, -m_ref));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(S[8 * i + e + 1], c_l2, -m_ref));
            lsum += p0;   // two running sums: half the dependent chain
            lsum2 += p1;
            p_cur[i][e / 2] = pack_bf16x2(p0, p1);
            // pin the work here, between the output MFMAs: left alone, the
            // compiler sinks it to the end of the step where nothing hides it
            asm volatile("" : "+v"(p_cur[i][e / 2]), "+v"(lsum), "+v"(lsum2));
          }
        }
      };

      if constexpr (kPVOn) {
#pragma unroll
        for (int n = 0; n < kPV; ++n) {
          mfma_pv(O[n >> 1], vr[n % kRV], p_prev[n & 1]);
          if (n + kRV < kPV) vr[n % kRV] = vfrag(n + kRV);
          softmax_part(n);
          if constexpr (kP2 && kQKOn) {
            if (n >= 10 && n < 26 && (n - 10) % 4 == 0) v_read((n - 10) / 4);
            if (n >= 12 && n < 28 && (n - 12) % 4 == 0) v_write((n - 12) / 4);
          }
          after_pv_mfma(n);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 10; ++k) softmax_part(k);
        if constexpr (kP2 && kQKOn) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            v_read(i);
            v_write(i);
          }
        }
      }
      if constexpr (kQKOn) {
        if (h == 0 || __any(!(lsum + lsum2 <= kPSumLimit))) {
          // Exact path: the step's maximum per head (the other 16 tokens of
          // the head sit in lane ^ 32: a lane-half swap), the reference moved
          // to it, and the step's p recomputed.  On a later step (a score far
          // above the reference) the wave's accumulated output and sum are
          // rescaled by 2^(old - new): the exact online-softmax update.
          const float a0 = fmaxf(fmaxf(S[0], S[1]), S[2]), a1 = fmaxf(fmaxf(S[3], S[4]), S[5]);
          const float a2 = fmaxf(fmaxf(S[6], S[7]), S[8]), a3 = fmaxf(fmaxf(S[9], S[10]), S[11]);
          const float a4 = fmaxf(fmaxf(S[12], S[13]), S[14]);
          float mx = fmaxf(fmaxf(fmaxf(a0, a1), fmaxf(a2, a3)), fmaxf(a4, S[15]));
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * c_l2;
          const float m_new = h == 0 ? mx : fmaxf(m_ref, mx);
          const float corr = h == 0 ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
          m_ref = m_new;
          lsum = lsum2 = 0.f;
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const float p0 = __builtin_amdgcn_exp2f(fmaf(S[8 * i + e], c_l2, -m_ref));
              const float p1 = __builtin_amdgcn_exp2f(fmaf(S[8 * i + e + 1], c_l2, -m_ref));
              lsum += p0;
              lsum2 += p1;
              p_cur[i][e / 2] = pack_bf16x2(p0, p1);
            }
          if (h != 0) {  // (wave-uniform) O holds earlier steps: rescale it
            o_ready(O);
#pragma unroll
            for (int cb = 0; cb < kDC / 32; ++cb) {
              O[cb] *= corr;                        // through VGPRs ...
              asm volatile("" : "+a"(O[cb]));       // ... and back into the AGPRs
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

    // block of the next step to prefetch, looked up one step early
    int blk_nx = nsteps > 2 ? block_of(1) : 0;
    // Past the staged window of the page table, every wave first refills
    // sm.ptab (at most once per kPtab blocks: a piece longer than 65536
    // tokens).  Called right after a step barrier, when no wave still reads
    // the old window.
    auto ptab_window = [&](int i) __attribute__((always_inline)) {
      if (i - pbase >= kPtab) {
        wait_vm<0>();
        pbase += kPtab;
        fill_ptab(pbase);
        step_barrier();
      }
    };
    auto next_block = [&](int h) __attribute__((always_inline)) {  // the block of step h + 3
      ptab_window((h + 3) >> 1);
      blk_nx = block_of((h + 3) >> 1);
    };
    auto no_hook = [](int) __attribute__((always_inline)) {};
    if constexpr (kMode == 0) {
      if (nsteps > 1) load_step(bbuf(1), step_at(blk0, 1), valid_in(1), wave, loff);
      // Iteration h: wait until step h's own loads are done (at most the loads
      // of step h+1, issued one iteration earlier, still pending); a barrier
      // makes every wave's share visible and frees buffer (h+2)%4.  The K
      // fragments of step h are read first; the nine loads of step h+2 are
      // spread over the score MFMAs (issued back to back by all four waves
      // at once, they would queue on the compute unit's address unit for
      // several hundred cycles).  The page-table entry of step h+3 is read
      // from LDS here and resolved one iteration later, so its latency is
      // never waited for on its own.
      int blk_raw = 0;  // sm.ptab entry of step h+2, read in iteration h-1
      for (int h = 0; h < nsteps; ++h) {
        if (h + 1 < nsteps)
          wait_vm<kLoadsPerWave>();
        else
          wait_vm<0>();
        step_barrier();
        if (h > 0) blk_nx = __builtin_amdgcn_readfirstlane(blk_raw);
        const bool nx = h + 3 < nsteps;
        if (nx) ptab_window((h + 3) >> 1);
        // past the last step the descriptor is empty: the nine loads still run
        // (no branch around each) and only write zeros into a free buffer
        const bool ld = h + 2 < nsteps;
        const __amdgpu_buffer_rsrc_t r = step_rsrc(ld ? step_at(blk_nx, h + 2) : cache, ld ? valid_in(h + 2) : 0);
        unsigned char* const dst = bbuf((h + 2) % kNBuf);
        // Step 0 runs the same code with P = 0 against its own (finite,
        // zero-filled past the length) buffer: a second specialisation without
        // PV costs the register allocator more than these 32 MFMAs cost.
        run_step(std::true_type{}, std::true_type{}, h, [&](int n) __attribute__((always_inline)) {
          if (n % 4 == 1) load_piece(r, dst, wave, loff, n / 4);
          if (n == 2 && nx) blk_raw = sm.ptab[((h + 3) >> 1) - pbase];
        }, no_hook);
      }
    } else if constexpr (kP2) {
      // Iteration h: step h's codes have landed (at most the next step's
      // loads, 4 or 5 per wave, still pending) and the barrier also publishes
      // V of step h-1 and frees code buffer (h+2) % 3 and V buffer h % 2.
      // Scores of step h, then the output MFMAs of step h-1 with the softmax
      // of step h, the conversion of step h's V and the loads of step h+2
      // spread between them.
      int blk_raw = 0;
      for (int h = 0; h < nsteps; ++h) {
        wait_vm<4>();
        step_barrier();
        if (h > 0) blk_nx = __builtin_amdgcn_readfirstlane(blk_raw);
        const bool nx = h + 3 < nsteps;
        if (nx) ptab_window((h + 3) >> 1);
        const bool ld = h + 2 < nsteps;
        const auto rc = rsrc_codes(ld ? blk_nx : 0, h + 2, ld), rs = rsrc_scales(ld ? blk_nx : 0, h + 2, ld);
        unsigned char* const dst = cbuf((h + 2) % 3);
        run_step(std::true_type{}, std::true_type{}, h, [&](int n) __attribute__((always_inline)) {
          if (n == 2 && nx) blk_raw = sm.ptab[((h + 3) >> 1) - pbase];
        }, [&](int n) __attribute__((always_inline)) {
          if (n % 6 == 2) load_piece_p2(rc, rs, dst, wave, loff8_at(), lane, n / 6);
        });
      }
      step_barrier();  // V of the last step is complete
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
        if (h + 3 < nsteps) next_block(h);
        run_step(std::true_type{}, std::true_type{}, h, no_hook, no_hook);
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
    run_step(std::false_type{}, std::true_type{}, nsteps, no_hook, no_hook);  // PV of the last step
    wait_vm<0>();  // the last iterations' empty loads, before the LDS is reused
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
      (is_fp8_cache(a.cache_dtype) && a.scales != nullptr && (reinterpret_cast<uintptr_t>(a.scales) % 16) == 0);
  return a.H == kH && a.d_latent == kDC && a.D == kD && a.block_size == kBS && a.act_dtype == MLA_BF16 &&
         cache_ok && (reinterpret_cast<uintptr_t>(a.cache) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.q) % 16) == 0;
}

template <int kMode>
hipError_t launch_decode_mfma_t(const DecodeArgs& a, hipStream_t st) {
  const size_t smem = sizeof(Smem);
  if (hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(decode_mfma_kernel<kMode>), int(smem));
      e != hipSuccess)
    return e;
  dim3 grid(unsigned(a.G) * unsigned(a.n_q));
  hipLaunchKernelGGL(decode_mfma_kernel<kMode>, grid, dim3(kNT), smem, st, a);
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  if (a.cache_dtype == MLA_FP8_E4M3_PO2) return launch_decode_mfma_t<2>(a, st);
  if (a.cache_dtype == MLA_FP8_E4M3) return launch_decode_mfma_t<1>(a, st);
  return launch_decode_mfma_t<0>(a, st);
}

}  // namespace mla
