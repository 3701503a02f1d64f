// Split-KV MLA decode on gfx950 matrix cores, DeepSeek-V3 dims:
// H = 128 heads, d_c = 512, d_R = 64 (row D = 576), 64-token cache blocks,
// bf16 queries and cache, fp32 accumulation.
//
// What it computes ([MLA-93] Core Mechanics 3, decoding listing STEPs 4-5):
// for every head i, s_t = scale * ([q~_i ; q^R_i] . [c_t ; k^R_t]),
// p = softmax(s), u_i = sum_t p_t c_t -- here per piece of a partition of the
// cache blocks, written as (normalised u, log-sum-exp) partials.
//
// Design (one workgroup of 4 waves per (partition, query token)):
//  * All 128 heads share one 64-token tile of the cache.  The tile
//    (64 x 576 bf16 = 72 KB) moves HBM -> LDS once with direct-to-LDS 16-byte
//    loads (global_load_lds_dwordx4), double-buffered, and every wave reads it
//    for its own 32 heads, so each cache byte crosses HBM once per step.
//  * Scores as S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: the K fragment (32
//    tokens x 16 channels) comes from LDS as one ds_read_b128 per lane, Q^T
//    (16 channels x 32 heads) stays in registers for the whole piece.  In the
//    S^T accumulator a lane owns one head and 32 of the 64 tokens, so the
//    softmax row max is an in-lane reduction plus one exchange with lane^32,
//    and the accumulator already has the A-operand layout of the P.V product
//    (the token order inside each K=16 step is a permutation we mirror on V).
//  * P.V: O[32 heads x 512] += P[32 x 16 tokens] . V[16 tokens x 32 channels]
//    with V read from the same token-major tile by ds_read_b64_tr_b16 (each
//    16-lane group turns a 4-token x 16-channel block into per-lane columns).
//  * Softmax in log2 units against a per-head reference m_ref taken from the
//    head's first tile: p = 2^(s' - m_ref).  While every later score stays
//    below m_ref + kHeadroom (32), p <= 2^32 and nothing can overflow in fp32
//    or bf16, so O never needs rescaling and is only ever touched by MFMA.  If
//    some head exceeds its headroom, the workgroup raises that head's
//    reference and recomputes the piece (correct for any input; it does not
//    happen for ordinary logits).
//  * Masked (past-length) tokens: their score is -inf, and their tile rows are
//    outside the load's buffer range, which fills them with zeros, so
//    0 * (stale value / NaN) never reaches the accumulators.
//  * LDS tile layout: 8-token x 8-chunk sub-blocks (one 1 KB direct load
//    each), 16-byte chunks XOR-swizzled by token so both the b128 K reads and
//    the transposed V reads spread over all banks.
#include <utility>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kH = 128, kDC = 512, kDR = 64, kD = kDC + kDR, kBS = 64;
constexpr int kNT = 256;                  // 4 waves x 32 heads
constexpr int kChunks = kD / 8;           // 72 chunks of 16 B per token row
constexpr int kRowBytes = kD * 2;         // 1152
constexpr int kTileBytes = kBS * kRowBytes;  // 73728
constexpr int kLoadsPerWave = (kTileBytes / 1024) / 4;  // 18 direct loads of 1 KB
constexpr float kHeadroom = 32.0f;        // log2 headroom above the reference max

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16-byte-chunk swizzle: chunk slot (c & 7) ^ swz(t) within token t's sub-row.
MLA_DEV int swz(int t) { return ((((t & 3) << 1) | ((t >> 2) & 1)) ^ ((t >> 2) & 2)) & 7; }

// Byte offset of chunk c (0..71) of token t (0..63) inside a tile buffer.
MLA_DEV int tile_off(int t, int c) {
  return (((t >> 3) * 9 + (c >> 3)) * 64 + (t & 7) * 8 + ((c & 7) ^ swz(t))) * 16;
}

struct Smem {
  alignas(16) unsigned char tile[2][kTileBytes];
  PlanScratch<kNT> plan;
  int redo;  // a head exceeded its headroom: recompute the piece
};

MLA_DEV void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Per-lane byte offset, inside an 8-token group, of the chunk this lane loads
// in sub-block column cg: token row lane/8, swizzled chunk slot lane%8.  The
// group parity p = (token group & 1) selects the swizzle variant.
MLA_DEV int load_lane_off(int lane, int p) {
  const int t = 8 * p + lane / 8;
  return (lane / 8) * kRowBytes + ((lane & 7) ^ swz(t)) * 16;
}

// Issue this wave's 18 direct HBM->LDS loads (1 KB sub-blocks) of one cache
// block.  The buffer descriptor covers only the `nvalid` live rows: lanes whose
// row is past it read out of range, which writes zeros into LDS, so masked
// rows never carry stale or NaN data into the products.
template <int M>
MLA_DEV void load_one(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int wave, const int (&loff)[2]) {
  constexpr int cg = M % 9, par = M / 9;  // k = 18*wave + M -> tg = 2*wave + M/9
  const int k = wave * kLoadsPerWave + M;
  // the column-group offset goes into soffset: the instruction's immediate
  // offset would also shift the LDS destination
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + k * 1024),
                                           16, loff[par], (2 * wave + par) * 9216 + cg * 128, 0, 0);
}
template <int... Ms>
MLA_DEV void load_all(__amdgpu_buffer_rsrc_t r, unsigned char* dst, int wave, const int (&loff)[2],
                      std::integer_sequence<int, Ms...>) {
  (load_one<Ms>(r, dst, wave, loff), ...);
}
MLA_DEV void load_tile(unsigned char* dst, const unsigned char* src, int nvalid, int wave,
                       const int (&loff)[2]) {
  __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, nvalid * kRowBytes, 0x00020000);
  load_all(r, dst, wave, loff, std::make_integer_sequence<int, kLoadsPerWave>{});
}

MLA_DEV bf16x8 lds_b128(const unsigned char* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Score MFMAs are written as inline asm with the accumulator constrained to
// arch VGPRs: O needs the whole AGPR file, and the compiler would otherwise
// place the scores in AGPRs and shuttle O blocks through VGPRs every tile.
// Hazards the compiler cannot see are handled explicitly: the chain starts
// from a literal-zero accumulator (no VALU->MFMA dependency), successive
// accumulations into one block are always separated by an independent MFMA,
// and scores_ready() puts 24 wait states (more than the longest
// MFMA-write -> VALU-read requirement) between the last write and the softmax.
MLA_DEV void mfma_qk_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
MLA_DEV void mfma_qk(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
MLA_DEV void scores_ready(f32x16& s0, f32x16& s1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0), "+v"(s1));
}

MLA_DEV bf16x8 lds_tr_pair(const unsigned char* p0, const unsigned char* p1) {
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(kNT, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int g = lane / 32;       // lane group: which 8-wide half of a 16-wide k step
  const int hl = lane % 32;      // head within the wave (S^T column)

  // XCD-aware mapping: consecutive logical ids share an XCD (workgroups are
  // dealt round-robin to the 8 XCDs), so the n_q workgroups of a partition and
  // neighbouring partitions of one sequence share that XCD's L2.
  const int P = gridDim.x, xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int per = P / 8, rem = P % 8;
  const int logical = xcd * per + min(xcd, rem) + idx;
  const int part = logical / a.n_q, j = logical % a.n_q;

  const float c_log2 = a.scale * 1.4426950408889634f;  // scores -> log2 units

  plan_for_each_piece<kNT>(a.seq_lens, a.batch, kBS, a.G, part, sm.plan,
                           [&](int b_, int ulo_, int uhi_, int slot_) {
    // piece bounds come from LDS: tell the compiler they are wave-uniform
    const int b = __builtin_amdgcn_readfirstlane(b_), ulo = __builtin_amdgcn_readfirstlane(ulo_);
    const int uhi = __builtin_amdgcn_readfirstlane(uhi_), slot = __builtin_amdgcn_readfirstlane(slot_);
    const int L = a.seq_lens[b];
    const int nvis = L - a.n_q + j + 1;
    const int u_end = min(uhi, (nvis + kBS - 1) / kBS);
    const int ntiles = max(0, u_end - ulo);
    const size_t orow0 = (size_t(slot) * a.n_q + j) * kH + wave * 32;
    if (ntiles == 0) {  // nothing visible to this query in the piece
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.ws_o) + orow0 * kDC);
      for (int e = lane; e < 32 * kDC / 8; e += kWave) dst[e] = uint4{0u, 0u, 0u, 0u};
      if (lane < 32) a.ws_lse[orow0 + lane] = -INFINITY;
      return;
    }
    const int32_t* pt = a.page_table + int64_t(b) * a.max_blocks;
    const unsigned char* cache = static_cast<const unsigned char*>(a.cache);
    auto block_ptr = [&](int u) {
      return cache + int64_t(__builtin_amdgcn_readfirstlane(pt[u])) * kTileBytes;
    };
    auto block_at = [&](int blk) { return cache + int64_t(blk) * kTileBytes; };
    auto valid_in = [&](int u) { return min(kBS, nvis - u * kBS); };

    const int loff[2] = {load_lane_off(lane, 0), load_lane_off(lane, 1)};
    // first tile in flight while Q is fetched
    load_tile(sm.tile[0], block_ptr(ulo), valid_in(ulo), wave, loff);
    const __bf16* qrow = static_cast<const __bf16*>(a.q) +
                         ((size_t(b) * a.n_q + j) * kH + wave * 32 + hl) * kD;
    bf16x8 qf[kD / 16];
#pragma unroll
    for (int s = 0; s < kD / 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * g);

    // per-lane LDS offsets (tile-independent parts)
    //  K fragment: token t = 32*bt + hl, chunk c = 2*s + g
    int koff[4];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) koff[a4] = tile_off(hl, 2 * a4 + g);
    //  V fragment (transposed read): token 16*i + 8*sec + 4*g + s16/4,
    //  channel 32*cb + 16*h + 4*(s16%4)
    const int h16 = (lane / 16) & 1, s16 = lane % 16;
    int voff[2][2];
#pragma unroll
    for (int sec = 0; sec < 2; ++sec)
#pragma unroll
      for (int cbo = 0; cbo < 2; ++cbo)
        voff[sec][cbo] = tile_off(8 * sec + 4 * g + s16 / 4, 4 * cbo + 2 * h16 + (s16 % 4) / 2) +
                         8 * (s16 % 2);

    f32x16 O[kDC / 32];
    float m_ref = -INFINITY, l_run = 0.f;
    for (;;) {  // one pass per reference choice; normally exactly one
#pragma unroll
      for (int cb = 0; cb < kDC / 32; ++cb) O[cb] = f32x16{};
      l_run = 0.f;
      bool redo = false;
      if (threadIdx.x == 0) sm.redo = 0;
      // page-table entry of the tile after next, fetched one iteration early
      // so the lookup never sits on the critical path of a prefetch
      int blk_next = ntiles > 1 ? pt[ulo + 1] : 0;
      for (int it = 0; it < ntiles; ++it) {
        const int u = ulo + it;
        wait_vm();
        __syncthreads();  // tile `it` landed for every wave; buffer (it+1)%2 is free
        if (sm.redo) { redo = true; break; }
        if (it + 1 < ntiles)
          load_tile(sm.tile[(it + 1) & 1], block_at(__builtin_amdgcn_readfirstlane(blk_next)),
                    valid_in(u + 1), wave, loff);
        if (it + 2 < ntiles) blk_next = pt[u + 2];
        const unsigned char* tb = sm.tile[it & 1];
        const int nv = valid_in(u);

        // ---- S^T = K . Q^T  (two 32-token blocks, interleaved) ----
        // Step n = 2*s + bt reads the K fragment of channel step s for token
        // block bt (token 32*bt + hl sits in sub-block row 4*bt + hl/8, i.e.
        // +36 KB per bt).  A 4-deep ring keeps 3 LDS reads in flight behind
        // each MFMA; sched_barrier pins that order.
        f32x16 S[2];
        auto kaddr = [&](int n) {
          const int s_ = n >> 1, bt = n & 1;
          return tb + koff[s_ & 3] + (s_ >> 2) * 1024 + bt * 36864;
        };
        constexpr int kQK = 2 * (kD / 16);  // 72 MFMAs
        bf16x8 kr[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) kr[n] = lds_b128(kaddr(n));
#pragma unroll
        for (int n = 0; n < kQK; ++n) {
          const int s_ = n >> 1, bt = n & 1;
          if (s_ == 0)
            mfma_qk_first(S[bt], kr[n & 3], qf[s_]);
          else
            mfma_qk(S[bt], kr[n & 3], qf[s_]);
          if (n + 4 < kQK) kr[n & 3] = lds_b128(kaddr(n + 4));
          __builtin_amdgcn_sched_barrier(0);
        }
        scores_ready(S[0], S[1]);

        // ---- softmax (lane = one head; 32 of the 64 tokens) ----
        if (nv < kBS) {  // partial last tile: mask tokens >= nv
          const int lim = nv - 4 * g;
#pragma unroll
          for (int bt = 0; bt < 2; ++bt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * bt + 8 * (r / 4) + (r % 4) >= lim) S[bt][r] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int bt = 0; bt < 2; ++bt)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[bt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c_log2;
        if (m_ref == -INFINITY) m_ref = mx;  // first tile of the piece
        if (__any(mx > m_ref + kHeadroom)) {
          m_ref = fmaxf(m_ref, mx);
          sm.redo = 1;  // seen by every wave after the next barrier
          continue;
        }
        bf16x8 pf[4];
        float lsum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(S[i / 2][8 * (i % 2) + e], c_log2, -m_ref));
            lsum += p;
            pf[i][e] = (__bf16)p;
          }
        l_run += lsum;

        // ---- O += P . V  (consecutive MFMAs update different O blocks) ----
        // Step n = 16*i + cb: token step i, channel block cb; V fragments come
        // from two transposed reads, kept 3 steps ahead in a 4-deep ring.
        auto vfrag = [&](int n) {
          const int i = n >> 4, cb = n & 15;
          const int base = (2 * i) * 9216 + (cb >> 1) * 1024;  // voff[1] adds row 2i+1
          return lds_tr_pair(tb + base + voff[0][cb & 1], tb + base + voff[1][cb & 1]);
        };
        constexpr int kPV = 4 * (kDC / 32);  // 64 MFMAs
        bf16x8 vr[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) vr[n] = vfrag(n);
#pragma unroll
        for (int n = 0; n < kPV; ++n) {
          // O^T[channel][head] += V^T . P^T: the lane keeps one head, so the
          // normalisation and the partial store need no cross-lane traffic
          O[n & 15] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[n & 3], pf[n >> 4], O[n & 15], 0, 0, 0);
          if (n + 4 < kPV) vr[n & 3] = vfrag(n + 4);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (!redo) {
        __syncthreads();
        if (!sm.redo) break;  // a wave may have flagged on the very last tile
      }
      // recompute the piece with the raised references
      wait_vm();
      __syncthreads();
      load_tile(sm.tile[0], block_ptr(ulo), valid_in(ulo), wave, loff);
    }
    __syncthreads();  // buffers are reused by the next piece

    // ---- epilogue: normalise and write the partial (bf16) ----
    // lane (g, hl) holds O^T rows = channels 32*cb + 8*rg + 4*g + {0..3} of head hl
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = 1.f / l_tot;
    if (lane < 32) a.ws_lse[orow0 + lane] = (m_ref + log2f(l_tot)) * 0.6931471805599453f;
    uint16_t* orow = static_cast<uint16_t*>(a.ws_o) + (orow0 + hl) * kDC + 4 * g;
#pragma unroll
    for (int cb = 0; cb < kDC / 32; ++cb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint32_t lo = uint32_t(f32_to_bf16(O[cb][4 * rg + 0] * inv)) |
                            (uint32_t(f32_to_bf16(O[cb][4 * rg + 1] * inv)) << 16);
        const uint32_t hi = uint32_t(f32_to_bf16(O[cb][4 * rg + 2] * inv)) |
                            (uint32_t(f32_to_bf16(O[cb][4 * rg + 3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + 32 * cb + 8 * rg) = uint2{lo, hi};
      }
  });
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs& a) {
  return a.H == kH && a.d_latent == kDC && a.D == kD && a.block_size == kBS &&
         a.act_dtype == MLA_BF16 && a.cache_dtype == MLA_BF16 &&
         (reinterpret_cast<uintptr_t>(a.cache) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.q) % 16) == 0;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  static bool attr_set = false;
  const size_t smem = sizeof(Smem);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_mfma_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(smem));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid(unsigned(a.G) * unsigned(a.n_q));
  hipLaunchKernelGGL(decode_mfma_kernel, grid, dim3(kNT), smem, st, a);
  return hipGetLastError();
}

}  // namespace mla
