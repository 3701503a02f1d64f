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
//  2. prefill_expand_kernel: the expansion K^C = c W^UK^T and V = c W^UV^T,
//     one persistent GEMM launch for both, written head-major [H][T][128];
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

// The chunk's queries with q^R rotated at each token's position (rotate-half
// pairs (j, j + 32), angle pos * base^(-j/32) in fp64, cos/sin rounded to
// fp32).  One workgroup per chunk token: the 32 angles are computed once and
// shared by the token's 128 heads through LDS; one thread per (head, 16-byte
// piece): q^C pieces are copied, q^R pieces (8 pairs: chunk c with chunk
// c + 4) are rotated.
__global__ __launch_bounds__(kNT) void prefill_rope_kernel(PrefillArgs a) {
  __shared__ float cs[kDR / 2], sn[kDR / 2];
  const int tok = blockIdx.x;
  const int pos = a.seq_len - a.n_tokens + tok;
  if (threadIdx.x < kDR / 2) {
    const int j = threadIdx.x;
    double sd, cd;
    sincos(double(pos) * pow(double(a.rope_base), -double(j) / double(kDR / 2)), &sd, &cd);
    cs[j] = float(cd);
    sn[j] = float(sd);
  }
  __syncthreads();
  const uint4* src = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.q) + int64_t(tok) * kH * kDK);
  uint4* dst = reinterpret_cast<uint4*>(static_cast<__bf16*>(a.ws_q) + int64_t(tok) * kH * kDK);
  constexpr int kPieces = kDN / 8 + kDR / 16;  // 16 q^C pieces + 4 q^R piece pairs per head
  for (int i = threadIdx.x; i < kH * kPieces; i += kNT) {
    const int h = i / kPieces, k = i % kPieces;
    const int row = h * (kDK / 8);  // 24 pieces of 16 bytes per head
    if (k < kDN / 8) {
      dst[row + k] = src[row + k];
      continue;
    }
    const int c = k - kDN / 8;      // q^R pieces c and c + 4: pairs (8c + e, 8c + e + 32)
    const uint4 lo = src[row + kDN / 8 + c], hi = src[row + kDN / 8 + c + 4];
    const __bf16* x = reinterpret_cast<const __bf16*>(&lo);
    const __bf16* z = reinterpret_cast<const __bf16*>(&hi);
    uint4 olo, ohi;
    __bf16* y0 = reinterpret_cast<__bf16*>(&olo);
    __bf16* y1 = reinterpret_cast<__bf16*>(&ohi);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float xv = float(x[e]), zv = float(z[e]), c_ = cs[8 * c + e], s_ = sn[8 * c + e];
      y0[e] = (__bf16)(xv * c_ - zv * s_);
      y1[e] = (__bf16)(zv * c_ + xv * s_);
    }
    dst[row + kDN / 8 + c] = olo;
    dst[row + kDN / 8 + c + 4] = ohi;
  }
}

__global__ __launch_bounds__(kNT) void prefill_gather_kernel(PrefillArgs a) {
  // one 16-byte piece of the bf16 row per thread: row t, piece k of 72 (64
  // latent + 8 RoPE); an e4m3 row gives each piece from 8 codes x the scale
  // of their 128-channel tile (fp32 product, one bf16 rounding)
  const int64_t i = int64_t(blockIdx.x) * kNT + threadIdx.x;
  if (i >= int64_t(a.seq_len) * 72) return;
  const int t = int(i / 72), k = int(i % 72);
  const int blk = a.page_table[t / a.block_size];
  const int64_t row = int64_t(blk) * a.block_size + t % a.block_size;
  uint4 v;
  if (a.cache_scales) {
    const uint2 codes = reinterpret_cast<const uint2*>(static_cast<const unsigned char*>(a.cache) + row * (kDC + kDR))[k];
    const float sc = a.cache_scales[row * 5 + k / 16];
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const uint32_t w[2] = {codes.x, codes.y};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[e]), false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[e]), true);
      o[2 * e] = pack_bf16x2(lo[0] * sc, lo[1] * sc);
      o[2 * e + 1] = pack_bf16x2(hi[0] * sc, hi[1] * sc);
    }
    v = uint4{o[0], o[1], o[2], o[3]};
  } else {
    v = reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(a.cache) + row * (kDC + kDR) * 2)[k];
  }
  if (k < 64)
    reinterpret_cast<uint4*>(a.ws_c)[int64_t(t) * 64 + k] = v;
  else
    reinterpret_cast<uint4*>(a.ws_kr)[int64_t(t) * 8 + (k - 64)] = v;
}

// The expansion, Y = c . W^T for W = W^UK (Y = K^C) and W = W^UV (Y = V),
// W viewed as [H*128][512]: a GEMM of T x 16384 outputs over a 512-deep
// reduction, both operands contiguous along it.  One launch covers both
// matrices.  A workgroup of eight waves computes a tile of 256 weight rows x
// 256 tokens; each wave owns 128 x 64 (4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16, weight rows as the MFMA's rows so that a lane's
// outputs are 4 consecutive columns of one token's row).  The reduction runs
// in 8 stages of 64 (128 bytes of every row: whole cache lines, which halves
// the requests in flight per byte against 64-byte pieces).  A stage (64 KB)
// is loaded into registers one stage ahead and written to one of two LDS
// buffers, rows swizzled by 16-byte piece so the fragment reads hit
// distinct banks.  The workgroups are persistent, one per compute unit: the
// next tile's first stage loads while a tile's outputs are written.  Tiles
// are assigned so that each XCD keeps its own token tiles (in its L2) and
// walks the weight tiles, its workgroups sharing one weight tile at a time.
constexpr int kENT = 512;                                  // eight waves
constexpr int kEN = 256;                                   // weight rows per tile
constexpr int kET = 256;                                   // tokens per tile
constexpr int kEK = 64;                                    // reduction per stage
constexpr int kERowBytes = kEK * 2;                        // 128 bytes of a row per stage
constexpr int kEStageBytes = (kEN + kET) * kERowBytes;     // 65536
constexpr int kEChunks = kDC / kEK;                        // 8
constexpr int kELoads = (kEN + kET) / 8;                   // 64 loads of 8 rows per stage
constexpr int kELoadsPerWave = kELoads / (kENT / kWave);   // 8
constexpr int kEWTiles = kH * kDN / kEN;                   // 64 weight tiles per matrix
constexpr int kEOutRow = kDN * 2 + 16;                     // epilogue row in LDS (padded)
constexpr int kELds = 2 * kEStageBytes > (kENT / kWave) * 64 * kEOutRow ? 2 * kEStageBytes
                                                                       : (kENT / kWave) * 64 * kEOutRow;
static_assert(kDN == kDV && kELoads % (kENT / kWave) == 0 && (kEN / 8) % kELoadsPerWave == 0 && kEChunks % 2 == 0,
              "expansion tiling: a wave's loads are all weight rows or all token rows");

// 16-byte piece p of row r of a stage sits in slot p ^ ((r >> 1) & 7)
MLA_DEV int exp_slot(int r, int p) { return p ^ ((r >> 1) & 7); }

__global__ __launch_bounds__(kENT, 1) void prefill_expand_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(128))) unsigned char smem[];
  const int T = a.seq_len;
  const int ntt = (T + kET - 1) / kET;
  // persistent: the workgroups of one XCD (blockIdx % 8) walk that XCD's
  // tiles in order, r = wt * ns + s for weight tile wt and the XCD's token
  // tile s (token tiles xcd, xcd + 8, ...)
  const int xcd = blockIdx.x % 8, wg = blockIdx.x / 8, nwg = gridDim.x / 8;
  const int ns = (ntt - xcd + 7) / 8;
  const int ntiles = 2 * kEWTiles * ns;
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wn = wave & 1, wtk = wave >> 1;
  const bool w_loads = wave * kELoadsPerWave < kEN / 8;  // wave-uniform: the wave loads weight rows
  // the wave's rows: stage rows srow0 .. srow0 + 63; lane l takes row l / 8 of
  // each group of 8, piece l % 8 (8 lanes read one row's 128 contiguous bytes)
  const int srow0 = wave * kELoadsPerWave * 8;
  const int lrow = lane >> 3, lpiece = lane & 7;
  const int voff0 = ((w_loads ? srow0 : srow0 - kEN) + lrow) * (kDC * 2) + lpiece * 16;
  // fragment reads: lane (g, i) takes row i of a 32-row block, piece 2 ks + g
  const int fr = lane & 31, fg = lane >> 5;
  uint32_t cofs[kEK / 16];
#pragma unroll
  for (int ks = 0; ks < kEK / 16; ++ks) cofs[ks] = uint32_t(fr * kERowBytes + exp_slot(fr, 2 * ks + fg) * 16);

  struct Tile {
    int m, n0, t0;
    __amdgpu_buffer_rsrc_t rsrc;  // this wave's operand: weight rows or token rows
  };
  auto tile_of = [&](int r) __attribute__((always_inline)) {
    Tile t;
    const int wt = r / ns;
    t.m = wt / kEWTiles;
    t.n0 = (wt % kEWTiles) * kEN;
    t.t0 = (xcd + 8 * (r % ns)) * kET;
    if (w_loads) {
      const unsigned char* wbase =
          static_cast<const unsigned char*>(t.m == 0 ? a.w_uk : a.w_uv) + int64_t(t.n0) * kDC * 2;
      t.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)wbase, (short)0, kEN * kDC * 2, 0x00020000);
    } else {
      // token rows past T lie outside the descriptor and load as zeros
      const unsigned char* xbase = static_cast<const unsigned char*>(a.ws_c) + int64_t(t.t0) * kDC * 2;
      t.rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)xbase, (short)0, min(kET, T - t.t0) * kDC * 2, 0x00020000);
    }
    return t;
  };
  auto fetch = [&](const Tile& t, int kc, u32x4 (&R)[kELoadsPerWave]) __attribute__((always_inline)) {
#pragma unroll
    for (int mm = 0; mm < kELoadsPerWave; ++mm)
      R[mm] = __builtin_amdgcn_raw_buffer_load_b128(t.rsrc, voff0 + mm * 8 * (kDC * 2), kc * kERowBytes, 0);
  };
  auto put = [&](int kc, const u32x4 (&R)[kELoadsPerWave]) __attribute__((always_inline)) {
    unsigned char* buf = smem + (kc & 1) * kEStageBytes;
#pragma unroll
    for (int mm = 0; mm < kELoadsPerWave; ++mm) {
      const int row = srow0 + mm * 8 + lrow;
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(
          (lds_u8*)(buf + row * kERowBytes + exp_slot(row, lpiece) * 16)) = R[mm];
    }
  };
  f32x16 acc[4][2];
  // the fragments of k step ks + 1 are read while the MFMAs of step ks run
  // (two fragment sets, 48 registers; the scheduling barriers keep the
  // compiler from hoisting more reads, which the 256-register budget of two
  // waves per SIMD cannot hold next to the 128 accumulators)
  auto compute = [&](int kc) __attribute__((always_inline)) {
    const uint32_t base = lds_addr(smem) + uint32_t((kc & 1) * kEStageBytes);
    bf16x8 af[2][4], bf[2][2];
    auto read = [&](int ks, int j) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        af[j][nb] = lds_b128_at(base + uint32_t((wn * 128 + nb * 32) * kERowBytes) + cofs[ks]);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        bf[j][tb] = lds_b128_at(base + uint32_t((kEN + wtk * 64 + tb * 32) * kERowBytes) + cofs[ks]);
    };
    read(0, 0);
#pragma unroll
    for (int ks = 0; ks < kEK / 16; ++ks) {
      if (ks + 1 < kEK / 16) read(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
          acc[nb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][nb], bf[ks & 1][tb], acc[nb][tb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (wg >= ntiles) return;
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x4 R[kELoadsPerWave];
  Tile cur = tile_of(wg);
  fetch(cur, 0, R);
  for (int r = wg; r < ntiles; r += nwg) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) acc[nb][tb] = f32x16{};
    // stage s is fetched into registers one stage ahead and written to LDS
    // buffer s & 1, which the barrier after the computation of stage s - 1
    // (or after the previous tile's epilogue) freed
    put(0, R);
    fetch(cur, 1, R);
    __syncthreads();
    for (int kc = 0; kc < kEChunks; ++kc) {
      compute(kc);
      if (kc + 1 < kEChunks) {
        put(kc + 1, R);
        if (kc + 2 < kEChunks) fetch(cur, kc + 2, R);
      }
      __syncthreads();
    }
    // Epilogue.  Lane (g, i) holds weight rows 8 (q / 4) + 4 g + q % 4 of
    // block nb, token i of block tb; a wave's 128 weight rows are one head's,
    // and Y is head-major, [H][T][128], so the wave's 64 tokens are one
    // contiguous 16 KB run.  The tile goes through LDS (rows padded against
    // bank conflicts) and leaves as whole 1 KB pieces with non-temporal
    // stores, which keep the operand tiles in L2.
    unsigned char* stage = smem + wave * 64 * kEOutRow;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x2 v = {pack_bf16x2(acc[nb][tb][4 * q + 0], acc[nb][tb][4 * q + 1]),
                           pack_bf16x2(acc[nb][tb][4 * q + 2], acc[nb][tb][4 * q + 3])};
          *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(
              (lds_u8*)(stage + (tb * 32 + fr) * kEOutRow + (nb * 32 + 8 * q + 4 * fg) * 2)) = v;
        }
    // the next tile's first stage loads while this tile's outputs leave
    const Tile nxt = tile_of(r + nwg < ntiles ? r + nwg : r);
    if (r + nwg < ntiles) fetch(nxt, 0, R);
    // lane l stores piece l % 16 of rows 4 i + l / 16; the lane's offsets are
    // made opaque per tile so the compiler keeps them out of the main loop
    int er = lane >> 4, ec = lane & 15;
    asm volatile("" : "+v"(er), "+v"(ec));
    const int head = (cur.n0 >> 7) + wn;
    unsigned char* y = static_cast<unsigned char*>(cur.m == 0 ? a.ws_kc : a.ws_v) +
                       (int64_t(head) * T + cur.t0 + wtk * 64) * (kDN * 2) + (er * (kDN * 2) + ec * 16);
    const unsigned char* src = stage + er * kEOutRow + ec * 16;
    const int lim = min(64, T - cur.t0 - wtk * 64) - er;  // rows 4 i + er < nrows
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (4 * i < lim) {
        const u32x4 v = *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(
            (const lds_u8*)(src + 4 * i * kEOutRow));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(y + 4 * i * (kDN * 2)));
      }
    }
    __syncthreads();  // the staging rows are read before the next tile's stage 0 lands
    cur = nxt;
  }
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
  // keys up to here are visible to every query of the wave: steps that end
  // there need no causal mask
  const int wave_vis = p0 + min(qb * kRowsPerWG + wave * 32, C - 1);
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
  // and 8 value sub-blocks per step, five per wave ----
  // K^C and V are head-major, [H][T][128]: a head's rows are contiguous
  constexpr int row_bytes = kDN * 2;
  const unsigned char* kc_head = static_cast<const unsigned char*>(a.ws_kc) + int64_t(h) * T * row_bytes;
  const unsigned char* v_head = static_cast<const unsigned char*>(a.ws_v) + int64_t(h) * T * row_bytes;
  // One descriptor per operand for the whole key range: a step's rows are
  // addressed by soffset (step start) + voffset (this lane's row and chunk),
  // and the range check counts both, so rows past T still read as zeros.
  // Built once, outside the step loop (per step they cost about 20 scalar
  // instructions in a loop bound by instruction issue).
  const __amdgpu_buffer_rsrc_t rkc =
      __builtin_amdgcn_make_buffer_rsrc((void*)kc_head, (short)0, T * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)v_head, (short)0, T * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rkr =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.ws_kr, (short)0, T * kDR * 2, 0x00020000);
  auto issue_step = [&](int s) __attribute__((always_inline)) {
    const int t0 = s * kStep;
    unsigned char* buf = smem + (s % kNBuf) * kBufBytes;
    // wave w loads token group w (8 tokens) of every column group: K^C
    // twice, k^R, V twice -- the same five loads in every wave, no branches
    const int t = wave * 8 + lane / 8;  // token inside the step
    const int chunk = (lane % 8) ^ swz(t);
    const uint32_t kdst = lds_addr(buf) + uint32_t(wave * kKG * 1024);
    const uint32_t vdst = lds_addr(buf) + uint32_t(kKBytes + wave * kVG * 1024);
    const int so = t0 * row_bytes, sor = t0 * kDR * 2;
    load_sub(rkc, kdst, t * row_bytes + chunk * 16, so);
    load_sub(rkc, kdst + 1024u, t * row_bytes + chunk * 16, so + 128);
    load_sub(rkr, kdst + 2048u, t * kDR * 2 + chunk * 16, sor);
    load_sub(rv, vdst, t * row_bytes + chunk * 16, so);
    load_sub(rv, vdst + 1024u, t * row_bytes + chunk * 16, so + 128);
  };
  static_assert(kLoadsPerWave == 5 && kKG == 3 && kVG == 2 && kStep / 8 == kNT / kWave,
                "one token group of every column group per wave");

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
          if (h_ * kStep + kStep - 1 > wave_vis) {  // wave-uniform
            const int lim = q_lim - (h_ * kStep + 4 * g);  // causal: token index <= q_lim
#pragma unroll
            for (int r = 0; r < 16; ++r) S[r] = (8 * (r / 4) + (r % 4) > lim) ? -INFINITY : S[r];
          }
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
  static_assert((kDC + kDR) % 16 == 0 && kDC % 128 == 0, "e4m3 rows: 8-byte pieces, 16 pieces a tile");
  return a.H == kH && a.d_latent == kDC && a.d_rope == kDR && a.d_nope == kDN && a.d_v == kDV &&
         (reinterpret_cast<uintptr_t>(a.q) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.cache) % 16) == 0 &&
         (reinterpret_cast<uintptr_t>(a.out) % 8) == 0;
}

hipError_t launch_prefill_gather(const PrefillArgs& a, hipStream_t st) {
  const int64_t n = int64_t(a.seq_len) * 72;
  hipLaunchKernelGGL(prefill_gather_kernel, dim3(unsigned((n + kNT - 1) / kNT)), dim3(kNT), 0, st, a);
  hipLaunchKernelGGL(prefill_rope_kernel, dim3(unsigned(a.n_tokens)), dim3(kNT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill_expand(const PrefillArgs& a, hipStream_t st) {
  const int smem = kELds;
  if (hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(prefill_expand_kernel), smem); e != hipSuccess)
    return e;
  // one persistent workgroup per compute unit (the LDS allows no second),
  // the same number on every XCD; never more than the tiles of an XCD need
  const int ntt = (a.seq_len + kET - 1) / kET;
  const int per_xcd_tiles = 2 * kEWTiles * ((ntt + 7) / 8);
  const int per_xcd = std::max(1, std::min(mla_device_cu_count() / 8, per_xcd_tiles));
  hipLaunchKernelGGL(prefill_expand_kernel, dim3(unsigned(8 * per_xcd)), dim3(kENT), smem, st, a);
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
