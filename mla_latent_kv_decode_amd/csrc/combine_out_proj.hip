// Log-sum-exp merge of the decode partials followed by the per-head value
// up-projection, in one pass: for every row r = (b, j) and head i,
//   u = sum_s w_s o_s / sum_s w_s,  w_s = exp(lse_s - max_s lse_s)
//   o[r, i, :] = W^UV_i u
// ([MLA-93] decoding section: attention output aggregated in latent space,
// then up-projected by W^UV).  u never has to leave the chip.
//
// One workgroup per (head, 32 rows); d_latent = 512, d_v <= 128 (multiple of
// 32), bf16 partials and weights, fp32 accumulation.
//  * Where each sequence's pieces sit (first slot, count) is read from the
//    table mla_decode records beside the partials, so no plan is recomputed.
//  * The head's W^UV_i (d_v rows of 1 KB) is copied into LDS by direct 1 KB
//    loads (16-byte chunks XOR-swizzled by row), issued right after the table
//    is in: it streams in while the workgroup merges.
//  * Each wave merges 8 rows: every lane owns 8 channels; the lse values and
//    partial rows of a chunk of 4 pieces are loaded for all 8 rows before any
//    is used.  The merged u row is rounded to bf16 (as mla_decode_combine
//    stores it) and written to an LDS tile with the same swizzle.
//  * Wave w then computes output columns 32w..32w+31 with 32
//    v_mfma_f32_32x32x16_bf16 (A = u rows, B = W rows, both from LDS).
//  * Workgroup ids are remapped so the row groups of one head run on one XCD
//    and share its L2 for W^UV_i.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

constexpr int kNT = 256;
constexpr int kRows = 32;                 // rows per workgroup
constexpr int kRowsPerWave = kRows / (kNT / kWave);
constexpr int kDC = 512;
constexpr int kRowBytes = kDC * 2;        // one 1 KB row of u or W
constexpr int kMaxDV = 128;
constexpr int kPC = 4;                    // pieces merged per chunk

struct Smem {
  alignas(128) unsigned char w[kMaxDV * kRowBytes];  // W^UV_i
  alignas(128) unsigned char u[kRows * kRowBytes];   // merged rows (bf16)
};
constexpr int kMaxGroups = 8;         // row groups per workgroup (W^UV_i loaded once for all)

MLA_DEV uint32_t lds_addr(const unsigned char* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_u8*)p));
}
// byte offset of 16-byte chunk c of row `row` (chunks XOR-swizzled by row)
MLA_DEV uint32_t chunk_off(int row, int c) { return uint32_t(row * kRowBytes + ((c ^ (row & 15)) << 4)); }

// W^UV_i -> LDS: dv/4 rows per wave, one 1 KB direct load each; lane l fills
// chunk slot l of its row with source chunk l ^ (row & 15).
MLA_DEV void load_w_rows(unsigned char* dst, const void* w_uv, int h, int dv, int wave, int lane) {
  const unsigned char* wsrc = static_cast<const unsigned char*>(w_uv) + size_t(h) * dv * kRowBytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)wsrc, (short)0, dv * kRowBytes, 0x00020000);
  const int per = dv / (kNT / kWave);
  for (int i = 0; i < per; ++i) {
    const int row = wave * per + i;
    const uint32_t voff = uint32_t((lane ^ (row & 15)) << 4);
    asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(rs), "s"(row * kRowBytes), "{m0}"(lds_addr(dst + row * kRowBytes))
                 : "memory");
  }
}

// One workgroup per (head, gpw consecutive groups of 32 rows): W^UV_i is
// loaded once and serves every group.
__global__ __launch_bounds__(kNT, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void combine_out_proj_kernel(CombineProjArgs a, int gpw) {
  extern __shared__ __attribute__((aligned(128))) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane / 32, m = lane % 32;
  const int R = a.batch * a.n_q, H = a.H, dv = a.d_v;
  const int ngroups = (R + kRows - 1) / kRows;
  const int nblk = (ngroups + gpw - 1) / gpw;  // workgroups per head
  // consecutive logical ids share an XCD (workgroups are dealt round-robin)
  const int NB = gridDim.x, xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int logical = xcd * (NB / 8) + min(xcd, NB % 8) + idx;
  const int h = logical / nblk, gb = logical % nblk;
  const int R0 = gb * gpw * kRows, Rend = min(R, R0 + gpw * kRows);
  const int ngr = (Rend - R0 + kRows - 1) / kRows;  // groups of this workgroup


  // ---- 0. first slot and piece count of this wave's rows, from the table
  // the decode recorded; lane l keeps those of row l % 8 in group l / 8 ----
  static_assert(kMaxGroups * kRowsPerWave <= kWave, "one row per lane");
  int l_slot0 = 0, l_np = 0;
  {
    const int row = R0 + (lane / kRowsPerWave) * kRows + wave * kRowsPerWave + lane % kRowsPerWave;
    if (lane / kRowsPerWave < ngr && row < Rend) {
      const int2 t = *reinterpret_cast<const int2*>(a.ws_tab + 2 * (row / a.n_q));
      l_slot0 = t.x;
      l_np = t.y;
    }
  }
  // consumed here, so the wait for the table comes before the W loads
  // (waiting for it later would also wait for them)
  asm volatile("" ::"v"(l_slot0), "v"(l_np));

  // ---- 1. W^UV_i into LDS: it streams in while the rows merge ----
  load_w_rows(sm.w, a.w_uv, h, dv, wave, lane);

  for (int k = 0; k < ngr; ++k) {
  const int r0 = R0 + k * kRows, nrows = min(kRows, R - r0);
  int slot0[kRowsPerWave], np[kRowsPerWave], maxnp = 0;
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    slot0[i] = __builtin_amdgcn_readlane(l_slot0, k * kRowsPerWave + i);
    np[i] = __builtin_amdgcn_readlane(l_np, k * kRowsPerWave + i);
    maxnp = max(maxnp, np[i]);
  }

  // ---- 2. merge the pieces of this wave's 8 rows (lane = 8 channels) ----
  float M[kRowsPerWave], wsum[kRowsPerWave], acc[kRowsPerWave][8];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    M[i] = -INFINITY;
    wsum[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  }
  // per row: the lse / partial row of its first piece; pieces of one
  // (sequence, query) are n_q * H rows apart
  const size_t pstride = size_t(a.n_q) * H;
  const float* lrow[kRowsPerWave];
  const uint16_t* orow_ws[kRowsPerWave];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int j = (r0 + wave * kRowsPerWave + i) % a.n_q;
    const size_t r = (size_t(slot0[i]) * a.n_q + j) * H + h;
    lrow[i] = a.ws_lse + r;
    orow_ws[i] = static_cast<const uint16_t*>(a.ws_o) + r * kDC + 8 * lane;
  }
  static_assert(kRowsPerWave * kPC <= kWave, "one lse per lane");
  // lane l < 32 fetches the lse of (row l / kPC, piece s0 + l % kPC)
  const int li = min(lane / kPC, kRowsPerWave - 1), lsp = lane % kPC;
  int ln_np = 0;
  const float* l_lrow = lrow[0];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
    if (li == i) {
      ln_np = np[i];
      l_lrow = lrow[i];
    }
  for (int s0 = 0; s0 < maxnp; s0 += kPC) {
    uint4 x[kRowsPerWave][kPC];
    // Loads are unconditional (a branch around each would make the wave wait
    // for every load before issuing the next): a piece past the row's count
    // reads the row's last piece (a row with none reads slot 0) and is masked
    // below by lse = -inf.
    const int lp = max(0, min(s0 + lsp, ln_np - 1));
    const float lse_l = l_lrow[ln_np > 0 ? size_t(lp) * pstride : 0];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
      for (int s = 0; s < kPC; ++s) {
        const int p = max(0, min(s0 + s, np[i] - 1));
        const size_t off = size_t(p) * pstride;
        x[i][s] = *reinterpret_cast<const uint4*>(orow_ws[i] + (np[i] > 0 ? off * kDC : 0));
      }
    __builtin_amdgcn_sched_barrier(0);  // every load of the chunk is issued before the first use
    // The chunk's weights are computed one (row, piece) per lane, lane l < 32
    // holding row l / kPC and piece s0 + l % kPC: the same expf of the same
    // operands as a per-row loop would take (so the merge stays bit-identical
    // to mla_decode_combine's), two per lane instead of forty wave-uniform
    // ones, then read back per row.
    const float ls_l = s0 + lsp < ln_np ? lse_l : -INFINITY;  // mask pieces past the row's count
    float mc_l = fmaxf(ls_l, __shfl_xor(ls_l, 1, kWave));     // the row's four lanes
    mc_l = fmaxf(mc_l, __shfl_xor(mc_l, 2, kWave));
    float m_l = M[0];
#pragma unroll
    for (int i = 1; i < kRowsPerWave; ++i)
      if (li == i) m_l = M[i];
    const float mn_l = fmaxf(m_l, mc_l);
    const float sc_l = m_l == -INFINITY ? 0.f : expf(m_l - mn_l);  // rescale earlier chunks
    const float w_l = ls_l == -INFINITY ? 0.f : expf(ls_l - mn_l);
    auto lane_f = [](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const float sc = lane_f(sc_l, i * kPC);
      M[i] = lane_f(mn_l, i * kPC);
      wsum[i] *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] *= sc;
#pragma unroll
      for (int s = 0; s < kPC; ++s) {
        const float w = lane_f(w_l, i * kPC + s);
        wsum[i] += w;
        if (w != 0.f) {
          const uint32_t v[4] = {x[i][s].x, x[i][s].y, x[i][s].z, x[i][s].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[i][2 * e] += w * __uint_as_float(v[e] << 16);
            acc[i][2 * e + 1] += w * __uint_as_float(v[e] & 0xffff0000u);
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int r = wave * kRowsPerWave + i;
    const float inv = wsum[i] > 0.f ? 1.f / wsum[i] : 0.f;
    uint4 pk;
    pk.x = pack_bf16x2(acc[i][0] * inv, acc[i][1] * inv);
    pk.y = pack_bf16x2(acc[i][2] * inv, acc[i][3] * inv);
    pk.z = pack_bf16x2(acc[i][4] * inv, acc[i][5] * inv);
    pk.w = pack_bf16x2(acc[i][6] * inv, acc[i][7] * inv);
    // rows past the end get zeros: they feed MFMA rows that are never stored
    *reinterpret_cast<uint4*>(sm.u + chunk_off(r, lane)) = pk;
    if (r < nrows) {
      const size_t orow = size_t(r0 + r) * H + h;  // (b * n_q + j) * H + h
      if (a.u) *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.u) + orow * kDC + 8 * lane) = pk;
      if (a.lse_out && lane == 0) a.lse_out[orow] = wsum[i] > 0.f ? M[i] + logf(wsum[i]) : -INFINITY;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's W rows have landed
  __syncthreads();                                  // u tile and all W rows visible

  // ---- 3. o[rows, h, 32w..32w+31] = u . W^T on MFMA ----
  const int v0 = wave * 32;
  if (v0 < dv) {
  f32x16 o = {};
  const uint32_t ub = lds_addr(sm.u), wb = lds_addr(sm.w);
  auto afrag = [&](int s) { return *(lds_bf16x8*)(uintptr_t)(ub + chunk_off(m, 2 * s + g)); };
  auto bfrag = [&](int s) { return *(lds_bf16x8*)(uintptr_t)(wb + chunk_off(v0 + m, 2 * s + g)); };
  constexpr int kK = kDC / 16;
  bf16x8 ar[4], br[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    ar[s] = afrag(s);
    br[s] = bfrag(s);
  }
#pragma unroll
  for (int s = 0; s < kK; ++s) {
    o = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[s & 3], br[s & 3], o, 0, 0, 0);
    if (s + 4 < kK) {
      ar[s & 3] = afrag(s + 4);
      br[s & 3] = bfrag(s + 4);
    }
  }
  // lane (g, m) holds rows 8*(k/4) + 4*g + k%4 of column v0 + m
  __bf16* out = static_cast<__bf16*>(a.out);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int r = 8 * (q / 4) + 4 * g + (q % 4);
    if (r < nrows) out[(size_t(r0 + r) * H + h) * dv + v0 + m] = (__bf16)o[q];
  }
  }
  lds_barrier();  // every wave is done with the u tile before the next group writes it
  }
}


// ---------------------------------------------------------------------------
// Few rows (R <= 32, e.g. a handful of long sequences): one workgroup per
// (head, RPW rows), RPW = 1 or 2.  The 4 / RPW waves of a row split its
// pieces (wave w of the row merges pieces w, w + 4 / RPW, ...), meet in LDS,
// and the 256 threads then form the d_v outputs of each row as dot products
// against W^UV_i in LDS (two threads per output, 256 channels each).  With 64
// pieces a row this spreads the merge over many workgroups of busy waves
// instead of H workgroups with one; two rows per workgroup (when that still
// leaves about one workgroup per compute unit) read each head's W^UV_i half
// as often.
// ---------------------------------------------------------------------------
constexpr int kMaxRowModeRows = 32;
constexpr int kMaxRPW = 2;
struct RowSmem {
  alignas(128) unsigned char w[kMaxDV * kRowBytes];  // W^UV_i, rows swizzled as above
  alignas(16) float acc[kNT / kWave][kDC];           // per-wave unnormalised sums
  alignas(16) unsigned char u[kMaxRPW][kRowBytes];   // merged rows (bf16)
  float mw[kNT / kWave], sw[kNT / kWave];
};

template <int kRPW>
__global__ __launch_bounds__(kNT, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void combine_out_proj_row_kernel(CombineProjArgs a) {
  constexpr int kWPR = (kNT / kWave) / kRPW;  // waves per row
  static_assert(kRPW >= 1 && kRPW <= kMaxRPW && kWPR * kRPW == kNT / kWave, "rows per workgroup");
  extern __shared__ __attribute__((aligned(128))) unsigned char smem_raw[];
  RowSmem& sm = *reinterpret_cast<RowSmem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int R = a.batch * a.n_q, H = a.H, dv = a.d_v;
  const int nrb = (R + kRPW - 1) / kRPW;  // row blocks per head
  const int NB = gridDim.x, xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int logical = xcd * (NB / 8) + min(xcd, NB % 8) + idx;  // rows of one head share an XCD
  const int h = logical / nrb, r0 = (logical % nrb) * kRPW;
  const int nr = min(kRPW, R - r0);  // rows of this workgroup
  // this wave's row and its place among the row's waves
  const int q = wave / kWPR, wr = wave % kWPR;
  const int r = r0 + min(q, nr - 1);
  const int b = r / a.n_q, j = r % a.n_q;

  // ---- 0. the row's first slot and piece count (as the decode recorded
  // them), then W^UV_i into LDS ----
  const int slot0 = __builtin_amdgcn_readfirstlane(a.ws_tab[2 * b]);
  const int np = q < nr ? __builtin_amdgcn_readfirstlane(a.ws_tab[2 * b + 1]) : 0;
  asm volatile("" ::"s"(slot0), "s"(np));  // waited for before the W loads are issued
  load_w_rows(sm.w, a.w_uv, h, dv, wave, lane);

  // ---- 2. this wave's pieces: wr, wr + kWPR, ... (lane = 8 channels) ----
  const size_t pstride = size_t(a.n_q) * H;
  const size_t rbase = (size_t(slot0) * a.n_q + j) * H + h;
  const float* lrow = a.ws_lse + rbase;
  const uint16_t* orow = static_cast<const uint16_t*>(a.ws_o) + rbase * kDC + 8 * lane;
  const int npw = np > wr ? (np - wr + kWPR - 1) / kWPR : 0;
  float Mw = -INFINITY, swv = 0.f, acc[8] = {};
  for (int k0 = 0; k0 < npw; k0 += kPC) {
    // unconditional loads of clamped pieces, masked after (see the row-group kernel)
    const int pl = wr + kWPR * min(k0 + lane % kPC, npw - 1);
    const float lse_l = lrow[size_t(pl) * pstride];
    uint4 x[kPC];
#pragma unroll
    for (int s = 0; s < kPC; ++s) {
      const int p = wr + kWPR * min(k0 + s, npw - 1);
      x[s] = *reinterpret_cast<const uint4*>(orow + size_t(p) * pstride * kDC);
    }
    __builtin_amdgcn_sched_barrier(0);
    // the chunk's weights one piece per lane (lanes 0 .. kPC - 1; the rest
    // repeat them), read back per piece
    const float ls_l = k0 + lane % kPC < npw ? lse_l : -INFINITY;
    float mc = fmaxf(ls_l, __shfl_xor(ls_l, 1, kWave));
    mc = fmaxf(mc, __shfl_xor(mc, 2, kWave));
    const float Mn = fmaxf(Mw, __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(mc))));
    const float sc = Mw == -INFINITY ? 0.f : expf(Mw - Mn);
    const float w_l = ls_l == -INFINITY ? 0.f : expf(ls_l - Mn);
    Mw = Mn;
    if (k0 > 0) {  // (the first chunk finds zeros: nothing to rescale)
      swv *= sc;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= sc;
    }
#pragma unroll
    for (int s = 0; s < kPC; ++s) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), s));
      swv += w;
      if (w != 0.f) {
        const uint32_t v[4] = {x[s].x, x[s].y, x[s].z, x[s].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += w * __uint_as_float(v[e] << 16);
          acc[2 * e + 1] += w * __uint_as_float(v[e] & 0xffff0000u);
        }
      }
    }
  }

  // ---- 3. merge each row's waves (thread = 2 channels of every row) ----
  *reinterpret_cast<float4*>(&sm.acc[wave][8 * lane]) = float4{acc[0], acc[1], acc[2], acc[3]};
  *reinterpret_cast<float4*>(&sm.acc[wave][8 * lane + 4]) = float4{acc[4], acc[5], acc[6], acc[7]};
  if (lane == 0) {
    sm.mw[wave] = Mw;
    sm.sw[wave] = swv;
  }
  lds_barrier();
#pragma unroll
  for (int qq = 0; qq < kRPW; ++qq) {
    if (qq >= nr) break;  // (workgroup-uniform)
    float M = -INFINITY;
#pragma unroll
    for (int w = qq * kWPR; w < (qq + 1) * kWPR; ++w) M = fmaxf(M, sm.mw[w]);
    float tot = 0.f, u0 = 0.f, u1 = 0.f;
#pragma unroll
    for (int w = qq * kWPR; w < (qq + 1) * kWPR; ++w) {
      const float scw = sm.mw[w] == -INFINITY ? 0.f : expf(sm.mw[w] - M);
      tot += sm.sw[w] * scw;
      u0 += sm.acc[w][2 * tid] * scw;
      u1 += sm.acc[w][2 * tid + 1] * scw;
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    const uint32_t pk = pack_bf16x2(u0 * inv, u1 * inv);
    reinterpret_cast<uint32_t*>(sm.u[qq])[tid] = pk;
    const size_t orow_out = size_t(r0 + qq) * H + h;  // (b * n_q + j) * H + h
    if (a.u) reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.u) + orow_out * kDC)[tid] = pk;
    if (a.lse_out && tid == 0) a.lse_out[orow_out] = tot > 0.f ? M + logf(tot) : -INFINITY;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's W rows have landed
  __syncthreads();                                  // u rows and all W rows visible

  // ---- 4. o[r, h, v] = W^UV_i[v] . u (two threads per output) ----
  const int v = tid >> 1, half = tid & 1;
  if (v < dv) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const u32x4 lds_u4;
    const uint32_t wb = lds_addr(sm.w);
#pragma unroll
    for (int qq = 0; qq < kRPW; ++qq) {
      if (qq >= nr) break;
      const uint32_t ub = lds_addr(sm.u[qq]);
      float d = 0.f;
#pragma unroll 8
      for (int x = 0; x < kDC / 16; ++x) {
        const int xc = (kDC / 16) * half + x;  // 16-byte chunk of channels
        const u32x4 wv = *(lds_u4*)(uintptr_t)(wb + chunk_off(v, xc));
        const u32x4 uv = *(lds_u4*)(uintptr_t)(ub + xc * 16);
        const uint32_t wa[4] = {wv[0], wv[1], wv[2], wv[3]}, ua[4] = {uv[0], uv[1], uv[2], uv[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          d = fmaf(__uint_as_float(wa[e] << 16), __uint_as_float(ua[e] << 16), d);
          d = fmaf(__uint_as_float(wa[e] & 0xffff0000u), __uint_as_float(ua[e] & 0xffff0000u), d);
        }
      }
      d += __shfl_xor(d, 1, 64);
      if (half == 0) static_cast<__bf16*>(a.out)[(size_t(r0 + qq) * H + h) * dv + v] = (__bf16)d;
    }
  }
}

}  // namespace

bool combine_out_proj_supported(const CombineProjArgs& a) {
  return a.d_latent == kDC && a.d_v > 0 && a.d_v <= kMaxDV && a.d_v % 32 == 0 &&
         (reinterpret_cast<uintptr_t>(a.w_uv) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.ws_o) % 16) == 0 &&
         (a.u == nullptr || (reinterpret_cast<uintptr_t>(a.u) % 16) == 0);
}

hipError_t launch_combine_out_proj(const CombineProjArgs& a, hipStream_t st) {
  hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(combine_out_proj_kernel), int(sizeof(Smem)));
  if (e == hipSuccess)
    e = ensure_dynamic_lds(reinterpret_cast<const void*>(combine_out_proj_row_kernel<1>), int(sizeof(RowSmem)));
  if (e == hipSuccess)
    e = ensure_dynamic_lds(reinterpret_cast<const void*>(combine_out_proj_row_kernel<2>), int(sizeof(RowSmem)));
  if (e != hipSuccess) return e;
  const int R = a.batch * a.n_q;
  if (R <= kMaxRowModeRows) {  // few rows: one workgroup per (head, one or two rows)
    if (a.H * ((R + 1) / 2) >= 256)
      hipLaunchKernelGGL(combine_out_proj_row_kernel<2>, dim3(unsigned(a.H) * unsigned((R + 1) / 2)), dim3(kNT),
                         sizeof(RowSmem), st, a);
    else
      hipLaunchKernelGGL(combine_out_proj_row_kernel<1>, dim3(unsigned(a.H) * unsigned(R)), dim3(kNT),
                         sizeof(RowSmem), st, a);
    return hipGetLastError();
  }
  // enough row groups per workgroup to keep about 256 workgroups (one per
  // compute unit) while reading each head's W^UV_i as few times as possible
  const int ngroups = (R + kRows - 1) / kRows;
  const int gpw = max(1, min(kMaxGroups, ngroups * a.H / 256));
  const unsigned n = unsigned(a.H) * unsigned((ngroups + gpw - 1) / gpw);
  hipLaunchKernelGGL(combine_out_proj_kernel, dim3(n), dim3(kNT), sizeof(Smem), st, a, gpw);
  return hipGetLastError();
}

}  // namespace mla
