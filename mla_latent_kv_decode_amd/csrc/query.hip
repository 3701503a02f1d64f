// Matrix-absorbed query ([MLA-93] Core Mechanics 3 and its decoding
// section): for every (row, head i)
//   q~_i  = (W^UK_i)^T q^C_i      (d_nope -> d_latent)
//   q^R_i = RoPE(q^R_i, position) (rotate-half pairs (j, j + d_R/2), angle
//                                  pos * base^(-j/(d_R/2)) in fp64, cos/sin
//                                  rounded to fp32)
// written packed as [q~_i ; q^R_i], the layout the decode kernels read.
//
// Matrix-core form (bf16, d_latent = 512, d_nope = 128):
// one workgroup per (head, quarter of the 512 columns, split of the rows:
// up to four groups of 32 rows each).
//  * The W^UK_i quarter (d_nope rows of 256 bytes) is copied into LDS by
//    direct 1 KB loads, the 16-byte chunks of row n XOR-swizzled by
//    (n & 3) << 2; every W byte is read once per row split.
//  * The product is out[rows][c] = q^C[rows][n] . W^UK_i[n][c]: the
//    A operand (q^C, 16 contiguous bytes along n per lane) comes straight
//    from global memory; the B operand needs 8 consecutive n of one column
//    per lane, which two ds_read_b64_tr_b16 deliver from the row-major tile
//    (each 16-lane group turns a 4-row x 16-column block into per-lane
//    columns).  The swizzle puts the 4 rows x 4 chunks of a half-wave in 16
//    distinct bank groups.
//  * Wave w owns 32 of the quarter's columns: its B fragments (all of
//    d_nope) stay in registers while it walks the rows in groups of 32, one
//    MFMA per 16 of d_nope; the outputs are staged in LDS and written as
//    256-byte row segments.
//  * The quarter-cq workgroup also rotates q^R of the rows r = cq (mod 4)
//    of its head, on the VALU while the W tile is in flight.
// Other shapes and fp32 run a VALU kernel, one workgroup per (row, head).
#include "append_finalize.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kNT = 256;
constexpr int kRows = 32;
constexpr int kDL = 512;               // d_latent of the matrix-core form
constexpr int kMaxNope = 128;
constexpr int kMaxRope = 64;
constexpr int kRopePerThread = kRows * kMaxRope / 2 / kNT;  // RoPE pairs per thread and 32-row block
constexpr int kQuarters = 4;                  // column quarters of d_latent, one workgroup each
constexpr int kQCols = kDL / kQuarters;         // 128 columns, one 32-column tile per wave
constexpr int kQRow = kQCols * 2;               // 256-byte rows of the W quarter and the stage

MLA_DEV uint32_t lds_addr(const unsigned char* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const lds_u8*)p));
}
// swizzle of the 16-byte chunks of W row n
MLA_DEV int wswz(int n) { return (n & 3) << 2; }

// rotate-half RoPE of one pair (x at j, z at j + half) at angle pos * inv_freq
// (inv_freq = base^(-j/half) in fp64; angle, cos and sin in fp64, cos/sin
// then rounded to fp32)
MLA_DEV void rope_pair(float x, float z, int pos, double inv_freq, float* y0, float* y1) {
  double sd, cd;
  sincos(double(pos) * inv_freq, &sd, &cd);
  const float cs = float(cd), sn = float(sd);
  *y0 = x * cs - z * sn;
  *y1 = z * cs + x * sn;
}
MLA_DEV double rope_inv_freq(int j, int half, float base) { return pow(double(base), -double(j) / double(half)); }

// Row splits: each workgroup takes up to kGroupsPerSplit groups of 32 rows
// (a longer serial walk over the row groups leaves the compute unit waiting
// on each group's loads); the W quarter is then read once per split, the
// later ones from L2.
constexpr int kGroupsPerSplit = 4;
MLA_HD int absorb_row_splits(int rows) {
  const int groups = (rows + kRows - 1) / kRows;
  return max(1, (groups + kGroupsPerSplit - 1) / kGroupsPerSplit);
}

// Block blk of NB (NB = 4 H x row splits); blk % 8 is the XCD the block runs on.
MLA_DEV void query_absorb_mfma_body(const QueryArgs& a, int blk, int NB) {
  __shared__ __attribute__((aligned(128))) unsigned char w_lds[kMaxNope * kQRow];    // W^UK_i quarter
  __shared__ __attribute__((aligned(128))) unsigned char o_lds[kRows * kQRow];       // output stage
  __shared__ __attribute__((aligned(128))) unsigned char r_lds[kRows * kMaxRope * 2]; // RoPE stage
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int H = a.H, dn = a.d_nope, dr = a.d_rope, R = a.rows;
  const int in_stride = dn + dr, out_stride = kDL + dr;
  // the column quarters and row splits of one head run on one XCD and share
  // its L2 for q^C (per split) and the W quarters (per quarter)
  const int xcd = blk % 8, idx = blk / 8;
  const int logical = xcd * (NB / 8) + min(xcd, NB % 8) + idx;
  const int RS = absorb_row_splits(R);
  const int h = __builtin_amdgcn_readfirstlane(logical / (kQuarters * RS));
  const int rs = __builtin_amdgcn_readfirstlane((logical / kQuarters) % RS);
  const int cq = __builtin_amdgcn_readfirstlane(logical % kQuarters);
  // this workgroup's rows [r_lo, r_hi): whole groups of 32
  const int rows_per = ((R + kRows - 1) / kRows + RS - 1) / RS * kRows;
  const int r_lo = rs * rows_per, r_hi = min(R, r_lo + rows_per);
  if (r_lo >= R) return;  // (workgroup-uniform: no barrier is left waiting)

  // ---- RoPE inputs of this workgroup's first 32 rows r = cq (mod 4), loaded
  //      before anything else: loads complete in order, so behind the W tile
  //      they would wait for all of it (unconditional loads of clamped
  //      indices; the unused ones are never stored) ----
  const int half = dr / 2;
  const int rope_rows = max(0, (r_hi - r_lo - cq + kQuarters - 1) / kQuarters);  // rows r_lo + cq + 4k
  const __bf16* qin = static_cast<const __bf16*>(a.q_in);
  float rx[kRopePerThread], rz[kRopePerThread];
  int rpos[kRopePerThread];
#pragma unroll
  for (int k = 0; k < kRopePerThread; ++k) {
    const int it = tid + kNT * k, hh = max(half, 1);
    const int kk = min(it / hh, max(rope_rows - 1, 0)), j = it % hh;
    const int rr = min(r_lo + cq + kQuarters * kk, R - 1);
    const size_t ib = (size_t(rr) * H + h) * in_stride + dn;
    rx[k] = float(qin[ib + min(j, max(dr - 1, 0))]);
    rz[k] = float(qin[ib + min(j + half, max(dr - 1, 0))]);
    rpos[k] = a.positions[rr];
  }

  // ---- A fragments of the first row group, also ahead of the W tile (the
  //      RoPE inputs' wait then counts them, not the tile) ----
  const int m = lane % 32, g = lane / 32, s16 = lane % 16, h16 = (lane / 16) & 1;
  auto load_a = [&](int r0, bf16x8 (&af)[kMaxNope / 16]) __attribute__((always_inline)) {
    const __bf16* arow = qin + (size_t(min(r0 + m, R - 1)) * H + h) * in_stride + 8 * g;
#pragma unroll
    for (int s = 0; s < kMaxNope / 16; ++s) af[s] = *reinterpret_cast<const bf16x8*>(arow + 16 * s);
  };
  bf16x8 af_cur[kMaxNope / 16], af_nxt[kMaxNope / 16];
  load_a(r_lo, af_cur);

  // ---- W^UK_i[:, 128 cq .. 128 cq + 127] -> LDS: rows of 256 bytes, four
  //      rows per direct 1 KB load, chunks of row n swizzled by (n & 3) << 2 ----
  {
    const unsigned char* wsrc =
        static_cast<const unsigned char*>(a.w_uk) + (size_t(h) * dn * kDL + size_t(cq) * kQCols) * 2;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)wsrc, (short)0, (dn - 1) * kDL * 2 + kQRow, 0x00020000);
    for (int i = wave; i < dn / 4; i += kNT / kWave) {
      const int n = 4 * i + (lane >> 4), c = lane & 15;
      const uint32_t voff = uint32_t(n * kDL * 2 + ((c ^ wswz(n)) << 4));
      asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rs), "{m0}"(lds_addr(w_lds + i * 1024))
                   : "memory");
    }
  }

  // ---- RoPE of the rows r = cq (mod 4) of this head, on the VALU while the
  //      tile is in flight; staged and written as whole 2 * d_R-byte rows ----
  __bf16* qout = static_cast<__bf16*>(a.q_out);
  {
    // the pair index j = (tid + 256 k) % half is tid % half for every k when
    // half divides 256 (one fp64 power per thread); otherwise it is per k
    const bool j_fixed = kNT % max(half, 1) == 0;
    const double inv_freq0 = rope_inv_freq(tid % max(half, 1), max(half, 1), a.rope_base);
    // one block of 32 rows from inputs already in registers (no loads here:
    // a conditional load would make the wave wait for the W tile as well)
    auto emit = [&](int rb, const float (&X)[kRopePerThread], const float (&Z)[kRopePerThread],
                    const int (&P)[kRopePerThread]) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < kRopePerThread; ++k) {
        const int it = tid + kNT * k;
        if (it < kRows * half && rb + it / half < rope_rows) {
          const int j = it % half;
          float y0, y1;
          rope_pair(X[k], Z[k], P[k], j_fixed ? inv_freq0 : rope_inv_freq(j, half, a.rope_base), &y0, &y1);
          reinterpret_cast<__bf16*>(r_lds)[(it / half) * dr + j] = (__bf16)y0;
          reinterpret_cast<__bf16*>(r_lds)[(it / half) * dr + j + half] = (__bf16)y1;
        }
      }
      // LDS-only barriers: __syncthreads() would also wait for the W tile
      lds_barrier();
      const int cpr = dr * 2 / 16;  // 16-byte chunks per RoPE row
      for (int i = tid; i < kRows * cpr; i += kNT) {
        const int k = rb + i / cpr, c = i % cpr;
        if (k < rope_rows) {
          const int rr = r_lo + cq + kQuarters * k;
          *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(qout) +
                                    ((size_t(rr) * H + h) * out_stride + kDL) * 2 + c * 16) =
              *reinterpret_cast<const uint4*>(r_lds + (i / cpr) * dr * 2 + c * 16);
        }
      }
      lds_barrier();
    };
    // a split's rows r = cq (mod 4) fit one block of 32
    static_assert(kGroupsPerSplit * kRows / kQuarters <= kRows, "one RoPE block per workgroup");
    if (rope_rows > 0) emit(0, rx, rz, rpos);
  }

  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- B fragments (the wave's 32 columns, all of d_nope), kept in registers ----
  bf16x8 bf[kMaxNope / 16];
  {
    const uint32_t wb = lds_addr(w_lds);
    const int cl = 4 * wave + 2 * h16 + ((s16 & 3) >> 1);  // logical chunk of the 256-byte row
#pragma unroll
    for (int s = 0; s < kMaxNope / 16; ++s) {
      {
        const int n1 = 16 * s + 8 * g + (s16 >> 2), n2 = n1 + 4;
        const uint32_t p1 = wb + uint32_t(n1 * kQRow + ((cl ^ wswz(n1)) << 4) + 8 * (s16 & 1));
        const uint32_t p2 = wb + uint32_t(n2 * kQRow + ((cl ^ wswz(n2)) << 4) + 8 * (s16 & 1));
        const i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p1);
        const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(uintptr_t)p2);
        const i16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        bf[s] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }

  // ---- row groups of 32: A from global, 8 MFMAs, staged, written in
  //      256-byte row segments ----
  for (int r0 = r_lo; r0 < r_hi; r0 += kRows) {
    const int nrows = min(kRows, r_hi - r0);
    if (r0 + kRows < r_hi) load_a(r0 + kRows, af_nxt);  // the next group's A, in flight meanwhile
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < kMaxNope / 16; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_cur[s], bf[s], acc, 0, 0, 0);
#pragma unroll
    for (int s = 0; s < kMaxNope / 16; ++s) af_cur[s] = af_nxt[s];
    // lane (g, m) holds rows 8*(q/4) + 4*g + q%4 of column 32 * wave + m
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int r = 8 * (q / 4) + 4 * g + (q % 4);
      *reinterpret_cast<__bf16*>(o_lds + r * kQRow + (32 * wave + m) * 2) = (__bf16)acc[q];
    }
    __syncthreads();
    for (int i = tid; i < nrows * (kQRow / 16); i += kNT) {
      const int r = i / (kQRow / 16), c = i % (kQRow / 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(qout) +
                                ((size_t(r0 + r) * H + h) * out_stride + cq * kQCols) * 2 + c * 16) =
          *reinterpret_cast<const uint4*>(o_lds + r * kQRow + c * 16);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kNT) void query_absorb_mfma_kernel(QueryArgs a) {
  query_absorb_mfma_body(a, blockIdx.x, gridDim.x);
}

// The same blocks first, then the cache append's second step
// (append_finalize.h), two units per block, in one launch.
template <int CDT>
__global__ __launch_bounds__(kNT) void append_finalize_query_kernel(AppendArgs ap, const float* ws, int nk,
                                                                    QueryArgs q, int nq) {
  if (int(blockIdx.x) < nq)
    query_absorb_mfma_body(q, blockIdx.x, nq);
  else
    append_finalize_pair<CDT>(ap, ws, nk, blockIdx.x - nq);
}

// VALU form: one workgroup per (row, head); thread c accumulates column c.
template <int ADT>
__global__ __launch_bounds__(kNT) void query_absorb_generic_kernel(QueryArgs a) {
  extern __shared__ float qc[];  // [d_nope]
  const int r = blockIdx.x / a.H, h = blockIdx.x % a.H, tid = threadIdx.x;
  const int dn = a.d_nope, dr = a.d_rope, dl = a.d_latent;
  const size_t ib = (size_t(r) * a.H + h) * (dn + dr), ob = (size_t(r) * a.H + h) * (dl + dr);
  auto ld = [&](size_t i) -> float {
    if constexpr (ADT == MLA_FP32) return static_cast<const float*>(a.q_in)[i];
    else return bf16_to_f32(static_cast<const uint16_t*>(a.q_in)[i]);
  };
  auto st = [&](size_t i, float v) {
    if constexpr (ADT == MLA_FP32) static_cast<float*>(a.q_out)[i] = v;
    else static_cast<uint16_t*>(a.q_out)[i] = f32_to_bf16(v);
  };
  for (int n = tid; n < dn; n += kNT) qc[n] = ld(ib + n);
  __syncthreads();
  const size_t wb = size_t(h) * dn * dl;
  for (int c = tid; c < dl; c += kNT) {
    float acc = 0.f;
    for (int n = 0; n < dn; ++n) {
      const float w = ADT == MLA_FP32 ? static_cast<const float*>(a.w_uk)[wb + size_t(n) * dl + c]
                                      : bf16_to_f32(static_cast<const uint16_t*>(a.w_uk)[wb + size_t(n) * dl + c]);
      acc = fmaf(qc[n], w, acc);
    }
    st(ob + c, acc);
  }
  const int half = dr / 2;
  for (int j = tid; j < half; j += kNT) {
    float y0, y1;
    rope_pair(ld(ib + dn + j), ld(ib + dn + j + half), a.positions[r], rope_inv_freq(j, half, a.rope_base),
              &y0, &y1);
    st(ob + dl + j, y0);
    st(ob + dl + j + half, y1);
  }
}

}  // namespace

bool query_absorb_mfma_supported(const QueryArgs& a) {
  return a.act_dtype == MLA_BF16 && a.d_latent == kDL && a.d_nope == kMaxNope &&
         a.d_rope > 0 && a.d_rope <= kMaxRope && a.d_rope % 8 == 0 && (a.d_nope + a.d_rope) % 8 == 0 &&
         (reinterpret_cast<uintptr_t>(a.q_in) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.w_uk) % 16) == 0 &&
         (reinterpret_cast<uintptr_t>(a.q_out) % 16) == 0;
}

hipError_t launch_query_absorb_mfma(const QueryArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(query_absorb_mfma_kernel, dim3(unsigned(a.H) * kQuarters * unsigned(absorb_row_splits(a.rows))),
                     dim3(kNT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_append_finalize_query_mfma(const AppendArgs& ap, const void* ws, const QueryArgs& q,
                                             hipStream_t st) {
  const int nk = append_mfma_slices(ap), nq = q.H * kQuarters * absorb_row_splits(q.rows);
  const dim3 grid(unsigned(nq + (append_finalize_units(ap) + 1) / 2));
  const float* w = static_cast<const float*>(ws);
  if (ap.cache_dtype == MLA_BF16)
    hipLaunchKernelGGL(append_finalize_query_kernel<MLA_BF16>, grid, dim3(kNT), 0, st, ap, w, nk, q, nq);
  else if (ap.cache_dtype == MLA_FP32)
    hipLaunchKernelGGL(append_finalize_query_kernel<MLA_FP32>, grid, dim3(kNT), 0, st, ap, w, nk, q, nq);
  else if (ap.cache_dtype == MLA_FP8_E4M3_PO2)
    hipLaunchKernelGGL(append_finalize_query_kernel<MLA_FP8_E4M3_PO2>, grid, dim3(kNT), 0, st, ap, w, nk, q, nq);
  else
    hipLaunchKernelGGL(append_finalize_query_kernel<MLA_FP8_E4M3>, grid, dim3(kNT), 0, st, ap, w, nk, q, nq);
  return hipGetLastError();
}

hipError_t launch_query_absorb_generic(const QueryArgs& a, hipStream_t st) {
  const dim3 grid(unsigned(a.rows) * unsigned(a.H));
  const size_t smem = size_t(a.d_nope) * sizeof(float);
  if (a.act_dtype == MLA_FP32)
    hipLaunchKernelGGL(query_absorb_generic_kernel<MLA_FP32>, grid, dim3(kNT), smem, st, a);
  else
    hipLaunchKernelGGL(query_absorb_generic_kernel<MLA_BF16>, grid, dim3(kNT), smem, st, a);
  return hipGetLastError();
}

}  // namespace mla
