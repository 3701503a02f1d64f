// Bias-free linear layer y = x W^T with fp32 accumulation: the query-side
// projections of the [MLA-93] decoding section (c^Q = W^DQ h, then
// q^C = W^UQ c^Q and q^R = W^QR c^Q) and its final W^O projection; with a
// single W^Q it is the one-matrix query path of the small workload.
//
// Matrix-core form (bf16, k a multiple of 512, n of 32).  At decode batch
// sizes x has few rows and the weight is the stream: every weight byte is
// read once, as whole 1 KB pieces of its rows.
//  * One workgroup per (32 or 64 weight rows = output columns, up to 64 rows
//    of x, k range).  Per 512-deep stage its four waves copy the weight row
//    pieces into LDS by direct 1 KB loads (the 16-byte chunks of row r
//    XOR-swizzled by r & 31) while they fetch their x fragments from global
//    memory (x is small and stays in L2); then each wave runs the MFMAs of
//    its share of the stage (64 rows of x: row block w & 1, k half w >> 1;
//    32 rows: k quarter w) for every 32-column block, the weight fragments
//    read from LDS.  With 64 columns the x fragments serve two blocks.  Two
//    or four workgroups share a CU, so one's loads overlap another's MFMAs.
//    (Fragments loaded straight into registers, 16 bytes per lane from 32
//    rows at once, streamed the weight at half this rate or less.)
//  * The waves' 32 x 32 accumulators meet in LDS and are summed in k order;
//    the workgroup writes y (one k range) or an fp32 partial, which a second
//    kernel sums over the ranges in range order.  Results are deterministic
//    for given shapes.
// Other shapes and fp32 run a VALU kernel: one wave per output element.
#include <algorithm>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

constexpr int kNT = 256;
constexpr int kWaves = kNT / kWave;
constexpr int kNB = 32;         // weight rows (output columns) per MFMA block
constexpr int kStage = 512;     // k per stage: one 1 KB piece of each weight row
constexpr int kRowB = kStage * 2;
constexpr int kMaxSplits = 16;

MLA_DEV uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) unsigned char*)p));
}

// kRB 32-row blocks of x and kCB 32-column blocks (weight rows) per workgroup
template <int kRB, int kCB>
__global__ __launch_bounds__(kNT, 4 / kCB) void linear_mfma_kernel(LinearArgs a, float* ws, int ks, int row_tiles) {
  constexpr int kCols = kNB * kCB;
  // the weight stage; reused at the end for the cross-wave sums
  __shared__ __attribute__((aligned(1024))) unsigned char wt[kCols * kRowB];
  constexpr int kKW = kWaves / kRB;         // waves sharing a row block (each a k part)
  constexpr int kKS = kStage / kKW / 16;    // MFMA k steps per wave and stage
  const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane / 32, m = lane % 32;
  const int rb = wave % kRB, kp = wave / kRB;
  const int M = a.rows, K = a.k, N = a.n;
  // The row tiles of one weight tile are consecutive logical workgroups of
  // one XCD (workgroups are dealt to the 8 XCDs round-robin), so they run
  // together and the second reads the weight from that XCD's L2.
  const int NB = gridDim.x, xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
  const int logical = xcd * (NB / 8) + min(xcd, NB % 8) + idx;
  const int n0 = (logical / row_tiles) * kCols, split = blockIdx.y, r0 = (logical % row_tiles) * 32 * kRB;
  const int kb = split * ks, nst = (min(K, kb + ks) - kb) / kStage;

  // direct loads of this wave's 8 weight rows: lane l fills chunk slot l of
  // row r with source chunk l ^ (r & 31)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const unsigned char*>(a.w) + size_t(n0) * K * 2), (short)0, kCols * K * 2, 0x00020000);
  const __bf16* xrow = static_cast<const __bf16*>(a.x) + size_t(min(r0 + 32 * rb + m, M - 1)) * K +
                       kp * (kStage / kKW) + 8 * g;
  const uint32_t wb = lds_addr(wt) + uint32_t(m * kRowB);
  f32x16 acc[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) acc[cb] = f32x16{};
  for (int s = 0; s < nst; ++s) {
    const int k0 = kb + s * kStage;
#pragma unroll
    for (int i = 0; i < kCols / kWaves; ++i) {
      const int r = wave * (kCols / kWaves) + i;
      const uint32_t voff = uint32_t(r * K * 2 + k0 * 2 + ((lane ^ (r & 31)) << 4));
      asm volatile(MLA_ASM_VMEM_WAIT "buffer_load_dwordx4 %0, %1, 0 offen lds"
                   :
                   : "v"(voff), "s"(rs), "{m0}"(lds_addr(wt + r * kRowB))
                   : "memory");
    }
    bf16x8 xa[kKS];
#pragma unroll
    for (int t = 0; t < kKS; ++t) xa[t] = *reinterpret_cast<const bf16x8*>(xrow + k0 + 16 * t);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // lane (g, m): weight row m, k = kp * (stage / kKW) + 16 t + 8 g of the stage
#pragma unroll
    for (int t = 0; t < kKS; ++t) {
      const int c = kp * (kKS * 2) + 2 * t + g;  // 16-byte chunk of the row
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const bf16x8 bv = *(lds_bf16x8*)(uintptr_t)(wb + uint32_t(cb * kNB * kRowB + ((c ^ m) << 4)));
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[t], bv, acc[cb], 0, 0, 0);
      }
    }
    __syncthreads();  // every wave is done with the stage before the next one lands
  }

  // ---- the k parts' accumulators, summed in k order ----
  // lane (g, m) holds rows 8 (q / 4) + 4 g + q % 4 of block rb, column 32 cb + m
  float (*red)[32 * kRB][kCols] = reinterpret_cast<float (*)[32 * kRB][kCols]>(wt);
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int q = 0; q < 16; ++q) red[kp][32 * rb + 8 * (q / 4) + 4 * g + q % 4][kNB * cb + m] = acc[cb][q];
  __syncthreads();
  constexpr int kE = 32 * kRB * kCols / kNT;  // outputs per thread, consecutive columns
  const int row = threadIdx.x / (kCols / kE), col = (threadIdx.x % (kCols / kE)) * kE;
  float v[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) v[e] = red[0][row][col + e];
#pragma unroll
  for (int p = 1; p < kKW; ++p)
#pragma unroll
    for (int e = 0; e < kE; ++e) v[e] += red[p][row][col + e];
  const int r = r0 + row;
  if (r >= M) return;
  if (gridDim.y > 1) {
    float* p = ws + (size_t(split) * M + r) * N + n0 + col;
#pragma unroll
    for (int e = 0; e < kE; e += 4) *reinterpret_cast<float4*>(p + e) = float4{v[e], v[e + 1], v[e + 2], v[e + 3]};
  } else {
    uint32_t* p = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.y) + size_t(r) * N + n0 + col);
#pragma unroll
    for (int e = 0; e < kE; e += 2) p[e / 2] = pack_bf16x2(v[e], v[e + 1]);
  }
}

// y = sum over the k ranges of their fp32 partials, in range order; four
// consecutive outputs per thread, the partials of up to 16 ranges loaded
// before any is added
__global__ __launch_bounds__(kNT) void linear_reduce_kernel(LinearArgs a, const float* ws, int S) {
  const size_t total4 = size_t(a.rows) * a.n / 4;  // n is a multiple of 64
  const size_t i = size_t(blockIdx.x) * kNT + threadIdx.x;
  if (i >= total4) return;
  const float4* p = reinterpret_cast<const float4*>(ws) + i;
  float4 x[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) x[s] = p[size_t(min(s, S - 1)) * total4];
  float4 v = x[0];
#pragma unroll
  for (int s = 1; s < kMaxSplits; ++s)
    if (s < S) {
      v.x += x[s].x;
      v.y += x[s].y;
      v.z += x[s].z;
      v.w += x[s].w;
    }
  reinterpret_cast<uint2*>(a.y)[i] = uint2{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}

// VALU form: one wave per output element, lanes strided over k, tree sum
template <int ADT>
__global__ __launch_bounds__(kNT) void linear_generic_kernel(LinearArgs a) {
  const int lane = threadIdx.x % kWave;
  const int64_t o = int64_t(blockIdx.x) * kWaves + threadIdx.x / kWave;
  if (o >= int64_t(a.rows) * a.n) return;
  const int64_t r = o / a.n, c = o % a.n;
  auto ld = [&](const void* base, int64_t i) -> float {
    if constexpr (ADT == MLA_FP32) return static_cast<const float*>(base)[i];
    else return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  };
  float acc = 0.f;
  for (int k = lane; k < a.k; k += kWave) acc = fmaf(ld(a.x, r * a.k + k), ld(a.w, c * a.k + k), acc);
  acc = wave_sum(acc);
  if (lane == 0) {
    if constexpr (ADT == MLA_FP32) static_cast<float*>(a.y)[o] = acc;
    else static_cast<uint16_t*>(a.y)[o] = f32_to_bf16(acc);
  }
}

int row_blocks(int rows) { return rows <= 32 ? 1 : 2; }

}  // namespace

bool linear_mfma_supported(const LinearArgs& a) {
  return a.act_dtype == MLA_BF16 && a.k % kStage == 0 && a.n % kNB == 0 &&
         int64_t(2 * kNB) * a.k * 2 < (int64_t(1) << 31) &&
         (reinterpret_cast<uintptr_t>(a.x) % 16) == 0 && (reinterpret_cast<uintptr_t>(a.w) % 16) == 0 &&
         (reinterpret_cast<uintptr_t>(a.y) % 16) == 0;
}

// Launch shape: column blocks per workgroup (two share each x fragment, one
// gives more workgroups), k ranges, row tiles.  The workgroups should fill
// the GPU (256 CUs, 4 / cb workgroups each) in one round: a second, partial
// round would run at a fraction of the machine.  More k ranges add fp32
// partials (written and read back: 8 bytes per range, row and column), kept
// within a quarter of the weight's bytes.
struct LinPlan {
  int rb, cb, S, ks, row_tiles;
};
LinPlan linear_plan(const LinearArgs& a) {
  constexpr int kCUs = 256;
  LinPlan best{};
  for (int cb : {2, 1}) {
    if (a.n % (kNB * cb)) continue;
    LinPlan p;
    p.rb = row_blocks(a.rows);
    p.cb = cb;
    p.row_tiles = (a.rows + 32 * p.rb - 1) / (32 * p.rb);
    const int64_t tiles = int64_t(a.n / (kNB * cb)) * p.row_tiles;
    const int stages = a.k / kStage;
    const int64_t cap = std::max<int64_t>(1, int64_t(a.k) / (16 * int64_t(std::max(a.rows, 1))));
    int64_t want = std::max<int64_t>(1, kCUs * 4 / cb / tiles);
    want = std::min<int64_t>({want, cap, int64_t(kMaxSplits), int64_t(stages)});
    const int per = int((stages + want - 1) / want);
    p.ks = per * kStage;
    p.S = (stages + per - 1) / per;
    best = p;
    if (tiles * p.S >= kCUs) break;  // fills every CU at least once
  }
  return best;
}

size_t linear_mfma_workspace(const LinearArgs& a) {
  const LinPlan p = linear_plan(a);
  return p.S > 1 ? size_t(p.S) * size_t(a.rows) * size_t(a.n) * sizeof(float) : 0;
}

hipError_t launch_linear_mfma(const LinearArgs& a, void* ws, hipStream_t st) {
  const LinPlan p = linear_plan(a);
  const dim3 grid(unsigned(a.n / (kNB * p.cb) * p.row_tiles), unsigned(p.S));
  float* w = static_cast<float*>(ws);
  if (p.rb == 1 && p.cb == 1) hipLaunchKernelGGL((linear_mfma_kernel<1, 1>), grid, dim3(kNT), 0, st, a, w, p.ks, p.row_tiles);
  if (p.rb == 1 && p.cb == 2) hipLaunchKernelGGL((linear_mfma_kernel<1, 2>), grid, dim3(kNT), 0, st, a, w, p.ks, p.row_tiles);
  if (p.rb == 2 && p.cb == 1) hipLaunchKernelGGL((linear_mfma_kernel<2, 1>), grid, dim3(kNT), 0, st, a, w, p.ks, p.row_tiles);
  if (p.rb == 2 && p.cb == 2) hipLaunchKernelGGL((linear_mfma_kernel<2, 2>), grid, dim3(kNT), 0, st, a, w, p.ks, p.row_tiles);
  if (p.S > 1) {
    const size_t total4 = size_t(a.rows) * a.n / 4;
    hipLaunchKernelGGL(linear_reduce_kernel, dim3(unsigned((total4 + kNT - 1) / kNT)), dim3(kNT), 0, st, a,
                       static_cast<const float*>(ws), p.S);
  }
  return hipGetLastError();
}

hipError_t launch_linear_generic(const LinearArgs& a, hipStream_t st) {
  const int64_t outs = int64_t(a.rows) * a.n;
  const dim3 grid(unsigned((outs + kWaves - 1) / kWaves));
  if (a.act_dtype == MLA_FP32)
    hipLaunchKernelGGL(linear_generic_kernel<MLA_FP32>, grid, dim3(kNT), 0, st, a);
  else
    hipLaunchKernelGGL(linear_generic_kernel<MLA_BF16>, grid, dim3(kNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace mla
