// Opt-in checks of the device-data preconditions of a call (lengths,
// positions and the page-table entries the call would read), run before the
// call's kernels.  One workgroup scans the data and writes the first
// violation it meets (kind, index, value) to a device-side result; the host
// reads it back after a stream synchronisation.  A debugging aid: it costs a
// launch and a synchronisation per call.
#include <map>
#include <mutex>

#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kNT = 256;

// kind (0 = none), index, value of the first violation
__device__ int g_validate_result[3];

__global__ __launch_bounds__(kNT) void validate_kernel(ValidateArgs a) {
  __shared__ int first;  // smallest violating item index
  __shared__ int info[3];
  if (threadIdx.x == 0) {
    first = INT32_MAX;
    info[0] = info[1] = info[2] = 0;
  }
  __syncthreads();
  const int cap = a.max_blocks * a.block_size;  // positions one sequence can hold
  int my_kind = 0, my_i = INT32_MAX, my_value = 0;  // this thread's first violation
  for (int i = threadIdx.x; i < a.n_items && !my_kind; i += kNT) {
    int kind = 0, value = 0;
    if (a.seq_lens) {  // decode-side call: item i = sequence i
      const int L = a.seq_lens[i];
      if (L < a.n_q || L > cap) {
        kind = 1;
        value = L;
      } else if (a.page_table) {
        const int nb = (L + a.block_size - 1) / a.block_size;
        for (int blk = 0; blk < nb && !kind; ++blk) {
          const int e = a.page_table[int64_t(i) * a.max_blocks + blk];
          if (e < 0) {
            kind = 2;
            value = e;
          }
        }
      }
    } else {  // token-side call: item i = token i
      const int p = a.positions[i];
      if (p < 0 || (a.page_table && p >= cap)) {
        kind = 3;
        value = p;
      } else if (a.seq_ids && a.seq_ids[i] < 0) {
        // (the table's row count is not an argument of the token-side calls,
        // so their entries are not read here: an out-of-range sequence id
        // would make this check itself read out of bounds)
        kind = 4;
        value = a.seq_ids[i];
      }
    }
    if (kind) {
      my_kind = kind;
      my_i = i;
      my_value = value;
    }
  }
  if (my_kind) atomicMin(&first, my_i);
  __syncthreads();
  if (my_kind && my_i == first) {  // the smallest violating index records the details
    info[0] = my_kind;
    info[1] = my_i;
    info[2] = my_value;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    g_validate_result[0] = info[0];
    g_validate_result[1] = info[1];
    g_validate_result[2] = info[2];
  }
}

}  // namespace

hipError_t run_validate(const ValidateArgs& a, hipStream_t st, int out[3]) {
  static std::mutex mu;  // one check at a time: they share the device-side result
  std::lock_guard<std::mutex> lock(mu);
  static std::map<int, int*> addr;  // the result's address on each device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  auto it = addr.find(dev);
  if (it == addr.end()) {
    int* p = nullptr;
    e = hipGetSymbolAddress(reinterpret_cast<void**>(&p), HIP_SYMBOL(g_validate_result));
    if (e != hipSuccess) return e;
    it = addr.emplace(dev, p).first;
  }
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(kNT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(out, it->second, 3 * sizeof(int), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
  return hipStreamSynchronize(st);
}

}  // namespace mla
