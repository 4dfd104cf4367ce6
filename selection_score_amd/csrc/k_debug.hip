// Debug-mode checks (KVSEL_DEBUG=1 only): a count of the NaN and Inf values
// of a float array, for the score arrays the library reads and writes.
#include "common.h"

#include <algorithm>
#include <mutex>

namespace kvsel {

// Under KVSEL_DEBUG=1, the scores a selection reads and the scores a scoring
// call writes are checked for NaN and Inf (outside the contract).  The count
// lives in one device word per GPU; the host reads it back synchronously,
// under a lock, so concurrent debug calls do not share a count.
__device__ unsigned long long g_debug_nonfinite;

__global__ void nonfinite_clear_kernel(unsigned long long* count) { *count = 0ull; }

__global__ __launch_bounds__(256) void nonfinite_count_kernel(const float* __restrict__ x, int64_t rows, int64_t cols,
                                                              int64_t stride, unsigned long long* count) {
  const int64_t total = rows * cols;
  unsigned long long c = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / cols, j = i - r * cols;
    c += (__float_as_uint(x[r * stride + j]) & 0x7f800000u) == 0x7f800000u;   // exponent all ones
  }
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  if ((threadIdx.x & 63) == 0 && c != 0) atomicAdd(count, c);
}

hipError_t debug_count_nonfinite(const float* x, int64_t rows, int64_t cols, int64_t stride, hipStream_t st,
                                 uint64_t* count) {
  static std::mutex mu;
  std::lock_guard<std::mutex> lock(mu);
  *count = 0;
  if (x == nullptr || rows <= 0 || cols <= 0) return hipSuccess;
  unsigned long long* d = nullptr;   // this device's copy of the word
  hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&d), HIP_SYMBOL(g_debug_nonfinite));
  if (e != hipSuccess) return e;
  nonfinite_clear_kernel<<<1, 1, 0, st>>>(d);
  const int64_t blocks = std::min<int64_t>(ceil_div(rows * cols, 256), 4096);
  nonfinite_count_kernel<<<static_cast<unsigned>(blocks), 256, 0, st>>>(x, rows, cols, stride, d);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  unsigned long long h = 0;
  if ((e = hipMemcpyAsync(&h, d, sizeof(h), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
  *count = h;
  return hipSuccess;
}

}  // namespace kvsel
