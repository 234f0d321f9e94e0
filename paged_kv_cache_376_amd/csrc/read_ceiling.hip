// Measurement aid, not part of the library's interface: the practical HBM read ceiling of the
// device, for the benchmark to report beside each kernel's roofline.  A plain contiguous read
// of a large buffer, 16-byte loads with 8 of them in flight per thread, 2048 work-groups
// striding over the buffer; each thread folds what it read into one value so that the loads
// stay live, and no work-group writes anything unless the folded value hits a sentinel.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;
constexpr int kGrid = 2048;

__global__ __launch_bounds__(kThreads) void read_kernel(const uint4* __restrict__ p, size_t n_vec, unsigned* sink) {
  unsigned acc = 0;
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads * kInFlight;
  for (size_t base = static_cast<size_t>(blockIdx.x) * kThreads * kInFlight + threadIdx.x; base < n_vec;
       base += stride) {
    uint4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const size_t i = base + static_cast<size_t>(u) * kThreads;
      v[u] = i < n_vec ? p[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) at `p` once, on `stream`.  `sink` is device memory of at
// least 2048 unsigned ints, written only in the unlikely case that a work-group's folded value
// equals a sentinel.  Returns 0, or a hipError_t code.
extern "C" __attribute__((visibility("default"))) int pkv_read_ceiling_pass(const void* p, size_t bytes, void* sink,
                                                                            void* stream) {
  if (!p || !sink || bytes % 16 != 0) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(read_kernel, dim3(kGrid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(p), bytes / 16, static_cast<unsigned*>(sink));
  return static_cast<int>(hipGetLastError());
}
