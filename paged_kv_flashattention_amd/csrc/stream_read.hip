// A plain streaming read of a device buffer, for the benchmark only: it measures
// the HBM read bandwidth a simple kernel reaches on this GPU, the reference the
// decode kernel's bandwidth is compared with.  Built into its own library
// (libpa_stream.so), not into libpaged_attn.so.
//
//   pa_stream_read(buf, bytes, sink, blocks, stream): every 16-byte word of buf
//   (bytes a multiple of 16 * blocks) is loaded once, non-temporally, by a grid of
//   `blocks` work-groups of 256 threads, each streaming one contiguous chunk of
//   bytes / blocks with eight loads in flight per thread (on MI355X this reached
//   7.0-7.1 TB/s, against 6.6-7.0 TB/s for the same loads striding over the whole
//   buffer).  The words are folded into one value per thread that is written to
//   sink[block] only if it equals a constant no real buffer produces, so the loads
//   cannot be dropped and nothing else is written.  Returns 0, or 1 for bad
//   arguments, 2 for a launch error.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

constexpr int kInFlight = 8;         // loads in flight per thread

// n = words per work-group's chunk
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* buf, size_t n,
                                                               uint32_t* sink) {
  const u32x4* p = buf + (size_t)blockIdx.x * n;
  uint32_t acc = 0;
  size_t i = threadIdx.x;
  for (; i + (kInFlight - 1) * kThreads < n; i += kInFlight * kThreads) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n; i += kThreads) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                              void* stream) {
  if (!buf || !sink || blocks < 1 || (bytes & 15) || (bytes / 16) % (size_t)blocks ||
      (reinterpret_cast<uintptr_t>(buf) & 15))
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                     bytes / 16 / (size_t)blocks, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
