// A plain streaming read of a device buffer, for the benchmark only: it measures
// the HBM read bandwidth a simple kernel reaches on this GPU, the reference the
// decode kernel's bandwidth is compared with.  Built into its own library
// (libpa_stream.so), not into libpaged_attn.so.
//
//   pa_stream_read(buf, bytes, sink, blocks, stream): every 16-byte word of buf
//   (bytes a multiple of 16) is loaded once, non-temporally, by a grid of `blocks`
//   work-groups of 256 threads striding over the buffer.  The words are folded
//   into one value per thread that is written to sink[block] only if it equals a
//   constant no real buffer produces, so the loads cannot be dropped and nothing
//   else is written.  Returns 0, or 1 for bad arguments, 2 for a launch error.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* buf, size_t n,
                                                               uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    const u32x4 b = __builtin_nontemporal_load(buf + i + stride);
    const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3];
    acc ^= c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^ d[3];
  }
  for (; i < n; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" int pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks,
                              void* stream) {
  if (!buf || !sink || blocks < 1 || (bytes & 15) ||
      (reinterpret_cast<uintptr_t>(buf) & 15))
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
