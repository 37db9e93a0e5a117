// KV page writer: new tokens' K and V rows scattered into their pages, bit for
// bit (eager KV writeback of "Inside Ion", "IonAttention in One Paragraph").
// One thread moves one 16-byte piece of one (token, head) row for both pools;
// consecutive threads cover consecutive pieces of a row, so each warp of work
// reads and writes whole contiguous rows.
#include <stdio.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pa {

constexpr int kKvWriteBlock = 256;

__global__ __launch_bounds__(kKvWriteBlock) void kv_page_write_kernel(KvWriteArgs a) {
  const int pieces_per_row = a.D >> 3;                   // 16-byte pieces per head row
  const int pieces_per_tok = a.Hkv * pieces_per_row;
  const long long idx = (long long)blockIdx.x * kKvWriteBlock + threadIdx.x;
  if (idx >= (long long)a.T * pieces_per_tok) return;
  const int t = (int)(idx / pieces_per_tok);
  const int rem = (int)(idx - (long long)t * pieces_per_tok);   // = head * pieces + piece

  // sequence owning token t: the last b with cu_new[b] <= t
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_new[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int pos = a.start_pos[b] + (t - a.cu_new[b]);
  if (pos < 0) return;
  const int pidx = pos >> a.ps_shift;
  if (pidx >= a.max_pages) return;
  const int page = a.block_tables[(size_t)b * a.max_pages + pidx];
  if ((unsigned)page >= (unsigned)a.num_pages) return;

  const size_t src = (size_t)t * a.Hkv * a.D + (size_t)rem * 8;
  const size_t dst = (((size_t)page << a.ps_shift) + (pos & (a.page_size - 1))) * a.Hkv * a.D +
                     (size_t)rem * 8;
  const u32x4 k = *reinterpret_cast<const u32x4*>(a.k_new + src);
  const u32x4 v = *reinterpret_cast<const u32x4*>(a.v_new + src);
  *reinterpret_cast<u32x4*>(a.k_pool + dst) = k;
  *reinterpret_cast<u32x4*>(a.v_pool + dst) = v;
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream, char* desc,
                           size_t desc_len) {
  const long long work = (long long)a.T * a.Hkv * (a.D >> 3);
  const unsigned blocks = (unsigned)((work + kKvWriteBlock - 1) / kKvWriteBlock);
  hipLaunchKernelGGL(kv_page_write_kernel, dim3(blocks), dim3(kKvWriteBlock), 0, stream, a);
  snprintf(desc, desc_len, "kv_page_write grid=%u block=%d tokens=%d", blocks, kKvWriteBlock,
           a.T);
  return hipGetLastError();
}

}  // namespace pa
