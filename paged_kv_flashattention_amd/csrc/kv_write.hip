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

// E4M3 code pair (byte 0 = lo, byte 1 = hi) of two float32 values already scaled
// and clamped to [-448, 448]; the conversion rounds to nearest, ties to even.
template <bool HIGH_WORD>
__device__ __forceinline__ uint32_t fp8_pair(float lo, float hi, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(lo, hi, (int)old, HIGH_WORD);
}

__device__ __forceinline__ float q_clamp(float x) { return fminf(fmaxf(x, -448.f), 448.f); }

// 16 bf16 values -> 16 E4M3 codes of x * inv (float32 product, clamped)
__device__ __forceinline__ u32x4 quantize16(const u32x4& x0, const u32x4& x1, float inv) {
  float f[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = q_clamp(bf16_lo(x0[i]) * inv);
    f[2 * i + 1] = q_clamp(bf16_hi(x0[i]) * inv);
    f[8 + 2 * i] = q_clamp(bf16_lo(x1[i]) * inv);
    f[8 + 2 * i + 1] = q_clamp(bf16_hi(x1[i]) * inv);
  }
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t d = fp8_pair<false>(f[4 * w], f[4 * w + 1], 0u);
    r[w] = fp8_pair<true>(f[4 * w + 2], f[4 * w + 3], d);
  }
  return r;
}

// The same placement, with the FP8 quantisation fused in ("The Stack Below the
// Stack (Part 2)", 2.1: quantisation as part of the KV-insert kernel).  One thread
// writes one 16-byte piece (16 codes) of one (token, head) row of each pool.
__global__ __launch_bounds__(kKvWriteBlock) void kv_page_write_fp8_kernel(KvWriteArgs a) {
  const int pieces_per_row = a.D >> 4;
  const int pieces_per_tok = a.Hkv * pieces_per_row;
  const long long idx = (long long)blockIdx.x * kKvWriteBlock + threadIdx.x;
  if (idx >= (long long)a.T * pieces_per_tok) return;
  const int t = (int)(idx / pieces_per_tok);
  const int rem = (int)(idx - (long long)t * pieces_per_tok);

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

  const size_t src = (size_t)t * a.Hkv * a.D + (size_t)rem * 16;
  const size_t dst = (((size_t)page << a.ps_shift) + (pos & (a.page_size - 1))) * a.Hkv * a.D +
                     (size_t)rem * 16;
  const u32x4 k0 = *reinterpret_cast<const u32x4*>(a.k_new + src);
  const u32x4 k1 = *reinterpret_cast<const u32x4*>(a.k_new + src + 8);
  const u32x4 v0 = *reinterpret_cast<const u32x4*>(a.v_new + src);
  const u32x4 v1 = *reinterpret_cast<const u32x4*>(a.v_new + src + 8);
  uint8_t* kp = reinterpret_cast<uint8_t*>(a.k_pool);
  uint8_t* vp = reinterpret_cast<uint8_t*>(a.v_pool);
  // scales per (page, KV head): the reciprocal of this page's scale, in float32 as
  // for a pool scale
  float k_inv = a.k_inv, v_inv = a.v_inv;
  if (a.k_scales) {
    const size_t s = (size_t)page * a.Hkv + rem / pieces_per_row;
    k_inv = 1.0f / a.k_scales[s];
    v_inv = 1.0f / a.v_scales[s];
  }
  *reinterpret_cast<u32x4*>(kp + dst) = quantize16(k0, k1, k_inv);
  *reinterpret_cast<u32x4*>(vp + dst) = quantize16(v0, v1, v_inv);
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream, char* desc,
                           size_t desc_len) {
  const long long work = (long long)a.T * a.Hkv * (a.D >> (a.fp8 ? 4 : 3));
  const unsigned blocks = (unsigned)((work + kKvWriteBlock - 1) / kKvWriteBlock);
  if (a.fp8)
    hipLaunchKernelGGL(kv_page_write_fp8_kernel, dim3(blocks), dim3(kKvWriteBlock), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_page_write_kernel, dim3(blocks), dim3(kKvWriteBlock), 0, stream, a);
  snprintf(desc, desc_len, "kv_page_write%s grid=%u block=%d tokens=%d", a.fp8 ?
           (a.k_scales ? "_fp8 (scales per page and KV head)" : "_fp8") : "", blocks,
           kKvWriteBlock, a.T);
  return hipGetLastError();
}

}  // namespace pa
