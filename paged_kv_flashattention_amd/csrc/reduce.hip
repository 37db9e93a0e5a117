// Split-K merge of decode partials ("The Stack Below the Stack (Part 2)", section
// 2.2, step 3): each row's S partition outputs are reweighted by their local
// log-sum-exps.  One wave per row; each lane owns D/64 output columns.  The
// partitions' weights exp(lse_c - max) are computed once per row into LDS.
#include <stdio.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pa {

constexpr int kReduceRowsPerBlock = 4;
constexpr int kReduceMaxChunk = 64;     // partition weights staged per pass

template <int D>
__global__ __launch_bounds__(64 * kReduceRowsPerBlock) void splitk_reduce_kernel(ReduceArgs a) {
  constexpr int PER = D / 64;           // output columns per lane
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = blockIdx.x * kReduceRowsPerBlock + wave;
  __shared__ float w_sm[kReduceRowsPerBlock][kReduceMaxChunk];
  if (r >= a.R) return;                 // whole wave leaves; no block barrier below

  const float* lse_row = a.part_lse + (size_t)r * a.S;
  float m = kNegInf;
  for (int c = lane; c < a.S; c += 64) m = fmaxf(m, lse_row[c]);
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));

  float acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  float tot = 0.f;
  if (m != kNegInf) {
    const float* o_row = a.part_o + (size_t)r * a.S * D + PER * lane;
    for (int c0 = 0; c0 < a.S; c0 += kReduceMaxChunk) {
      const int cn = min(kReduceMaxChunk, a.S - c0);
      float w = 0.f;
      if (lane < cn) w = __expf(lse_row[c0 + lane] - m);
      float ws = w;
      for (int off = 32; off >= 1; off >>= 1) ws += __shfl_xor(ws, off);
      tot += ws;
      w_sm[wave][lane] = w;
      __builtin_amdgcn_wave_barrier();
      for (int c = 0; c < cn; ++c) {
        const float wc = w_sm[wave][c];
        const float* src = o_row + (size_t)(c0 + c) * D;
        if constexpr (PER == 2) {
          const float2 v = *reinterpret_cast<const float2*>(src);
          acc[0] += wc * v.x;
          acc[1] += wc * v.y;
        } else {
          acc[0] += wc * src[0];
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  const bool live = tot > 0.f;
  const float inv = live ? 1.f / tot : 0.f;
  uint16_t* op = a.out + (size_t)r * D + PER * lane;
  if constexpr (PER == 2) {
    *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    __bf16 v = (__bf16)(acc[0] * inv);
    *op = __builtin_bit_cast(uint16_t, v);
  }
  if (lane == 0 && a.lse_out) a.lse_out[r] = live ? m + __logf(tot) : kNegInf;
}

// Few partitions (S <= SMAX, the common case): every load of a row -- its S lse
// values and S partial outputs -- is issued before any is used, so a row costs
// one memory round trip instead of a chain of dependent ones.  Each thread owns 4
// consecutive output columns of one row (D / 4 threads per row).
constexpr int kReduceFewThreads = 256;

template <int D, int SMAX>
__global__ __launch_bounds__(kReduceFewThreads) void splitk_reduce_few_kernel(ReduceArgs a) {
  constexpr int CH = D / 4;
  const long long i = (long long)blockIdx.x * kReduceFewThreads + threadIdx.x;
  const int r = (int)(i / CH);
  const int c = (int)(i - (long long)r * CH);
  if (r >= a.R) return;
  const float* lse_row = a.part_lse + (size_t)r * a.S;
  const float* o_row = a.part_o + (size_t)r * a.S * D + 4 * c;
  float lse[SMAX];
  f32x4 o[SMAX];
#pragma unroll
  for (int k = 0; k < SMAX; ++k) lse[k] = k < a.S ? lse_row[k] : kNegInf;
#pragma unroll
  for (int k = 0; k < SMAX; ++k)
    if (k < a.S) o[k] = *reinterpret_cast<const f32x4*>(o_row + (size_t)k * D);
  float m = kNegInf;
#pragma unroll
  for (int k = 0; k < SMAX; ++k) m = fmaxf(m, lse[k]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float tot = 0.f;
  if (m != kNegInf) {
#pragma unroll
    for (int k = 0; k < SMAX; ++k)
      if (k < a.S) {
        const float w = __expf(lse[k] - m);
        tot += w;
        acc += w * o[k];
      }
  }
  const bool live = tot > 0.f;
  const float inv = live ? 1.f / tot : 0.f;
  *reinterpret_cast<u32x2*>(a.out + (size_t)r * D + 4 * c) =
      u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  if (c == 0 && a.lse_out) a.lse_out[r] = live ? m + __logf(tot) : kNegInf;
}

template <int D>
static void launch_reduce_d(const ReduceArgs& a, hipStream_t stream, unsigned& blocks,
                            bool& few) {
  few = a.S <= 8;
  if (few) {
    blocks = (unsigned)(((long long)a.R * (D / 4) + kReduceFewThreads - 1) / kReduceFewThreads);
    if (a.S <= 4)
      hipLaunchKernelGGL((splitk_reduce_few_kernel<D, 4>), dim3(blocks), dim3(kReduceFewThreads),
                         0, stream, a);
    else
      hipLaunchKernelGGL((splitk_reduce_few_kernel<D, 8>), dim3(blocks), dim3(kReduceFewThreads),
                         0, stream, a);
    return;
  }
  blocks = (a.R + kReduceRowsPerBlock - 1) / kReduceRowsPerBlock;
  hipLaunchKernelGGL(splitk_reduce_kernel<D>, dim3(blocks), dim3(64 * kReduceRowsPerBlock), 0,
                     stream, a);
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream, char* desc, size_t desc_len) {
  unsigned blocks = 0;
  bool few = false;
  if (a.D == 128) launch_reduce_d<128>(a, stream, blocks, few);
  else launch_reduce_d<64>(a, stream, blocks, few);
  snprintf(desc, desc_len, "splitk_reduce%s<D=%d> grid=%u rows=%d splits=%d", few ? "_few" : "",
           a.D, blocks, a.R, a.S);
  return hipGetLastError();
}

}  // namespace pa
