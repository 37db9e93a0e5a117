// Split-K paged decode attention for gfx950: the partition kernel (one work-group
// of W waves per (KV head, partition, sequence) item; the item's walk is in
// decode_item.hpp) and its launch.
#include <stdio.h>

#include "decode_item.hpp"

namespace pa {

// BM: a block map is given (a.block_map); PS: FP8 pools with scales per (page, KV
// head) (a.k_scales).  Each is compiled in only when used.
template <int D, int W, bool F8, bool BM = false, bool PS = false>
__global__ __launch_bounds__(64 * W) void decode_partition_kernel(DecodeArgs a) {
  constexpr bool DYN = false;
  constexpr bool GP = false;
  const int kvh = blockIdx.x;
  const int split = blockIdx.y;
  const int b = blockIdx.z;
#include "decode_walk.inc"
}

// Grouped partitions: a one-wave work-group walks a.group consecutive partitions of
// one (KV head, sequence) as one run of chunks, the loads running on across partition
// boundaries, and writes each partition's partial as it leaves it, with the state
// and arithmetic of a walk over that partition alone (so the partials are the same
// bits as one one-wave work-group per partition).  It replaces the partition grid
// when the caller's split count would launch several times more one-wave
// work-groups than the grid that streams HBM fastest (decode_waves).
template <int D, bool F8, bool BM = false, bool PS = false>
__global__ __launch_bounds__(64) void decode_group_kernel(DecodeArgs a) {
  decode_item<D, 1, F8, BM, PS, false, true>(a, blockIdx.x, blockIdx.y * a.group, blockIdx.z);
}

template <int D>
static hipError_t launch_group_d(const DecodeArgs& a, hipStream_t stream,
                                 const KernelEvents& ev) {
  dim3 grid(a.Hkv, (a.S + a.group - 1) / a.group, a.B);
  const dim3 block(64);
  if (a.kv_fp8 && a.k_scales) {
    if (a.block_map)
      launch_kernel(decode_group_kernel<D, true, true, true>, grid, block, 0, stream, ev, a);
    else
      launch_kernel(decode_group_kernel<D, true, false, true>, grid, block, 0, stream, ev, a);
  } else if (a.kv_fp8) {
    if (a.block_map)
      launch_kernel(decode_group_kernel<D, true, true>, grid, block, 0, stream, ev, a);
    else
      launch_kernel(decode_group_kernel<D, true>, grid, block, 0, stream, ev, a);
  } else if (a.block_map) {
    launch_kernel(decode_group_kernel<D, false, true>, grid, block, 0, stream, ev, a);
  } else {
    launch_kernel(decode_group_kernel<D, false>, grid, block, 0, stream, ev, a);
  }
  return hipGetLastError();
}

template <int D, int W>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream,
                                  const KernelEvents& ev) {
  dim3 grid(a.Hkv, a.S, a.B);
  const dim3 block(64 * W);
  if (a.kv_fp8 && a.k_scales) {
    if (a.block_map)
      launch_kernel(decode_partition_kernel<D, W, true, true, true>, grid, block, 0, stream, ev, a);
    else
      launch_kernel(decode_partition_kernel<D, W, true, false, true>, grid, block, 0, stream, ev, a);
  } else if (a.kv_fp8) {
    if (a.block_map)
      launch_kernel(decode_partition_kernel<D, W, true, true>, grid, block, 0, stream, ev, a);
    else
      launch_kernel(decode_partition_kernel<D, W, true>, grid, block, 0, stream, ev, a);
  } else if (a.block_map) {
    launch_kernel(decode_partition_kernel<D, W, false, true>, grid, block, 0, stream, ev, a);
  } else {
    launch_kernel(decode_partition_kernel<D, W, false>, grid, block, 0, stream, ev, a);
  }
  return hipGetLastError();
}

// Waves per work-group: enough waves in the whole grid (about two per CU, 512 on
// MI355X) and no more, so that each wave streams as long a run of keys as
// possible (measured on MI355X: fewer, longer streams read HBM faster; one
// wave per CU is too few).  A wave over FP8 pools moves half the bytes per chunk
// for the same work, so it takes twice the waves (about four per CU) to keep as
// many bytes in flight.
static long long decode_wave_target(bool fp8) { return fp8 ? 1024 : 512; }
int decode_waves(long long groups, bool fp8) {
  const long long target = decode_wave_target(fp8);
  return groups >= target ? 1 : (2 * groups >= target ? 2 : 4);
}
static int decode_waves(const DecodeArgs& a) {
  return decode_waves((long long)a.Hkv * a.S * a.B, a.kv_fp8 != 0);
}
// Partitions per work-group: 1, or (at least twice the target's one-wave work-groups)
// as many as bring the grid down to about the target, at most kGpMaxParts (measured
// on MI355X, 8 x 131072 keys, Hkv 8, 64 partitions: 4,096 one-wave work-groups stream
// slower than 512).
static int decode_group(long long items, int S, bool fp8) {
  long long g = items / decode_wave_target(fp8);
  if (g > S) g = S;
  if (g > kGpMaxParts) g = kGpMaxParts;
  return g < 2 ? 1 : (int)g;
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream, int W,
                                  const KernelEvents& ev) {
  if (W == 4) return launch_decode_t<D, 4>(a, stream, ev);
  if (W == 2) return launch_decode_t<D, 2>(a, stream, ev);
  return launch_decode_t<D, 1>(a, stream, ev);
}

hipError_t launch_decode(const DecodeArgs& a_in, hipStream_t stream, char* desc,
                         size_t desc_len, const KernelEvents& ev) {
  DecodeArgs a = a_in;
  const int W = decode_waves(a);
  a.group = a.S > 1 ? decode_group((long long)a.Hkv * a.S * a.B, a.S, a.kv_fp8 != 0) : 1;
  const char* pool = a.kv_fp8 ? (a.k_scales ? "fp8-e4m3 scales per page" : "fp8-e4m3") : "bf16";
  if (a.group > 1) {
    hipError_t e = a.D == 128 ? launch_group_d<128>(a, stream, ev) : launch_group_d<64>(a, stream, ev);
    snprintf(desc, desc_len,
             "decode_group<D=%d,W=1,%s%s> grid=(%d,%d,%d) block=64 part_len=%d splits=%d "
             "partitions per work-group=%d",
             a.D, pool, a.block_map ? ",block map" : "", a.Hkv, (a.S + a.group - 1) / a.group,
             a.B, a.part_len, a.S, a.group);
    return e;
  }
  hipError_t e = a.D == 128 ? launch_decode_d<128>(a, stream, W, ev)
                            : launch_decode_d<64>(a, stream, W, ev);
  snprintf(desc, desc_len,
           "decode_partition<D=%d,W=%d,%s%s> grid=(%d,%d,%d) block=%d part_len=%d splits=%d", a.D,
           W, pool, a.block_map ? ",block map" : "", a.Hkv, a.S, a.B, 64 * W, a.part_len, a.S);
  return e;
}

}  // namespace pa
