// Shared device types and helpers for the gfx950 kernels of libpaged_attn.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// 16x16x32 bf16 matrix-core product with fp32 accumulation (gfx950).
// Lane l supplies A[l % 16][8 (l/16) .. 8 (l/16) + 7] and B[8 (l/16) ..][l % 16];
// it receives C[4 (l/16) + i][l % 16] for i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 32x32x16 bf16 matrix-core product with fp32 accumulation (gfx950).
// Lane l supplies A[l % 32][8 (l/32) .. + 7] and B[8 (l/32) ..][l % 32];
// it receives C[8 j + 4 (l/32) + i][l % 32] in element 4 j + i (j, i = 0..3).
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two fp32 values to a packed bf16 pair (round to nearest even), low half = lo.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Byte-select of two dwords: result byte k = byte sel_k of {hi:lo} (0-3 lo, 4-7 hi).
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// {low halves of x and y} and {high halves of x and y}
__device__ __forceinline__ uint32_t pack_lo_halves(uint32_t x, uint32_t y) {
  return perm_b32(y, x, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi_halves(uint32_t x, uint32_t y) {
  return perm_b32(y, x, 0x07060302u);
}

// Cross-lane combines without LDS: gfx950's v_permlane32_swap exchanges the upper
// 32 lanes of one register with the lower 32 of another, so with both operands
// equal to v the pair holds v[l] and v[l ^ 32] in every lane (v_permlane16_swap
// does the same for l ^ 16 within each half).
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_max_xor16_32(float v) { return xor32_max(xor16_max(v)); }
__device__ __forceinline__ float wave_sum_xor16_32(float v) { return xor32_sum(xor16_sum(v)); }

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const uint16_t* p) {
  return *reinterpret_cast<const u32x2*>(p);
}
// Streaming loads for data read exactly once (decode's K/V): non-temporal, so
// they do not displace reusable lines in the caches.
__device__ __forceinline__ u32x4 ld16_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld8_nt(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

// Page id of logical key `key` of a sequence, clamped into the pool and the
// table row so that a malformed table cannot send a load outside the buffers.
__device__ __forceinline__ int page_of(const int32_t* table_row, int key, int ps_shift,
                                       int max_pages, int num_pages) {
  int idx = key >> ps_shift;
  idx = idx < max_pages ? idx : max_pages - 1;
  int page = table_row[idx];
  return (unsigned)page < (unsigned)num_pages ? page : 0;
}

// A window of 64 consecutive block-table entries of one sequence, held one per
// lane, plus the next 64 already in flight.  Page lookups are made with a
// wave-uniform table index (readlane, so the page id lands in a scalar register)
// and must not decrease from call to call; crossing the window end shifts it
// and fetches the following 64 entries.  Entries are clamped into the table row
// and page ids into the pool.
struct PageWindow {
  const int32_t* row;
  int max_pages, num_pages;
  int base;       // table index held by lane 0 of `cur` (multiple of 64)
  int cur, nxt;

  __device__ __forceinline__ int fetch(int idx) const {
    idx = idx < max_pages ? idx : max_pages - 1;
    return row[idx];
  }
  __device__ __forceinline__ void init(const int32_t* r, int max_p, int num_p, int first_idx,
                                       int lane) {
    row = r;
    max_pages = max_p;
    num_pages = num_p;
    base = first_idx & ~63;
    cur = fetch(base + lane);
    nxt = fetch(base + 64 + lane);
  }
  __device__ __forceinline__ int page(int idx, int lane) {
    while (idx >= base + 64) {
      base += 64;
      cur = nxt;
      nxt = fetch(base + 64 + lane);
    }
    const int p = __builtin_amdgcn_readlane(cur, idx - base);
    return (unsigned)p < (unsigned)num_pages ? p : 0;
  }
};

// 16 bytes per lane from global memory straight into LDS: lane i reads
// sbase + voff_i (a wave-uniform base address in SGPRs plus a 32-bit per-lane byte
// offset) and its bytes land at lds_wave_base + 16 i (gfx950
// global_load_lds_dwordx4, LDS base in M0).  Written as inline assembly so that
// the compiler, which cannot tell which LDS reads such a load may feed, does not
// wait for every outstanding one before each LDS read; completion is waited for
// explicitly (vmcnt_wait) before the barrier that publishes a tile.  M0 is listed as
// clobbered although the compiler reserves it (it warns so): no code it generates for
// these kernels reads or writes M0 (every M0 write in their assembly is this block's),
// and saving and restoring M0 around each copy instead cost 2 % of the dense causal
// prefill kernel on MI355X.
__device__ __forceinline__ void dma16(const uint16_t* sbase, uint32_t voff,
                                      uint16_t* lds_wave_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "m0", "memory");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Work-group barrier that the compiler may not move memory operations across
// (the hardware barrier alone; the waits it needs are issued explicitly).
__device__ __forceinline__ void block_sync() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace pa
