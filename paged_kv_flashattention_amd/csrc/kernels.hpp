// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <atomic>
#include <stddef.h>
#include <stdint.h>

namespace pa {

struct DecodeArgs {
  const uint16_t* q;             // [B, Hq, D]
  const uint16_t* k_pool;        // [num_pages, page_size, Hkv, D]
  const uint16_t* v_pool;
  const int32_t* block_tables;   // [B, max_pages]
  const int32_t* seq_lens;       // [B]
  uint16_t* out;                 // [B, Hq, D]           (S == 1)
  float* lse_out;                // [B, Hq] or null      (S == 1)
  float* part_o;                 // [B * Hq, S, D]       (S > 1)
  float* part_lse;               // [B * Hq, S]          (S > 1)
  int force_partials;            // write partials even when S == 1
  int B, Hq, Hkv, G, D;
  int max_pages, num_pages, page_size, ps_shift;
  int part_len, S;
  float scale_log2;              // softmax scale * log2(e) (* k_scale for FP8 pools)
  int kv_fp8;                    // pools hold FP8 E4M3 codes (uint8) instead of bf16
  float v_scale;                 // value of one V code unit (1 for bf16 pools)
  int window;                    // sliding window: keys j >= seq_len - window only (0: none)
  const float* alibi;            // [Hq] ALiBi slopes, or null: score += slope * (j - pos)
  const int32_t* key_lo;         // [B] first key of the row's document, or null (none)
  const float* k_scales;         // FP8 pools: [num_pages, Hkv] scales per (page, KV head),
  const float* v_scales;         //   or null: one scale per pool (folded as above)
  const uint8_t* block_map;      // [B, bm_kb] listed 64-key tiles of each row, or null
  int bm_kb;
  int group;                     // partitions per one-wave work-group (0 or 1: one)
};

struct ReduceArgs {
  uint16_t* out;                 // [R, D]
  float* lse_out;                // [R] or null
  const float* part_o;           // [R, S, D]
  const float* part_lse;         // [R, S]
  int R, S, D;
};

struct KvWriteArgs {
  uint16_t* k_pool;
  uint16_t* v_pool;
  const uint16_t* k_new;         // [T, Hkv, D]
  const uint16_t* v_new;
  const int32_t* cu_new;         // [B + 1]
  const int32_t* start_pos;      // [B]
  const int32_t* block_tables;   // [B, max_pages]
  int B, T, max_pages, num_pages, page_size, ps_shift, Hkv, D;
  int fp8;                       // quantise into FP8 E4M3 pools (uint8 codes)
  float k_inv, v_inv;            // 1 / k_scale, 1 / v_scale (float32)
  const float* k_scales;         // [num_pages, Hkv] scales per (page, KV head), or null
  const float* v_scales;
};

struct PrefillArgs {
  const uint16_t* q;             // [Tq, Hq, D]
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* cu_seqlens_q;   // [B + 1]
  const int32_t* seq_lens_k;     // [B]
  const int32_t* block_tables;   // [B, max_pages]
  uint16_t* out;                 // [Tq, Hq, D]
  float* lse_out;                // [Tq, Hq] or null
  int B, Tq, max_q_len, Hq, Hkv, G, D;
  int max_pages, num_pages, page_size, ps_shift;
  int causal;
  float scale_log2;
  int n_qt;                      // query tiles per sequence (of the longest)
  int xcd_groups;                // XCD units per XCD, or 0: plain order
  int xcd_split;                 // a (sequence, KV head) group's tile ranks are dealt over
                                 // this many XCD units (1, 2, 4 or 8)
  int window;                    // sliding window: position p sees keys j > p - window (0: none)
  const float* alibi;            // [Hq] ALiBi slopes, or null: score += slope * (j - pos)
  int kv_fp8;                    // pools hold FP8 E4M3 codes (uint8) instead of bf16
  float v_scale;                 // value of one V code unit (1 for bf16 pools)
  int S;                         // key-range parts per query tile at most (1: no split)
  int part_min;                  // 64-key tiles per part at least
  float* part_o;                 // [Tq * Hq, S, D] partial outputs        (S > 1)
  float* part_lse;               // [Tq * Hq, S] partial natural-log lse   (S > 1)
  const int32_t* key_lo;         // [Tq] document range [key_lo, key_hi) of each query
  const int32_t* key_hi;         //   row, or both null (no document masks)
  const float* k_scales;         // FP8 pools: [num_pages, Hkv] scales per (page, KV head),
  const float* v_scales;         //   or null: one scale per pool
  int persist;                   // persistent work-groups (plain bf16 variant, 8 waves)
  int hp;                        // paired heads: a work-group of 8 waves takes two query
                                 //   heads of one KV group x 128 rows (set by the launcher)
  const uint8_t* block_map;      // [B, bm_qb, bm_kb] visible 64 x 64 blocks, or null
  int bm_qb, bm_kb;
};

// Optional events stamped with one kernel's own start and end: the dispatch
// carries them (hipExtLaunchKernel), so measuring adds no work to the stream.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

constexpr int kMaxDevices = 64;

// More than 64 KiB of dynamic LDS is requested for a kernel once per device (the
// first launch on each device sets it; concurrent first launches both set it, which
// is harmless).  state (one per kernel and device): 0 not yet, 1 set, 2 + error code
// otherwise.
inline hipError_t lds_attribute_once(std::atomic<int>* state, const void* kernel,
                                     size_t bytes) {
  int dev = 0;
  const hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return de;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  const int st = state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    const hipError_t e =
        hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    state[dev].store(e == hipSuccess ? 1 : 2 + (int)e, std::memory_order_release);
    return e;
  }
  return st == 1 ? hipSuccess : (hipError_t)(st - 2);
}

template <typename... Args>
inline void launch_kernel(void (*kernel)(Args...), dim3 grid, dim3 block, uint32_t lds,
                          hipStream_t stream, const KernelEvents& ev, Args... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev.start, ev.stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
}

// Each launcher enqueues on `stream` and returns hipGetLastError() of the launch;
// `desc` (>= 256 bytes) receives a one-line description of what was launched.  The
// decode and prefill launchers stamp `ev` around their main kernel.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, char* desc, size_t desc_len,
                         const KernelEvents& ev = KernelEvents());
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream, char* desc, size_t desc_len);
hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream, char* desc,
                           size_t desc_len);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream, char* desc,
                          size_t desc_len, const KernelEvents& ev = KernelEvents());
// with S > 1: merges the rows whose query tile was split (after launch_prefill; waves
// > 0: after a launch of work-groups of that many waves, as launch_mixed's 8)
hipError_t launch_prefill_merge(const PrefillArgs& a, hipStream_t stream, char* desc,
                                size_t desc_len, int waves = 0);
// One kernel for a prefill batch (plain bf16 variant, 256-row query tiles; p.B = 0:
// none) and a decode batch (bf16, d.B = 0: none) over the same pools; the merges of
// their key parts and partitions are the caller's (launch_prefill_merge with 8 waves,
// launch_reduce).  `ev` is stamped around the kernel.
hipError_t launch_mixed(const PrefillArgs& p, const DecodeArgs& d, hipStream_t stream,
                        char* desc, size_t desc_len, const KernelEvents& ev = KernelEvents());
// work-groups of the prefill part of launch_mixed (from p's B, Hq, Hkv, max_q_len and S;
// 0 for no prefill part)
long long mixed_prefill_items(const PrefillArgs& p);
// waves per prefill work-group (32 query rows each) for the longest query run (and
// whether the pools are FP8 with ALiBi slopes)
int prefill_waves(int max_q_len, bool fp8_alibi = false);
// waves per decode work-group for a grid of `groups` (KV head, partition, sequence)
// items
int decode_waves(long long groups, bool fp8);

}  // namespace pa
