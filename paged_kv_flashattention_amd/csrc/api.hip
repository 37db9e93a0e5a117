// C-ABI entry points of libpaged_attn.so: argument validation, launch sizing,
// error reporting.  Every check runs on the host before anything is enqueued, so
// a failing call leaves outputs untouched; the only device work is the kernels'.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>
#include <functional>
#include <mutex>
#include <queue>
#include <vector>
#include <string.h>

#include "../../include/paged_attn.h"
#include "kernels.hpp"

namespace {

thread_local char g_last_error[512] = "";
thread_local char g_last_launch[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int log2_exact(int v) {
  if (v <= 0 || (v & (v - 1))) return -1;
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

bool head_dim_ok(int D) { return D == 64 || D == 128; }
bool page_size_ok(int ps) { return ps == 16 || ps == 32 || ps == 64; }

// Shared checks of the paged-KV description.
int check_pool(int32_t B, int32_t max_pages, int32_t num_pages, int32_t page_size,
               int32_t Hq, int32_t Hkv, int32_t D) {
  if (B < 0 || max_pages < 1 || num_pages < 1 || Hq < 1 || Hkv < 1)
    return fail(PA_ERR_SHAPE, "sizes must be positive (B=%d max_pages=%d num_pages=%d Hq=%d Hkv=%d)",
                B, max_pages, num_pages, Hq, Hkv);
  if (!head_dim_ok(D)) return fail(PA_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", D);
  if (!page_size_ok(page_size))
    return fail(PA_ERR_UNSUPPORTED, "page size %d not in {16, 32, 64}", page_size);
  if (Hq % Hkv) return fail(PA_ERR_UNSUPPORTED, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (Hq / Hkv > 16) return fail(PA_ERR_UNSUPPORTED, "GQA group %d exceeds 16", Hq / Hkv);
  if ((long long)num_pages * page_size * Hkv * D > (1ll << 40))
    return fail(PA_ERR_SHAPE, "pool larger than 2^40 elements");
  return PA_OK;
}

constexpr int kChunk = 32;   // keys per decode chunk; partitions are multiples of it
constexpr int32_t kMaxSplits = 65535;   // the split index is the grid's y dimension

int32_t resolve_splits(int32_t B, int32_t Hkv, int32_t max_seq_len, int32_t num_splits) {
  const int32_t chunks = max_seq_len > 0 ? (max_seq_len + kChunk - 1) / kChunk : 1;
  if (num_splits <= 0) {
    // About one work-group per CU (256 on MI355X), each streaming one long
    // partition, measured fastest; partitions keep >= 8 chunks.
    const long long groups = (long long)(B > 0 ? B : 1) * Hkv;
    long long s = (256 + groups / 2) / groups;
    const long long max_by_len = chunks / 8 > 0 ? chunks / 8 : 1;
    if (s > max_by_len) s = max_by_len;
    if (s < 1) s = 1;
    num_splits = (int32_t)s;
  }
  if (num_splits > chunks) num_splits = chunks;
  if (num_splits > kMaxSplits) num_splits = kMaxSplits;
  return num_splits < 1 ? 1 : num_splits;
}

// Keys a decode row walks at most: max_seq_len, or with a sliding window of w keys
// at most w + 31 (the window's start is rounded down to a 32-key chunk).
int32_t effective_len(int32_t max_seq_len, int32_t window) {
  if (window <= 0) return max_seq_len;
  const long long w = (long long)window + kChunk - 1;
  return w < max_seq_len ? (int32_t)w : max_seq_len;
}

bool scales_ok(float k_scale, float v_scale) {
  return k_scale > 0.f && k_scale <= 3.0e38f && v_scale > 0.f && v_scale <= 3.0e38f;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Split-K workspace: fp32 partial outputs [B, Hq, S, D] then fp32 partial lse
// [B, Hq, S].
size_t workspace_for(int32_t B, int32_t Hq, int32_t D, int32_t S) {
  if (S <= 1) return 0;
  const size_t rows = (size_t)B * Hq * S;
  return align256(rows * D * sizeof(float)) + align256(rows * sizeof(float));
}

// Scales per (page, KV head) of FP8 pools: both or neither, FP8 pools only, 4-byte
// aligned.
int page_scales_ok(const char* what, bool fp8, const float* k_scales, const float* v_scales) {
  if (!k_scales && !v_scales) return PA_OK;
  if (!k_scales || !v_scales)
    return fail(PA_ERR_NULL, "%s: k_scales and v_scales must both be given or both be NULL",
                what);
  if (!fp8)
    return fail(PA_ERR_UNSUPPORTED, "%s: scales per page need FP8 pools (kv_fp8 = 1)", what);
  if ((reinterpret_cast<uintptr_t>(k_scales) & 3u) || (reinterpret_cast<uintptr_t>(v_scales) & 3u))
    return fail(PA_ERR_MISALIGNED, "%s: k_scales and v_scales must be 4-byte aligned", what);
  return PA_OK;
}

// Checks and argument packing shared by paged_attn_decode and
// paged_attn_decode_partials.  `what` names the entry point in messages.
int decode_args(pa::DecodeArgs& a, const char* what, const void* q, const void* k_pool,
                const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                int32_t B, int32_t max_pages, int32_t num_pages, int32_t page_size, int32_t Hq,
                int32_t Hkv, int32_t D, float softmax_scale, int32_t max_seq_len,
                int32_t num_splits, bool fp8 = false, float k_scale = 1.f,
                float v_scale = 1.f, int32_t window = 0, const float* alibi = nullptr,
                const int32_t* key_lo = nullptr, const float* k_scales = nullptr,
                const float* v_scales = nullptr, const uint8_t* block_map = nullptr,
                int32_t bm_kb = 0) {
  if (B < 0 || max_seq_len < 0 || window < 0)
    return fail(PA_ERR_SHAPE, "%s: B=%d max_seq_len=%d", what, B, max_seq_len);
  int st = check_pool(B, max_pages, num_pages, page_size, Hq, Hkv, D);
  if (st) return st;
  if (B > 0) {
    if (!q || !k_pool || !v_pool || !block_tables || !seq_lens)
      return fail(PA_ERR_NULL, "%s: a required pointer is NULL", what);
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
      return fail(PA_ERR_MISALIGNED, "%s: data pointers must be 16-byte aligned", what);
  }
  if (!(softmax_scale > 0.f) || softmax_scale > 3.0e38f)
    return fail(PA_ERR_SHAPE, "%s: softmax scale must be positive and finite", what);
  if (alibi && (reinterpret_cast<uintptr_t>(alibi) & 3u))
    return fail(PA_ERR_MISALIGNED, "%s: alibi_slopes must be 4-byte aligned", what);
  if (key_lo && (reinterpret_cast<uintptr_t>(key_lo) & 3u))
    return fail(PA_ERR_MISALIGNED, "%s: key_lo must be 4-byte aligned", what);
  st = page_scales_ok(what, fp8, k_scales, v_scales);
  if (st) return st;
  if (block_map && bm_kb < 1)
    return fail(PA_ERR_SHAPE, "%s: block map of %d key blocks per sequence", what, bm_kb);
  // with scales per page the pool scales are not used
  if (k_scales) k_scale = v_scale = 1.f;
  if (fp8 && !(scales_ok(k_scale, v_scale) && softmax_scale * k_scale <= 3.0e38f))
    return fail(PA_ERR_SHAPE, "%s: k_scale and v_scale must be positive and finite", what);
  // with a window every row walks at most window + 31 keys (its lower bound rounded
  // down to a 32-key chunk): partitions are sized for that
  const int32_t len = effective_len(max_seq_len, window);
  const int32_t S = resolve_splits(B, Hkv, len, num_splits);
  const int32_t chunks = len > 0 ? (len + kChunk - 1) / kChunk : 1;
  a = pa::DecodeArgs{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.D = D;
  a.max_pages = max_pages; a.num_pages = num_pages; a.page_size = page_size;
  a.ps_shift = log2_exact(page_size);
  a.S = S;
  a.part_len = ((chunks + S - 1) / S) * kChunk;
  // FP8 pools: scores use the codes, so k_scale folds into the softmax scale and
  // v_scale into the final normalisation
  a.scale_log2 = softmax_scale * (fp8 ? k_scale : 1.f) * 1.4426950408889634f;
  a.kv_fp8 = fp8 ? 1 : 0;
  a.v_scale = fp8 ? v_scale : 1.f;
  a.window = window;
  a.alibi = alibi;
  a.key_lo = key_lo;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.block_map = block_map;
  a.bm_kb = bm_kb;
  return PA_OK;
}


// Checks and launch shared by the bf16 and FP8 page writes.
int kv_write_impl(const char* what, void* k_pool, void* v_pool, const void* k_new,
                  const void* v_new, const int32_t* cu_new, const int32_t* start_pos,
                  const int32_t* block_tables, int32_t B, int32_t T, int32_t max_pages,
                  int32_t num_pages, int32_t page_size, int32_t Hkv, int32_t D, bool fp8,
                  float k_scale, float v_scale, void* stream, const float* k_scales = nullptr,
                  const float* v_scales = nullptr) {
  g_last_error[0] = 0;
  if (B < 0 || T < 0) return fail(PA_ERR_SHAPE, "%s: B=%d T=%d must be >= 0", what, B, T);
  int st0 = page_scales_ok(what, fp8, k_scales, v_scales);
  if (st0) return st0;
  if (k_scales) k_scale = v_scale = 1.f;
  if (fp8 && !scales_ok(k_scale, v_scale))
    return fail(PA_ERR_SHAPE, "%s: k_scale and v_scale must be positive and finite", what);
  if (B == 0 || T == 0) {
    snprintf(g_last_launch, sizeof(g_last_launch), "%s: nothing to do", what);
    return PA_OK;
  }
  int st = check_pool(B, max_pages, num_pages, page_size, Hkv, Hkv, D);
  if (st) return st;
  if (!k_pool || !v_pool || !k_new || !v_new || !cu_new || !start_pos || !block_tables)
    return fail(PA_ERR_NULL, "%s: a required pointer is NULL", what);
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PA_ERR_MISALIGNED, "%s: data pointers must be 16-byte aligned", what);
  pa::KvWriteArgs a{};
  a.k_pool = static_cast<uint16_t*>(k_pool);
  a.v_pool = static_cast<uint16_t*>(v_pool);
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.cu_new = cu_new;
  a.start_pos = start_pos;
  a.block_tables = block_tables;
  a.B = B; a.T = T; a.max_pages = max_pages; a.num_pages = num_pages;
  a.page_size = page_size; a.ps_shift = log2_exact(page_size); a.Hkv = Hkv; a.D = D;
  a.fp8 = fp8 ? 1 : 0;
  // the reciprocal is taken once, in float32, as the quantiser's definition does
  a.k_inv = fp8 ? 1.0f / k_scale : 1.f;
  a.v_inv = fp8 ? 1.0f / v_scale : 1.f;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  hipError_t e = pa::launch_kv_write(a, static_cast<hipStream_t>(stream), g_last_launch,
                                     sizeof(g_last_launch));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "%s launch: %s", what, hipGetErrorString(e));
  return PA_OK;
}

// Checks, workspace carving and the partition + reduce launches shared by the
// bf16 and FP8 decode entry points.
int decode_impl(const char* what, void* out, float* lse_out, const void* q, const void* k_pool,
                const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                int32_t B, int32_t max_pages, int32_t num_pages, int32_t page_size, int32_t Hq,
                int32_t Hkv, int32_t D, float softmax_scale, int32_t max_seq_len,
                int32_t num_splits, void* workspace, size_t workspace_bytes, bool fp8,
                float k_scale, float v_scale, void* stream, int32_t window = 0,
                const float* alibi = nullptr, const pa::KernelEvents& ev = pa::KernelEvents(),
                const int32_t* key_lo = nullptr, const float* k_scales = nullptr,
                const float* v_scales = nullptr, const uint8_t* block_map = nullptr,
                int32_t bm_kb = 0) {
  g_last_error[0] = 0;
  pa::DecodeArgs a;
  int st = decode_args(a, what, q, k_pool, v_pool, block_tables, seq_lens, B, max_pages,
                       num_pages, page_size, Hq, Hkv, D, softmax_scale, max_seq_len,
                       num_splits, fp8, k_scale, v_scale, window, alibi, key_lo, k_scales,
                       v_scales, block_map, bm_kb);
  if (st) return st;
  if (B == 0) {
    snprintf(g_last_launch, sizeof(g_last_launch), "%s: nothing to do", what);
    return PA_OK;
  }
  if (!out) return fail(PA_ERR_NULL, "%s: out is NULL", what);
  if (!aligned16(out)) return fail(PA_ERR_MISALIGNED, "%s: out must be 16-byte aligned", what);
  const int32_t S = a.S;
  const size_t need = workspace_for(B, Hq, D, S);
  if (need && (!workspace || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed for %d splits, got %zu",
                what, need, S, workspace ? workspace_bytes : (size_t)0);
  if (need && !aligned16(workspace))
    return fail(PA_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", what);
  a.out = static_cast<uint16_t*>(out);
  a.lse_out = lse_out;
  const size_t rows = (size_t)B * Hq * S;
  if (S > 1) {
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_lse = reinterpret_cast<float*>(ws + align256(rows * D * sizeof(float)));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char d1[256], d2[256];
  hipError_t e = pa::launch_decode(a, s, d1, sizeof(d1), ev);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "%s launch: %s", what, hipGetErrorString(e));
  if (S > 1) {
    pa::ReduceArgs r{};
    r.out = a.out; r.lse_out = lse_out; r.part_o = a.part_o; r.part_lse = a.part_lse;
    r.R = B * Hq; r.S = S; r.D = D;
    e = pa::launch_reduce(r, s, d2, sizeof(d2));
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "reduce launch: %s", hipGetErrorString(e));
    snprintf(g_last_launch, sizeof(g_last_launch), "%s; %s", d1, d2);
  } else {
    snprintf(g_last_launch, sizeof(g_last_launch), "%s", d1);
  }
  return PA_OK;
}

constexpr int32_t kPrefillMaxSplits = 16;      // the merge kernel's part limit
constexpr int kPrefillPartMinTiles = 16;       // 64-key tiles per key-range part at least

// Key-range parts per prefill query tile when the caller passes num_splits <= 0:
// none while the launch fills every work-group slot of the chip (256 CUs; one
// 8-wave or two 4-wave work-groups per CU) -- measured on MI355X, splitting a
// launch that already fills the chip gains less than the partial-result traffic
// and the merge cost -- else enough parts for one work-group per slot, at most 8.
// (The slot count takes the work-group size from max_q_len alone, as the workspace
// query does, so both give the same S; FP8 pools with ALiBi launch 8-wave work-groups
// whatever the length, for which the count is then only an estimate.)
// (waves > 0: work-groups of that many waves, as the mixed step's 8.)
int32_t resolve_prefill_splits(int32_t B, int32_t Hq, int32_t max_q_len, int32_t num_splits,
                               int waves = 0) {
  if (num_splits > 0) return num_splits < kPrefillMaxSplits ? num_splits : kPrefillMaxSplits;
  if (B <= 0 || Hq <= 0 || max_q_len <= 0) return 1;
  const int W = waves > 0 ? waves : pa::prefill_waves(max_q_len);
  const long long n_qt = (max_q_len + 32 * W - 1) / (32 * W);
  const long long wgs = (long long)Hq * B * n_qt;
  const long long slots = 256ll * (8 / W);
  if (wgs >= slots) return 1;
  const long long s = (slots + wgs - 1) / wgs;
  return (int32_t)(s < 8 ? s : 8);
}

// Key-split workspace: fp32 partial outputs [Tq * Hq, S, D], then fp32 partial lse
// [Tq * Hq, S].
size_t prefill_workspace_for(int32_t Tq, int32_t Hq, int32_t D, int32_t S) {
  if (S <= 1 || Tq <= 0) return 0;
  const size_t rows = (size_t)Tq * Hq * S;
  return align256(rows * D * sizeof(float)) + align256(rows * sizeof(float));
}

// Checks and argument packing shared by the prefill entry points and the mixed step
// (waves > 0: work-groups of that many waves, for the key-part count); the key parts
// S are resolved (1: the plain one-pass prefill) and their workspace checked.  With no
// query row to compute, *nothing is set and a is left empty.
int prefill_args(pa::PrefillArgs& a, bool* nothing, const char* what, void* out,
                 float* lse_out, const void* q, const void* k_pool, const void* v_pool,
                 const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                 const int32_t* block_tables, int32_t B, int32_t Tq, int32_t max_q_len,
                 int32_t max_pages, int32_t num_pages, int32_t page_size, int32_t Hq,
                 int32_t Hkv, int32_t D, float softmax_scale, int32_t causal, int32_t num_splits,
                 void* workspace, size_t workspace_bytes, int32_t window = 0,
                 const float* alibi = nullptr, bool fp8 = false, float k_scale = 1.f,
                 float v_scale = 1.f, const int32_t* key_lo = nullptr,
                 const int32_t* key_hi = nullptr, const float* k_scales = nullptr,
                 const float* v_scales = nullptr, int32_t persistent = 0,
                 const uint8_t* block_map = nullptr, int32_t bm_qb = 0, int32_t bm_kb = 0,
                 int waves = 0) {
  a = pa::PrefillArgs{};
  *nothing = false;
  if (B < 0 || Tq < 0 || max_q_len < 0 || window < 0)
    return fail(PA_ERR_SHAPE, "%s: B=%d Tq=%d max_q_len=%d window=%d", what, B, Tq, max_q_len,
                window);
  int st = check_pool(B, max_pages, num_pages, page_size, Hq, Hkv, D);
  if (st) return st;
  if (B == 0 || Tq == 0 || max_q_len == 0) {
    *nothing = true;
    return PA_OK;
  }
  if (!out || !q || !k_pool || !v_pool || !cu_seqlens_q || !seq_lens_k || !block_tables)
    return fail(PA_ERR_NULL, "%s: a required pointer is NULL", what);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PA_ERR_MISALIGNED, "%s: data pointers must be 16-byte aligned", what);
  if (!(softmax_scale > 0.f) || softmax_scale > 3.0e38f)
    return fail(PA_ERR_SHAPE, "%s: softmax scale must be positive and finite", what);
  if (alibi && (reinterpret_cast<uintptr_t>(alibi) & 3u))
    return fail(PA_ERR_MISALIGNED, "%s: alibi_slopes must be 4-byte aligned", what);
  if (!key_lo != !key_hi)
    return fail(PA_ERR_NULL, "%s: key_lo and key_hi must both be given or both be NULL", what);
  if ((key_lo && (reinterpret_cast<uintptr_t>(key_lo) & 3u)) ||
      (key_hi && (reinterpret_cast<uintptr_t>(key_hi) & 3u)))
    return fail(PA_ERR_MISALIGNED, "%s: key_lo and key_hi must be 4-byte aligned", what);
  st = page_scales_ok(what, fp8, k_scales, v_scales);
  if (st) return st;
  if (k_scales && alibi)
    return fail(PA_ERR_UNSUPPORTED, "%s: FP8 scales per page with ALiBi slopes are not "
                "supported in prefill", what);
  if (k_scales) k_scale = v_scale = 1.f;
  if (fp8 && !(scales_ok(k_scale, v_scale) && softmax_scale * k_scale <= 3.0e38f))
    return fail(PA_ERR_SHAPE, "%s: k_scale and v_scale must be positive and finite", what);
  if (block_map) {
    if (bm_qb < 1 || bm_kb < 1)
      return fail(PA_ERR_SHAPE, "%s: block map of %d x %d blocks per sequence", what, bm_qb,
                  bm_kb);
    if (num_splits > 1)
      return fail(PA_ERR_UNSUPPORTED, "%s: block maps take no key parts (num_splits %d)", what,
                  num_splits);
    if ((long long)max_pages * page_size > 262144)
      return fail(PA_ERR_UNSUPPORTED, "%s: block maps cover at most 262144 keys per sequence "
                  "(max_pages x page_size = %lld)", what, (long long)max_pages * page_size);
    num_splits = 1;
  }
  if (max_q_len > Tq) max_q_len = Tq;
  const int32_t S = resolve_prefill_splits(B, Hq, max_q_len, num_splits, waves);
  // one work-group per (query head, sequence, 128- or 256-row query tile, key
  // part); the launch holds at most 2^32 - 1 work-items
  if ((long long)Hq * B * ((max_q_len + 127) / 128 + 1) * 256 * S > 0xffffffffll)
    return fail(PA_ERR_SHAPE, "%s: %d heads x %d sequences x %d query rows x %d key parts is "
                "too many work-groups for one launch", what, Hq, B, max_q_len, S);
  const size_t need = prefill_workspace_for(Tq, Hq, D, S);
  if (need && (!workspace || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed for %d key parts, got %zu",
                what, need, S, workspace ? workspace_bytes : (size_t)0);
  if (need && !aligned16(workspace))
    return fail(PA_ERR_MISALIGNED, "%s: workspace must be 16-byte aligned", what);
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.cu_seqlens_q = cu_seqlens_q;
  a.seq_lens_k = seq_lens_k;
  a.block_tables = block_tables;
  a.out = static_cast<uint16_t*>(out);
  a.lse_out = lse_out;
  a.B = B; a.Tq = Tq; a.max_q_len = max_q_len; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.D = D;
  a.max_pages = max_pages; a.num_pages = num_pages; a.page_size = page_size;
  a.ps_shift = log2_exact(page_size);
  a.causal = causal ? 1 : 0;
  // FP8 pools: scores use the codes, so k_scale folds into the softmax scale and
  // v_scale into the final normalisation
  a.scale_log2 = softmax_scale * (fp8 ? k_scale : 1.f) * 1.4426950408889634f;
  a.window = window;
  a.alibi = alibi;
  a.kv_fp8 = fp8 ? 1 : 0;
  a.v_scale = fp8 ? v_scale : 1.f;
  a.key_lo = key_lo;
  a.key_hi = key_hi;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.persist = persistent ? 1 : 0;
  a.block_map = block_map;
  a.bm_qb = bm_qb;
  a.bm_kb = bm_kb;
  a.S = S;
  a.part_min = kPrefillPartMinTiles;
  if (S > 1) {
    char* ws = static_cast<char*>(workspace);
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_lse = reinterpret_cast<float*>(ws + align256((size_t)Tq * Hq * S * D * sizeof(float)));
  }
  return PA_OK;
}

// Checks and launches shared by the prefill entry points; S == 1 is the plain
// one-pass prefill.
int prefill_impl(const char* what, void* out, float* lse_out, const void* q, const void* k_pool,
                 const void* v_pool, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                 const int32_t* block_tables, int32_t B, int32_t Tq, int32_t max_q_len,
                 int32_t max_pages, int32_t num_pages, int32_t page_size, int32_t Hq,
                 int32_t Hkv, int32_t D, float softmax_scale, int32_t causal, int32_t num_splits,
                 void* workspace, size_t workspace_bytes, void* stream, int32_t window = 0,
                 const float* alibi = nullptr, bool fp8 = false, float k_scale = 1.f,
                 float v_scale = 1.f, const pa::KernelEvents& ev = pa::KernelEvents(),
                 const int32_t* key_lo = nullptr, const int32_t* key_hi = nullptr,
                 const float* k_scales = nullptr, const float* v_scales = nullptr,
                 int32_t persistent = 0, const uint8_t* block_map = nullptr,
                 int32_t bm_qb = 0, int32_t bm_kb = 0) {
  g_last_error[0] = 0;
  pa::PrefillArgs a;
  bool nothing = false;
  const int st = prefill_args(a, &nothing, what, out, lse_out, q, k_pool, v_pool, cu_seqlens_q,
                              seq_lens_k, block_tables, B, Tq, max_q_len, max_pages, num_pages,
                              page_size, Hq, Hkv, D, softmax_scale, causal, num_splits,
                              workspace, workspace_bytes, window, alibi, fp8, k_scale, v_scale,
                              key_lo, key_hi, k_scales, v_scales, persistent, block_map, bm_qb,
                              bm_kb);
  if (st) return st;
  if (nothing) {
    snprintf(g_last_launch, sizeof(g_last_launch), "%s: nothing to do", what);
    return PA_OK;
  }
  const int32_t S = a.S;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char d1[320], d2[256];
  hipError_t e = pa::launch_prefill(a, hs, d1, sizeof(d1), ev);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "%s launch: %s", what, hipGetErrorString(e));
  if (S > 1) {
    e = pa::launch_prefill_merge(a, hs, d2, sizeof(d2));
    if (e != hipSuccess)
      return fail(PA_ERR_LAUNCH, "%s merge launch: %s", what, hipGetErrorString(e));
    snprintf(g_last_launch, sizeof(g_last_launch), "%s; %s", d1, d2);
  } else {
    snprintf(g_last_launch, sizeof(g_last_launch), "%s", d1);
  }
  return PA_OK;
}

// Scratch of paged_attn_decode_noalloc: the split-K partials of callers that cannot
// allocate.  It lives in the library's code object, so every GPU the library runs
// on holds its own copy from the library's first use there until the process ends.
// In host code `scratch` only stands for the device array: its address on the
// current device comes from hipGetSymbolAddress, taken once per device and kept.
constexpr size_t kNoallocScratchBytes = PA_DECODE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up on the first call on each
// device); PA_OK or a failure status with the reason recorded.
int scratch_on_current_device(const char* what, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(PA_ERR_UNSUPPORTED, "%s: device %d beyond the %d devices with scratch", what, dev,
                kMaxScratchDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(PA_ERR_LAUNCH, "%s: hipGetSymbolAddress(scratch) on device %d: %s", what, dev,
                    hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return PA_OK;
}

}  // namespace

// The caller's optional kernel-timing events of an options struct.
template <typename Opts>
static pa::KernelEvents events_of(const Opts* o) {
  pa::KernelEvents ev;
  ev.start = static_cast<hipEvent_t>(o->kernel_start_event);
  ev.stop = static_cast<hipEvent_t>(o->kernel_stop_event);
  return ev;
}

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_MISALIGNED: return "PA_ERR_MISALIGNED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH";
    default: return "PA_ERR_UNKNOWN";
  }
}

const char* pa_last_error(void) { return g_last_error; }
const char* pa_describe_launch(void) { return g_last_launch; }

int kv_page_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                  const int32_t* cu_new, const int32_t* start_pos,
                  const int32_t* block_tables, int32_t B, int32_t T, int32_t max_pages,
                  int32_t num_pages, int32_t page_size, int32_t Hkv, int32_t D,
                  void* stream) {
  return kv_write_impl("kv_page_write", k_pool, v_pool, k_new, v_new, cu_new, start_pos,
                       block_tables, B, T, max_pages, num_pages, page_size, Hkv, D, false, 1.f,
                       1.f, stream);
}

int kv_page_write_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                      const int32_t* cu_new, const int32_t* start_pos,
                      const int32_t* block_tables, int32_t B, int32_t T, int32_t max_pages,
                      int32_t num_pages, int32_t page_size, int32_t Hkv, int32_t D,
                      float k_scale, float v_scale, void* stream) {
  return kv_write_impl("kv_page_write_fp8", k_pool, v_pool, k_new, v_new, cu_new, start_pos,
                       block_tables, B, T, max_pages, num_pages, page_size, Hkv, D, true,
                       k_scale, v_scale, stream);
}

int kv_page_write_fp8_scales(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                             const int32_t* cu_new, const int32_t* start_pos,
                             const int32_t* block_tables, int32_t B, int32_t T,
                             int32_t max_pages, int32_t num_pages, int32_t page_size, int32_t Hkv,
                             int32_t D, const float* k_scales, const float* v_scales,
                             void* stream) {
  if (!k_scales || !v_scales)
    return fail(PA_ERR_NULL, "kv_page_write_fp8_scales: k_scales and v_scales are required");
  return kv_write_impl("kv_page_write_fp8_scales", k_pool, v_pool, k_new, v_new, cu_new,
                       start_pos, block_tables, B, T, max_pages, num_pages, page_size, Hkv, D,
                       true, 1.f, 1.f, stream, k_scales, v_scales);
}

int paged_attn_decode(void* out, float* lse_out, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_tables,
                      const int32_t* seq_lens, int32_t B, int32_t max_pages,
                      int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv,
                      int32_t D, float softmax_scale, int32_t max_seq_len,
                      int32_t num_splits, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return decode_impl("decode", out, lse_out, q, k_pool, v_pool, block_tables, seq_lens, B,
                     max_pages, num_pages, page_size, Hq, Hkv, D, softmax_scale, max_seq_len,
                     num_splits, workspace, workspace_bytes, false, 1.f, 1.f, stream);
}

int paged_attn_decode_fp8(void* out, float* lse_out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables,
                          const int32_t* seq_lens, int32_t B, int32_t max_pages,
                          int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv,
                          int32_t D, float softmax_scale, float k_scale, float v_scale,
                          int32_t max_seq_len, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, void* stream) {
  return decode_impl("decode_fp8", out, lse_out, q, k_pool, v_pool, block_tables, seq_lens, B,
                     max_pages, num_pages, page_size, Hq, Hkv, D, softmax_scale, max_seq_len,
                     num_splits, workspace, workspace_bytes, true, k_scale, v_scale, stream);
}

int32_t paged_attn_decode_num_splits(int32_t B, int32_t Hkv, int32_t max_seq_len) {
  return resolve_splits(B, Hkv > 0 ? Hkv : 1, max_seq_len, 0);
}

size_t paged_attn_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                         int32_t max_seq_len, int32_t num_splits) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return 0;
  return workspace_for(B, Hq, D, resolve_splits(B, Hkv, max_seq_len, num_splits));
}

int paged_attn_splitk_reduce(void* out, float* lse_out, const float* partial_out,
                             const float* partial_lse, int32_t R, int32_t S, int32_t D,
                             void* stream) {
  g_last_error[0] = 0;
  if (R < 0 || S < 1) return fail(PA_ERR_SHAPE, "splitk_reduce: R=%d S=%d", R, S);
  if (!head_dim_ok(D)) return fail(PA_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", D);
  if (R == 0) {
    snprintf(g_last_launch, sizeof(g_last_launch), "splitk_reduce: nothing to do");
    return PA_OK;
  }
  if (!out || !partial_out || !partial_lse)
    return fail(PA_ERR_NULL, "splitk_reduce: a required pointer is NULL");
  if (!aligned16(out) || !aligned16(partial_out))
    return fail(PA_ERR_MISALIGNED, "splitk_reduce: data pointers must be 16-byte aligned");
  pa::ReduceArgs r{};
  r.out = static_cast<uint16_t*>(out);
  r.lse_out = lse_out;
  r.part_o = partial_out;
  r.part_lse = partial_lse;
  r.R = R; r.S = S; r.D = D;
  hipError_t e = pa::launch_reduce(r, static_cast<hipStream_t>(stream), g_last_launch,
                                   sizeof(g_last_launch));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "splitk_reduce launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int paged_attn_decode_noalloc(void* out, float* lse_out, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_tables,
                              const int32_t* seq_lens, int32_t B, int32_t max_pages,
                              int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv,
                              int32_t D, float softmax_scale, int32_t max_seq_len,
                              int32_t num_splits, void* stream) {
  g_last_error[0] = 0;
  // the same checks and split resolution as paged_attn_decode, then the size rule,
  // all on the host before the device is touched
  pa::DecodeArgs a;
  int st = decode_args(a, "decode_noalloc", q, k_pool, v_pool, block_tables, seq_lens, B,
                       max_pages, num_pages, page_size, Hq, Hkv, D, softmax_scale, max_seq_len,
                       num_splits);
  if (st) return st;
  const size_t need = workspace_for(B, Hq, D, a.S);
  if (need > kNoallocScratchBytes)
    return fail(PA_ERR_WORKSPACE, "decode_noalloc: %d splits need %zu bytes of partials, more "
                "than the library's %zu-byte scratch (use fewer splits, or paged_attn_decode "
                "with a workspace)", a.S, need, kNoallocScratchBytes);
  void* ws = nullptr;
  if (need && B > 0) {
    st = scratch_on_current_device("decode_noalloc", &ws);
    if (st) return st;
  }
  return decode_impl("decode_noalloc", out, lse_out, q, k_pool, v_pool, block_tables, seq_lens,
                     B, max_pages, num_pages, page_size, Hq, Hkv, D, softmax_scale, max_seq_len,
                     num_splits, ws, ws ? kNoallocScratchBytes : 0, false, 1.f, 1.f, stream);
}

int paged_attn_decode_partials(float* partial_out, float* partial_lse, const void* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t B, int32_t max_pages, int32_t num_pages,
                               int32_t page_size, int32_t Hq, int32_t Hkv, int32_t D,
                               float softmax_scale, int32_t max_seq_len, int32_t num_splits,
                               void* stream) {
  g_last_error[0] = 0;
  pa::DecodeArgs a;
  if (num_splits < 1) return fail(PA_ERR_SHAPE, "decode_partials: num_splits=%d < 1", num_splits);
  int st = decode_args(a, "decode_partials", q, k_pool, v_pool, block_tables, seq_lens, B,
                       max_pages, num_pages, page_size, Hq, Hkv, D, softmax_scale, max_seq_len,
                       num_splits);
  if (st) return st;
  if (a.S != num_splits)
    return fail(PA_ERR_SHAPE, "decode_partials: %d splits exceed the %d 32-key chunks of max_seq_len",
                num_splits, a.S);
  if (B == 0) {
    snprintf(g_last_launch, sizeof(g_last_launch), "decode_partials: nothing to do");
    return PA_OK;
  }
  if (!partial_out || !partial_lse) return fail(PA_ERR_NULL, "decode_partials: NULL partials");
  if (!aligned16(partial_out))
    return fail(PA_ERR_MISALIGNED, "decode_partials: partial_out must be 16-byte aligned");
  // the partition kernel writes partials whenever S > 1; with S == 1 route the
  // single partition through the same path by presenting it as split 0 of 1
  a.part_o = partial_out;
  a.part_lse = partial_lse;
  a.force_partials = 1;
  hipError_t e = pa::launch_decode(a, static_cast<hipStream_t>(stream), g_last_launch,
                                   sizeof(g_last_launch));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "decode_partials launch: %s", hipGetErrorString(e));
  return PA_OK;
}

int paged_attn_prefill_varlen(void* out, float* lse_out, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* cu_seqlens_q,
                              const int32_t* seq_lens_k, const int32_t* block_tables,
                              int32_t B, int32_t Tq, int32_t max_q_len, int32_t max_pages,
                              int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv,
                              int32_t D, float softmax_scale, int32_t causal, void* stream) {
  return prefill_impl("prefill", out, lse_out, q, k_pool, v_pool, cu_seqlens_q, seq_lens_k,
                      block_tables, B, Tq, max_q_len, max_pages, num_pages, page_size, Hq, Hkv,
                      D, softmax_scale, causal, 1, nullptr, 0, stream);
}

int32_t paged_attn_prefill_num_splits(int32_t B, int32_t Hq, int32_t max_q_len) {
  return resolve_prefill_splits(B, Hq, max_q_len, 0);
}

// Host planning of the key-part count from the lengths themselves.  Each query tile
// is counted in 64-key tiles exactly as the kernel bounds it (causal limit, window
// start) and cut into parts exactly as the kernel cuts it.  A launch lasts at least
// its heaviest piece and at least the mean load per work-group slot, so the count
// starts at ceil(heaviest / mean) (less 5 % of slack for rounding); from there up to
// 8 each count is priced by list-scheduling its work-groups heaviest-first onto the
// slots (the grid's own order), each work-group charged kPlanWgTiles for its start
// and drain and the launch kPlanMergeTiles for the merge when anything is cut.  The
// cheapest count wins, the smallest within 3 % of it.
constexpr long long kPlanWgTiles = 2;
constexpr long long kPlanMergeTiles = 3;

static long long plan_makespan(const std::vector<long long>& tiles, int32_t Hq, int s,
                               long long slots, std::vector<long long>& jobs) {
  jobs.clear();
  bool cut = false;
  for (const long long t : tiles) {
    long long p = 1;
    if (s > 1) {
      p = t / kPrefillPartMinTiles;
      if (p > s) p = s;
      if (p < 1) p = 1;
    }
    cut |= p > 1;
    for (long long k = 0; k < p; ++k) {
      const long long len = (k + 1) * t / p - k * t / p + kPlanWgTiles;
      for (int32_t h = 0; h < Hq; ++h) jobs.push_back(len);
    }
  }
  std::sort(jobs.begin(), jobs.end(), std::greater<long long>());
  std::priority_queue<long long, std::vector<long long>, std::greater<long long>> load;
  for (long long i = 0; i < slots; ++i) load.push(0);
  long long span = 0;
  for (const long long j : jobs) {
    const long long x = load.top() + j;
    load.pop();
    load.push(x);
    if (x > span) span = x;
  }
  return span + (cut ? kPlanMergeTiles : 0);
}

int32_t paged_attn_prefill_plan_splits(int32_t B, const int32_t* q_lens, const int32_t* k_lens,
                                       int32_t Hq, int32_t causal, int32_t window_left) {
  g_last_error[0] = 0;
  if (B < 0 || Hq <= 0 || window_left < 0) {
    fail(PA_ERR_SHAPE, "prefill_plan_splits: B=%d Hq=%d window_left=%d", B, Hq, window_left);
    return 0;
  }
  if (B == 0) return 1;
  if (!q_lens || !k_lens) {
    fail(PA_ERR_NULL, "prefill_plan_splits: q_lens or k_lens is NULL");
    return 0;
  }
  int32_t max_q = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (q_lens[b] < 0 || k_lens[b] < 0) {
      fail(PA_ERR_SHAPE, "prefill_plan_splits: sequence %d has q_len %d, k_len %d", b,
           q_lens[b], k_lens[b]);
      return 0;
    }
    if (q_lens[b] > max_q) max_q = q_lens[b];
  }
  if (max_q == 0) return 1;
  const int W = pa::prefill_waves(max_q);
  const int bm = 32 * W;
  std::vector<long long> tiles;
  long long total = 0, heavy = 0;
  for (int32_t b = 0; b < B; ++b) {
    const long long q = q_lens[b], L = k_lens[b];
    for (long long r0 = 0; r0 < q; r0 += bm) {
      const long long rows = q - r0 < bm ? q - r0 : bm;
      long long k_lim = L;
      if (causal) {
        const long long lim = L - q + r0 + rows;
        k_lim = lim < 0 ? 0 : (lim < L ? lim : L);
      }
      const long long n = (k_lim + 63) / 64;
      long long first = 0;
      if (window_left > 0) {
        const long long lo = L - q + r0 - window_left + 1;
        first = lo > 0 ? lo / 64 : 0;
        if (first > n) first = n;
      }
      tiles.push_back(n - first);
      total += n - first;
      if (n - first > heavy) heavy = n - first;
    }
  }
  const long long slots = 256ll * (8 / W);
  // r = heaviest / mean = heavy * slots / work; the count starts at ceil(r - 0.05)
  const long long work = total * Hq;
  if (heavy < 2 * kPrefillPartMinTiles || heavy * slots <= work) return 1;
  long long s_lo = (heavy * slots * 20 - work + work * 20 - 1) / (work * 20);
  if (s_lo < 1) s_lo = 1;
  if (s_lo > 8) return 8;
  // a grid this large is priced by the bound alone
  if ((long long)tiles.size() * Hq > (1ll << 14)) return (int32_t)s_lo;
  std::vector<long long> jobs;
  long long cost[9] = {0};
  long long best = -1;
  for (long long s = s_lo; s <= 8; ++s) {
    cost[s] = plan_makespan(tiles, Hq, (int)s, slots, jobs);
    if (best < 0 || cost[s] < best) best = cost[s];
  }
  for (long long s = s_lo; s <= 8; ++s)
    if (cost[s] * 100 <= best * 103) return (int32_t)s;
  return 8;
}

size_t paged_attn_prefill_workspace_bytes(int32_t B, int32_t Tq, int32_t max_q_len, int32_t Hq,
                                          int32_t D, int32_t num_splits) {
  if (B <= 0 || Tq <= 0 || max_q_len <= 0 || Hq <= 0 || D <= 0) return 0;
  if (max_q_len > Tq) max_q_len = Tq;
  return prefill_workspace_for(Tq, Hq, D, resolve_prefill_splits(B, Hq, max_q_len, num_splits));
}

int paged_attn_prefill_varlen_splitk(void* out, float* lse_out, const void* q,
                                     const void* k_pool, const void* v_pool,
                                     const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                     const int32_t* block_tables, int32_t B, int32_t Tq,
                                     int32_t max_q_len, int32_t max_pages, int32_t num_pages,
                                     int32_t page_size, int32_t Hq, int32_t Hkv, int32_t D,
                                     float softmax_scale, int32_t causal, int32_t num_splits,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl("prefill_splitk", out, lse_out, q, k_pool, v_pool, cu_seqlens_q,
                      seq_lens_k, block_tables, B, Tq, max_q_len, max_pages, num_pages,
                      page_size, Hq, Hkv, D, softmax_scale, causal, num_splits, workspace,
                      workspace_bytes, stream);
}

int paged_attn_decode_ex(void* out, float* lse_out, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_tables,
                         const int32_t* seq_lens, int32_t B, int32_t max_pages,
                         int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv,
                         int32_t D, float softmax_scale, int32_t max_seq_len,
                         const pa_decode_opts* opts, void* workspace, size_t workspace_bytes,
                         void* stream) {
  g_last_error[0] = 0;
  if (!opts) return fail(PA_ERR_NULL, "decode_ex: opts is NULL");
  if (opts->kv_fp8 != 0 && opts->kv_fp8 != 1)
    return fail(PA_ERR_UNSUPPORTED, "decode_ex: kv_fp8=%d", opts->kv_fp8);
  return decode_impl("decode_ex", out, lse_out, q, k_pool, v_pool, block_tables, seq_lens, B,
                     max_pages, num_pages, page_size, Hq, Hkv, D, softmax_scale, max_seq_len,
                     opts->num_splits, workspace, workspace_bytes, opts->kv_fp8 == 1,
                     opts->kv_fp8 ? opts->k_scale : 1.f, opts->kv_fp8 ? opts->v_scale : 1.f,
                     stream, opts->window_left, opts->alibi_slopes, events_of(opts),
                     opts->key_lo, opts->k_scales, opts->v_scales, opts->block_map,
                     opts->block_map_k_blocks);
}

size_t paged_attn_decode_ex_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                            int32_t max_seq_len, const pa_decode_opts* opts) {
  if (!opts || B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || opts->window_left < 0) return 0;
  const int32_t len = effective_len(max_seq_len, opts->window_left);
  return workspace_for(B, Hq, D, resolve_splits(B, Hkv, len, opts->num_splits));
}

int paged_attn_prefill_ex(void* out, float* lse_out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* cu_seqlens_q,
                          const int32_t* seq_lens_k, const int32_t* block_tables, int32_t B,
                          int32_t Tq, int32_t max_q_len, int32_t max_pages, int32_t num_pages,
                          int32_t page_size, int32_t Hq, int32_t Hkv, int32_t D,
                          float softmax_scale, const pa_prefill_opts* opts, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  if (!opts) return fail(PA_ERR_NULL, "prefill_ex: opts is NULL");
  if (opts->kv_fp8 != 0 && opts->kv_fp8 != 1)
    return fail(PA_ERR_UNSUPPORTED, "prefill_ex: kv_fp8=%d", opts->kv_fp8);
  return prefill_impl("prefill_ex", out, lse_out, q, k_pool, v_pool, cu_seqlens_q, seq_lens_k,
                      block_tables, B, Tq, max_q_len, max_pages, num_pages, page_size, Hq, Hkv,
                      D, softmax_scale, opts->causal, opts->num_splits, workspace,
                      workspace_bytes, stream, opts->window_left, opts->alibi_slopes,
                      opts->kv_fp8 == 1, opts->k_scale, opts->v_scale, events_of(opts),
                      opts->key_lo, opts->key_hi, opts->k_scales, opts->v_scales,
                      opts->persistent, opts->block_map, opts->block_map_q_blocks,
                      opts->block_map_k_blocks);
}

// The mixed step's parts: the prefill's key-part count for 256-row work-groups, and
// the workspace regions of both parts.
static int32_t mixed_prefill_splits(const pa_mixed_prefill& p, int32_t Hq) {
  const int32_t mq = p.max_q_len < p.Tq ? p.max_q_len : p.Tq;
  return resolve_prefill_splits(p.B, Hq, mq, p.num_splits, 8);
}

// The decode part's split count: the caller's, or (num_splits <= 0) the larger of two
// counts.  (1) The decode's own count times the waves per work-group its own launch
// would give each item: every item of the mixed launch is walked by one wave, so each
// wave keeps the run of keys it would stream in paged_attn_decode (measured on MI355X,
// the mixed ragged step: 116.5-120.7 us with 4 splits, 152.5-154.5 us with the
// decode's own 2, whose one-wave items of 1,760 keys then outlast the prefill).
// (2) Enough items for the CUs the prefill's work-groups leave: eight items (one
// work-group) per CU of MI355X's 256 beyond the prefill's work-group count, partitions
// kept at 8 chunks or more -- a work-group holds eight items on one CU, so a decode
// alone with (1)'s count read its KV through a quarter of the CUs (32 x 8192 keys, Hq 28
// / Hkv 4: 166.5 us with 64 work-groups, 93.4 us with 256, against 85.4 us for
// paged_attn_decode).  prefill_wgs: the prefill part's work-groups.
static int32_t mixed_decode_splits(const pa_mixed_decode& d, int32_t Hkv, bool fp8,
                                   long long prefill_wgs) {
  if (d.num_splits > 0) return d.num_splits;
  const int32_t s0 = resolve_splits(d.B, Hkv, d.max_seq_len, 0);
  const int w = pa::decode_waves((long long)Hkv * s0 * (d.B > 0 ? d.B : 1), fp8);
  long long s = (long long)s0 * w;
  const long long free_cus = 256 - prefill_wgs;
  if (free_cus > 0 && d.B > 0) {
    const long long groups = (long long)d.B * Hkv;
    const int32_t chunks = d.max_seq_len > 0 ? (d.max_seq_len + kChunk - 1) / kChunk : 1;
    long long spread = (8 * free_cus + groups - 1) / groups;
    const long long cap = chunks / 8 > 0 ? chunks / 8 : 1;
    if (spread > cap) spread = cap;
    if (spread > s) s = spread;
  }
  return resolve_splits(d.B, Hkv, d.max_seq_len, (int32_t)(s < kMaxSplits ? s : kMaxSplits));
}

// Work-groups of the mixed launch's prefill part, from the host scalars the split
// count and the grid depend on.
static long long mixed_prefill_wgs(const pa_mixed_prefill& p, int32_t Hq, int32_t Hkv) {
  if (p.B <= 0 || p.Tq <= 0 || p.max_q_len <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return 0;
  pa::PrefillArgs a{};
  a.B = p.B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.max_q_len = p.max_q_len < p.Tq ? p.max_q_len : p.Tq;
  a.S = mixed_prefill_splits(p, Hq);
  return pa::mixed_prefill_items(a);
}

static size_t mixed_prefill_bytes(const pa_mixed_prefill& p, int32_t Hq, int32_t D) {
  if (p.B <= 0 || p.Tq <= 0 || p.max_q_len <= 0) return 0;
  return prefill_workspace_for(p.Tq, Hq, D, mixed_prefill_splits(p, Hq));
}

size_t paged_attn_mixed_workspace_bytes(const pa_mixed_prefill* prefill,
                                        const pa_mixed_decode* decode, const pa_mixed_fp8* fp8,
                                        int32_t Hq, int32_t Hkv, int32_t D) {
  if (!prefill || !decode || Hq <= 0 || Hkv <= 0 || D <= 0) return 0;
  const size_t pf = mixed_prefill_bytes(*prefill, Hq, D);
  const size_t dec =
      decode->B > 0 && decode->max_seq_len >= 0
          ? workspace_for(decode->B, Hq, D,
                          mixed_decode_splits(*decode, Hkv, fp8 != nullptr,
                                              mixed_prefill_wgs(*prefill, Hq, Hkv)))
          : 0;
  return pf + dec;
}

int paged_attn_mixed(const pa_mixed_prefill* prefill, const pa_mixed_decode* decode,
                     const pa_mixed_fp8* fp8, const void* k_pool, const void* v_pool,
                     int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv, int32_t D,
                     float softmax_scale, void* workspace, size_t workspace_bytes,
                     void* stream) {
  g_last_error[0] = 0;
  if (!prefill || !decode) return fail(PA_ERR_NULL, "mixed: prefill or decode is NULL");
  const pa_mixed_prefill& p = *prefill;
  const pa_mixed_decode& dc = *decode;
  // FP8 pools: the scales of both parts (checked by each part's own checks below)
  const bool f8 = fp8 != nullptr;
  const float ks = f8 ? fp8->k_scale : 1.f, vs = f8 ? fp8->v_scale : 1.f;
  const float* kss = f8 ? fp8->k_scales : nullptr;
  const float* vss = f8 ? fp8->v_scales : nullptr;
  // the prefill's partials come first in the workspace, the decode's after them; a
  // part with B == 0 is not checked
  const size_t pf_need = Hq > 0 && D > 0 ? mixed_prefill_bytes(p, Hq, D) : 0;
  pa::PrefillArgs a{};
  if (p.B != 0) {
    bool no_prefill = false;
    const int st = prefill_args(a, &no_prefill, "mixed (prefill part)", p.out, p.lse_out, p.q,
                                k_pool, v_pool, p.cu_seqlens_q, p.seq_lens_k, p.block_tables,
                                p.B, p.Tq, p.max_q_len, p.max_pages, num_pages, page_size, Hq,
                                Hkv, D, softmax_scale, p.causal, p.num_splits, workspace,
                                workspace_bytes < pf_need ? workspace_bytes : pf_need, 0,
                                nullptr, f8, ks, vs, nullptr, nullptr, kss, vss, 0, nullptr, 0,
                                0, 8);
    if (st) return st;
    if (no_prefill) a = pa::PrefillArgs{};
  }
  pa::DecodeArgs d{};
  if (dc.B != 0) {
    const int st = decode_args(d, "mixed (decode part)", dc.q, k_pool, v_pool, dc.block_tables,
                               dc.seq_lens, dc.B, dc.max_pages, num_pages, page_size, Hq, Hkv,
                               D, softmax_scale, dc.max_seq_len,
                               dc.max_seq_len >= 0
                                   ? mixed_decode_splits(dc, Hkv, f8,
                                                         a.B > 0 ? pa::mixed_prefill_items(a) : 0)
                                   : 0,
                               f8,
                               ks, vs, 0, nullptr, nullptr, kss, vss);
    if (st) return st;
    if (!dc.out) return fail(PA_ERR_NULL, "mixed (decode part): out is NULL");
    if (!aligned16(dc.out))
      return fail(PA_ERR_MISALIGNED, "mixed (decode part): out must be 16-byte aligned");
    const size_t need = workspace_for(dc.B, Hq, D, d.S);
    char* ws = workspace ? static_cast<char*>(workspace) + pf_need : nullptr;
    const size_t have = workspace_bytes > pf_need ? workspace_bytes - pf_need : 0;
    if (need && (!workspace || have < need))
      return fail(PA_ERR_WORKSPACE, "mixed: workspace of %zu bytes needed (%zu prefill, %zu "
                  "decode for %d splits), got %zu", pf_need + need, pf_need, need, d.S,
                  workspace ? workspace_bytes : (size_t)0);
    if (need && !aligned16(workspace))
      return fail(PA_ERR_MISALIGNED, "mixed: workspace must be 16-byte aligned");
    d.out = static_cast<uint16_t*>(dc.out);
    d.lse_out = dc.lse_out;
    if (d.S > 1) {
      d.part_o = reinterpret_cast<float*>(ws);
      d.part_lse = reinterpret_cast<float*>(
          ws + align256((size_t)dc.B * Hq * d.S * D * sizeof(float)));
    }
  }
  if (a.B == 0 && d.B == 0) {
    snprintf(g_last_launch, sizeof(g_last_launch), "mixed: nothing to do");
    return PA_OK;
  }
  hipStream_t hs = static_cast<hipStream_t>(stream);
  char d1[400], d2[256] = "", d3[256] = "";
  hipError_t e = pa::launch_mixed(a, d, hs, d1, sizeof(d1));
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "mixed launch: %s", hipGetErrorString(e));
  if (a.B > 0 && a.S > 1) {
    e = pa::launch_prefill_merge(a, hs, d2, sizeof(d2), 8);
    if (e != hipSuccess)
      return fail(PA_ERR_LAUNCH, "mixed prefill merge launch: %s", hipGetErrorString(e));
  }
  if (d.B > 0 && d.S > 1) {
    pa::ReduceArgs r{};
    r.out = d.out; r.lse_out = d.lse_out; r.part_o = d.part_o; r.part_lse = d.part_lse;
    r.R = d.B * Hq; r.S = d.S; r.D = D;
    e = pa::launch_reduce(r, hs, d3, sizeof(d3));
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "mixed reduce launch: %s", hipGetErrorString(e));
  }
  snprintf(g_last_launch, sizeof(g_last_launch), "%s%s%s%s%s", d1, d2[0] ? "; " : "", d2,
           d3[0] ? "; " : "", d3);
  return PA_OK;
}

size_t paged_attn_prefill_ex_workspace_bytes(int32_t B, int32_t Tq, int32_t max_q_len,
                                             int32_t Hq, int32_t D,
                                             const pa_prefill_opts* opts) {
  if (!opts || opts->block_map) return 0;     // block maps take no key parts
  return paged_attn_prefill_workspace_bytes(B, Tq, max_q_len, Hq, D, opts->num_splits);
}

}  // extern "C"
