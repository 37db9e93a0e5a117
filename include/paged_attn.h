/*
 * paged_attn.h -- exact attention over a paged KV cache on AMD MI355X (gfx950).
 *
 * C ABI of libpaged_attn.so.  Every entry point takes plain device pointers and
 * sizes; the library never allocates, frees or synchronises, and enqueues all of
 * its work on the caller's HIP stream (`stream`, a hipStream_t passed as void*;
 * NULL means the default stream).
 *
 * Problem statement followed (the source pages, cited by title and section):
 *   - queries Q[tokens, Hq, D], key/value page pools [pages, page_size, Hkv, D],
 *     per-sequence block tables and lengths ("8. Kernels and Attention Backends",
 *     chapter intro and "Attention is an I/O problem": ragged sequences, KV blocks
 *     scattered through memory, KV state may be paged);
 *   - exact softmax attention softmax(scale * Q K^T + mask) V, computed tile by tile
 *     with an online softmax ("The Stack Below the Stack (Part 2)", section 2.1);
 *   - decode split along the KV length with a log-sum-exp merge (same page,
 *     section 2.2 "Flash-Decoding");
 *   - causal mask q_idx >= kv_idx (same page, section 5), in absolute positions;
 *   - eager KV page writeback ("Inside Ion", "IonAttention in One Paragraph").
 *
 * Common conventions
 *   - bf16 data (Q, K/V pools, new K/V, outputs), int32 indices, fp32 lse.
 *   - All tensors are dense and row-major in the order written; data pointers must
 *     be 16-byte aligned.
 *   - GQA: query head h reads KV head h / (Hq / Hkv).
 *   - softmax_scale must be positive and finite (PA_ERR_SHAPE otherwise).
 *   - lse outputs are natural-log log-sum-exps of the scaled visible scores.
 *   - A query row that sees no key (sequence length 0, or an empty causal window)
 *     yields O = 0 and lse = -inf, never NaN.
 *   - Supported envelope: D in {64, 128}; page_size in {16, 32, 64};
 *     Hq % Hkv == 0 and 1 <= Hq/Hkv <= 16.  Anything else returns
 *     PA_ERR_UNSUPPORTED and enqueues nothing: there is no fallback path.
 *   - A failing call enqueues nothing and leaves every output untouched.  A launch
 *     error reported by the runtime becomes PA_ERR_LAUNCH.  pa_last_error() gives
 *     a thread-local description of the last failure.
 *   - Device-resident metadata is a precondition, not checked on the device:
 *     block-table entries used must lie in [0, num_pages); a sequence's keys must
 *     fit its table row (seq_len <= max_pages * page_size); kv_page_write's
 *     destination slots must be distinct.  The kernels clamp page ids and table
 *     indices into range so that a violation reads or skips wrong-but-valid
 *     memory instead of faulting; results are then undefined.
 *   - The library keeps no state between calls except thread-local strings; calls
 *     on different streams may run concurrently unless they write the same memory.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL                       */
  PA_ERR_SHAPE = 2,       /* a size is negative or inconsistent               */
  PA_ERR_UNSUPPORTED = 3, /* outside the supported envelope (D, page size, GQA) */
  PA_ERR_MISALIGNED = 4,  /* a data pointer is not 16-byte aligned            */
  PA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required       */
  PA_ERR_LAUNCH = 6       /* the HIP runtime rejected a launch                */
} pa_status;

/*
 * kv_page_write -- place new tokens' keys and values into their pages.
 *
 * Eager KV writeback ("Inside Ion", "IonAttention in One Paragraph"; KV-cache
 * insertion in "The Stack Below the Stack (Part 2)", section 2.1).  New token t of
 * sequence b (cu_new[b] <= t < cu_new[b+1]) has logical position
 *   pos = start_pos[b] + (t - cu_new[b])
 * and is copied, all Hkv heads, bit for bit, to row pos % page_size of page
 * block_tables[b * max_pages + pos / page_size] in both pools.
 *
 *   k_pool, v_pool : [num_pages, page_size, Hkv, D] bf16, modified in place
 *   k_new, v_new   : [T, Hkv, D] bf16
 *   cu_new         : [B+1] int32 prefix sums of new tokens per sequence (cu_new[B] == T)
 *   start_pos      : [B] int32 logical position of each sequence's first new token
 *   block_tables   : [B, max_pages] int32
 * Tokens whose position falls outside the table row, or whose page id is outside
 * [0, num_pages), are skipped (precondition violation; see above).  T == 0 or
 * B == 0 is a no-op returning PA_OK.
 */
int kv_page_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                  const int32_t* cu_new, const int32_t* start_pos,
                  const int32_t* block_tables, int32_t B, int32_t T, int32_t max_pages,
                  int32_t num_pages, int32_t page_size, int32_t Hkv, int32_t D,
                  void* stream);

/*
 * FP8 key/value pages.
 *
 * Quantising the KV cache to FP8 at insertion is named as a fusion target and as
 * part of a serving recipe ("The Stack Below the Stack (Part 2)", section 2.1 and
 * its closing pointer to Part 3); the pages fix no format or scaling, so this
 * library defines them:
 *   - a code is one byte in the OCP 8-bit E4M3 ("fn") format: sign, 4 exponent
 *     bits with bias 7, 3 mantissa bits, subnormals, no infinities, largest
 *     finite magnitude 448, codes 0x7F/0xFF are NaN;
 *   - each pool has one float32 scale (k_scale for K, v_scale for V): code c
 *     stands for decode(c) * scale;
 *   - quantisation computes y = x * (1 / scale) in float32 (the reciprocal taken
 *     once, in float32), clamps y to [-448, 448] and rounds to the nearest E4M3
 *     value, ties to even.  NaN inputs give unspecified codes.
 * FP8 pools have the bf16 pools' shape [num_pages, page_size, Hkv, D], one byte
 * per element (uint8 storage), and the same 16-byte alignment rule.
 *
 * Finer scaling (the caller's choice): one float32 scale per (page, KV head),
 * arrays k_scales / v_scales of shape [num_pages, Hkv] on the device, owned by the
 * caller; a code of page p, head h stands for decode(c) * scales[p * Hkv + h], and a
 * token row is quantised with the scale of the page and head it lands in.  Scales
 * must be positive and finite (device data, not checked).  Decode and prefill fold
 * each page's key scale into the score multiplier of that page's keys and apply
 * each page's value scale to P before P V (the row sums stay unscaled), so the
 * per-pool k_scale / v_scale arguments are then ignored.
 */

/*
 * kv_page_write_fp8 -- kv_page_write with the quantisation fused in: token t's
 * keys are written as the E4M3 codes of k_new[t] under k_scale, its values under
 * v_scale, at the same place kv_page_write would put them.
 *
 *   k_pool, v_pool   : [num_pages, page_size, Hkv, D] uint8 E4M3 codes, modified in place
 *   k_new, v_new     : [T, Hkv, D] bf16
 *   k_scale, v_scale : positive finite float32 (PA_ERR_SHAPE otherwise)
 * Every other argument, precondition and status is kv_page_write's.
 */
int kv_page_write_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                      const int32_t* cu_new, const int32_t* start_pos,
                      const int32_t* block_tables, int32_t B, int32_t T, int32_t max_pages,
                      int32_t num_pages, int32_t page_size, int32_t Hkv, int32_t D,
                      float k_scale, float v_scale, void* stream);

/*
 * kv_page_write_fp8_scales -- kv_page_write_fp8 with scales per (page, KV head):
 * token t's head h is quantised under k_scales[page * Hkv + h] (keys) and
 * v_scales[page * Hkv + h] (values) of the page it is written to.
 *
 *   k_scales, v_scales : device [num_pages, Hkv] float32 (4-byte aligned), required
 * Every other argument, precondition and status is kv_page_write_fp8's.
 */
int kv_page_write_fp8_scales(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                             const int32_t* cu_new, const int32_t* start_pos,
                             const int32_t* block_tables, int32_t B, int32_t T,
                             int32_t max_pages, int32_t num_pages, int32_t page_size, int32_t Hkv,
                             int32_t D, const float* k_scales, const float* v_scales,
                             void* stream);

/*
 * paged_attn_decode_num_splits -- the split count paged_attn_decode uses when it is
 * passed num_splits <= 0: enough (sequence, KV head, split) work-groups to fill the
 * chip, each covering at least a few 32-key chunks ("The Stack Below the Stack
 * (Part 2)", section 2.2: decode has parallelism to spare only along the KV length).
 * Never more than the number of 32-key chunks of max_seq_len; at least 1.
 */
int32_t paged_attn_decode_num_splits(int32_t B, int32_t Hkv, int32_t max_seq_len);

/*
 * paged_attn_decode_workspace_bytes -- bytes of workspace paged_attn_decode needs for
 * this shape and split count (after resolving num_splits <= 0 as above): fp32
 * partial outputs [B, Hq, S, D] followed by fp32 partial lse [B, Hq, S], each region
 * 256-byte aligned.  0 when S == 1.  Split counts are capped at 65535.
 */
size_t paged_attn_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                         int32_t max_seq_len, int32_t num_splits);

/*
 * paged_attn_decode -- one query row per sequence against its paged KV history.
 *
 * out[b, h, :] = softmax(scale * q[b, h] . K_b^T) V_b over keys 0..seq_lens[b]-1
 * of sequence b, where K_b/V_b are gathered through block_tables row b
 * ("8. Kernels and Attention Backends", "Counting attention's traffic": decode is
 * bound by reading the whole history).  The keys are cut into S = num_splits
 * partitions of part_len = roundup(ceil(max_seq_len / S), 32) keys; each
 * partition's partial output and log-sum-exp go to the workspace and a second
 * kernel merges them exactly ("The Stack Below the Stack (Part 2)", section 2.2).
 * With S == 1 the first kernel writes out/lse_out directly and no workspace is used.
 * How partitions map to work-groups is the library's choice and does not change a
 * bit of the results: when B * Hkv * S is several times the number of one-wave
 * work-groups that stream HBM best on MI355X, each work-group walks up to 8
 * consecutive partitions of one (sequence, KV head) as one run of keys.
 *
 *   out       : [B, Hq, D] bf16                 lse_out : [B, Hq] fp32 or NULL
 *   q         : [B, Hq, D] bf16
 *   k_pool, v_pool : [num_pages, page_size, Hkv, D] bf16 (read only)
 *   block_tables   : [B, max_pages] int32       seq_lens : [B] int32 keys attended
 *   max_seq_len    : host-side upper bound of seq_lens (sizes the partitions; keys
 *                    past S * part_len are not attended)
 *   num_splits     : S, or <= 0 for paged_attn_decode_num_splits()
 *   workspace      : device buffer of at least paged_attn_decode_workspace_bytes()
 *                    (may be NULL when that is 0); contents are scratch.  Calls that
 *                    share a workspace must not run concurrently.
 */
int paged_attn_decode(void* out, float* lse_out, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_tables,
                      const int32_t* seq_lens, int32_t B, int32_t max_pages,
                      int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv,
                      int32_t D, float softmax_scale, int32_t max_seq_len,
                      int32_t num_splits, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The split-K partials go to a fixed scratch area inside the
 * library instead of a caller workspace; the call allocates nothing (no hipMalloc,
 * no hipFree, no allocating library routine) and records no memset.
 *
 *   - The scratch is PA_DECODE_NOALLOC_SCRATCH_BYTES (32 MiB) of device memory in
 *     the library's code object: each GPU the library runs on holds its own copy
 *     until the process ends.  Its address on a device is looked up on the first
 *     call on that device (make one call outside graph capture first).
 *   - Arguments, split resolution, results and statuses are paged_attn_decode's
 *     with no workspace.  When the resolved split count needs more partials than
 *     the scratch holds (paged_attn_decode_workspace_bytes above 32 MiB), the call
 *     returns PA_ERR_WORKSPACE and enqueues nothing.  The library's own split
 *     choice (num_splits <= 0) always fits.
 *   - Nothing in the scratch needs clearing: every call writes each partial it
 *     reads.  Every call on a GPU shares that GPU's scratch, so calls that overlap
 *     on one GPU (other streams, other threads) race and their results are
 *     undefined; calls in one stream are ordered and safe.
 */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)
int paged_attn_decode_noalloc(void* out, float* lse_out, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* block_tables,
                              const int32_t* seq_lens, int32_t B, int32_t max_pages,
                              int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv,
                              int32_t D, float softmax_scale, int32_t max_seq_len,
                              int32_t num_splits, void* stream);

/*
 * paged_attn_decode_fp8 -- paged_attn_decode over FP8 E4M3 pools (format above):
 * the attention of q against keys decode(k_code) * k_scale and values
 * decode(v_code) * v_scale.  The codes are widened to bf16 exactly on their way to
 * the same MFMA path; k_scale folds into the softmax scale and v_scale into the
 * final normalisation, so lse_out is the log-sum-exp of the scaled scores against
 * the dequantised keys.
 *
 *   k_pool, v_pool   : [num_pages, page_size, Hkv, D] uint8 E4M3 codes (read only)
 *   k_scale, v_scale : positive finite float32, with softmax_scale * k_scale finite
 *                      (PA_ERR_SHAPE otherwise)
 * Every other argument, the split-K workspace (same size as paged_attn_decode's)
 * and every status are paged_attn_decode's.
 */
int paged_attn_decode_fp8(void* out, float* lse_out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* block_tables,
                          const int32_t* seq_lens, int32_t B, int32_t max_pages,
                          int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv,
                          int32_t D, float softmax_scale, float k_scale, float v_scale,
                          int32_t max_seq_len, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * paged_attn_decode_partials -- the first phase of paged_attn_decode on its own:
 * per-partition results, to be merged later by paged_attn_splitk_reduce (possibly
 * after gathering partials of the same rows computed elsewhere, e.g. on other GPUs
 * holding other parts of the KV history; the merge is associative).
 *
 * Same arguments and partitioning as paged_attn_decode, with num_splits >= 1 given
 * explicitly (it must not exceed the number of 32-key chunks of max_seq_len).  For
 * row r = b * Hq + h and partition c (keys [c * part_len, (c+1) * part_len) of the
 * sequence), partial_out[r, c, :] is the attention output over that partition alone
 * and partial_lse[r, c] its natural-log log-sum-exp ("The Stack Below the Stack
 * (Part 2)", section 2.2, step 2); an empty partition gives 0 and -inf.
 *
 *   partial_out : [B * Hq, S, D] fp32 (16-byte aligned)   partial_lse : [B * Hq, S] fp32
 */
int paged_attn_decode_partials(float* partial_out, float* partial_lse, const void* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t B, int32_t max_pages, int32_t num_pages,
                               int32_t page_size, int32_t Hq, int32_t Hkv, int32_t D,
                               float softmax_scale, int32_t max_seq_len, int32_t num_splits,
                               void* stream);

/*
 * paged_attn_splitk_reduce -- merge S partial results per row into the exact one.
 *
 * "The Stack Below the Stack (Part 2)", section 2.2, step 3: with m = max_c lse_c,
 *   lse = m + ln sum_c exp(lse_c - m),   out = sum_c exp(lse_c - lse) * partial_out[c].
 * A partial with lse_c = -inf (an empty partition) contributes nothing; if every
 * partial of a row is empty the row gets out = 0, lse = -inf.
 *
 *   out         : [R, D] bf16              lse_out     : [R] fp32 or NULL
 *   partial_out : [R, S, D] fp32 (each row normalised by its own partition's sum)
 *   partial_lse : [R, S] fp32 natural-log lse of each partition
 */
int paged_attn_splitk_reduce(void* out, float* lse_out, const float* partial_out,
                             const float* partial_lse, int32_t R, int32_t S, int32_t D,
                             void* stream);

/*
 * paged_attn_prefill_varlen -- ragged (causal) attention of many query rows per
 * sequence over paged keys, on MFMA.
 *
 * Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of q and
 * attends keys 0..seq_lens_k[b]-1 of its table row.  With causal != 0 the q_len
 * rows of a sequence are its LAST q_len positions: row i sits at absolute position
 * p_i = seq_lens_k[b] - q_len + i and sees keys j <= p_i (the q_idx >= kv_idx mask
 * of "The Stack Below the Stack (Part 2)", section 5, bottom-right aligned over the
 * history).  Without causal every row sees all seq_lens_k[b] keys.  q_len == 1 is
 * a valid decode row.  Prefill is compute-heavy ("8. Kernels and Attention
 * Backends", "Counting attention's traffic"): scores and P V run on bf16 MFMA with
 * fp32 accumulation; P is rounded to bf16 before P V.
 *
 *   out        : [Tq, Hq, D] bf16               lse_out : [Tq, Hq] fp32 or NULL
 *   q          : [Tq, Hq, D] bf16               cu_seqlens_q : [B+1] int32 (cu[B] == Tq)
 *   seq_lens_k : [B] int32                      block_tables : [B, max_pages] int32
 *   max_q_len  : host-side upper bound of the per-sequence q_len (sizes the grid;
 *                rows past it are not computed)
 * One launch covers Hq * B * ceil(max_q_len / R) work-groups of 2 R threads
 * (R = 128 query rows, or 256 when max_q_len >= 512 or the pools are FP8 with ALiBi
 * slopes); when
 * Hq * B * (ceil(max_q_len / 128) + 1) * 256 exceeds 2^32 - 1 the call is refused
 * with PA_ERR_SHAPE.
 */
int paged_attn_prefill_varlen(void* out, float* lse_out, const void* q, const void* k_pool,
                              const void* v_pool, const int32_t* cu_seqlens_q,
                              const int32_t* seq_lens_k, const int32_t* block_tables,
                              int32_t B, int32_t Tq, int32_t max_q_len, int32_t max_pages,
                              int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv,
                              int32_t D, float softmax_scale, int32_t causal, void* stream);

/*
 * paged_attn_prefill_varlen_splitk -- paged_attn_prefill_varlen with long key
 * ranges cut into parts, so that a batch whose sequences differ widely in length
 * (a long history next to short ones) does not wait on a few long work-groups.
 *
 * Each query tile (R rows as above) of sequence b needs the keys up to its last
 * row's position (all seq_lens_k[b] keys without causal): n tiles of 64 keys.
 * With S = num_splits > 1 those tiles are cut into P = min(S, max(1, n / 16))
 * parts of consecutive tiles (so a part spans at least 1,024 keys); each part is
 * computed by its own work-group into the workspace (partial output and natural-log
 * lse, as paged_attn_decode_partials does for decode), and a second kernel merges
 * the parts of every split row exactly ("The Stack Below the Stack (Part 2)",
 * section 2.2: the log-sum-exp merge is exact for any partition of the keys).
 * Rows of tiles with P == 1 are written directly.  The result equals
 * paged_attn_prefill_varlen's up to rounding; with S == 1 it is the same launch.
 *
 *   num_splits : S (at most 16), or <= 0 for paged_attn_prefill_num_splits()
 *   workspace  : device buffer of at least paged_attn_prefill_workspace_bytes()
 *                (may be NULL when that is 0); contents are scratch.  Calls that share
 *                a workspace must not run concurrently.
 * Every other argument and status is paged_attn_prefill_varlen's; the launch bound
 * on work-items includes the factor S.
 */
int paged_attn_prefill_varlen_splitk(void* out, float* lse_out, const void* q,
                                     const void* k_pool, const void* v_pool,
                                     const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                     const int32_t* block_tables, int32_t B, int32_t Tq,
                                     int32_t max_q_len, int32_t max_pages, int32_t num_pages,
                                     int32_t page_size, int32_t Hq, int32_t Hkv, int32_t D,
                                     float softmax_scale, int32_t causal, int32_t num_splits,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attn_prefill_num_splits -- the key-part count paged_attn_prefill_varlen_splitk
 * uses for num_splits <= 0: 1 while the launch fills every work-group slot of MI355X
 * (256 CUs; one 256-row or two 128-row work-groups per CU), else enough parts for
 * one work-group per slot, at most 8.  Depends only on host scalars.
 */
int32_t paged_attn_prefill_num_splits(int32_t B, int32_t Hq, int32_t max_q_len);

/*
 * paged_attn_prefill_plan_splits -- a key-part count for
 * paged_attn_prefill_varlen_splitk planned from host copies of the lengths (a
 * scheduler knows them before it launches): q_lens[b] query rows over k_lens[b]
 * keys, b < B, with the same causal flag and window_left as the launch.  Every
 * query tile is counted in 64-key tiles and cut into parts as the kernel does.  A
 * launch lasts at least its heaviest piece and at least the mean load per
 * work-group slot of MI355X (256 CUs; one 256-row or two 128-row work-groups each),
 * so the count starts at ceil(heaviest / mean - 0.05); each count from there to 8 is
 * priced by placing its work-groups heaviest-first on the slots (as the grid is
 * ordered), charging each work-group 2 tiles for its start and drain and the merge
 * 3 tiles, and the cheapest count (the smallest within 3 % of it) is returned.  It is
 * 1 when the heaviest tile is at most the mean or shorter than two 16-tile parts.
 * Ragged batches of chunks over unequal histories ("The Stack Below the Stack
 * (Part 2)", section 2.2; "8. Kernels and Attention Backends", chapter intro: a
 * step holds ragged requests of very different lengths) are the case it serves.  Host work grows with the work-group count
 * (about 0.6 ms for 640 work-groups); beyond 16,384 (query tile, head) work-groups
 * the starting bound is returned unpriced.
 *
 *   q_lens, k_lens : host arrays of B non-negative int32 (read only, not kept)
 *
 * Returns the count (>= 1), or 0 with pa_last_error() set when B < 0, Hq <= 0,
 * window_left < 0, a length is negative, or an array is NULL with B > 0.
 */
int32_t paged_attn_prefill_plan_splits(int32_t B, const int32_t* q_lens, const int32_t* k_lens,
                                       int32_t Hq, int32_t causal, int32_t window_left);

/*
 * paged_attn_prefill_workspace_bytes -- workspace bytes of paged_attn_prefill_varlen_splitk
 * for this shape and num_splits (after resolving num_splits <= 0 as above): fp32
 * partial outputs [Tq * Hq, S, D] followed by fp32 partial lse [Tq * Hq, S], each
 * region 256-byte aligned.  0 when S == 1.
 */
size_t paged_attn_prefill_workspace_bytes(int32_t B, int32_t Tq, int32_t max_q_len, int32_t Hq,
                                          int32_t D, int32_t num_splits);

/*
 * Sliding-window attention and the general entry points.
 *
 * The pages list sliding windows among the masks a serving backend must support
 * ("8. Kernels and Attention Backends", "Attention is an I/O problem"; sliding-window
 * and document masks as FlexAttention mask functions in "The Stack Below the Stack
 * (Part 2)", section 5) without fixing the predicate.  This library's: with
 * window_left = w > 0 a query at absolute position p sees key j only if p - w < j
 * (its last w positions, itself included), on top of the causal bound when causal;
 * without causal only this lower bound applies.  A decode row sits at position
 * seq_len - 1, so it sees keys seq_len - w .. seq_len - 1.  w = 0: no window.
 * Without document ranges (below) every sequence of a ragged batch is one document.
 *
 * ALiBi: the same section names ALiBi among the score modifications, again without
 * a formula.  This library's: with alibi_slopes (device float32 [Hq], one slope per
 * query head, 4-byte aligned) the score of query head h at absolute position p
 * against key j becomes softmax_scale * q . k + slope_h * (j - p); NULL: no bias.
 * lse outputs include the bias.  The bias composes with the causal bound and the
 * window.
 *
 * Document masks: the same section names document masking among the mask
 * functions (several documents packed into one sequence, a query seeing only its
 * own document's keys), again without a representation.  This library's: the
 * documents of a sequence are contiguous runs of positions, and the caller gives
 * every query row the half-open range [key_lo, key_hi) of key positions of its
 * own document (absolute positions of its sequence, as seq_lens_k counts them);
 * the row sees key j only if key_lo <= j < key_hi, on top of the causal bound and
 * the window.  A decode row (the last position of its sequence) needs only key_lo.
 * Ranges are data, not checked on the device: a range outside 0 .. seq_len masks
 * accordingly.  Document masks select the prefill kernel's general variant; the
 * host planner paged_attn_prefill_plan_splits does not see them.
 *
 * Together the causal bound, the window and the document range are one mask
 * predicate per row, lo <= key <= lim, that the general variant applies to the
 * blocks where some row's bound falls and uses to skip the key tiles outside every
 * row's range.  Any mask that is an interval of keys per query row (prefix-LM
 * masks, chunked local attention, ...) is such a predicate: give its bounds as
 * key_lo / key_hi, with causal off where the interval reaches past the row.
 *
 * Block maps: the same section shows a mask written as a predicate of (sequence,
 * head, query index, key index) and compiled by create_block_mask, which records
 * per (query block, key block) whether the block is needed at all.  This
 * library's: a block map is such a mask given in block form, block_map[b][i / 64]
 * [j / 64] nonzero when row i of sequence b's query run (0-based within the run)
 * may see key j; entries outside the map's block_map_q_blocks x block_map_k_blocks
 * count as zero.  It combines (and) with the causal bound, the window, the
 * document ranges and ALiBi.  The prefill walks only the 64-key tiles that one of
 * its four 64-row query blocks lists (256-row work-groups) and masks a listed tile
 * whole for the rows of a query block that does not list it; there block maps take
 * bf16 or FP8 pools (scales per pool or per page), no key parts, and at most 262144
 * keys per sequence (max_pages x page_size); other requests are PA_ERR_UNSUPPORTED.
 * The decode takes a map of one
 * query block per sequence (its row is query index 0 of a one-row run),
 * block_map[b][j / 64], and walks only the 32-key chunks of listed tiles, with bf16
 * or FP8 pools and any split count.  The map is data, read on the device.
 *
 * The _ex entry points take every option of an operation in one struct; the
 * entry points above are these with fixed options.  A NULL opts is PA_ERR_NULL; a
 * negative window PA_ERR_SHAPE.
 *
 * Kernel timing: kernel_start_event / kernel_stop_event, when not NULL, are HIP
 * events (created beforehand, timing enabled, on the launch's device) that the
 * dispatch of the operation's main kernel (decode: the partition kernel, or the
 * kernel of grouped partitions; prefill:
 * the prefill kernel, not the merge) stamps with that kernel's own start and end
 * (hipExtLaunchKernel).  hipEventElapsedTime on the pair then gives the kernel's
 * duration inside a stream of work, with no event records added between launches.
 * The library neither creates, records otherwise, nor destroys them.
 */
typedef struct {
  int32_t num_splits;   /* as paged_attn_decode's (<= 0: the library's choice)            */
  int32_t window_left;  /* 0, or w > 0: keys seq_len - w .. seq_len - 1 only              */
  int32_t kv_fp8;       /* 0: bf16 pools; 1: E4M3 code pools (paged_attn_decode_fp8)      */
  float k_scale;        /* kv_fp8 only                                                    */
  float v_scale;        /* kv_fp8 only                                                    */
  const float* alibi_slopes;  /* NULL, or device [Hq] float32 slopes (ALiBi above)        */
  void* kernel_start_event;   /* NULL, or a created hipEvent_t (timing enabled) that the
                                 partition kernel's dispatch stamps with its start       */
  void* kernel_stop_event;    /* NULL, or a hipEvent_t stamped with that kernel's end     */
  const int32_t* key_lo;      /* NULL, or device [B] int32: first key of the document the
                                 decode row belongs to (document masks above)            */
  const float* k_scales;      /* kv_fp8 only: NULL (the pool scales above), or device
                                 [num_pages, Hkv] float32 scales per (page, KV head)     */
  const float* v_scales;      /* with k_scales (both or neither)                          */
  const uint8_t* block_map;   /* NULL, or device uint8 [B, block_map_k_blocks]: the 64-key
                                 tiles each sequence's decode row sees (block maps above;
                                 the row is query index 0 of its one-row run)             */
  int32_t block_map_k_blocks; /* key blocks of 64 keys per sequence in the map (>= 1)     */
} pa_decode_opts;

typedef struct {
  int32_t causal;       /* as paged_attn_prefill_varlen's                                 */
  int32_t window_left;  /* 0, or w > 0: row at position p sees keys j > p - w only        */
  int32_t num_splits;   /* key parts as paged_attn_prefill_varlen_splitk's: 1 plain,
                           <= 0 the library's choice (may need a workspace)               */
  const float* alibi_slopes;  /* NULL, or device [Hq] float32 slopes (ALiBi above)        */
  int32_t kv_fp8;       /* 0: bf16 pools; 1: E4M3 code pools (format above)               */
  float k_scale;        /* kv_fp8 only                                                    */
  float v_scale;        /* kv_fp8 only                                                    */
  void* kernel_start_event;   /* NULL, or a created hipEvent_t (timing enabled) that the
                                 prefill kernel's dispatch stamps with its start         */
  void* kernel_stop_event;    /* NULL, or a hipEvent_t stamped with that kernel's end     */
  const int32_t* key_lo;      /* NULL, or device [Tq] int32: key_lo of every query row    */
  const int32_t* key_hi;      /* NULL, or device [Tq] int32: key_hi of every query row
                                 (both or neither; document masks above)                 */
  const float* k_scales;      /* kv_fp8 only: NULL (the pool scales above), or device
                                 [num_pages, Hkv] float32 scales per (page, KV head); not
                                 with ALiBi slopes (PA_ERR_UNSUPPORTED)                  */
  const float* v_scales;      /* with k_scales (both or neither)                          */
  int32_t persistent;   /* 1: persistent work-groups (plain bf16 variant with 256-row query
                           tiles only, else ignored): one per CU, each taking the grid's
                           work items in turn and fetching the next item's Q rows and
                           first K/V tile during the current item's last tile.  The
                           results are the same bits as the plain grid's.  0: plain grid */
  const uint8_t* block_map;   /* NULL, or device uint8 [B, block_map_q_blocks,
                                 block_map_k_blocks]: a mask in block form (block maps
                                 above); no key parts                                     */
  int32_t block_map_q_blocks; /* query blocks of 64 rows per sequence in the map (>= 1)   */
  int32_t block_map_k_blocks; /* key blocks of 64 keys per sequence in the map (>= 1)     */
} pa_prefill_opts;

/*
 * paged_attn_decode_ex -- paged_attn_decode / paged_attn_decode_fp8 with options.
 * With a window every row walks at most window_left + 31 keys (its first key rounded
 * down to a 32-key chunk), and the split count and workspace are sized for
 * min(max_seq_len, window_left + 31): use paged_attn_decode_ex_workspace_bytes.
 */
int paged_attn_decode_ex(void* out, float* lse_out, const void* q, const void* k_pool,
                         const void* v_pool, const int32_t* block_tables,
                         const int32_t* seq_lens, int32_t B, int32_t max_pages,
                         int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv,
                         int32_t D, float softmax_scale, int32_t max_seq_len,
                         const pa_decode_opts* opts, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Workspace bytes of paged_attn_decode_ex for these options (0 for NULL opts). */
size_t paged_attn_decode_ex_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                            int32_t max_seq_len, const pa_decode_opts* opts);

/*
 * paged_attn_prefill_ex -- paged_attn_prefill_varlen(_splitk) with options.  With a
 * window, a query tile starts at the 64-key tile holding its first row's lower
 * bound, so key tiles wholly below every row's window are never read.  A window or
 * ALiBi selects a kernel variant with those steps compiled in (two more vector
 * operations per score for ALiBi); without them the plain kernel runs.  With
 * kv_fp8 the pools hold E4M3 codes: each tile's codes are loaded into registers and
 * widened to bf16 (exactly) into the same LDS tile the bf16 path fills, k_scale
 * folds into the softmax scale and v_scale into the final normalisation, as in
 * paged_attn_decode_fp8.
 */
int paged_attn_prefill_ex(void* out, float* lse_out, const void* q, const void* k_pool,
                          const void* v_pool, const int32_t* cu_seqlens_q,
                          const int32_t* seq_lens_k, const int32_t* block_tables, int32_t B,
                          int32_t Tq, int32_t max_q_len, int32_t max_pages, int32_t num_pages,
                          int32_t page_size, int32_t Hq, int32_t Hkv, int32_t D,
                          float softmax_scale, const pa_prefill_opts* opts, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes of paged_attn_prefill_ex for these options (0 for NULL opts). */
size_t paged_attn_prefill_ex_workspace_bytes(int32_t B, int32_t Tq, int32_t max_q_len,
                                             int32_t Hq, int32_t D,
                                             const pa_prefill_opts* opts);

/*
 * The mixed step: one step of a serving engine holds prefill chunks and decode rows
 * side by side ("8. Kernels and Attention Backends", chapter intro: one step of 23
 * ragged requests), and one kernel can serve both kinds ("Inside Ion: Custom
 * Attention Kernels for NVIDIA Grace", "IonAttention in One Paragraph").
 * paged_attn_mixed computes a prefill batch (as paged_attn_prefill_varlen_splitk) and
 * a decode batch (as paged_attn_decode) over the same bf16 pools in one kernel
 * launch: its first work-groups each run eight decode items (a (sequence, KV head,
 * partition) item per wave, as the decode with one-wave work-groups runs it), and
 * the work-groups after them run the prefill's items (256-row query tiles,
 * whatever max_q_len) in the prefill grid's order, so the decode's short items
 * take CUs while the prefill's heaviest tiles start and free them for the rest.
 * Where the prefill has key parts or the decode has partitions, their merge kernels
 * follow on the same stream (the prefill merge, then the split-K reduce).  The
 * prefill rows are bit for bit those of paged_attn_prefill_varlen_splitk with the same
 * key-part count when that launch takes 256-row tiles too (max_q_len >= 512); the
 * decode rows those of paged_attn_decode with the same split count when that launch
 * takes one-wave work-groups (Hkv x splits x B >= 512), and otherwise equal up to
 * rounding (its waves then split a partition's chunks and merge them).
 * FP8 pools are taken (pa_mixed_fp8 below); the other options (windows, ALiBi,
 * document ranges, block maps) are not: use the separate entry points for them.
 */
typedef struct {
  void* out;                    /* bf16 [Tq, Hq, D]                                     */
  float* lse_out;               /* fp32 [Tq, Hq] or NULL                                */
  const void* q;                /* bf16 [Tq, Hq, D]                                     */
  const int32_t* cu_seqlens_q;  /* [B + 1] int32, cu[B] == Tq                           */
  const int32_t* seq_lens_k;    /* [B] int32                                            */
  const int32_t* block_tables;  /* [B, max_pages] int32                                 */
  int32_t B, Tq, max_q_len, max_pages;   /* B == 0: no prefill part                     */
  int32_t causal;               /* as paged_attn_prefill_varlen's                       */
  int32_t num_splits;           /* key parts as paged_attn_prefill_varlen_splitk's (<= 0:
                                   the library's count for 256-row work-groups)         */
} pa_mixed_prefill;

typedef struct {
  void* out;                    /* bf16 [B, Hq, D]                                      */
  float* lse_out;               /* fp32 [B, Hq] or NULL                                 */
  const void* q;                /* bf16 [B, Hq, D], one query row per sequence          */
  const int32_t* block_tables;  /* [B, max_pages] int32                                 */
  const int32_t* seq_lens;      /* [B] int32                                            */
  int32_t B, max_pages;         /* B == 0: no decode part                               */
  int32_t max_seq_len;          /* host-side bound of seq_lens, as paged_attn_decode's  */
  int32_t num_splits;           /* > 0: as paged_attn_decode's; <= 0: the larger of
                                   paged_attn_decode's (or paged_attn_decode_fp8's) own
                                   count times the waves per work-group its launch would
                                   give each item (1, 2 or 4), so that each one-wave item
                                   here walks as many keys as a wave does there, and the
                                   count that gives the CUs the prefill's work-groups
                                   leave free (of 256) eight items each, partitions kept
                                   at 8 chunks of 32 keys or more                       */
} pa_mixed_decode;

/* FP8 E4M3 pools for paged_attn_mixed (a NULL pointer there: bf16 pools), with the
 * scales paged_attn_decode_ex and paged_attn_prefill_ex take: one per pool, or per
 * (page, KV head) when k_scales / v_scales are given (both or neither). */
typedef struct {
  float k_scale, v_scale;       /* one scale per pool (with k_scales NULL)              */
  const float* k_scales;        /* NULL, or device [num_pages, Hkv] float32             */
  const float* v_scales;        /* with k_scales                                        */
} pa_mixed_fp8;

/*
 * Workspace bytes of paged_attn_mixed: the prefill's key-part partials (as
 * paged_attn_prefill_workspace_bytes with 256-row tiles) followed by the decode's
 * split-K partials (as paged_attn_decode_workspace_bytes), each region 256-byte
 * aligned, with the split counts paged_attn_mixed resolves; 0 when neither part
 * needs one or an argument is NULL or not positive.
 */
size_t paged_attn_mixed_workspace_bytes(const pa_mixed_prefill* prefill,
                                        const pa_mixed_decode* decode, const pa_mixed_fp8* fp8,
                                        int32_t Hq, int32_t Hkv, int32_t D);

/*
 * paged_attn_mixed -- the prefill and decode batches above in one launch (plus their
 * merges).  Both parts share the pools (num_pages, page_size, Hkv, D; bf16, or with
 * fp8 non-NULL E4M3 codes under fp8's scales), Hq and the softmax scale.  prefill or
 * decode NULL: PA_ERR_NULL.  Each part is checked as its own entry point checks it (the
 * same statuses; the message names the part); a part with B == 0 is skipped, and with
 * both skipped nothing is launched.  The workspace is scratch (calls that share one
 * must not run concurrently).
 */
int paged_attn_mixed(const pa_mixed_prefill* prefill, const pa_mixed_decode* decode,
                     const pa_mixed_fp8* fp8, const void* k_pool, const void* v_pool,
                     int32_t num_pages, int32_t page_size, int32_t Hq, int32_t Hkv, int32_t D,
                     float softmax_scale, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Human-readable name of a pa_status value (static string). */
const char* pa_status_string(int status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* pa_last_error(void);

/* Thread-local description of the last successful launch on this thread: kernel
 * variant, grid, split count.  The selected path is part of the contract, so it is
 * reported rather than implied ("8. Kernels and Attention Backends", "Backends are
 * compatibility decisions"). */
const char* pa_describe_launch(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
