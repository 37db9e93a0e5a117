// Ragged causal prefill over paged K/V on gfx950 matrix cores.
//
// Work-group = 4 waves = 128 consecutive query rows of one query head of one
// sequence; each wave owns 32 rows.  Keys are walked in 64-key tiles that the
// waves copy from the page pool straight into LDS (global_load_lds, through the
// block table; double buffered, so the next tile is in flight while the current
// one is consumed).  Per 32-key block a wave computes
//   S^T[32 keys x 32 queries] = K Q^T           32x32x16 bf16 MFMA, fp32 accumulate
//   running max / running sum per query         ("The Stack Below the Stack (Part 2)",
//                                                 section 2.1, online softmax)
//   O^T[D x 32 queries] += V^T P^T               P rounded to bf16
// Keys sit on the MFMA's M side so that every per-query statistic lives in lane %
// 32 and the S^T accumulator is already laid out as the P^T operand.  K and V are
// both stored row-major; the V^T operand comes from transposing LDS reads
// (ds_read_b64_tr_b16).
//
// Causal rows are the LAST q_len positions of their sequence (query row i at
// absolute position seq_len - q_len + i sees keys j <= that position); key
// blocks wholly above a wave's rows are skipped, and only blocks that cross the
// diagonal are masked.  Work-groups with the most keys are dispatched first.
#include <limits.h>
#include <stdio.h>

#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "decode_item.hpp"
#include "kernels.hpp"

namespace pa {

constexpr int kPfBN = 64;              // keys per LDS tile
constexpr float kRescaleSlack = 8.f;   // log2 headroom before the reference moves
constexpr float kSumLimit = 256.f;     // 2^kRescaleSlack: bound on a lane's block row sum
#ifndef PF_W8_MIN
#define PF_W8_MIN 512
#endif

// Document masks: the smallest key_lo and the largest key_hi over query rows
// r0 .. r0 + rows - 1 of the sequence whose rows start at token t0, reduced over
// one wave (each lane reads every 64th row).  The union of those rows' documents
// lies in [lo, hi).
struct DocSpan {
  int lo, hi;
};
__device__ __forceinline__ DocSpan pf_doc_span(const PrefillArgs& a, int t0, int r0, int rows,
                                               int lane) {
  int lo = INT_MAX, hi = INT_MIN;
  for (int r = lane; r < rows; r += 64) {
    lo = min(lo, a.key_lo[t0 + r0 + r]);
    hi = max(hi, a.key_hi[t0 + r0 + r]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    lo = min(lo, __shfl_xor(lo, off));
    hi = max(hi, __shfl_xor(hi, off));
  }
  return DocSpan{__builtin_amdgcn_readfirstlane(lo), __builtin_amdgcn_readfirstlane(hi)};
}

// The key tiles a query tile needs and how many parts they are cut into.  A
// query tile of rows r0 .. r0 + rows - 1 of a sequence with L keys and q_len query
// rows needs keys up to k_lim - 1 (causal: up to its last row's position) and,
// with a sliding window, from its first row's lower bound on; with document masks
// only keys inside the span of its rows' documents: tiles first .. n - 1.  With key
// splitting on (S > 1) those tiles are cut into min(S, count / part_min) parts of
// consecutive tiles (at least one), each computed by its own work-group; the prefill
// merge recomputes the same count for every row.
struct PfTiles {
  int first;   // first 64-key tile
  int n;       // one past the last tile
  int parts;   // key-range parts
};

template <bool GEN>
__device__ __forceinline__ PfTiles pf_tiles(const PrefillArgs& a, int L, int q_len, int r0,
                                            int bm, int t0, int lane) {
  const int rows = min(bm, q_len - r0);
  int k_lim = L;
  if (a.causal) k_lim = min(L, max(0, L - q_len + r0 + rows));
  // only the general variant (window, ALiBi, documents) sees a window or documents
  int k_lo = GEN && a.window > 0 ? max(0, L - q_len + r0 - a.window + 1) : 0;
  if (GEN && a.key_lo) {
    const DocSpan d = pf_doc_span(a, t0, r0, min(rows, a.Tq - t0 - r0), lane);
    k_lim = min(k_lim, max(0, d.hi));
    k_lo = max(k_lo, min(d.lo, k_lim));
  }
  PfTiles t;
  t.n = (k_lim + kPfBN - 1) / kPfBN;
  t.first = min(k_lo / kPfBN, t.n);
  t.parts = a.S > 1 ? max(1, min(a.S, (t.n - t.first) / a.part_min)) : 1;
  return t;
}

// LDS tiles of 64 keys.  Each wave's 16 rows (keys 16 w .. 16 w + 15, one run of
// one page) form a region of 16 x D bf16 stored chunk-major: the 16-byte chunk c
// (columns 8 c .. 8 c + 7) of the region's rows sits in the 256-byte line c, one
// slot per row.  The LDS serves 256 bytes (all 64 banks) per clock.
//   K: row s of the region in slot s.  A K operand read (one chunk of 16
//      consecutive rows per 16 lanes) covers one whole line.
//   V: row s in slot (s + 4 c) mod 16 of line c.  A transposing V read (per 32
//      lanes: 4 consecutive rows x 4 consecutive chunks, 8 bytes each) then hits
//      16 distinct slots of 4 lines.
// Both layouts make every operand address a fixed per-lane offset plus a
// compile-time constant; the DMA (one 1024-byte run of 64 slots per instruction)
// fetches, per lane, whichever global chunk belongs in its slot.
template <int D>
struct PfLds {
  static constexpr int TILE = kPfBN * D;          // bf16 elements of one K or V tile
  static constexpr int REGION = 16 * D;           // one wave's 16 rows
  static constexpr int K_STAGES = 2;              // K of tiles t and t + 1
  static constexpr int V_STAGES = 3;              // V of tiles t - 1 .. t + 1
  static constexpr int V0 = K_STAGES * TILE;      // first V stage
  static constexpr size_t BYTES = (size_t)(K_STAGES + V_STAGES) * TILE * sizeof(uint16_t);
  // persistent work-groups: the next item's Q rows (32 per wave) after the stages
  static constexpr int Q0 = (K_STAGES + V_STAGES) * TILE;
  static constexpr size_t q_bytes(int W) { return (size_t)32 * W * D * sizeof(uint16_t); }
};

// max(a, b, c) in one instruction.  The scores compared here come from MFMA
// accumulators and cannot be signalling NaNs, so the quieting that fmaxf needs
// before each comparison is not needed.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Keeps a value computed where it is written: later passes may not sink its
// computation past this point (used to hold vector work between MFMAs).
__device__ __forceinline__ void pin(float v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void pin(uint32_t v) { asm volatile("" ::"v"(v)); }


// Transposing 8-byte LDS read: within each 16-lane group, lane j receives element
// (j % 4) of the 8-byte rows that lanes j/4, 4 + j/4, 8 + j/4 and 12 + j/4 point at.
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// How the W waves of a work-group split the DMA of a 64-key tile: the tile has
// four 16-row regions of D / 8 lines; wave w fills lines line0 .. line0 + LPW - 1
// of region w * 4 / W, with LPW / 4 load instructions per matrix (each covers four
// lines of 16 slots).  The 16 rows of a region are keys k0 + 16 r .., all in one
// page, which starts the run at in-page row (16 r) & (page_size - 1) since tiles
// start on page boundaries.
template <int D, int W>
struct PfDma {
  static constexpr int LPW = (D / 8) * 4 / W;     // lines per wave
  static constexpr int NJ = LPW / 4;              // load instructions per matrix
  static __device__ __forceinline__ int region(int wave) { return wave * 4 / W; }
  static __device__ __forceinline__ int line0(int wave) { return (wave % (W / 4)) * LPW; }
};

// DMA loads of one 64-key tile into LDS (K into kst, V into vst).  The per-lane
// byte offsets koff / voff (row and chunk within the run of the slot the lane
// fills) are fixed for the whole kernel, so a tile costs only scalar address
// arithmetic.
template <int D, int W>
__device__ __forceinline__ void pf_issue_tile(uint16_t* kst, uint16_t* vst,
                                              const uint16_t* kbase, const uint16_t* vbase,
                                              size_t page_row0, int rs, const uint32_t* koff,
                                              const uint32_t* voff, int wave) {
  using M = PfDma<D, W>;
  const size_t base = page_row0 * rs;
#pragma unroll
  for (int j = 0; j < M::NJ; ++j) {
    const int slot0 = M::region(wave) * PfLds<D>::REGION + 128 * (M::line0(wave) + 4 * j);
    dma16(kbase + base, koff[j], kst + slot0);
    dma16(vbase + base, voff[j], vst + slot0);
  }
}

// Zero this wave's V slots whose rows are at or past the sequence end (the last
// tile only): they hold other data, and P = 0 times NaN would not be 0.  The
// slots are the ones this wave's DMA fills.
template <int D, int W>
__device__ __forceinline__ void pf_zero_tail(uint16_t* vst, int k0, int L, int wave, int lane) {
  using M = PfDma<D, W>;
#pragma unroll
  for (int j = 0; j < M::NJ; ++j) {
    const int c = M::line0(wave) + 4 * j + (lane >> 4);
    const int row = ((lane & 15) - 4 * c) & 15;
    if (k0 + 16 * M::region(wave) + row >= L)
      *reinterpret_cast<u32x4*>(vst + M::region(wave) * PfLds<D>::REGION + 128 * c +
                                8 * (lane & 15)) = u32x4{0u, 0u, 0u, 0u};
  }
}

// Four E4M3 codes (bytes 0..3) -> two packed bf16 pairs, exactly (every E4M3 value
// is a bf16 value).
__device__ __forceinline__ u32x2 pf_fp8x4_to_bf16(uint32_t w) {
  return u32x2{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

// A work item: query rows 32 W qt .. 32 W qt + 32 W - 1 of query head h of sequence
// b, over key part `part` of their key tiles.
struct PfWork {
  int h, b, qt, part;
};

__device__ __forceinline__ PfWork pf_work_of(const PrefillArgs& a, int p) {
  // Item p -> (query head h, sequence b, query tile qt, key part).  Items (one per
  // work-group of the plain grid, whose id is p) are handed to the 8 XCDs round-robin (id % 8), each XCD with its own L2.  With
  // xcd_groups set, the work is cut into units -- a (sequence, KV head) group or,
  // when the group count is not a multiple of 8, one of xcd_split classes of its
  // query-tile ranks, so that the units divide evenly among the XCDs (ranks are
  // dealt to the classes zig-zag, so every class carries as much causal work) --
  // and each XCD runs its units one after the other (unit-major): all query
  // heads, tiles and key parts of a unit, heaviest tile first, then the next unit,
  // so the group's K/V stays in that XCD's L2 while the unit's tiles use it, and the
  // next unit's heavy tiles start while the previous one's light ones finish.
  // Without it the order is head-major, heaviest tiles first.  Either way all key
  // parts of a tile start together and every XCD keeps its share of the unsplit work.
  // With paired heads (a.hp) an item takes query heads h and h + 1 (h even within its
  // KV group), so the head dimension of the grid has half the entries.
  PfWork w;
  {
    const int hs = a.hp ? 2 : 1;
    if (a.xcd_groups) {
      const int m = a.xcd_split;
      const int gh = a.G / hs;                   // head slots of a group
      const int tpu = (a.n_qt + m - 1) / m;      // tile ranks per unit
      const int k = p >> 3;                      // this work-group's place on its XCD
      const int per_unit = gh * tpu * a.S;       // work-groups of one unit
      const int ui = k / per_unit;               // the XCD's ui-th unit
      const int rem = k - ui * per_unit;
      const int r2 = rem / gh;                   // (tile rank in unit, part), heaviest first
      const int rl = r2 / a.S;
      w.part = r2 - rl * a.S;
      const int u = (p & 7) + 8 * ui;            // unit = group g, rank class j
      const int g = u / m;
      const int j = u - g * m;
      // ranks dealt to the classes zig-zag (0 .. m-1, then m-1 .. 0, ...), so every
      // class holds as much heavy as light causal work
      const int rank = rl * m + ((rl & 1) ? m - 1 - j : j);
      w.b = g / a.Hkv;
      w.h = (g - w.b * a.Hkv) * a.G + hs * (rem % gh);
      w.qt = a.n_qt - 1 - rank;                    // below 0: past the unit's last tile
    } else {
      const int hq = a.Hq / hs;
      w.h = hs * (p % hq);
      const int r = p / hq;
      w.b = r % a.B;
      const int r2 = r / a.B;
      const int rank = r2 / a.S;
      w.part = r2 - rank * a.S;
      w.qt = a.n_qt - 1 - rank;
    }
  }

  return w;
}

// What an item covers: its sequence's query rows start at token t0, q_len of them,
// over L keys; its first row r_wg; its KV head; the key tiles tile_lo .. tile_hi - 1
// (part `part` of `parts`).  ok = 0 for an item past its sequence's last query tile
// or key part.
struct PfSetup {
  int ok, t0, q_len, L, r_wg, kvh, tile_lo, tile_hi, parts;
};

template <bool GEN>
__device__ __forceinline__ PfSetup pf_setup(const PrefillArgs& a, const PfWork& w, int bm,
                                            int lane) {
  PfSetup s{};
  if (w.qt < 0) return s;
  s.t0 = a.cu_seqlens_q[w.b];
  s.q_len = a.cu_seqlens_q[w.b + 1] - s.t0;
  s.r_wg = w.qt * bm;
  if (s.r_wg >= s.q_len) return s;
  const int L = a.seq_lens_k[w.b];
  const int cap = a.max_pages * a.page_size;
  s.L = L < 0 ? 0 : (L > cap ? cap : L);
  s.kvh = w.h / a.G;
  // keys past the item's last row are never needed; with key splitting the item
  // covers tiles tile_lo .. tile_hi - 1 of them
  const PfTiles tw = pf_tiles<GEN>(a, s.L, s.q_len, s.r_wg, bm, s.t0, lane);
  if (w.part >= tw.parts) return s;
  s.parts = tw.parts;
  s.tile_lo = tw.first + w.part * (tw.n - tw.first) / tw.parts;
  s.tile_hi = tw.first + (w.part + 1) * (tw.n - tw.first) / tw.parts;
  s.ok = 1;
  return s;
}

// Hand-over between consecutive items of a persistent work-group: during an item's
// last tile the work-group already issues the next item's first K/V tile (into the
// stages that follow the item's own), copies the next item's Q rows into the LDS Q
// area and holds its block-table window, so that the next item starts on data in LDS
// instead of waiting for its table, Q and first tile in turn.
struct PfHand {
  int has;        // this item's first tile was issued by the previous item
  int q_lds;      //   and its Q rows sit in the LDS Q area
  int kc, vc;     // K and V stage of this item's first tile
  int tab;        // this item's block-table window (per lane), when has
  int pn;         // the item after this one (its id), or -1
};

// Block maps (a mask given in block form, 64 query rows x 64 keys per block): the
// listed key tiles of a work-group are gathered into a list in LDS, after the
// K/V stages; entry 0 holds the count, entry 1 + i the i-th listed tile in
// ascending order, with bit 16 + k set when the work-group's k-th 64-row query
// block lists it.
constexpr int kBsMaxTiles = 4096;           // 262,144 keys
constexpr size_t kBsListBytes = (kBsMaxTiles + 16) * sizeof(int);

// W waves (32 W query rows) per work-group; 8 W waves per CU.  GEN: the general
// variant (sliding window, ALiBi); F8: FP8 E4M3 pools; REV: key tiles walked
// downwards, which is how the ALiBi variants (general only) walk, so REV also
// compiles the bias in.  PER: an item of a persistent work-group (hand-over in hd).
// BS: a block map (general variant, 8 waves, no key parts).  HP: paired heads (plain
// bf16 variant, 8 waves): waves 0-3 take query head w.h and waves 4-7 head w.h + 1,
// both over the same 128 rows, so each K/V tile in LDS serves two heads.
template <int D, int W, bool GEN, bool F8, bool REV, bool PS, bool PER, bool BS = false,
          bool HP = false>
__device__ __forceinline__ void pf_item(const PrefillArgs& a, const PfWork& w,
                                        const PfSetup& s, PfHand& hd, uint16_t* pf_lds) {
  static_assert(!REV || GEN, "the downward walk is a general-variant feature");
  static_assert(!PS || (F8 && GEN && !REV), "scales per page: FP8 general variant, no ALiBi");
  static_assert(!PER || (!GEN && !F8), "persistent work-groups: plain bf16 variant");
  static_assert(!BS || (GEN && !PER && W == 8), "block maps: general variant, 8 waves");
  static_assert(!HP || (!PER && W == 8),
                "paired heads: plain bf16 variant, 8 waves");
  constexpr bool ALI = REV;          // ALiBi slopes present (a.alibi != nullptr)
  using L_ = PfLds<D>;
  using M_ = PfDma<D, W>;
  constexpr int kPfBM = HP ? 128 : 32 * W;   // query rows per work-group
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;         // query column of S^T / O^T
  const int hh = lane >> 5;          // k-half of the MFMA operands
  const int g16 = lane & 15;
  const int h = w.h + (HP ? wave / 4 : 0), b = w.b, part = w.part;
  const int t0 = s.t0, q_len = s.q_len, r_wg = s.r_wg, L = s.L, kvh = s.kvh;
  const int tile_lo = s.tile_lo, tile_hi = s.tile_hi;
  const uint16_t* kbase = a.k_pool + (size_t)kvh * D;
  const uint16_t* vbase = a.v_pool + (size_t)kvh * D;
  const int shift = L - q_len;                 // position of row r is shift + r
  // what the previous item of a persistent work-group prefetched for this one
  const bool pre = PER && hd.has;
  const bool q_pre = PER && hd.q_lds;
  const int kc = PER ? hd.kc : 0, vc = PER ? hd.vc : 0;
  if constexpr (PER) hd.has = hd.q_lds = 0;

  // this wave's rows and the position bound of its rows
  const int r_w = r_wg + 32 * (HP ? wave % 4 : wave);
  const int my_row = r_w + col;
  const bool row_ok = my_row < q_len && t0 + my_row < a.Tq;
  const int my_pos = shift + my_row;          // causal: keys <= my_pos are visible
  // Which keys this row sees (the mask, as one predicate): lo_row <= key <= lim.
  // lim is the sequence end, the causal bound and (documents) its document's end;
  // lo_row the window's start and (documents) its document's start.  w_lim_min and
  // w_lo_max are the smallest lim and the largest lo_row among the wave's rows: a
  // block needs the per-key mask only where one of them falls inside it.
  int lim = a.causal ? min(L - 1, my_pos) : L - 1;         // last visible key
  int lo_row = GEN && a.window > 0 ? my_pos - a.window + 1 : INT_MIN;
  int w_lim_min = a.causal ? shift + r_w : L - 1;
  int w_lo_max = GEN && a.window > 0 ? shift + r_w + 31 - a.window + 1 : INT_MIN;
  int w_hi_max = L;                            // one past the wave's last visible key
  if (GEN && a.key_lo) {
    // rows past the query run take neutral bounds (their outputs are not written)
    const int dlo = row_ok ? a.key_lo[t0 + my_row] : 0;
    const int dhi = row_ok ? a.key_hi[t0 + my_row] : L;
    lim = min(lim, dhi - 1);
    lo_row = max(lo_row, dlo);
    int mn = lim, mx = lo_row, hx = row_ok ? min(lim + 1, L) : 0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      mn = min(mn, __shfl_xor(mn, off));
      mx = max(mx, __shfl_xor(mx, off));
      hx = max(hx, __shfl_xor(hx, off));
    }
    w_lim_min = __builtin_amdgcn_readfirstlane(mn);
    w_lo_max = __builtin_amdgcn_readfirstlane(mx);
    w_hi_max = __builtin_amdgcn_readfirstlane(hx);
  }
  // ALiBi, slope_h * (key - row position), in two parts that cost nothing per score:
  // the key's offset within its block (8 j + 4 hh + i for element 4 j + i) is the
  // same for every block, so it is the initial value of the score accumulator
  // (raw units; the scores are scaled later); the block start less the row's
  // position is one value per block and row, added with the softmax reference
  // (log2 units, `boff`, set when a block's scores are masked).
  const float slope_log2 = ALI ? a.alibi[h] * kLog2e : 0.f;
  f32x16 ebias;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ebias[4 * j + i] = ALI ? slope_log2 / a.scale_log2 * (float)(8 * j + 4 * hh + i) : 0.f;
  float boff = 0.f;

  // Q^T operand: lane holds Q[row col][16 kk + 8 hh + j]
  u32x4 qb[D / 16];
  if (!q_pre) {
    const uint16_t* qp = a.q + ((size_t)(t0 + (row_ok ? my_row : 0)) * a.Hq + h) * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qb[kk] = row_ok ? ld16(qp + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
  }

  // Fixed per-lane LDS offsets (elements within a tile).  K operand of step kk
  // of block kb: row 32 kb + col, chunk 2 kk + hh, at k_lane + 32 kb D + 256 kk.
  // V^T operand of d-tile t, 16-key half u of block kb: two transposing reads,
  // rows 8 j + 4 hh + g16 / 4 of region 2 kb + u, columns 32 t + dsub .., at
  // v_lane[j] + (2 kb + u) 16 D + 512 t.
  const uint32_t k_lane = (col >> 4) * PfLds<D>::REGION + hh * 128 + (col & 15) * 8;
  uint32_t v_lane[2];
  {
    const int e = 2 * ((lane >> 4) & 1) + ((g16 & 3) >> 1);   // chunk within 4
#pragma unroll
    for (int j = 0; j < 2; ++j)
      v_lane[j] = e * 128 + (((8 * j + 4 * hh + (g16 >> 2) + 4 * e) & 15) << 3) + 4 * (g16 & 1);
  }

  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;

  // Block-table window: lane j holds the page of this wave's 16 keys of tile
  // base_t + j; it is reloaded every 64 tiles.
  const int32_t* bt = a.block_tables + (size_t)b * a.max_pages;
  int base_t = 0;
  int tab = 0;
  auto load_tab_of = [&](const int32_t* bt_, int first_tile) {
    int idx = ((first_tile + lane) * kPfBN + 16 * M_::region(wave)) >> a.ps_shift;
    idx = idx < a.max_pages ? idx : a.max_pages - 1;
    return bt_[idx];
  };
  auto load_tab = [&](int first_tile) { return load_tab_of(bt, first_tile); };
  const int run0 = (16 * M_::region(wave)) & (a.page_size - 1);
  const int rs = a.Hkv * D;
  // the global chunk each lane's DMA slot receives: slot 64 j + lane = line c,
  // slot s; K holds row s there, V row (s - 4 c) mod 16
  uint32_t k_dma[M_::NJ], v_dma[M_::NJ];
#pragma unroll
  for (int j = 0; j < M_::NJ; ++j) {
    const int c = M_::line0(wave) + 4 * j + (lane >> 4), sl = lane & 15;
    k_dma[j] = (uint32_t)(sl * rs + c * 8) * 2u;
    v_dma[j] = (uint32_t)((((sl - 4 * c) & 15) * rs) + c * 8) * 2u;
  }
  auto kst = [&](int kt) { return pf_lds + (kt & 1) * L_::TILE; };
  auto vst = [&](int vs) { return pf_lds + L_::V0 + vs * L_::TILE; };
  // FP8 pools: each wave covers the pieces (16 consecutive codes of one row) of its
  // region, row-major so that a row's pieces are neighbouring lanes; they are
  // loaded into registers one tile ahead, like the DMA, and widened to bf16 into the
  // tile's slots during the step before the tile is published (in the steady loop)
  // or at the publish (the walk's first tile and the tiles after a wave's last block).
  constexpr int F8_PPR = D / 16;                  // pieces per row
  constexpr int F8_IPW = 4 * D / W;               // pieces per wave per matrix
  constexpr int F8_NP = F8 ? (F8_IPW + 63) / 64 : 1;
  const uint8_t* kbase8 = reinterpret_cast<const uint8_t*>(a.k_pool) + (size_t)kvh * D;
  const uint8_t* vbase8 = reinterpret_cast<const uint8_t*>(a.v_pool) + (size_t)kvh * D;
  u32x4 k8[F8_NP], v8[F8_NP];
  // FP8 pools with scales per (page, KV head): each wave reads the key and value
  // scales of its own 16-row region's page when it issues a tile and, when the tile
  // is published, writes them to a small table kept per V stage: for each 32-key
  // block of the tile (k of its first and second 16 keys, v of both).  After the
  // barrier every wave finds there the scales of every block it computes.
  __shared__ __align__(16) float pg_scales[PS ? 3 : 1][8];
  float ks_next = 1.f, vs_next = 1.f;
  // DMA of tile n (tiles are issued in increasing order) into V stage vs
  // DMA of the tile of page pg (KV head kvh_) into K stage ks and V stage vs
  auto issue_page = [&](int pg, int kvh_, int ks, int vs) {
    pg = (unsigned)pg < (unsigned)a.num_pages ? pg : 0;
    if constexpr (PS) {
      ks_next = a.k_scales[(size_t)pg * a.Hkv + kvh_];
      vs_next = a.v_scales[(size_t)pg * a.Hkv + kvh_];
    }
    if constexpr (F8) {
      const size_t base = ((size_t)pg * a.page_size + run0) * rs;
#pragma unroll
      for (int k = 0; k < F8_NP; ++k) {
        const int i = lane + 64 * k;
        if (F8_IPW % 64 == 0 || i < F8_IPW) {
          const int piece = (wave % (W / 4)) * F8_IPW + i;
          const size_t off = base + (size_t)(piece / F8_PPR) * rs + 16 * (piece % F8_PPR);
          k8[k] = *reinterpret_cast<const u32x4*>(kbase8 + off);
          v8[k] = *reinterpret_cast<const u32x4*>(vbase8 + off);
          (void)kvh_;
        }
      }
    } else {
      pf_issue_tile<D, W>(kst(ks), vst(vs), a.k_pool + (size_t)kvh_ * D,
                          a.v_pool + (size_t)kvh_ * D, (size_t)pg * a.page_size + run0, rs,
                          k_dma, v_dma, wave);
    }
  };
  auto issue = [&](int n, int ks, int vs) {
    if (REV ? n < base_t : n - base_t >= 64) {
      base_t = REV ? max(0, n - 63) : (BS ? n : base_t + 64);
      tab = load_tab(base_t);
    }
    issue_page(__builtin_amdgcn_readlane(tab, n - base_t), kvh, ks, vs);
  };
  // FP8 pools: quarter q (0, 1: K; 2, 3: V) of this wave's share of tile n, widened
  // from the codes in registers into K stage ks and V stage vs
  auto widen = [&](int n, int ks, int vs, int q) {
    uint16_t* kr = kst(ks) + M_::region(wave) * PfLds<D>::REGION;
    uint16_t* vr = vst(vs) + M_::region(wave) * PfLds<D>::REGION;
    const int row0 = n * kPfBN + 16 * M_::region(wave);
#pragma unroll
    for (int k = 0; k < F8_NP; ++k) {
      const int i = lane + 64 * k;
      if (F8_IPW % 64 == 0 || i < F8_IPW) {
        const int piece = (wave % (W / 4)) * F8_IPW + i;
        const int sl = piece / F8_PPR, c = 2 * (piece % F8_PPR) + (q & 1);
        const int h2 = 2 * (q & 1);              // the piece's first or second 8 codes
        if (q < 2) {
          const u32x2 k0 = pf_fp8x4_to_bf16(k8[k][h2]), k1 = pf_fp8x4_to_bf16(k8[k][h2 + 1]);
          *reinterpret_cast<u32x4*>(kr + 128 * c + 8 * sl) = u32x4{k0[0], k0[1], k1[0], k1[1]};
        } else {
          // V rows at or past the sequence end are zeroed (P = 0 times NaN is not 0)
          u32x4 va = {0u, 0u, 0u, 0u};
          if (row0 + sl < L) {
            const u32x2 v0 = pf_fp8x4_to_bf16(v8[k][h2]), v1 = pf_fp8x4_to_bf16(v8[k][h2 + 1]);
            va = u32x4{v0[0], v0[1], v1[0], v1[1]};
          }
          *reinterpret_cast<u32x4*>(vr + 128 * c + 8 * ((sl + 4 * c) & 15)) = va;
        }
      }
    }
  };
  // tile n's loads (this wave's) have landed; tail rows zeroed; then everyone's.
  // widened: (FP8) this wave's share of tile n was widened during the step before.
  auto publish = [&](int n, int ks, int vs, bool widened = false) {
    // widened tiles went through registers, whose loads the compiler waits for
    if (!widened) vmcnt_wait<0>();
    if constexpr (PS) {
      // region r holds keys 16 r .. 16 r + 15 of the tile: half r % 2 of block r / 2
      const int r = M_::region(wave);
      if (lane == 0 && wave % (W / 4) == 0) {
        pg_scales[vs][4 * (r >> 1) + (r & 1)] = ks_next;
        pg_scales[vs][4 * (r >> 1) + 2 + (r & 1)] = vs_next;
      }
    }
    if constexpr (F8) {
      if (!widened) {
#pragma unroll
        for (int q = 0; q < 4; ++q) widen(n, ks, vs, q);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the tile is in LDS
    } else if (n * kPfBN + kPfBN > L) {
      pf_zero_tail<D, W>(vst(vs), n * kPfBN, L, wave, lane);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the zeros are in LDS
    }
    block_sync();
  };

  // ---- the per-block steps ----
  // S^T of the 32 keys of block kb of a K tile
  auto qk = [&](const uint16_t* kt_lds, int kb) {
    const uint16_t* kl = kt_lds + k_lane + kb * 32 * D;
    f32x16 sc = ebias;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      sc = mfma32x32x16(*reinterpret_cast<const u32x4*>(kl + 256 * kk), qb[kk], sc);
    return sc;
  };
  // Score multipliers of a block's two 16-key halves (elements 0..7 are keys 0..15
  // of the block, elements 8..15 keys 16..31) and, with scales per page, the value
  // scales that go onto P: the softmax scale (times the pool's k_scale for FP8
  // pools) or, per (page, KV head), times each half's page scale.
  struct BlkScale {
    float ca, cb, va, vb;
  };
  auto blk_scale = [&](int vs, int kb) {
    if constexpr (PS) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(&pg_scales[vs][4 * kb]);
      return BlkScale{a.scale_log2 * t[0], a.scale_log2 * t[1], t[2], t[3]};
    } else {
      return BlkScale{a.scale_log2, a.scale_log2, 1.f, 1.f};
    }
  };
  // scaled row maximum of a block (log2 units)
  auto rowmax = [&](const f32x16& sc, const BlkScale& bs) {
    float ma = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
    for (int e = 3; e < 7; e += 2) ma = fmaxf(fmaxf(ma, sc[e]), sc[e + 1]);
    ma = fmaxf(ma, sc[7]);
    float mb = fmaxf(fmaxf(sc[8], sc[9]), sc[10]);
#pragma unroll
    for (int e = 11; e < 15; e += 2) mb = fmaxf(fmaxf(mb, sc[e]), sc[e + 1]);
    mb = fmaxf(mb, sc[15]);
    // both multipliers are positive, so scaling commutes with the maximum
    const float r = PS ? xor32_max(fmaxf(ma * bs.ca, mb * bs.cb))
                       : xor32_max(fmaxf(ma, mb)) * bs.ca;
    return ALI ? r + boff : r;
  };
  // Block map: the walk's tiles come from the list (entry of walk index u), and a
  // tile that this wave's query block does not list is masked whole.
  int* const bs_list = reinterpret_cast<int*>(pf_lds + L_::Q0);
  int bs_n = 0;
  auto bs_entry = [&](int u) { return bs_list[1 + (REV ? bs_n - 1 - u : u)]; };
  // The block's ALiBi offset (general variant), then -inf for keys past the end,
  // (causal) above the diagonal and (window) below a row's window; only blocks that
  // touch one of these boundaries need the second part.  Called once per block
  // (walk index u of its tile), right after its scores are formed and before they
  // are used.
  auto mask = [&](f32x16& sc, int kb0, int u) {
    if (ALI) boff = slope_log2 * (float)(kb0 - my_pos);
    if constexpr (BS) {
      // the wave's query block: bit 16 + (its first row - r_wg) / 64 of the entry
      if (!((bs_entry(u) >> (16 + (HP ? wave & 3 : wave) / 2)) & 1)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[e] = kNegInf;
        return;
      }
    }
    const bool need = (kb0 + 32 > L) || (kb0 + 31 > w_lim_min) || (GEN && kb0 < w_lo_max);
    if (__builtin_expect(need, 0)) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb0 + 8 * j + 4 * hh + i;
          if (key > lim || (GEN && key < lo_row)) sc[4 * j + i] = kNegInf;
        }
    }
  };
  // Online softmax in log2 units with a lazily moved reference: the running
  // reference m_run only moves (rescaling l and the accumulator) when a row's
  // scaled maximum exceeds it by more than kRescaleSlack, so P stays below
  // 2^kRescaleSlack and the result is unchanged -- the final normalisation uses
  // the same reference ("The Stack Below the Stack (Part 2)", 2.1 and 2.3).
  auto decide = [&](float mt) {
    const bool grow = mt > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mt : m_run;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
      m_run = m_new;
    }
  };
  // O^T += V^T P^T over block kb of a V tile
  auto pv = [&](const uint16_t* vt_lds, int kb, const u32x4& pb0, const u32x4& pb1) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint16_t* vl = vt_lds + (2 * kb + u) * PfLds<D>::REGION;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        const u32x2 lo = ds_read_tr16(vl + v_lane[0] + 512 * t);
        const u32x2 hi = ds_read_tr16(vl + v_lane[1] + 512 * t);
        acc[t] = mfma32x32x16(u32x4{lo[0], lo[1], hi[0], hi[1]}, u == 0 ? pb0 : pb1, acc[t]);
      }
    }
  };

  // exp2(s * scale_log2 - m_run) of a block, packed to the P^T operand layout
  // (pw[0..3]: keys 16 u + 4 hh + 0..3 with u = 0, pw[4..7] with u = 1), and the
  // lane's share of the block's row sum, added in fp32 before P is rounded to bf16
  // for P V.  (A row sum of the rounded pairs through v_dot2_f32_bf16 against
  // (1, 1) forms a serial chain that does not issue under the matrix cores' work
  // on gfx950: with one pipeline step's MFMAs in flight it held the matrix cores
  // at 68 % of their peak against 82 % with plain fp32 adds, two waves per SIMD.)
  auto exps = [&](const f32x16& sc, const BlkScale& bs, uint32_t* pw, float& ps) {
    const float neg_m0 = m_run == kNegInf ? 0.f : -m_run;
    const float neg_m = ALI ? neg_m0 + boff : neg_m0;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float c = e < 8 ? bs.ca : bs.cb;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], c, neg_m));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e + 1], c, neg_m));
      if constexpr (PS) {
        const float v = e < 8 ? bs.va : bs.vb;
        pw[e / 2] = pack_bf16x2(p0 * v, p1 * v);
      } else {
        pw[e / 2] = pack_bf16x2(p0, p1);
      }
      ps0 += p0;
      ps1 += p1;
    }
    ps = ps0 + ps1;
  };
  // The reference m_run is only checked after the fact: a block is exponentiated
  // against the current reference, and only when some lane's partial row sum
  // exceeds 2^kRescaleSlack (so P may have grown past that) does the wave take
  // the row maximum, move the reference, rescale l and the accumulator and redo
  // the block.  The accepted P are therefore bounded by 2^kRescaleSlack and the
  // result is the same as with an exact running maximum ("The Stack Below the
  // Stack (Part 2)", 2.1 and 2.3: any common reference gives the same quotient).
  auto settle = [&](const f32x16& sc, const BlkScale& bs, uint32_t* pw, float& ps) {
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(!(ps <= kSumLimit) || m_run == kNegInf), 0)) {
      const float m_new = fmaxf(m_run, rowmax(sc, bs));
      const float alpha = m_run == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
      m_run = m_new;
      exps(sc, bs, pw, ps);
    }
    l_run += ps;
  };
  // One pipeline step: exponentiate the pending block against the current
  // reference and accumulate its P V from V tile vp (block kbp), while computing
  // the scores of the next block from K tile kq (block kbq).  The instruction
  // order is written out: each MFMA is followed by the vector work that does not
  // depend on it, so the matrix cores and the vector ALU of one wave overlap;
  // operand reads run two MFMAs ahead.  sched_barrier keeps the compiler from
  // regrouping the chunks.
  //
  // FP8 pools: with wn >= 0 the step also widens this wave's share of tile wn (codes in
  // registers) into K stage wks and V stage wvs, a quarter after every other P V MFMA,
  // where the vector ALU has nothing else to do; the tile's publish then only waits.
  // The stages of the tile published next are not read during the step before it.
  auto step = [&](f32x16& s_pend, const uint16_t* kq, int kbq, int vsi, int kbp, int wn = -1,
                  int wks = 0, int wvs = 0) {
    constexpr int NK = D / 16;                 // QK MFMAs
    constexpr int EPK = 16 / NK;               // exponentials per QK MFMA
    constexpr int NV = 2 * (D / 32);           // PV MFMAs
    const uint16_t* vp = vst(vsi);
    const BlkScale bs = blk_scale(vsi, kbp);
    const float neg_m0 = m_run == kNegInf ? 0.f : -m_run;
    const float neg_m = ALI ? neg_m0 + boff : neg_m0;
    const uint16_t* kl = kq + k_lane + kbq * 32 * D;
    u32x4 kf[NK];
    kf[0] = *reinterpret_cast<const u32x4*>(kl);
    kf[1] = *reinterpret_cast<const u32x4*>(kl + 256);
    f32x16 sn = ebias;
    uint32_t pw[8];
    float pe[16];
    float ps0 = 0.f, ps1 = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      if (i + 2 < NK) kf[i + 2] = *reinterpret_cast<const u32x4*>(kl + 256 * (i + 2));
      sn = mfma32x32x16(kf[i], qb[i], sn);
#pragma unroll
      for (int e = EPK * i; e < EPK * (i + 1); e += 2) {
        const float c = e < 8 ? bs.ca : bs.cb;
        pe[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_pend[e], c, neg_m));
        pe[e + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_pend[e + 1], c, neg_m));
        if constexpr (PS) {
          const float v = e < 8 ? bs.va : bs.vb;
          pw[e / 2] = pack_bf16x2(pe[e] * v, pe[e + 1] * v);
        } else {
          pw[e / 2] = pack_bf16x2(pe[e], pe[e + 1]);
        }
        pin(pw[e / 2]);
      }
      // row sum (fp32, two chains) of the exponentials formed one chunk earlier
      if (i > 0) {
#pragma unroll
        for (int e = EPK * (i - 1); e < EPK * i; e += 2) {
          ps0 = e == 0 ? pe[e] : ps0 + pe[e];
          ps1 = e == 0 ? pe[e + 1] : ps1 + pe[e + 1];
        }
      }
      pin(ps0);
      pin(ps1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = EPK * (NK - 1); e < 16; e += 2) {
      ps0 += pe[e];
      ps1 += pe[e + 1];
    }
    float ps = ps0 + ps1;
    settle(s_pend, bs, pw, ps);
    const u32x4 pb0 = {pw[0], pw[1], pw[2], pw[3]};
    const u32x4 pb1 = {pw[4], pw[5], pw[6], pw[7]};
    // O^T += V^T P^T: MFMA i covers d-tile i % (D / 32) of 16-key half i / (D / 32)
    auto vfrag = [&](int i) {
      const uint16_t* vl =
          vp + (2 * kbp + i / (D / 32)) * PfLds<D>::REGION + 512 * (i % (D / 32));
      const u32x2 lo = ds_read_tr16(vl + v_lane[0]);
      const u32x2 hi = ds_read_tr16(vl + v_lane[1]);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 vf[NV];
    vf[0] = vfrag(0);
    vf[1] = vfrag(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i + 2 < NV) vf[i + 2] = vfrag(i + 2);
      const int t = i % (D / 32);
      acc[t] = mfma32x32x16(vf[i], i < D / 32 ? pb0 : pb1, acc[t]);
      if constexpr (F8) {
        // NV / 4 MFMAs per quarter (NV is 4 or 8)
        if (wn >= 0 && (i + 1) % (NV / 4) == 0) widen(wn, wks, wvs, i / (NV / 4));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    s_pend = sn;
  };

  // Software pipeline over 32-key blocks: while the matrix cores compute S of
  // block i + 1 and then O += P V of block i, the vector unit exponentiates block
  // i.  K of tiles t, t + 1 and V of tiles t - 1 .. t + 1 are resident, so one
  // barrier per tile suffices.
  // Key tiles are walked upwards, or (REV) from the last one down: with ALiBi the
  // scores grow towards a row's own position, so walking down sets the softmax
  // reference at the first block instead of moving it at nearly every block.  B0, B1:
  // the first and second 32-key block of a tile in walk order.
  constexpr int B0 = REV ? 1 : 0, B1 = 1 - B0;
  if constexpr (BS) {
    // the list: wave 0 reads the map entries of its query blocks for 1,024 tiles per
    // pass (lane l: tiles t + 64 i + l) and compacts the listed ones in order
    if (wave == 0) {
      const uint8_t* mrow = a.block_map + (size_t)b * a.bm_qb * a.bm_kb;
      const int qb0 = r_wg / 64;
      int count = 0;
      for (int tb = tile_lo; tb < tile_hi; tb += 64 * 16) {
        int f[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = tb + 64 * i + lane;
          const bool t_ok = t < tile_hi && t < a.bm_kb;
          int fl = 0;
#pragma unroll
          for (int k = 0; k < kPfBM / 64; ++k) {
            const int qb = qb0 + k;
            const uint8_t v =
                mrow[(size_t)min(qb, a.bm_qb - 1) * a.bm_kb + min(t, a.bm_kb - 1)];
            fl |= (t_ok && qb < a.bm_qb && v != 0) ? 1 << k : 0;
          }
          f[i] = fl;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint64_t bal = __builtin_amdgcn_ballot_w64(f[i] != 0);
          const int below = __builtin_amdgcn_mbcnt_hi(
              (uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
          if (f[i]) bs_list[1 + count + below] = (tb + 64 * i + lane) | (f[i] << 16);
          count += __builtin_popcountll(bal);
        }
      }
      if (lane == 0) bs_list[0] = count;
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the list is in LDS
    }
    block_sync();
    bs_n = __builtin_amdgcn_readfirstlane(bs_list[0]);
  }
  auto tile_at = [&](int u) {
    return BS ? bs_entry(u) & 0xffff : (REV ? tile_hi - 1 - u : tile_lo + u);
  };
  const int nt = BS ? bs_n : tile_hi - tile_lo;
  // Walking upwards, the blocks from the first key past this wave's last valid row
  // on are masked for all of its rows (causal), as are blocks past the sequence end:
  // the wave computes only its first G blocks (finishing the last of them) and for
  // the remaining tiles only moves its share and meets the barriers.  In the
  // diagonal region of a 256-row tile that leaves 28 of the 64 (wave, block) steps
  // to the other waves.  The steady loop below is the same for every wave; only
  // where a wave's blocks end does it take the short tail.
  const int w_last = min(r_w + 31, q_len - 1);              // last valid row of the wave
  const int w_key_end = __builtin_amdgcn_readfirstlane(min(
      w_hi_max, !a.causal ? L : (w_last < r_w ? 0 : min(L, shift + w_last + 1))));
  // finish the pending block (P from its scores, P V from V tile vp, block kbp)
  auto finish = [&](f32x16& sp, int vsi, int kbp) {
    const BlkScale bs = blk_scale(vsi, kbp);
    uint32_t pw[8];
    float ps;
    exps(sp, bs, pw, ps);
    settle(sp, bs, pw, ps);
    pv(vst(vsi), kbp, u32x4{pw[0], pw[1], pw[2], pw[3]}, u32x4{pw[4], pw[5], pw[6], pw[7]});
  };
  // stages of the walk's k-th tile: K (kc + k) mod 2, V (vc + k) mod 3; the next
  // item of a persistent work-group takes the stages after this item's last tile
  if constexpr (PER) {
    hd.kc = (kc + nt) & 1;
    hd.vc = (vc + nt) % 3;
  }
  // The next item of a persistent work-group, as far as its prefetch needs it: its
  // KV head, its block-table window and where this wave's share of its Q rows is.
  int nx_do = 0, nx_kvh = 0, nx_qok = 0, tab_nx = 0;
  const uint16_t* nx_q = a.q;
  uint32_t nx_qoff = 0;
  auto next_item = [&]() {
    if (hd.pn < 0) return;
    const PfWork nw = pf_work_of(a, hd.pn);
    const PfSetup ns = pf_setup<GEN>(a, nw, kPfBM, lane);
    if (!(ns.tile_hi > ns.tile_lo)) return;
    nx_do = 1;
    nx_kvh = ns.kvh;
    tab_nx = load_tab_of(a.block_tables + (size_t)nw.b * a.max_pages, ns.tile_lo);
    // Q rows r_wg + 32 wave .. of the next item, 16 bytes per lane and instruction:
    // lane i takes row i % 32, columns 16 kk + 8 (i / 32) .. (the Q^T operand's
    // layout), rows past the query run clamped to its last row (zeroed when read)
    const int lim_row = min(ns.q_len, a.Tq - ns.t0) - 1;
    nx_qok = lim_row >= 0;
    const int row0 = max(0, min(ns.r_wg + 32 * wave, lim_row));
    const int rel = max(0, min(ns.r_wg + 32 * wave + col, lim_row) - row0);
    nx_q = a.q + ((size_t)(ns.t0 + row0) * a.Hq + nw.h) * D;
    nx_qoff = (uint32_t)((rel * a.Hq * D + hh * 8) * 2);
  };
  // the next item's first tile and Q rows, issued as the tile after this item's last
  auto prefetch = [&](int ks, int vs) {
    issue_page(__builtin_amdgcn_readlane(tab_nx, 0), nx_kvh, ks, vs);
    hd.has = 1;
    hd.tab = tab_nx;
    if (nx_qok) {
      uint16_t* ql = pf_lds + L_::Q0 + wave * 32 * D;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) dma16(nx_q, nx_qoff + 32u * kk, ql + 512 * kk);
      hd.q_lds = 1;
    }
  };
  // DMA of the walk's k-th tile, or past the last one the next item's first
  auto issue_walk = [&](int k) {
    if (k < nt) {
      issue(tile_at(k), (kc + k) & 1, (vc + k) % 3);
    } else if constexpr (PER) {
      if (k == nt && nx_do) prefetch((kc + k) & 1, (vc + k) % 3);
    }
  };
  if (nt > 0) {
    base_t = BS ? (REV ? max(0, tile_at(0) - 63) : tile_at(0))
                : (REV ? max(0, tile_hi - 64) : tile_lo);
    tab = pre ? hd.tab : load_tab(base_t);
    int vs_cur = vc;                      // V stage of the walk's current tile
    int ks_cur = kc;                      // K stage of the walk's current tile
    if (!pre) issue(tile_at(0), kc, vc);
    publish(tile_at(0), kc, vc);
    if (q_pre) {
      const uint16_t* ql = pf_lds + L_::Q0 + wave * 32 * D + 8 * lane;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        qb[kk] = row_ok ? *reinterpret_cast<const u32x4*>(ql + 512 * kk) : u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (PER) next_item();
    issue_walk(1);
    // G: blocks this wave computes, in walk order (wave-uniform); with a block map,
    // the listed tiles' blocks that start below the wave's key end
    int G = REV ? 2 * nt : min(2 * nt, max(0, (w_key_end - tile_lo * kPfBN + 31) / 32));
    if constexpr (BS && !REV) {
      int c = 0;
      for (int i = lane; i < nt; i += 64) {
        const int k0 = (bs_list[1 + i] & 0xffff) * kPfBN;
        c += (k0 < w_key_end ? 1 : 0) + (k0 + 32 < w_key_end ? 1 : 0);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off);
      G = __builtin_amdgcn_readfirstlane(c);
    }
    // first block: scores, mask, first reference
    f32x16 s_pend;
    if (G > 0) {
      s_pend = qk(kst(ks_cur), B0);
      mask(s_pend, tile_at(0) * kPfBN + 32 * B0, 0);
      decide(rowmax(s_pend, blk_scale(vs_cur, B0)));
    }
    // iterations u whose two steps both score a computed block (2 u + 2 < G)
    const int U1 = G > 0 ? min(nt - 1, (G - 1) / 2) : 0;
    int u = 0;
    for (; u < U1; ++u) {
      const int kt = tile_at(u), kn = tile_at(u + 1);
      const int vs_next = vs_cur == 2 ? 0 : vs_cur + 1;
      // Waves w and w + 4 share a SIMD, and the older one wins its issue slots: left
      // alone it finishes each barrier interval first and waits while the younger one
      // runs by itself.  Issue priority instead goes to one wave group from here to
      // the next such point and to the other group after it, alternating per tile, so
      // each barrier interval's two steps are led by different waves (bf16: with FP8
      // pools, whose widening shares the P V phase, this measured slower).
      if constexpr (W == 8 && !F8) {
        if ((wave >= 4) == (u & 1)) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
      // first block of tile kt (pending) -> its second block (FP8: widening tile kn)
      step(s_pend, kst(ks_cur), B1, vs_cur, B0, F8 ? kn : -1, ks_cur ^ 1, vs_next);
      mask(s_pend, kt * kPfBN + 32 * B1, u);
      // second block of tile kt -> first block of tile kn.  FP8 pools: tile kn's codes
      // are in LDS already, so the registers take tile u + 2's codes before the barrier
      // (with scales per page the scale registers of tile kn are still to be published)
      if constexpr (F8 && !PS) {
        issue_walk(u + 2);
        publish(kn, ks_cur ^ 1, vs_next, true);
      } else {
        publish(kn, ks_cur ^ 1, vs_next, F8);
        issue_walk(u + 2);
      }
      step(s_pend, kst(ks_cur ^ 1), B0, vs_cur, B1);
      mask(s_pend, kn * kPfBN + 32 * B0, u + 1);
      vs_cur = vs_next;
      ks_cur ^= 1;
    }
    if constexpr (W == 8 && !F8) __builtin_amdgcn_s_setprio(0);
    if (u == nt - 1) {
      // the last tile: both of its blocks (G = 2 nt), only its first (G = 2 nt - 1),
      // or none (G = 0, one tile)
      const int kl = tile_at(u);
      if (G == 2 * nt) {
        step(s_pend, kst(ks_cur), B1, vs_cur, B0);
        mask(s_pend, kl * kPfBN + 32 * B1, u);
        finish(s_pend, vs_cur, B1);
      } else if (G == 2 * nt - 1) {
        finish(s_pend, vs_cur, B0);
      }
    } else {
      // this wave's blocks end in tile u (G = 2 u + 1 or 2 u + 2) or there are none
      const int kt = tile_at(u), kn = tile_at(u + 1);
      const int vs_next = vs_cur == 2 ? 0 : vs_cur + 1;
      if (G == 2 * u + 2) {
        step(s_pend, kst(ks_cur), B1, vs_cur, B0);
        mask(s_pend, kt * kPfBN + 32 * B1, u);
      } else if (G == 2 * u + 1) {
        finish(s_pend, vs_cur, B0);
      }
      publish(kn, ks_cur ^ 1, vs_next);
      issue_walk(u + 2);
      if (G == 2 * u + 2) finish(s_pend, vs_cur, B1);
      vs_cur = vs_next;
      ks_cur ^= 1;
      // the remaining tiles: this wave's share of each is moved, nothing computed
      for (++u; u + 1 < nt; ++u) {
        const int vs_n = vs_cur == 2 ? 0 : vs_cur + 1;
        publish(tile_at(u + 1), ks_cur ^ 1, vs_n);
        issue_walk(u + 2);
        vs_cur = vs_n;
        ks_cur ^= 1;
      }
    }
  }

  if (!row_ok) return;
  const float l_tot = xor32_sum(l_run);
  const bool live = l_tot > 0.f;
  const float inv = live ? (F8 ? a.v_scale : 1.f) / l_tot : 0.f;
  const float lse = live ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  if (s.parts > 1) {
    // this part's normalised output and lse, merged by the prefill merge kernel
    const size_t prow = ((size_t)(t0 + my_row) * a.Hq + h) * a.S + part;
    float* po = a.part_o + prow * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(po + 32 * t + 8 * j + 4 * hh) =
            f32x4{acc[t][4 * j] * inv, acc[t][4 * j + 1] * inv, acc[t][4 * j + 2] * inv,
                  acc[t][4 * j + 3] * inv};
    if (hh == 0) a.part_lse[prow] = lse;
    return;
  }
  uint16_t* op = a.out + ((size_t)(t0 + my_row) * a.Hq + h) * D;
  // lane holds O^T[32 t + 8 j + 4 hh + i][col]
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x2 w = {pack_bf16x2(acc[t][4 * j] * inv, acc[t][4 * j + 1] * inv),
                       pack_bf16x2(acc[t][4 * j + 2] * inv, acc[t][4 * j + 3] * inv)};
      *reinterpret_cast<u32x2*>(op + 32 * t + 8 * j + 4 * hh) = w;
    }
  if (hh == 0 && a.lse_out) a.lse_out[(size_t)(t0 + my_row) * a.Hq + h] = lse;
}

// One work-group per item of the plain grid (item = blockIdx.x).
template <int D, int W, bool GEN, bool F8, bool REV, bool PS = false, bool BS = false,
          bool HP = false>
__global__ __launch_bounds__(64 * W, 8 / W) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) uint16_t pf_lds[];
  const PfWork w = pf_work_of(a, blockIdx.x);
  const PfSetup s = pf_setup<GEN>(a, w, HP ? 128 : 32 * W, threadIdx.x & 63);
  if (!s.ok) return;
  PfHand hd{};
  pf_item<D, W, GEN, F8, REV, PS, false, BS, HP>(a, w, s, hd, pf_lds);
}

// Persistent work-groups: one per CU, a multiple of 8 of them, each working through
// items of the plain grid's order one after the other, with the hand-over above.  The
// work-group j sits on XCD j mod 8 and takes only that XCD's items (ids p with
// p mod 8 = j mod 8, the ids the plain grid sends there), in rounds over the XCD's
// work-groups that alternate in direction (round r hands the XCD's items
// r P8 .. r P8 + P8 - 1, P8 work-groups per XCD, to its work-groups in ascending, then
// descending order), so that the heaviest-first order of the items pairs heavy with
// light ones on every work-group.
template <int D, int W>
__global__ __launch_bounds__(64 * W, 1) void prefill_persist_kernel(PrefillArgs a,
                                                                    int n_items) {
  extern __shared__ __align__(16) uint16_t pf_lds[];
  const int x = blockIdx.x & 7, jx = blockIdx.x >> 3, p8 = gridDim.x >> 3;
  const int lane = threadIdx.x & 63;
  auto item_at = [&](int r) { return 8 * (r * p8 + ((r & 1) ? p8 - 1 - jx : jx)) + x; };
  // the first item of round r or later that has work, or -1
  auto find = [&](int r) {
    for (;; ++r) {
      const int p = item_at(r);
      if (p >= n_items) return -1;
      if (pf_setup<false>(a, pf_work_of(a, p), 32 * W, lane).ok) return r;
    }
  };
  int r = find(0);
  if (r < 0) return;
  PfHand hd{};
  for (;;) {
    const PfWork w = pf_work_of(a, item_at(r));
    const PfSetup s = pf_setup<false>(a, w, 32 * W, lane);
    const int rn = find(r + 1);
    hd.pn = rn < 0 ? -1 : item_at(rn);
    pf_item<D, W, false, false, false, false, true>(a, w, s, hd, pf_lds);
    if (rn < 0) return;
    r = rn;
  }
}

// One launch for a step's prefill query runs and decode rows over the same pools (a
// kernel that serves both kinds of request of a step: "Inside Ion: Custom Attention
// Kernels for NVIDIA Grace", "IonAttention in One Paragraph").  Work-groups 0 ..
// n_dg - 1 each run eight decode items, one per wave, as the one-wave decode
// partition kernel runs them (item 8 x work-group + wave; KV head fastest, then
// partition, then sequence), staging their K rows in the start of the dynamic LDS; the
// work-groups after them run the plain prefill grid's items (256-row query tiles,
// plain bf16 variant) in its order.  The decode items come first so that they run
// while the prefill's heaviest tiles start, and the CUs they free take prefill
// items; n_dg is a multiple of 8, so prefill item p runs on XCD p mod 8 as in the
// plain grid.
// F8: FP8 E4M3 pools (the plain FP8 prefill variant, or with PS, scales per (page, KV
// head), the general one, which reads them).
template <int D, bool F8 = false, bool PS = false>
__global__ __launch_bounds__(512, 1) void mixed_kernel(PrefillArgs a, DecodeArgs d, int n_dg) {
  extern __shared__ __align__(16) uint16_t pf_lds[];
  static_assert(8 * 32 * KRows<D>::LROW <= PfLds<D>::TILE * 5, "decode staging fits the LDS");
  if ((int)blockIdx.x < n_dg) {
    const int i = 8 * blockIdx.x + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int per_b = d.Hkv * d.S;
    if (i >= per_b * d.B) return;
    const int b = i / per_b;
    const int r = i - b * per_b;
    const int split = r / d.Hkv;
    decode_item<D, 1, F8, false, PS, true>(d, r - split * d.Hkv, split, b);
    return;
  }
  const PfWork w = pf_work_of(a, blockIdx.x - n_dg);
  const PfSetup s = pf_setup<PS>(a, w, 256, threadIdx.x & 63);
  if (!s.ok) return;
  PfHand hd{};
  pf_item<D, 8, PS, F8, false, PS, false>(a, w, s, hd, pf_lds);
}

// Merge of the query tiles that were cut into key-range parts ("The Stack Below
// the Stack (Part 2)", section 2.2, step 3: with m the largest part lse, weights
// exp(lse_c - m), lse = m + ln sum).  A work-group covers kMergePasses * 256 / (D / 4)
// rows of one (query head, sequence, query tile); each thread merges 4 output columns
// of one row per pass, with all of that row's loads issued before any is used, so a
// pass costs about two memory round trips.  Work-groups of tiles with one part
// (written by the prefill kernel) return at once.
constexpr int kMergeThreads = 256;
constexpr int kMergePasses = 4;     // rows per thread: most work-groups of a launch only
                                    // find their tile unsplit and return, so fewer,
                                    // larger work-groups finish the launch sooner
constexpr int kMaxParts = 16;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(PrefillArgs a, int bm) {
  constexpr int CH = D / 4;                  // 4-column chunks per row
  constexpr int RPP = kMergeThreads / CH;    // rows per pass
  constexpr int RPB = RPP * kMergePasses;    // rows per work-group
  const int rblocks = bm / RPB;
  const int p = blockIdx.x / rblocks;
  const int rb = blockIdx.x - p * rblocks;
  const int h = p % a.Hq;
  const int r = p / a.Hq;
  const int b = r % a.B;
  const int qt = r / a.B;
  const int t0 = a.cu_seqlens_q[b];
  const int q_len = a.cu_seqlens_q[b + 1] - t0;
  const int r_wg = qt * bm;
  if (r_wg >= q_len) return;
  int L = a.seq_lens_k[b];
  const int cap = a.max_pages * a.page_size;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const PfTiles tw = a.window > 0 || a.key_lo
                        ? pf_tiles<true>(a, L, q_len, r_wg, bm, t0, threadIdx.x & 63)
                        : pf_tiles<false>(a, L, q_len, r_wg, bm, t0, threadIdx.x & 63);
  if (tw.parts <= 1) return;
  const int c = threadIdx.x % CH;
  for (int pass = 0; pass < kMergePasses; ++pass) {
    const int row = r_wg + rb * RPB + pass * RPP + threadIdx.x / CH;
    if (row >= q_len || t0 + row >= a.Tq) return;
    const size_t orow = (size_t)(t0 + row) * a.Hq + h;
    const size_t prow = orow * a.S;
    float lse[kMaxParts];
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k) lse[k] = k < tw.parts ? a.part_lse[prow + k] : kNegInf;
    f32x4 o[kMaxParts];
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k)
      if (k < tw.parts) o[k] = *reinterpret_cast<const f32x4*>(a.part_o + (prow + k) * D + 4 * c);
    float m = kNegInf;
#pragma unroll
    for (int k = 0; k < kMaxParts; ++k) m = fmaxf(m, lse[k]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float tot = 0.f;
    if (m != kNegInf) {
#pragma unroll
      for (int k = 0; k < kMaxParts; ++k)
        if (k < tw.parts) {
          const float w = __expf(lse[k] - m);
          tot += w;
          acc += w * o[k];
        }
    }
    const bool live = tot > 0.f;
    const float inv = live ? 1.f / tot : 0.f;
    *reinterpret_cast<u32x2*>(a.out + orow * D + 4 * c) =
        u32x2{pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    if (c == 0 && a.lse_out) a.lse_out[orow] = live ? m + __logf(tot) : kNegInf;
  }
}

// query-tile slots per (head, sequence) in the grid: n_qt, rounded up to a multiple of
// xcd_split in the unit-major order (the surplus work-groups return at once)
static int prefill_grid_tiles(const PrefillArgs& a) {
  return a.xcd_groups ? (a.n_qt + a.xcd_split - 1) / a.xcd_split * a.xcd_split : a.n_qt;
}

// compute units of the current device (read once per device)
static hipError_t device_cus(int* cus) {
  static std::atomic<int> known[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int n = known[dev].load(std::memory_order_acquire);
  if (n == 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    known[dev].store(n, std::memory_order_release);
  }
  *cus = n;
  return hipSuccess;
}

// items of the plain grid (one per work-group there)
static int prefill_items(const PrefillArgs& a) {
  return a.Hq / (a.hp ? 2 : 1) * a.B * prefill_grid_tiles(a) * a.S;
}

// persistent work-groups for a launch: one per CU, a multiple of 8, no more than
// the items need
static int prefill_persist_groups(const PrefillArgs& a, int cus) {
  const int n = prefill_items(a);
  return std::max(8, std::min(cus / 8 * 8, (n + 7) / 8 * 8));
}

template <int D>
static hipError_t launch_prefill_persist(const PrefillArgs& a, hipStream_t stream,
                                         const KernelEvents& ev) {
  constexpr size_t lds = PfLds<D>::BYTES + PfLds<D>::q_bytes(8);
  static std::atomic<int> state[kMaxDevices];
  hipError_t e = lds_attribute_once(
      state, reinterpret_cast<const void*>(prefill_persist_kernel<D, 8>), lds);
  if (e != hipSuccess) return e;
  int cus = 0;
  e = device_cus(&cus);
  if (e != hipSuccess) return e;
  launch_kernel(prefill_persist_kernel<D, 8>, dim3(prefill_persist_groups(a, cus)), dim3(512),
                (uint32_t)lds, stream, ev, a, prefill_items(a));
  return hipGetLastError();
}

template <int D, int W, bool GEN, bool F8, bool REV, bool PS = false, bool BS = false,
          bool HP = false>
static hipError_t launch_prefill_w(const PrefillArgs& a, hipStream_t stream,
                                   const KernelEvents& ev) {
  constexpr size_t lds = PfLds<D>::BYTES + (BS ? kBsListBytes : 0);
  if constexpr (lds > 65536) {
    static std::atomic<int> state[kMaxDevices];
    const hipError_t e = lds_attribute_once(
        state, reinterpret_cast<const void*>(prefill_kernel<D, W, GEN, F8, REV, PS, BS, HP>),
        lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(prefill_items(a));
  launch_kernel(prefill_kernel<D, W, GEN, F8, REV, PS, BS, HP>, grid, dim3(64 * W),
                (uint32_t)lds, stream, ev, a);
  return hipGetLastError();
}

// the sliding-window bound and the ALiBi bias are compiled only into the general
// variant
template <int D, int W>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream,
                                   const KernelEvents& ev) {
  if (a.kv_fp8) {
    if constexpr (W == 8) {
      if (a.hp) {
        if (a.block_map) {
          if (a.k_scales)
            return launch_prefill_w<D, 8, true, true, false, true, true, true>(a, stream, ev);
          return a.alibi ? launch_prefill_w<D, 8, true, true, true, false, true, true>(a, stream, ev)
                         : launch_prefill_w<D, 8, true, true, false, false, true, true>(a, stream, ev);
        }
        if (a.k_scales)
          return launch_prefill_w<D, 8, true, true, false, true, false, true>(a, stream, ev);
        if (a.alibi) return launch_prefill_w<D, 8, true, true, true, false, false, true>(a, stream, ev);
        return a.window > 0 || a.key_lo
                   ? launch_prefill_w<D, 8, true, true, false, false, false, true>(a, stream, ev)
                   : launch_prefill_w<D, 8, false, true, false, false, false, true>(a, stream, ev);
      }
    }
    if (a.block_map) {
      // block maps take 256-row work-groups (prefill_waves)
      if constexpr (W == 8) {
        if (a.k_scales) return launch_prefill_w<D, 8, true, true, false, true, true>(a, stream, ev);
        return a.alibi ? launch_prefill_w<D, 8, true, true, true, false, true>(a, stream, ev)
                       : launch_prefill_w<D, 8, true, true, false, false, true>(a, stream, ev);
      } else {
        return hipErrorInvalidValue;
      }
    }
    // scales per (page, KV head) (the entry point refuses them with ALiBi slopes)
    if (a.k_scales) return launch_prefill_w<D, W, true, true, false, true>(a, stream, ev);
    if (a.alibi) return launch_prefill_w<D, W, true, true, true>(a, stream, ev);
    return a.window > 0 || a.key_lo ? launch_prefill_w<D, W, true, true, false>(a, stream, ev)
                                    : launch_prefill_w<D, W, false, true, false>(a, stream, ev);
  }
  if (a.block_map) {
    // block maps take 256-row work-groups (prefill_waves)
    if constexpr (W == 8) {
      if (a.hp)
        return a.alibi ? launch_prefill_w<D, 8, true, false, true, false, true, true>(a, stream, ev)
                       : launch_prefill_w<D, 8, true, false, false, false, true, true>(a, stream, ev);
      return a.alibi ? launch_prefill_w<D, 8, true, false, true, false, true>(a, stream, ev)
                     : launch_prefill_w<D, 8, true, false, false, false, true>(a, stream, ev);
    } else {
      return hipErrorInvalidValue;
    }
  }
  if constexpr (W == 8) {
    if (a.hp && a.alibi)
      return launch_prefill_w<D, 8, true, false, true, false, false, true>(a, stream, ev);
    if (a.hp && (a.window > 0 || a.key_lo))
      return launch_prefill_w<D, 8, true, false, false, false, false, true>(a, stream, ev);
  }
  if (a.alibi) return launch_prefill_w<D, W, true, false, true>(a, stream, ev);
  if (a.window > 0 || a.key_lo) return launch_prefill_w<D, W, true, false, false>(a, stream, ev);
  if (W == 8 && a.persist) return launch_prefill_persist<D>(a, stream, ev);
  if constexpr (W == 8) {
    if (a.hp) return launch_prefill_w<D, 8, false, false, false, false, false, true>(a, stream, ev);
  }
  return launch_prefill_w<D, W, false, false, false>(a, stream, ev);
}

// Waves per work-group: 8 (256 query rows, half the K/V traffic per row) when the
// longest query run fills two of them, else 4 (on MI355X, 512-row chunks over long
// histories ran 8 % faster with 256-row work-groups than with 128-row ones).  FP8 pools with ALiBi always take 8: the
// 4-wave variant stages twice the codes per lane in registers, and with the bias
// terms on top it would not fit the 256 registers of a two-wave-per-SIMD launch.
int prefill_waves(int max_q_len, bool fp8_alibi) {
  return max_q_len >= PF_W8_MIN || fp8_alibi ? 8 : 4;
}
static int prefill_waves(const PrefillArgs& a) {
  if (a.block_map) return 8;
  return prefill_waves(a.max_q_len, a.kv_fp8 && a.alibi != nullptr);
}

// Paired heads (a work-group of 8 waves takes two query heads of one KV group over 128
// rows instead of one head over 256): for every unsplit 8-wave launch with an even
// GQA group, bf16 or FP8 pools, with or without a window, ALiBi, document masks or a
// block map: a work-group then walks the union of 128 rows' key ranges (windows,
// documents) or of two query blocks' listed tiles instead of 256 rows' or four
// blocks'.  Each K/V tile copied into LDS then serves two heads' rows, the
// work-groups are as many as with 256-row tiles, and a causal
// work-group's diagonal spans 128 keys instead of 256, so fewer of its (wave, block)
// steps are masked whole.  A row's result does not depend on the tile height when
// the keys are not split, so the output bits are those of the 256-row launch; with
// key parts the parts follow the tile height, and the planner and the merge count
// 256-row tiles, so split launches keep them.
static bool prefill_pairs(const PrefillArgs& a, int W) {
  return W == 8 && a.S <= 1 && !a.persist && a.G % 2 == 0;
}

static PrefillArgs prefill_shape(const PrefillArgs& a_in, int W, bool pairs = false) {
  PrefillArgs a = a_in;
  a.hp = pairs ? 1 : 0;
  const int rows = pairs ? 128 : 32 * W;       // query rows per tile
  a.n_qt = (a.max_q_len + rows - 1) / rows;
  // XCD units: groups, or m rank classes of each group with groups * m a multiple of
  // 8.  Only for m <= 2 and when every unit gets a tile rank (n_qt >= m), else the
  // plain order: with 4 or 8 classes most XCDs fetch most of a group's K/V anyway,
  // while the unit order gives up the global heaviest-first packing (measured on
  // MI355X: 5 x 2048 causal rows, Hq 16 / Hkv 2, 127 us in 4 classes against 112.5 us
  // head-major; 1 x 8192 and 3 x 4096 at Hkv 4 in 2 classes 2-2.5 % faster than
  // head-major).
  const int groups = a.B * a.Hkv;
  int m = 1;
  while ((groups * m) % 8) m *= 2;
  a.xcd_split = m;
  a.xcd_groups = a.n_qt >= m && m <= 2 ? groups * m / 8 : 0;
  if (a.S < 1) a.S = 1;
  return a;
}

hipError_t launch_prefill_merge(const PrefillArgs& a_in, hipStream_t stream, char* desc,
                                size_t desc_len, int waves) {
  const int W = waves > 0 ? waves : prefill_waves(a_in);
  const PrefillArgs a = prefill_shape(a_in, W);
  const int rows_per_wg = kMergeThreads / (a.D / 4) * kMergePasses;
  dim3 grid(a.Hq * a.B * a.n_qt * (32 * W / rows_per_wg));
  if (a.D == 128)
    hipLaunchKernelGGL(prefill_merge_kernel<128>, grid, dim3(kMergeThreads), 0, stream, a,
                       32 * W);
  else
    hipLaunchKernelGGL(prefill_merge_kernel<64>, grid, dim3(kMergeThreads), 0, stream, a,
                       32 * W);
  snprintf(desc, desc_len, "prefill_merge<D=%d> grid=%u (query tiles x heads x %d-row blocks) "
           "parts<=%d", a.D, grid.x, rows_per_wg, a.S);
  return hipGetLastError();
}

template <int D, bool F8, bool PS>
static hipError_t launch_mixed_v(const PrefillArgs& a, const DecodeArgs& d, int n_dg, int n_pf,
                                 hipStream_t stream, const KernelEvents& ev) {
  constexpr size_t lds = PfLds<D>::BYTES;
  static std::atomic<int> state[kMaxDevices];
  const hipError_t e =
      lds_attribute_once(state, reinterpret_cast<const void*>(mixed_kernel<D, F8, PS>), lds);
  if (e != hipSuccess) return e;
  launch_kernel(mixed_kernel<D, F8, PS>, dim3(n_dg + n_pf), dim3(512), (uint32_t)lds, stream,
                ev, a, d, n_dg);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_mixed_d(const PrefillArgs& a, const DecodeArgs& d, int n_dg, int n_pf,
                                 hipStream_t stream, const KernelEvents& ev) {
  const bool fp8 = a.kv_fp8 || d.kv_fp8;
  const bool ps = a.k_scales || d.k_scales;
  if (fp8 && ps) return launch_mixed_v<D, true, true>(a, d, n_dg, n_pf, stream, ev);
  if (fp8) return launch_mixed_v<D, true, false>(a, d, n_dg, n_pf, stream, ev);
  return launch_mixed_v<D, false, false>(a, d, n_dg, n_pf, stream, ev);
}

long long mixed_prefill_items(const PrefillArgs& p) {
  if (p.B <= 0 || p.max_q_len <= 0) return 0;
  return prefill_items(prefill_shape(p, 8));
}

hipError_t launch_mixed(const PrefillArgs& p_in, const DecodeArgs& d, hipStream_t stream,
                        char* desc, size_t desc_len, const KernelEvents& ev) {
  const int D = p_in.B > 0 ? p_in.D : d.D;
  PrefillArgs a = p_in;
  int n_pf = 0;
  if (a.B > 0) {
    a = prefill_shape(p_in, 8);
    n_pf = prefill_items(a);
  }
  const long long n_dec = d.B > 0 ? (long long)d.Hkv * d.S * d.B : 0;
  const int n_dg = (int)(((n_dec + 7) / 8 + 7) / 8 * 8);
  if (n_dg + (long long)n_pf > 0x7fffffffll) return hipErrorInvalidValue;
  if (n_dg + n_pf == 0) {
    snprintf(desc, desc_len, "mixed: nothing to do");
    return hipSuccess;
  }
  const hipError_t e = D == 128 ? launch_mixed_d<128>(a, d, n_dg, n_pf, stream, ev)
                                : launch_mixed_d<64>(a, d, n_dg, n_pf, stream, ev);
  const bool fp8 = a.kv_fp8 || d.kv_fp8;
  snprintf(desc, desc_len,
           "mixed<D=%d,%s> grid=%d: %d decode work-groups (%lld one-wave items: %d KV heads x %d "
           "splits x %d rows) then %d prefill items (256-row tiles, %d key parts, %s) "
           "block=512 lds=%zu",
           D,
           fp8 ? (a.k_scales || d.k_scales ? "fp8-e4m3 scales per page" : "fp8-e4m3") : "bf16",
           n_dg + n_pf, n_dg, n_dec, d.Hkv, d.S, d.B, n_pf, a.S,
           a.xcd_groups ? "KV groups per XCD" : "head-major",
           D == 128 ? PfLds<128>::BYTES : PfLds<64>::BYTES);
  return e;
}

hipError_t launch_prefill(const PrefillArgs& a_in, hipStream_t stream, char* desc,
                          size_t desc_len, const KernelEvents& ev) {
  const int W = prefill_waves(a_in);
  const PrefillArgs a = prefill_shape(a_in, W, prefill_pairs(a_in, W));
  hipError_t e;
  if (a.D == 128)
    e = W == 8 ? launch_prefill_t<128, 8>(a, stream, ev) : launch_prefill_t<128, 4>(a, stream, ev);
  else
    e = W == 8 ? launch_prefill_t<64, 8>(a, stream, ev) : launch_prefill_t<64, 4>(a, stream, ev);
  char order[64];
  if (!a.xcd_groups)
    snprintf(order, sizeof(order), "head-major");
  else if (a.xcd_split == 1)
    snprintf(order, sizeof(order), "KV groups per XCD, group-major");
  else
    snprintf(order, sizeof(order), "KV groups in %d rank classes per XCD, unit-major",
             a.xcd_split);
  const bool per = W == 8 && a.persist && !a.kv_fp8 && !a.alibi && a.window == 0 && !a.key_lo &&
                   !a.block_map;
  char pers[96] = "";
  int cus = 0;
  if (per && device_cus(&cus) == hipSuccess)
    snprintf(pers, sizeof(pers), ", persistent: %d work-groups with next-item prefetch",
             prefill_persist_groups(a, cus));
  const size_t lds = (a.D == 128 ? PfLds<128>::BYTES : PfLds<64>::BYTES) +
                     (per ? (a.D == 128 ? PfLds<128>::q_bytes(8) : PfLds<64>::q_bytes(8)) : 0) +
                     (a.block_map ? kBsListBytes : 0);
  snprintf(desc, desc_len,
           "prefill<D=%d,BM=%d,BN=%d,mfma32x32x16,%s%s%s> grid=%d (%d heads x %d seqs x %d "
           "q-tiles x %d key parts, %s%s) block=%d lds=%zu",
           a.D, a.hp ? 128 : 32 * W, kPfBN,
           a.kv_fp8 ? (a.k_scales ? "fp8-e4m3-widened,scales per page" : "fp8-e4m3-widened")
                    : "lds-dma",
           a.block_map ? ",block map" : "", a.hp ? ",paired heads" : "",
           prefill_items(a), a.Hq, a.B, a.n_qt, a.S, order, pers, 64 * W, lds);
  return e;
}

}  // namespace pa
