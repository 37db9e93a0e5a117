// The decode item: the per-chunk loads, the K staging through LDS and the walk of one
// (sequence, KV head, partition) item, shared by the decode partition kernel and the
// mixed-step kernel.
//
// One work-group of W waves owns one (sequence b, KV head, partition) triple.
// The partition's keys are walked in 32-key chunks, each wave taking a contiguous
// run of them; each wave streams its chunks straight from the page pools into registers
// (16-byte loads, next chunk in flight while the current one computes), so the
// kernel reads every attended K/V byte exactly once -- decode is bound by those
// reads ("8. Kernels and Attention Backends", "Counting attention's traffic").
//
// Per chunk, with G = Hq / Hkv query heads sharing the KV head (padded to 16):
//   S^T[32 keys x 16 heads] = K Q^T      two 16x16x32 bf16 MFMA tiles per 32 d
//   online softmax over keys per head    running max and sum, rescale on growth
//                                        ("The Stack Below the Stack (Part 2)", 2.1)
//   O^T[D x 16 heads] += V^T P^T         P rounded to bf16, 16x16x32 MFMA per 16 d
// Orientation is chosen so that every per-head statistic lives in lane % 16 and
// no operand needs a cross-lane move: the S^T accumulator is already the B operand
// layout of P^T, and V is transposed inside each lane with byte permutes
// (each lane loads 8 keys x D/16 contiguous values and regroups them per d).
//
// At the end the W waves merge through LDS and the work-group writes either the
// final bf16 output (one partition) or the partition's normalised partial output
// and natural-log lse, which the split-K reduce kernel merges ("The Stack Below the
// Stack (Part 2)", section 2.2: a second kernel combines the chunks).  Merging in
// the last-arriving work-group instead was measured slower on MI355X: the partials
// must then bypass the per-XCD L2 caches.
#pragma once
#include <limits.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pa {

// Key and value scales of the two 16-key halves of a chunk (FP8 pools with scales
// per (page, KV head)).
struct ChunkScales {
  float k0, k1, v0, v1;
};

template <int D>
struct DecodeChunk {
  u32x4 ka[D / 32];          // K row (chunk key l%16), d in [D/4 * g, D/4 * (g+1))
  u32x4 kb[D / 32];          // K row (chunk key 16 + l%16), same d range
  uint32_t v[8][D / 32];     // V rows of the lane's 8 keys, d in [D/16 * n, D/16 * (n+1))
  uint32_t v8[8][D / 64];    // FP8 pools: the same values as raw E4M3 codes
};

// K of a chunk in whole-row order: instruction i covers rows RPI*i .. RPI*i+RPI-1
// (RPI = 512 / D rows of D bf16), each row read by D/8 consecutive lanes, so every
// load instruction consumes whole cache lines and can stream past the caches.
// The rows are then regrouped through LDS into the MFMA operand layout.
template <int D>
struct KRows {
  static constexpr int LPR = D / 8;          // lanes per row (16 B each)
  static constexpr int RPI = 64 / LPR;       // rows per load instruction
  static constexpr int NI = 32 / RPI;        // load instructions per 32-key chunk
  static constexpr int LROW = D + 8;         // LDS row pitch (bf16), 16 B pad
  u32x4 r[NI];
};

// FP8 pools: a row is D bytes, read 16 bytes (16 codes) per lane, RPI8 rows per
// instruction; the codes are widened to bf16 (exactly: every E4M3 value is a bf16
// value) on their way into the same LDS tile.
template <int D>
struct KRows8 {
  static constexpr int LPR = D / 16;
  static constexpr int RPI = 64 / LPR;
  static constexpr int NI = 32 / RPI;
};

template <int D>
__device__ __forceinline__ void decode_load_k_rows8(KRows<D>& k, const uint8_t* kbase, int pg0,
                                                    int pg1, int c0, const DecodeArgs& a,
                                                    int lane) {
  using R = KRows8<D>;
  const int psm = a.page_size - 1;
  const int rs = a.Hkv * D;
  const size_t page_elems = (size_t)a.page_size * rs;
  const int sub = lane / R::LPR;
  const int off = (lane % R::LPR) * 16;
#pragma unroll
  for (int i = 0; i < R::NI; ++i) {
    const int row = R::RPI * i + sub;
    const int pg = row < 16 ? pg0 : pg1;
    k.r[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
        kbase + (size_t)pg * page_elems + ((c0 + row) & psm) * rs + off));
  }
}

// four E4M3 codes (bytes 0..3) -> two packed bf16 pairs (bytes 0,1 and 2,3)
__device__ __forceinline__ u32x2 fp8x4_to_bf16(uint32_t w) {
  return u32x2{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

template <int D>
__device__ __forceinline__ void decode_k8_to_lds(const KRows<D>& k, uint16_t* kl, int lane) {
  using R = KRows8<D>;
  const int sub = lane / R::LPR;
  const int off = (lane % R::LPR) * 16;
#pragma unroll
  for (int i = 0; i < R::NI; ++i) {
    const u32x2 w0 = fp8x4_to_bf16(k.r[i][0]), w1 = fp8x4_to_bf16(k.r[i][1]);
    const u32x2 w2 = fp8x4_to_bf16(k.r[i][2]), w3 = fp8x4_to_bf16(k.r[i][3]);
    const u32x4 a = {w0[0], w0[1], w1[0], w1[1]};
    const u32x4 b = {w2[0], w2[1], w3[0], w3[1]};
    uint16_t* p = kl + (R::RPI * i + sub) * KRows<D>::LROW + off;
    *reinterpret_cast<u32x4*>(p) = a;
    *reinterpret_cast<u32x4*>(p + 8) = b;
  }
}

template <int D>
__device__ __forceinline__ void decode_load_k_rows(KRows<D>& k, const uint16_t* kbase, int pg0,
                                                   int pg1, int c0, const DecodeArgs& a,
                                                   int lane) {
  const int psm = a.page_size - 1;
  const int rs = a.Hkv * D;
  const size_t page_elems = (size_t)a.page_size * rs;
  const int sub = lane / KRows<D>::LPR;
  const int off = (lane % KRows<D>::LPR) * 8;
#pragma unroll
  for (int i = 0; i < KRows<D>::NI; ++i) {
    const int row = KRows<D>::RPI * i + sub;           // key c0 + row
    const int pg = row < 16 ? pg0 : pg1;
    const uint16_t* p = kbase + (size_t)pg * page_elems + ((c0 + row) & psm) * rs + off;
    k.r[i] = ld16_nt(p);
  }
}

template <int D>
__device__ __forceinline__ void decode_k_to_lds(const KRows<D>& k, uint16_t* kl, int lane) {
  const int sub = lane / KRows<D>::LPR;
  const int off = (lane % KRows<D>::LPR) * 8;
#pragma unroll
  for (int i = 0; i < KRows<D>::NI; ++i)
    *reinterpret_cast<u32x4*>(kl + (KRows<D>::RPI * i + sub) * KRows<D>::LROW + off) = k.r[i];
}

template <int D>
__device__ __forceinline__ void decode_k_from_lds(DecodeChunk<D>& c, const uint16_t* kl, int n,
                                                  int g) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    c.ka[kk] = *reinterpret_cast<const u32x4*>(kl + n * KRows<D>::LROW + (D / 4) * g + 8 * kk);
    c.kb[kk] =
        *reinterpret_cast<const u32x4*>(kl + (16 + n) * KRows<D>::LROW + (D / 4) * g + 8 * kk);
  }
}

template <int D>
__device__ __forceinline__ void decode_load_v(DecodeChunk<D>& c, const uint16_t* vbase,
                                              int pg0, int pg1, int c0, const DecodeArgs& a,
                                              int n, int g) {
  constexpr int DPL = D / 16;
  const int psm = a.page_size - 1;
  const int rs = a.Hkv * D;
  const size_t page_elems = (size_t)a.page_size * rs;
  const uint16_t* va = vbase + (size_t)pg0 * page_elems + ((c0 + 4 * g) & psm) * rs + DPL * n;
  const uint16_t* vb = vbase + (size_t)pg1 * page_elems + ((c0 + 16 + 4 * g) & psm) * rs +
                       DPL * n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (D == 128) {
      u32x4 x = ld16_nt(va + i * rs);
      u32x4 y = ld16_nt(vb + i * rs);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        c.v[i][w] = x[w];
        c.v[4 + i][w] = y[w];
      }
    } else {
      u32x2 x = ld8_nt(va + i * rs);
      u32x2 y = ld8_nt(vb + i * rs);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        c.v[i][w] = x[w];
        c.v[4 + i][w] = y[w];
      }
    }
  }
}

// FP8 V: the lane's D/16 codes of each of its 8 key rows, kept as codes until
// P V needs them (widening them here would make the wave wait for the loads at
// once instead of one chunk later).
template <int D>
__device__ __forceinline__ void decode_load_v8(DecodeChunk<D>& c, const uint8_t* vbase,
                                               int pg0, int pg1, int c0, const DecodeArgs& a,
                                               int n, int g) {
  constexpr int DPL = D / 16;
  const int psm = a.page_size - 1;
  const int rs = a.Hkv * D;
  const size_t page_elems = (size_t)a.page_size * rs;
  const uint8_t* va = vbase + (size_t)pg0 * page_elems + ((c0 + 4 * g) & psm) * rs + DPL * n;
  const uint8_t* vb = vbase + (size_t)pg1 * page_elems + ((c0 + 16 + 4 * g) & psm) * rs +
                      DPL * n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (D == 128) {
      const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(va + i * rs));
      const u32x2 y = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vb + i * rs));
      c.v8[i][0] = x[0]; c.v8[i][1] = x[1];
      c.v8[4 + i][0] = y[0]; c.v8[4 + i][1] = y[1];
    } else {
      c.v8[i][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(va + i * rs));
      c.v8[4 + i][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(vb + i * rs));
    }
  }
}

// The codes widened to bf16 pairs in the layout decode_load_v produces.
template <int D>
__device__ __forceinline__ void decode_widen_v8(DecodeChunk<D>& c) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int w = 0; w < D / 64; ++w) {
      const u32x2 r = fp8x4_to_bf16(c.v8[j][w]);
      c.v[j][2 * w] = r[0];
      c.v[j][2 * w + 1] = r[1];
    }
}

// Grouped partitions: the LDS stage of a one-wave work-group's finished partials, at
// most kGpMaxParts partitions x 16 heads x (D + 4) floats, then their lse values.
constexpr int kGpMaxParts = 8;
template <int D>
__device__ __forceinline__ float* gp_stage() {
  __shared__ __align__(16) float buf[kGpMaxParts * 16 * (D + 4) + kGpMaxParts * 16];
  return buf;
}

// BM: a block map is given (a.block_map); PS: FP8 pools with scales per (page, KV
// head) (a.k_scales).  Each is compiled in only when used.
//
// One (KV head kvh, partition split, sequence b) item, walked by the W waves of a
// work-group.  Each wave stages its K rows in 32 rows of KRows<D>::LROW bf16 of LDS:
// its row of a static array, or (DYN) a slice at the start of the kernel's dynamic
// LDS chosen by its wave index in the work-group.  DYN takes W = 1: each wave's item
// is its own and meets no barrier, so the waves of one work-group may run different
// items.  GP: the item is a group of a.group partitions from `split` on, walked as one
// run of chunks, each partition's partial written as the walk leaves it.
template <int D, int W, bool F8, bool BM = false, bool PS = false, bool DYN = false,
          bool GP = false>
__device__ __forceinline__ void decode_item(const DecodeArgs& a, int kvh, int split, int b) {
#include "decode_walk.inc"
}

}  // namespace pa
