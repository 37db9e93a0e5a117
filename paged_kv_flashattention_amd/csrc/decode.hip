// Split-K paged decode attention for gfx950.
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
#include <limits.h>
#include <stdio.h>

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

// BM: a block map is given (a.block_map); PS: FP8 pools with scales per (page, KV
// head) (a.k_scales).  Each is compiled in only when used.
template <int D, int W, bool F8, bool BM = false, bool PS = false>
__global__ __launch_bounds__(64 * W) void decode_partition_kernel(DecodeArgs a) {
  constexpr int DPL = D / 16;   // d values per lane per V row = MFMA d-tiles
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;      // head column (S^T, O^T) / K row within a tile
  const int g = lane >> 4;      // k-group of the MFMA operands
  const int kvh = blockIdx.x;
  const int split = blockIdx.y;
  const int b = blockIdx.z;

  int L = a.seq_lens[b];
  const int cap = a.max_pages * a.page_size;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  // sliding window and document: the row (position L - 1) sees keys lo .. L - 1 (the
  // window's start, or its document's start if later); the walk starts at lo rounded
  // down to a chunk, so chunks keep their page alignment, and the keys below lo are
  // masked
  int lo = a.window > 0 ? max(0, L - a.window) : 0;
  if (a.key_lo) lo = max(lo, min(L, a.key_lo[b]));
  const int k_begin = (lo & ~31) + split * a.part_len;
  const int k_end = min(L, k_begin + a.part_len);
  const int n_chunks = k_end > k_begin ? (k_end - k_begin + 31) >> 5 : 0;

  const int32_t* bt = a.block_tables + (size_t)b * a.max_pages;
  const uint16_t* kbase = a.k_pool + (size_t)kvh * D;
  const uint16_t* vbase = a.v_pool + (size_t)kvh * D;
  const uint8_t* kbase8 = reinterpret_cast<const uint8_t*>(a.k_pool) + (size_t)kvh * D;
  const uint8_t* vbase8 = reinterpret_cast<const uint8_t*>(a.v_pool) + (size_t)kvh * D;
  auto load_k = [&](KRows<D>& kr, int p0, int p1, int c0) {
    if constexpr (F8) decode_load_k_rows8<D>(kr, kbase8, p0, p1, c0, a, lane);
    else decode_load_k_rows<D>(kr, kbase, p0, p1, c0, a, lane);
  };
  auto load_v = [&](DecodeChunk<D>& ch, int p0, int p1, int c0) {
    if constexpr (F8) decode_load_v8<D>(ch, vbase8, p0, p1, c0, a, n, g);
    else decode_load_v<D>(ch, vbase, p0, p1, c0, a, n, g);
  };

  // Q^T as the B operand of S^T = K Q^T: lane holds Q[head n][D/4 * g + 8 kk + j].
  const bool head_ok = n < a.G;
  const int h = kvh * a.G + n;
  // ALiBi: this head's slope in log2 units (the row sits at position L - 1)
  const float slope = a.alibi && head_ok ? a.alibi[h] * kLog2e : 0.f;
  u32x4 qb[D / 32];
  {
    const uint16_t* qp = a.q + ((size_t)b * a.Hq + (head_ok ? h : 0)) * D + (D / 4) * g;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      qb[kk] = head_ok ? ld16(qp + 8 * kk) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  // per-wave staging of one chunk's K rows
  __shared__ __align__(16) uint16_t k_lds_all[W][32 * KRows<D>::LROW];
  uint16_t* k_lds = k_lds_all[wave];

  float m_run = kNegInf;     // running max (log2 domain) of head n
  float l_run = 0.f;         // this lane's share of the running sum
  f32x4 acc[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each wave owns a contiguous run of chunks and keeps one chunk in registers.
  // The next chunk's K loads are issued as soon as this chunk's scores are formed
  // and its V loads as soon as P V has consumed the V registers, so every wave
  // keeps a chunk's worth of loads in flight while it computes; several waves per
  // SIMD cover the rest of the memory latency.  The next chunk index is clamped to
  // the wave's last chunk (a repeat of cached addresses) so the loads are issued
  // unconditionally.  Page ids come from a register window over the table row.
  const int per = (n_chunks + W - 1) / W;
  int c = min(n_chunks, wave * per);
  const int c_hi = min(n_chunks, c + per);
  // Block map (a mask in block form): the row, query index 0 of its one-row run, sees
  // the keys of the 64-key tiles that entry [b][tile] lists.  A chunk lies in one tile
  // (chunks are 32-key aligned), so the walk visits only the chunks of listed tiles:
  // lm holds the listed bits of tiles tb .. tb + 63 (one ballot over a load per lane).
  const uint8_t* bmap = BM ? a.block_map + (size_t)b * a.bm_kb : nullptr;
  int tb = INT_MIN;
  uint64_t lm = 0;
  auto next_listed = [&](int cc, int lim) {
    while (cc < lim) {
      const int t = (k_begin + 32 * cc) >> 6;
      if (t < tb || t >= tb + 64) {
        tb = t;
        const int tl = t + lane;
        lm = __builtin_amdgcn_ballot_w64(tl < a.bm_kb && bmap[min(tl, a.bm_kb - 1)] != 0);
      }
      const uint64_t m = lm >> (t - tb);
      if (m & 1) return cc;
      // the first chunk of the next listed tile (of tile tb + 64 when none is left)
      const int tn = m ? t + (int)__builtin_ctzll(m) : tb + 64;
      cc = max(cc + 1, ((tn << 6) - k_begin) >> 5);
    }
    return lim;
  };
  // Outer loop: one register window of 64 table entries per pass (lane j holds
  // entry base + j); the inner loop over the chunks it covers issues no other loads.
  while (c < c_hi) {
    if constexpr (BM) {
      c = next_listed(c, c_hi);
      if (c >= c_hi) break;
    }
    const int base = (k_begin + 32 * c) >> a.ps_shift;
    const int tab = bt[min(base + lane, a.max_pages - 1)];
    const int c_end = min(c_hi, (((base + 64) << a.ps_shift) - k_begin) >> 5);
    auto page = [&](int key) {
      const int pg = __builtin_amdgcn_readlane(tab, (key >> a.ps_shift) - base);
      return (unsigned)pg < (unsigned)a.num_pages ? pg : 0;
    };
    DecodeChunk<D> ch;
    KRows<D> kr;
    // FP8 pools with scales per (page, KV head): the scales of the two pages of the
    // chunk in registers, read (scalar loads) one chunk ahead like its data
    ChunkScales sc{1.f, 1.f, 1.f, 1.f};
    auto scales_of = [&](int p0, int p1) {
      ChunkScales r{1.f, 1.f, 1.f, 1.f};
      if constexpr (PS) {
        r.k0 = a.k_scales[(size_t)p0 * a.Hkv + kvh];
        r.k1 = a.k_scales[(size_t)p1 * a.Hkv + kvh];
        r.v0 = a.v_scales[(size_t)p0 * a.Hkv + kvh];
        r.v1 = a.v_scales[(size_t)p1 * a.Hkv + kvh];
      }
      return r;
    };
    {
      const int c0 = k_begin + 32 * c;
      const int p0 = page(c0), p1 = page(c0 + 16);
      sc = scales_of(p0, p1);
      load_k(kr, p0, p1, c0);
      // K before V: the first scores then wait only for the K loads
      __builtin_amdgcn_sched_barrier(0);
      load_v(ch, p0, p1, c0);
    }
    for (; c < c_end;) {
      // the next chunk to walk; its loads are issued during this one (the last chunk of
      // a window repeats its own addresses, so the loads are unconditional)
      int cn = c + 1;
      if constexpr (BM) cn = next_listed(c + 1, c_end);
      const int c0 = k_begin + 32 * c;
      const int c0n = k_begin + 32 * (BM ? (cn < c_end ? cn : c) : min(c + 1, c_end - 1));
      const int pn0 = page(c0n);
      const int pn1 = page(c0n + 16);
      const ChunkScales scn = scales_of(pn0, pn1);

      // this chunk's K rows -> LDS; the next chunk's K loads reuse the registers
      if constexpr (F8) decode_k8_to_lds<D>(kr, k_lds, lane);
      else decode_k_to_lds<D>(kr, k_lds, lane);
      load_k(kr, pn0, pn1, c0n);
      decode_k_from_lds<D>(ch, k_lds, n, g);
      f32x4 sa = {0.f, 0.f, 0.f, 0.f};
      f32x4 sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) {
        sa = mfma16x16x32(ch.ka[kk], qb[kk], sa);
        sb = mfma16x16x32(ch.kb[kk], qb[kk], sb);
      }

      if constexpr (F8) decode_widen_v8<D>(ch);

      // FP8 pools with scales per (page, KV head): the keys of the chunk's first 16
      // rows come from page p0, the next 16 from p1 (the same page when pages hold
      // 32 or more keys), so each half has its own key scale in the score multiplier
      const float sm0 = PS ? a.scale_log2 * sc.k0 : a.scale_log2;
      const float sm1 = PS ? a.scale_log2 * sc.k1 : a.scale_log2;
      float s[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = sa[i] * sm0;
        s[4 + i] = sb[i] * sm1;
      }
      if (a.alibi) {
        // score of key c0 + 4 g + o (o = j, or 12 + j for the second half) gets
        // slope * (key - (L - 1))
        const float fb = (float)(c0 + 4 * g - (L - 1));
#pragma unroll
        for (int j = 0; j < 8; ++j) s[j] = fmaf(slope, fb + (float)(j < 4 ? j : 12 + j), s[j]);
      }
      if (c0 + 32 > k_end || c0 < lo) {
        // keys past the end get -inf and V rows 0 (they may hold anything); keys
        // below the window get -inf (their V rows are real data)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = c0 + (j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4));
          if (key >= k_end) {
            s[j] = kNegInf;
#pragma unroll
            for (int w = 0; w < D / 32; ++w) ch.v[j][w] = 0u;
          } else if (key < lo) {
            s[j] = kNegInf;
          }
        }
      }
      float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                       fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      mt = wave_max_xor16_32(mt);
      const float m_new = fmaxf(m_run, mt);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = __builtin_amdgcn_exp2f(s[j] - m_use);
        psum += p[j];
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int t = 0; t < DPL; ++t) acc[t] *= alpha;
      // the value scale of each half's page goes onto P (the row sum above stays
      // unscaled): P V then sums p_j * v_scale(page of j) * decode(code_j)
      if constexpr (PS) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          p[j] *= sc.v0;
          p[4 + j] *= sc.v1;
        }
      }
      const u32x4 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                        pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
#pragma unroll
      for (int t = 0; t < DPL; ++t) {
        const int w = t >> 1;
        u32x4 va;
        if ((t & 1) == 0) {
          va = u32x4{pack_lo_halves(ch.v[0][w], ch.v[1][w]), pack_lo_halves(ch.v[2][w], ch.v[3][w]),
                     pack_lo_halves(ch.v[4][w], ch.v[5][w]), pack_lo_halves(ch.v[6][w], ch.v[7][w])};
        } else {
          va = u32x4{pack_hi_halves(ch.v[0][w], ch.v[1][w]), pack_hi_halves(ch.v[2][w], ch.v[3][w]),
                     pack_hi_halves(ch.v[4][w], ch.v[5][w]), pack_hi_halves(ch.v[6][w], ch.v[7][w])};
        }
        acc[t] = mfma16x16x32(va, pb, acc[t]);
      }
      load_v(ch, pn0, pn1, c0n);
      sc = scn;
      c = cn;
    }
  }

  float l_tot = wave_sum_xor16_32(l_run);
  float m_fin = m_run;

  if constexpr (W > 1) {
    __shared__ float sm_acc[W][DPL * 4][64];
    __shared__ float sm_m[W][16];
    __shared__ float sm_l[W][16];
#pragma unroll
    for (int t = 0; t < DPL; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_acc[wave][4 * t + i][lane] = acc[t][i];
    if (g == 0) {
      sm_m[wave][n] = m_run;
      sm_l[wave][n] = l_tot;
    }
    __syncthreads();
    if (wave != 0) return;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][n]);
    const float M_use = M == kNegInf ? 0.f : M;
    float Lsum = 0.f;
#pragma unroll
    for (int t = 0; t < DPL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float e = __builtin_amdgcn_exp2f(sm_m[w][n] - M_use);
      Lsum += e * sm_l[w][n];
#pragma unroll
      for (int t = 0; t < DPL; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] += e * sm_acc[w][4 * t + i][lane];
    }
    l_tot = Lsum;
    m_fin = M;
  }

  const bool live = l_tot > 0.f;
  const float inv = live ? a.v_scale / l_tot : 0.f;
  const float lse = live ? (m_fin + __log2f(l_tot)) * kLn2 : kNegInf;
  // lane holds d = DPL * (4 g + i) + t for i = 0..3, t = 0..DPL-1, i.e. the
  // DPL * 4 consecutive values starting at d = DPL * 4 * g
  if (a.S == 1 && !a.force_partials) {
    if (!head_ok) return;
    uint16_t* op = a.out + ((size_t)b * a.Hq + h) * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = DPL * (4 * g + i);
      if constexpr (DPL == 8) {
        u32x4 w;
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2)
          w[t2] = pack_bf16x2(acc[2 * t2][i] * inv, acc[2 * t2 + 1][i] * inv);
        *reinterpret_cast<u32x4*>(op + d0) = w;
      } else {
        u32x2 w;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
          w[t2] = pack_bf16x2(acc[2 * t2][i] * inv, acc[2 * t2 + 1][i] * inv);
        *reinterpret_cast<u32x2*>(op + d0) = w;
      }
    }
    if (g == 0 && a.lse_out) a.lse_out[(size_t)b * a.Hq + h] = lse;
    return;
  }

  // Split-K: this partition's normalised output and natural-log lse, merged by
  // the split-K reduce kernel.
  if (!head_ok) return;
  const size_t row = ((size_t)b * a.Hq + h) * a.S + split;
  float* op = a.part_o + row * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d0 = DPL * (4 * g + i);
#pragma unroll
    for (int t4 = 0; t4 < DPL / 4; ++t4) {
      f32x4 w = {acc[4 * t4][i] * inv, acc[4 * t4 + 1][i] * inv, acc[4 * t4 + 2][i] * inv,
                 acc[4 * t4 + 3][i] * inv};
      *reinterpret_cast<f32x4*>(op + d0 + 4 * t4) = w;
    }
  }
  if (g == 0) a.part_lse[row] = lse;
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
static int decode_waves(const DecodeArgs& a) {
  const long long groups = (long long)a.Hkv * a.S * a.B;
  const long long target = a.kv_fp8 ? 1024 : 512;
  return groups >= target ? 1 : (2 * groups >= target ? 2 : 4);
}

template <int D>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream, int W,
                                  const KernelEvents& ev) {
  if (W == 4) return launch_decode_t<D, 4>(a, stream, ev);
  if (W == 2) return launch_decode_t<D, 2>(a, stream, ev);
  return launch_decode_t<D, 1>(a, stream, ev);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, char* desc, size_t desc_len,
                         const KernelEvents& ev) {
  const int W = decode_waves(a);
  hipError_t e = a.D == 128 ? launch_decode_d<128>(a, stream, W, ev)
                            : launch_decode_d<64>(a, stream, W, ev);
  snprintf(desc, desc_len,
           "decode_partition<D=%d,W=%d,%s%s> grid=(%d,%d,%d) block=%d part_len=%d splits=%d", a.D,
           W, a.kv_fp8 ? (a.k_scales ? "fp8-e4m3 scales per page" : "fp8-e4m3") : "bf16",
           a.block_map ? ",block map" : "", a.Hkv, a.S, a.B, 64 * W, a.part_len, a.S);
  return e;
}

}  // namespace pa
