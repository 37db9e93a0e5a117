// Split-K paged decode attention for gfx950.
//
// One work-group of W waves owns one (sequence b, KV head, partition) triple.
// The partition's keys are walked in 32-key chunks, chunk c going to wave c % W;
// each wave streams its chunks straight from the page pools into registers
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
// and natural-log lse for the split-K reduce ("The Stack Below the Stack (Part 2)",
// section 2.2).
#include <stdio.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pa {

template <int D>
struct DecodeChunk {
  u32x4 ka[D / 32];          // K row (chunk key l%16), d in [D/4 * g, D/4 * (g+1))
  u32x4 kb[D / 32];          // K row (chunk key 16 + l%16), same d range
  uint32_t v[8][D / 32];     // V rows of the lane's 8 keys, d in [D/16 * n, D/16 * (n+1))
};

template <int D>
__device__ __forceinline__ void decode_load_chunk(DecodeChunk<D>& c, const uint16_t* kbase,
                                                  const uint16_t* vbase, const int32_t* bt,
                                                  int c0, const DecodeArgs& a, int n, int g) {
  const int psm = a.page_size - 1;
  const size_t rs = (size_t)a.Hkv * D;
  const int pg0 = page_of(bt, c0, a.ps_shift, a.max_pages, a.num_pages);
  const int pg1 = page_of(bt, c0 + 16, a.ps_shift, a.max_pages, a.num_pages);
  const size_t base0 = (size_t)pg0 * a.page_size;
  const size_t base1 = (size_t)pg1 * a.page_size;
  const uint16_t* ka = kbase + (base0 + ((c0 + n) & psm)) * rs + (D / 4) * g;
  const uint16_t* kb = kbase + (base1 + ((c0 + 16 + n) & psm)) * rs + (D / 4) * g;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    c.ka[kk] = ld16(ka + 8 * kk);
    c.kb[kk] = ld16(kb + 8 * kk);
  }
  constexpr int DPL = D / 16;
  const uint16_t* va = vbase + (base0 + ((c0 + 4 * g) & psm)) * rs + DPL * n;
  const uint16_t* vb = vbase + (base1 + ((c0 + 16 + 4 * g) & psm)) * rs + DPL * n;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (D == 128) {
      u32x4 x = ld16(va + i * rs);
      u32x4 y = ld16(vb + i * rs);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        c.v[i][w] = x[w];
        c.v[4 + i][w] = y[w];
      }
    } else {
      u32x2 x = ld8(va + i * rs);
      u32x2 y = ld8(vb + i * rs);
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        c.v[i][w] = x[w];
        c.v[4 + i][w] = y[w];
      }
    }
  }
}

template <int D, int W>
__global__ __launch_bounds__(64 * W) void decode_partition_kernel(DecodeArgs a) {
  constexpr int DPL = D / 16;   // d values per lane per V row = MFMA d-tiles
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;      // head column (S^T, O^T) / K row within a tile
  const int g = lane >> 4;      // k-group of the MFMA operands
  const int kvh = blockIdx.x;
  const int split = blockIdx.y;
  const int b = blockIdx.z;

  int L = a.seq_lens[b];
  const int cap = a.max_pages * a.page_size;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int k_begin = split * a.part_len;
  const int k_end = min(L, k_begin + a.part_len);
  const int n_chunks = k_end > k_begin ? (k_end - k_begin + 31) >> 5 : 0;

  const int32_t* bt = a.block_tables + (size_t)b * a.max_pages;
  const uint16_t* kbase = a.k_pool + (size_t)kvh * D;
  const uint16_t* vbase = a.v_pool + (size_t)kvh * D;

  // Q^T as the B operand of S^T = K Q^T: lane holds Q[head n][D/4 * g + 8 kk + j].
  const bool head_ok = n < a.G;
  const int h = kvh * a.G + n;
  u32x4 qb[D / 32];
  {
    const uint16_t* qp = a.q + ((size_t)b * a.Hq + (head_ok ? h : 0)) * D + (D / 4) * g;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      qb[kk] = head_ok ? ld16(qp + 8 * kk) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m_run = kNegInf;     // running max (log2 domain) of head n
  float l_run = 0.f;         // this lane's share of the running sum
  f32x4 acc[DPL];
#pragma unroll
  for (int t = 0; t < DPL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](DecodeChunk<D>& c, int c0) {
    f32x4 sa = {0.f, 0.f, 0.f, 0.f};
    f32x4 sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      sa = mfma16x16x32(c.ka[kk], qb[kk], sa);
      sb = mfma16x16x32(c.kb[kk], qb[kk], sb);
    }
    float s[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = sa[i] * a.scale_log2;
      s[4 + i] = sb[i] * a.scale_log2;
    }
    if (c0 + 32 > k_end) {     // last chunk: keys past the end get -inf, their V rows 0
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = c0 + (j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4));
        if (key >= k_end) {
          s[j] = kNegInf;
#pragma unroll
          for (int w = 0; w < D / 32; ++w) c.v[j][w] = 0u;
        }
      }
    }
    float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                     fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mt = wave_max_xor16_32(mt);
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_use);
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = exp2f(s[j] - m_use);
      ps += p[j];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < DPL; ++t) acc[t] *= alpha;
    const u32x4 pb = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                      pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
#pragma unroll
    for (int t = 0; t < DPL; ++t) {
      const int w = t >> 1;
      u32x4 va;
      if ((t & 1) == 0) {
        va = u32x4{pack_lo_halves(c.v[0][w], c.v[1][w]), pack_lo_halves(c.v[2][w], c.v[3][w]),
                   pack_lo_halves(c.v[4][w], c.v[5][w]), pack_lo_halves(c.v[6][w], c.v[7][w])};
      } else {
        va = u32x4{pack_hi_halves(c.v[0][w], c.v[1][w]), pack_hi_halves(c.v[2][w], c.v[3][w]),
                   pack_hi_halves(c.v[4][w], c.v[5][w]), pack_hi_halves(c.v[6][w], c.v[7][w])};
      }
      acc[t] = mfma16x16x32(va, pb, acc[t]);
    }
  };

  // Software pipeline over this wave's chunks: two register buffers, the next
  // chunk's loads issued before the current chunk is consumed.
  DecodeChunk<D> c_a, c_b;
  int c = wave;
  if (c < n_chunks) decode_load_chunk<D>(c_a, kbase, vbase, bt, k_begin + 32 * c, a, n, g);
  while (c < n_chunks) {
    const int c_next = c + W;
    if (c_next < n_chunks)
      decode_load_chunk<D>(c_b, kbase, vbase, bt, k_begin + 32 * c_next, a, n, g);
    compute(c_a, k_begin + 32 * c);
    c = c_next;
    if (c >= n_chunks) break;
    const int c_next2 = c + W;
    if (c_next2 < n_chunks)
      decode_load_chunk<D>(c_a, kbase, vbase, bt, k_begin + 32 * c_next2, a, n, g);
    compute(c_b, k_begin + 32 * c);
    c = c_next2;
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
      const float e = exp2f(sm_m[w][n] - M_use);
      Lsum += e * sm_l[w][n];
#pragma unroll
      for (int t = 0; t < DPL; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][i] += e * sm_acc[w][4 * t + i][lane];
    }
    l_tot = Lsum;
    m_fin = M;
  }

  if (!head_ok) return;
  const bool live = l_tot > 0.f;
  const float inv = live ? 1.f / l_tot : 0.f;
  const float lse = live ? (m_fin + __log2f(l_tot)) * kLn2 : kNegInf;
  // lane holds d = DPL * (4 g + i) + t for i = 0..3, t = 0..DPL-1
  if (a.S == 1) {
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
  } else {
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
}

template <int D, int W>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  dim3 grid(a.Hkv, a.S, a.B);
  hipLaunchKernelGGL((decode_partition_kernel<D, W>), grid, dim3(64 * W), 0, stream, a);
  return hipGetLastError();
}

static constexpr int kDecodeWaves = 4;

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream, char* desc, size_t desc_len) {
  hipError_t e;
  if (a.D == 128)
    e = launch_decode_t<128, kDecodeWaves>(a, stream);
  else
    e = launch_decode_t<64, kDecodeWaves>(a, stream);
  snprintf(desc, desc_len,
           "decode_partition<D=%d,W=%d> grid=(%d,%d,%d) block=%d part_len=%d splits=%d", a.D,
           kDecodeWaves, a.Hkv, a.S, a.B, 64 * kDecodeWaves, a.part_len, a.S);
  return e;
}

}  // namespace pa
