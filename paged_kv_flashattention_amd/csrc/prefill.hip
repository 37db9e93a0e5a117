// Ragged causal prefill over paged K/V on gfx950 matrix cores.
//
// Work-group = 4 waves = 128 consecutive query rows of one query head of one
// sequence; each wave owns 32 rows.  Keys are walked in 64-key tiles gathered
// through the block table into LDS (double buffered: the next tile's global
// loads are in flight while the current tile is consumed).  Per 32-key block a
// wave computes
//   S^T[32 keys x 32 queries] = K Q^T           32x32x16 bf16 MFMA, fp32 accumulate
//   running max / running sum per query         ("The Stack Below the Stack (Part 2)",
//                                                 section 2.1, online softmax)
//   O^T[D x 32 queries] += V^T P^T               P rounded to bf16
// Keys sit on the MFMA's M side so that every per-query statistic lives in lane %
// 32 and the S^T accumulator is already laid out as the P^T operand; V is stored
// transposed in LDS (V^T[d][key], transposed in registers while staging) so the
// V^T operand is one 16-byte LDS read.  Within each group of 16 keys the V^T
// columns hold keys in the order 0-3, 8-11, 4-7, 12-15: the order in which the
// S^T accumulator hands P^T its keys.
//
// Causal rows are the LAST q_len positions of their sequence (query row i at
// absolute position seq_len - q_len + i sees keys j <= that position); key
// blocks wholly above a wave's rows are skipped, and only blocks that cross the
// diagonal are masked.  Work-groups with the most keys are dispatched first.
#include <stdio.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pa {

constexpr int kPfWaves = 4;
constexpr int kPfBM = 32 * kPfWaves;   // query rows per work-group
constexpr int kPfBN = 64;              // keys per LDS tile
constexpr int kPfThreads = 64 * kPfWaves;

template <int D>
struct PfLds {
  static constexpr int KROW = D + 8;          // bf16 per K row (16 B pad)
  static constexpr int VROW = kPfBN + 8;      // bf16 per V^T row (16 B pad)
  static constexpr int K_ELEMS = kPfBN * KROW;
  static constexpr int V_ELEMS = D * VROW;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr size_t BYTES = 2 * STAGE * sizeof(uint16_t);
};

// Position of key offset o (0..63) of a tile among the V^T columns.
__device__ __forceinline__ int vt_col(int o) {
  const int grp = (o >> 2) & 3;
  const int swapped = grp == 1 ? 2 : (grp == 2 ? 1 : grp);
  return (o & ~15) | (swapped << 2) | (o & 3);
}

template <int D>
struct PfStage {
  u32x4 k[D / 32];                 // K: one key row, D/4 values
  uint32_t v[4][D / 32];           // V: 4 key rows x D/16 values
};

// Global loads of one 64-key tile for this thread.  Wave w stages keys
// k0 + 16 w .. k0 + 16 w + 15, which share one page (`page`, wave-uniform); the
// loads are unconditional (page and slot are always inside the pool) and rows past
// the sequence end are zeroed afterwards.
template <int D>
__device__ __forceinline__ void pf_load_tile(PfStage<D>& st, const PrefillArgs& a,
                                             const uint16_t* kbase, const uint16_t* vbase,
                                             int page, int k0, int L, int tid) {
  const int psm = a.page_size - 1;
  const int rs = a.Hkv * D;
  const size_t page_off = (size_t)page * a.page_size * rs;
  // K: thread -> key tid/4, d range [(tid%4) * D/4, +D/4)
  {
    const int key = k0 + (tid >> 2);
    const uint16_t* p = kbase + page_off + (key & psm) * rs + (tid & 3) * (D / 4);
    const bool ok = key < L;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const u32x4 x = ld16(p + 8 * c);
      st.k[c] = ok ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // V: thread -> keys 4 (tid/16) .. +3, d range [(tid%16) * D/16, +D/16)
  {
    const int key0 = k0 + 4 * (tid >> 4);
    const uint16_t* p = vbase + page_off + (key0 & psm) * rs + (tid & 15) * (D / 16);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = key0 + r < L;
      if constexpr (D == 128) {
        const u32x4 x = ld16(p + r * rs);
#pragma unroll
        for (int w = 0; w < 4; ++w) st.v[r][w] = ok ? x[w] : 0u;
      } else {
        const u32x2 x = ld8(p + r * rs);
#pragma unroll
        for (int w = 0; w < 2; ++w) st.v[r][w] = ok ? x[w] : 0u;
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void pf_store_tile(const PfStage<D>& st, uint16_t* lds, int tid) {
  uint16_t* kl = lds;
  uint16_t* vl = lds + PfLds<D>::K_ELEMS;
  {
    uint16_t* p = kl + (tid >> 2) * PfLds<D>::KROW + (tid & 3) * (D / 4);
#pragma unroll
    for (int c = 0; c < D / 32; ++c) *reinterpret_cast<u32x4*>(p + 8 * c) = st.k[c];
  }
  {
    // 4 keys x D/16 d values -> for each d, 4 keys (8 bytes) at the key group's column
    const int col = vt_col(4 * (tid >> 4));
    const int d0 = (tid & 15) * (D / 16);
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const int w = t >> 1;
      u32x2 pr;
      if ((t & 1) == 0) {
        pr = u32x2{pack_lo_halves(st.v[0][w], st.v[1][w]), pack_lo_halves(st.v[2][w], st.v[3][w])};
      } else {
        pr = u32x2{pack_hi_halves(st.v[0][w], st.v[1][w]), pack_hi_halves(st.v[2][w], st.v[3][w])};
      }
      *reinterpret_cast<u32x2*>(vl + (d0 + t) * PfLds<D>::VROW + col) = pr;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) uint16_t pf_lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;         // query column of S^T / O^T
  const int hh = lane >> 5;          // k-half of the MFMA operands
  const int h = blockIdx.x;          // query head
  const int b = blockIdx.y;
  const int qt = gridDim.z - 1 - blockIdx.z;   // heaviest tiles first

  const int t0 = a.cu_seqlens_q[b];
  const int q_len = a.cu_seqlens_q[b + 1] - t0;
  const int r_wg = qt * kPfBM;
  if (r_wg >= q_len) return;
  int L = a.seq_lens_k[b];
  const int cap = a.max_pages * a.page_size;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int kvh = h / a.G;
  const uint16_t* kbase = a.k_pool + (size_t)kvh * D;
  const uint16_t* vbase = a.v_pool + (size_t)kvh * D;

  // absolute position of this work-group's last row; keys past it are never needed
  const int rows_wg = min(kPfBM, q_len - r_wg);
  const int shift = L - q_len;                 // position of row r is shift + r
  int k_lim = L;
  if (a.causal) k_lim = min(L, max(0, shift + r_wg + rows_wg));
  const int n_tiles = (k_lim + kPfBN - 1) / kPfBN;

  // this wave's rows and the position bound of its rows
  const int r_w = r_wg + 32 * wave;
  const int my_row = r_w + col;
  const bool row_ok = my_row < q_len && t0 + my_row < a.Tq;
  const int my_pos = shift + my_row;          // causal: keys <= my_pos are visible
  const int w_pos_max = shift + min(r_w + 31, q_len - 1);
  const int w_pos_min = shift + r_w;

  // Q^T operand: lane holds Q[row col][16 kk + 8 hh + j]
  u32x4 qb[D / 16];
  {
    const uint16_t* qp = a.q + ((size_t)(t0 + (row_ok ? my_row : 0)) * a.Hq + h) * D + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qb[kk] = row_ok ? ld16(qp + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
  }

  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;

  // Block-table window: lane j holds the page of this wave's 16 keys of tile
  // base_t + j, so the 64 tiles of a window need no further table reads; the
  // tile loop runs one window at a time.
  const int32_t* bt = a.block_tables + (size_t)b * a.max_pages;
  int base_t = 0;
  int tab = 0;
  auto load_tab = [&](int first_tile) {
    int idx = ((first_tile + lane) * kPfBN + 16 * wave) >> a.ps_shift;
    idx = idx < a.max_pages ? idx : a.max_pages - 1;
    return bt[idx];
  };
  auto tile_page = [&](int kt) {
    const int pg = __builtin_amdgcn_readlane(tab, kt - base_t);
    return (unsigned)pg < (unsigned)a.num_pages ? pg : 0;
  };

  PfStage<D> st;
  while (base_t < n_tiles) {
    tab = load_tab(base_t);
    const int win_end = min(n_tiles, base_t + 64);
    // stage the window's first tile
    pf_load_tile<D>(st, a, kbase, vbase, tile_page(base_t), base_t * kPfBN, L, tid);
    pf_store_tile<D>(st, pf_lds + (base_t & 1) * PfLds<D>::STAGE, tid);
    __syncthreads();

    for (int kt = base_t; kt < win_end; ++kt) {
      const uint16_t* cur = pf_lds + (kt & 1) * PfLds<D>::STAGE;
      // next tile's loads in flight during this tile's math (clamped to the window:
      // the window's last iteration stages a repeat that nobody reads)
      const int nt = min(kt + 1, win_end - 1);
      pf_load_tile<D>(st, a, kbase, vbase, tile_page(nt), nt * kPfBN, L, tid);

#pragma unroll
      for (int kb = 0; kb < kPfBN / 32; ++kb) {
        const int kb0 = kt * kPfBN + kb * 32;
        const bool skip = kb0 >= L || (a.causal && kb0 > w_pos_max) || r_w >= q_len;
        if (skip) continue;
        // S^T = K Q^T
        f32x16 s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
        const uint16_t* kl = cur + (kb * 32 + col) * PfLds<D>::KROW + 8 * hh;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(kl + 16 * kk);
          s = mfma32x32x16(ka, qb[kk], s);
        }
        // scale to log2 units; mask keys past the end and (causal) above the diagonal
        const bool need_mask = (kb0 + 32 > L) || (a.causal && kb0 + 31 > w_pos_min);
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] *= a.scale_log2;
        if (need_mask) {
          const int lim = a.causal ? min(L - 1, my_pos) : L - 1;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = kb0 + 8 * j + 4 * hh + i;
              if (key > lim) s[4 * j + i] = kNegInf;
            }
        }
        float mt = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mt = fmaxf(mt, s[e]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[e] = exp2f(s[e] - m_use);
          psum += s[e];
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
        const u32x4 pb0 = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]),
                           pack_bf16x2(s[4], s[5]), pack_bf16x2(s[6], s[7])};
        const u32x4 pb1 = {pack_bf16x2(s[8], s[9]), pack_bf16x2(s[10], s[11]),
                           pack_bf16x2(s[12], s[13]), pack_bf16x2(s[14], s[15])};
        // O^T += V^T P^T
        const uint16_t* vl = cur + PfLds<D>::K_ELEMS + col * PfLds<D>::VROW + kb * 32 + 8 * hh;
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          const uint16_t* vrow = vl + 32 * t * PfLds<D>::VROW;
          const u32x4 va0 = *reinterpret_cast<const u32x4*>(vrow);
          const u32x4 va1 = *reinterpret_cast<const u32x4*>(vrow + 16);
          acc[t] = mfma32x32x16(va0, pb0, acc[t]);
          acc[t] = mfma32x32x16(va1, pb1, acc[t]);
        }
      }
      pf_store_tile<D>(st, pf_lds + ((kt + 1) & 1) * PfLds<D>::STAGE, tid);
      __syncthreads();
    }
    base_t = win_end;
  }

  if (!row_ok) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const bool live = l_tot > 0.f;
  const float inv = live ? 1.f / l_tot : 0.f;
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
  if (hh == 0 && a.lse_out)
    a.lse_out[(size_t)(t0 + my_row) * a.Hq + h] = live ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
}

template <int D>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream, int n_qt) {
  dim3 grid(a.Hq, a.B, n_qt);
  hipLaunchKernelGGL(prefill_kernel<D>, grid, dim3(kPfThreads), PfLds<D>::BYTES, stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream, char* desc,
                          size_t desc_len) {
  const int n_qt = (a.max_q_len + kPfBM - 1) / kPfBM;
  hipError_t e;
  if (a.D == 128) {
    // more than 64 KiB of dynamic LDS must be requested once per process
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(prefill_kernel<128>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)PfLds<128>::BYTES);
    if (attr != hipSuccess) return attr;
    e = launch_prefill_t<128>(a, stream, n_qt);
  } else {
    e = launch_prefill_t<64>(a, stream, n_qt);
  }
  snprintf(desc, desc_len,
           "prefill<D=%d,BM=%d,BN=%d,mfma32x32x16> grid=(%d,%d,%d) block=%d lds=%zu", a.D,
           kPfBM, kPfBN, a.Hq, a.B, n_qt, kPfThreads,
           a.D == 128 ? PfLds<128>::BYTES : PfLds<64>::BYTES);
  return e;
}

}  // namespace pa
