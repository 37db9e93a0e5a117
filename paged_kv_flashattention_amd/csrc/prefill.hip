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
#include <stdio.h>

#include "common.hpp"
#include "kernels.hpp"

namespace pa {

constexpr int kPfWaves = 4;
constexpr int kPfBM = 32 * kPfWaves;   // query rows per work-group
constexpr int kPfBN = 64;              // keys per LDS tile
constexpr int kPfThreads = 64 * kPfWaves;
constexpr float kRescaleSlack = 8.f;   // log2 headroom before the reference moves

// LDS tile: K and V rows of 64 keys, row-major [key][D] with no padding; the
// 16-byte chunks of row r are stored permuted (chunk c at c ^ chunk_swz(r)).  The
// LDS serves 256 bytes (all 64 banks) per clock: a K operand read covers one chunk
// of 16 consecutive rows per clock, a transposing V read four chunks of 4
// consecutive rows per 32 lanes, and the permutation keeps both on distinct banks
// (for D = 128 a row spans all banks, so rows r .. r + 3 must differ in the
// permutation's upper two bits; for D = 64 two rows share a bank line).
template <int D>
struct PfLds {
  static constexpr int TILE = kPfBN * D;          // bf16 elements of K (or V) per tile
  static constexpr int STAGE = 2 * TILE;          // K then V
  static constexpr size_t BYTES = 2 * STAGE * sizeof(uint16_t);   // two stages
};

template <int D>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land at
// lds_wave_base + 16 i (gfx950 global_load_lds_dwordx4, LDS base in M0).  Written
// as inline assembly so that the compiler, which cannot tell which LDS reads such
// a load may feed, does not wait for every outstanding one before each LDS read;
// completion is waited for explicitly (vmcnt_wait) before the barrier that
// publishes a tile.
__device__ __forceinline__ void dma16(const uint16_t* gsrc, uint16_t* lds_wave_base) {
  const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_wave_base;
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "s"(lds)
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

// Transposing 8-byte LDS read: within each 16-lane group, lane j receives element
// (j % 4) of the 8-byte rows that lanes j/4, 4 + j/4, 8 + j/4 and 12 + j/4 point at.
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// DMA loads of one 64-key tile into one LDS stage.  Wave w fills rows 16 w ..
// 16 w + 15 of K and of V (keys k0 + 16 w .., all in one page `page`); each load
// instruction covers RPI = 512 / D rows, lane i fetching the global chunk that
// belongs at LDS position i of the permuted layout.
template <int D>
__device__ __forceinline__ void pf_issue_tile(uint16_t* stage, const PrefillArgs& a,
                                              const uint16_t* kbase, const uint16_t* vbase,
                                              int page, int k0, int wave, int lane) {
  constexpr int LPR = D / 8;               // 16-byte chunks per row
  constexpr int RPI = 64 / LPR;            // rows per instruction
  const int psm = a.page_size - 1;
  const int rs = a.Hkv * D;
  const size_t page_off = (size_t)page * a.page_size * rs;
#pragma unroll
  for (int i = 0; i < 16 / RPI; ++i) {
    const int r = 16 * wave + RPI * i + lane / LPR;          // tile row = key - k0
    const int c = (lane % LPR) ^ chunk_swz<D>(r);            // global chunk for this slot
    const size_t src = page_off + (size_t)((k0 + r) & psm) * rs + c * 8;
    uint16_t* dst = stage + (16 * wave + RPI * i) * D;       // wave-uniform
    dma16(kbase + src, dst);
    dma16(vbase + src, dst + PfLds<D>::TILE);
  }
}

// Zero this wave's V rows at or past the sequence end (the last tile only): they
// hold other data, and P = 0 times NaN would not be 0.
template <int D>
__device__ __forceinline__ void pf_zero_tail(uint16_t* stage, int k0, int L, int wave, int lane) {
  constexpr int LPR = D / 8;
  constexpr int RPI = 64 / LPR;
#pragma unroll
  for (int i = 0; i < 16 / RPI; ++i) {
    const int r = 16 * wave + RPI * i + lane / LPR;
    if (k0 + r >= L)
      *reinterpret_cast<u32x4*>(stage + PfLds<D>::TILE + r * D + (lane % LPR) * 8) =
          u32x4{0u, 0u, 0u, 0u};
  }
}

template <int D>
__global__ __launch_bounds__(kPfThreads, 2) void prefill_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) uint16_t pf_lds[];
  constexpr int NDMA = 2 * (16 * D / 512);  // DMA instructions per wave per tile
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

  while (base_t < n_tiles) {
    tab = load_tab(base_t);
    const int win_end = min(n_tiles, base_t + 64);
    // every wave has finished reading both stages before they are refilled
    block_sync();
    pf_issue_tile<D>(pf_lds + (base_t & 1) * PfLds<D>::STAGE, a, kbase, vbase,
                     tile_page(base_t), base_t * kPfBN, wave, lane);

    for (int kt = base_t; kt < win_end; ++kt) {
      uint16_t* cur = pf_lds + (kt & 1) * PfLds<D>::STAGE;
      // next tile's DMA in flight during this tile's math (clamped to the window:
      // the window's last iteration stages a repeat that nobody reads)
      const int nt = min(kt + 1, win_end - 1);
      pf_issue_tile<D>(pf_lds + ((kt + 1) & 1) * PfLds<D>::STAGE, a, kbase, vbase,
                       tile_page(nt), nt * kPfBN, wave, lane);
      vmcnt_wait<NDMA>();                 // this wave's loads of tile kt have landed
      if (kt * kPfBN + kPfBN > L) {
        pf_zero_tail<D>(cur, kt * kPfBN, L, wave, lane);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the zeros are in LDS
      }
      block_sync();                        // ... and every other wave's

      // Scores of both 32-key blocks, their two MFMA chains interleaved and each K
      // fragment read one step ahead, so the softmax of the first block overlaps
      // the matrix cores' work on the second.  A block wholly outside this wave's
      // causal window is computed anyway and then ignored.
      f32x16 sblk[kPfBN / 32];
      bool act[kPfBN / 32];
#pragma unroll
      for (int kb = 0; kb < kPfBN / 32; ++kb) {
        const int kb0 = kt * kPfBN + kb * 32;
        act[kb] = !(kb0 >= L || (a.causal && kb0 > w_pos_max) || r_w >= q_len);
#pragma unroll
        for (int e = 0; e < 16; ++e) sblk[kb][e] = 0.f;
      }
      if (act[0] || act[1]) {
        const uint16_t* kl0 = cur + col * D;
        const uint16_t* kl1 = cur + (32 + col) * D;
        const int sw0 = chunk_swz<D>(col), sw1 = chunk_swz<D>(32 + col);
        auto kfrag = [&](const uint16_t* kl, int sw, int kk) {
          return *reinterpret_cast<const u32x4*>(kl + (((2 * kk + hh) ^ sw) << 3));
        };
        u32x4 n0 = kfrag(kl0, sw0, 0), n1 = kfrag(kl1, sw1, 0);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const u32x4 f0 = n0, f1 = n1;
          if (kk + 1 < D / 16) {
            n0 = kfrag(kl0, sw0, kk + 1);
            n1 = kfrag(kl1, sw1, kk + 1);
          }
          sblk[0] = mfma32x32x16(f0, qb[kk], sblk[0]);
          sblk[1] = mfma32x32x16(f1, qb[kk], sblk[1]);
        }
        // Scheduling order: the fragment reads run two MFMA pairs ahead of their use.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // 4 LDS reads
#pragma unroll
        for (int i = 0; i < D / 16 - 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // 2 LDS reads
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
#pragma unroll
      for (int kb = 0; kb < kPfBN / 32; ++kb) {
        if (!act[kb]) continue;
        const int kb0 = kt * kPfBN + kb * 32;
        f32x16& s = sblk[kb];
        // Keys past the end and (causal) above the diagonal get -inf; only blocks
        // that touch the boundary need it.
        const bool need_mask = (kb0 + 32 > L) || (a.causal && kb0 + 31 > w_pos_min);
        if (__builtin_expect(need_mask, 0)) {
          const int lim = a.causal ? min(L - 1, my_pos) : L - 1;
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = kb0 + 8 * j + 4 * hh + i;
              if (key > lim) s[4 * j + i] = kNegInf;
            }
        }
        // Online softmax in log2 units with a lazily moved reference: the running
        // reference m_ref only moves (rescaling l and the accumulator) when a row's
        // scaled maximum exceeds it by more than kRescaleSlack, so P stays below
        // 2^kRescaleSlack and the result is unchanged -- the final normalisation
        // uses the same reference ("The Stack Below the Stack (Part 2)", 2.1 and 2.3).
        float mt = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
        for (int e = 3; e < 15; e += 2) mt = fmaxf(fmaxf(mt, s[e]), s[e + 1]);
        mt = fmaxf(mt, s[15]);
        mt = xor32_max(mt) * a.scale_log2;
        const bool grow = mt > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float m_new = grow ? mt : m_run;
          const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
          l_run *= alpha;
#pragma unroll
          for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
          m_run = m_new;
        }
        const float neg_m = m_run == kNegInf ? 0.f : -m_run;
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], a.scale_log2, neg_m));
          psum += s[e];
        }
        l_run += psum;
        // P^T operand halves: keys 16u + 4 hh + (0..3) and 16u + 8 + 4 hh + (0..3)
        const u32x4 pb0 = {pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]),
                           pack_bf16x2(s[4], s[5]), pack_bf16x2(s[6], s[7])};
        const u32x4 pb1 = {pack_bf16x2(s[8], s[9]), pack_bf16x2(s[10], s[11]),
                           pack_bf16x2(s[12], s[13]), pack_bf16x2(s[14], s[15])};
        // The V^T operand (8 keys of one d per lane) comes from two transposing
        // reads of row-major V: in each 16-lane group, lane i points at key row
        // key0 + i/4, columns d0 + 4 (i % 4) .. + 3.
        const int g16 = lane & 15;
        const int dsub = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
        auto vfrag = [&](int t, int u) {
          const int dd = 32 * t + dsub;                      // first d of this lane's piece
          const int r0 = kb * 32 + 16 * u + 4 * hh + (g16 >> 2);
          const int r1 = r0 + 8;
          const u32x2 lo = ds_read_tr16(cur + PfLds<D>::TILE + r0 * D +
                                        (((dd >> 3) ^ chunk_swz<D>(r0)) << 3) + (dd & 7));
          const u32x2 hi = ds_read_tr16(cur + PfLds<D>::TILE + r1 * D +
                                        (((dd >> 3) ^ chunk_swz<D>(r1)) << 3) + (dd & 7));
          return u32x4{lo[0], lo[1], hi[0], hi[1]};
        };
        // O^T += V^T P^T over the block's two 16-key halves; the four d-tiles are
        // independent accumulators, so each half issues four MFMAs back to back.
        u32x4 vnext = vfrag(0, 0);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int t = 0; t < D / 32; ++t) {
            const u32x4 va = vnext;
            if (u * (D / 32) + t + 1 < 2 * (D / 32)) {
              const int n = u * (D / 32) + t + 1;
              vnext = vfrag(n % (D / 32), n / (D / 32));
            }
            acc[t] = mfma32x32x16(va, u == 0 ? pb0 : pb1, acc[t]);
          }
      }
      block_sync();                        // stage kt is free for tile kt + 2
    }
    vmcnt_wait<0>();                       // no DMA outstanding into a reused stage
    base_t = win_end;
  }

  if (!row_ok) return;
  const float l_tot = xor32_sum(l_run);
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
           "prefill<D=%d,BM=%d,BN=%d,mfma32x32x16,lds-dma> grid=(%d,%d,%d) block=%d lds=%zu",
           a.D, kPfBM, kPfBN, a.Hq, a.B, n_qt, kPfThreads,
           a.D == 128 ? PfLds<128>::BYTES : PfLds<64>::BYTES);
  return e;
}

}  // namespace pa
