// Page criticality scores (LServe, section 4.2; PRR, section 5 for the
// GQA query; PRR, section 3.1 for the EMA update, done by the lane that
// holds the page's state):
// the score workgroup as a device function, its grid, and its tuning
// constants, shared by the score kernel and kernels that run score
// workgroups beside other work.
#pragma once

#include "dsa_common.hpp"
#include "dsa_host.hpp"

#ifndef DSA_SCORE_LOADS
#define DSA_SCORE_LOADS 8  // metadata loads in flight per lane
#endif
#ifndef DSA_SCORE_PIPE
#define DSA_SCORE_PIPE 1  // 1: the next rows' loads overlap the current rows' scores
#endif
#ifndef DSA_SCORE_MIN_PPW
#define DSA_SCORE_MIN_PPW 8  // fewest physical pages per wave while the grid keeps >= 1024 waves
#endif
#ifndef DSA_SCORE_WAVES
#define DSA_SCORE_WAVES 8192  // target waves of the score grid
#endif
#ifndef DSA_SCORE_NT
#define DSA_SCORE_NT 1  // 1: metadata loads are non-temporal (read once per step)
#endif

namespace dsa {

struct EmaArgs {
  float* level;
  float* trend;
  float* pred;
  float alpha, beta, gamma;
  int init;
};

// ============================================================ page score
// A wave walks a contiguous range of physical pages (one page-table load
// for the whole range).  Row r of the wave takes logical page 4u + r of the
// range in load pair u and each of its lanes loads the same 16 B channel
// slice of that page's kmin and kmax.  With qpos = max(qbar, 0) and
// qneg = min(qbar, 0) the lane term sum_c qpos*kmax + qneg*kmin summed over
// the row (4 DPP steps) is sum_c max(qbar_c*kmax_c, qbar_c*kmin_c): no
// cross-row traffic.  Loads of invalid pages are redirected to a valid
// address and masked, so the loop has no divergent branches.  The physical
// max over g = 2 or 4 logical pages combines rows with two swizzles.
// One 256-thread workgroup of the score grid; (bx, by, bz) is its place in
// the grid (wgs_per_row, n_kv_heads, batch), or (compact index, 0, batch)
// with streaming heads.  A __device__ body so that other kernels can run
// score workgroups beside their own.
template <typename T, int D, int G, int GL>
__device__ __forceinline__ void score_body(
    const T* __restrict__ q, const T* __restrict__ meta, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, int n_kv_heads, int P, int Pl, int max_pages, int num_slots,
    unsigned long long streaming, int pages_per_wave, int wgs_per_row, float* __restrict__ scores,
    const EmaArgs& ema, int bx, int by, int bz) {
  using L_ = Lay<T, D>;
  constexpr int CPL = L_::CPL, DW = L_::DW;
  constexpr int U = DSA_SCORE_LOADS / 2;     // load pairs in flight per lane
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int b = bz;
  // with streaming heads the grid is compact: wgs_per_row workgroups for each
  // dense head (in head order), then one workgroup per streaming head
  int h = by, xb = bx;
  if (streaming) {
    const int n_dense_wg = wgs_per_row * (n_kv_heads - __popcll(streaming));
    const bool dense = bx < n_dense_wg;
    int want = dense ? bx / wgs_per_row : bx - n_dense_wg;
    xb = dense ? bx % wgs_per_row : 0;
    for (h = 0; h < n_kv_heads; ++h) {   // the want-th head of its kind
      if ((((streaming >> h) & 1ull) == 0) == dense) {
        if (want == 0) break;
        --want;
      }
    }
  }
  const size_t rowbase = ((size_t)b * n_kv_heads + h) * max_pages;
  float* srow = scores + rowbase;
  auto put = [&](int j, float sc) {
    srow[j] = sc;
    if (ema.level) {
      const size_t x = rowbase + j;
      float nl = sc, nt = 0.0f, pr = sc;
      if (!ema.init) ema_step(sc, ema.level[x], ema.trend[x], ema.alpha, ema.beta, ema.gamma, nl, nt, pr);
      ema.level[x] = nl;
      ema.trend[x] = nt;
      ema.pred[x] = pr;
    }
  };
  if ((streaming >> h) & 1ull) {   // the whole row by one workgroup
    for (int j = threadIdx.x; j < max_pages; j += 256) put(j, kNegInf);
    return;
  }
  const int j0 = (xb * 4 + wave) * pages_per_wave;
  if (j0 >= max_pages) return;
  const int j1 = min(max_pages, j0 + pages_per_wave);
  const int L = clamp_len(seq_lens[b], max_pages, P);
  const int np = (L + P - 1) / P;

  const int r = lane >> 4, cg = lane & 15;
  // slots of this wave's pages (pages_per_wave <= 64)
  const int my_slot = (j0 + lane < min(j1, np)) ? page_table[(size_t)b * max_pages + j0 + lane] : -1;
  // lane i keeps page j0 + i's EMA state, loaded now and updated at the end
  float my_level = 0.0f, my_trend = 0.0f;
  if (ema.level && !ema.init && j0 + lane < j1) {
    my_level = ema.level[rowbase + j0 + lane];
    my_trend = ema.trend[rowbase + j0 + lane];
  }
  // the wave's scores, one per page, gathered here and written once at the
  // end: one coalesced store per output row instead of a 4-byte store per page
  __shared__ float s_wave_sc[4][64];
  // group-mean query, this lane's channels, split by sign
  float qpos[CPL], qneg[CPL];
  {
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      uint32_t w[DW];
      load_dw<DW>(q + ((size_t)b * n_kv_heads * G + (size_t)h * G + gg) * D + cg * CPL, w);
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] += chan<T>(w, c);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float qb = acc[c] * (1.0f / G);
      qpos[c] = fmaxf(qb, 0.0f);
      qneg[c] = fminf(qb, 0.0f);
    }
  }
  const size_t head_stride = (size_t)GL * 2 * D;  // elements of one (slot, head) metadata block
  const int n_pairs = ((j1 - j0) * GL + 3) / 4;    // uniform
  // loads of U rows (kmin and kmax per lane) ...
  auto issue = [&](int u0, uint32_t (&wmin)[U][DW], uint32_t (&wmax)[U][DW], bool (&ok)[U]) {
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      if (u0 + uu >= n_pairs) break;                 // uniform: no loads past the range
      const int lp = 4 * (u0 + uu) + r;            // logical page within the range
      const int pl = lp / GL, sub = lp % GL;
      const int slot = __shfl(my_slot, pl & 63, 64);
      const int pg = j0 + pl;
      ok[uu] = pg < j1 && pg < np && slot >= 0 && slot < num_slots && pg * P + sub * Pl < L;
      const T* src = ok[uu] ? meta + ((size_t)slot * n_kv_heads + h) * head_stride + (size_t)sub * 2 * D + cg * CPL
                            : meta + cg * CPL;        // valid address, result discarded
#if DSA_SCORE_NT
      load_dw_stream<DW>(src, wmin[uu]);
      load_dw_stream<DW>(src + D, wmax[uu]);
#else
      load_dw<DW>(src, wmin[uu]);
      load_dw<DW>(src + D, wmax[uu]);
#endif
    }
  };
  // ... and their scores
  auto consume = [&](int u0, const uint32_t (&wmin)[U][DW], const uint32_t (&wmax)[U][DW], const bool (&ok)[U]) {
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      if (u0 + uu >= n_pairs) break;
      float part = 0.0f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        part = fmaf(qpos[c], chan<T>(wmax[uu], c), part);
        part = fmaf(qneg[c], chan<T>(wmin[uu], c), part);
      }
      float sc = row_sum(part);
      if (!ok[uu]) sc = kNegInf;                  // invalid sub-page takes no part in the max
      const int pl = (4 * (u0 + uu) + r) / GL;
      if constexpr (GL == 2) {
        sc = fmaxf(sc, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(sc), 0x401F)));  // rows ^1
      } else if constexpr (GL == 4) {
        sc = fmaxf(sc, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(sc), 0x401F)));  // rows ^1
        sc = fmaxf(sc, __shfl_xor(sc, 32, 64));                                                     // rows ^2
      }
      const bool writer = cg == 0 && (r % GL) == 0;
      if (writer && j0 + pl < j1) s_wave_sc[wave][pl] = sc;
    }
  };
#if DSA_SCORE_PIPE
  // two register sets: the next U rows are loading while the current are scored
  uint32_t amin[U][DW], amax[U][DW], bmin[U][DW], bmax[U][DW];
  bool aok[U], bok[U];
  issue(0, amin, amax, aok);
  for (int u0 = 0; u0 < n_pairs; u0 += 2 * U) {
    if (u0 + U < n_pairs) issue(u0 + U, bmin, bmax, bok);
    consume(u0, amin, amax, aok);
    if (u0 + U >= n_pairs) break;
    if (u0 + 2 * U < n_pairs) issue(u0 + 2 * U, amin, amax, aok);
    consume(u0 + U, bmin, bmax, bok);
  }
#else
  for (int u0 = 0; u0 < n_pairs; u0 += U) {
    uint32_t wmin[U][DW], wmax[U][DW];
    bool ok[U];
    issue(u0, wmin, wmax, ok);
    consume(u0, wmin, wmax, ok);
  }
#endif
  // every page of [j0, j1) was scored by one writer lane of this wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (j0 + lane < j1) {
    const int j = j0 + lane;
    const float sc = s_wave_sc[wave][lane];
    srow[j] = sc;
    if (ema.level) {
      const size_t x = rowbase + j;
      float nl = sc, nt = 0.0f, pr = sc;
      if (!ema.init) ema_step(sc, my_level, my_trend, ema.alpha, ema.beta, ema.gamma, nl, nt, pr);
      ema.level[x] = nl;
      ema.trend[x] = nt;
      ema.pred[x] = pr;
    }
  }
}


// Grid of the score kernel: each wave walks a range of <= 64 physical pages
// (one page-table load); aim for DSA_SCORE_WAVES waves over the grid.
struct ScorePlan {
  int ppw, wgs;   // pages per wave, workgroups per dense row
  dim3 grid;
};
template <int G>
inline ScorePlan score_plan(const dsa_kv* kv, uint64_t smask) {
  const long long units = (long long)kv->batch * kv->n_kv_heads;
  // every wave forms the group-mean query itself: with many heads per group
  // fewer, longer waves read less of it
  const long long target_waves = (long long)DSA_SCORE_WAVES * 4 / (G > 4 ? G : 4);
  long long ppw = (units * kv->max_pages + target_waves - 1) / target_waves;
  // small grids take fewer, longer waves, unless that would leave under 1024
  const long long min_ppw = units * kv->max_pages >= (long long)DSA_SCORE_MIN_PPW * 1024 ? DSA_SCORE_MIN_PPW : 4;
  ppw = ppw < min_ppw ? min_ppw : (ppw > 64 ? 64 : ppw);
  ppw = (ppw + 3) / 4 * 4;
  ScorePlan p;
  p.ppw = (int)ppw;
  p.wgs = ceil_div(ceil_div(kv->max_pages, p.ppw), 4);
  const int n_stream = __builtin_popcountll(smask);
  p.grid = smask ? dim3(p.wgs * (kv->n_kv_heads - n_stream) + n_stream, 1, kv->batch)
                 : dim3(p.wgs, kv->n_kv_heads, kv->batch);
  return p;
}

}  // namespace dsa
