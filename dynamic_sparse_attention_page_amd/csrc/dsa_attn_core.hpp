// Online-softmax attention over 16-token KV tiles for the G q heads of one
// KV head, on one wave.
//
// The (O, l, m) state and its update follow the online-softmax recurrence of
// PRR ("Predict, Reuse, and Repair", section 3.3): a new block moves the
// running max to max(m, m~), rescales the old denominator and output by
// exp(m - m_new) and adds the block's exp(s - m_new) terms.
//
// Work split inside the wave.  Each of the 4 DPP rows (16 lanes) owns token
// 4i + row (i = 0..3) of every tile and keeps its own running state, so no
// cross-row traffic is needed per tile; rows are merged once at the end with
// the same recurrence.  In a row, lane j holds channels [j*CPL, +CPL) of the
// 4 tokens and of every q head.  Per tile:
//   1. 4G partial dot products per lane (v_dot2_f32_bf16 for bf16 KV),
//   2. a row reduce-scatter leaves lane j with the full logits of token
//      i = j/4 for heads [(j%4)*G/4, +G/4) (G >= 4),
//   3. max over the row's 4 tokens per head (row rotations), new running
//      max, p = exp2((s - m) * scale * log2 e),
//   4. the row's p values and rescale factors go through LDS so every lane
//      can update its output channels for all heads.
// Logits are kept as raw q.k; `c` = scale * log2(e) converts differences.
#pragma once

#include "dsa_common.hpp"

namespace dsa {

template <typename T, int D, int G>
struct AttnWave {
  static constexpr int CPL = Lay<T, D>::CPL;
  static constexpr int DW = Lay<T, D>::DW;
  static constexpr int NV = 4 * G;
  static constexpr int NOWN = G >= 4 ? G / 4 : 1;
  static constexpr int LDS_ROW = (6 * G + 3) / 4 * 4;  // p[4G], alpha/l[G], m[G]; 16 B aligned
  static constexpr int LDS_FLOATS = 4 * LDS_ROW;   // per wave

  int lane, r, j, i_own, hbase;
  uint32_t qd[G][DW];
  float o[G][CPL];
  float m_own[NOWN];
  float lp[NOWN];
  float* lds;  // this wave's LDS_FLOATS floats

  __device__ __forceinline__ void init(const T* __restrict__ q_heads /* [G][D] of this KV head */, float* lds_) {
    lane = threadIdx.x & 63;
    r = lane >> 4;
    j = lane & 15;
    i_own = j >> 2;
    hbase = G >= 4 ? (j & 3) * (G / 4) : (G == 2 ? ((j >> 1) & 1) : 0);
    lds = lds_;
#pragma unroll
    for (int h = 0; h < G; ++h) load_dw<DW>(q_heads + (size_t)h * D + j * CPL, qd[h]);
    reset();
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[h][c] = 0.0f;
#pragma unroll
    for (int u = 0; u < NOWN; ++u) { m_own[u] = kNegInf; lp[u] = 0.0f; }
  }

  // Raw loads of this lane's part of a 16-token tile (rows 4i + r).
  __device__ __forceinline__ static void load_tile(const T* __restrict__ tile, int lane_, uint32_t (&d)[4][DW]) {
    const int rr = lane_ >> 4, jj = lane_ & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_dw_kv<DW>(tile + (size_t)(4 * i + rr) * D + jj * CPL, d[i]);
  }

  // Token t (0..15) of the tile takes part iff t < nvalid and, for a
  // streaming head, its sequence position is a sink or local token.
  __device__ __forceinline__ static bool tok_ok(int t, int nvalid, bool smask, int tok0, int L, int sink,
                                                int local) {
    bool ok = t < nvalid;
    if (smask) {
      const int gt = tok0 + t;
      ok = ok && (gt < sink || gt >= L - local);
    }
    return ok;
  }

  __device__ __forceinline__ void tile(const uint32_t (&kd)[4][DW], uint32_t (&vd)[4][DW], int nvalid, bool smask,
                                       int tok0, int L, int sink, int local, float c) {
    float s[NV];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int h = 0; h < G; ++h) s[i * G + h] = lane_dot<T, DW>(kd[i], qd[h]);
    row_sum_scatter<NV>(s, j);
    const bool ok = tok_ok(4 * i_own + r, nvalid, smask, tok0, L, sink, local);
    float* pb = lds + r * LDS_ROW;
#pragma unroll
    for (int u = 0; u < NOWN; ++u) {
      const float su = ok ? s[u] : kNegInf;
      const float mn = fmaxf(m_own[u], ror_max4(su));
      const float alpha = (mn == kNegInf) ? 1.0f : fast_exp2((m_own[u] - mn) * c);
      const float p = exp2_diff(su, mn, c);
      lp[u] = fmaf(lp[u], alpha, p);
      m_own[u] = mn;
      pb[i_own * G + hbase + u] = p;
      if (i_own == 0) pb[4 * G + hbase + u] = alpha;
    }
    wave_sync();
    float pr[4 * G], al[G];
#pragma unroll
    for (int x = 0; x < 4 * G; x += 4) {
      const float4 t4 = *reinterpret_cast<const float4*>(pb + x);
      pr[x] = t4.x; pr[x + 1] = t4.y; pr[x + 2] = t4.z; pr[x + 3] = t4.w;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) al[h] = pb[4 * G + h];
    wave_sync();
    if (nvalid < 16 || smask) {  // masked rows may hold non-finite garbage: keep 0 * v finite
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!tok_ok(4 * i + r, nvalid, smask, tok0, L, sink, local))
#pragma unroll
          for (int x = 0; x < DW; ++x) vd[i][x] = 0u;
    }
    bool moved = false;
#pragma unroll
    for (int h = 0; h < G; ++h) moved |= al[h] != 1.0f;
    if (__builtin_amdgcn_read_exec() & __ballot(moved)) {  // skip the rescale once the maxima settle
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) o[h][cc] *= al[h];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        const float v = chan<T>(vd[i], cc);
#pragma unroll
        for (int h = 0; h < G; ++h) o[h][cc] = fmaf(pr[i * G + h], v, o[h][cc]);
      }
    }
  }

  // Row totals without the cross-row merge: every lane gets m[h] (raw max)
  // and l[h] of its own row; o stays per row.
  __device__ __forceinline__ void row_totals(float (&m)[G], float (&l)[G]) {
    float* pb = lds + r * LDS_ROW;
#pragma unroll
    for (int u = 0; u < NOWN; ++u) {
      const float ls = ror_sum4(lp[u]);
      if (i_own == 0) {
        pb[4 * G + hbase + u] = ls;
        pb[5 * G + hbase + u] = m_own[u];
      }
    }
    wave_sync();
#pragma unroll
    for (int h = 0; h < G; ++h) { l[h] = pb[4 * G + h]; m[h] = pb[5 * G + h]; }
    wave_sync();
  }

  // Collapse the 4 row states into one wave state.  Afterwards every lane
  // holds m[h] (raw max), l[h] for all heads and o[h][channels of j]
  // (unnormalised), identical in the 4 rows.
  __device__ __forceinline__ void finish(float (&m)[G], float (&l)[G], float c) {
    float* pb = lds + r * LDS_ROW;
#pragma unroll
    for (int u = 0; u < NOWN; ++u) {
      const float ls = ror_sum4(lp[u]);
      if (i_own == 0) {
        pb[4 * G + hbase + u] = ls;
        pb[5 * G + hbase + u] = m_own[u];
      }
    }
    wave_sync();
#pragma unroll
    for (int h = 0; h < G; ++h) { l[h] = pb[4 * G + h]; m[h] = pb[5 * G + h]; }
    wave_sync();
#pragma unroll
    for (int step = 16; step <= 32; step <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mp = shfl_xor_f(m[h], step);
        const float lq = shfl_xor_f(l[h], step);
        const float mm = fmaxf(m[h], mp);
        const float a = exp2_diff(m[h], mm, c);
        const float bq = exp2_diff(mp, mm, c);
        l[h] = l[h] * a + lq * bq;
        m[h] = mm;
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) o[h][cc] = o[h][cc] * a + shfl_xor_f(o[h][cc], step) * bq;
      }
    }
  }
};

}  // namespace dsa
