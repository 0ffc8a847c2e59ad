// Sparse decode attention over selected pages, its split-KV combine, PRR's
// repair and PSA's progressive selection.
//
// sparse_decode_attn (LServe, section 3.3: the decode kernel iterates only
//   over the needed pages, loop step -> page index -> cache slot; PRR,
//   section 3.3: the speculative kernel also emits l and m per head).
//   Split-KV: a workgroup of 4 waves takes one (sequence, KV head, range of
//   16-token tiles of the selected pages), computes all G q heads of the
//   group from one read of each K/V tile, merges its waves through LDS and
//   writes one unnormalised partial (o, l, m); the combine kernel folds the
//   partials of a head with the online-softmax merge.
// attn_repair (PRR, sections 3.3-3.4): the split-KV path runs over A with
//   an LDS bitmap of P in each workgroup, so only the missing set M = A \ P
//   is attended, and the combine folds the caller's speculative (O, l, m) in
//   as one more partial.
// page_select_progressive (PSA, section 3.2, with the GPU-side weight check
//   of section 3.3): one workgroup per (sequence, KV head) selects the next
//   pages by score in rounds, computes the (o, l, m) of 16 of them at a time
//   in parallel and applies the stop test to them in rank order with prefix
//   scans; no host sync.
#include "dsa_attn_core.hpp"
#include "dsa_attn_mfma.hpp"
#include "dsa_host.hpp"
#include "dsa_select.hpp"

#include <mutex>

#ifndef DSA_TILES_PER_WAVE
#define DSA_TILES_PER_WAVE 2  // 16-token K/V tiles per wave of the VALU partial kernel (all in flight at once)
#endif
#ifndef DSA_TILES_PER_WAVE_MFMA
#define DSA_TILES_PER_WAVE_MFMA 4  // the same for the matrix-core partial kernel
#endif

namespace dsa {

constexpr int kWgWaves = 4;
constexpr int kTilesPerWave = DSA_TILES_PER_WAVE;
constexpr int kTilesPerWaveMfma = DSA_TILES_PER_WAVE_MFMA;

// Fused selection (dsa_sparse_decode_attn_topk): each split workgroup ranks
// its row of scores itself and takes the entries of its range; split 0
// writes the ids and count.  e == 0: ids/counts are inputs.
struct SelectArgs {
  const float* scores;
  int k;
  int32_t* ids_out;
  int32_t* counts_out;
  int e;      // scores per thread: max_pages <= 256 * e
  int fine;   // split as finely as possible: the ids are a short prefix of a long row
};

// ============================================================ split-KV partial
template <typename T, int D, int G, bool FILTER, int SEL_E>
__global__ __launch_bounds__(256) void attn_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ counts, int ids_stride, int n_kv_heads, int P,
    int max_pages, int num_slots, unsigned long long streaming, int sink, int local, float scale, float c,
    int tiles_per_split, int n_splits, const int32_t* __restrict__ skip_ids,
    const int32_t* __restrict__ skip_counts, SelectArgs sel, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  using A = AttnWave<T, D, G>;
  constexpr int CPL = A::CPL, DW = A::DW;
  __shared__ __align__(16) float lds_rows[kWgWaves][A::LDS_FLOATS];
  // row-state merge buffers: 16 row states for G <= 4, 4 wave states above
  constexpr int NSTATE = G <= 4 ? 16 : 1;
  constexpr int NWS = G <= 4 ? 1 : kWgWaves;
  __shared__ __align__(16) float rs_o[NSTATE][G][D];
  __shared__ float rs_ml[NSTATE][G][2];
  __shared__ __align__(16) float lds_o[NWS][G][D];
  __shared__ float lds_ml[NWS][G][2];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  // the wave index is uniform: loop bounds and branches derived from it stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int unit = b * n_kv_heads + h;
  const int TPP = P / 16;
  const int t_begin = split * tiles_per_split;
  const int first_entry = t_begin / TPP;
  int pg_raw = -1, sl_raw = -1;
  int cnt;
  if constexpr (SEL_E > 0) {
    // the selection of dsa_page_select_topk, recomputed by every split of
    // the row (no cross-workgroup traffic); entries are in ascending order
    __shared__ SelectSmem<SEL_E, kWgWaves> ssm;
    __shared__ int s_pages[64];
    const int tid = threadIdx.x;
    const int L0 = clamp_len(seq_lens[b], max_pages, P);
    const int np0 = (L0 + P - 1) / P;
    const int nslot = tiles_per_split / TPP;
    int32_t* out = sel.ids_out + (size_t)unit * sel.k;
    if ((streaming >> h) & 1ull) {
      const int n_sink = min(np0, (min(sink, L0) + P - 1) / P);
      const int l_first = max(n_sink, (local > 0 && L0 > 0) ? max(0, L0 - local) / P : np0);
      cnt = min(sel.k, n_sink + (np0 - l_first));
      const int x = first_entry + lane;
      if (lane < nslot && x < cnt) pg_raw = x < n_sink ? x : l_first + (x - n_sink);
      if (split == 0) {
        for (int y = tid; y < sel.k; y += 256) out[y] = y < cnt ? (y < n_sink ? y : l_first + (y - n_sink)) : -1;
        if (tid == 0) sel.counts_out[unit] = cnt;
      }
    } else {
      cnt = min(sel.k, np0);
      const float* srow = sel.scores + (size_t)unit * max_pages;
      float sv[SEL_E];
#pragma unroll
      for (int e = 0; e < SEL_E; ++e) sv[e] = (e * 256 + tid < max_pages) ? srow[e * 256 + tid] : 0.0f;
      uint32_t key[SEL_E];
      unsigned long long actm = 0ull;
#pragma unroll
      for (int e = 0; e < SEL_E; ++e) {
        key[e] = order_key(sv[e]);
        if (e * 256 + tid < np0) actm |= 1ull << e;
      }
      const unsigned long long selm = block_select_top<SEL_E, kWgWaves>(key, actm, np0, cnt, ssm);
      int rk[SEL_E];
      ordered_ranks<SEL_E, kWgWaves>(selm, rk, ssm.rank, ssm.scan);
#pragma unroll
      for (int e = 0; e < SEL_E; ++e)
        if ((selm >> e) & 1ull) {
          const int r = rk[e];
          if (r >= first_entry && r < first_entry + nslot) s_pages[r - first_entry] = e * 256 + tid;
          if (split == 0 && r < cnt) out[r] = e * 256 + tid;
        }
      if (split == 0) {
        for (int y = cnt + tid; y < sel.k; y += 256) out[y] = -1;
        if (tid == 0) sel.counts_out[unit] = cnt;
      }
      __syncthreads();
      if (lane < nslot && first_entry + lane < cnt) pg_raw = s_pages[lane];
    }
    if (pg_raw >= 0 && pg_raw < max_pages) sl_raw = page_table[(size_t)b * max_pages + pg_raw];
  } else {
    // The id and its slot are fetched together with the count (the count
    // only decides later which of them are used): entry -> page -> slot is
    // one dependent hop instead of two.
    if (lane < tiles_per_split / TPP && first_entry + lane < ids_stride) {
      pg_raw = ids[(size_t)unit * ids_stride + first_entry + lane];
      if (pg_raw >= 0 && pg_raw < max_pages) sl_raw = page_table[(size_t)b * max_pages + pg_raw];
    }
    cnt = counts[unit];
    cnt = cnt < 0 ? 0 : (cnt > ids_stride ? ids_stride : cnt);
  }
  const int n_tiles = cnt * TPP;
  if (t_begin >= n_tiles) return;  // whole workgroup: the combine reads only active splits
  const int t_end = min(n_tiles, t_begin + tiles_per_split);
  const int L = clamp_len(seq_lens[b], max_pages, P);
  const int np = (L + P - 1) / P;
  const bool smask = (streaming >> h) & 1ull;
  if constexpr (FILTER) {
    // pages listed in skip_ids (PRR's speculative set P) are left out: an
    // LDS bitmap of them filters this split's entries (M = A \ P in place)
    extern __shared__ uint32_t skip_bits[];
    const int nwords = (max_pages + 31) >> 5;
    for (int x = threadIdx.x; x < nwords; x += 256) skip_bits[x] = 0u;
    __syncthreads();
    int pc = skip_counts[unit];
    pc = pc < 0 ? 0 : (pc > ids_stride ? ids_stride : pc);
    for (int x = threadIdx.x; x < pc; x += 256) {
      const int pg = skip_ids[(size_t)unit * ids_stride + x];
      if (pg >= 0 && pg < max_pages) atomicOr(&skip_bits[pg >> 5], 1u << (pg & 31));
    }
    __syncthreads();
    if (pg_raw >= 0 && pg_raw < max_pages && ((skip_bits[pg_raw >> 5] >> (pg_raw & 31)) & 1u)) sl_raw = -1;
  }

  A st;
  st.init(q + ((size_t)b * n_kv_heads * G + (size_t)h * G) * D, lds_rows[wave]);

  const int n_entries = (t_end - 1) / TPP - first_entry + 1;
  int my_page = -1, my_slot = -1;
  if (lane < n_entries && pg_raw >= 0 && pg_raw < np && sl_raw >= 0 && sl_raw < num_slots) {
    my_page = pg_raw;
    my_slot = sl_raw;
  }
  const size_t slot_stride = (size_t)n_kv_heads * P * D;
  const size_t head_off = (size_t)h * P * D;

  // The TW tiles of this wave (t_begin + wave + 4i) are loaded together and
  // then computed in order: every load is issued before the first wait, and
  // unconditionally (a tile past the split's end, or of a page without a
  // slot, re-reads tile 0 of slot 0 of this head and is skipped), so no
  // wait covers a load that is not needed yet.
  constexpr int TW = kTilesPerWave;
  uint32_t kd[TW][4][DW], vd[TW][4][DW];
  int nv[TW], tk[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const int t = t_begin + wave + kWgWaves * i;
    const int e = t / TPP - first_entry, tin = t % TPP;   // e < 64: a split holds at most 64 entries
    const int page = __builtin_amdgcn_readlane(my_page, e);
    const int slot = __builtin_amdgcn_readlane(my_slot, e);
    const bool ok = t < t_end && slot >= 0;
    tk[i] = page * P + tin * 16;
    nv[i] = ok ? min(16, L - tk[i]) : 0;
    const size_t off = ok ? (size_t)slot * slot_stride + head_off + (size_t)tin * 16 * D : head_off;
    A::load_tile(k + off, lane, kd[i]);
    A::load_tile(v + off, lane, vd[i]);
    __builtin_amdgcn_sched_barrier(0);   // keep the issue order tile by tile (K, V, next tile)
  }
#pragma unroll
  for (int i = 0; i < TW; ++i)
    if (nv[i] > 0) st.tile(kd[i], vd[i], nv[i], smask, tk[i], L, sink, local, c);

  const size_t pbase = ((size_t)unit * n_splits + split) * G;
  if constexpr (G <= 4) {
    // 16 row states (4 waves x 4 rows) meet in LDS; one pass merges them
    float m[G], l[G];
    st.row_totals(m, l);
    const int row = wave * 4 + (lane >> 4);
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) rs_o[row][hh][(lane & 15) * CPL + cc] = st.o[hh][cc];
    if ((lane & 15) == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) { rs_ml[row][hh][0] = m[hh]; rs_ml[row][hh][1] = l[hh]; }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
      const int hh = idx / D, cc = idx % D;
      float mm = kNegInf;
#pragma unroll
      for (int w = 0; w < 16; ++w) mm = fmaxf(mm, rs_ml[w][hh][0]);
      float acc = 0.0f, ls = 0.0f;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const float wt = exp2_diff(rs_ml[w][hh][0], mm, c);
        acc = fmaf(rs_o[w][hh][cc], wt, acc);
        ls = fmaf(rs_ml[w][hh][1], wt, ls);
      }
      part_o[(pbase + hh) * D + cc] = acc;
      if (cc == 0) {
        part_ml[(pbase + hh) * 2 + 0] = (mm == kNegInf) ? kNegInf : mm * scale;  // natural-log units
        part_ml[(pbase + hh) * 2 + 1] = ls;
      }
    }
  } else {
    float m[G], l[G];
    st.finish(m, l, c);
    if (lane < 16) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) lds_o[wave][hh][lane * CPL + cc] = st.o[hh][cc];
    }
    if (lane == 0) {
#pragma unroll
      for (int hh = 0; hh < G; ++hh) { lds_ml[wave][hh][0] = m[hh]; lds_ml[wave][hh][1] = l[hh]; }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
      const int hh = idx / D, cc = idx % D;
      float mm = kNegInf;
#pragma unroll
      for (int w = 0; w < kWgWaves; ++w) mm = fmaxf(mm, lds_ml[w][hh][0]);
      float acc = 0.0f, ls = 0.0f;
#pragma unroll
      for (int w = 0; w < kWgWaves; ++w) {
        const float wt = exp2_diff(lds_ml[w][hh][0], mm, c);
        acc = fmaf(lds_o[w][hh][cc], wt, acc);
        ls = fmaf(lds_ml[w][hh][1], wt, ls);
      }
      part_o[(pbase + hh) * D + cc] = acc;
      if (cc == 0) {
        part_ml[(pbase + hh) * 2 + 0] = (mm == kNegInf) ? kNegInf : mm * scale;  // natural-log units
        part_ml[(pbase + hh) * 2 + 1] = ls;
      }
    }
  }
}

// ============================================================ split-KV partial, matrix cores
// Same split and output as attn_partial_kernel, for bf16 KV with 8 or 16 q
// heads per KV head: each wave runs the MFMA tile of dsa_attn_mfma.hpp over
// its tiles, and the 4 wave states meet in LDS.
template <int D, int G, bool FILTER>
__global__ __launch_bounds__(256) void attn_partial_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ counts, int ids_stride, int n_kv_heads, int P,
    int max_pages, int num_slots, unsigned long long streaming, int sink, int local, float scale, float c,
    int tiles_per_split, int n_splits, const int32_t* __restrict__ skip_ids,
    const int32_t* __restrict__ skip_counts, SelectArgs, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  using M = MfmaWave<D, G>;
  constexpr int NK = M::NK, NB = M::NB;
  constexpr int OS = D + 4;   // LDS row stride of the merge buffer (floats)
  __shared__ __align__(16) uint16_t lds_v[kWgWaves][M::LDS_ELEMS];
  __shared__ __align__(16) float lds_o[kWgWaves][G][OS];
  __shared__ float lds_ml[kWgWaves][G][2];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  // the wave index is uniform: loop bounds and branches derived from it stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int unit = b * n_kv_heads + h;
  const int TPP = P / 16;
  const int t_begin = split * tiles_per_split;
  const int first_entry = t_begin / TPP;
  int pg_raw = -1, sl_raw = -1;
  if (lane < tiles_per_split / TPP && first_entry + lane < ids_stride) {
    pg_raw = ids[(size_t)unit * ids_stride + first_entry + lane];
    if (pg_raw >= 0 && pg_raw < max_pages) sl_raw = page_table[(size_t)b * max_pages + pg_raw];
  }
  int cnt = counts[unit];
  cnt = cnt < 0 ? 0 : (cnt > ids_stride ? ids_stride : cnt);
  const int n_tiles = cnt * TPP;
  if (t_begin >= n_tiles) return;  // whole workgroup: the combine reads only active splits
  const int t_end = min(n_tiles, t_begin + tiles_per_split);
  const int L = clamp_len(seq_lens[b], max_pages, P);
  const int np = (L + P - 1) / P;
  const bool smask = (streaming >> h) & 1ull;
  if constexpr (FILTER) {
    // pages listed in skip_ids (PRR's speculative set P) are left out: an
    // LDS bitmap of them filters this split's entries (M = A \ P in place)
    extern __shared__ uint32_t skip_bits[];
    const int nwords = (max_pages + 31) >> 5;
    for (int x = threadIdx.x; x < nwords; x += 256) skip_bits[x] = 0u;
    __syncthreads();
    int pc = skip_counts[unit];
    pc = pc < 0 ? 0 : (pc > ids_stride ? ids_stride : pc);
    for (int x = threadIdx.x; x < pc; x += 256) {
      const int pg = skip_ids[(size_t)unit * ids_stride + x];
      if (pg >= 0 && pg < max_pages) atomicOr(&skip_bits[pg >> 5], 1u << (pg & 31));
    }
    __syncthreads();
    if (pg_raw >= 0 && pg_raw < max_pages && ((skip_bits[pg_raw >> 5] >> (pg_raw & 31)) & 1u)) sl_raw = -1;
  }

  M st;
  st.init(q + ((size_t)b * n_kv_heads * G + (size_t)h * G) * D, lds_v[wave]);

  const int n_entries = (t_end - 1) / TPP - first_entry + 1;
  int my_page = -1, my_slot = -1;
  if (lane < n_entries && pg_raw >= 0 && pg_raw < np && sl_raw >= 0 && sl_raw < num_slots) {
    my_page = pg_raw;
    my_slot = sl_raw;
  }
  const size_t slot_stride = (size_t)n_kv_heads * P * D;
  const size_t head_off = (size_t)h * P * D;

  // The TW tiles of this wave, loaded together and computed in order (see
  // attn_partial_kernel).
  constexpr int TW = kTilesPerWaveMfma;
  uint4 kr[TW][NK], vr[TW][NK];
  int nv[TW], tk[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i) {
    const int t = t_begin + wave + kWgWaves * i;
    const int e = t / TPP - first_entry, tin = t % TPP;   // e < 64: a split holds at most 64 entries
    const int page = __builtin_amdgcn_readlane(my_page, e);
    const int slot = __builtin_amdgcn_readlane(my_slot, e);
    const bool ok = t < t_end && slot >= 0;
    tk[i] = page * P + tin * 16;
    nv[i] = ok ? min(16, L - tk[i]) : 0;
    const size_t off = ok ? (size_t)slot * slot_stride + head_off + (size_t)tin * 16 * D : head_off;
    M::load_k(k + off, lane, kr[i]);
    M::load_v(v + off, lane, vr[i]);
    __builtin_amdgcn_sched_barrier(0);   // keep the issue order tile by tile (K, V, next tile)
  }
#pragma unroll
  for (int i = 0; i < TW; ++i)
    if (nv[i] > 0) st.tile(kr[i], vr[i], nv[i], smask, tk[i], L, sink, local, c);

  // wave states meet in LDS: lane holds O[head h][16n + 4g + j]
  const float lsum = st.total_l();
  if (st.h < G) {
#pragma unroll
    for (int n = 0; n < NB; ++n)
      *reinterpret_cast<float4*>(&lds_o[wave][st.h][16 * n + 4 * st.g]) =
          make_float4(st.acc[n][0], st.acc[n][1], st.acc[n][2], st.acc[n][3]);
    if (st.g == 0) { lds_ml[wave][st.h][0] = st.m; lds_ml[wave][st.h][1] = lsum; }
  }
  __syncthreads();
  const size_t pbase = ((size_t)unit * n_splits + split) * G;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int hh = idx / D, cc = idx % D;
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < kWgWaves; ++w) mm = fmaxf(mm, lds_ml[w][hh][0]);
    float acc = 0.0f, ls = 0.0f;
#pragma unroll
    for (int w = 0; w < kWgWaves; ++w) {
      const float wt = exp2_diff(lds_ml[w][hh][0], mm, c);
      acc = fmaf(lds_o[w][hh][cc], wt, acc);
      ls = fmaf(lds_ml[w][hh][1], wt, ls);
    }
    part_o[(pbase + hh) * D + cc] = acc;
    if (cc == 0) {
      part_ml[(pbase + hh) * 2 + 0] = (mm == kNegInf) ? kNegInf : mm * scale;  // natural-log units
      part_ml[(pbase + hh) * 2 + 1] = ls;
    }
  }
}

// ============================================================ combine
// One workgroup per (sequence, q head).  The active splits are merged with
// the online-softmax rule in chunks of 64: every thread first issues the
// loads of all the O values it needs from the chunk (thread (sub, c) takes
// channel c of splits sub, sub + SPT, ...), wave 0 loads the chunk's
// (m, l) pairs, one per lane, and turns them into merge weights against the
// running maximum (wave reductions, no barrier), and after one barrier every
// thread folds its values.  So a chunk costs one memory round trip, and
// rows of up to 64 splits (every top-k and repair call here) exactly one.
// For repair the caller's (O, l, m) is one more term.  Writes normalised O.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, const int32_t* __restrict__ counts,
    int ids_stride, int n_kv_heads, int G, int TPP, int tiles_per_split, int n_splits, int fold,
    float* __restrict__ O, float* __restrict__ l, float* __restrict__ m) {
  constexpr int SPT = 256 / D;   // split lanes per channel
  constexpr int CH = 64;         // splits per chunk
  constexpr int PER = CH / SPT;  // O values per thread and chunk
  __shared__ float s_w[CH];
  __shared__ float s_acc[SPT][D];
  __shared__ float s_alpha, s_M, s_L;
  const int hq = blockIdx.x, b = blockIdx.y;
  const int Hq = n_kv_heads * G;
  const int h = hq / G, g = hq % G;
  const int unit = b * n_kv_heads + h;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = tid % D, sub = tid / D;   // sub is uniform within a wave
  const size_t row = (size_t)b * Hq + hq;
  int cnt = counts[unit];
  cnt = cnt < 0 ? 0 : (cnt > ids_stride ? ids_stride : cnt);
  const int active = min(n_splits, (cnt * TPP + tiles_per_split - 1) / tiles_per_split);
  const size_t base = (size_t)unit * n_splits * G + g;   // split s: partial row base + s * G
  // the caller's (O, l, m) for repair, read before any of it is rewritten
  // (the writes follow the last barrier)
  float o_in = 0.0f, m_in = kNegInf, l_in = 0.0f;
  if (fold && tid < D) {
    o_in = O[row * D + c];
    m_in = m[row];
    l_in = l[row];
  }

  float acc = 0.0f;
  float M = kNegInf, Lw = 0.0f;   // running max and denominator (wave 0)
  for (int s0 = 0; s0 < active; s0 += CH) {
    const int n = min(CH, active - s0);
    float ov[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int sp = s0 + min(sub + SPT * j, n - 1);   // in bounds; the surplus is weighted out
      ov[j] = part_o[(base + (size_t)sp * G) * D + c];
    }
    if (wave == 0) {
      const int sp = s0 + min(lane, n - 1);
      float ms = part_ml[(base + (size_t)sp * G) * 2];
      const float ls = part_ml[(base + (size_t)sp * G) * 2 + 1];
      if (lane >= n || !(ls > 0.0f)) ms = kNegInf;    // surplus lanes and empty splits drop out
      float mb = ms;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) mb = fmaxf(mb, __shfl_xor(mb, d, 64));
      const float Mn = fmaxf(M, mb);
      const float w = (ms == kNegInf) ? 0.0f : expf(ms - Mn);
      const float alpha = (M == kNegInf) ? 0.0f : expf(M - Mn);
      float lw = w * (ms == kNegInf ? 0.0f : ls);
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) lw += __shfl_xor(lw, d, 64);
      Lw = fmaf(Lw, alpha, lw);
      M = Mn;
      s_w[lane] = w;
      if (lane == 0) s_alpha = alpha;
    }
    __syncthreads();
    const float alpha = s_alpha;
    acc *= alpha;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc = fmaf(ov[j], s_w[sub + SPT * j], acc);   // s_w is 0 past n
    __syncthreads();   // s_w and s_alpha are rewritten by the next chunk
  }
  if (wave == 0 && lane == 0) { s_M = M; s_L = Lw; }
  s_acc[sub][c] = acc;
  __syncthreads();
  if (tid < D) {
    float Mf = s_M, Lf = s_L, o = 0.0f;
#pragma unroll
    for (int x = 0; x < SPT; ++x) o += s_acc[x][c];
    if (fold && l_in > 0.0f && m_in != kNegInf) {   // the caller's term: its O is normalised
      const float Mn = fmaxf(Mf, m_in);
      const float a = (Mf == kNegInf) ? 0.0f : expf(Mf - Mn);
      const float wt = expf(m_in - Mn) * l_in;
      o = fmaf(o, a, o_in * wt);
      Lf = fmaf(Lf, a, wt);
      Mf = Mn;
    }
    O[row * D + c] = Lf > 0.0f ? o / Lf : 0.0f;
    if (c == 0) {
      l[row] = Lf;
      m[row] = Lf > 0.0f ? Mf : kNegInf;
    }
  }
}

// ============================================================ PSA progressive
// One workgroup of NWV waves per (sequence, KV head).  Pages are taken in
// rounds: the block radix select picks the next 64 (then 256) pages by score
// among those not yet taken, a counting sort puts them in rank order (score
// descending, lower index first on ties), and the walk attends to them NWV
// at a time -- wave w computes the (o, l, m) of the page at rank cs + w.
// The stop test of each group runs as prefix scans over NWV lanes of wave
// 0: running log-sum of the block masses and running minimum, then the first
// rank whose test passes ends the walk.  The visited blocks are folded into
// the output with the online-softmax merge, in rank order.
constexpr int kPsaMaxPages = 8192;
constexpr int kPsaFirst = 64;    // pages of the first round
constexpr int kPsaRound = 256;   // pages of each later round

// 16 waves where a wave's tile state fits 128 registers, else 8
template <typename T, int G>
constexpr int psa_waves() { return (G == 1 && sizeof(T) == 2) ? 16 : 8; }

__device__ __forceinline__ float log_add(float a, float b) {
  const float mx = fmaxf(a, b), mn = fminf(a, b);
  if (mn == kNegInf) return mx;
  return mx + log1pf(expf(mn - mx));
}

// E scores per thread: rows up to E * NT pages (the launch takes the
// smallest E that holds max_pages, so short rows carry no padding).
template <typename T, int D, int G, int E>
__global__ __launch_bounds__((psa_waves<T, G>() * 64)) void psa_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens, const float* __restrict__ scores,
    int n_kv_heads, int P, int max_pages, int num_slots, int stop_mode, int never_stop, int always_stop,
    float ln_odds, float scale, float c, int32_t* __restrict__ ids, int32_t* __restrict__ counts,
    float* __restrict__ O, float* __restrict__ l, float* __restrict__ m) {
  using A = AttnWave<T, D, G>;
  constexpr int CPL = A::CPL, DW = A::DW;
  constexpr int NWV = psa_waves<T, G>();
  constexpr int NT = NWV * 64;
  static_assert(E * NT <= kPsaMaxPages, "row capacity");
  static_assert(G * D <= NT, "one output element per thread");
  __shared__ SelectSmem<E, NWV> sm;
  __shared__ unsigned long long s_key[kPsaRound];  // picks of the round: score key << 32 | ~index
  __shared__ uint32_t s_keys[E * NT];                  // score keys, element order
  __shared__ int s_page[kPsaRound], s_slot[kPsaRound];  // in rank order
  __shared__ __align__(16) float lds_rows[NWV][A::LDS_FLOATS];
  __shared__ __align__(16) float ch_o[NWV][G][D];
  __shared__ float ch_ml[NWV][G][2];
  __shared__ int s_take, s_stop, s_left;
  __shared__ float s_lnacc, s_lnmin;
  __shared__ float s_wt[NWV][G], s_alpha[G], s_accm[G];  // merge weights; running max per head

  const int h = blockIdx.x, b = blockIdx.y;
  const int unit = b * n_kv_heads + h;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int L = clamp_len(seq_lens[b], max_pages, P);
  const int np = (L + P - 1) / P;
  const float* srow = scores + (size_t)unit * max_pages;
  int32_t* irow = ids + (size_t)unit * max_pages;
  const int32_t* ptrow = page_table + (size_t)b * max_pages;

  // scores are loaded up to max_pages, so the loads do not wait for seq_lens
  float sv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sv[e] = (e * NT + tid < max_pages) ? srow[e * NT + tid] : 0.0f;
  uint32_t key[E];
  unsigned long long remm = 0ull;  // bit e: page e * NT + tid not taken yet
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int idx = e * NT + tid;
    key[e] = order_key(sv[e]);
    if (idx < np) remm |= 1ull << e;
  }

  A st;
  st.init(q + ((size_t)b * n_kv_heads * G + (size_t)h * G) * D, lds_rows[wave]);
  const size_t slot_stride = (size_t)n_kv_heads * P * D;
  const size_t head_off = (size_t)h * P * D;
  const int TPP = P / 16;
  float acc_o = 0.0f, acc_l = 0.0f;  // thread tid < G*D owns element tid
  const int my_h = tid / D, my_c = tid % D;
  if (tid == 0) { s_lnacc = kNegInf; s_lnmin = __builtin_huge_valf(); s_left = np; s_stop = 0; }
  if (tid < G) s_accm[tid] = kNegInf;
  int visited = 0, n_rem = np;
  bool stop = false;
  for (int round = 0; !stop && n_rem > 0; ++round) {
    // 1. the next pages by score, in rank order (the keys wait in LDS
    //    while a round is walked)
    if (round > 0) {
#pragma unroll
      for (int e = 0; e < E; ++e) key[e] = s_keys[e * NT + tid];
    }
    const int n_pick = min(round == 0 ? kPsaFirst : kPsaRound, n_rem);
    const unsigned long long pick = block_select_top<E, NWV>(key, remm, n_rem, n_pick, sm);
    remm &= ~pick;
    n_rem -= n_pick;
    {
      if (round == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) s_keys[e * NT + tid] = key[e];
      }
      int rk[E];
      ordered_ranks<E, NWV>(pick, rk, sm.rank, sm.scan);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((pick >> e) & 1ull)
          s_key[rk[e]] = ((unsigned long long)key[e] << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)(e * NT + tid));
    }
    __syncthreads();
    if (tid < n_pick) {
      const unsigned long long mine = s_key[tid];
      const int page = (int)(0xFFFFFFFFu - (uint32_t)(mine & 0xFFFFFFFFull));
      const int slot = ptrow[page];   // in flight during the ranking loop
      int r = 0;
#pragma unroll 8
      for (int x = 0; x < n_pick; ++x) r += s_key[x] > mine ? 1 : 0;   // keys are distinct
      s_page[r] = page;
      s_slot[r] = slot;
    }
    __syncthreads();

    // 2. walk the round NWV pages at a time
    for (int cs = 0; cs < n_pick; cs += NWV) {
      const int pos = cs + wave;
      st.reset();
      float pm[G], pl[G];
      if (pos < n_pick) {
        const int page = s_page[pos], slot = s_slot[pos];
        if (slot >= 0 && slot < num_slots) {
          for (int tin = 0; tin < TPP; ++tin) {
            const int tok0 = page * P + tin * 16;
            const int nvalid = min(16, L - tok0);
            if (nvalid <= 0) break;
            uint32_t kd[4][DW], vd[4][DW];
            const size_t off = (size_t)slot * slot_stride + head_off + (size_t)tin * 16 * D;
            A::load_tile(k + off, lane, kd);
            A::load_tile(v + off, lane, vd);
            st.tile(kd, vd, nvalid, false, tok0, L, 0, 0, c);
          }
        }
      }
      st.finish(pm, pl, c);
      if (lane < 16) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc) ch_o[wave][hh][lane * CPL + cc] = st.o[hh][cc];
      }
      if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          ch_ml[wave][hh][0] = (pm[hh] == kNegInf) ? kNegInf : pm[hh] * scale;
          ch_ml[wave][hh][1] = pl[hh];
        }
      }
      __syncthreads();
      // stop test in rank order: lane w of row 0 of wave 0 stands for rank
      // cs + w.  Block masses are summed over the group's heads, kept as
      // logs; prefix sums run in the linear domain relative to the largest.
      if (wave == 0) {
        const int n_here = min(NWV, n_pick - cs);
        const bool here = lane < n_here;
        float mh[G];
        float ln_as = kNegInf;
        {
          float mx = kNegInf;
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            mh[hh] = here ? ch_ml[lane & (NWV - 1)][hh][0] : kNegInf;
            mx = fmaxf(mx, mh[hh]);
          }
          if (mx != kNegInf) {
            float sum = 0.0f;
#pragma unroll
            for (int hh = 0; hh < G; ++hh)
              if (mh[hh] != kNegInf) sum = fmaf(ch_ml[lane & (NWV - 1)][hh][1], __expf(mh[hh] - mx), sum);
            ln_as = sum > 0.0f ? mx + __logf(sum) : kNegInf;
          }
        }
        const float acc0 = s_lnacc;
        const float big = fmaxf(acc0, row_max(ln_as));
        float lnacc = kNegInf;
        {
          const float x = (ln_as == kNegInf) ? 0.0f : __expf(ln_as - big);
          const float pre = row_scan_sum(x) + ((acc0 == kNegInf) ? 0.0f : __expf(acc0 - big));
          if (big != kNegInf && pre > 0.0f) lnacc = big + __logf(pre);
        }
        const float lnmin = fminf(s_lnmin, row_scan_min(here ? ln_as : __builtin_huge_valf()));
        const int left = s_left - (lane + 1);
        bool pass;
        if (never_stop) pass = false;
        else if (always_stop) pass = true;
        else if (stop_mode == 0) pass = lnacc - lnmin >= ln_odds;
        else pass = (left == 0) || (lnacc - (lnmin + __logf((float)left)) >= ln_odds);
        const unsigned long long hit = __ballot(here && pass);
        const int take = hit ? (__ffsll((long long)hit)) : n_here;   // 1-based rank of the first pass
        // merge weights of the taken blocks, per head: exp(m_w - M), M the new running max
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float mo = s_accm[hh];
          const float mt = lane < take ? mh[hh] : kNegInf;
          const float M = fmaxf(mo, row_max(mt));
          if (lane < NWV) s_wt[lane][hh] = (mt == kNegInf) ? 0.0f : __expf(mt - M);
          if (lane == 0) {
            s_alpha[hh] = (mo == kNegInf) ? (M == kNegInf ? 1.0f : 0.0f) : __expf(mo - M);
            s_accm[hh] = M;
          }
        }
        if (lane == take - 1) {
          s_lnacc = lnacc;
          s_lnmin = lnmin;
          s_left = left;
          s_take = take;
          s_stop = hit ? 1 : 0;
        }
      }
      __syncthreads();
      const int take = s_take;
      if (tid < G * D) {
        const float a = s_alpha[my_h];
        acc_o *= a;
        acc_l *= a;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
          if (w < take) {
            const float wt = s_wt[w][my_h];
            acc_o = fmaf(ch_o[w][my_h][my_c], wt, acc_o);
            acc_l = fmaf(ch_ml[w][my_h][1], wt, acc_l);
          }
        }
      }
      if (tid < take) irow[visited + tid] = s_page[cs + tid];
      visited += take;
      stop = s_stop != 0;
      __syncthreads();   // ch_o / ch_ml / s_* are rewritten next
      if (stop) break;
    }
  }

  // 3. outputs
  for (int x = visited + tid; x < max_pages; x += NT) irow[x] = -1;
  if (tid == 0) counts[unit] = visited;
  if (tid < G * D) {
    const size_t row = (size_t)b * n_kv_heads * G + (size_t)h * G + my_h;
    O[row * D + my_c] = acc_l > 0.0f ? acc_o / acc_l : 0.0f;
    if (my_c == 0) {
      l[row] = acc_l;
      m[row] = acc_l > 0.0f ? s_accm[my_h] : kNegInf;
    }
  }
}

// ============================================================ host planning
struct SplitPlan {
  int tiles_per_split, n_splits, TPP;
};

// A split is one workgroup: 4 waves of TW tiles each, all in flight at once
// (TW = kTilesPerWaveMfma for the matrix-core kernel, 8+ heads per KV head
// with bf16 KV), so the grid grows with the selection: counts live on the
// device, so it is sized for ids_stride entries, and splits past a row's
// count exit at once.
inline SplitPlan plan_splits(const dsa_kv* kv, int ids_stride, bool mfma) {
  SplitPlan p;
  p.TPP = kv->page_size / 16;
  const long long tiles_max = (long long)ids_stride * p.TPP;
  p.tiles_per_split = kWgWaves * (mfma ? kTilesPerWaveMfma : kTilesPerWave);
  p.n_splits = (int)((tiles_max + p.tiles_per_split - 1) / p.tiles_per_split);
  if (p.n_splits < 1) p.n_splits = 1;
  return p;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace for any plan of this shape: the smallest split gives the most
// splits.
inline size_t max_splits_of(const dsa_kv* kv, int ids_stride) {
  constexpr int kMinTiles = kWgWaves * (kTilesPerWave < kTilesPerWaveMfma ? kTilesPerWave : kTilesPerWaveMfma);
  const size_t tiles_max = (size_t)ids_stride * (kv->page_size / 16);
  return (tiles_max + kMinTiles - 1) / kMinTiles;
}

inline size_t partial_bytes(const dsa_kv* kv, int G, int ids_stride) {
  const size_t units = (size_t)kv->batch * kv->n_kv_heads;
  const size_t ms = max_splits_of(kv, ids_stride);
  return align256(units * ms * G * kv->head_dim * sizeof(float)) + align256(units * ms * G * 2 * sizeof(float));
}

template <typename T, int D, int G>
static int launch_attn_g(const void* q, const dsa_kv* kv, const int32_t* ids, const int32_t* counts,
                         int ids_stride, uint64_t smask, int sink, int local, float scale, float* O, float* l,
                         float* m, void* ws, int fold, const int32_t* skip_ids, const int32_t* skip_counts,
                         const SelectArgs& sel, hipStream_t st) {
  const SplitPlan p = plan_splits(kv, ids_stride, sizeof(T) == 2 && G >= 8);
  const size_t units = (size_t)kv->batch * kv->n_kv_heads;
  float* part_o = (float*)ws;
  float* part_ml = (float*)((char*)ws + align256(units * max_splits_of(kv, ids_stride) * G * D * sizeof(float)));
  const float c = scale * kLog2e;
  dim3 grid(p.n_splits, kv->n_kv_heads, kv->batch);
  const size_t dyn = skip_ids ? (size_t)((kv->max_pages + 31) / 32) * sizeof(uint32_t) : 0;
#define DSA_PARTIAL(KERNEL, TT, ...)                                                                             \
  hipLaunchKernelGGL((KERNEL<__VA_ARGS__>), grid, dim3(256), dyn, st, (const TT*)q, (const TT*)kv->k,           \
                     (const TT*)kv->v, kv->page_table, kv->seq_lens, ids, counts, ids_stride, kv->n_kv_heads,   \
                     kv->page_size, kv->max_pages, kv->num_slots, (unsigned long long)smask, sink, local, scale, \
                     c, p.tiles_per_split, p.n_splits, skip_ids, skip_counts, sel, part_o, part_ml)
  if constexpr (sizeof(T) == 2 && G >= 8) {
    if (sel.e) return DSA_ERR_UNSUPPORTED;
    if (skip_ids) DSA_PARTIAL(attn_partial_mfma_kernel, uint16_t, D, G, true);
    else DSA_PARTIAL(attn_partial_mfma_kernel, uint16_t, D, G, false);
  } else {
    if (sel.e == 8) DSA_PARTIAL(attn_partial_kernel, T, T, D, G, false, 8);
    else if (sel.e == 16) DSA_PARTIAL(attn_partial_kernel, T, T, D, G, false, 16);
    else if (sel.e) return DSA_ERR_UNSUPPORTED;
    else if (skip_ids) DSA_PARTIAL(attn_partial_kernel, T, T, D, G, true, 0);
    else DSA_PARTIAL(attn_partial_kernel, T, T, D, G, false, 0);
  }
#undef DSA_PARTIAL
  int rc = launch_status();
  if (rc) return rc;
  hipLaunchKernelGGL((attn_combine_kernel<D>), dim3(kv->n_kv_heads * G, kv->batch), dim3(256), 0, st, part_o,
                     part_ml, sel.e ? sel.counts_out : counts, ids_stride, kv->n_kv_heads, G, p.TPP, p.tiles_per_split, p.n_splits, fold, O,
                     l, m);
  return launch_status();
}

template <typename T, int D>
static int launch_attn_d(const void* q, int G, const dsa_kv* kv, const int32_t* ids, const int32_t* counts,
                         int ids_stride, uint64_t smask, int sink, int local, float scale, float* O, float* l,
                         float* m, void* ws, int fold, const int32_t* skip_ids, const int32_t* skip_counts,
                         const SelectArgs& sel, hipStream_t st) {
  switch (G) {
    case 1: return launch_attn_g<T, D, 1>(q, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, fold, skip_ids, skip_counts, sel, st);
    case 2: return launch_attn_g<T, D, 2>(q, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, fold, skip_ids, skip_counts, sel, st);
    case 4: return launch_attn_g<T, D, 4>(q, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, fold, skip_ids, skip_counts, sel, st);
    case 8: return launch_attn_g<T, D, 8>(q, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, fold, skip_ids, skip_counts, sel, st);
    case 16: return launch_attn_g<T, D, 16>(q, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, fold, skip_ids, skip_counts, sel, st);
  }
  return DSA_ERR_UNSUPPORTED;
}

static int launch_attn(const void* q, int G, const dsa_kv* kv, const int32_t* ids, const int32_t* counts,
                       int ids_stride, uint64_t smask, int sink, int local, float scale, float* O, float* l,
                       float* m, void* ws, int fold, const int32_t* skip_ids, const int32_t* skip_counts,
                       const SelectArgs& sel, hipStream_t st) {
  const bool bf = kv->dtype == DSA_BF16;
  if (kv->head_dim == 128)
    return bf ? launch_attn_d<uint16_t, 128>(q, G, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, fold, skip_ids, skip_counts, sel, st)
              : launch_attn_d<float, 128>(q, G, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, fold, skip_ids, skip_counts, sel, st);
  return bf ? launch_attn_d<uint16_t, 64>(q, G, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, fold, skip_ids, skip_counts, sel, st)
            : launch_attn_d<float, 64>(q, G, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, fold, skip_ids, skip_counts, sel, st);
}

static int check_attn_common(const void* q, int n_q_heads, const dsa_kv* kv, float scale, int* G) {
  int rc = check_kv(kv, true);
  if (rc) return rc;
  if (n_q_heads < 1 || n_q_heads % kv->n_kv_heads) return DSA_ERR_SHAPE;
  *G = n_q_heads / kv->n_kv_heads;
  if (!pow2_group(*G)) return DSA_ERR_UNSUPPORTED;
  if (!(scale > 0.0f) || !(scale < __builtin_huge_valf())) return DSA_ERR_SHAPE;
  if (kv->batch > 0) {
    if (!q) return DSA_ERR_NULL;
    if (!aligned16(q)) return DSA_ERR_ALIGN;
  }
  return DSA_OK;
}

static int max_lds_per_block() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) v = 65536;
    cached[dev] = v;
  }
  return cached[dev];
}

template <typename T, int D, int G>
static int launch_psa_g(const void* q, const dsa_kv* kv, const float* scores, float thr, int stop_mode, float scale,
                        int32_t* ids, int32_t* counts, float* O, float* l, float* m, hipStream_t st) {
  const int never_stop = thr >= 1.0f;
  const int always_stop = thr <= 0.0f;
  const float ln_odds = (never_stop || always_stop) ? 0.0f : (float)log((double)thr / (1.0 - (double)thr));
  const float c = scale * kLog2e;
  constexpr int NT = psa_waves<T, G>() * 64;
  constexpr int EMAX = kPsaMaxPages / NT;
#define DSA_PSA(E_)                                                                                                \
  hipLaunchKernelGGL((psa_kernel<T, D, G, E_>), dim3(kv->n_kv_heads, kv->batch), dim3(NT), 0, st, (const T*)q,     \
                     (const T*)kv->k, (const T*)kv->v, kv->page_table, kv->seq_lens, scores, kv->n_kv_heads,       \
                     kv->page_size, kv->max_pages, kv->num_slots, stop_mode, never_stop, always_stop, ln_odds,     \
                     scale, c, ids, counts, O, l, m)
  if (kv->max_pages <= NT * (EMAX / 4)) DSA_PSA(EMAX / 4);
  else if (kv->max_pages <= NT * (EMAX / 2)) DSA_PSA(EMAX / 2);
  else DSA_PSA(EMAX);
#undef DSA_PSA
  return launch_status();
}

template <typename T, int D>
static int launch_psa_d(const void* q, int G, const dsa_kv* kv, const float* scores, float thr, int stop_mode,
                        float scale, int32_t* ids, int32_t* counts, float* O, float* l, float* m, hipStream_t st) {
  switch (G) {
    case 1: return launch_psa_g<T, D, 1>(q, kv, scores, thr, stop_mode, scale, ids, counts, O, l, m, st);
    case 2: return launch_psa_g<T, D, 2>(q, kv, scores, thr, stop_mode, scale, ids, counts, O, l, m, st);
    case 4: return launch_psa_g<T, D, 4>(q, kv, scores, thr, stop_mode, scale, ids, counts, O, l, m, st);
  }
  return DSA_ERR_UNSUPPORTED;
}

}  // namespace dsa

using namespace dsa;

// ============================================================ C ABI
extern "C" size_t dsa_workspace_bytes(int32_t op, const dsa_kv* kv, int32_t n_q_heads, int32_t ids_stride) {
  if (check_kv(kv, false) != DSA_OK || n_q_heads < 1 || n_q_heads % kv->n_kv_heads || ids_stride < 1) return 0;
  const int G = n_q_heads / kv->n_kv_heads;
  if (!pow2_group(G)) return 0;
  const size_t part = partial_bytes(kv, G, ids_stride);
  if (op == DSA_OP_SPARSE_DECODE_ATTN) return part;
  if (op == DSA_OP_ATTN_REPAIR) return part;
  return 0;
}

// Validation shared by dsa_sparse_decode_attn and its no-allocation variant;
// on success *need holds the scratch bytes of the call (0 when nothing runs).
static int check_sparse_decode_attn(const void* q, int32_t n_q_heads, const dsa_kv* kv, const int32_t* ids,
                                    const int32_t* counts, int32_t ids_stride, const dsa_stream_cfg* stream_cfg,
                                    float scale, const float* O, const float* l, const float* m, int* G,
                                    uint64_t* smask, size_t* need) {
  *need = 0;
  int rc = check_attn_common(q, n_q_heads, kv, scale, G);
  if (rc) return rc;
  if (ids_stride < 1) return DSA_ERR_SHAPE;
  if ((rc = streaming_mask(stream_cfg, kv->n_kv_heads, smask))) return rc;
  if (kv->batch == 0) return DSA_OK;
  if (!ids || !counts || !O || !l || !m) return DSA_ERR_NULL;
  *need = dsa_workspace_bytes(DSA_OP_SPARSE_DECODE_ATTN, kv, n_q_heads, ids_stride);
  return DSA_OK;
}

extern "C" int dsa_sparse_decode_attn(const void* q, int32_t n_q_heads, const dsa_kv* kv, const int32_t* ids,
                                      const int32_t* counts, int32_t ids_stride, const dsa_stream_cfg* stream_cfg,
                                      float scale, float* O, float* l, float* m, void* ws, size_t ws_bytes,
                                      void* stream) {
  int G = 0;
  uint64_t smask = 0;
  size_t need = 0;
  int rc = check_sparse_decode_attn(q, n_q_heads, kv, ids, counts, ids_stride, stream_cfg, scale, O, l, m, &G,
                                    &smask, &need);
  if (rc || kv->batch == 0) return rc;
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  const int sink = stream_cfg ? stream_cfg->sink : 0, local = stream_cfg ? stream_cfg->local : 0;
  return launch_attn(q, G, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, 0, nullptr,
                     nullptr, SelectArgs{}, (hipStream_t)stream);
}

// ------------------------------------------------------------ no-allocation variant
// The split partials of dsa_sparse_decode_attn_noalloc live in this
// file-scope device array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy, at its own address, until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: kernels get the address that hipGetSymbolAddress returns for the
// device, looked up once per device and kept in scratch_dev.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex scratch_mu;
static void* scratch_dev[kMaxDevices];

// Device address of `scratch` on the device that owns `stream`, looked up
// with that device current the first time (the caller's current device is
// restored afterwards).
static int scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return DSA_ERR_LAUNCH;
  hipDevice_t dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return DSA_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return DSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return DSA_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return DSA_ERR_LAUNCH;
    if (e != hipSuccess || !p) return DSA_ERR_LAUNCH;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return DSA_OK;
}

extern "C" int dsa_sparse_decode_attn_noalloc(const void* q, int32_t n_q_heads, const dsa_kv* kv,
                                              const int32_t* ids, const int32_t* counts, int32_t ids_stride,
                                              const dsa_stream_cfg* stream_cfg, float scale, float* O, float* l,
                                              float* m, void* stream) {
  int G = 0;
  uint64_t smask = 0;
  size_t need = 0;
  int rc = check_sparse_decode_attn(q, n_q_heads, kv, ids, counts, ids_stride, stream_cfg, scale, O, l, m, &G,
                                    &smask, &need);
  if (rc || kv->batch == 0) return rc;
  if (need > (size_t)DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_SCRATCH;
  void* ws = nullptr;
  if ((rc = scratch_address((hipStream_t)stream, &ws))) return rc;
  const int sink = stream_cfg ? stream_cfg->sink : 0, local = stream_cfg ? stream_cfg->local : 0;
  return launch_attn(q, G, kv, ids, counts, ids_stride, smask, sink, local, scale, O, l, m, ws, 0, nullptr,
                     nullptr, SelectArgs{}, (hipStream_t)stream);
}

extern "C" int dsa_sparse_decode_attn_topk(const void* q, int32_t n_q_heads, const dsa_kv* kv, const float* scores,
                                           int32_t k, const dsa_stream_cfg* stream_cfg, float scale, int32_t* ids,
                                           int32_t* counts, float* O, float* l, float* m, void* ws, size_t ws_bytes,
                                           void* stream) {
  int G = 0;
  int rc = check_attn_common(q, n_q_heads, kv, scale, &G);
  if (rc) return rc;
  if (k < 1) return DSA_ERR_SHAPE;
  uint64_t smask;
  if ((rc = streaming_mask(stream_cfg, kv->n_kv_heads, &smask))) return rc;
  if (smask) {
    // the sink/local page list of a streaming head must fit in k
    long long worst = (stream_cfg->sink + (long long)kv->page_size - 1) / kv->page_size +
                      (stream_cfg->local + (long long)kv->page_size - 1) / kv->page_size + 1;
    if (worst > kv->max_pages) worst = kv->max_pages;
    if (worst > k) return DSA_ERR_SHAPE;
  }
  if (kv->batch == 0) return DSA_OK;
  if (!scores || !ids || !counts || !O || !l || !m) return DSA_ERR_NULL;
  const size_t need = dsa_workspace_bytes(DSA_OP_SPARSE_DECODE_ATTN, kv, n_q_heads, k);
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  const int sink = stream_cfg ? stream_cfg->sink : 0, local = stream_cfg ? stream_cfg->local : 0;
  hipStream_t st = (hipStream_t)stream;
  const int e = kv->max_pages <= 2048 ? 8 : (kv->max_pages <= 4096 ? 16 : 0);
  if (G <= 4 && e) {
    const SelectArgs sel{scores, k, ids, counts, e};
    return launch_attn(q, G, kv, nullptr, nullptr, k, smask, sink, local, scale, O, l, m, ws, 0, nullptr, nullptr,
                       sel, st);
  }
  // large rows or large groups: the two calls in sequence
  if ((rc = dsa_page_select_topk(scores, kv->batch, kv->n_kv_heads, kv->max_pages, kv->seq_lens, kv->page_size, k,
                                 stream_cfg, ids, counts, stream)))
    return rc;
  return launch_attn(q, G, kv, ids, counts, k, smask, sink, local, scale, O, l, m, ws, 0, nullptr, nullptr,
                     SelectArgs{}, st);
}

extern "C" int dsa_attn_repair(const void* q, int32_t n_q_heads, const dsa_kv* kv, const int32_t* a_ids,
                               const int32_t* a_counts, const int32_t* p_ids, const int32_t* p_counts,
                               int32_t ids_stride, float scale, float* O, float* l, float* m, void* ws,
                               size_t ws_bytes, void* stream) {
  int G = 0;
  int rc = check_attn_common(q, n_q_heads, kv, scale, &G);
  if (rc) return rc;
  if (ids_stride < 1) return DSA_ERR_SHAPE;
  if (kv->batch == 0) return DSA_OK;
  if (!a_ids || !a_counts || !O || !l || !m) return DSA_ERR_NULL;
  if (!p_ids != !p_counts) return DSA_ERR_NULL;
  const size_t need = dsa_workspace_bytes(DSA_OP_ATTN_REPAIR, kv, n_q_heads, ids_stride);
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  if (p_ids) {
    const size_t lds = (size_t)((kv->max_pages + 31) / 32) * sizeof(uint32_t);
    if ((int)lds + 52 * 1024 > max_lds_per_block()) return DSA_ERR_UNSUPPORTED;
  }
  // without P the a_ids are M already (usually a short prefix of the row):
  // the plain split-KV path, folded; splits past the count exit at once
  return launch_attn(q, G, kv, a_ids, a_counts, ids_stride, 0, 0, 0, scale, O, l, m, ws, 1, p_ids, p_counts,
                     SelectArgs{}, (hipStream_t)stream);
}

extern "C" int dsa_page_select_progressive(const void* q, int32_t n_q_heads, const dsa_kv* kv, const float* scores,
                                           float threshold, int32_t stop_mode, float scale, int32_t* ids,
                                           int32_t* counts, float* O, float* l, float* m, void* stream) {
  int G = 0;
  int rc = check_attn_common(q, n_q_heads, kv, scale, &G);
  if (rc) return rc;
  if (stop_mode != 0 && stop_mode != 1) return DSA_ERR_SHAPE;
  if (threshold != threshold) return DSA_ERR_SHAPE;
  if (kv->max_pages > kPsaMaxPages) return DSA_ERR_UNSUPPORTED;
  if (kv->batch == 0) return DSA_OK;
  if (!scores || !ids || !counts || !O || !l || !m) return DSA_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  const bool bf = kv->dtype == DSA_BF16;
  if (kv->head_dim == 128)
    return bf ? launch_psa_d<uint16_t, 128>(q, G, kv, scores, threshold, stop_mode, scale, ids, counts, O, l, m, st)
              : launch_psa_d<float, 128>(q, G, kv, scores, threshold, stop_mode, scale, ids, counts, O, l, m, st);
  return bf ? launch_psa_d<uint16_t, 64>(q, G, kv, scores, threshold, stop_mode, scale, ids, counts, O, l, m, st)
            : launch_psa_d<float, 64>(q, G, kv, scores, threshold, stop_mode, scale, ids, counts, O, l, m, st);
}
