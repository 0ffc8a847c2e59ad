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
#include "dsa_score.hpp"
#include "dsa_select.hpp"

#include <mutex>

#ifndef DSA_TILES_PER_WAVE
#define DSA_TILES_PER_WAVE 2  // 16-token K/V tiles per wave of the VALU partial kernel (all in flight at once)
#endif
#ifndef DSA_TILES_PER_WAVE_WIDE
#define DSA_TILES_PER_WAVE_WIDE 3  // the same when the grid would hold more splits than the GPU has CUs
#endif
#ifndef DSA_TILES_PER_WAVE_MFMA
#define DSA_TILES_PER_WAVE_MFMA 4  // the same for the matrix-core partial kernel
#endif

namespace dsa {

constexpr int kWgWaves = 4;
constexpr int kTilesPerWave = DSA_TILES_PER_WAVE;
constexpr int kTilesPerWaveWide = DSA_TILES_PER_WAVE_WIDE;
static_assert(kTilesPerWaveWide >= kTilesPerWave, "the narrow split is the smallest");
constexpr int kTilesPerWaveMfma = DSA_TILES_PER_WAVE_MFMA;
#ifndef DSA_TILES_PER_WAVE_REPAIR
#define DSA_TILES_PER_WAVE_REPAIR 1  // the same for the repair over a compacted M (both kernels): M is short
#endif
constexpr int kTilesPerWaveRepair = DSA_TILES_PER_WAVE_REPAIR;

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
// The workgroup (split, h, b) as a device function (kernels that run these
// splits beside other work call it too).
template <typename T, int D, int G, bool FILTER, int SEL_E, int TW>
__device__ __forceinline__ void attn_partial_body(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ counts, int ids_stride, int n_kv_heads, int P,
    int max_pages, int num_slots, unsigned long long streaming, int sink, int local, float scale, float c,
    int tiles_per_split, int n_splits, const int32_t* __restrict__ skip_ids,
    const int32_t* __restrict__ skip_counts, const SelectArgs& sel, float* __restrict__ part_o,
    float* __restrict__ part_ml, int split, int h, int b) {
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

template <typename T, int D, int G, bool FILTER, int SEL_E, int TW>
__global__ __launch_bounds__(256) void attn_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ counts, int ids_stride, int n_kv_heads, int P,
    int max_pages, int num_slots, unsigned long long streaming, int sink, int local, float scale, float c,
    int tiles_per_split, int n_splits, const int32_t* __restrict__ skip_ids,
    const int32_t* __restrict__ skip_counts, SelectArgs sel, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  attn_partial_body<T, D, G, FILTER, SEL_E, TW>(q, k, v, page_table, seq_lens, ids, counts, ids_stride, n_kv_heads,
                                                P, max_pages, num_slots, streaming, sink, local, scale, c,
                                                tiles_per_split, n_splits, skip_ids, skip_counts, sel, part_o,
                                                part_ml, (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z);
}

// ============================================================ split-KV partial, matrix cores
// Same split and output as attn_partial_kernel, for bf16 KV with 8 or 16 q
// heads per KV head: each wave runs the MFMA tile of dsa_attn_mfma.hpp over
// its tiles, and the 4 wave states meet in LDS.
// The workgroup (split, h, b) as a device function, so that other kernels
// can run these splits beside their own workgroups.
template <int D, int G, bool FILTER, int TW>
__device__ __forceinline__ void attn_partial_mfma_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ counts, int ids_stride, int n_kv_heads, int P,
    int max_pages, int num_slots, unsigned long long streaming, int sink, int local, float scale, float c,
    int tiles_per_split, int n_splits, const int32_t* __restrict__ skip_ids,
    const int32_t* __restrict__ skip_counts, float* __restrict__ part_o, float* __restrict__ part_ml, int split,
    int h, int b) {
  using M = MfmaWave<D, G>;
  constexpr int NK = M::NK, NB = M::NB;
  constexpr int OS = D + 4;   // LDS row stride of the merge buffer (floats)
  // a wave's V staging (during its tiles) and its merge rows (after them)
  // share one LDS region: the wave writes its rows only once its own tiles
  // are done, and the merge reads them after the barrier
  constexpr int kVFloats = (M::LDS_ELEMS + 1) / 2, kOFloats = G * OS;
  constexpr int kWaveFloats = kVFloats > kOFloats ? kVFloats : kOFloats;
  __shared__ __align__(16) float lds_wave[kWgWaves][kWaveFloats];
  __shared__ float lds_ml[kWgWaves][G][2];
  auto lds_o = [&](int w, int hh) { return &lds_wave[w][hh * OS]; };

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
  st.init(q + ((size_t)b * n_kv_heads * G + (size_t)h * G) * D, reinterpret_cast<uint16_t*>(lds_wave[wave]));

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
      *reinterpret_cast<float4*>(lds_o(wave, st.h) + 16 * n + 4 * st.g) =
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
      acc = fmaf(lds_o(w, hh)[cc], wt, acc);
      ls = fmaf(lds_ml[w][hh][1], wt, ls);
    }
    part_o[(pbase + hh) * D + cc] = acc;
    if (cc == 0) {
      part_ml[(pbase + hh) * 2 + 0] = (mm == kNegInf) ? kNegInf : mm * scale;  // natural-log units
      part_ml[(pbase + hh) * 2 + 1] = ls;
    }
  }
}

template <int D, int G, bool FILTER, int TW>
__global__ __launch_bounds__(256) void attn_partial_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ ids, const int32_t* __restrict__ counts, int ids_stride, int n_kv_heads, int P,
    int max_pages, int num_slots, unsigned long long streaming, int sink, int local, float scale, float c,
    int tiles_per_split, int n_splits, const int32_t* __restrict__ skip_ids,
    const int32_t* __restrict__ skip_counts, SelectArgs, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  attn_partial_mfma_body<D, G, FILTER, TW>(q, k, v, page_table, seq_lens, ids, counts, ids_stride, n_kv_heads, P,
                                           max_pages, num_slots, streaming, sink, local, scale, c, tiles_per_split,
                                           n_splits, skip_ids, skip_counts, part_o, part_ml, (int)blockIdx.x,
                                           (int)blockIdx.y, (int)blockIdx.z);
}

// ============================================================ combine
// One workgroup per (sequence, q head).  The active splits are merged with
// the online-softmax rule in chunks of 64: every thread first issues the
// loads of all the O values it needs from the chunk (thread (sub, c) takes
// channel c of splits sub, sub + SPT, ...), wave 0 loads the chunk's
// (m, l) pairs, one per lane, and turns them into merge weights against the
// running maximum (wave reductions, no barrier), and after one barrier every
// thread folds its values.  So a chunk costs one memory round trip, and
// rows of up to 64 splits exactly one.  (Chunks of 128 measured slower on
// the whole: a round trip fewer for rows of 65-128 splits, but twice the
// loads per thread for every row.)
// For repair the caller's (O, l, m) is one more term.  Writes normalised O.
template <int D>
__device__ __forceinline__ void attn_combine_body(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, const int32_t* __restrict__ counts,
    int ids_stride, int n_kv_heads, int G, int TPP, int tiles_per_split, int n_splits, int fold,
    float* __restrict__ O, float* __restrict__ l, float* __restrict__ m, int hq, int b) {
  constexpr int SPT = 256 / D;   // split lanes per channel
  constexpr int CH = 64;         // splits per chunk
  constexpr int PER = CH / SPT;  // O values per thread and chunk
  __shared__ float s_w[CH];
  __shared__ float s_acc[SPT][D];
  __shared__ float s_alpha, s_M, s_L;
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

template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, const int32_t* __restrict__ counts,
    int ids_stride, int n_kv_heads, int G, int TPP, int tiles_per_split, int n_splits, int fold,
    float* __restrict__ O, float* __restrict__ l, float* __restrict__ m) {
  attn_combine_body<D>(part_o, part_ml, counts, ids_stride, n_kv_heads, G, TPP, tiles_per_split, n_splits, fold, O,
                       l, m, (int)blockIdx.x, (int)blockIdx.y);
}

// ============================================================ PSA progressive
// One workgroup of NWV waves per (sequence, KV head).  Pages are taken in
// rounds: the first round picks the 64 highest-ranked pages, each later
// round the next 256 (rank: score descending, lower index first on equal
// scores).  Rank order is the order of the 64-bit value
// (score key << 32 | ~index), so the pages still in play are exactly those
// whose value lies below that of the last page taken: a round keeps no
// per-page state and re-reads the score row.
//
// A round's pick: when at most kPsaCand pages are in play they all become
// candidates; otherwise radix passes over the pages in play (min / max,
// a 2048-bucket LDS histogram, and a bucket search that every wave does for
// itself from the histogram) narrow the range around the n_pick-th value
// until the pages above the cut bucket plus those in it number at most
// kPsaCand.  The candidates are ranked by counting, and the first n_pick
// ranks are the round's pages in rank order.  The first pass maps the
// score values linearly onto the buckets, later ones shift the key; once
// the keys in play are all equal the passes run on the index.
//
// The walk attends to NWV pages at a time -- wave w to the page at rank
// cs + w -- and every wave then evaluates the stop test of the group on the
// same values (prefix scans over NWV lanes: running log-sum of the block
// masses and running minimum), so the group needs one barrier.  The visited
// blocks are folded into the output with the online-softmax merge, in rank
// order.
constexpr int kPsaMaxPages = 65536;
constexpr int kPsaFirst = 64;     // pages of the first round
constexpr int kPsaRound = 256;    // pages of each later round
constexpr int kPsaCand = 512;     // most candidates ranked directly
constexpr int kPsaRegKeys = 16;   // score keys a thread holds at once

// 16 waves where a wave's tile state fits 128 registers, else 8
template <typename T, int G>
constexpr int psa_waves() { return (G == 1 && sizeof(T) == 2) ? 16 : 8; }

__device__ __forceinline__ float log_add(float a, float b) {
  const float mx = fmaxf(a, b), mn = fminf(a, b);
  if (mn == kNegInf) return mx;
  return mx + log1pf(expf(mn - mx));
}

__device__ __forceinline__ float readlane_f(float x, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), src));
}

__device__ __forceinline__ unsigned long long page_order(uint32_t key, int idx) {
  return ((unsigned long long)key << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)idx);
}

template <int NW>
struct PsaSmem {
  unsigned hist[2][kHistWords];      // alternate passes use alternate buffers
  uint32_t mm[2][2 * NW];
  __align__(16) unsigned long long cand[kPsaCand];
  int cand_slot[kPsaCand];
  int n_cand[2];                     // candidate counters of alternate rounds
  unsigned long long kbound;         // order value of the round's last page
  int page[kPsaRound], slot[kPsaRound];   // the round's pages in rank order
};

// This thread's pages are idx = e * NT + tid, e < E.  Rows of at most
// 8 * NT pages hold their keys and page-table entries in registers for a
// whole round; longer rows stream the keys from the score row in chunks of
// kPsaRegKeys per pass.
template <int E, int NT>
struct PsaKeys {
  static constexpr bool kResident = E <= 8;
  static constexpr int R = kResident ? E : kPsaRegKeys;
  uint32_t key[R];
  int slot[kResident ? R : 1];
  const float* srow;
  const int32_t* ptrow;
  int max_pages, np, tid;

  // every load is issued before the first use (addresses clamped into the row)
  __device__ __forceinline__ void load(int e0) {
    float v[R];
    int t = tid;
    // streamed keys are re-read by every pass: the empty asm hides that the
    // addresses repeat, so the compiler does not keep them all live instead
    if constexpr (!kResident) asm volatile("" : "+v"(t));
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = min((e0 + r) * NT + t, max_pages - 1);
      v[r] = srow[c];
      if constexpr (kResident) slot[r] = ptrow[c];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) key[r] = order_key(v[r]);
  }
  __device__ __forceinline__ void round_start() {
    if constexpr (kResident) load(0);
  }
  // f(e0) once per chunk of R element slots e0 .. e0 + R - 1 of this
  // thread, with their keys (and, when resident, page-table entries) in
  // key[] / slot[]; e0 is the same across the workgroup
  template <class F>
  __device__ __forceinline__ void each_chunk(F&& f) {
    if constexpr (kResident) {
      f(0);
    } else {
      for (int e0 = 0; e0 < E && e0 * NT < np; e0 += R) {
        load(e0);
        f(e0);
      }
    }
  }
  // f(key, idx, slot, valid) for every element slot of this thread, in
  // step across the wave (valid: idx < np; slot only when resident)
  template <class F>
  __device__ __forceinline__ void each(F&& f) {
    if constexpr (kResident) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int idx = r * NT + tid;
        f(key[r], idx, slot[r], idx < np);
      }
    } else {
      for (int e0 = 0; e0 < E && e0 * NT < np; e0 += R) {
        load(e0);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int idx = (e0 + r) * NT + tid;
          f(key[r], idx, 0, idx < np);
        }
      }
    }
  }
};

// The n_pick highest-ranked of the n_act pages in play in round `round`
// (all valid pages in round 0, FIRST; later, those whose order value is below kb),
// in rank order into sm.page / sm.slot; kb becomes the order value of the
// last one.  Candidates are ranked by counting.  Rounds
// alternate candidate counters: a round clears the one of the round after
// it, which every thread read before the ranking barrier of the round before.
template <int E, int NW, bool FIRST>
__device__ __forceinline__ void psa_pick(PsaKeys<E, NW * 64>& ks, int round, unsigned long long& kb, int n_act,
                                         int n_pick, PsaSmem<NW>& sm) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x, lane = tid & 63;
  int* n_cand_p = &sm.n_cand[round & 1];
  if (tid == 0) sm.n_cand[(round + 1) & 1] = 0;
  const unsigned long long below = (1ull << lane) - 1ull;
  const unsigned long long kb_in = kb;
  auto live = [&](uint32_t key, int idx, bool valid) {
    if constexpr (FIRST) return valid;
    else return valid & (page_order(key, idx) < kb_in);
  };
  // range in play: level 0, keys in [lo, hi] (and, after a linear pass until
  // the next min / max, in bucket pb of map pm); level 1, key t and ~index in
  // [lo, hi].  The tests below are written without branches: both levels'
  // terms are computed and the uniform level selects.
  bool lvl1 = false;
  uint32_t lo = 0u, hi = 0xFFFFFFFFu, t = 0u, pb = 0u;
  bool pend = false;
  BucketMap pm{}, map{};
  uint32_t bstar = 0u;
  bool cut = false;
  int need = n_pick;
  auto field = [&](uint32_t key, int idx) { return lvl1 ? 0xFFFFFFFFu - (uint32_t)idx : key; };
  auto in_range = [&](uint32_t key, int idx) {
    const uint32_t f = field(key, idx);
    return (f >= lo) & (f <= hi) & (!lvl1 | (key == t)) & (!pend | (pm.linear(key) == pb));
  };
  auto above = [&](uint32_t key, int idx) {
    const uint32_t f = field(key, idx);
    return lvl1 ? ((key > t) | ((key == t) & (f > hi))) : (key > hi);
  };
  auto bucket = [&](uint32_t key, int idx) {
    const uint32_t a = map.linear(key), b = map.shifted(field(key, idx));
    return map.lin ? a : b;
  };

  if (n_pick < n_act && n_act > kPsaCand) {
    bool first_hist = true;
    // at most: a linear pass, three shift passes on the key, a min / max
    // that finds the key equal, one shift pass on the index (< 2^16 apart)
    for (int pass = 0; pass < 8; ++pass) {
      unsigned* hist = sm.hist[pass & 1];
      for (int x = tid; x < kHistWords; x += NT) hist[x] = 0u;   // last read two barriers ago
      uint32_t mn = 0xFFFFFFFFu, mx = 0u;
      ks.each([&](uint32_t key, int idx, int, bool valid) {
        if (live(key, idx, valid) && in_range(key, idx)) {
          const uint32_t f = field(key, idx);
          mn = min(mn, f);
          mx = max(mx, f);
        }
      });
      block_minmax_1b<NW>(mn, mx, sm.mm[pass & 1]);   // also orders the zeroing before the atomics
      lo = mn;
      hi = mx;
      pend = false;
      if (lo == hi) {
        if (lvl1) break;   // one page left in range: the cut takes the whole range
        lvl1 = true;
        t = lo;
        lo = 0u;
        hi = 0xFFFFFFFFu;
        continue;
      }
      const uint32_t span = hi - lo;
      map.lo = lo;
      map.shift = span < (uint32_t)kBuckets ? 0 : (32 - __clz((int)span) - 11);
      map.lin = false;
      map.f0 = 0.0f;
      map.inv = 0.0f;
      if (!lvl1 && first_hist && span >= (uint32_t)kBuckets) {
        const float f0 = key_value(lo), f1 = key_value(hi);
        const float inv = (float)(kBuckets - 1) / (f1 - f0);
        if (__builtin_isfinite(f0) && __builtin_isfinite(f1) && __builtin_isfinite(f1 - f0) && f1 > f0 &&
            __builtin_isfinite(inv) && inv > 0.0f) {
          map.lin = true;
          map.f0 = f0;
          map.inv = inv;
        }
      }
      first_hist = false;
      ks.each([&](uint32_t key, int idx, int, bool valid) {
        if (live(key, idx, valid) && in_range(key, idx)) atomicAdd(&hist[hist_at(bucket(key, idx))], 1u);
      });
      __syncthreads();
      // every wave finds the cut bucket from the histogram itself
      const BucketCut bc = bucket_search(hist, need);
      bstar = bc.b;
      const int above_b = bc.above, nb = bc.n;
      if ((n_pick - need) + above_b + nb <= kPsaCand) {
        cut = true;
        break;
      }
      need -= above_b;
      if (map.lin) {
        pend = true;
        pm = map;
        pb = bstar;
      } else {
        const uint32_t l2 = lo + (bstar << map.shift);
        const unsigned long long h2 = (unsigned long long)l2 + (1ull << map.shift) - 1ull;
        lo = l2;
        hi = (uint32_t)min((unsigned long long)hi, h2);
      }
    }
  }
  // candidates: every page in play above the range, and those of the range
  // at or above the cut; a wave reserves room for a chunk's hits with one atomic
  ks.each_chunk([&](int e0) {
    constexpr int R = PsaKeys<E, NT>::R;
    bool hit[R];
    unsigned long long bm[R];
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = (e0 + r) * NT + tid;
      const uint32_t key = ks.key[r];
      hit[r] = live(key, idx, idx < ks.np) &&
               (above(key, idx) || (in_range(key, idx) && (!cut || bucket(key, idx) >= bstar)));
      bm[r] = __ballot(hit[r]);
      cnt += __popcll(bm[r]);
    }
    if (cnt) {
      int base = 0;
      if (lane == 0) base = atomicAdd(n_cand_p, cnt);
      base = __builtin_amdgcn_readlane(base, 0);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int p = base + __popcll(bm[r] & below);
        if (hit[r] && p < kPsaCand) {
          sm.cand[p] = page_order(ks.key[r], (e0 + r) * NT + tid);
          sm.cand_slot[p] = PsaKeys<E, NT>::kResident ? ks.slot[PsaKeys<E, NT>::kResident ? r : 0] : 0;
        }
        base += __popcll(bm[r]);
      }
    }
  });
  __syncthreads();
  // ranks by counting: lpc lanes per candidate (a power of two, up to 16)
  // each count a share of the candidates above it and sum across the group
  const int n_cand = min(*n_cand_p, kPsaCand);
  int lpc = 16;
  while (lpc > 1 && n_cand * lpc > NT) lpc >>= 1;
  const int ci = tid / lpc, part = tid & (lpc - 1);
  if (ci < n_cand) {
    const unsigned long long mine_o = sm.cand[ci];
    const int idx = (int)(0xFFFFFFFFu - (uint32_t)(mine_o & 0xFFFFFFFFull));
    int slot = 0;
    if (part == 0) slot = PsaKeys<E, NT>::kResident ? sm.cand_slot[ci] : ks.ptrow[idx];   // in flight during the count
    int r = 0;
    for (int x = part; x < n_cand; x += lpc) r += sm.cand[x] > mine_o ? 1 : 0;   // order values are distinct
    for (int msk = 1; msk < lpc; msk <<= 1) r += __shfl_xor(r, msk, 64);
    if (part == 0) {
      if (r < n_pick) {
        sm.page[r] = idx;
        sm.slot[r] = slot;
      }
      if (r == n_pick - 1) sm.kbound = mine_o;
    }
  }
  __syncthreads();
  kb = sm.kbound;
}

// The progressive selection and walk of one (b, KV head): srow is the
// row's scores and ptrow its page-table row (global memory, or the LDS copy
// of the fused kernel).  E pages per thread at most: rows up to E * NT pages
// (the launch takes the smallest E that holds max_pages).
template <typename T, int D, int G, int E>
__device__ __forceinline__ void psa_body(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* srow,
    const int32_t* ptrow, int L, int h, int b, int n_kv_heads, int P, int max_pages, int num_slots, int stop_mode,
    int never_stop, int always_stop, float ln_odds, float scale, float c, int32_t* __restrict__ ids,
    int32_t* __restrict__ counts, float* __restrict__ O, float* __restrict__ l, float* __restrict__ m,
    int streaming = 0, int sink = 0, int local = 0) {
  using A = AttnWave<T, D, G>;
  constexpr int CPL = A::CPL, DW = A::DW;
  constexpr int NWV = psa_waves<T, G>();
  constexpr int NT = NWV * 64;
  static_assert(E * NT <= kPsaMaxPages, "row capacity");
  static_assert(G * D <= NT && D >= 64, "one output element per thread, one head per wave");
  __shared__ PsaSmem<NWV> sm;
  __shared__ __align__(16) float lds_rows[NWV][A::LDS_FLOATS];
  __shared__ __align__(16) float ch_o[2][NWV][G][D];   // alternate groups use alternate buffers
  __shared__ float ch_ml[2][NWV][G][2];

  const int unit = b * n_kv_heads + h;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int np = (L + P - 1) / P;
  int32_t* irow = ids + (size_t)unit * max_pages;

  PsaKeys<E, NT> ks;
  ks.srow = srow;
  ks.ptrow = ptrow;
  ks.max_pages = max_pages;
  ks.np = np;
  ks.tid = tid;
  ks.round_start();

  A st;
  st.init(q + ((size_t)b * n_kv_heads * G + (size_t)h * G) * D, lds_rows[wave]);
  if (tid == 0) { sm.n_cand[0] = 0; sm.n_cand[1] = 0; }
  __syncthreads();
  const size_t slot_stride = (size_t)n_kv_heads * P * D;
  const size_t head_off = (size_t)h * P * D;
  const int TPP = P / 16;
  float acc_o = 0.0f, acc_l = 0.0f;  // thread tid < G*D owns element tid
  const int my_h = tid / D, my_c = tid % D;   // my_h is uniform over a wave
  // stop-test state, the same in every wave
  float lnacc_run = kNegInf, lnmin_run = __builtin_huge_valf();
  int left_run = np;
  float accm[G];   // running max per head of the merged blocks
#pragma unroll
  for (int hh = 0; hh < G; ++hh) accm[hh] = kNegInf;
  int visited = 0, n_rem = np, grp = 0;
  unsigned long long kb = 0ull;
  bool stop = false;
  // A streaming head (LServe section 4.1) attends to the pages holding a
  // sink or a local token, in ascending order, with the token mask; it is
  // not ranked and never stops early.  The list is [0, n_sink) then
  // [l_first, np).
  const int n_sink = min(np, (min(sink, L) + P - 1) / P);
  const int l_first = max(n_sink, (local > 0 && L > 0) ? max(0, L - local) / P : np);
  const int n_fixed = n_sink + (np - l_first);
  if (streaming) n_rem = n_fixed;
  const bool no_stop = never_stop || streaming;
  for (int round = 0; !stop && n_rem > 0; ++round) {
    const int n_pick = min(round == 0 ? kPsaFirst : kPsaRound, n_rem);
    if (streaming) {
      __syncthreads();   // the last round's reads of the page list are done
      const int e0 = (streaming ? n_fixed : np) - n_rem;
      for (int x = tid; x < n_pick; x += NT) {
        const int e = e0 + x;
        const int pg = e < n_sink ? e : l_first + (e - n_sink);
        sm.page[x] = pg;
        sm.slot[x] = ptrow[pg];
      }
      __syncthreads();
    } else if (round == 0) {
      psa_pick<E, NWV, true>(ks, round, kb, n_rem, n_pick, sm);
    } else {
      psa_pick<E, NWV, false>(ks, round, kb, n_rem, n_pick, sm);
    }
    n_rem -= n_pick;

    for (int cs = 0; cs < n_pick; cs += NWV) {
      const int buf = grp & 1;
      ++grp;
      const int pos = cs + wave;
      st.reset();
      float pm[G], pl[G];
      if (pos < n_pick) {
        const int page = sm.page[pos], slot = sm.slot[pos];
        if (slot >= 0 && slot < num_slots) {
          for (int tin = 0; tin < TPP; ++tin) {
            const int tok0 = page * P + tin * 16;
            const int nvalid = min(16, L - tok0);
            if (nvalid <= 0) break;
            uint32_t kd[4][DW], vd[4][DW];
            const size_t off = (size_t)slot * slot_stride + head_off + (size_t)tin * 16 * D;
            A::load_tile(k + off, lane, kd);
            A::load_tile(v + off, lane, vd);
            st.tile(kd, vd, nvalid, streaming != 0, tok0, L, sink, local, c);
          }
        }
      }
      st.finish(pm, pl, c);
      if (lane < 16) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc) ch_o[buf][wave][hh][lane * CPL + cc] = st.o[hh][cc];
      }
      if (lane == 0) {
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          ch_ml[buf][wave][hh][0] = (pm[hh] == kNegInf) ? kNegInf : pm[hh] * scale;
          ch_ml[buf][wave][hh][1] = pl[hh];
        }
      }
      __syncthreads();
      // stop test in rank order, in every wave: lane w of row 0 stands for
      // rank cs + w.  Block masses are summed over the group's heads, kept
      // as logs; prefix sums run in the linear domain relative to the largest.
      const int n_here = min(NWV, n_pick - cs);
      const bool here = lane < n_here;
      const int wl = lane & (NWV - 1);
      float mh[G];
      float ln_as = kNegInf;
      {
        float mx = kNegInf;
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          mh[hh] = here ? ch_ml[buf][wl][hh][0] : kNegInf;
          mx = fmaxf(mx, mh[hh]);
        }
        if (mx != kNegInf) {
          float sum = 0.0f;
#pragma unroll
          for (int hh = 0; hh < G; ++hh)
            if (mh[hh] != kNegInf) sum = fmaf(ch_ml[buf][wl][hh][1], __expf(mh[hh] - mx), sum);
          ln_as = sum > 0.0f ? mx + __logf(sum) : kNegInf;
        }
      }
      const float big = fmaxf(lnacc_run, row_max(ln_as));
      float lnacc = kNegInf;
      {
        const float x = (ln_as == kNegInf) ? 0.0f : __expf(ln_as - big);
        const float pre = row_scan_sum(x) + ((lnacc_run == kNegInf) ? 0.0f : __expf(lnacc_run - big));
        if (big != kNegInf && pre > 0.0f) lnacc = big + __logf(pre);
      }
      const float lnmin = fminf(lnmin_run, row_scan_min(here ? ln_as : __builtin_huge_valf()));
      const int left = left_run - (lane + 1);
      bool pass;
      if (no_stop) pass = false;
      else if (always_stop) pass = true;
      else if (stop_mode == 0) pass = lnacc - lnmin >= ln_odds;
      else pass = (left == 0) || (lnacc - (lnmin + __logf((float)left)) >= ln_odds);
      const unsigned long long hit = __ballot(here && pass);
      const int take = hit ? __ffsll((long long)hit) : n_here;   // 1-based rank of the first pass
      lnacc_run = readlane_f(lnacc, take - 1);
      lnmin_run = readlane_f(lnmin, take - 1);
      left_run = __builtin_amdgcn_readlane(left, take - 1);
      // merge weights of the taken blocks: lane w holds exp(m_w - M) for
      // every head, M the new running max (the same in every lane)
      float wt[G], alpha[G];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float mo = accm[hh];
        const float mt = lane < take ? mh[hh] : kNegInf;
        const float M = fmaxf(mo, readlane_f(row_max(mt), 0));
        wt[hh] = (mt == kNegInf) ? 0.0f : __expf(mt - M);
        alpha[hh] = (mo == kNegInf) ? (M == kNegInf ? 1.0f : 0.0f) : __expf(mo - M);
        accm[hh] = M;
      }
      if (tid < G * D) {
        float w_h = wt[0], a_h = alpha[0];
#pragma unroll
        for (int hh = 1; hh < G; ++hh)
          if (my_h == hh) { w_h = wt[hh]; a_h = alpha[hh]; }
        acc_o *= a_h;
        acc_l *= a_h;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
          if (w < take) {
            const float ww = readlane_f(w_h, w);
            acc_o = fmaf(ch_o[buf][w][my_h][my_c], ww, acc_o);
            acc_l = fmaf(ch_ml[buf][w][my_h][1], ww, acc_l);
          }
        }
      }
      if (tid < take) irow[visited + tid] = sm.page[cs + tid];
      visited += take;
      if (hit) {
        stop = true;
        break;
      }
    }
    if (!stop && n_rem > 0 && !streaming) ks.round_start();   // the next round's keys (not held during the walk)
  }

  // outputs
  for (int x = visited + tid; x < max_pages; x += NT) irow[x] = -1;
  if (tid == 0) counts[unit] = visited;
  if (tid < G * D) {
    float m_h = accm[0];
#pragma unroll
    for (int hh = 1; hh < G; ++hh)
      if (my_h == hh) m_h = accm[hh];
    const size_t row = (size_t)b * n_kv_heads * G + (size_t)h * G + my_h;
    O[row * D + my_c] = acc_l > 0.0f ? acc_o / acc_l : 0.0f;
    if (my_c == 0) {
      l[row] = acc_l;
      m[row] = acc_l > 0.0f ? m_h : kNegInf;
    }
  }
}

template <typename T, int D, int G, int E>
__global__ __launch_bounds__((psa_waves<T, G>() * 64)) void psa_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens, const float* __restrict__ scores,
    int n_kv_heads, int P, int max_pages, int num_slots, int stop_mode, int never_stop, int always_stop,
    float ln_odds, float scale, float c, int32_t* __restrict__ ids, int32_t* __restrict__ counts,
    float* __restrict__ O, float* __restrict__ l, float* __restrict__ m, unsigned long long streaming, int sink,
    int local) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int L = clamp_len(seq_lens[b], max_pages, P);
  psa_body<T, D, G, E>(q, k, v, scores + ((size_t)b * n_kv_heads + h) * max_pages, page_table + (size_t)b * max_pages,
                       L, h, b, n_kv_heads, P, max_pages, num_slots, stop_mode, never_stop, always_stop, ln_odds, scale,
                       c, ids, counts, O, l, m, (int)((streaming >> h) & 1ull), sink, local);
}

// ============================================================ PSA with its own scores
// dsa_psa_decode: one workgroup per (b, KV head) scores its own row into LDS
// and goes straight on to the progressive selection and walk -- no second
// launch and no global round trip of the scores.  Worth it when there are
// at least as many rows as CUs (each workgroup streams its row's metadata
// on one CU).  The scores are the page_score kernel's, operation for
// operation (group-mean query split by sign, kmax / kmin terms in channel
// order, DPP row sum), so both paths select the same pages; they are also
// written to global memory, after the walk.  Page-table row and scores live
// in dynamic LDS.
constexpr int kPsaFusedMaxPages = 8192;
#ifndef DSA_PSA_FUSED_LOADS
#define DSA_PSA_FUSED_LOADS 8
#endif
constexpr int kPsaFusedLoads = DSA_PSA_FUSED_LOADS;   // load pairs in flight per lane

template <typename T, int D, int G, int E>
__global__ __launch_bounds__((psa_waves<T, G>() * 64)) void psa_fused_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ meta,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens, int n_kv_heads, int P,
    int max_pages, int num_slots, int stop_mode, int never_stop, int always_stop, float ln_odds, float scale,
    float c, float* __restrict__ scores, int32_t* __restrict__ ids, int32_t* __restrict__ counts,
    float* __restrict__ O, float* __restrict__ l, float* __restrict__ m, unsigned long long streaming, int sink,
    int local) {
  using L_ = Lay<T, D>;
  constexpr int CPL = L_::CPL, DW = L_::DW;
  constexpr int NWV = psa_waves<T, G>();
  constexpr int NT = NWV * 64;
  constexpr int U = kPsaFusedLoads;
  extern __shared__ __align__(16) unsigned char psa_dyn[];
  float* s_score = reinterpret_cast<float*>(psa_dyn);                                  // [max_pages]
  int32_t* s_slot = reinterpret_cast<int32_t*>(psa_dyn + (((size_t)max_pages * 4 + 15) & ~(size_t)15));
  const int h = blockIdx.x, b = blockIdx.y;
  const int unit = b * n_kv_heads + h;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane >> 4, cg = lane & 15;
  const int L = clamp_len(seq_lens[b], max_pages, P);
  const int np = (L + P - 1) / P;
  const int32_t* ptg = page_table + (size_t)b * max_pages;
  for (int x = tid; x < max_pages; x += NT) s_slot[x] = ptg[x];
  if ((streaming >> h) & 1ull) {   // a streaming head: no scores (-inf, as page_score writes), fixed pages
    for (int x = tid; x < max_pages; x += NT) scores[(size_t)unit * max_pages + x] = kNegInf;
    __syncthreads();
    psa_body<T, D, G, E>(q, k, v, s_score, s_slot, L, h, b, n_kv_heads, P, max_pages, num_slots, stop_mode,
                         never_stop, always_stop, ln_odds, scale, c, ids, counts, O, l, m, 1, sink, local);
    return;
  }
  // group-mean query, this lane's channels, split by sign
  float qpos[CPL], qneg[CPL];
  {
    float acc[CPL];
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) acc[cc] = 0.0f;
#pragma unroll
    for (int gg = 0; gg < G; ++gg) {
      uint32_t w[DW];
      load_dw<DW>(q + ((size_t)b * n_kv_heads * G + (size_t)h * G + gg) * D + cg * CPL, w);
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) acc[cc] += chan<T>(w, cc);
    }
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) {
      const float qb = acc[cc] * (1.0f / G);
      qpos[cc] = fmaxf(qb, 0.0f);
      qneg[cc] = fminf(qb, 0.0f);
    }
  }
  __syncthreads();
  // row r of wave w scores page 4 (it * NWV + w) + r; U iterations' loads
  // are issued together (invalid pages read a valid address and score -inf)
  float* sg = scores + (size_t)unit * max_pages;
  const size_t head_stride = (size_t)2 * D;
  const int n_it = (max_pages + 4 * NWV - 1) / (4 * NWV);
  for (int it0 = 0; it0 < n_it; it0 += U) {
    uint32_t wmin[U][DW], wmax[U][DW];
    bool ok[U];
    int jj[U];
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      const int j = 4 * ((it0 + uu) * NWV + wave) + r;
      jj[uu] = j;
      const int slot = j < max_pages ? s_slot[j] : -1;
      ok[uu] = j < np && slot >= 0 && slot < num_slots;
      const T* src = ok[uu] ? meta + ((size_t)slot * n_kv_heads + h) * head_stride + cg * CPL : meta + cg * CPL;
      load_dw_stream<DW>(src, wmin[uu]);
      load_dw_stream<DW>(src + D, wmax[uu]);
    }
#pragma unroll
    for (int uu = 0; uu < U; ++uu) {
      float part = 0.0f;
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) {
        part = fmaf(qpos[cc], chan<T>(wmax[uu], cc), part);
        part = fmaf(qneg[cc], chan<T>(wmin[uu], cc), part);
      }
      float sc = row_sum(part);
      if (!ok[uu]) sc = kNegInf;
      if (cg == 0 && jj[uu] < max_pages) s_score[jj[uu]] = sc;
    }
  }
  __syncthreads();
  psa_body<T, D, G, E>(q, k, v, s_score, s_slot, L, h, b, n_kv_heads, P, max_pages, num_slots, stop_mode,
                       never_stop, always_stop, ln_odds, scale, c, ids, counts, O, l, m);
  // the row's scores leave LDS once, coalesced, after the walk: the scoring
  // loads then share the memory system with no scattered 4-byte stores
  for (int x = tid; x < max_pages; x += NT) sg[x] = s_score[x];
}

// ============================================================ PRR step on one stream
// A speculative PRR step ("Predict, Reuse, and Repair", sections 2-3) has
// two pairs of independent parts: the page scores (with the EMA update) and
// the speculative attention over P^t; later the speculative combine and the
// repair's partials over M^t = A^t \ P^t.  Run on two streams, each
// dependency between the HIP graph's hardware queues costs several µs here,
// so each pair instead shares one launch: the first workgroups of the grid
// run one part, the rest the other (both parts use 256-thread workgroups).
struct PrrStepArgs {
  const void *q, *kp, *vp, *meta;   // query, K and V pools, page metadata (bf16 or fp32)
  const int32_t *page_table, *seq_lens;
  int n_kv_heads, P, Pl, max_pages, num_slots, batch;
  float scale, c;
  // scores and EMA
  float* scores;
  EmaArgs ema;
  int score_ppw, score_wgs;
  // speculative attention over P^t (row stride k), its partials
  const int32_t *p_ids, *p_counts;
  int k, spec_tps, spec_splits;   // k: entries per id row
  float *spec_o, *spec_ml;
  // repair over M^t (row stride k), its partials
  const int32_t *m_ids, *m_counts;
  int rep_tps, rep_splits;
  float *rep_o, *rep_ml;
  float *O, *l, *m;
};

// The partials of one split: the matrix-core body for bf16 with 8 or 16 q
// heads per KV head, else the VALU body (TW tiles per wave either way).
template <typename T, int D, int G, int TW>
__device__ __forceinline__ void prr_partial(const PrrStepArgs& a, const int32_t* ids, const int32_t* counts, int tps,
                                            int n_splits, float* po, float* pm, int split, int h, int b) {
  if constexpr (sizeof(T) == 2 && G >= 8) {
    attn_partial_mfma_body<D, G, false, TW>((const uint16_t*)a.q, (const uint16_t*)a.kp, (const uint16_t*)a.vp,
                                            a.page_table, a.seq_lens, ids, counts, a.k, a.n_kv_heads, a.P,
                                            a.max_pages, a.num_slots, 0ull, 0, 0, a.scale, a.c, tps, n_splits,
                                            nullptr, nullptr, po, pm, split, h, b);
  } else {
    attn_partial_body<T, D, G, false, 0, TW>((const T*)a.q, (const T*)a.kp, (const T*)a.vp, a.page_table,
                                             a.seq_lens, ids, counts, a.k, a.n_kv_heads, a.P, a.max_pages,
                                             a.num_slots, 0ull, 0, 0, a.scale, a.c, tps, n_splits, nullptr, nullptr,
                                             SelectArgs{}, po, pm, split, h, b);
  }
}

template <typename T, int D, int G, int GL, int SPEC_TW>
__global__ __launch_bounds__(256) void prr_score_spec_kernel(PrrStepArgs a) {
  const int n_spec = a.spec_splits * a.n_kv_heads * a.batch;   // speculative splits first: the longer chains
  const int x = blockIdx.x;
  if (x < n_spec) {
    const int split = x % a.spec_splits, h = (x / a.spec_splits) % a.n_kv_heads, b = x / (a.spec_splits * a.n_kv_heads);
    prr_partial<T, D, G, SPEC_TW>(a, a.p_ids, a.p_counts, a.spec_tps, a.spec_splits, a.spec_o, a.spec_ml, split, h, b);
  } else {
    const int i = x - n_spec;
    score_body<T, D, G, GL>((const T*)a.q, (const T*)a.meta, a.page_table, a.seq_lens, a.n_kv_heads, a.P, a.Pl,
                            a.max_pages, a.num_slots, 0ull, a.score_ppw, a.score_wgs, a.scores, a.ema, i % a.score_wgs,
                            (i / a.score_wgs) % a.n_kv_heads, i / (a.score_wgs * a.n_kv_heads));
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void prr_combine_repair_kernel(PrrStepArgs a) {
  const int Hq = a.n_kv_heads * G;
  const int n_comb = Hq * a.batch;
  const int x = blockIdx.x;
  if (x < n_comb) {   // the speculative result over P^t into (O, l, m)
    attn_combine_body<D>(a.spec_o, a.spec_ml, a.p_counts, a.k, a.n_kv_heads, G, a.P / 16, a.spec_tps, a.spec_splits,
                         0, a.O, a.l, a.m, x % Hq, x / Hq);
  } else {            // the repair's partials over M^t
    const int i = x - n_comb;
    const int split = i % a.rep_splits, h = (i / a.rep_splits) % a.n_kv_heads, b = i / (a.rep_splits * a.n_kv_heads);
    prr_partial<T, D, G, kTilesPerWaveRepair>(a, a.m_ids, a.m_counts, a.rep_tps, a.rep_splits, a.rep_o, a.rep_ml,
                                              split, h, b);
  }
}

// ============================================================ host planning
static int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

struct SplitPlan {
  int tiles_per_split, n_splits, TPP;
};

// A split is one workgroup: 4 waves of TW tiles each, all in flight at once
// (TW = kTilesPerWaveMfma for the matrix-core kernel, 8+ heads per KV head
// with bf16 KV; for the VALU kernel kTilesPerWave, or kTilesPerWaveWide when
// that would give more splits than the GPU has CUs: fewer, longer splits
// then repeat the fused selection less often), so the grid grows with the
// selection: counts live on the device, so it is sized for ids_stride
// entries, and splits past a row's count exit at once.
inline SplitPlan plan_splits(const dsa_kv* kv, int ids_stride, int tw) {
  SplitPlan p;
  p.TPP = kv->page_size / 16;
  const long long tiles_max = (long long)ids_stride * p.TPP;
  p.tiles_per_split = kWgWaves * tw;
  p.n_splits = (int)((tiles_max + p.tiles_per_split - 1) / p.tiles_per_split);
  if (p.n_splits < 1) p.n_splits = 1;
  return p;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace for any plan of this shape whose waves take at least min_tw
// tiles: the smallest split gives the most splits.  The partial O values
// come first, then the (m, l) pairs at an offset set by the plan's own
// split count.
inline size_t max_splits_of(const dsa_kv* kv, int ids_stride, int min_tw) {
  const size_t min_tiles = (size_t)kWgWaves * min_tw;
  const size_t tiles_max = (size_t)ids_stride * (kv->page_size / 16);
  return (tiles_max + min_tiles - 1) / min_tiles;
}

constexpr int kMinTwAttn = kTilesPerWave < kTilesPerWaveMfma ? kTilesPerWave : kTilesPerWaveMfma;
constexpr int kMinTwRepair = kMinTwAttn < kTilesPerWaveRepair ? kMinTwAttn : kTilesPerWaveRepair;

inline size_t partial_bytes(const dsa_kv* kv, int G, int ids_stride, int min_tw) {
  const size_t units = (size_t)kv->batch * kv->n_kv_heads;
  const size_t ms = max_splits_of(kv, ids_stride, min_tw);
  return align256(units * ms * G * kv->head_dim * sizeof(float)) + align256(units * ms * G * 2 * sizeof(float));
}

template <typename T, int D, int G>
static int launch_attn_g(const void* q, const dsa_kv* kv, const int32_t* ids, const int32_t* counts,
                         int ids_stride, uint64_t smask, int sink, int local, float scale, float* O, float* l,
                         float* m, void* ws, int fold, const int32_t* skip_ids, const int32_t* skip_counts,
                         const SelectArgs& sel, hipStream_t st) {
  constexpr bool kMfma = sizeof(T) == 2 && G >= 8;
  const size_t units = (size_t)kv->batch * kv->n_kv_heads;
  // the repair over a compacted M (fold, no P to filter) reads a short
  // prefix of a long id row: many short splits, each one latency chain,
  // finish it sooner than a few long ones.  With P to filter every split
  // builds P's bitmap first, so that path keeps the usual splits.
  const bool repair = fold != 0 && skip_ids == nullptr;
  int tw = repair ? kTilesPerWaveRepair : (kMfma ? kTilesPerWaveMfma : kTilesPerWave);
  if (!kMfma && !repair) {
    const long long tiles = (long long)units * ids_stride * (kv->page_size / 16);
    if ((tiles + kWgWaves * tw - 1) / (kWgWaves * tw) > cu_count()) tw = kTilesPerWaveWide;
  }
  const SplitPlan p = plan_splits(kv, ids_stride, tw);
  float* part_o = (float*)ws;
  float* part_ml = (float*)((char*)ws + align256(units * (size_t)p.n_splits * G * D * sizeof(float)));
  const float c = scale * kLog2e;
  dim3 grid(p.n_splits, kv->n_kv_heads, kv->batch);
  const size_t dyn = skip_ids ? (size_t)((kv->max_pages + 31) / 32) * sizeof(uint32_t) : 0;
#define DSA_PARTIAL(KERNEL, TT, ...)                                                                             \
  hipLaunchKernelGGL((KERNEL<__VA_ARGS__>), grid, dim3(256), dyn, st, (const TT*)q, (const TT*)kv->k,           \
                     (const TT*)kv->v, kv->page_table, kv->seq_lens, ids, counts, ids_stride, kv->n_kv_heads,   \
                     kv->page_size, kv->max_pages, kv->num_slots, (unsigned long long)smask, sink, local, scale, \
                     c, p.tiles_per_split, p.n_splits, skip_ids, skip_counts, sel, part_o, part_ml)
  if constexpr (sizeof(T) == 2 && G >= 8) {
    constexpr int WM = kTilesPerWaveMfma, WR = kTilesPerWaveRepair;
    if (sel.e) return DSA_ERR_UNSUPPORTED;
    if (repair) DSA_PARTIAL(attn_partial_mfma_kernel, uint16_t, D, G, false, WR);
    else if (skip_ids) DSA_PARTIAL(attn_partial_mfma_kernel, uint16_t, D, G, true, WM);
    else DSA_PARTIAL(attn_partial_mfma_kernel, uint16_t, D, G, false, WM);
  } else {
    constexpr int W1 = kTilesPerWave, W2 = kTilesPerWaveWide, WR = kTilesPerWaveRepair;
    const bool wide = tw == W2 && W2 != W1;
    if (repair) {
      if (sel.e) return DSA_ERR_UNSUPPORTED;
      DSA_PARTIAL(attn_partial_kernel, T, T, D, G, false, 0, WR);
    } else if (sel.e == 8) {
      if (wide) DSA_PARTIAL(attn_partial_kernel, T, T, D, G, false, 8, W2);
      else DSA_PARTIAL(attn_partial_kernel, T, T, D, G, false, 8, W1);
    } else if (sel.e == 16) {
      if (wide) DSA_PARTIAL(attn_partial_kernel, T, T, D, G, false, 16, W2);
      else DSA_PARTIAL(attn_partial_kernel, T, T, D, G, false, 16, W1);
    } else if (sel.e) {
      return DSA_ERR_UNSUPPORTED;
    } else if (skip_ids) {
      if (wide) DSA_PARTIAL(attn_partial_kernel, T, T, D, G, true, 0, W2);
      else DSA_PARTIAL(attn_partial_kernel, T, T, D, G, true, 0, W1);
    } else {
      if (wide) DSA_PARTIAL(attn_partial_kernel, T, T, D, G, false, 0, W2);
      else DSA_PARTIAL(attn_partial_kernel, T, T, D, G, false, 0, W1);
    }
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

// Streaming heads of a PSA call: flags per KV head, sink and local tokens.
struct PsaStream {
  unsigned long long mask;
  int sink, local;
};

template <typename T, int D, int G>
static int launch_psa_g(const void* q, const dsa_kv* kv, const float* scores, float thr, int stop_mode, float scale,
                        int32_t* ids, int32_t* counts, float* O, float* l, float* m, const PsaStream& ps,
                        hipStream_t st) {
  const int never_stop = thr >= 1.0f;
  const int always_stop = thr <= 0.0f;
  const float ln_odds = (never_stop || always_stop) ? 0.0f : (float)log((double)thr / (1.0 - (double)thr));
  const float c = scale * kLog2e;
  constexpr int NT = psa_waves<T, G>() * 64;
  constexpr int EMAX = kPsaMaxPages / NT;
  constexpr int ESHORT = 4096 / NT;   // rows of up to 4096 pages
#define DSA_PSA(E_)                                                                                                \
  hipLaunchKernelGGL((psa_kernel<T, D, G, E_>), dim3(kv->n_kv_heads, kv->batch), dim3(NT), 0, st, (const T*)q,     \
                     (const T*)kv->k, (const T*)kv->v, kv->page_table, kv->seq_lens, scores, kv->n_kv_heads,       \
                     kv->page_size, kv->max_pages, kv->num_slots, stop_mode, never_stop, always_stop, ln_odds,     \
                     scale, c, ids, counts, O, l, m, ps.mask, ps.sink, ps.local)
  if (kv->max_pages <= NT * ESHORT) DSA_PSA(ESHORT);
  else if (kv->max_pages <= NT * kPsaRegKeys) DSA_PSA(kPsaRegKeys);
  else DSA_PSA(EMAX);
#undef DSA_PSA
  return launch_status();
}

template <typename T, int D>
static int launch_psa_d(const void* q, int G, const dsa_kv* kv, const float* scores, float thr, int stop_mode,
                        float scale, int32_t* ids, int32_t* counts, float* O, float* l, float* m, const PsaStream& ps,
                        hipStream_t st) {
  switch (G) {
    case 1: return launch_psa_g<T, D, 1>(q, kv, scores, thr, stop_mode, scale, ids, counts, O, l, m, ps, st);
    case 2: return launch_psa_g<T, D, 2>(q, kv, scores, thr, stop_mode, scale, ids, counts, O, l, m, ps, st);
    case 4: return launch_psa_g<T, D, 4>(q, kv, scores, thr, stop_mode, scale, ids, counts, O, l, m, ps, st);
  }
  return DSA_ERR_UNSUPPORTED;
}


inline size_t psa_fused_lds(int max_pages) {
  return (((size_t)max_pages * 4 + 15) & ~(size_t)15) + (size_t)max_pages * 4;
}

// The fused kernel for this shape, or DSA_ERR_UNSUPPORTED when its LDS
// (static + page-table row + scores) does not fit a workgroup.
template <typename T, int D, int G>
static int launch_psa_fused_g(const void* q, const dsa_kv* kv, const void* meta, float thr, int stop_mode,
                              float scale, float* scores, int32_t* ids, int32_t* counts, float* O, float* l, float* m,
                              const PsaStream& ps, hipStream_t st) {
  const int never_stop = thr >= 1.0f;
  const int always_stop = thr <= 0.0f;
  const float ln_odds = (never_stop || always_stop) ? 0.0f : (float)log((double)thr / (1.0 - (double)thr));
  const float c = scale * kLog2e;
  constexpr int NT = psa_waves<T, G>() * 64;
  const size_t dyn = psa_fused_lds(kv->max_pages);
  auto go = [&](auto kernel) -> int {
    hipFuncAttributes fa{};
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kernel)) != hipSuccess) return DSA_ERR_LAUNCH;
    if (fa.sharedSizeBytes + dyn > (size_t)max_lds_per_block()) return DSA_ERR_UNSUPPORTED;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)dyn) != hipSuccess)
      return DSA_ERR_LAUNCH;
    hipLaunchKernelGGL(kernel, dim3(kv->n_kv_heads, kv->batch), dim3(NT), dyn, st, (const T*)q, (const T*)kv->k,
                       (const T*)kv->v, (const T*)meta, kv->page_table, kv->seq_lens, kv->n_kv_heads, kv->page_size,
                       kv->max_pages, kv->num_slots, stop_mode, never_stop, always_stop, ln_odds, scale, c, scores,
                       ids, counts, O, l, m, ps.mask, ps.sink, ps.local);
    return launch_status();
  };
  if (kv->max_pages <= 4096) return go(psa_fused_kernel<T, D, G, 4096 / NT>);
  return go(psa_fused_kernel<T, D, G, kPsaFusedMaxPages / NT>);
}

template <typename T, int D>
static int launch_psa_fused_d(const void* q, int G, const dsa_kv* kv, const void* meta, float thr, int stop_mode,
                              float scale, float* scores, int32_t* ids, int32_t* counts, float* O, float* l, float* m,
                              const PsaStream& ps, hipStream_t st) {
  switch (G) {
    case 1: return launch_psa_fused_g<T, D, 1>(q, kv, meta, thr, stop_mode, scale, scores, ids, counts, O, l, m, ps, st);
    case 2: return launch_psa_fused_g<T, D, 2>(q, kv, meta, thr, stop_mode, scale, scores, ids, counts, O, l, m, ps, st);
    case 4: return launch_psa_fused_g<T, D, 4>(q, kv, meta, thr, stop_mode, scale, scores, ids, counts, O, l, m, ps, st);
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
  if (op == DSA_OP_SPARSE_DECODE_ATTN) return partial_bytes(kv, G, ids_stride, kMinTwAttn);
  if (op == DSA_OP_ATTN_REPAIR) return partial_bytes(kv, G, ids_stride, kMinTwRepair);
  if (op == DSA_OP_PRR_DECODE_STEP)   // speculative partials, then the repair's
    return partial_bytes(kv, G, ids_stride, kMinTwAttn) + partial_bytes(kv, G, ids_stride, kTilesPerWaveRepair);
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
                               int32_t ids_stride, const dsa_stream_cfg* stream_cfg, float scale, float* O, float* l,
                               float* m, void* ws, size_t ws_bytes, void* stream) {
  int G = 0;
  int rc = check_attn_common(q, n_q_heads, kv, scale, &G);
  if (rc) return rc;
  if (ids_stride < 1) return DSA_ERR_SHAPE;
  uint64_t smask;
  if ((rc = streaming_mask(stream_cfg, kv->n_kv_heads, &smask))) return rc;
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
  const int sink = stream_cfg ? stream_cfg->sink : 0, local = stream_cfg ? stream_cfg->local : 0;
  return launch_attn(q, G, kv, a_ids, a_counts, ids_stride, smask, sink, local, scale, O, l, m, ws, 1, p_ids, p_counts,
                     SelectArgs{}, (hipStream_t)stream);
}

// One PRR speculative step on one stream: scores + EMA beside the
// speculative partials, the selection, the speculative combine beside the
// repair's partials, the repair's fold.  The speculative split is the one
// dsa_sparse_decode_attn would take for these rows, so the results are
// those of the separate calls bit for bit.
template <typename T, int D, int G, int GL>
static int launch_prr_step(PrrStepArgs a, const dsa_kv* kv, float alpha, float beta, float gamma, int32_t* a_ids,
                           int32_t* a_counts, int32_t* m_ids, int32_t* m_counts, int32_t* p_ids, int32_t* p_counts,
                           void* ws, hipStream_t st) {
  constexpr bool kMfma = sizeof(T) == 2 && G >= 8;
  const size_t units = (size_t)kv->batch * kv->n_kv_heads;
  int tw = kMfma ? kTilesPerWaveMfma : kTilesPerWave;
  if (!kMfma) {
    const long long tiles = (long long)units * a.k * (kv->page_size / 16);
    if ((tiles + kWgWaves * tw - 1) / (kWgWaves * tw) > cu_count()) tw = kTilesPerWaveWide;
  }
  const SplitPlan ps = plan_splits(kv, a.k, tw);
  const SplitPlan pr = plan_splits(kv, a.k, kTilesPerWaveRepair);
  const ScorePlan sp = score_plan<G>(kv, 0);
  char* w = (char*)ws;
  a.spec_o = (float*)w;
  a.spec_ml = (float*)(w + align256(units * ps.n_splits * G * D * sizeof(float)));
  w += partial_bytes(kv, G, a.k, kMinTwAttn);
  a.rep_o = (float*)w;
  a.rep_ml = (float*)(w + align256(units * pr.n_splits * G * D * sizeof(float)));
  a.spec_tps = ps.tiles_per_split;
  a.spec_splits = ps.n_splits;
  a.rep_tps = pr.tiles_per_split;
  a.rep_splits = pr.n_splits;
  a.score_ppw = sp.ppw;
  a.score_wgs = sp.wgs;
  const long long n_spec = (long long)ps.n_splits * units, n_score = (long long)sp.wgs * units;
  const long long n_comb = (long long)kv->n_kv_heads * G * kv->batch, n_rep = (long long)pr.n_splits * units;
  if (n_spec + n_score > 0x7FFFFFFFLL || n_comb + n_rep > 0x7FFFFFFFLL) return DSA_ERR_UNSUPPORTED;
  const dim3 g1((unsigned)(n_spec + n_score));
  if constexpr (kMfma) {
    hipLaunchKernelGGL((prr_score_spec_kernel<T, D, G, GL, kTilesPerWaveMfma>), g1, dim3(256), 0, st, a);
  } else if (tw == kTilesPerWaveWide && kTilesPerWaveWide != kTilesPerWave) {
    hipLaunchKernelGGL((prr_score_spec_kernel<T, D, G, GL, kTilesPerWaveWide>), g1, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((prr_score_spec_kernel<T, D, G, GL, kTilesPerWave>), g1, dim3(256), 0, st, a);
  }
  int rc = launch_status();
  if (rc) return rc;
  rc = dsa_prr_select(a.scores, kv->batch, kv->n_kv_heads, kv->max_pages, kv->seq_lens, kv->page_size, a.k, a_ids,
                      a_counts, nullptr, nullptr, a.ema.pred, alpha, beta, gamma, 0, a.k, p_ids, p_counts, a.p_ids,
                      a.p_counts, m_ids, m_counts, nullptr, 0, st);
  if (rc) return rc;
  a.m_ids = m_ids;
  a.m_counts = m_counts;
  hipLaunchKernelGGL((prr_combine_repair_kernel<T, D, G>), dim3((unsigned)(n_comb + n_rep)), dim3(256), 0, st, a);
  if ((rc = launch_status())) return rc;
  hipLaunchKernelGGL((attn_combine_kernel<D>), dim3(kv->n_kv_heads * G, kv->batch), dim3(256), 0, st, a.rep_o,
                     a.rep_ml, m_counts, a.k, kv->n_kv_heads, G, kv->page_size / 16, pr.tiles_per_split, pr.n_splits,
                     1, a.O, a.l, a.m);
  return launch_status();
}

// (logical page = physical page only: PRR's pages carry one score each)
template <typename T, int D, int G>
static int launch_prr_step_gl(const PrrStepArgs& a, const dsa_kv* kv, float alpha, float beta, float gamma,
                              int32_t* a_ids, int32_t* a_counts, int32_t* m_ids, int32_t* m_counts, int32_t* p_ids,
                              int32_t* p_counts, void* ws, hipStream_t st) {
  if (kv->page_size != a.Pl) return DSA_ERR_UNSUPPORTED;
  return launch_prr_step<T, D, G, 1>(a, kv, alpha, beta, gamma, a_ids, a_counts, m_ids, m_counts, p_ids, p_counts, ws,
                                     st);
}

template <typename T, int D>
static int launch_prr_step_d(int G, const PrrStepArgs& a, const dsa_kv* kv, float alpha, float beta, float gamma,
                             int32_t* a_ids, int32_t* a_counts, int32_t* m_ids, int32_t* m_counts, int32_t* p_ids,
                             int32_t* p_counts, void* ws, hipStream_t st) {
  switch (G) {
    case 1: return launch_prr_step_gl<T, D, 1>(a, kv, alpha, beta, gamma, a_ids, a_counts, m_ids, m_counts, p_ids, p_counts, ws, st);
    case 2: return launch_prr_step_gl<T, D, 2>(a, kv, alpha, beta, gamma, a_ids, a_counts, m_ids, m_counts, p_ids, p_counts, ws, st);
    case 4: return launch_prr_step_gl<T, D, 4>(a, kv, alpha, beta, gamma, a_ids, a_counts, m_ids, m_counts, p_ids, p_counts, ws, st);
    case 8: return launch_prr_step_gl<T, D, 8>(a, kv, alpha, beta, gamma, a_ids, a_counts, m_ids, m_counts, p_ids, p_counts, ws, st);
    case 16: return launch_prr_step_gl<T, D, 16>(a, kv, alpha, beta, gamma, a_ids, a_counts, m_ids, m_counts, p_ids, p_counts, ws, st);
  }
  return DSA_ERR_UNSUPPORTED;
}

extern "C" int dsa_prr_decode_step(const void* q, int32_t n_q_heads, const dsa_kv* kv, const void* meta,
                                   int32_t logical_page, float* scores, float* level, float* trend, float* pred,
                                   float alpha, float beta, float gamma, int32_t k, const int32_t* p_cur_ids,
                                   const int32_t* p_cur_counts, int32_t* a_ids, int32_t* a_counts, int32_t* m_ids,
                                   int32_t* m_counts, int32_t* p_ids, int32_t* p_counts, float scale, float* O,
                                   float* l, float* m, void* ws, size_t ws_bytes, void* stream) {
  int G = 0;
  int rc = check_attn_common(q, n_q_heads, kv, scale, &G);
  if (rc) return rc;
  if ((rc = check_logical(kv, logical_page))) return rc;
  if (k < 1) return DSA_ERR_SHAPE;
  // bf16 KV, logical page = physical page, rows within the selection's limit
  if (kv->dtype != DSA_BF16 || logical_page != kv->page_size || kv->max_pages > 65536) return DSA_ERR_UNSUPPORTED;
  if (kv->batch == 0) return DSA_OK;
  if (!meta || !scores || !level || !trend || !pred || !p_cur_ids || !p_cur_counts || !a_ids || !a_counts ||
      !m_ids || !m_counts || !p_ids || !p_counts || !O || !l || !m)
    return DSA_ERR_NULL;
  if (pred == level || pred == trend || level == trend || scores == pred || scores == level || scores == trend)
    return DSA_ERR_SHAPE;
  if (p_cur_ids == p_ids || p_cur_counts == p_counts) return DSA_ERR_SHAPE;   // P^t is read while P^{t+1} is written
  if (!aligned16(meta)) return DSA_ERR_ALIGN;
  const size_t need = dsa_workspace_bytes(DSA_OP_PRR_DECODE_STEP, kv, n_q_heads, k);
  if (!ws || ws_bytes < need) return DSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return DSA_ERR_ALIGN;
  PrrStepArgs a{};
  a.q = q;
  a.kp = kv->k;
  a.vp = kv->v;
  a.meta = meta;
  a.page_table = kv->page_table;
  a.seq_lens = kv->seq_lens;
  a.n_kv_heads = kv->n_kv_heads;
  a.P = kv->page_size;
  a.Pl = logical_page;
  a.max_pages = kv->max_pages;
  a.num_slots = kv->num_slots;
  a.batch = kv->batch;
  a.scale = scale;
  a.c = scale * kLog2e;
  a.scores = scores;
  a.ema = EmaArgs{level, trend, pred, alpha, beta, gamma, 0};
  a.p_ids = p_cur_ids;
  a.p_counts = p_cur_counts;
  a.k = k;
  a.O = O;
  a.l = l;
  a.m = m;
  hipStream_t st = (hipStream_t)stream;
  if (kv->head_dim == 128)
    return launch_prr_step_d<uint16_t, 128>(G, a, kv, alpha, beta, gamma, a_ids, a_counts, m_ids, m_counts, p_ids,
                                            p_counts, ws, st);
  return launch_prr_step_d<uint16_t, 64>(G, a, kv, alpha, beta, gamma, a_ids, a_counts, m_ids, m_counts, p_ids,
                                         p_counts, ws, st);
}

extern "C" int dsa_page_select_progressive(const void* q, int32_t n_q_heads, const dsa_kv* kv, const float* scores,
                                           float threshold, int32_t stop_mode, const dsa_stream_cfg* stream_cfg,
                                           float scale, int32_t* ids, int32_t* counts, float* O, float* l, float* m,
                                           void* stream) {
  int G = 0;
  int rc = check_attn_common(q, n_q_heads, kv, scale, &G);
  if (rc) return rc;
  if (stop_mode != 0 && stop_mode != 1) return DSA_ERR_SHAPE;
  if (threshold != threshold) return DSA_ERR_SHAPE;
  uint64_t smask;
  if ((rc = streaming_mask(stream_cfg, kv->n_kv_heads, &smask))) return rc;
  if (kv->max_pages > kPsaMaxPages) return DSA_ERR_UNSUPPORTED;
  if (kv->batch == 0) return DSA_OK;
  if (!scores || !ids || !counts || !O || !l || !m) return DSA_ERR_NULL;
  const PsaStream ps{(unsigned long long)smask, stream_cfg ? stream_cfg->sink : 0, stream_cfg ? stream_cfg->local : 0};
  hipStream_t st = (hipStream_t)stream;
  const bool bf = kv->dtype == DSA_BF16;
  if (kv->head_dim == 128)
    return bf ? launch_psa_d<uint16_t, 128>(q, G, kv, scores, threshold, stop_mode, scale, ids, counts, O, l, m, ps, st)
              : launch_psa_d<float, 128>(q, G, kv, scores, threshold, stop_mode, scale, ids, counts, O, l, m, ps, st);
  return bf ? launch_psa_d<uint16_t, 64>(q, G, kv, scores, threshold, stop_mode, scale, ids, counts, O, l, m, ps, st)
            : launch_psa_d<float, 64>(q, G, kv, scores, threshold, stop_mode, scale, ids, counts, O, l, m, ps, st);
}

extern "C" int dsa_psa_decode(const void* q, int32_t n_q_heads, const dsa_kv* kv, const void* meta, float threshold,
                              int32_t stop_mode, const dsa_stream_cfg* stream_cfg, float scale, float* scores,
                              int32_t* ids, int32_t* counts, float* O, float* l, float* m, void* stream) {
  int G = 0;
  int rc = check_attn_common(q, n_q_heads, kv, scale, &G);
  if (rc) return rc;
  if (stop_mode != 0 && stop_mode != 1) return DSA_ERR_SHAPE;
  if (threshold != threshold) return DSA_ERR_SHAPE;
  uint64_t smask;
  if ((rc = streaming_mask(stream_cfg, kv->n_kv_heads, &smask))) return rc;
  if (kv->max_pages > kPsaMaxPages) return DSA_ERR_UNSUPPORTED;
  if (G > 4) return DSA_ERR_UNSUPPORTED;
  if (kv->batch == 0) return DSA_OK;
  if (!meta || !scores || !ids || !counts || !O || !l || !m) return DSA_ERR_NULL;
  if (!aligned16(meta)) return DSA_ERR_ALIGN;
  const PsaStream ps{(unsigned long long)smask, stream_cfg ? stream_cfg->sink : 0, stream_cfg ? stream_cfg->local : 0};
  hipStream_t st = (hipStream_t)stream;
  const bool bf = kv->dtype == DSA_BF16;
  if (kv->max_pages <= kPsaFusedMaxPages && (long long)kv->batch * kv->n_kv_heads >= cu_count()) {
    if (kv->head_dim == 128)
      rc = bf ? launch_psa_fused_d<uint16_t, 128>(q, G, kv, meta, threshold, stop_mode, scale, scores, ids, counts, O, l, m, ps, st)
              : launch_psa_fused_d<float, 128>(q, G, kv, meta, threshold, stop_mode, scale, scores, ids, counts, O, l, m, ps, st);
    else
      rc = bf ? launch_psa_fused_d<uint16_t, 64>(q, G, kv, meta, threshold, stop_mode, scale, scores, ids, counts, O, l, m, ps, st)
              : launch_psa_fused_d<float, 64>(q, G, kv, meta, threshold, stop_mode, scale, scores, ids, counts, O, l, m, ps, st);
    if (rc != DSA_ERR_UNSUPPORTED) return rc;
  }
  // fewer rows than CUs, long rows, or an LDS budget that does not fit: the two calls
  if ((rc = dsa_page_score(q, n_q_heads, kv, meta, kv->page_size, stream_cfg, scores, stream))) return rc;
  return dsa_page_select_progressive(q, n_q_heads, kv, scores, threshold, stop_mode, stream_cfg, scale, ids, counts,
                                     O, l, m, stream);
}
