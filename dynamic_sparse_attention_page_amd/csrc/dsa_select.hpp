// Block-wide radix selection of the largest keys, shared by the fixed top-k
// (PSA, section 2.2; PRR, section 2), the fused top-k attention and the
// PRR calibration.
//
// A workgroup of NT = NW * 64 threads holds E keys per thread; thread t owns
// element indices t, t + NT, t + 2NT, ... (bit e of a 64-bit mask stands for
// element e * NT + t).  Keys are 32-bit with the order of the float scores
// (-0 and +0 equal).  Radix select over the elements still in play, whose
// keys span [lo, hi]: each pass maps them to at most 2048 buckets with a
// map that is monotone in the key (equal keys share a bucket) and builds an
// LDS histogram; every wave then finds the bucket holding the wanted rank
// from the histogram by itself (no block scan).  Elements in higher buckets
// are chosen, lower ones dropped; if the bucket is taken whole the
// selection ends, else the pass repeats on that bucket.  The first pass maps
// the score values linearly onto the buckets (when they are finite), later
// passes take (key - lo) >> s, which removes 11 bits of span per pass.  Once
// at most 64 elements are left they are ranked directly by (key, lower
// index first); if more are left with equal keys, they are taken in index
// order -- the lower-index tie rule either way.  Index-order ranks come from
// per-(element slot, wave) ballot counts that every wave scans itself.
#pragma once

#include <type_traits>

#include "dsa_common.hpp"

namespace dsa {

constexpr int kBuckets = 2048;
constexpr int kSmall = 64;  // elements left that are ranked directly

// Histogram buckets are stored with one pad word after every 32, so the 64
// lanes of a wave reading 32 consecutive buckets each hit distinct banks.
constexpr int kHistWords = kBuckets + kBuckets / 32;
__device__ __forceinline__ int hist_at(uint32_t b) { return (int)(b + (b >> 5)); }

// The bucket holding the need-th largest element (1 <= need <= total count),
// found by one wave from a complete histogram: lane x sums buckets
// [kBuckets - 32(x+1), kBuckets - 32x), a wave scan finds the lane whose
// buckets hold the need-th, then lanes 0..31 scan that lane's buckets from
// the top down.  Returns the bucket, the elements in higher buckets and the
// elements in it (the same values in every lane).
struct BucketCut {
  uint32_t b;
  int above, n;
};
__device__ __forceinline__ BucketCut bucket_search(const unsigned* hist, int need) {
  static_assert(kBuckets == 64 * 32, "32 buckets per lane");
  const int lane = threadIdx.x & 63;
  int mine = 0;
  {
    const unsigned* h0 = hist + hist_at(kBuckets - 32 * (lane + 1));
#pragma unroll
    for (int x = 0; x < 32; ++x) mine += (int)h0[x];
  }
  const int incl = wave_incl_scan(mine);
  const unsigned long long hm = __ballot(incl - mine < need && need <= incl);
  const int src = __ffsll((long long)hm) - 1;
  const int acc0 = __builtin_amdgcn_readlane(incl - mine, src);   // elements in higher lanes' buckets
  const int sb0 = kBuckets - 32 * (src + 1);
  const int hb = lane < 32 ? (int)hist[hist_at(sb0 + 31 - lane)] : 0;
  const int pre = wave_incl_scan(hb);
  const unsigned long long fm = __ballot(lane < 32 && acc0 + pre >= need);
  const int fl = __ffsll((long long)fm) - 1;
  BucketCut c;
  c.b = (uint32_t)(sb0 + 31 - fl);
  c.above = acc0 + __builtin_amdgcn_readlane(pre - hb, fl);
  c.n = __builtin_amdgcn_readlane(hb, fl);
  return c;
}

// Per-thread element masks: 32 bits when a thread holds at most 32 elements
// (half the mask arithmetic), else 64.
template <int E>
struct MaskOf {
  using type = typename std::conditional<(E <= 32), uint32_t, unsigned long long>::type;
};

template <int E, int NW>
struct SelectSmem {
  __align__(16) unsigned hist[2][kHistWords];   // alternate passes use alternate buffers
  unsigned long long small[kSmall];
  int scan[NW];                      // ordered_ranks
  int rank[E * NW];
  uint32_t mm[2][2 * NW];            // pass min/max, alternating
  int bstar, above, n_small;
  unsigned long long kappa;
};

// Workgroup-wide LDS ordering point: a barrier, or for one wave a fence.
template <int NW>
__device__ __forceinline__ void group_sync() {
  if constexpr (NW == 1) wave_sync();
  else __syncthreads();
}

// Exclusive prefix sum over the block (threads in index order) and the total.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int x, int* smem /* NW ints */, int& total) {
  const int incl = wave_incl_scan(x);
  if constexpr (NW == 1) {
    total = __builtin_amdgcn_readlane(incl, 63);
    return incl - x;
  } else {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 63) smem[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int s = smem[w];
      if (w < wave) before += s;
      total += s;
    }
    __syncthreads();
    return before + incl - x;
  }
}

// Index-order rank of every set bit of `mask` among all set bits of the
// workgroup, and their total.  Slots (e, wave) are counted with ballots;
// with at most 64 slots every wave scans the counts itself (one barrier),
// else one block scan orders them.  Consecutive calls on the same buffers
// must be separated by a workgroup barrier.
template <int E, int NW>
__device__ __forceinline__ int ordered_ranks(unsigned long long mask64, int (&rank)[E], int* cnt /* E*NW */,
                                             int* scan_smem /* NW */) {
  static_assert(E * NW <= NW * 64, "one (element, wave) slot per thread");
  using M = typename MaskOf<E>::type;
  const M mask = (M)mask64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const unsigned long long b = __ballot((mask >> e) & 1u);
    rank[e] = __popcll(b & below);
    if (lane == 0) cnt[e * NW + wave] = __popcll(b);
  }
  group_sync<NW>();
  if constexpr (E * NW <= 64) {
    const int v = lane < E * NW ? cnt[lane] : 0;
    const int incl = wave_incl_scan(v);
#pragma unroll
    for (int e = 0; e < E; ++e) rank[e] += __builtin_amdgcn_readlane(incl - v, e * NW + wave);
    return __builtin_amdgcn_readlane(incl, 63);
  } else {
    const int tid = threadIdx.x;
    const int v = tid < E * NW ? cnt[tid] : 0;
    int total;
    const int before = block_excl_scan<NW>(v, scan_smem, total);
    if (tid < E * NW) cnt[tid] = before;
    group_sync<NW>();
#pragma unroll
    for (int e = 0; e < E; ++e) rank[e] += cnt[e * NW + wave];
    return total;
  }
}

// float -> uint32 with the same order; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key (the value of -0 comes back as +0).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Bucket map of one pass: linear in the score value, or a key shift.
struct BucketMap {
  bool lin;
  float f0, inv;
  uint32_t lo;
  int shift;
  __device__ __forceinline__ uint32_t linear(uint32_t k) const {
    return (uint32_t)fminf((key_value(k) - f0) * inv, (float)(kBuckets - 1));
  }
  __device__ __forceinline__ uint32_t shifted(uint32_t k) const { return (k - lo) >> shift; }
};

// Among the elements whose bit is set in `actm` (n_act of them over the
// workgroup), choose the `need` with the largest keys, equal keys going to
// the lower index.  Returns this thread's chosen bits.  All threads call it
// with the same n_act and need; consecutive calls on one SelectSmem must be
// separated by a workgroup barrier.
// Min / max over the block with one barrier (smem alternates between calls
// that are not separated by another barrier).
template <int NW>
__device__ __forceinline__ void block_minmax_1b(uint32_t& lo, uint32_t& hi, uint32_t* smem /* 2*NW */) {
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  if constexpr (NW > 1) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) { smem[2 * wave] = lo; smem[2 * wave + 1] = hi; }
    __syncthreads();
    lo = smem[0];
    hi = smem[1];
#pragma unroll
    for (int w = 1; w < NW; ++w) { lo = min(lo, smem[2 * w]); hi = max(hi, smem[2 * w + 1]); }
  }
}

// Exclusive block scan with one barrier (smem alternates like above).
template <int NW>
__device__ __forceinline__ int block_excl_scan_1b(int x, int* smem /* NW */) {
  const int incl = wave_incl_scan(x);
  if constexpr (NW == 1) {
    return incl - x;
  } else {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 63) smem[wave] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) before += smem[w];
    return before + incl - x;
  }
}

template <int E, int NW>
__device__ __forceinline__ unsigned long long block_select_top(const uint32_t (&key)[E], unsigned long long actm64,
                                                               int n_act, int need, SelectSmem<E, NW>& sm) {
  using M = typename MaskOf<E>::type;
  M actm = (M)actm64;
  constexpr int NT = NW * 64;
  if (need <= 0) return 0ull;
  if (need >= n_act) return actm;
  const int tid = threadIdx.x;
  M selm = 0;
  // at most: a linear pass and three shift passes narrow the keys to one
  // value, whose min / max then ends the loop
  for (int pass = 0; pass < 5; ++pass) {
    if (n_act == need) return selm | actm;
    if (n_act <= kSmall) {
      // rank the few left by (key, lower index first); the need-th largest
      // composite value is the cut.  n_small was cleared before the last
      // pass's barriers (on pass 0 here).
      if (pass == 0) {
        if (tid == 0) sm.n_small = 0;
        group_sync<NW>();
      }
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((actm >> e) & 1u) {
          const int p = atomicAdd(&sm.n_small, 1);
          sm.small[p] = ((unsigned long long)key[e] << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)(e * NT + tid));
        }
      group_sync<NW>();
      if (tid < n_act) {
        const unsigned long long mine = sm.small[tid];
        int r = 0;
        for (int x = 0; x < n_act; ++x) r += sm.small[x] > mine ? 1 : 0;
        if (r == need - 1) sm.kappa = mine;
      }
      group_sync<NW>();
      const uint32_t cut_key = (uint32_t)(sm.kappa >> 32);
      const int cut_idx = (int)(0xFFFFFFFFu - (uint32_t)(sm.kappa & 0xFFFFFFFFull));
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (((actm >> e) & 1u) && (key[e] > cut_key || (key[e] == cut_key && e * NT + tid <= cut_idx)))
          selm |= (M)1 << e;
      return selm;   // the next writer of small / kappa / n_small passes a barrier first
    }
    unsigned* hist = sm.hist[pass & 1];
    static_assert(kHistWords % 4 == 0, "16-byte clears");
    for (int x = tid; x < kHistWords / 4; x += NT)   // last read two barriers ago
      reinterpret_cast<uint4*>(hist)[x] = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) sm.n_small = 0;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((actm >> e) & 1u) { lo = min(lo, key[e]); hi = max(hi, key[e]); }
    block_minmax_1b<NW>(lo, hi, sm.mm[pass & 1]);   // also orders the zeroing before the atomics
    if (lo == hi) break;
    BucketMap map;
    const uint32_t span = hi - lo;
    map.lo = lo;
    map.shift = span < (uint32_t)kBuckets ? 0 : (32 - __clz((int)span) - 11);
    map.lin = false;
    map.f0 = 0.0f;
    map.inv = 0.0f;
    if (pass == 0 && span >= (uint32_t)kBuckets) {
      const float f0 = key_value(lo), f1 = key_value(hi);
      const float inv = (float)(kBuckets - 1) / (f1 - f0);
      if (__builtin_isfinite(f0) && __builtin_isfinite(f1) && __builtin_isfinite(f1 - f0) && f1 > f0 &&
          __builtin_isfinite(inv) && inv > 0.0f) {
        map.lin = true;
        map.f0 = f0;
        map.inv = inv;
      }
    }
    // each element's bucket, kept for the classification after the search
    uint32_t bk[E];
    if (map.lin) {
#pragma unroll
      for (int e = 0; e < E; ++e) bk[e] = map.linear(key[e]);
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) bk[e] = map.shifted(key[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((actm >> e) & 1u) atomicAdd(&hist[hist_at(bk[e])], 1u);
    group_sync<NW>();
    const BucketCut cut = bucket_search(hist, need);
    M above = 0, at = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      above |= (M)(bk[e] > cut.b) << e;
      at |= (M)(bk[e] == cut.b) << e;
    }
    selm |= actm & above;
    actm &= at;
    need -= cut.above;
    n_act = cut.n;
    // no barrier: this hist buffer is next zeroed two passes later, after
    // two more barriers
  }
  // the keys still in play are equal: take them in index order
  int rk[E];
  ordered_ranks<E, NW>(actm, rk, sm.rank, sm.scan);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (((actm >> e) & 1u) && rk[e] < need) selm |= (M)1 << e;
  group_sync<NW>();   // every wave has read the counts: the caller may rank with sm.rank next
  return selm;
}

}  // namespace dsa
