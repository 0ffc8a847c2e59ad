// Block-wide radix selection of the largest keys, shared by the fixed top-k
// (PSA, section 2.2; PRR, section 2) and the rounds of PSA's progressive
// selection (section 3.2).
//
// A workgroup of NT = NW * 64 threads holds E keys per thread; thread t owns
// element indices t, t + NT, t + 2NT, ... (bit e of a 64-bit mask stands for
// element e * NT + t).  Keys are 32-bit with the order of the float scores
// (-0 and +0 equal).  Adaptive radix select: the keys still in play span
// [lo, hi]; bucket (key - lo) >> s, with s chosen so the span fills at most
// 2048 buckets, is monotone in the key and equal keys share a bucket.  An
// LDS histogram and a block suffix scan find the bucket holding the wanted
// rank; elements in higher buckets are chosen, lower ones dropped, and the
// pass repeats on that bucket (each pass removes 11 bits of span, so at
// most 3) until it holds exactly the elements still needed or only equal
// keys.  Those are taken in index order -- the lower-index tie rule.
// Index-order ranks come from per-(element slot, wave) ballot counts and one
// block scan over them.
#pragma once

#include "dsa_common.hpp"

namespace dsa {

constexpr int kBuckets = 2048;

template <int E, int NW>
struct SelectSmem {
  unsigned hist[kBuckets];
  int scan[NW];
  int rank[E * NW];
  uint32_t mm[2 * NW];
  int bstar, above;
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

template <int NW>
__device__ __forceinline__ void block_minmax_u32(uint32_t& lo, uint32_t& hi, uint32_t* smem /* 2*NW */) {
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
    __syncthreads();
  }
}

// Index-order rank of every set bit of `mask` among all set bits of the
// workgroup, and their total.  Slots (e, wave) are counted with ballots, one
// block scan orders them, lanes add their rank in the ballot.
template <int E, int NW>
__device__ __forceinline__ int ordered_ranks(unsigned long long mask, int (&rank)[E], int* cnt /* E*NW */,
                                             int* scan_smem /* NW */) {
  static_assert(E * NW <= NW * 64, "one (element, wave) slot per thread");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const unsigned long long b = __ballot((mask >> e) & 1ull);
    rank[e] = __popcll(b & below);
    if (lane == 0) cnt[e * NW + wave] = __popcll(b);
  }
  group_sync<NW>();
  const int tid = threadIdx.x;
  const int v = tid < E * NW ? cnt[tid] : 0;
  int total;
  const int before = block_excl_scan<NW>(v, scan_smem, total);
  if (tid < E * NW) cnt[tid] = before;
  group_sync<NW>();
#pragma unroll
  for (int e = 0; e < E; ++e) rank[e] += cnt[e * NW + wave];
  group_sync<NW>();   // cnt is reused by the next call
  return total;
}

// float -> uint32 with the same order; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Among the elements whose bit is set in `actm` (n_act of them over the
// workgroup), choose the `need` with the largest keys, equal keys going to
// the lower index.  Returns this thread's chosen bits.  All threads call it
// with the same n_act and need.
template <int E, int NW>
__device__ __forceinline__ unsigned long long block_select_top(const uint32_t (&key)[E], unsigned long long actm,
                                                               int n_act, int need, SelectSmem<E, NW>& sm) {
  constexpr int NT = NW * 64;
  constexpr int BPT = kBuckets / NT;  // buckets per thread in the suffix scan
  static_assert(kBuckets % NT == 0, "bucket split");
  if (need <= 0) return 0ull;
  if (need >= n_act) return actm;
  const int tid = threadIdx.x;
  unsigned long long selm = 0ull;
  for (int iter = 0; iter < 4; ++iter) {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((actm >> e) & 1ull) { lo = min(lo, key[e]); hi = max(hi, key[e]); }
    block_minmax_u32<NW>(lo, hi, sm.mm);
    if (n_act == need || lo == hi) break;
    const uint32_t span = hi - lo;
    const int shift = span < (uint32_t)kBuckets ? 0 : (32 - __clz((int)span) - 11);
    for (int x = tid; x < kBuckets; x += NT) sm.hist[x] = 0u;
    group_sync<NW>();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((actm >> e) & 1ull) atomicAdd(&sm.hist[(key[e] - lo) >> shift], 1u);
    group_sync<NW>();
    // suffix scan: thread t owns buckets [(NT-1-t)*BPT, +BPT), so lower t = higher buckets
    const int b0 = (NT - 1 - tid) * BPT;
    int mine = 0;
#pragma unroll
    for (int x = 0; x < BPT; ++x) mine += (int)sm.hist[b0 + x];
    int tot;
    int acc = block_excl_scan<NW>(mine, sm.scan, tot);
    if (acc < need && need <= acc + mine) {
      for (int x = BPT - 1; x >= 0; --x) {
        const int hb = (int)sm.hist[b0 + x];
        if (acc + hb >= need) { sm.bstar = b0 + x; sm.above = acc; break; }
        acc += hb;
      }
    }
    group_sync<NW>();
    const uint32_t bstar = (uint32_t)sm.bstar;
    const int above = sm.above;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const unsigned long long bit = 1ull << e;
      if (actm & bit) {
        const uint32_t bk = (key[e] - lo) >> shift;
        if (bk > bstar) { selm |= bit; actm &= ~bit; }
        else if (bk < bstar) actm &= ~bit;
      }
    }
    need -= above;
    n_act = (int)sm.hist[bstar];
    group_sync<NW>();  // hist is rewritten by the next pass
  }
  // the keys still in play are equal (or exactly `need` of them are left):
  // take them in index order
  int rk[E];
  ordered_ranks<E, NW>(actm, rk, sm.rank, sm.scan);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (((actm >> e) & 1ull) && rk[e] < need) selm |= 1ull << e;
  return selm;
}

}  // namespace dsa
