// Fixed top-k page selection (PSA, section 2.2; PRR, section 2: the
// selection stage of a dynamic sparse attention step) and the fixed
// sink/local page lists of streaming heads (LServe, section 4.1).
//
// One workgroup per (sequence, KV head) of NT threads; thread t owns page
// indices t, t + NT, t + 2NT, ... (coalesced loads) in registers, as 32-bit
// keys with the order of the float scores (-0 and +0 equal).  Adaptive radix
// select: the keys still in play span [klo, khi]; bucket (key - klo) >> s,
// with s chosen so the span fills at most 2048 buckets, is monotone in the
// score and equal scores share a bucket.  An LDS histogram and a block
// suffix scan find the bucket holding the k-th largest score; pages in
// higher buckets are kept, lower ones dropped, and the pass repeats on that
// bucket (each pass removes 11 bits of span, so at most 3) until it holds
// exactly the pages still needed or only equal keys.  Those are taken in
// index order -- the lower-index tie rule.  Index-order ranks come from
// per-(element slot, wave) ballot counts and one block scan over them; the
// kept indices are written in ascending order the same way.
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

constexpr int kBuckets = 2048;

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

// Index-order rank of every set bit of `mask` (bit e = element e * NT + tid)
// among all set bits of the workgroup, and their total.  Slots (e, wave) are
// counted with ballots, one block scan orders them, lanes add their rank in
// the ballot.  cnt: E * NW ints of LDS.
template <int E, int NW>
__device__ __forceinline__ int ordered_ranks(unsigned long long mask, int (&rank)[E], int* cnt, int* scan_smem);

// Workgroup-wide LDS ordering point: a barrier, or for one wave a fence.
template <int NW>
__device__ __forceinline__ void group_sync() {
  if constexpr (NW == 1) wave_sync();
  else __syncthreads();
}

template <int NW>
__device__ __forceinline__ void group_sync();

template <int E, int NW>
__device__ __forceinline__ int ordered_ranks(unsigned long long mask, int (&rank)[E], int* cnt, int* scan_smem) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const unsigned long long b = __ballot((mask >> e) & 1ull);
    rank[e] = __popcll(b & below);
    if (lane == 0) cnt[e * NW + wave] = __popcll(b);
  }
  group_sync<NW>();
  // E * NW <= NT: one slot per thread, scanned in (e, wave) order
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

template <int E, int NW>
__global__ __launch_bounds__(NW * 64) void topk_kernel(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ seq_lens, int n_kv_heads,
                                                         int max_pages, int P, int k, unsigned long long streaming,
                                                         int sink, int local, int32_t* __restrict__ ids,
                                                         int32_t* __restrict__ counts) {
  constexpr int NT = NW * 64;
  constexpr int BPT = kBuckets / NT;  // buckets per thread in the suffix scan
  __shared__ unsigned hist[kBuckets];
  __shared__ int scan_smem[NW];
  __shared__ int rank_smem[E * NW];
  __shared__ uint32_t mm_smem[2 * NW];
  __shared__ int s_bstar, s_above;
  const int h = blockIdx.x, b = blockIdx.y;
  const int unit = b * n_kv_heads + h;
  const int tid = threadIdx.x;
  const int L = clamp_len(seq_lens[b], max_pages, P);
  const int np = (L + P - 1) / P;
  int32_t* out = ids + (size_t)unit * k;

  if ((streaming >> h) & 1ull) {
    // pages holding a sink token or a local token, ascending: the list is
    // [0, n_sink) followed by [l_first, np), so entry x is computed directly
    const int n_sink = min(np, (min(sink, L) + P - 1) / P);
    const int l_first = max(n_sink, (local > 0 && L > 0) ? max(0, L - local) / P : np);
    const int n = min(k, n_sink + (np - l_first));
    for (int x = tid; x < k; x += NT) out[x] = x < n ? (x < n_sink ? x : l_first + (x - n_sink)) : -1;
    if (tid == 0) counts[unit] = n;
    return;
  }

  const int keff = min(k, np);
  uint32_t key[E];
  unsigned long long actm = 0ull, selm = 0ull;  // bit e: page tid*E+e still in play / kept
  const float* srow = scores + (size_t)unit * max_pages;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int idx = e * NT + tid;
    key[e] = idx < np ? order_key(srow[idx]) : 0u;
    if (idx < np) actm |= 1ull << e;
  }
  int need = keff, n_act = np;
  if (need > 0) {
    for (int iter = 0; iter < 4; ++iter) {
      uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((actm >> e) & 1ull) { lo = min(lo, key[e]); hi = max(hi, key[e]); }
      block_minmax_u32<NW>(lo, hi, mm_smem);
      if (n_act == need || lo == hi) break;
      const uint32_t span = hi - lo;
      const int shift = span < (uint32_t)kBuckets ? 0 : (32 - __clz((int)span) - 11);
      for (int x = tid; x < kBuckets; x += NT) hist[x] = 0u;
      group_sync<NW>();
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((actm >> e) & 1ull) atomicAdd(&hist[(key[e] - lo) >> shift], 1u);
      group_sync<NW>();
      // suffix scan: thread t owns buckets [(NT-1-t)*BPT, +BPT), so lower t = higher buckets
      const int b0 = (NT - 1 - tid) * BPT;
      int mine = 0;
#pragma unroll
      for (int x = 0; x < BPT; ++x) mine += (int)hist[b0 + x];
      int tot;
      int acc = block_excl_scan<NW>(mine, scan_smem, tot);
      if (acc < need && need <= acc + mine) {
        for (int x = BPT - 1; x >= 0; --x) {
          const int hb = (int)hist[b0 + x];
          if (acc + hb >= need) { s_bstar = b0 + x; s_above = acc; break; }
          acc += hb;
        }
      }
      group_sync<NW>();
      const uint32_t bstar = (uint32_t)s_bstar;
      const int above = s_above;
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
      n_act = (int)hist[bstar];
      group_sync<NW>();  // hist is rewritten by the next pass
    }
  } else {
    actm = 0ull;
  }
  // the keys still in play are equal (or exactly `need` of them are left):
  // take them in index order
  {
    int rk[E];
    ordered_ranks<E, NW>(actm, rk, rank_smem, scan_smem);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (((actm >> e) & 1ull) && rk[e] < need) selm |= 1ull << e;
  }
  {
    int rk[E];
    ordered_ranks<E, NW>(selm, rk, rank_smem, scan_smem);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (((selm >> e) & 1ull) && rk[e] < keff) out[rk[e]] = e * NT + tid;
  }
  for (int x = keff + tid; x < k; x += NT) out[x] = -1;
  if (tid == 0) counts[unit] = keff;
}

template <int E, int NW>
static int launch_topk_e(const float* scores, int B, int Hkv, int max_pages, const int32_t* seq_lens, int P, int k,
                         uint64_t smask, int sink, int local, int32_t* ids, int32_t* counts, hipStream_t st) {
  hipLaunchKernelGGL((topk_kernel<E, NW>), dim3(Hkv, B), dim3(NW * 64), 0, st, scores, seq_lens, Hkv, max_pages, P,
                     k, (unsigned long long)smask, sink, local, ids, counts);
  return launch_status();
}

}  // namespace dsa

using namespace dsa;

extern "C" int dsa_page_select_topk(const float* scores, int32_t batch, int32_t n_kv_heads, int32_t max_pages,
                                    const int32_t* seq_lens, int32_t page_size, int32_t k,
                                    const dsa_stream_cfg* stream_cfg, int32_t* ids, int32_t* counts, void* stream) {
  if (batch < 0 || n_kv_heads < 1 || max_pages < 1 || page_size < 1 || k < 1) return DSA_ERR_SHAPE;
  if (max_pages > 65536) return DSA_ERR_UNSUPPORTED;
  uint64_t smask;
  int rc = streaming_mask(stream_cfg, n_kv_heads, &smask);
  if (rc) return rc;
  if (smask) {
    // the sink/local page list of a streaming head must fit in k
    long long worst = (stream_cfg->sink + (long long)page_size - 1) / page_size +
                      (stream_cfg->local + (long long)page_size - 1) / page_size + 1;
    if (worst > max_pages) worst = max_pages;
    if (worst > k) return DSA_ERR_SHAPE;
  }
  if (batch == 0) return DSA_OK;
  if (!scores || !seq_lens || !ids || !counts) return DSA_ERR_NULL;
  const int sink = stream_cfg ? stream_cfg->sink : 0, local = stream_cfg ? stream_cfg->local : 0;
  hipStream_t st = (hipStream_t)stream;
  // ~8 pages per thread; one wave up to 512 pages, up to 16 waves above
  const int N = max_pages;
#define DSA_TOPK(E, NW) return launch_topk_e<E, NW>(scores, batch, n_kv_heads, max_pages, seq_lens, page_size, k, \
                                                     smask, sink, local, ids, counts, st)
  if (N <= 256) DSA_TOPK(4, 1);
  if (N <= 512) DSA_TOPK(8, 1);
  if (N <= 1024) DSA_TOPK(4, 4);
  if (N <= 2048) DSA_TOPK(8, 4);
  if (N <= 4096) DSA_TOPK(8, 8);
  if (N <= 8192) DSA_TOPK(8, 16);
  if (N <= 16384) DSA_TOPK(16, 16);
  if (N <= 32768) DSA_TOPK(32, 16);
  DSA_TOPK(64, 16);
#undef DSA_TOPK
}
