// Fixed top-k page selection (PSA, section 2.2; PRR, section 2: the
// selection stage of a dynamic sparse attention step) and the fixed
// sink/local page lists of streaming heads (LServe, section 4.1).
//
// One workgroup per (sequence, KV head) of NT threads; thread t owns page
// indices t, t + NT, t + 2NT, ... (coalesced loads) in registers.  The
// block radix select of dsa_select.hpp picks the k largest scores (lower
// index on ties); the kept indices are written in ascending order through
// the same ballot ranks.
#include "dsa_host.hpp"
#include "dsa_select.hpp"

namespace dsa {

// Top keff of the valid elements (index < np) of one row held in registers,
// written ascending into out[0..k) with -1 after, and the count.
template <int E, int NW>
__device__ __forceinline__ void select_and_write(const uint32_t (&key)[E], int np, int keff, int k,
                                                 int32_t* __restrict__ out, int32_t* __restrict__ count,
                                                 SelectSmem<E, NW>& sm) {
  constexpr int NT = NW * 64;
  const int tid = threadIdx.x;
  unsigned long long actm = 0ull;  // bit e: element e * NT + tid is valid
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (e * NT + tid < np) actm |= 1ull << e;
  const unsigned long long selm = block_select_top<E, NW>(key, actm, np, keff, sm);
  int rk[E];
  ordered_ranks<E, NW>(selm, rk, sm.rank, sm.scan);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (((selm >> e) & 1ull) && rk[e] < keff) out[rk[e]] = e * NT + tid;
  for (int x = keff + tid; x < k; x += NT) out[x] = -1;
  if (tid == 0) *count = keff;
}

template <int E, int NW>
__global__ __launch_bounds__(NW * 64) void topk_kernel(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ seq_lens, int n_kv_heads,
                                                         int max_pages, int P, int k, unsigned long long streaming,
                                                         int sink, int local, int32_t* __restrict__ ids,
                                                         int32_t* __restrict__ counts) {
  constexpr int NT = NW * 64;
  __shared__ SelectSmem<E, NW> sm;
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
  const float* srow = scores + (size_t)unit * max_pages;
  // scores are loaded up to max_pages, so the loads do not wait for seq_lens
  float sv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sv[e] = (e * NT + tid < max_pages) ? srow[e * NT + tid] : 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = order_key(sv[e]);
  select_and_write<E, NW>(key, np, keff, k, out, counts + unit, sm);
}

// PRR's two selections side by side ("Predict, Reuse, and Repair",
// sections 2 and 3.1): blockIdx.z == 0 selects A^t = top-k of the scores
// IS^t, blockIdx.z == 1 selects P^{t+1} = top-k_spec of the prediction
// (already updated with IS^t).  With m_ids, the A workgroup also writes the
// missing set M^t = A^t \ P^t of the repair (section 3.4): P^t, the
// speculative set of this step, goes into an LDS bitmap, and the chosen
// pages without a bit are written ascending through the same ballot ranks.
template <int E, int NW>
__global__ __launch_bounds__(NW * 64) void prr_select_kernel(
    const float* __restrict__ scores, const float* __restrict__ pred, const int32_t* __restrict__ seq_lens,
    int n_kv_heads, int max_pages, int P, int k, int32_t* __restrict__ a_ids, int32_t* __restrict__ a_counts,
    int k_spec, int32_t* __restrict__ p_ids, int32_t* __restrict__ p_counts, const int32_t* __restrict__ pc_ids,
    const int32_t* __restrict__ pc_counts, int32_t* __restrict__ m_ids, int32_t* __restrict__ m_counts) {
  constexpr int NT = NW * 64;
  __shared__ SelectSmem<E, NW> sm;
  __shared__ uint32_t pbits[E * NT / 32];   // P^t, one bit per page
  const int h = blockIdx.x, b = blockIdx.y;
  const int unit = b * n_kv_heads + h;
  const int tid = threadIdx.x;
  const int L = clamp_len(seq_lens[b], max_pages, P);
  const int np = (L + P - 1) / P;
  const bool spec = blockIdx.z != 0;
  const float* src = (spec ? pred : scores) + (size_t)unit * max_pages;
  const int kk = spec ? k_spec : k;
  float sv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) sv[e] = (e * NT + tid < max_pages) ? src[e * NT + tid] : 0.0f;
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = order_key(sv[e]);
  select_and_write<E, NW>(key, np, min(kk, np), kk, (spec ? p_ids : a_ids) + (size_t)unit * kk,
                          (spec ? p_counts : a_counts) + unit, sm);
  if (spec || !m_ids) return;
  // P^t as an LDS bitmap
  for (int x = tid; x < E * NT / 32; x += NT) pbits[x] = 0u;
  __syncthreads();
  const int pc = min(max(pc_counts[unit], 0), k_spec);
  for (int x = tid; x < pc; x += NT) {
    const int pg = pc_ids[(size_t)unit * k_spec + x];
    if (pg >= 0 && pg < max_pages) atomicOr(&pbits[pg >> 5], 1u << (pg & 31));
  }
  const int keff = min(k, np);
  const int32_t* out = a_ids + (size_t)unit * k;
  // M^t: the entries of A (ascending, just written) without a bit of P^t,
  // compacted in order -- thread t re-reads its own run of entries, one
  // block scan places them (nothing of the selection stays live)
  __syncthreads();   // the bitmap is complete and the workgroup's a_ids stores are visible to it
  const int per = (keff + NT - 1) / NT, x0 = min(keff, tid * per), x1 = min(keff, x0 + per);
  int mine = 0;
  for (int x = x0; x < x1; ++x) {
    const int pg = out[x];
    mine += (pbits[pg >> 5] >> (pg & 31)) & 1u ? 0 : 1;
  }
  int nm;
  int w = block_excl_scan<NW>(mine, sm.scan, nm);
  int32_t* mo = m_ids + (size_t)unit * k;
  for (int x = x0; x < x1; ++x) {
    const int pg = out[x];
    if (!((pbits[pg >> 5] >> (pg & 31)) & 1u)) mo[w++] = pg;
  }
  for (int x = nm + tid; x < k; x += NT) mo[x] = -1;
  if (tid == 0) m_counts[unit] = nm;
}

// ============================================================ split-row selection
// PRR's selections over long rows (tens of thousands of pages) on many CUs.
// One workgroup takes a row at a time only up to a few thousand elements:
// beyond that it is bound by one CU's issue rate and its memory parallelism.
// Here each row is cut into chunks of kSrC elements, one workgroup each, in
// two launches:
//  1. sr_hist_kernel: every workgroup of a row derives the same monotone
//     bucket map (linear in the value over the range of a fixed sample of the
//     row), histograms its chunk into kSrNB buckets and writes the bucket
//     offsets and its elements sorted by bucket (key, index) to the
//     workspace.
//  2. sr_select_kernel: every workgroup of a row sums the chunk histograms,
//     finds the bucket b* holding the k-th largest element, ranks the
//     elements of b* (gathered from all chunks) by (key, lower index first)
//     and so obtains the exact cut (kappa, cut index): an element is chosen
//     iff its key is above kappa, or equal with an index not above the cut
//     index.  It then writes its own chunk's chosen ids at the offset given
//     by the chunks before it (ascending overall).
// Row 2u of unit u is the score row (A^t), row 2u + 1 the EMA prediction
// (P^{t+1}); the prediction of an element is recomputed from (IS, level,
// trend) wherever it is needed, and level / trend are rewritten only by the
// second launch, so no workgroup reads state another one has updated.
constexpr int kSrNW = 4;                    // waves per workgroup
constexpr int kSrNT = kSrNW * 64;
constexpr int kSrE = 8;                     // elements per thread
constexpr int kSrC = kSrE * kSrNT;          // 2048 elements per chunk
constexpr int kSrNB = 256;                  // buckets of the chunk histograms
constexpr int kSrMaxW = 32;                 // chunks per row: max_pages <= 65536
constexpr int kSrReg = kSrE * kSrNT;        // elements of b* ranked in registers
static_assert(kSrNB == kSrNT, "one bucket per thread");

// Order keys of +inf and -inf: keys beyond them are NaNs.
constexpr uint32_t kKeyPosInf = 0xFF800000u;
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;

// Value of element j of a row: the score, or for the prediction row the
// EMA update with it (level', trend' and the prediction).
struct SrRow {
  const float* is;
  const float* level;   // nullptr: the prediction is already in pred_in
  const float* trend;
  const float* pred_in;
  float alpha, beta, gamma;
  int pred, init;
  __device__ __forceinline__ float value(int j, float& nl, float& nt) const {
    if (pred && !level) { nl = nt = 0.0f; return pred_in[j]; }
    const float x = is[j];
    if (!pred || init) { nl = x; nt = 0.0f; return x; }
    float pr;
    ema_step(x, level[j], trend[j], alpha, beta, gamma, nl, nt, pr);
    return pr;
  }
  __device__ __forceinline__ float value(int j) const {
    float nl, nt;
    return value(j, nl, nt);
  }
};

// Monotone map of order keys onto kSrNB buckets: linear in the value over
// [f0, f0 + kSrNB / inv] (clamped), else the top 8 key bits.
struct SrMap {
  int lin;
  float f0, inv;
  __device__ __forceinline__ uint32_t operator()(uint32_t k) const {
    if (!lin) return k >> 24;
    if (k > kKeyPosInf) return kSrNB - 1;
    if (k < kKeyNegInf) return 0;
    const float x = (key_value(k) - f0) * inv;
    return (uint32_t)fminf(fmaxf(x, 0.0f), (float)(kSrNB - 1));
  }
};

struct SrWs {
  int32_t* off;    // [rows][W][kSrNB + 1] exclusive bucket offsets of each chunk, then its count
  uint32_t* key;   // [rows][N] each chunk's valid keys sorted by bucket
  int32_t* idx;    // [rows][N] their page indices
};

inline size_t sr_align(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t sr_ws_bytes(size_t rows, int N) {
  const size_t W = (size_t)((N + kSrC - 1) / kSrC);
  return sr_align(rows * W * (kSrNB + 1) * sizeof(int32_t)) + 2 * sr_align(rows * (size_t)N * sizeof(uint32_t));
}
inline SrWs sr_ws(void* ws, size_t rows, int N) {
  const size_t W = (size_t)((N + kSrC - 1) / kSrC);
  char* p = (char*)ws;
  SrWs s;
  s.off = (int32_t*)p;
  p += sr_align(rows * W * (kSrNB + 1) * sizeof(int32_t));
  s.key = (uint32_t*)p;
  p += sr_align(rows * (size_t)N * sizeof(uint32_t));
  s.idx = (int32_t*)p;
  return s;
}

__global__ __launch_bounds__(kSrNT) void sr_hist_kernel(const float* __restrict__ scores,
                                                        const float* __restrict__ level,
                                                        const float* __restrict__ trend,
                                                        const float* __restrict__ pred,
                                                        const int32_t* __restrict__ seq_lens, int n_kv_heads, int N,
                                                        int P, float alpha, float beta, float gamma, int init,
                                                        SrWs ws) {
  __shared__ unsigned hist[kSrNB];
  __shared__ int cursor[kSrNB];
  __shared__ uint32_t mm[2 * kSrNW];
  __shared__ int scan[kSrNW];
  const int w = blockIdx.x, unit = blockIdx.y, arr = blockIdx.z;
  const int W = gridDim.x, tid = threadIdx.x;
  const int b = unit / n_kv_heads;
  const int L = clamp_len(seq_lens[b], N, P);
  const int np = (L + P - 1) / P;
  const size_t rb = (size_t)unit * N;
  const SrRow row{scores + rb, level ? level + rb : nullptr, trend ? trend + rb : nullptr, pred + rb, alpha, beta,
                  gamma, arr, init};
  const int r = unit * 2 + arr;

  // loads up to N, so they do not wait for the sequence length
  uint32_t key[kSrE];
#pragma unroll
  for (int e = 0; e < kSrE; ++e) {
    const int j = w * kSrC + e * kSrNT + tid;
    key[e] = j < N ? order_key(row.value(j)) : 0u;
  }
  // the same sample in every workgroup of the row: kSrNT evenly spaced
  // elements, of which the valid finite ones set the range (infinities and
  // NaNs fall into the end buckets)
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  {
    const int j = N > kSrNT ? (int)((long long)tid * N / kSrNT) : tid;
    if (j < N) {
      const float v = row.value(j);
      if (j < np && __builtin_isfinite(v)) lo = hi = order_key(v);
    }
  }
  hist[tid] = 0u;
  block_minmax_1b<kSrNW>(lo, hi, mm);   // its barrier also orders the zeroing
  SrMap map{0, 0.0f, 0.0f};
  {
    const float f0 = key_value(lo), f1 = key_value(hi);
    if (lo <= hi && __builtin_isfinite(f0) && __builtin_isfinite(f1) && f1 > f0 && __builtin_isfinite(f1 - f0)) {
      const float inv = (float)kSrNB / (f1 - f0);
      if (__builtin_isfinite(inv) && inv > 0.0f) map = SrMap{1, f0, inv};
    }
  }
  uint32_t bk[kSrE];
#pragma unroll
  for (int e = 0; e < kSrE; ++e) {
    bk[e] = map(key[e]);
    if (w * kSrC + e * kSrNT + tid < np) atomicAdd(&hist[bk[e]], 1u);
  }
  __syncthreads();
  int total;
  const int ex = block_excl_scan<kSrNW>((int)hist[tid], scan, total);
  cursor[tid] = ex;
  int32_t* off = ws.off + ((size_t)r * W + w) * (kSrNB + 1);
  off[tid] = ex;
  if (tid == 0) off[kSrNB] = total;
  __syncthreads();
  uint32_t* okey = ws.key + (size_t)r * N + (size_t)w * kSrC;
  int32_t* oidx = ws.idx + (size_t)r * N + (size_t)w * kSrC;
#pragma unroll
  for (int e = 0; e < kSrE; ++e) {
    const int j = w * kSrC + e * kSrNT + tid;
    if (j < np) {
      const int pos = atomicAdd(&cursor[bk[e]], 1);   // < the chunk's count: inside the chunk's slice
      okey[pos] = key[e];
      oidx[pos] = j;
    }
  }
}

struct SrSmem {
  SelectSmem<kSrE, kSrNW> sel;
  int32_t tab[kSrMaxW * (kSrNB + 1)];   // the row's chunk offsets
  int chunk_sel[kSrMaxW];               // chosen elements per chunk
  int chunk_inp[kSrMaxW];               // ... of which in P^t
  int mstart[kSrMaxW + 1];              // b* members before each chunk
  unsigned h8[256];                     // digit histogram of the long-b* path
  unsigned long long comp[kSrNT];       // (key, ~index) of a short b*
  uint32_t mm[2][2 * kSrNW];
  int scan[2][kSrNW];
  int bstar, above, nstar, digit, need, base, base_m, n_m;
  uint32_t kappa;
  int cut;
};

// Chunk holding member m of b* (mstart ascending, mstart[0] = 0).
__device__ __forceinline__ int sr_member_chunk(const int* mstart, int W, int m) {
  int lo = 0, hi = W - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mstart[mid] <= m) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kSrNT) void sr_select_kernel(
    const float* __restrict__ scores, float* __restrict__ level, float* __restrict__ trend,
    float* __restrict__ pred, const int32_t* __restrict__ seq_lens, int n_kv_heads, int N, int P, int k, int k_spec,
    float alpha, float beta, float gamma, int init, SrWs ws, int32_t* __restrict__ a_ids,
    int32_t* __restrict__ a_counts, int32_t* __restrict__ p_ids, int32_t* __restrict__ p_counts,
    const int32_t* __restrict__ pc_ids, const int32_t* __restrict__ pc_counts, int32_t* __restrict__ m_ids,
    int32_t* __restrict__ m_counts) {
  __shared__ SrSmem sm;
  extern __shared__ uint32_t pbits[];   // P^t bitmap (the score row's workgroups with m_ids)
  const int w = blockIdx.x, unit = blockIdx.y, arr = blockIdx.z;
  const int W = gridDim.x, tid = threadIdx.x;
  const int b = unit / n_kv_heads;
  const int L = clamp_len(seq_lens[b], N, P);
  const int np = (L + P - 1) / P;
  const size_t rb = (size_t)unit * N;
  const SrRow row{scores + rb, level ? level + rb : nullptr, trend ? trend + rb : nullptr, pred + rb, alpha, beta,
                  gamma, arr, init};
  const int r = unit * 2 + arr;
  const int kk = arr ? k_spec : k;
  const int keff = min(kk, np);
  const bool with_m = arr == 0 && m_ids != nullptr;
  int32_t* out = (arr ? p_ids : a_ids) + (size_t)unit * kk;

  // own chunk; the prediction row also writes the EMA state and prediction
  uint32_t key[kSrE];
#pragma unroll
  for (int e = 0; e < kSrE; ++e) {
    const int j = w * kSrC + e * kSrNT + tid;
    key[e] = 0u;
    if (j < N) {
      float nl, nt;
      const float v = row.value(j, nl, nt);
      key[e] = order_key(v);
      if (arr && level) { level[rb + j] = nl; trend[rb + j] = nt; pred[rb + j] = v; }
    }
  }
  // P^t entries (the first kSrReg) and their scores, loaded up front
  int pc = 0;
  int pgv[kSrE];
  uint32_t pkey[kSrE];
  if (with_m) {
    pc = min(max(pc_counts[unit], 0), k_spec);
#pragma unroll
    for (int e = 0; e < kSrE; ++e) {
      const int x = e * kSrNT + tid;
      pgv[e] = x < pc ? pc_ids[(size_t)unit * k_spec + x] : -1;
    }
#pragma unroll
    for (int e = 0; e < kSrE; ++e) pkey[e] = (pgv[e] >= 0 && pgv[e] < N) ? order_key(scores[rb + pgv[e]]) : 0u;
    for (int x = tid; x < (N + 31) / 32; x += kSrNT) pbits[x] = 0u;
  }
  if (tid < kSrMaxW) { sm.chunk_inp[tid] = 0; sm.chunk_sel[tid] = 0; }

  if (keff <= 0) {   // nothing chosen (uniform)
    for (int x = w * kSrNT + tid; x < kk; x += W * kSrNT) out[x] = -1;
    if (w == 0 && tid == 0) (arr ? p_counts : a_counts)[unit] = 0;
    if (with_m) {
      for (int x = w * kSrNT + tid; x < k; x += W * kSrNT) m_ids[(size_t)unit * k + x] = -1;
      if (w == 0 && tid == 0) m_counts[unit] = 0;
    }
    return;
  }

  // 1. the row's histogram: sum of the chunk histograms
  const int32_t* offr = ws.off + (size_t)r * W * (kSrNB + 1);
  {
    constexpr int NTAB = (kSrMaxW * (kSrNB + 1) + kSrNT - 1) / kSrNT;
    int32_t tv[NTAB];   // all loads in flight together
#pragma unroll
    for (int u = 0; u < NTAB; ++u) {
      const int x = u * kSrNT + tid;
      tv[u] = x < W * (kSrNB + 1) ? offr[x] : 0;
    }
#pragma unroll
    for (int u = 0; u < NTAB; ++u) {
      const int x = u * kSrNT + tid;
      if (x < W * (kSrNB + 1)) sm.tab[x] = tv[u];
    }
  }
  __syncthreads();
  const int bt = kSrNB - 1 - tid;   // thread t takes bucket kSrNB-1-t: lower threads, higher buckets
  int cnt_b = 0;
#pragma unroll
  for (int c = 0; c < kSrMaxW; ++c)
    if (c < W) cnt_b += sm.tab[c * (kSrNB + 1) + bt + 1] - sm.tab[c * (kSrNB + 1) + bt];
  int tot;
  const int above_b = block_excl_scan<kSrNW>(cnt_b, sm.scan[0], tot);
  if (above_b < keff && keff <= above_b + cnt_b) { sm.bstar = bt; sm.above = above_b; sm.nstar = cnt_b; }
  __syncthreads();
  const int bstar = sm.bstar, nstar = sm.nstar;
  const int need1 = keff - sm.above;   // 1 <= need1 <= nstar
  if (tid < 64) {   // members of b* before each chunk: one wave scan over the chunks
    const int c = tid;
    const int n = c < W ? sm.tab[c * (kSrNB + 1) + bstar + 1] - sm.tab[c * (kSrNB + 1) + bstar] : 0;
    const int incl = wave_incl_scan(n);
    if (c < W) sm.mstart[c] = incl - n;
    if (c == W - 1) sm.mstart[W] = incl;
  }
  __syncthreads();
  auto member = [&](int m, uint32_t& kv, int& iv) {
    const int c = sr_member_chunk(sm.mstart, W, m);
    const size_t pos = (size_t)r * N + (size_t)c * kSrC + sm.tab[c * (kSrNB + 1) + bstar] + (m - sm.mstart[c]);
    kv = ws.key[pos];
    iv = ws.idx[pos];
  };

  // 2. the cut among the members of b*: the need1-th largest (key, lower index first)
  if (nstar <= kSrNT) {
    // one member per thread, ranked against all others through LDS
    unsigned long long* comp = sm.comp;
    uint32_t kv = 0u;
    int iv = 0;
    if (tid < nstar) {
      member(tid, kv, iv);
      comp[tid] = ((unsigned long long)kv << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)iv);
    }
    __syncthreads();
    if (tid < nstar) {
      const unsigned long long mine = comp[tid];
      int rank = 0;
#pragma unroll 8
      for (int x = 0; x < nstar; ++x) rank += comp[x] > mine ? 1 : 0;
      if (rank == need1 - 1) { sm.kappa = kv; sm.cut = iv; }
    }
    __syncthreads();
    if (tid < nstar && (kv > sm.kappa || (kv == sm.kappa && iv <= sm.cut)))
      atomicAdd(&sm.chunk_sel[sr_member_chunk(sm.mstart, W, tid)], 1);
  } else if (nstar <= kSrReg) {
    uint32_t mk[kSrE];
    int mi[kSrE];
    unsigned long long act = 0ull;
#pragma unroll
    for (int e = 0; e < kSrE; ++e) {
      const int m = e * kSrNT + tid;
      mk[e] = 0u;
      mi[e] = 0;
      if (m < nstar) { member(m, mk[e], mi[e]); act |= 1ull << e; }
    }
    uint32_t kappa;
    int cut;
    if (need1 >= nstar) {   // all of b*
      uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
      for (int e = 0; e < kSrE; ++e)
        if ((act >> e) & 1ull) lo = min(lo, mk[e]);
      block_minmax_1b<kSrNW>(lo, hi, sm.mm[0]);
      kappa = lo;
      cut = 0x7FFFFFFF;
    } else {
      // the need1 largest keys (equal keys in any order), their smallest key kappa ...
      const unsigned long long s1 = block_select_top<kSrE, kSrNW>(mk, act, nstar, need1, sm.sel);
      uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
      for (int e = 0; e < kSrE; ++e)
        if ((s1 >> e) & 1ull) lo = min(lo, mk[e]);
      block_minmax_1b<kSrNW>(lo, hi, sm.mm[0]);
      kappa = lo;
      // ... then among the members equal to kappa the lowest indices
      int n_gt = 0, n_eq = 0;
      unsigned long long eq = 0ull;
      uint32_t ik[kSrE];
#pragma unroll
      for (int e = 0; e < kSrE; ++e) {
        const bool on = (act >> e) & 1ull;
        n_gt += (on && mk[e] > kappa) ? 1 : 0;
        if (on && mk[e] == kappa) { eq |= 1ull << e; ++n_eq; }
        ik[e] = 0xFFFFFFFFu - (uint32_t)mi[e];
      }
      int gt_all, eq_all;
      block_excl_scan<kSrNW>(n_gt, sm.scan[0], gt_all);
      block_excl_scan<kSrNW>(n_eq, sm.scan[1], eq_all);
      const int need2 = need1 - gt_all;   // 1 <= need2 <= eq_all
      if (need2 >= eq_all) {
        cut = 0x7FFFFFFF;
      } else {
        const unsigned long long s2 = block_select_top<kSrE, kSrNW>(ik, eq, eq_all, need2, sm.sel);
        uint32_t lo2 = 0xFFFFFFFFu, hi2 = 0u;
#pragma unroll
        for (int e = 0; e < kSrE; ++e)
          if ((s2 >> e) & 1ull) hi2 = max(hi2, (uint32_t)mi[e]);
        block_minmax_1b<kSrNW>(lo2, hi2, sm.mm[1]);
        cut = (int)hi2;
      }
    }
    // chosen members per chunk
#pragma unroll
    for (int e = 0; e < kSrE; ++e) {
      const int m = e * kSrNT + tid;
      if (((act >> e) & 1ull) && (mk[e] > kappa || (mk[e] == kappa && mi[e] <= cut)))
        atomicAdd(&sm.chunk_sel[sr_member_chunk(sm.mstart, W, m)], 1);
    }
    if (tid == 0) { sm.kappa = kappa; sm.cut = cut; }
  } else {
    // many members (large runs of equal or clustered scores): radix select
    // on the 64-bit composite (key, ~index) in 8-bit digits, reading the
    // members from the workspace in every pass
    unsigned long long prefix = 0ull;
    int need = need1;
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      sm.h8[tid] = 0u;
      __syncthreads();
      for (int m = tid; m < nstar; m += kSrNT) {
        uint32_t kv;
        int iv;
        member(m, kv, iv);
        const unsigned long long comp = ((unsigned long long)kv << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)iv);
        if (pass == 0 || (comp >> (shift + 8)) == prefix) atomicAdd(&sm.h8[(comp >> shift) & 255u], 1u);
      }
      __syncthreads();
      const int d = 255 - tid;
      const int hc = (int)sm.h8[d];
      int t2;
      const int ab = block_excl_scan<kSrNW>(hc, sm.scan[0], t2);
      if (ab < need && need <= ab + hc) { sm.digit = d; sm.need = need - ab; }
      __syncthreads();
      prefix = (prefix << 8) | (unsigned long long)sm.digit;
      need = sm.need;
    }
    const uint32_t kappa = (uint32_t)(prefix >> 32);
    const int cut = (int)(0xFFFFFFFFu - (uint32_t)(prefix & 0xFFFFFFFFull));
    for (int m = tid; m < nstar; m += kSrNT) {
      uint32_t kv;
      int iv;
      member(m, kv, iv);
      if (kv > kappa || (kv == kappa && iv <= cut)) atomicAdd(&sm.chunk_sel[sr_member_chunk(sm.mstart, W, m)], 1);
    }
    if (tid == 0) { sm.kappa = kappa; sm.cut = cut; }
  }
  __syncthreads();
  const uint32_t kappa = sm.kappa;
  const int cut = sm.cut;
  auto chosen = [&](uint32_t kv, int j) { return j < np && (kv > kappa || (kv == kappa && j <= cut)); };

  // 3. P^t (score row with m_ids): bitmap, and its chosen pages per chunk
  //    (each page counted once, by the thread that set its bit)
  if (with_m) {
    auto mark = [&](int pg, uint32_t kv) {
      if (pg >= 0 && pg < N) {
        const uint32_t bit = 1u << (pg & 31);
        const uint32_t old = atomicOr(&pbits[pg >> 5], bit);
        if (!(old & bit) && chosen(kv, pg)) atomicAdd(&sm.chunk_inp[pg / kSrC], 1);
      }
    };
#pragma unroll
    for (int e = 0; e < kSrE; ++e) mark(pgv[e], pkey[e]);
    for (int x = kSrReg + tid; x < pc; x += kSrNT) {
      const int pg = pc_ids[(size_t)unit * k_spec + x];
      mark(pg, (pg >= 0 && pg < N) ? order_key(scores[rb + pg]) : 0u);
    }
  }
  __syncthreads();
  // chosen elements per chunk (those of buckets above b* plus chosen
  // members) and their offsets: one wave scan over the chunks
  if (tid < 64) {
    const int c = tid;
    int sc = 0, mc = 0;
    if (c < W) {
      const int32_t* t = sm.tab + c * (kSrNB + 1);
      sc = sm.chunk_sel[c] + t[kSrNB] - t[bstar + 1];
      mc = sc - sm.chunk_inp[c];
    }
    const int is = wave_incl_scan(sc), im = wave_incl_scan(mc);
    if (c == w) { sm.base = is - sc; sm.base_m = im - mc; }
    if (c == 63) sm.n_m = im;
  }
  __syncthreads();

  // 4. this chunk's chosen ids, ascending, after those of the chunks before it
  const int base = sm.base, base_m = sm.base_m, n_m = sm.n_m;
  unsigned long long selm = 0ull, mselm = 0ull;
#pragma unroll
  for (int e = 0; e < kSrE; ++e) {
    const int j = w * kSrC + e * kSrNT + tid;
    if (chosen(key[e], j)) {
      selm |= 1ull << e;
      if (with_m && !((pbits[j >> 5] >> (j & 31)) & 1u)) mselm |= 1ull << e;
    }
  }
  int rk[kSrE];
  ordered_ranks<kSrE, kSrNW>(selm, rk, sm.sel.rank, sm.sel.scan);
#pragma unroll
  for (int e = 0; e < kSrE; ++e)
    if (((selm >> e) & 1ull) && base + rk[e] < keff) out[base + rk[e]] = w * kSrC + e * kSrNT + tid;
  for (int x = keff + w * kSrNT + tid; x < kk; x += W * kSrNT) out[x] = -1;
  if (w == 0 && tid == 0) (arr ? p_counts : a_counts)[unit] = keff;
  if (with_m) {
    __syncthreads();   // the first ranking's counts are read
    ordered_ranks<kSrE, kSrNW>(mselm, rk, sm.sel.rank, sm.sel.scan);
    int32_t* mo = m_ids + (size_t)unit * k;
#pragma unroll
    for (int e = 0; e < kSrE; ++e)
      if (((mselm >> e) & 1ull) && base_m + rk[e] < n_m) mo[base_m + rk[e]] = w * kSrC + e * kSrNT + tid;
    for (int x = n_m + w * kSrNT + tid; x < k; x += W * kSrNT) mo[x] = -1;
    if (w == 0 && tid == 0) m_counts[unit] = n_m;
  }
}

template <int E, int NW>
static int launch_topk_e(const float* scores, int B, int Hkv, int max_pages, const int32_t* seq_lens, int P, int k,
                         uint64_t smask, int sink, int local, int32_t* ids, int32_t* counts, hipStream_t st) {
  hipLaunchKernelGGL((topk_kernel<E, NW>), dim3(Hkv, B), dim3(NW * 64), 0, st, scores, seq_lens, Hkv, max_pages, P,
                     k, (unsigned long long)smask, sink, local, ids, counts);
  return launch_status();
}

template <int E, int NW>
static int launch_prr_select_e(const float* scores, const float* pred, int B, int Hkv, int max_pages,
                               const int32_t* seq_lens, int P, int k, int32_t* a_ids, int32_t* a_counts, int k_spec,
                               int32_t* p_ids, int32_t* p_counts, const int32_t* pc_ids, const int32_t* pc_counts,
                               int32_t* m_ids, int32_t* m_counts, hipStream_t st) {
  hipLaunchKernelGGL((prr_select_kernel<E, NW>), dim3(Hkv, B, 2), dim3(NW * 64), 0, st, scores, pred, seq_lens, Hkv,
                     max_pages, P, k, a_ids, a_counts, k_spec, p_ids, p_counts, pc_ids, pc_counts, m_ids, m_counts);
  return launch_status();
}

#ifndef DSA_SR_MIN_PAGES
#define DSA_SR_MIN_PAGES 4096  // rows longer than this take the split-row selection (given a workspace)
#endif

inline bool sr_applies(int max_pages) { return max_pages > DSA_SR_MIN_PAGES; }

static int launch_prr_split(const float* scores, float* level, float* trend, float* pred, int B, int Hkv, int N,
                            const int32_t* seq_lens, int P, int k, int32_t* a_ids, int32_t* a_counts, float alpha,
                            float beta, float gamma, int init, int k_spec, int32_t* p_ids, int32_t* p_counts,
                            const int32_t* pc_ids, const int32_t* pc_counts, int32_t* m_ids, int32_t* m_counts,
                            void* ws, hipStream_t st) {
  const int units = B * Hkv;
  const int W = (N + kSrC - 1) / kSrC;
  const SrWs s = sr_ws(ws, (size_t)units * 2, N);
  const dim3 grid(W, units, 2);
  hipLaunchKernelGGL(sr_hist_kernel, grid, dim3(kSrNT), 0, st, scores, level, trend, pred, seq_lens, Hkv, N, P, alpha,
                     beta, gamma, init, s);
  int rc = launch_status();
  if (rc) return rc;
  const size_t dyn = m_ids ? (size_t)((N + 31) / 32) * sizeof(uint32_t) : 0;
  hipLaunchKernelGGL(sr_select_kernel, grid, dim3(kSrNT), dyn, st, scores, level, trend, pred, seq_lens, Hkv, N, P, k,
                     k_spec, alpha, beta, gamma, init, s, a_ids, a_counts, p_ids, p_counts, pc_ids, pc_counts, m_ids,
                     m_counts);
  return launch_status();
}

}  // namespace dsa

using namespace dsa;

extern "C" int dsa_prr_select(const float* scores, int32_t batch, int32_t n_kv_heads, int32_t max_pages,
                              const int32_t* seq_lens, int32_t page_size, int32_t k, int32_t* a_ids,
                              int32_t* a_counts, float* level, float* trend, float* pred, float alpha, float beta,
                              float gamma, int32_t init, int32_t k_spec, int32_t* p_ids, int32_t* p_counts,
                              const int32_t* p_cur_ids, const int32_t* p_cur_counts, int32_t* m_ids,
                              int32_t* m_counts, void* ws, size_t ws_bytes, void* stream) {
  if (batch < 0 || n_kv_heads < 1 || max_pages < 1 || page_size < 1 || k < 1 || k_spec < 1) return DSA_ERR_SHAPE;
  if (max_pages > 65536) return DSA_ERR_UNSUPPORTED;
  if (batch == 0) return DSA_OK;
  if (!scores || !seq_lens || !a_ids || !a_counts || !pred || !p_ids || !p_counts) return DSA_ERR_NULL;
  if (!level != !trend) return DSA_ERR_NULL;   // both NULL: pred already holds the updated prediction
  const bool ema = level != nullptr;
  if (ema && (pred == level || pred == trend || level == trend)) return DSA_ERR_SHAPE;
  if (m_ids && (!m_counts || !p_cur_ids || !p_cur_counts)) return DSA_ERR_NULL;
  if (m_ids && (p_cur_ids == p_ids || p_cur_counts == p_counts)) return DSA_ERR_SHAPE;   // P^t is read while P^{t+1} is written
  hipStream_t st = (hipStream_t)stream;
  if (ws && sr_applies(max_pages) && (long long)batch * n_kv_heads <= 65535) {
    // long rows: chunk histograms, then the cut and the writes, each over
    // all chunks of all rows; the EMA update is part of both launches
    if (ws_bytes < sr_ws_bytes((size_t)batch * n_kv_heads * 2, max_pages)) return DSA_ERR_WORKSPACE;
    if (!aligned16(ws)) return DSA_ERR_ALIGN;
    return launch_prr_split(scores, level, trend, pred, batch, n_kv_heads, max_pages, seq_lens, page_size, k, a_ids,
                            a_counts, alpha, beta, gamma, init ? 1 : 0, k_spec, p_ids, p_counts, p_cur_ids,
                            p_cur_counts, m_ids, m_counts, ws, st);
  }
  // the EMA update is elementwise and spread over the whole GPU; the two
  // selections then run in one grid
  if (ema) {
    const int rc = dsa_ema_predict_update(scores, level, trend, pred, (int64_t)batch * n_kv_heads * max_pages, alpha,
                                          beta, gamma, init, stream);
    if (rc) return rc;
  }
  const int N = max_pages;
#define DSA_PRR(E, NW) return launch_prr_select_e<E, NW>(scores, pred, batch, n_kv_heads, max_pages, seq_lens, \
                                                          page_size, k, a_ids, a_counts, k_spec, p_ids, p_counts, \
                                                          p_cur_ids, p_cur_counts, m_ids, m_counts, st)
  if (N <= 256) DSA_PRR(4, 1);
  if (N <= 512) DSA_PRR(8, 1);
  if (N <= 1024) DSA_PRR(4, 4);
  if (N <= 2048) DSA_PRR(8, 4);
  if (N <= 4096) DSA_PRR(8, 8);
  if (N <= 8192) DSA_PRR(8, 16);
  if (N <= 16384) DSA_PRR(16, 16);
  if (N <= 32768) DSA_PRR(32, 16);
  DSA_PRR(64, 16);
#undef DSA_PRR
}

extern "C" size_t dsa_prr_select_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t max_pages) {
  if (batch < 1 || n_kv_heads < 1 || max_pages < 1 || max_pages > 65536 || !sr_applies(max_pages)) return 0;
  return sr_ws_bytes((size_t)batch * n_kv_heads * 2, max_pages);
}

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
