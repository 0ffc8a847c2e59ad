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

}  // namespace dsa

using namespace dsa;

extern "C" int dsa_prr_select(const float* scores, int32_t batch, int32_t n_kv_heads, int32_t max_pages,
                              const int32_t* seq_lens, int32_t page_size, int32_t k, int32_t* a_ids,
                              int32_t* a_counts, float* level, float* trend, float* pred, float alpha, float beta,
                              float gamma, int32_t init, int32_t k_spec, int32_t* p_ids, int32_t* p_counts,
                              const int32_t* p_cur_ids, const int32_t* p_cur_counts, int32_t* m_ids,
                              int32_t* m_counts, void* stream) {
  if (batch < 0 || n_kv_heads < 1 || max_pages < 1 || page_size < 1 || k < 1 || k_spec < 1) return DSA_ERR_SHAPE;
  if (max_pages > 65536) return DSA_ERR_UNSUPPORTED;
  if (batch == 0) return DSA_OK;
  if (!scores || !seq_lens || !a_ids || !a_counts || !level || !trend || !pred || !p_ids || !p_counts)
    return DSA_ERR_NULL;
  if (pred == level || pred == trend || level == trend) return DSA_ERR_SHAPE;
  if (m_ids && (!m_counts || !p_cur_ids || !p_cur_counts)) return DSA_ERR_NULL;
  if (m_ids && (p_cur_ids == p_ids || p_cur_counts == p_counts)) return DSA_ERR_SHAPE;   // P^t is read while P^{t+1} is written
  // the EMA update is elementwise and spread over the whole GPU; the two
  // selections then run in one grid
  int rc = dsa_ema_predict_update(scores, level, trend, pred, (int64_t)batch * n_kv_heads * max_pages, alpha, beta,
                                  gamma, init, stream);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
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
