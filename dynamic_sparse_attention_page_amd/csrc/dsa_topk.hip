// Fixed top-k page selection (PSA, section 2.2; PRR, section 2: the
// selection stage of a dynamic sparse attention step) and the fixed
// sink/local page lists of streaming heads (LServe, section 4.1).
//
// One workgroup per (sequence, KV head).  Thread t owns the E consecutive
// page indices [t*E, (t+1)*E) of the score row, held in registers as
// order-preserving 32-bit keys.  The k-th largest key is found MSB-first,
// 4 bits per pass (8 passes): per-thread digit counters packed into 8-bit
// fields, a DPP row reduce-scatter plus two cross-row shuffles turn them
// into per-wave histograms, 16 LDS atomics per wave make the block
// histogram.  Keys above the threshold are all kept; keys equal to it are
// kept in index order until k is reached, which implements the lower-index
// tie rule exactly.  Two block scans then compact the kept indices in
// ascending order.
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

// float -> uint32 with the same order; -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the block (threads in index order) and the total.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int x, int* smem /* NW ints */, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
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

template <int E, int NW>
__global__ __launch_bounds__(NW * 64) void topk_kernel(const float* __restrict__ scores,
                                                         const int32_t* __restrict__ seq_lens, int n_kv_heads,
                                                         int max_pages, int P, int k, unsigned long long streaming,
                                                         int sink, int local, int32_t* __restrict__ ids,
                                                         int32_t* __restrict__ counts) {
  constexpr int NT = NW * 64;
  __shared__ unsigned hist[8][16];
  __shared__ int scan_smem[NW];
  const int h = blockIdx.x, b = blockIdx.y;
  const int unit = b * n_kv_heads + h;
  const int tid = threadIdx.x, lane = tid & 63;
  const int L = clamp_len(seq_lens[b], max_pages, P);
  const int np = (L + P - 1) / P;
  int32_t* out = ids + (size_t)unit * k;

  if ((streaming >> h) & 1ull) {
    // pages holding a sink token or a local token, ascending
    if (tid == 0) {
      const int s_end = min(sink, L);
      const int sink_pages = (s_end + P - 1) / P;
      const int l_begin = max(0, L - local);
      const int loc_first = (local > 0 && L > 0) ? l_begin / P : np;
      int n = 0;
      for (int pg = 0; pg < np && n < k; ++pg)
        if (pg < sink_pages || pg >= loc_first) out[n++] = pg;
      counts[unit] = n;
      for (int x = n; x < k; ++x) out[x] = -1;
    }
    return;
  }

  for (int x = tid; x < 8 * 16; x += NT) (&hist[0][0])[x] = 0u;
  const int keff = min(k, np);
  uint32_t key[E];
  bool valid[E];
  const float* srow = scores + (size_t)unit * max_pages;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int idx = tid * E + e;
    valid[e] = idx < np;
    key[e] = valid[e] ? order_key(srow[idx]) : 0u;
  }
  __syncthreads();

  uint32_t prefix = 0u, pmask = 0u;
  int krem = keff;
  if (keff > 0) {
    const int j = lane & 15;
#pragma unroll 1
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 28 - 4 * pass;
      unsigned long long c_lo = 0ull, c_hi = 0ull;  // 8-bit counters for digits 0-7 / 8-15
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool act = valid[e] && ((key[e] & pmask) == prefix);
        const uint32_t d = (key[e] >> shift) & 15u;
        const unsigned long long inc = act ? (1ull << (8 * (d & 7u))) : 0ull;
        if (d < 8) c_lo += inc; else c_hi += inc;
      }
      float v[16];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        v[d] = (float)((c_lo >> (8 * d)) & 0xffull);
        v[d + 8] = (float)((c_hi >> (8 * d)) & 0xffull);
      }
      row_sum_scatter<16>(v, j);  // lane j of each row: that row's count of digit j
      float t = v[0];
      t += shfl_xor_f(t, 16);
      t += shfl_xor_f(t, 32);
      if (lane < 16 && t > 0.0f) atomicAdd(&hist[pass][lane], (unsigned)t);
      __syncthreads();
      unsigned above = 0u;
      int dsel = 0;
      for (int d = 15; d >= 0; --d) {
        const unsigned hd = hist[pass][d];
        if (above + hd >= (unsigned)krem) { dsel = d; break; }
        above += hd;
      }
      krem -= (int)above;
      prefix |= (uint32_t)dsel << shift;
      pmask |= 15u << shift;
    }
  }
  // prefix is now the k-th largest key; krem keys equal to it are kept.
  int eq_local = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) eq_local += (keff > 0 && valid[e] && key[e] == prefix) ? 1 : 0;
  int eq_total;
  const int eq_before = block_excl_scan<NW>(eq_local, scan_smem, eq_total);
  bool take[E];
  int sel_local = 0, eq_seen = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bool tk = false;
    if (keff > 0 && valid[e]) {
      if (key[e] > prefix) tk = true;
      else if (key[e] == prefix) { tk = (eq_before + eq_seen) < krem; ++eq_seen; }
    }
    take[e] = tk;
    sel_local += tk ? 1 : 0;
  }
  int sel_total;
  int pos = block_excl_scan<NW>(sel_local, scan_smem, sel_total);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (take[e] && pos < keff) out[pos++] = tid * E + e;
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
  // ~8 keys per thread; 64..1024 threads
  if (max_pages <= 128) return launch_topk_e<2, 1>(scores, batch, n_kv_heads, max_pages, seq_lens, page_size, k, smask, sink, local, ids, counts, st);
  if (max_pages <= 512) return launch_topk_e<8, 1>(scores, batch, n_kv_heads, max_pages, seq_lens, page_size, k, smask, sink, local, ids, counts, st);
  if (max_pages <= 1024) return launch_topk_e<8, 2>(scores, batch, n_kv_heads, max_pages, seq_lens, page_size, k, smask, sink, local, ids, counts, st);
  if (max_pages <= 2048) return launch_topk_e<8, 4>(scores, batch, n_kv_heads, max_pages, seq_lens, page_size, k, smask, sink, local, ids, counts, st);
  if (max_pages <= 4096) return launch_topk_e<8, 8>(scores, batch, n_kv_heads, max_pages, seq_lens, page_size, k, smask, sink, local, ids, counts, st);
  if (max_pages <= 8192) return launch_topk_e<8, 16>(scores, batch, n_kv_heads, max_pages, seq_lens, page_size, k, smask, sink, local, ids, counts, st);
  if (max_pages <= 16384) return launch_topk_e<16, 16>(scores, batch, n_kv_heads, max_pages, seq_lens, page_size, k, smask, sink, local, ids, counts, st);
  if (max_pages <= 32768) return launch_topk_e<32, 16>(scores, batch, n_kv_heads, max_pages, seq_lens, page_size, k, smask, sink, local, ids, counts, st);
  return launch_topk_e<64, 16>(scores, batch, n_kv_heads, max_pages, seq_lens, page_size, k, smask, sink, local, ids, counts, st);
}
