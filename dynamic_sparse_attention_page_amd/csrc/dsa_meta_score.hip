// Page key metadata and page criticality scores.
//
// page_meta_build: LServe, section 4.2 and Figure 7 -- every physical page
//   carries kmin/kmax vectors of its logical sub-pages, built once when the
//   page is filled (prefill / earlier decode steps).
// page_score: LServe, section 4.2 -- a logical page's importance is
//   sum_c max(q_c*kmax_c, q_c*kmin_c), a physical page takes the max of its
//   logical pages; PRR, section 5 -- with GQA the query is one representative
//   vector per KV head (here the mean of the group's q heads).
// page_score_ema: the same, with PRR's EMA update (section 3.1) applied to
//   each page's new score in the lane that writes it.
//
// Both kernels stream their input once with coalesced 16 B loads; the score
// kernel is HBM-bound (one multiply-add per metadata element): its metadata
// loads carry the non-temporal hint and are software-pipelined (the next
// rows load while the current rows are scored).
#include "dsa_common.hpp"
#include "dsa_host.hpp"
#include "dsa_score.hpp"

namespace dsa {

// ============================================================ metadata build
// One wave per (sequence, page, KV head).  Lane (row r, position cg) reads
// tokens 4i + r (i = 0..3) of each 16-token tile, channels [cg*CPL, +CPL).
template <typename T, int D>
__global__ __launch_bounds__(256) void meta_build_kernel(
    const T* __restrict__ k, const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    int n_kv_heads, int P, int Pl, int max_pages, int num_slots, int first_page, int n_pages_req,
    T* __restrict__ meta) {
  using L_ = Lay<T, D>;
  constexpr int CPL = L_::CPL, DW = L_::DW;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int b = blockIdx.z, h = blockIdx.y;
  const int j = first_page + blockIdx.x * 4 + wave;
  const int L = clamp_len(seq_lens[b], max_pages, P);
  const int np = (L + P - 1) / P;
  const int last = (n_pages_req < 0) ? np : min(np, first_page + n_pages_req);
  if (j < first_page || j >= last) return;
  const int slot = page_table[(size_t)b * max_pages + j];
  if (slot < 0 || slot >= num_slots) return;

  const int r = lane >> 4, cg = lane & 15;
  const int g = P / Pl, tiles_per_sub = Pl / 16;
  const T* page = k + ((size_t)slot * n_kv_heads + h) * (size_t)P * D;
  T* out = meta + ((size_t)slot * n_kv_heads + h) * (size_t)g * 2 * D;
  const int valid = min(P, L - j * P);

  for (int s = 0; s < g; ++s) {
    float mn[CPL], mx[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) { mn[c] = __builtin_huge_valf(); mx[c] = kNegInf; }
    for (int tt = 0; tt < tiles_per_sub; ++tt) {
      const int tile = s * tiles_per_sub + tt;
      uint32_t w[4][DW];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        load_dw<DW>(page + (size_t)(tile * 16 + 4 * i + r) * D + cg * CPL, w[i]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (tile * 16 + 4 * i + r < valid) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const float x = chan<T>(w[i], c);
            mn[c] = fminf(mn[c], x);
            mx[c] = fmaxf(mx[c], x);
          }
        }
      }
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      mn[c] = fminf(mn[c], shfl_xor_f(mn[c], 16));
      mn[c] = fminf(mn[c], shfl_xor_f(mn[c], 32));
      mx[c] = fmaxf(mx[c], shfl_xor_f(mx[c], 16));
      mx[c] = fmaxf(mx[c], shfl_xor_f(mx[c], 32));
    }
    if (r < 2) {  // row 0 writes kmin, row 1 writes kmax
      const bool any = s * Pl < valid;
      uint32_t o[DW];
#pragma unroll
      for (int x = 0; x < DW; ++x) {
        if constexpr (sizeof(T) == 2) {
          const float a = any ? (r == 0 ? mn[2 * x] : mx[2 * x]) : 0.0f;
          const float bb = any ? (r == 0 ? mn[2 * x + 1] : mx[2 * x + 1]) : 0.0f;
          o[x] = (__float_as_uint(a) >> 16) | (__float_as_uint(bb) & 0xffff0000u);
        } else {
          o[x] = __float_as_uint(any ? (r == 0 ? mn[x] : mx[x]) : 0.0f);
        }
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(out + (size_t)(s * 2 + r) * D + cg * CPL);
#pragma unroll
      for (int x = 0; x < DW; ++x) dst[x] = o[x];
    }
  }
}

// PRR's EMA update fused into the score launch: the lane that writes a
// page's score also updates its level and trend and writes the prediction
// (the same float operations as dsa_ema_predict_update).  level == nullptr:
// scores only.
template <typename T, int D, int G, int GL>
__global__ __launch_bounds__(256) void score_kernel(
    const T* __restrict__ q, const T* __restrict__ meta, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, int n_kv_heads, int P, int Pl, int max_pages, int num_slots,
    unsigned long long streaming, int pages_per_wave, int wgs_per_row, float* __restrict__ scores, EmaArgs ema) {
  score_body<T, D, G, GL>(q, meta, page_table, seq_lens, n_kv_heads, P, Pl, max_pages, num_slots, streaming,
                          pages_per_wave, wgs_per_row, scores, ema, (int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z);
}

}  // namespace dsa

using namespace dsa;

// ============================================================ C ABI
template <typename T, int D>
static int launch_meta(const dsa_kv* kv, int Pl, void* meta, int first_page, int n_pages, hipStream_t st) {
  int span = n_pages < 0 ? kv->max_pages - first_page : min(n_pages, kv->max_pages - first_page);
  if (span <= 0) return DSA_OK;
  dim3 grid(ceil_div(span, 4), kv->n_kv_heads, kv->batch);
  hipLaunchKernelGGL((meta_build_kernel<T, D>), grid, dim3(256), 0, st, (const T*)kv->k, kv->page_table,
                     kv->seq_lens, kv->n_kv_heads, kv->page_size, Pl, kv->max_pages, kv->num_slots, first_page,
                     n_pages, (T*)meta);
  return launch_status();
}

extern "C" int dsa_page_meta_build(const dsa_kv* kv, int32_t logical_page, void* meta, int32_t first_page,
                                   int32_t n_pages, void* stream) {
  int rc = check_kv(kv, true);
  if (rc) return rc;
  if ((rc = check_logical(kv, logical_page))) return rc;
  if (first_page < 0) return DSA_ERR_SHAPE;
  if (kv->batch == 0 || n_pages == 0 || first_page >= kv->max_pages) return DSA_OK;
  if (!meta) return DSA_ERR_NULL;
  if (!aligned16(meta)) return DSA_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const bool bf = kv->dtype == DSA_BF16;
  if (kv->head_dim == 128)
    return bf ? launch_meta<uint16_t, 128>(kv, logical_page, meta, first_page, n_pages, st)
              : launch_meta<float, 128>(kv, logical_page, meta, first_page, n_pages, st);
  return bf ? launch_meta<uint16_t, 64>(kv, logical_page, meta, first_page, n_pages, st)
            : launch_meta<float, 64>(kv, logical_page, meta, first_page, n_pages, st);
}

template <typename T, int D, int G, int GL>
static int launch_score_g(const void* q, const dsa_kv* kv, const void* meta, int Pl, uint64_t smask,
                          float* scores, const EmaArgs& ema, hipStream_t st) {
  const ScorePlan p = score_plan<G>(kv, smask);
  hipLaunchKernelGGL((score_kernel<T, D, G, GL>), p.grid, dim3(256), 0, st, (const T*)q, (const T*)meta,
                     kv->page_table, kv->seq_lens, kv->n_kv_heads, kv->page_size, Pl, kv->max_pages,
                     kv->num_slots, (unsigned long long)smask, p.ppw, p.wgs, scores, ema);
  return launch_status();
}

template <typename T, int D, int G>
static int launch_score_gl(const void* q, const dsa_kv* kv, const void* meta, int Pl, uint64_t smask,
                           float* scores, const EmaArgs& ema, hipStream_t st) {
  switch (kv->page_size / Pl) {
    case 1: return launch_score_g<T, D, G, 1>(q, kv, meta, Pl, smask, scores, ema, st);
    case 2: return launch_score_g<T, D, G, 2>(q, kv, meta, Pl, smask, scores, ema, st);
    case 4: return launch_score_g<T, D, G, 4>(q, kv, meta, Pl, smask, scores, ema, st);
  }
  return DSA_ERR_UNSUPPORTED;
}

template <typename T, int D>
static int launch_score_d(const void* q, int G, const dsa_kv* kv, const void* meta, int Pl, uint64_t smask,
                          float* scores, const EmaArgs& ema, hipStream_t st) {
  switch (G) {
    case 1: return launch_score_gl<T, D, 1>(q, kv, meta, Pl, smask, scores, ema, st);
    case 2: return launch_score_gl<T, D, 2>(q, kv, meta, Pl, smask, scores, ema, st);
    case 4: return launch_score_gl<T, D, 4>(q, kv, meta, Pl, smask, scores, ema, st);
    case 8: return launch_score_gl<T, D, 8>(q, kv, meta, Pl, smask, scores, ema, st);
    case 16: return launch_score_gl<T, D, 16>(q, kv, meta, Pl, smask, scores, ema, st);
  }
  return DSA_ERR_UNSUPPORTED;
}

static int page_score_impl(const void* q, int32_t n_q_heads, const dsa_kv* kv, const void* meta, int32_t logical_page,
                           const dsa_stream_cfg* stream_cfg, float* scores, const EmaArgs& ema, void* stream) {
  int rc = check_kv(kv, false);
  if (rc) return rc;
  if ((rc = check_logical(kv, logical_page))) return rc;
  if (n_q_heads < 1 || n_q_heads % kv->n_kv_heads) return DSA_ERR_SHAPE;
  const int G = n_q_heads / kv->n_kv_heads;
  if (!pow2_group(G)) return DSA_ERR_UNSUPPORTED;
  uint64_t smask;
  if ((rc = streaming_mask(stream_cfg, kv->n_kv_heads, &smask))) return rc;
  if (kv->batch == 0) return DSA_OK;
  if (!q || !meta || !scores) return DSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(meta)) return DSA_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const bool bf = kv->dtype == DSA_BF16;
  if (kv->head_dim == 128)
    return bf ? launch_score_d<uint16_t, 128>(q, G, kv, meta, logical_page, smask, scores, ema, st)
              : launch_score_d<float, 128>(q, G, kv, meta, logical_page, smask, scores, ema, st);
  return bf ? launch_score_d<uint16_t, 64>(q, G, kv, meta, logical_page, smask, scores, ema, st)
            : launch_score_d<float, 64>(q, G, kv, meta, logical_page, smask, scores, ema, st);
}

extern "C" int dsa_page_score(const void* q, int32_t n_q_heads, const dsa_kv* kv, const void* meta,
                              int32_t logical_page, const dsa_stream_cfg* stream_cfg, float* scores,
                              void* stream) {
  const EmaArgs none{nullptr, nullptr, nullptr, 0.0f, 0.0f, 0.0f, 0};
  return page_score_impl(q, n_q_heads, kv, meta, logical_page, stream_cfg, scores, none, stream);
}

extern "C" int dsa_page_score_ema(const void* q, int32_t n_q_heads, const dsa_kv* kv, const void* meta,
                                  int32_t logical_page, const dsa_stream_cfg* stream_cfg, float* scores, float* level,
                                  float* trend, float* pred, float alpha, float beta, float gamma, int32_t init,
                                  void* stream) {
  if (!level || !trend || !pred) return DSA_ERR_NULL;
  if (pred == level || pred == trend || level == trend || scores == pred || scores == level || scores == trend)
    return DSA_ERR_SHAPE;
  const EmaArgs ema{level, trend, pred, alpha, beta, gamma, init ? 1 : 0};
  return page_score_impl(q, n_q_heads, kv, meta, logical_page, stream_cfg, scores, ema, stream);
}
