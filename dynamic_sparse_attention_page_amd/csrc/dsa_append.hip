// Decode-time append: the new token's K/V rows go into the last page of
// their sequence and that page's key metadata follows in place.
//
// PSA, section 3.1 (system design): the KV cache manager writes every newly
//   generated token's K/V into its block on the GPU, and the blocks'
//   metadata stays in GPU memory for the next criticality estimate.
// LServe, section 4.2 and Figure 7: the kmin/kmax vectors of a physical page
//   come from the prefill and from the earlier decoding steps, i.e. they are
//   maintained token by token.
//
// One workgroup per sequence, one thread per 16-byte chunk of the
// (KV head, channel) rows: each chunk is one load of k_new, v_new and of the
// logical page's kmin/kmax, and one store of each; the min/max update is the
// only arithmetic.  The sequence length is read by every thread before the
// barrier and written after it, so the length array may be updated in place.
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

// Element-wise min / max of two 16-byte chunks of stored values.
template <typename T>
__device__ __forceinline__ void chunk_minmax(const uint4& a, const uint4& x, uint4& lo, uint4& hi);

template <>
__device__ __forceinline__ void chunk_minmax<float>(const uint4& a, const uint4& x, uint4& lo, uint4& hi) {
  const uint32_t* pa = reinterpret_cast<const uint32_t*>(&a);
  const uint32_t* px = reinterpret_cast<const uint32_t*>(&x);
  uint32_t* pl = reinterpret_cast<uint32_t*>(&lo);
  uint32_t* ph = reinterpret_cast<uint32_t*>(&hi);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pl[i] = __float_as_uint(fminf(__uint_as_float(pa[i]), __uint_as_float(px[i])));
    ph[i] = __float_as_uint(fmaxf(__uint_as_float(pa[i]), __uint_as_float(px[i])));
  }
}

// bf16: each 32-bit word holds two values; min/max of bf16 values is a bf16
// value, so widening, comparing and narrowing by truncation is exact.
template <>
__device__ __forceinline__ void chunk_minmax<uint16_t>(const uint4& a, const uint4& x, uint4& lo, uint4& hi) {
  const uint32_t* pa = reinterpret_cast<const uint32_t*>(&a);
  const uint32_t* px = reinterpret_cast<const uint32_t*>(&x);
  uint32_t* pl = reinterpret_cast<uint32_t*>(&lo);
  uint32_t* ph = reinterpret_cast<uint32_t*>(&hi);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a0 = bf_lo(pa[i]), a1 = bf_hi(pa[i]), x0 = bf_lo(px[i]), x1 = bf_hi(px[i]);
    pl[i] = (__float_as_uint(fminf(a0, x0)) >> 16) | (__float_as_uint(fminf(a1, x1)) & 0xffff0000u);
    ph[i] = (__float_as_uint(fmaxf(a0, x0)) >> 16) | (__float_as_uint(fmaxf(a1, x1)) & 0xffff0000u);
  }
}

template <typename T>
__global__ __launch_bounds__(1024) void append_kernel(
    T* __restrict__ k, T* __restrict__ v, const int32_t* __restrict__ page_table, const int32_t* seq_lens,
    int n_kv_heads, int P, int Pl, int D, int max_pages, int num_slots, const T* __restrict__ k_new,
    const T* __restrict__ v_new, T* __restrict__ meta, int32_t* new_lens, int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int p = seq_lens[b];
  const int j = p >= 0 ? p / P : max_pages;
  const int slot = j < max_pages ? page_table[(size_t)b * max_pages + j] : -1;
  const bool ok = slot >= 0 && slot < num_slots;
  __syncthreads();   // every thread holds p before the length is rewritten
  if (threadIdx.x == 0) {
    new_lens[b] = ok ? p + 1 : p;
    if (status) status[b] = ok ? 1 : 0;
  }
  if (!ok) return;
  constexpr int V = 16 / sizeof(T);   // values per 16-byte chunk
  const int o = p % P, s = o / Pl, g = P / Pl;
  const bool opens = (o % Pl) == 0;   // first token of its logical page
  const int cpr = D / V;
  const int n = n_kv_heads * cpr;
  for (int x = threadIdx.x; x < n; x += blockDim.x) {
    const int h = x / cpr, c0 = (x % cpr) * V;
    const size_t src = ((size_t)b * n_kv_heads + h) * D + c0;
    const uint4 kn = *reinterpret_cast<const uint4*>(k_new + src);
    const uint4 vn = *reinterpret_cast<const uint4*>(v_new + src);
    const size_t row = (((size_t)slot * n_kv_heads + h) * P + o) * D + c0;
    *reinterpret_cast<uint4*>(k + row) = kn;
    *reinterpret_cast<uint4*>(v + row) = vn;
    T* box = meta + (((size_t)slot * n_kv_heads + h) * g + s) * 2 * D + c0;   // [0] kmin, [D] kmax
    uint4 lo = kn, hi = kn;
    if (!opens) {
      uint4 t;
      chunk_minmax<T>(*reinterpret_cast<const uint4*>(box), kn, lo, t);
      chunk_minmax<T>(*reinterpret_cast<const uint4*>(box + D), kn, t, hi);
    }
    *reinterpret_cast<uint4*>(box) = lo;
    *reinterpret_cast<uint4*>(box + D) = hi;
  }
}

}  // namespace dsa

using namespace dsa;

extern "C" int dsa_kv_append(const dsa_kv* kv, int32_t logical_page, const void* k_new, const void* v_new,
                             void* meta, int32_t* new_seq_lens, int32_t* status, void* stream) {
  int rc = check_kv(kv, true);
  if (rc) return rc;
  if ((rc = check_logical(kv, logical_page))) return rc;
  if (kv->batch == 0) return DSA_OK;
  if (!k_new || !v_new || !meta || !new_seq_lens) return DSA_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(meta)) return DSA_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid(kv->batch);
  // one thread per 16-byte chunk of a sequence's rows, so all of its loads
  // are in flight at once (up to 1024 threads)
  const long long chunks = (long long)kv->n_kv_heads * kv->head_dim * (kv->dtype == DSA_BF16 ? 2 : 4) / 16;
  const dim3 block((unsigned)(chunks >= 1024 ? 1024 : (chunks + 63) / 64 * 64));
  if (kv->dtype == DSA_BF16)
    hipLaunchKernelGGL((append_kernel<uint16_t>), grid, block, 0, st, (uint16_t*)kv->k, (uint16_t*)kv->v,
                       kv->page_table, kv->seq_lens, kv->n_kv_heads, kv->page_size, logical_page, kv->head_dim,
                       kv->max_pages, kv->num_slots, (const uint16_t*)k_new, (const uint16_t*)v_new,
                       (uint16_t*)meta, new_seq_lens, status);
  else
    hipLaunchKernelGGL((append_kernel<float>), grid, block, 0, st, (float*)kv->k, (float*)kv->v,
                       kv->page_table, kv->seq_lens, kv->n_kv_heads, kv->page_size, logical_page, kv->head_dim,
                       kv->max_pages, kv->num_slots, (const float*)k_new, (const float*)v_new, (float*)meta,
                       new_seq_lens, status);
  return launch_status();
}
