// Block-sparse prefill attention ("LServe: Efficient Long-sequence LLM
// Serving with Unified Sparse Attention"): section 2.3 -- every T_Q x T_K
// tile of the attention map is either skipped or computed like causal
// attention; section 3.3 and Figure 5 -- dense and streaming heads run in one
// kernel whose iterator visits only the tiles it needs; section 4.1 -- a
// streaming head keeps the Lambda mask of sink and local tokens.
//
// One workgroup per (64-query tile, q head); wave w owns queries
// 16w .. 16w+15 of the tile.  The key tiles (64 keys) the tile needs are
// visited in order: all of 0 .. qt for a dense head (causal), the sink tiles
// and the tiles of the local window for a streaming head; a skipped tile
// holds no attended (query, key) pair.  Inside a visited tile the token mask
// is exact.  Per tile the workgroup stages K (row-major) and V (transposed)
// in LDS, and every wave runs the online-softmax recurrence on the matrix
// cores with the layouts of the decode tile (dsa_attn_mfma.hpp), queries in
// place of heads:
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16, D/32 steps per 16 keys;
//                    lane (h = l%16, g = l/16) holds S[query h][keys 4g+j]
//   O^T += V^T P^T   v_mfma_f32_16x16x16_bf16, P as bf16 hi + lo parts;
//                    A = V^T is one 8-byte read of the transposed V tile
// Heaviest query tiles (most key tiles) are launched first.
#include "dsa_attn_mfma.hpp"
#include "dsa_host.hpp"

namespace dsa {

constexpr int kPfTile = 64;   // T_Q = T_K

template <int D>
struct PrefillSmem {
  static constexpr int KS = D + 8;          // K row stride (bf16): rows of a read spread over banks
  static constexpr int VS = kPfTile + 8;    // V^T row stride (bf16), 8-byte aligned rows
  __align__(16) uint16_t k[kPfTile * KS];
  __align__(16) uint16_t vt[D * VS];
};

__device__ __forceinline__ uint32_t bf16_at(const uint4& x, int i) {
  const uint32_t w = i < 2 ? x.x : i < 4 ? x.y : i < 6 ? x.z : x.w;
  return (i & 1) ? (w >> 16) : (w & 0xFFFFu);
}

template <int D>
__global__ __launch_bounds__(256) void prefill_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, int L, int Hq, int Hkv,
                                                      unsigned long long streaming, int sink, int local, float scale,
                                                      float c, float* __restrict__ O, float* __restrict__ lout,
                                                      float* __restrict__ mout) {
  constexpr int NK = D / 32, NB = D / 16;
  using S = PrefillSmem<D>;
  __shared__ S sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane & 15, g = lane >> 4;
  const int qt = gridDim.x - 1 - blockIdx.x;   // heaviest tiles first
  const int hq = blockIdx.y, G = Hq / Hkv, hk = hq / G;
  const bool smask = (streaming >> hk) & 1ull;
  const int iq = qt * kPfTile + wave * 16 + h;  // this lane's query
  const size_t kv_row = (size_t)Hkv * D;

  // Q^T operand: query iq, channels 32i + 8g
  bf16x8_t qb[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (iq < L) w = *reinterpret_cast<const uint4*>(q + ((size_t)iq * Hq + hq) * D + 32 * i + 8 * g);
    qb[i] = __builtin_bit_cast(bf16x8_t, w);
  }
  f32x4_t acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = kNegInf, lpart = 0.0f;

  // key tiles: dense [0, qt]; streaming: sink tiles, then the local window's
  int n_first = qt + 1, lo2 = qt + 1;
  if (smask) {
    n_first = min(qt + 1, (sink + kPfTile - 1) / kPfTile);
    lo2 = local > 0 ? max(n_first, max(0, qt * kPfTile + 1 - local) / kPfTile) : qt + 1;
  }
  const int n_iter = n_first + max(0, qt + 1 - lo2);

  for (int it = 0; it < n_iter; ++it) {
    const int kb = it < n_first ? it : lo2 + (it - n_first);
    const int key0 = kb * kPfTile;
    __syncthreads();   // the previous tile's LDS reads are done
    // K tile, row-major: 16-byte chunk tid + 256x
#pragma unroll
    for (int x = 0; x < D / 32; ++x) {
      const int chunk = tid + 256 * x;
      const int row = chunk / (D / 8), col = (chunk % (D / 8)) * 8;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (key0 + row < L) w = *reinterpret_cast<const uint4*>(k + (size_t)(key0 + row) * kv_row + (size_t)hk * D + col);
      *reinterpret_cast<uint4*>(sm.k + row * S::KS + col) = w;
    }
    // V tile, transposed: a half-wave takes keys (2p, 2p+1), p = lane % 32,
    // and D/64 channel chunks; each channel row gets one 32-bit word
    {
      const int hw = tid >> 5, p = tid & 31;
#pragma unroll
      for (int x = 0; x < D / 64; ++x) {
        const int col = (hw * (D / 64) + x) * 8;
        uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
        const int t0 = key0 + 2 * p;
        if (t0 < L) a = *reinterpret_cast<const uint4*>(v + (size_t)t0 * kv_row + (size_t)hk * D + col);
        if (t0 + 1 < L) b = *reinterpret_cast<const uint4*>(v + (size_t)(t0 + 1) * kv_row + (size_t)hk * D + col);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<uint32_t*>(sm.vt + (col + i) * S::VS + 2 * p) = bf16_at(a, i) | (bf16_at(b, i) << 16);
      }
    }
    __syncthreads();

    // logits of 4 sub-tiles of 16 keys
    f32x4_t s[4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      s[sub] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(sm.k + (16 * sub + h) * S::KS + 32 * i + 8 * g);
        s[sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[i], s[sub], 0, 0, 0);
      }
    }
    float tm = kNegInf;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = key0 + 16 * sub + 4 * g + j;
        const bool ok = key <= iq && key < L && (!smask || key < sink || key > iq - local);
        if (!ok) s[sub][j] = kNegInf;
        tm = fmaxf(tm, s[sub][j]);
      }
    tm = fmaxf(tm, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(tm), 0x401F)));  // lanes ^ 16
    tm = fmaxf(tm, shfl_xor_f(tm, 32));
    const float mn = fmaxf(m, tm);
    const float alpha = (mn == kNegInf) ? 1.0f : fast_exp2((m - mn) * c);
    if (__builtin_amdgcn_read_exec() & __ballot(alpha != 1.0f)) {
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] *= alpha;
    }
    float psum = 0.0f;
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = exp2_diff(s[sub][j], mn, c);
        psum += p[j];
      }
      const uint32_t h01 = pack_bf16(p[0], p[1]), h23 = pack_bf16(p[2], p[3]);
      const uint32_t l01 = pack_bf16(p[0] - bf_lo(h01), p[1] - bf_hi(h01));
      const uint32_t l23 = pack_bf16(p[2] - bf_lo(h23), p[3] - bf_hi(h23));
      const s16x4_t bhi = __builtin_bit_cast(s16x4_t, make_uint2(h01, h23));
      const s16x4_t blo = __builtin_bit_cast(s16x4_t, make_uint2(l01, l23));
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const s16x4_t a = *reinterpret_cast<const s16x4_t*>(sm.vt + (16 * n + h) * S::VS + 16 * sub + 4 * g);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bhi, acc[n], 0, 0, 0);
        acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, blo, acc[n], 0, 0, 0);
      }
    }
    lpart = fmaf(lpart, alpha, psum);
    m = mn;
  }

  float lt = lpart + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(lpart), 0x401F));
  lt += shfl_xor_f(lt, 32);
  if (iq < L) {
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    float* orow = O + ((size_t)iq * Hq + hq) * D;
#pragma unroll
    for (int n = 0; n < NB; ++n)
      *reinterpret_cast<float4*>(orow + 16 * n + 4 * g) =
          make_float4(acc[n][0] * inv, acc[n][1] * inv, acc[n][2] * inv, acc[n][3] * inv);
    if (g == 0) {
      lout[(size_t)iq * Hq + hq] = lt;
      mout[(size_t)iq * Hq + hq] = lt > 0.0f ? m * scale : kNegInf;
    }
  }
}

}  // namespace dsa

using namespace dsa;

extern "C" int dsa_block_sparse_prefill(const void* q, const void* k, const void* v, int32_t L, int32_t n_q_heads,
                                        int32_t n_kv_heads, int32_t head_dim, const dsa_stream_cfg* stream_cfg,
                                        float scale, float* O, float* l, float* m, void* stream) {
  if (L < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads) return DSA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return DSA_ERR_UNSUPPORTED;
  if (!(scale > 0.0f) || !__builtin_isfinite(scale)) return DSA_ERR_SHAPE;
  uint64_t smask;
  int rc = streaming_mask(stream_cfg, n_kv_heads, &smask);
  if (rc) return rc;
  if (L == 0) return DSA_OK;
  if (!q || !k || !v || !O || !l || !m) return DSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(O)) return DSA_ERR_ALIGN;
  const int sink = stream_cfg ? stream_cfg->sink : 0, local = stream_cfg ? stream_cfg->local : 0;
  const float c = scale * kLog2e;
  const dim3 grid((L + kPfTile - 1) / kPfTile, n_q_heads);
  hipStream_t st = (hipStream_t)stream;
  if (head_dim == 128)
    hipLaunchKernelGGL((prefill_kernel<128>), grid, dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (int)L, (int)n_q_heads, (int)n_kv_heads, (unsigned long long)smask, sink,
                       local, scale, c, O, l, m);
  else
    hipLaunchKernelGGL((prefill_kernel<64>), grid, dim3(256), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (int)L, (int)n_q_heads, (int)n_kv_heads, (unsigned long long)smask, sink,
                       local, scale, c, O, l, m);
  return launch_status();
}
