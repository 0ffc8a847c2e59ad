// Block-sparse prefill attention ("LServe: Efficient Long-sequence LLM
// Serving with Unified Sparse Attention"): section 2.3 -- every T_Q x T_K
// tile of the attention map is either skipped or computed like causal
// attention; section 3.3 and Figure 5 -- dense and streaming heads run in one
// kernel whose iterator visits only the tiles it needs; section 4.1 -- a
// streaming head keeps the Lambda mask of sink and local tokens.
//
// One workgroup of NWQ waves per (query tile of 16 QS NWQ queries, q head);
// wave w owns QS sets of 16 consecutive queries, and every K or V read from
// LDS feeds the matrix-core products of all its sets.  The key tiles (64 keys)
// the query tile needs are visited in order: every tile up to the one of the
// last query for a dense head (causal), the sink tiles and the tiles of the
// local window for a streaming head; a skipped tile holds no attended
// (query, key) pair.  Inside a visited tile the token mask
// is exact.  Per tile the workgroup stages K and V row-major in LDS (V is
// read back transposed by the gfx950 transposed LDS reads), and every wave runs the online-softmax recurrence on the matrix
// cores with the layouts of the decode tile (dsa_attn_mfma.hpp), queries in
// place of heads:
//   S^T = K Q^T      v_mfma_f32_16x16x32_bf16, D/32 steps per 16 keys;
//                    lane (h = l%16, g = l/16) holds S[query h][keys 4g+j]
//   O^T += V^T P^T   v_mfma_f32_16x16x32_bf16 over 32 keys, P as bf16 hi +
//                    lo parts; the k index 8g + j stands for key 4g + j of
//                    the chunk's first 16 keys (j < 4) and 16 + 4g + j - 4 of
//                    its second, so B is the lane's own logits and A two
//                    transposed 8-byte reads of the row-major V tile
// Tiles below the diagonal of a dense head (and sink tiles below it) need
// no token mask.
// Heaviest query tiles (most key tiles) are launched first.
#include "dsa_attn_mfma.hpp"
#include "dsa_host.hpp"

namespace dsa {

#ifndef DSA_PREFILL_WAVES
#define DSA_PREFILL_WAVES 8   // waves per workgroup
#endif
#ifndef DSA_PREFILL_QSETS
#define DSA_PREFILL_QSETS 1   // sets of 16 queries per wave (each LDS read feeds all)
#endif

#ifndef DSA_PREFILL_KPAD
#define DSA_PREFILL_KPAD 16   // row padding of the K and V tiles in LDS (bf16 values; rows stay 16-byte aligned)
#endif

constexpr int kPfTile = 64;   // T_K

template <int D>
struct PrefillSmem {
  static constexpr int KS = D + DSA_PREFILL_KPAD;   // K and V row stride (bf16): rows of a read spread over banks
  static_assert((KS * 2) % 16 == 0, "16-byte aligned rows");
  __align__(16) uint16_t k[kPfTile * KS];
  __align__(16) uint16_t v[kPfTile * KS];   // row-major; read transposed
};

template <int D, int NWQ, int QS>
__global__ __launch_bounds__(NWQ * 64) void prefill_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, int L, int Hq, int Hkv,
                                                      unsigned long long streaming, int sink, int local, float scale,
                                                      float c, float* __restrict__ O, float* __restrict__ lout,
                                                      float* __restrict__ mout) {
  constexpr int NK = D / 32, NB = D / 16;
  constexpr int NT = NWQ * 64, QT = 16 * QS * NWQ;   // threads; queries per tile
  constexpr int NCH = kPfTile * D / 8;         // 16-byte chunks of a K (or V) tile
  constexpr int KCH = (NCH + NT - 1) / NT;     // K (and V) chunks per thread
  using S = PrefillSmem<D>;
  __shared__ S sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int h = lane & 15, g = lane >> 4;
  const int qt = gridDim.x - 1 - blockIdx.x;   // heaviest tiles first
  const int hq = blockIdx.y, G = Hq / Hkv, hk = hq / G;
  const bool smask = (streaming >> hk) & 1ull;
  const int q_first = qt * QT;
  int iq[QS];                                  // this lane's query in each set
#pragma unroll
  for (int u = 0; u < QS; ++u) iq[u] = q_first + (wave * QS + u) * 16 + h;
  const size_t kv_row = (size_t)Hkv * D;

  // Q^T operands: query iq[u], channels 32i + 8g
  bf16x8_t qb[QS][NK];
  f32x4_t acc[QS][NB];
  float m[QS], lpart[QS];
#pragma unroll
  for (int u = 0; u < QS; ++u) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (iq[u] < L) w = *reinterpret_cast<const uint4*>(q + ((size_t)iq[u] * Hq + hq) * D + 32 * i + 8 * g);
      qb[u][i] = __builtin_bit_cast(bf16x8_t, w);
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[u][n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m[u] = kNegInf;
    lpart[u] = 0.0f;
  }

  // key tiles: dense [0, kb_max]; streaming: sink tiles, then the local window's
  const int kb_max = (min(L, q_first + QT) - 1) / kPfTile;
  int n_first = kb_max + 1, lo2 = kb_max + 1;
  if (smask) {
    n_first = min(kb_max + 1, (sink + kPfTile - 1) / kPfTile);
    lo2 = local > 0 ? max(n_first, max(0, q_first + 1 - local) / kPfTile) : kb_max + 1;
  }
  const int n_iter = n_first + max(0, kb_max + 1 - lo2);

  // Global -> register staging of a key tile; the next tile's loads are in
  // flight while the current one is computed.  K and V: 16-byte chunk
  // tid + NT x of the row-major tile.
  uint4 kr[KCH], vr4[KCH];
  auto fetch = [&](int key0) {
#pragma unroll
    for (int x = 0; x < KCH; ++x) {
      const int chunk = tid + NT * x;
      const int row = chunk / (D / 8), col = (chunk % (D / 8)) * 8;
      kr[x] = make_uint4(0u, 0u, 0u, 0u);
      vr4[x] = kr[x];
      if (chunk < NCH && key0 + row < L) {
        const size_t off = (size_t)(key0 + row) * kv_row + (size_t)hk * D + col;
        kr[x] = *reinterpret_cast<const uint4*>(k + off);
        vr4[x] = *reinterpret_cast<const uint4*>(v + off);
      }
    }
  };
  auto tile_of = [&](int it) { return it < n_first ? it : lo2 + (it - n_first); };
  if (n_iter > 0) fetch(tile_of(0) * kPfTile);

  for (int it = 0; it < n_iter; ++it) {
    const int kb = tile_of(it);
    const int key0 = kb * kPfTile;
    __syncthreads();   // the previous tile's LDS reads are done
#pragma unroll
    for (int x = 0; x < KCH; ++x) {
      const int chunk = tid + NT * x;
      const int row = chunk / (D / 8), col = (chunk % (D / 8)) * 8;
      if (chunk < NCH) {
        *reinterpret_cast<uint4*>(sm.k + row * S::KS + col) = kr[x];
        *reinterpret_cast<uint4*>(sm.v + row * S::KS + col) = vr4[x];
      }
    }
    __syncthreads();
    if (it + 1 < n_iter) fetch(tile_of(it + 1) * kPfTile);

    // logits of 4 sub-tiles of 16 keys; one K read serves every query set
    f32x4_t s[QS][4];
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
#pragma unroll
      for (int u = 0; u < QS; ++u) s[u][sub] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(sm.k + (16 * sub + h) * S::KS + 32 * i + 8 * g);
#pragma unroll
        for (int u = 0; u < QS; ++u) s[u][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[u][i], s[u][sub], 0, 0, 0);
      }
    }
    // every pair of a tile below the diagonal is attended (for a streaming
    // head only if the tile is all sink); others are masked per token
    const bool full = key0 + kPfTile <= q_first && (!smask || key0 + kPfTile <= sink);
    float alpha[QS], mn[QS], psum[QS], nmc[QS];
#pragma unroll
    for (int u = 0; u < QS; ++u) {
      float tm = kNegInf;
#pragma unroll
      for (int sub = 0; sub < 4; ++sub)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!full) {
            const int key = key0 + 16 * sub + 4 * g + j;
            const bool ok = key <= iq[u] && key < L && (!smask || key < sink || key > iq[u] - local);
            if (!ok) s[u][sub][j] = kNegInf;
          }
          tm = fmaxf(tm, s[u][sub][j]);
        }
      tm = fmaxf(tm, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(tm), 0x401F)));  // lanes ^ 16
      tm = fmaxf(tm, shfl_xor_f(tm, 32));
      mn[u] = fmaxf(m[u], tm);
      nmc[u] = exp2_offset(mn[u], c);
      alpha[u] = (mn[u] == kNegInf) ? 1.0f : fast_exp2((m[u] - mn[u]) * c);
      if (__builtin_amdgcn_read_exec() & __ballot(alpha[u] != 1.0f)) {
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[u][n] *= alpha[u];
      }
      psum[u] = 0.0f;
    }
#pragma unroll
    for (int ch = 0; ch < 2; ++ch) {   // 32-key chunks: sub-tiles 2ch and 2ch + 1
      bf16x8_t bhi[QS], blo[QS];
#pragma unroll
      for (int u = 0; u < QS; ++u) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {  // words: keys (4g, 4g+1), (4g+2, 4g+3) of each sub-tile
          const int sub = 2 * ch + (x >> 1), j = 2 * (x & 1);
          const float p0 = exp2_fma(s[u][sub][j], c, nmc[u]), p1 = exp2_fma(s[u][sub][j + 1], c, nmc[u]);
          psum[u] += p0 + p1;
          hw[x] = pack_bf16(p0, p1);
          lw[x] = pack_bf16(p0 - bf_lo(hw[x]), p1 - bf_hi(hw[x]));
        }
        bhi[u] = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        blo[u] = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
      // A = V^T by transposed LDS reads (see the decode tile): lane 16k + m
      // addresses V[key0 + 4k + m/4][16n + 4(m%4) .. +3] of the chunk's
      // first 16 keys, then of its second; each read hands the lane the
      // 4 keys 4g + t of channel 16n + h
      const uint16_t* vt = sm.v + (32 * ch + 4 * g + ((lane & 15) >> 2)) * S::KS + 4 * (lane & 3);
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const s16x4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vt + 16 * n));
        const s16x4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(vt + 16 * S::KS + 16 * n));
        const uint2 a0 = __builtin_bit_cast(uint2, r0), a1 = __builtin_bit_cast(uint2, r1);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(a0.x, a0.y, a1.x, a1.y));
#pragma unroll
        for (int u = 0; u < QS; ++u) {
          acc[u][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhi[u], acc[u][n], 0, 0, 0);
          acc[u][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, blo[u], acc[u][n], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < QS; ++u) {
      lpart[u] = fmaf(lpart[u], alpha[u], psum[u]);
      m[u] = mn[u];
    }
  }

#pragma unroll
  for (int u = 0; u < QS; ++u) {
    float lt = lpart[u] + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(lpart[u]), 0x401F));
    lt += shfl_xor_f(lt, 32);
    if (iq[u] < L) {
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      float* orow = O + ((size_t)iq[u] * Hq + hq) * D;
#pragma unroll
      for (int n = 0; n < NB; ++n)
        *reinterpret_cast<float4*>(orow + 16 * n + 4 * g) =
            make_float4(acc[u][n][0] * inv, acc[u][n][1] * inv, acc[u][n][2] * inv, acc[u][n][3] * inv);
      if (g == 0) {
        lout[(size_t)iq[u] * Hq + hq] = lt;
        mout[(size_t)iq[u] * Hq + hq] = lt > 0.0f ? m[u] * scale : kNegInf;
      }
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
  constexpr int NWQ = DSA_PREFILL_WAVES, QS = DSA_PREFILL_QSETS, QT = 16 * QS * NWQ;
  const dim3 grid((L + QT - 1) / QT, n_q_heads);
  hipStream_t st = (hipStream_t)stream;
  if (head_dim == 128)
    hipLaunchKernelGGL((prefill_kernel<128, NWQ, QS>), grid, dim3(NWQ * 64), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (int)L, (int)n_q_heads, (int)n_kv_heads, (unsigned long long)smask, sink,
                       local, scale, c, O, l, m);
  else
    hipLaunchKernelGGL((prefill_kernel<64, NWQ, QS>), grid, dim3(NWQ * 64), 0, st, (const uint16_t*)q, (const uint16_t*)k,
                       (const uint16_t*)v, (int)L, (int)n_q_heads, (int)n_kv_heads, (unsigned long long)smask, sink,
                       local, scale, c, O, l, m);
  return launch_status();
}
