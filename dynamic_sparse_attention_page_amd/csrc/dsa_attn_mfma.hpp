// Online-softmax attention over 16-token KV tiles on the matrix cores, for
// KV groups of 8 or 16 q heads with bf16 KV (one wave).
//
// The recurrence is the one of the VALU path (PRR, "Predict, Reuse, and
// Repair", section 3.3: running max, rescale by exp(m - m_new), add the
// block's exp(s - m_new) terms); only the two contractions move to MFMA.
// With 8+ heads per KV head the 16 x 16 logit tile and the 16 x D output
// update are dense enough for the matrix cores.
//
// Layouts (16 x 16 MFMA blocks; lane l, h = l % 16, g = l / 16):
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16 over D/32 channel steps.
//                 A = K: lane holds K[token h][channels 32i + 8g, +8)
//                 B = Q^T: lane holds Q[head h][same channels]
//                 result: lane holds S[head h][tokens 4g + j], j < 4
//   O^T += V^T P^T  v_mfma_f32_16x16x32_bf16, one per 16-channel block n,
//                 the K dimension holding P's bf16 hi parts then its lo parts.
//                 A = V^T: lane holds V[tokens 4g + j][channel 16n + h], twice
//                 B = P^T: lane holds P[head h][tokens 4g + j] (hi, then lo)
//                 -- exactly the logit layout, so the softmax stays lane-local
//                 result: lane holds O[head h][channels 16n + 4g + j]
// Softmax statistics of head h live in lanes h, h+16, h+32, h+48; the tile
// max needs two lane swaps.  V^T comes from the row-major LDS copy of the
// tile through transposed LDS reads.  P enters the product as bf16 hi + lo
// parts, so the weights keep ~16 mantissa bits; one 32-deep product takes
// both.
#pragma once

#include "dsa_common.hpp"

namespace dsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Two floats to packed bf16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int D, int G>
struct MfmaWave {
  static_assert(G == 8 || G == 16, "matrix-core path is for 8 or 16 heads per KV head");
  static_assert(D == 64 || D == 128, "head_dim");
  static constexpr int NK = D / 32;   // QK^T steps; also 16-byte loads per lane per K or V tile
  static constexpr int NB = D / 16;   // 16-channel output blocks
  static constexpr int VS = D + 8;    // LDS row stride of the V tile (bf16): spreads the 4 token rows of a read over banks
  static constexpr int LDS_ELEMS = 16 * VS;

  int h, g;
  bf16x8_t qb[NK];
  f32x4_t acc[NB];
  float m;      // running max of head h, raw q.k
  float lpart;  // this lane's part of head h's denominator
  uint16_t* vs; // this wave's V tile in LDS

  __device__ __forceinline__ void init(const uint16_t* __restrict__ q_heads /* [G][D] */, uint16_t* lds) {
    const int lane = threadIdx.x & 63;
    h = lane & 15;
    g = lane >> 4;
    vs = lds;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (h < G) w = *reinterpret_cast<const uint4*>(q_heads + (size_t)h * D + 32 * i + 8 * g);
      qb[i] = __builtin_bit_cast(bf16x8_t, w);
    }
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[n] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m = kNegInf;
    lpart = 0.0f;
  }

  // K in the MFMA A layout: token h, channels 32i + 8g.
  __device__ __forceinline__ static void load_k(const uint16_t* __restrict__ tile, int lane, uint4 (&kd)[NK]) {
    const int hh = lane & 15, gg = lane >> 4;
#pragma unroll
    for (int i = 0; i < NK; ++i) kd[i] = ld16_kv(tile + (size_t)hh * D + 32 * i + 8 * gg);
  }
  // V flat: 16-byte chunk lane + 64i of the tile (fully coalesced).
  __device__ __forceinline__ static void load_v(const uint16_t* __restrict__ tile, int lane, uint4 (&vd)[NK]) {
#pragma unroll
    for (int i = 0; i < NK; ++i) vd[i] = ld16_kv(reinterpret_cast<const uint4*>(tile) + lane + 64 * i);
  }

  __device__ __forceinline__ static bool tok_ok(int t, int nvalid, bool smask, int tok0, int L, int sink,
                                                int local) {
    bool ok = t < nvalid;
    if (smask) {
      const int gt = tok0 + t;
      ok = ok && (gt < sink || gt >= L - local);
    }
    return ok;
  }

  __device__ __forceinline__ void tile(const uint4 (&kd)[NK], const uint4 (&vd)[NK], int nvalid, bool smask,
                                       int tok0, int L, int sink, int local, float c) {
    const int lane = threadIdx.x & 63;
    // stage V in LDS (row-major, padded rows) while the logits are formed
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int chunk = lane + 64 * i;               // 16-byte chunk of the tile
      const int row = chunk / (D / 8), col = (chunk % (D / 8)) * 8;
      const uint4 x = vd[i];
      uint32_t* dst = reinterpret_cast<uint32_t*>(vs + row * VS + col);
      dst[0] = x.x; dst[1] = x.y; dst[2] = x.z; dst[3] = x.w;
    }
    f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < NK; ++i)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kd[i]), qb[i], s, 0, 0, 0);
    bool ok[4] = {true, true, true, true};
    const bool partial = nvalid < 16 || smask;   // uniform: full tiles skip the token mask
    if (partial) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ok[j] = tok_ok(4 * g + j, nvalid, smask, tok0, L, sink, local);
        if (!ok[j]) s[j] = kNegInf;
      }
    }
    float tm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    tm = fmaxf(tm, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(tm), 0x401F)));  // lanes ^ 16
    tm = fmaxf(tm, shfl_xor_f(tm, 32));
    const float mn = fmaxf(m, tm);
    const float alpha = (mn == kNegInf) ? 1.0f : fast_exp2((m - mn) * c);
    float p[4];
    const float nmc = exp2_offset(mn, c);
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = exp2_fma(s[j], c, nmc);
    lpart = fmaf(lpart, alpha, (p[0] + p[1]) + (p[2] + p[3]));
    m = mn;
    // P^T as bf16 hi + lo
    const uint32_t h01 = pack_bf16(p[0], p[1]), h23 = pack_bf16(p[2], p[3]);
    const uint32_t l01 = pack_bf16(p[0] - bf_lo(h01), p[1] - bf_hi(h01));
    const uint32_t l23 = pack_bf16(p[2] - bf_lo(h23), p[3] - bf_hi(h23));
    // B of one 16x16x32 product per channel block: k = 8g + j holds the hi
    // part of key 4g + j (j < 4), then its lo part (j >= 4); A repeats the
    // lane's 4 V values, so the product adds V (P_hi + P_lo)
    const bf16x8_t bhl = __builtin_bit_cast(bf16x8_t, make_uint4(h01, h23, l01, l23));
    if (__builtin_amdgcn_read_exec() & __ballot(alpha != 1.0f)) {   // skip once the maxima settle
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] *= alpha;
    }
    // masked tokens' V may be non-finite garbage: keep 0 * v finite
    uint32_t keep01 = 0xFFFFFFFFu, keep23 = 0xFFFFFFFFu;
    if (partial) {
      keep01 = (ok[0] ? 0x0000FFFFu : 0u) | (ok[1] ? 0xFFFF0000u : 0u);
      keep23 = (ok[2] ? 0x0000FFFFu : 0u) | (ok[3] ? 0xFFFF0000u : 0u);
    }
    wave_sync();
    // A = V^T by transposed LDS reads: lane 16k + m addresses the 4 values
    // V[4k + m/4][16n + 4(m%4) .. +3] of the row-major tile, and the read
    // hands lane 16k + 4a + b the b-th value of the blocks of lanes 16k + a +
    // 4t (t < 4): V[4k + t][16n + 4a + b], i.e. channel 16n + h of keys 4g + t
    const int lane16 = lane & 15;
    const uint16_t* vt = vs + (4 * g + (lane16 >> 2)) * VS + 4 * (lane16 & 3);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const s16x4_t raw = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(vt + 16 * n));
      const uint2 w = __builtin_bit_cast(uint2, raw);
      const uint32_t a01 = w.x & keep01, a23 = w.y & keep23;
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(a01, a23, a01, a23));
      acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bhl, acc[n], 0, 0, 0);
    }
    wave_sync();   // the next tile rewrites the LDS copy
  }

  // Denominator of head h over the whole wave (all four lanes of h get it).
  __device__ __forceinline__ float total_l() const {
    float x = lpart;
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
    return x + shfl_xor_f(x, 32);
  }
};

}  // namespace dsa
