// Shared device helpers of libdsa (gfx950, wave64).
//
// Lane layout used by every kernel that streams keys, values or metadata:
// a head_dim-long vector is covered by the 16 lanes of one DPP row, each
// lane holding CPL = head_dim/16 consecutive channels (8 B or 16 B of bf16,
// 16 B or 32 B of fp32).  A wave therefore holds 4 vectors per load, one per
// row, and consecutive lanes read consecutive bytes, so every wave-wide load
// is fully coalesced.  Reductions over a vector use DPP row operations; the
// 4 rows are combined with cross-row shuffles only when needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c with bf16 pairs packed in dwords (v_dot2_f32_bf16):
// the bf16 products are exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// ---------------------------------------------------------------- DPP
// Row = 16 consecutive lanes.  Partner patterns inside a row:
constexpr int DPP_ROW_MIRROR = 0x140;       // j <- j ^ 15
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // j <- j ^ 7
constexpr int DPP_QUAD_XOR3 = 0x1B;         // j <- j ^ 3   (quad_perm 3,2,1,0)
constexpr int DPP_QUAD_XOR1 = 0xB1;         // j <- j ^ 1   (quad_perm 1,0,3,2)
constexpr int DPP_ROW_ROR4 = 0x124;         // j <- (j + 4) & 15
constexpr int DPP_ROW_ROR8 = 0x128;         // j <- (j + 8) & 15

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

template <int N, int BIT, int CTRL>
__device__ __forceinline__ void rs_step(float* v, int j) {
  const bool up = (j >> BIT) & 1;
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float send = up ? v[k] : v[k + N / 2];
    const float keep = up ? v[k + N / 2] : v[k];
    v[k] = keep + dpp<CTRL>(send);
  }
}

// Sum NV values over the 16 lanes of each row (reduce-scatter).  Afterwards
// lane j of the row holds in v[0 .. max(1, NV/16)) the row totals of values
//   NV >= 16: [j*NV/16, (j+1)*NV/16)      NV == 8: j>>1      NV == 4: j>>2
// Each step pairs lanes that differ in one more bit (15, 7, 3, 1), keeping
// the half of the values selected by that bit of j.
template <int NV>
__device__ __forceinline__ void row_sum_scatter(float (&v)[NV], int j) {
  static_assert(NV == 4 || NV == 8 || NV == 16 || NV == 32 || NV == 64, "unsupported value count");
  rs_step<NV, 3, DPP_ROW_MIRROR>(v, j);
  if constexpr (NV / 2 >= 2) rs_step<NV / 2, 2, DPP_ROW_HALF_MIRROR>(v, j);
  else v[0] += dpp<DPP_ROW_HALF_MIRROR>(v[0]);
  if constexpr (NV / 4 >= 2) rs_step<NV / 4, 1, DPP_QUAD_XOR3>(v, j);
  else v[0] += dpp<DPP_QUAD_XOR3>(v[0]);
  if constexpr (NV / 8 >= 2) rs_step<NV / 8, 0, DPP_QUAD_XOR1>(v, j);
  else v[0] += dpp<DPP_QUAD_XOR1>(v[0]);
}

// All-reduce over the 16 lanes of a row.
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<DPP_ROW_MIRROR>(x);
  x += dpp<DPP_ROW_HALF_MIRROR>(x);
  x += dpp<DPP_QUAD_XOR3>(x);
  x += dpp<DPP_QUAD_XOR1>(x);
  return x;
}

// Row-wide max (all 16 lanes get it).
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, dpp<DPP_ROW_MIRROR>(x));
  x = fmaxf(x, dpp<DPP_ROW_HALF_MIRROR>(x));
  x = fmaxf(x, dpp<DPP_QUAD_XOR3>(x));
  return fmaxf(x, dpp<DPP_QUAD_XOR1>(x));
}

// DPP move whose lanes with no source in the row take `fill`.
template <int CTRL>
__device__ __forceinline__ float dpp_fill(float x, float fill) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Inclusive prefix sum / min over the 16 lanes of each row (row_shr 1, 2, 4, 8).
__device__ __forceinline__ float row_scan_sum(float x) {
  x += dpp_fill<0x111>(x, 0.0f);
  x += dpp_fill<0x112>(x, 0.0f);
  x += dpp_fill<0x114>(x, 0.0f);
  return x + dpp_fill<0x118>(x, 0.0f);
}
__device__ __forceinline__ float row_scan_min(float x) {
  const float inf = __builtin_huge_valf();
  x = fminf(x, dpp_fill<0x111>(x, inf));
  x = fminf(x, dpp_fill<0x112>(x, inf));
  x = fminf(x, dpp_fill<0x114>(x, inf));
  return fminf(x, dpp_fill<0x118>(x, inf));
}

// Max / sum over the 4 lanes j, j+4, j+8, j+12 of a row.
__device__ __forceinline__ float ror_max4(float x) {
  x = fmaxf(x, dpp<DPP_ROW_ROR4>(x));
  return fmaxf(x, dpp<DPP_ROW_ROR8>(x));
}
__device__ __forceinline__ float ror_sum4(float x) {
  x += dpp<DPP_ROW_ROR4>(x);
  return x + dpp<DPP_ROW_ROR8>(x);
}

// ---------------------------------------------------------------- wave scans
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xF, true);
}

// Inclusive prefix sum over the 64 lanes: shifts inside each row, then the
// last lane of row 0 (row 2) is added to row 1 (row 3) and the last lane of
// row 1 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_i<0x111>(x);        // row_shr:1
  x += dpp_i<0x112>(x);        // row_shr:2
  x += dpp_i<0x114>(x);        // row_shr:4
  x += dpp_i<0x118>(x);        // row_shr:8
  x += dpp_i<0x142, 0xA>(x);   // row_bcast:15 into rows 1, 3
  x += dpp_i<0x143, 0xC>(x);   // row_bcast:31 into rows 2, 3
  return x;
}

// Min / max of a uint32 over the wave, returned to every lane.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  x = min(x, (uint32_t)dpp_i<DPP_ROW_MIRROR>((int)x));
  x = min(x, (uint32_t)dpp_i<DPP_ROW_HALF_MIRROR>((int)x));
  x = min(x, (uint32_t)dpp_i<DPP_QUAD_XOR3>((int)x));
  x = min(x, (uint32_t)dpp_i<DPP_QUAD_XOR1>((int)x));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return min(min(a, b), min(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)dpp_i<DPP_ROW_MIRROR>((int)x));
  x = max(x, (uint32_t)dpp_i<DPP_ROW_HALF_MIRROR>((int)x));
  x = max(x, (uint32_t)dpp_i<DPP_QUAD_XOR3>((int)x));
  x = max(x, (uint32_t)dpp_i<DPP_QUAD_XOR1>((int)x));
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return max(max(a, b), max(c, d));
}

// Orders this wave's LDS writes before its later LDS reads (a wave's LDS
// operations complete in issue order; this keeps the compiler from moving
// them across the point).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) { return __shfl_xor(x, mask, 64); }

// 2^x on the transcendental unit (v_exp_f32; results below 2^-126 may
// flush to zero, which is below any tolerance here).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2 that maps the empty-set case (both operands -inf) to 0.
__device__ __forceinline__ float exp2_diff(float a, float m, float c) {
  return (m == kNegInf) ? 0.0f : fast_exp2((a - m) * c);
}

// The same weight as one fused multiply-add: 2^(a c + nmc) with
// nmc = exp2_offset(m, c) = -m c (0 when m = -inf, where every a is -inf).
__device__ __forceinline__ float exp2_offset(float m, float c) { return (m == kNegInf) ? 0.0f : -m * c; }
__device__ __forceinline__ float exp2_fma(float a, float c, float nmc) { return fast_exp2(fmaf(a, c, nmc)); }

// ---------------------------------------------------------------- layout
template <typename T, int D>
struct Lay {
  static constexpr int CPL = D / 16;                        // channels per lane
  static constexpr int DW = CPL * (int)sizeof(T) / 4;       // dwords per lane per vector
  static_assert(DW == 2 || DW == 4 || DW == 8, "unsupported layout");
};

// Load DW dwords at p (16-byte aligned when DW >= 4, 8-byte when DW == 2).
template <int DW>
__device__ __forceinline__ void load_dw(const void* p, uint32_t* out) {
  if constexpr (DW == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    out[0] = x.x; out[1] = x.y;
  } else {
#pragma unroll
    for (int u = 0; u < DW / 4; ++u) {
      const uint4 x = reinterpret_cast<const uint4*>(p)[u];
      out[4 * u + 0] = x.x; out[4 * u + 1] = x.y; out[4 * u + 2] = x.z; out[4 * u + 3] = x.w;
    }
  }
}

// Non-temporal variants for data read once per call (page metadata, the
// K/V rows of selected pages): the loads carry the streaming cache hint, so
// they do not displace reused lines, and HBM serves them at a higher rate.
using u32x2_t = unsigned int __attribute__((ext_vector_type(2)));
using u32x4_t = unsigned int __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x.x, x.y, x.z, x.w);
}
#ifndef DSA_KV_NT
#define DSA_KV_NT 1  // 1: K/V rows of selected pages load with the non-temporal hint
#endif
template <int DW>
__device__ __forceinline__ void load_dw_stream(const void* p, uint32_t* out) {
  if constexpr (DW == 2) {
    const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    out[0] = x.x; out[1] = x.y;
  } else {
#pragma unroll
    for (int u = 0; u < DW / 4; ++u) {
      const uint4 x = ld16_stream(reinterpret_cast<const uint4*>(p) + u);
      out[4 * u + 0] = x.x; out[4 * u + 1] = x.y; out[4 * u + 2] = x.z; out[4 * u + 3] = x.w;
    }
  }
}

// Loads of K/V rows.
template <int DW>
__device__ __forceinline__ void load_dw_kv(const void* p, uint32_t* out) {
#if DSA_KV_NT
  load_dw_stream<DW>(p, out);
#else
  load_dw<DW>(p, out);
#endif
}
__device__ __forceinline__ uint4 ld16_kv(const void* p) {
#if DSA_KV_NT
  return ld16_stream(p);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

// Channel c (0 <= c < CPL) of a lane's raw dwords as float.
template <typename T>
__device__ __forceinline__ float chan(const uint32_t* w, int c) {
  if constexpr (sizeof(T) == 2) return (c & 1) ? bf_hi(w[c >> 1]) : bf_lo(w[c >> 1]);
  else return __uint_as_float(w[c]);
}

// Dot product of a lane's CPL channels of a key with the same channels of q
// (stored the same way as the key).
template <typename T, int DW>
__device__ __forceinline__ float lane_dot(const uint32_t* k, const uint32_t* q) {
  float acc = 0.0f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int x = 0; x < DW; ++x) acc = dot2_bf16(k[x], q[x], acc);
  } else {
#pragma unroll
    for (int x = 0; x < DW; ++x) acc = fmaf(__uint_as_float(k[x]), __uint_as_float(q[x]), acc);
  }
  return acc;
}

// One EMA step of PRR's predictor ("Predict, Reuse, and Repair", section
// 3.1): trend and level both read the previous level; the prediction
// extrapolates the new level by gamma times the new trend.  Every product
// and sum is rounded to fp32 on its own (no fused multiply-add), in this
// order, so that any kernel -- and a float32 reference -- rounds the
// predictor the same way:
//   trend' = beta*(IS - level) + (1 - beta)*trend
//   level' = alpha*IS + (1 - alpha)*level
//   pred   = level' + gamma*trend'
__device__ __forceinline__ float ema_predict(float lv, float tr, float gamma) {
#pragma clang fp contract(off)
  return lv + gamma * tr;
}

__device__ __forceinline__ void ema_step(float is, float lv, float tr, float alpha, float beta, float gamma,
                                         float& nl, float& nt, float& pr) {
#pragma clang fp contract(off)
  nt = beta * (is - lv) + (1.0f - beta) * tr;
  nl = alpha * is + (1.0f - alpha) * lv;
  pr = ema_predict(nl, nt, gamma);
}

__device__ __forceinline__ int clamp_len(int L, int max_pages, int P) {
  const long long cap = (long long)max_pages * P;
  return L < 0 ? 0 : (L > cap ? (int)cap : L);
}

}  // namespace dsa
