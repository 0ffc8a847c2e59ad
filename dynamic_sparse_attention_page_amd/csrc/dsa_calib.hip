// PRR online predictor calibration ("Predict, Reuse, and Repair", section
// 3.2 of the page, the paper's section 4.2): the EMA hyper-parameters
// (alpha, beta, gamma) are chosen per prompt from a score trace by the
// score-weighted hit rate
//   H(theta) = mean over predicted steps phi of
//              sum_{b in P_phi(theta) & A_phi} IS_phi,b / sum_{b in A_phi} IS_phi,b
// over the printed grid alpha in {0.2 .. 0.8}, beta in {0.1 .. 0.5},
// gamma in {0 .. 0.75}: 80 candidates, searched exhaustively.
//
// calib_actual_kernel: one workgroup per (predicted step, unit) selects
//   A_phi = top-k of the true scores (the selection of dsa_page_select_topk)
//   and stores it as a bitmap (one ballot word per element slot and wave)
//   with its total weight.
// calib_kernel: one workgroup per (candidate, unit) carries the EMA state of
//   its unit through the trace -- in registers up to 8 elements per thread,
//   above that in a workspace slice of its own (a 1024-thread workgroup has
//   128 registers per thread) -- and per step predicts, absorbs the step's
//   scores (the update does not depend on P, so only the keys stay live
//   across the selection), selects P_phi = top-m of the prediction and
//   weighs P & A against the bitmap, reloading the scores it needs.
// calib_best_kernel: argmax over the candidates, lowest index on ties.
#include "dsa_host.hpp"
#include "dsa_select.hpp"

namespace dsa {

constexpr int kCalibCandidates = 80;

// Candidate c of the grid: alpha slowest, gamma fastest.
__device__ __forceinline__ void calib_theta(int c, float& alpha, float& beta, float& gamma) {
  const int ia = c / 20, ib = (c / 4) % 5, ig = c % 4;
  alpha = ia == 0 ? 0.2f : ia == 1 ? 0.4f : ia == 2 ? 0.6f : 0.8f;
  beta = ib == 0 ? 0.1f : ib == 1 ? 0.2f : ib == 2 ? 0.3f : ib == 3 ? 0.4f : 0.5f;
  gamma = 0.25f * (float)ig;
}

// Raw buffer over [p, p + bytes): loads past the end return 0, and every
// access of a thread shares one offset register (element slots differ by a
// scalar offset), so per-element addresses never occupy registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf(const void* p, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float ld_f32(__amdgpu_buffer_rsrc_t b, int vo, int so) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(b, vo, so, 0));
}

__device__ __forceinline__ void st_f32(float x, __amdgpu_buffer_rsrc_t b, int vo, int so) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), b, vo, so, 0);
}

// Block sum of one float per thread in a fixed order (wave trees, then the
// waves in index order); the total is returned to every thread.
template <int NW>
__device__ __forceinline__ float block_sum_f32(float x, float* smem /* NW */) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s, 64);
  if constexpr (NW == 1) {
    return x;
  } else {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) smem[wave] = x;
    __syncthreads();
    float t = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += smem[w];
    __syncthreads();
    return t;
  }
}

template <int E, int NW>
__global__ __launch_bounds__(NW * 64) void calib_actual_kernel(const float* __restrict__ trace, int units, int N,
                                                                 const int32_t* __restrict__ n_valid, int k,
                                                                 unsigned long long* __restrict__ a_bits,
                                                                 float* __restrict__ a_weight) {
  constexpr int NT = NW * 64;
  __shared__ SelectSmem<E, NW> sm;
  __shared__ float red[NW];
  const int phi = blockIdx.x + 1, u = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nv = min(max(n_valid[u], 0), N);
  const float* row = trace + ((size_t)phi * units + u) * N;
  uint32_t key[E];
  unsigned long long actm = 0ull;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    key[e] = order_key((e * NT + tid < N) ? row[e * NT + tid] : 0.0f);
    if (e * NT + tid < nv) actm |= 1ull << e;
  }
  const unsigned long long selm = block_select_top<E, NW>(key, actm, nv, min(k, nv), sm);
  unsigned long long* bits = a_bits + ((size_t)blockIdx.x * units + u) * (E * NW);
  float w = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool in = (selm >> e) & 1ull;
    const unsigned long long word = __ballot(in);   // elements e*NT + wave*64 + [0, 64)
    if (lane == 0) bits[e * NW + wave] = word;
    w += in ? key_value(key[e]) : 0.0f;   // the score itself (a -0 comes back as +0)
  }
  const float total = block_sum_f32<NW>(w, red);
  if (tid == 0) a_weight[(size_t)blockIdx.x * units + u] = total;
}

template <int E, int NW>
__global__ __launch_bounds__(NW * 64) void calib_kernel(const float* __restrict__ trace, int T, int units, int N,
                                                          const int32_t* __restrict__ n_valid, int m,
                                                          const unsigned long long* __restrict__ a_bits,
                                                          const float* __restrict__ a_weight, float* __restrict__ H,
                                                          float* __restrict__ state) {
  constexpr int NT = NW * 64;
  constexpr bool kRegs = E <= 8;   // state in registers, else in `state`
  __shared__ SelectSmem<E, NW> sm;
  __shared__ float red[NW];
  const int c = blockIdx.x, u = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float alpha, beta, gamma;
  calib_theta(c, alpha, beta, gamma);
  const int nv = min(max(n_valid[u], 0), N);
  unsigned long long actm = 0ull;
  constexpr int ER = kRegs ? E : 1;
  float lv[ER], tr[ER];
  const float* row0 = trace + (size_t)u * N;
  // this workgroup's state slice: level then trend, NT * E floats each
  float* s_lv = state + ((size_t)u * kCalibCandidates + c) * 2 * (E * NT);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if constexpr (kRegs) {
      lv[e] = (e * NT + tid < N) ? row0[e * NT + tid] : 0.0f;   // level = IS_0, trend = 0
      tr[e] = 0.0f;
    }
    if (e * NT + tid < nv) actm |= 1ull << e;
  }
  double acc = 0.0;
  const int vo = tid * 4;   // byte offset of this thread's element in every slot
  const auto bs = buf(s_lv, (size_t)2 * E * NT * sizeof(float));
  const auto b0 = buf(row0, (size_t)N * sizeof(float));
  for (int phi = 1; phi < T; ++phi) {
    const auto br = buf(trace + ((size_t)phi * units + u) * N, (size_t)N * sizeof(float));
    uint32_t key[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float is = ld_f32(br, vo, e * NT * 4);
      float l, tt;
      if constexpr (kRegs) {
        l = lv[e];
        tt = tr[e];
      } else if (phi == 1) {   // level = IS_0, trend = 0
        l = ld_f32(b0, vo, e * NT * 4);
        tt = 0.0f;
      } else {
        l = ld_f32(bs, vo, e * NT * 4);
        tt = ld_f32(bs, vo, (E + e) * NT * 4);
      }
      key[e] = order_key(ema_predict(l, tt, gamma));
      float pr;
      ema_step(is, l, tt, alpha, beta, gamma, l, tt, pr);
      if constexpr (kRegs) {
        lv[e] = l;
        tr[e] = tt;
      } else {
        st_f32(l, bs, vo, e * NT * 4);
        st_f32(tt, bs, vo, (E + e) * NT * 4);
      }
    }
    const unsigned long long selm = block_select_top<E, NW>(key, actm, nv, min(m, nv), sm);
    const unsigned long long* bits = a_bits + ((size_t)(phi - 1) * units + u) * (E * NW);
    float hit = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      // loads only under the selection: nothing of this loop stays live
      // across block_select_top (a set bit implies a valid element)
      if ((selm >> e) & 1ull) {
        if ((bits[e * NW + wave] >> lane) & 1ull) hit += ld_f32(br, vo, e * NT * 4);
      }
    }
    const float total = block_sum_f32<NW>(hit, red);   // also separates the selections
    const float den = a_weight[(size_t)(phi - 1) * units + u];
    acc += den == 0.0f ? 1.0 : (double)total / (double)den;
  }
  if (tid == 0) H[(size_t)u * kCalibCandidates + c] = (float)(acc / (double)(T - 1));
}

__global__ __launch_bounds__(64) void calib_best_kernel(const float* __restrict__ H, int32_t* __restrict__ best) {
  const int u = blockIdx.x, lane = threadIdx.x;
  const float* h = H + (size_t)u * kCalibCandidates;
  float v = h[lane];
  int i = lane;
  if (lane + 64 < kCalibCandidates && h[lane + 64] > v) { v = h[lane + 64]; i = lane + 64; }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const float ov = __shfl_xor(v, s, 64);
    const int oi = __shfl_xor(i, s, 64);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
  if (lane == 0) best[u] = i;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Capacity (elements per row) of the <E, NW> workgroup chosen for n.
inline int calib_capacity(int n) {
  int cap = 256;
  while (cap < n) cap <<= 1;
  return cap;
}

template <int E, int NW>
static int launch_calib(const float* trace, int T, int units, int N, const int32_t* n_valid, int k, int m, float* H,
                        int32_t* best, unsigned long long* a_bits, float* a_weight, float* state, hipStream_t st) {
  static_assert(E * NW * 64 >= 256, "capacity");
  hipLaunchKernelGGL((calib_actual_kernel<E, NW>), dim3(T - 1, units), dim3(NW * 64), 0, st, trace, units, N,
                     n_valid, k, a_bits, a_weight);
  int rc = launch_status();
  if (rc) return rc;
  hipLaunchKernelGGL((calib_kernel<E, NW>), dim3(kCalibCandidates, units), dim3(NW * 64), 0, st, trace, T, units, N,
                     n_valid, m, a_bits, a_weight, H, state);
  if ((rc = launch_status())) return rc;
  if (best) {
    hipLaunchKernelGGL(calib_best_kernel, dim3(units), dim3(64), 0, st, H, best);
    rc = launch_status();
  }
  return rc;
}

}  // namespace dsa

using namespace dsa;

// Workspace: A bitmaps, A weights, and for rows above 8192 elements the
// EMA state of every (unit, candidate) workgroup.
struct CalibWs {
  size_t bits, weight, state, total;
};

inline CalibWs calib_ws(int steps, int units, int n) {
  const size_t rows = (size_t)(steps - 1) * units;
  const size_t cap = (size_t)calib_capacity(n);
  CalibWs w;
  w.bits = 0;
  w.weight = align256(rows * (cap / 64) * sizeof(unsigned long long));
  w.state = w.weight + align256(rows * sizeof(float));
  w.total = w.state + (n > 8192 ? (size_t)units * kCalibCandidates * 2 * cap * sizeof(float) : 0);
  return w;
}

extern "C" size_t dsa_prr_calibrate_workspace_bytes(int32_t steps, int32_t units, int32_t n) {
  if (steps < 2 || units < 0 || n < 1 || n > 65536) return 0;
  return calib_ws(steps, units, n).total;
}

extern "C" int dsa_prr_calibrate(const float* trace, int32_t steps, int32_t units, int32_t n,
                                 const int32_t* n_valid, int32_t k, int32_t m, float* H, int32_t* best, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (steps < 2 || units < 0 || n < 1 || k < 0 || m < 0) return DSA_ERR_SHAPE;
  if (n > 65536) return DSA_ERR_UNSUPPORTED;
  if (units == 0) return DSA_OK;
  if (!trace || !n_valid || !H) return DSA_ERR_NULL;
  const CalibWs w = calib_ws(steps, units, n);
  if (!ws || ws_bytes < w.total) return DSA_ERR_WORKSPACE;
  unsigned long long* a_bits = (unsigned long long*)((char*)ws + w.bits);
  float* a_weight = (float*)((char*)ws + w.weight);
  float* state = (float*)((char*)ws + w.state);
  hipStream_t st = (hipStream_t)stream;
#define DSA_CAL(E, NW) \
  return launch_calib<E, NW>(trace, steps, units, n, n_valid, k, m, H, best, a_bits, a_weight, state, st)
  if (n <= 256) DSA_CAL(4, 1);
  if (n <= 512) DSA_CAL(8, 1);
  if (n <= 1024) DSA_CAL(4, 4);
  if (n <= 2048) DSA_CAL(8, 4);
  if (n <= 4096) DSA_CAL(8, 8);
  if (n <= 8192) DSA_CAL(8, 16);
  if (n <= 16384) DSA_CAL(16, 16);
  if (n <= 32768) DSA_CAL(32, 16);
  DSA_CAL(64, 16);
#undef DSA_CAL
}
