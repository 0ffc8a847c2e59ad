// PRR EMA page-score predictor ("Predict, Reuse, and Repair", section 3.1).
// Per block: a smoothed level and a trend; the prediction extrapolates the
// level by gamma times the trend, and an observed score updates trend and
// level, both from the previous level.  Elementwise and HBM-bound: 16-byte
// vector loads/stores over the flat arrays, scalar tail.
#include "dsa_common.hpp"
#include "dsa_host.hpp"

namespace dsa {

__device__ __forceinline__ void ema_one(const float* is_true, float* level, float* trend, float* pred, long long x,
                                        float alpha, float beta, float gamma, int init) {
  if (!is_true) {
    pred[x] = ema_predict(level[x], trend[x], gamma);
    return;
  }
  const float is = is_true[x];
  if (init) {
    level[x] = is;
    trend[x] = 0.0f;
    pred[x] = is;
    return;
  }
  float nl, nt, pr;
  ema_step(is, level[x], trend[x], alpha, beta, gamma, nl, nt, pr);
  level[x] = nl;
  trend[x] = nt;
  pred[x] = pr;
}

__global__ __launch_bounds__(256) void ema_kernel(const float* __restrict__ is_true, float* __restrict__ level,
                                                  float* __restrict__ trend, float* __restrict__ pred, long long n,
                                                  float alpha, float beta, float gamma, int init, int vec) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (vec) {
    const long long n4 = n / 4;
    for (long long x = i; x < n4; x += stride) {
      float4 lv = reinterpret_cast<float4*>(level)[x];
      float4 tr = reinterpret_cast<float4*>(trend)[x];
      float4 pr;
      if (!is_true) {
        pr = make_float4(ema_predict(lv.x, tr.x, gamma), ema_predict(lv.y, tr.y, gamma),
                         ema_predict(lv.z, tr.z, gamma), ema_predict(lv.w, tr.w, gamma));
      } else {
        const float4 is = reinterpret_cast<const float4*>(is_true)[x];
        if (init) {
          lv = is;
          tr = make_float4(0.f, 0.f, 0.f, 0.f);
          pr = is;
        } else {
          ema_step(is.x, lv.x, tr.x, alpha, beta, gamma, lv.x, tr.x, pr.x);
          ema_step(is.y, lv.y, tr.y, alpha, beta, gamma, lv.y, tr.y, pr.y);
          ema_step(is.z, lv.z, tr.z, alpha, beta, gamma, lv.z, tr.z, pr.z);
          ema_step(is.w, lv.w, tr.w, alpha, beta, gamma, lv.w, tr.w, pr.w);
        }
        reinterpret_cast<float4*>(level)[x] = lv;
        reinterpret_cast<float4*>(trend)[x] = tr;
      }
      reinterpret_cast<float4*>(pred)[x] = pr;
    }
    for (long long x = n4 * 4 + i; x < n; x += stride) ema_one(is_true, level, trend, pred, x, alpha, beta, gamma, init);
  } else {
    for (long long x = i; x < n; x += stride) ema_one(is_true, level, trend, pred, x, alpha, beta, gamma, init);
  }
}

}  // namespace dsa

using namespace dsa;

extern "C" int dsa_ema_predict_update(const float* is_true, float* level, float* trend, float* pred, int64_t n,
                                      float alpha, float beta, float gamma, int32_t init, void* stream) {
  if (n < 0) return DSA_ERR_SHAPE;
  if (n == 0) return DSA_OK;
  if (!level || !trend || !pred) return DSA_ERR_NULL;
  if (pred == level || pred == trend) return DSA_ERR_SHAPE;
  const int vec = aligned16(level) && aligned16(trend) && aligned16(pred) && (!is_true || aligned16(is_true));
  long long blocks = (n / (vec ? 4 : 1) + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(ema_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, is_true, level, trend,
                     pred, (long long)n, alpha, beta, gamma, (int)init, vec);
  return launch_status();
}
