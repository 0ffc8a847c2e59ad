// Host-side helpers of libdsa: argument validation and launch plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool pow2_group(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }

// Validates the pool descriptor; k/v are only checked when need_kv.
inline int check_kv(const dsa_kv* kv, bool need_kv) {
  if (!kv) return DSA_ERR_NULL;
  if (kv->dtype != DSA_F32 && kv->dtype != DSA_BF16) return DSA_ERR_DTYPE;
  if (kv->batch < 0 || kv->n_kv_heads < 1 || kv->max_pages < 1 || kv->num_slots < 0) return DSA_ERR_SHAPE;
  if (kv->page_size != 16 && kv->page_size != 32 && kv->page_size != 64) return DSA_ERR_UNSUPPORTED;
  if (kv->head_dim != 64 && kv->head_dim != 128) return DSA_ERR_UNSUPPORTED;
  if (kv->batch == 0) return DSA_OK;
  if (!kv->page_table || !kv->seq_lens) return DSA_ERR_NULL;
  if (need_kv) {
    if (!kv->k || !kv->v) return DSA_ERR_NULL;
    if (!aligned16(kv->k) || !aligned16(kv->v)) return DSA_ERR_ALIGN;
  }
  return DSA_OK;
}

inline int check_logical(const dsa_kv* kv, int logical_page) {
  if (logical_page < 16 || logical_page % 16 != 0 || logical_page > kv->page_size ||
      kv->page_size % logical_page != 0)
    return DSA_ERR_SHAPE;
  return DSA_OK;
}

// Streaming heads as a bit mask (bit h = KV head h streams).
inline int streaming_mask(const dsa_stream_cfg* st, int n_kv_heads, uint64_t* mask) {
  *mask = 0;
  if (!st || !st->kv_head_streaming) return DSA_OK;
  if (st->sink < 0 || st->local < 0) return DSA_ERR_SHAPE;
  for (int h = 0; h < n_kv_heads; ++h) {
    if (st->kv_head_streaming[h]) {
      if (h >= 64) return DSA_ERR_UNSUPPORTED;
      *mask |= (uint64_t)1 << h;
    }
  }
  return DSA_OK;
}

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace dsa
