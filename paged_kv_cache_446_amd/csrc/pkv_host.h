// Host-side argument checks shared by the libpkv entry points.
#pragma once

#include <stdint.h>

#include "pkv.h"

namespace pkv {

inline int elem_bytes(int32_t dtype) {
  return dtype == PKV_F32 ? 4 : (dtype == PKV_F16 || dtype == PKV_BF16) ? 2 : 0;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shapes the kernels are built for.
inline bool supported_head_dim(int32_t d) { return d == 64 || d == 128 || d == 256; }

inline int check_cache(const pkv_cache_t* c) {
  if (!c || !c->k_pool || !c->v_pool) return PKV_ERR_INVALID_ARGUMENT;
  if (c->num_layers <= 0 || c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
    return PKV_ERR_INVALID_ARGUMENT;
  if (elem_bytes(c->dtype) == 0) return PKV_ERR_UNSUPPORTED;
  if (!supported_head_dim(c->head_dim)) return PKV_ERR_UNSUPPORTED;
  if (!aligned16(c->k_pool) || !aligned16(c->v_pool)) return PKV_ERR_INVALID_ARGUMENT;
  return PKV_OK;
}

}  // namespace pkv
