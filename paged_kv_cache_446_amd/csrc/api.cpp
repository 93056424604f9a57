// Status strings and pool sizing for libpkv.
#include "pkv.h"
#include "pkv_host.h"

extern "C" const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PKV_ERR_OUT_OF_BLOCKS: return "out of blocks";
    case PKV_ERR_REFCOUNT: return "reference count out of range";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" size_t pkv_pool_bytes(const pkv_cache_t* c) {
  if (!c || c->num_layers <= 0 || c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->head_dim <= 0)
    return 0;
  const int eb = pkv::elem_bytes(c->dtype);
  if (!eb) return 0;
  return (size_t)c->num_layers * (size_t)c->num_blocks * (size_t)c->num_kv_heads *
         (size_t)PKV_BLOCK_SIZE * (size_t)c->head_dim * (size_t)eb;
}
