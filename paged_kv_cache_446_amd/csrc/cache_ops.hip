// kv_cache_write and copy_blocks for gfx950.
//
// kv_cache_write: each token processed appends one K entry and one V entry to
// the cache (devpress.csdn.net/amd/6a408ab810ee7a33f2834f35.html, prefill /
// decode / KV cache section).  copy_blocks: copy-on-write copies a shared
// block before a sequence modifies it and leaves the original as it was
// (blog.mckayzhao.com/?p=56, copy-on-write section).  Both are plain byte
// movement: bit-exact, no arithmetic on the data.
#include <hip/hip_runtime.h>

#include "pkv.h"
#include "pkv_device.h"
#include "pkv_host.h"

namespace pkv {

// One workgroup per token.  K: every 16-byte run of head dims stays contiguous
// in the tile (chunk (d/x) of token t sits at ((d/x)*16 + t)*x), so it is one
// 16-byte load and one 16-byte store.  V: four consecutive tokens of a dim
// are adjacent in the tile, so a single token's V entry is a strided scatter
// of elements.
template <int kBytes>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const u32x4* __restrict__ k_new, const void* __restrict__ v_new,
    const int64_t* __restrict__ slots, u32x4* __restrict__ k_pool, void* __restrict__ v_pool,
    int num_kv_heads, int head_dim, int64_t layer_elems) {
  typedef typename std::conditional<kBytes == 2, uint16_t, uint32_t>::type E;
  constexpr int x = 16 / kBytes;
  constexpr int x4 = x / 4;
  const int64_t tok = blockIdx.x;
  const int64_t slot = slots[tok];
  if (slot < 0) return;
  const int64_t blk = slot / kBlock;
  const int pos = (int)(slot % kBlock);
  const int chunks = head_dim / x;  // 16-byte chunks per (token, head)
  const int64_t tile = (int64_t)kBlock * head_dim;
  const int64_t blk_base = layer_elems + blk * num_kv_heads * tile;  // in elements
  // K: 16-byte chunks
  for (int i = threadIdx.x; i < num_kv_heads * chunks; i += blockDim.x) {
    const int h = i / chunks, ch = i - h * chunks;
    const u32x4 v = k_new[(tok * num_kv_heads + h) * chunks + ch];
    const int64_t dst = blk_base + h * tile + ((int64_t)ch * kBlock + pos) * x;  // elements
    k_pool[dst / x] = v;
  }
  // V: elements
  const E* vsrc = (const E*)v_new + tok * num_kv_heads * head_dim;
  E* vdst = (E*)v_pool;
  const int g = pos >> 2, j = pos & 3;
  for (int i = threadIdx.x; i < num_kv_heads * head_dim; i += blockDim.x) {
    const int h = i / head_dim, d = i - h * head_dim;
    const int n = d >> 4, c = d & 15, m = n / x4, r = n - m * x4;
    const int64_t off = ((((int64_t)m * 4 + g) * 16 + c) * x4 + r) * 4 + j;
    vdst[blk_base + h * tile + off] = vsrc[i];
  }
}

// grid (pair, layer, K|V): copy one block of one layer of one pool.  A block's
// source and destination never overlap (distinct blocks), so each thread issues
// all loads of a round before its stores: one memory round trip per kCopyBatch
// chunks instead of one per chunk.  Loads and stores are unconditional: a lane
// past the block's end copies its last chunk again (the same bytes to the same
// place).
constexpr int kCopyBatch = 8;

__global__ __launch_bounds__(256) void copy_blocks_kernel(const int32_t* __restrict__ pairs,
                                                          u32x4* __restrict__ k_pool,
                                                          u32x4* __restrict__ v_pool,
                                                          int64_t block_chunks,
                                                          int64_t layer_chunks) {
  const int p = blockIdx.x;
  const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  u32x4* pool = blockIdx.z ? v_pool : k_pool;
  const int64_t base = blockIdx.y * layer_chunks;
  const u32x4* __restrict__ s = pool + base + src * block_chunks;
  u32x4* __restrict__ d = pool + base + dst * block_chunks;
  for (int64_t i0 = threadIdx.x; i0 < block_chunks; i0 += (int64_t)blockDim.x * kCopyBatch) {
    u32x4 v[kCopyBatch];
#pragma unroll
    for (int k = 0; k < kCopyBatch; ++k) {  // unconditional (past the end: the last chunk)
      const int64_t i = i0 + (int64_t)k * blockDim.x;
      v[k] = s[i < block_chunks ? i : block_chunks - 1];
    }
#pragma unroll
    for (int k = 0; k < kCopyBatch; ++k) {  // past the end: the last chunk again, same bytes
      const int64_t i = i0 + (int64_t)k * blockDim.x;
      d[i < block_chunks ? i : block_chunks - 1] = v[k];
    }
  }
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_kv_cache_write(const pkv_cache_t* cache, int32_t layer, const void* k_new,
                                  const void* v_new, const int64_t* slot_mapping,
                                  int32_t num_tokens, void* stream) {
  int rc = check_cache(cache);
  if (rc != PKV_OK) return rc;
  if (layer < 0 || layer >= cache->num_layers || num_tokens < 0) return PKV_ERR_INVALID_ARGUMENT;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping) return PKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(k_new) || ((uintptr_t)v_new % elem_bytes(cache->dtype))) return PKV_ERR_INVALID_ARGUMENT;
  const int64_t layer_elems = (int64_t)layer * cache->num_blocks * cache->num_kv_heads *
                              kBlock * cache->head_dim;
  hipStream_t st = (hipStream_t)stream;
  dim3 grid(num_tokens), block(256);
  if (elem_bytes(cache->dtype) == 2)
    hipLaunchKernelGGL(kv_cache_write_kernel<2>, grid, block, 0, st, (const u32x4*)k_new, v_new,
                       slot_mapping, (u32x4*)cache->k_pool, cache->v_pool, cache->num_kv_heads,
                       cache->head_dim, layer_elems);
  else
    hipLaunchKernelGGL(kv_cache_write_kernel<4>, grid, block, 0, st, (const u32x4*)k_new, v_new,
                       slot_mapping, (u32x4*)cache->k_pool, cache->v_pool, cache->num_kv_heads,
                       cache->head_dim, layer_elems);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

extern "C" int pkv_copy_blocks(const pkv_cache_t* cache, const int32_t* pairs, int32_t num_pairs,
                               void* stream) {
  int rc = check_cache(cache);
  if (rc != PKV_OK) return rc;
  if (num_pairs < 0) return PKV_ERR_INVALID_ARGUMENT;
  if (num_pairs == 0) return PKV_OK;
  if (!pairs) return PKV_ERR_INVALID_ARGUMENT;
  const int64_t block_bytes =
      (int64_t)cache->num_kv_heads * kBlock * cache->head_dim * elem_bytes(cache->dtype);
  const int64_t block_chunks = block_bytes / 16;
  const int64_t layer_chunks = block_chunks * cache->num_blocks;
  dim3 grid(num_pairs, cache->num_layers, 2), block(256);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, block, 0, (hipStream_t)stream, pairs,
                     (u32x4*)cache->k_pool, (u32x4*)cache->v_pool, block_chunks, layer_chunks);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
