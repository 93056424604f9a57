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

// One workgroup per token, all KV heads.  Its loads do not wait for its slot: the
// token's K chunks and V elements are read at once, beside the slots of the token and of
// three neighbours on either side (scalar loads), so a decode token costs one memory
// round trip before its stores.
// Groups: when four consecutive tokens of the call hold positions 4g..4g+3 of one block
// (what the tokens of a prefill chunk form), the group's first token writes the whole
// group and the other three write nothing.  Its stores fill whole lines of the tiles:
//   K: every 16-byte run of head dims stays contiguous in the tile (chunk (d/x) of token t
//   sits at ((d/x)*16 + t)*x), so positions 4g..4g+3 of one chunk run are 64 contiguous
//   bytes;
//   V: four consecutive tokens of a dim are adjacent in the tile (a 16-byte chunk holds
//   tokens 4g..4g+3 of x4 dims), so each chunk is one 16-byte store, gathered from the
//   four tokens' elements.
// A token outside such a group (a single decode token, the ragged ends of a chunk)
// writes its own K chunks and its V element by element, so the other tokens of its V
// chunks keep their bytes.
// Slots at or past the pool's end (num_blocks * 16) are skipped like negative ones.
constexpr int kKPer = 2;  // K chunks per thread and pass (512 per pass: 8 heads of 256 fp32 dims)
constexpr int kEPer = 8;  // V elements per thread and pass (2048 per pass: 8 heads of 256 dims)

template <int kBytes>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const u32x4* __restrict__ k_new, const void* __restrict__ v_new,
    const int64_t* __restrict__ slots, int num_tokens, u32x4* __restrict__ k_pool,
    void* __restrict__ v_pool, int num_kv_heads, int head_dim, int64_t layer_elems,
    int64_t pool_slots) {
  typedef typename std::conditional<kBytes == 2, uint16_t, uint32_t>::type E;
  constexpr int x = 16 / kBytes;
  constexpr int x4 = x / 4;
  const int tok = blockIdx.x, tid = threadIdx.x;
  const int chunks = head_dim / x;                  // 16-byte chunks per (token, head)
  const int row = num_kv_heads * chunks;            // 16-byte chunks per token
  const int relems = num_kv_heads * head_dim;       // elements per token
  const E* vn = (const E*)v_new;
  // the first pass of K chunks and V elements, before the slots are known (past the end
  // of the row: its last entry again, never stored)
  u32v4 kv[kKPer];
#pragma unroll
  for (int j = 0; j < kKPer; ++j)
    kv[j] = *(const u32v4*)&k_new[(int64_t)tok * row + min(tid + 256 * j, row - 1)];
  E ve[kEPer];
#pragma unroll
  for (int j = 0; j < kEPer; ++j) ve[j] = vn[(int64_t)tok * relems + min(tid + 256 * j, relems - 1)];
  // slots of tokens tok-3 .. tok+3 (-1: none, skipped or outside the pool)
  int64_t sn[7];
#pragma unroll
  for (int j = 0; j < 7; ++j) {
    const int u = tok - 3 + j;
    const int64_t sl = (u >= 0 && u < num_tokens) ? slots[u] : -1;
    sn[j] = (sl >= 0 && sl < pool_slots) ? sl : -1;
  }
  const int64_t sl = sn[3];
  if (sl < 0) return;
  const int p = (int)(sl % kBlock);
  const int64_t tile = (int64_t)kBlock * head_dim;
  const int64_t blk_base = layer_elems + (sl / kBlock) * num_kv_heads * tile;  // elements
  // is the token in a group of four consecutive tokens holding positions 4g..4g+3?
  const int r = p & 3;
  bool grouped = true;
#pragma unroll
  for (int o = -3; o <= 3; ++o)  // token tok + o is the group's member o + r
    if (o + r >= 0 && o + r <= 3) grouped = grouped && sn[3 + o] == sl + o;
  E* vdst = (E*)v_pool + blk_base;
  if (!grouped) {
    // K: chunk i of the row is chunk ch = i % chunks of head i / chunks
    for (int i0 = 0; i0 < row; i0 += 256 * kKPer) {
      if (i0 > 0) {
#pragma unroll
        for (int j = 0; j < kKPer; ++j)
          kv[j] = *(const u32v4*)&k_new[(int64_t)tok * row + min(i0 + tid + 256 * j, row - 1)];
      }
#pragma unroll
      for (int j = 0; j < kKPer; ++j) {
        const int i = i0 + tid + 256 * j;
        if (i < row) {
          const int h = i / chunks, ch = i - h * chunks;
          *(u32v4*)&k_pool[(blk_base + h * tile) / x + (int64_t)ch * kBlock + p] = kv[j];
        }
      }
    }
    // V element by element: element i is dim d = i % head_dim of head i / head_dim
    const int g = p >> 2, jj = p & 3;
    for (int i0 = 0; i0 < relems; i0 += 256 * kEPer) {
      if (i0 > 0) {
#pragma unroll
        for (int j = 0; j < kEPer; ++j)
          ve[j] = vn[(int64_t)tok * relems + min(i0 + tid + 256 * j, relems - 1)];
      }
#pragma unroll
      for (int j = 0; j < kEPer; ++j) {
        const int i = i0 + tid + 256 * j;
        if (i < relems) {
          const int h = i / head_dim, d = i - h * head_dim;
          const int n = d >> 4, c = d & 15, m = n / x4, rr = n - m * x4;
          vdst[h * tile + ((((int64_t)m * 4 + g) * 16 + c) * x4 + rr) * 4 + jj] = ve[j];
        }
      }
    }
  } else if (r == 0) {
    // the group's first token writes the group.  K: entry i is token j = i % 4 of chunk
    // i / 4 of the row, so four neighbouring lanes fill the 64 bytes of positions
    // p .. p + 3 of one chunk run
    for (int i0 = 0; i0 < 4 * row; i0 += 256 * kKPer) {
      u32v4 kg[kKPer];
#pragma unroll
      for (int j = 0; j < kKPer; ++j) {
        const int i = min(i0 + tid + 256 * j, 4 * row - 1);
        kg[j] = *(const u32v4*)&k_new[(int64_t)(tok + (i & 3)) * row + (i >> 2)];
      }
#pragma unroll
      for (int j = 0; j < kKPer; ++j) {
        const int i = i0 + tid + 256 * j;
        if (i < 4 * row) {
          const int ci = i >> 2, h = ci / chunks, ch = ci - h * chunks;
          *(u32v4*)&k_pool[(blk_base + h * tile) / x + (int64_t)ch * kBlock + p + (i & 3)] = kg[j];
        }
      }
    }
    // V: whole chunks.  Chunk (m, c) of head h holds dims 16 (m x4 + rr) + c, rr < x4, of
    // the group's tokens j = 0..3, element rr * 4 + j
    const int g = p >> 2;
    const int per_head = head_dim / x4;  // chunks of one group in one head's tile
    for (int i = tid; i < num_kv_heads * per_head; i += blockDim.x) {
      const int h = i / per_head, q = i - h * per_head, m = q >> 4, c = q & 15;
      const E* src = vn + (int64_t)tok * relems + h * head_dim + 16 * m * x4 + c;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (kBytes == 2) {  // elements 2k and 2k+1: (rr, j) = (k / 2, 2 (k % 2)) and +1
          const int rr = k >> 1, j0 = 2 * (k & 1);
          w[k] = (uint32_t)src[(int64_t)j0 * relems + 16 * rr] |
                 ((uint32_t)src[(int64_t)(j0 + 1) * relems + 16 * rr] << 16);
        } else {
          w[k] = src[(int64_t)k * relems];
        }
      }
      *(u32v4*)&vdst[h * tile + (((int64_t)m * 4 + g) * 16 + c) * x] = u32v4{w[0], w[1], w[2], w[3]};
    }
  }
}

// grid (pair, layer, K|V): copy one block of one layer of one pool.  A block's
// source and destination never overlap (distinct blocks), so each thread issues
// all loads of a round before its stores: one memory round trip per kCopyBatch
// chunks instead of one per chunk.  Loads and stores are unconditional: a lane
// past the block's end copies its last chunk again (the same bytes to the same
// place).  A pair naming a block outside the pool is skipped.
constexpr int kCopyBatch = 8;

__global__ __launch_bounds__(256) void copy_blocks_kernel(const int32_t* __restrict__ pairs,
                                                          u32x4* __restrict__ k_pool,
                                                          u32x4* __restrict__ v_pool,
                                                          int64_t block_chunks,
                                                          int64_t layer_chunks, int num_blocks) {
  const int p = blockIdx.x;
  const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  u32x4* pool = blockIdx.z ? v_pool : k_pool;
  const int64_t base = blockIdx.y * layer_chunks;
  const u32x4* __restrict__ s = pool + base + src * block_chunks;
  u32x4* __restrict__ d = pool + base + dst * block_chunks;
  for (int64_t i0 = threadIdx.x; i0 < block_chunks; i0 += (int64_t)blockDim.x * kCopyBatch) {
    u32v4 v[kCopyBatch];  // a vector type: the batch stays in registers
#pragma unroll
    for (int k = 0; k < kCopyBatch; ++k) {  // unconditional (past the end: the last chunk)
      const int64_t i = i0 + (int64_t)k * blockDim.x;
      v[k] = *(const u32v4*)&s[i < block_chunks ? i : block_chunks - 1];
    }
#pragma unroll
    for (int k = 0; k < kCopyBatch; ++k) {  // past the end: the last chunk again, same bytes
      const int64_t i = i0 + (int64_t)k * blockDim.x;
      *(u32v4*)&d[i < block_chunks ? i : block_chunks - 1] = v[k];
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
  if (num_tokens > (1 << 30)) return PKV_ERR_UNSUPPORTED;  // grid limit
  const int64_t layer_elems = (int64_t)layer * cache->num_blocks * cache->num_kv_heads *
                              kBlock * cache->head_dim;
  const int64_t pool_slots = (int64_t)cache->num_blocks * kBlock;
  hipStream_t st = (hipStream_t)stream;
  dim3 grid(num_tokens), block(256);
  if (elem_bytes(cache->dtype) == 2)
    hipLaunchKernelGGL(kv_cache_write_kernel<2>, grid, block, 0, st, (const u32x4*)k_new, v_new,
                       slot_mapping, num_tokens, (u32x4*)cache->k_pool, cache->v_pool,
                       cache->num_kv_heads, cache->head_dim, layer_elems, pool_slots);
  else
    hipLaunchKernelGGL(kv_cache_write_kernel<4>, grid, block, 0, st, (const u32x4*)k_new, v_new,
                       slot_mapping, num_tokens, (u32x4*)cache->k_pool, cache->v_pool,
                       cache->num_kv_heads, cache->head_dim, layer_elems, pool_slots);
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
                     (u32x4*)cache->k_pool, (u32x4*)cache->v_pool, block_chunks, layer_chunks,
                     cache->num_blocks);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
