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

// grid (window of `win` consecutive tokens of the call, KV head); `win` is 1 to 16, chosen
// on the host so that the grid fills the GPU (single decode tokens: one token per
// workgroup; prefill chunks: 16).  A workgroup issues every load it needs at once (the
// slots of its tokens and of three on either side, its tokens' K chunks, the V rows of
// its tokens and of the three after them), then stores.
//   K: every 16-byte run of head dims stays contiguous in the tile (chunk (d/x) of token t
//   sits at ((d/x)*16 + t)*x), so a token's K is 16-byte stores.
//   V: four consecutive tokens of a dim are adjacent in the tile (a 16-byte chunk holds
//   tokens 4g..4g+3 of x4 dims).  When the call writes all four positions 4g..4g+3 of a
//   block through four consecutive tokens (a group: what the tokens of a prefill chunk
//   form), the workgroup holding the group's first token writes each of its chunks as one
//   16-byte store: whole lines of the tile.  A token outside such a group (a single decode
//   token, the ragged ends of a chunk) is written element by element, so the other tokens
//   of its chunks keep their bytes.  All tokens take that path when v_new is not 16-byte
//   aligned (stage == 0).
// Slots at or past the pool's end (num_blocks * 16) are skipped like negative ones.
constexpr int kWinMax = 16;                 // tokens per window, at most
constexpr int kAround = 3;                  // neighbours on each side a group check may need
constexpr int kRowsMax = kWinMax + kAround;  // V rows staged: the window and the three after it
constexpr int kKPer = 4;    // K chunks per thread: 16 tokens x (D * e / 16 <= 64) / 256
constexpr int kVPer = 5;    // V chunks staged per thread: 19 rows x (<= 64) / 256

template <int kBytes>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const u32x4* __restrict__ k_new, const void* __restrict__ v_new,
    const int64_t* __restrict__ slots, int num_tokens, u32x4* __restrict__ k_pool,
    void* __restrict__ v_pool, int num_kv_heads, int head_dim, int64_t layer_elems,
    int64_t pool_slots, int stage, int win) {
  typedef typename std::conditional<kBytes == 2, uint16_t, uint32_t>::type E;
  constexpr int x = 16 / kBytes;
  constexpr int x4 = x / 4;
  __shared__ int64_t sm_slot[kAround + kWinMax + kAround];  // tokens T0-3 .. T0+win+2; -1: none
  __shared__ int sm_grp[kWinMax];  // per window token: offset in its group, -1 none, -2 skipped
  extern __shared__ u32x4 sm_v[];  // V rows of tokens T0 .. T0+win+2, head h
  const int T0 = blockIdx.x * win, h = blockIdx.y, tid = threadIdx.x;
  const int chunks = head_dim / x;  // 16-byte chunks per (token, head)
  const int row = num_kv_heads * chunks;
  const int rows = win + kAround;
  // all loads first
  if (tid < win + 2 * kAround) {
    const int u = T0 - kAround + tid;
    const int64_t sl = (u >= 0 && u < num_tokens) ? slots[u] : -1;
    sm_slot[tid] = (sl >= 0 && sl < pool_slots) ? sl : -1;
  }
  // loads of chunks past the end read the call's last chunk instead (always in bounds, so
  // the loads need no branches and their registers stay registers); such values are
  // never stored
  const int64_t last_chunk = (int64_t)num_tokens * row - 1;
  u32v4 kv[kKPer];  // vector types: these batches stay in registers
#pragma unroll
  for (int j = 0; j < kKPer; ++j) {  // K chunk i: token i % win, chunk i / win (tokens fastest)
    const int i = tid + j * 256, k = i % win, ch = i / win;
    const int64_t src = (int64_t)(T0 + k) * row + h * chunks + ch;
    kv[j] = *(const u32v4*)&k_new[ch < chunks && T0 + k < num_tokens ? src : last_chunk];
  }
  if (stage) {
    const u32x4* vn = (const u32x4*)v_new;
    u32v4 vv[kVPer];
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int i = tid + j * 256, k = i / chunks, ch = i - k * chunks;
      const int64_t src = (int64_t)(T0 + k) * row + h * chunks + ch;
      vv[j] = *(const u32v4*)&vn[k < rows && T0 + k < num_tokens ? src : last_chunk];
    }
#pragma unroll
    for (int j = 0; j < kVPer; ++j) {
      const int i = tid + j * 256, k = i / chunks;
      if (k < rows && T0 + k < num_tokens) *(u32v4*)&sm_v[i] = vv[j];
    }
  }
  __syncthreads();
  // group(k): for window token k, its offset r inside a group of four consecutive tokens
  // holding positions 4g..4g+3 of one block, -1 when it is in no such group (always
  // without staging), -2 when its slot is skipped
  if (tid < win) {
    const int64_t sl = sm_slot[kAround + tid];
    int grp = -2;
    if (sl >= 0) {
      const int r = (int)(sl & 3);  // position % 4 (blocks hold 16 positions)
      grp = stage ? r : -1;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (sm_slot[kAround + tid - r + j] != sl - r + j) grp = -1;
    }
    sm_grp[tid] = grp;
  }
  const int64_t tile = (int64_t)kBlock * head_dim;
  auto tile_base = [&](int64_t sl) {  // first element of slot sl's (block, head h) tile
    return layer_elems + ((sl / kBlock) * num_kv_heads + h) * tile;
  };
#pragma unroll
  for (int j = 0; j < kKPer; ++j) {
    const int i = tid + j * 256, k = i % win, ch = i / win;
    const int64_t sl = sm_slot[kAround + k];
    if (ch < chunks && T0 + k < num_tokens && sl >= 0)
      *(u32v4*)&k_pool[tile_base(sl) / x + (int64_t)ch * kBlock + sl % kBlock] = kv[j];
  }
  __syncthreads();
  E* vdst = (E*)v_pool;
  const E* sv = (const E*)sm_v;
  // whole chunks of the groups that start in this window: chunk (m, c) of group g holds
  // dims 16 (m x4 + r) + c, r < x4, of tokens 4g..4g+3
  const int per_group = head_dim / x4;
  for (int i = tid; i < win * per_group; i += blockDim.x) {
    const int k = i / per_group, q = i - k * per_group;
    if (sm_grp[k] != 0) continue;
    const int64_t sl = sm_slot[kAround + k];
    const int m = q >> 4, c = q & 15, g = (int)(sl % kBlock) >> 2;
    // element r * 4 + j of the chunk: dim 16 (m x4 + r) + c of token k + j
    uint32_t w[4];
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      if constexpr (kBytes == 2) {
        const int e0 = 2 * i2, e1 = 2 * i2 + 1;  // r = e / 4, j = e % 4
        w[i2] = (uint32_t)sv[(k + e0 % 4) * head_dim + 16 * (m * x4 + e0 / 4) + c] |
                ((uint32_t)sv[(k + e1 % 4) * head_dim + 16 * (m * x4 + e1 / 4) + c] << 16);
      } else {
        w[i2] = sv[(k + i2) * head_dim + 16 * m + c];
      }
    }
    *(u32x4*)(vdst + tile_base(sl) + (((int64_t)m * 4 + g) * 16 + c) * x) = u32x4{w[0], w[1], w[2], w[3]};
  }
  // the other tokens, element by element
  const E* vsrc = (const E*)v_new + ((int64_t)T0 * num_kv_heads + h) * head_dim;
  for (int i = tid; i < win * head_dim; i += blockDim.x) {
    const int k = i / head_dim, d = i - k * head_dim;
    if (sm_grp[k] != -1) continue;
    const int64_t sl = sm_slot[kAround + k];
    const int p = (int)(sl % kBlock), g = p >> 2, j = p & 3;
    const int n = d >> 4, c = d & 15, m = n / x4, r = n - m * x4;
    const E val = stage ? sv[k * head_dim + d] : vsrc[(int64_t)k * num_kv_heads * head_dim + d];
    vdst[tile_base(sl) + ((((int64_t)m * 4 + g) * 16 + c) * x4 + r) * 4 + j] = val;
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
  if (num_tokens > (1 << 30) || cache->num_kv_heads > 65535) return PKV_ERR_UNSUPPORTED;  // grid limits
  const int64_t layer_elems = (int64_t)layer * cache->num_blocks * cache->num_kv_heads *
                              kBlock * cache->head_dim;
  const int64_t pool_slots = (int64_t)cache->num_blocks * kBlock;
  // window: the largest of 16, 8, 4, 2, 1 tokens that still gives 2048 workgroups (8 per
  // CU), so that a few decode tokens spread over the GPU and a prefill chunk's groups stay
  // in one workgroup
  int win = kWinMax;
  while (win > 1 && (int64_t)((num_tokens + win - 1) / win) * cache->num_kv_heads < 2048) win /= 2;
  // LDS for one head's V rows of a window and the three tokens after it (at most 19 KiB);
  // staged when v_new is 16-byte aligned
  const int stage = aligned16(v_new);
  const size_t lds =
      stage ? (size_t)(win + kAround) * cache->head_dim * elem_bytes(cache->dtype) : 0;
  hipStream_t st = (hipStream_t)stream;
  dim3 grid((num_tokens + win - 1) / win, cache->num_kv_heads), block(256);
  if (elem_bytes(cache->dtype) == 2)
    hipLaunchKernelGGL(kv_cache_write_kernel<2>, grid, block, lds, st, (const u32x4*)k_new, v_new,
                       slot_mapping, num_tokens, (u32x4*)cache->k_pool, cache->v_pool,
                       cache->num_kv_heads, cache->head_dim, layer_elems, pool_slots, stage, win);
  else
    hipLaunchKernelGGL(kv_cache_write_kernel<4>, grid, block, lds, st, (const u32x4*)k_new, v_new,
                       slot_mapping, num_tokens, (u32x4*)cache->k_pool, cache->v_pool,
                       cache->num_kv_heads, cache->head_dim, layer_elems, pool_slots, stage, win);
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
