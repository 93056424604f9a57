// Prefill chunks for gfx950: query rows with q_len > 1 attend to the whole
// cached context of their sequence plus the chunk's own earlier tokens
// (blog.mckayzhao.com/?p=56, chunked prefill under advanced features; the
// mixed {request_id: num_tokens} batch of the V1 section).  Keys are read block
// by block through the block table, as for decode (same page, section
// "PagedAttention").
//
// Two kernels:
//   * small chunks (q_len * G <= 64 (query token, head) columns, e.g. the
//     verify step of speculative decoding): one wavefront per 16 columns,
//     K/V tiles straight from memory into registers;
//   * large chunks: a plan kernel lists (sequence, 256-column query tile, KV
//     head) items, longest context first, and a persistent kernel takes them
//     from a queue.  Per item, K/V tiles of two blocks at a time are staged
//     in LDS (double buffered) and shared by 8 wavefronts of 32 columns; the
//     scores S^T = K.Q^T use 16x16x32 matrix instructions and the product
//     O^T += V^T.P^T runs over 32 tokens at a time, also 16x16x32.
#include "attn_common.h"

namespace pkv {

// ---------------------------------------------------------------------------
// Small chunks: grid (num_kv_heads * q_tiles, num_seqs), 4 wavefronts.  Each
// wavefront owns 16/G query tokens x G heads (one 16-column tile) and scans
// every block its last token can see, causal inside the chunk.  Chunks with
// more than max_cols columns are left to the tiled kernel.
// ---------------------------------------------------------------------------
template <class DT, int D, int G>
__global__ __launch_bounds__(256) void prefill_small_kernel(
    const typename DT::T* __restrict__ q, typename DT::T* __restrict__ out,
    const typename DT::T* __restrict__ kp, const typename DT::T* __restrict__ vp,
    const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ qsl, int num_kv_heads, float scale_log2, int max_cols) {
  typedef Geo<DT, D> Gm;
  constexpr int kTokW = 16 / G;            // query tokens per wavefront
  constexpr int kTokWG = kWaves * kTokW;   // query tokens per workgroup
  const int s = blockIdx.y;
  const int h = blockIdx.x % num_kv_heads;
  const int tile = blockIdx.x / num_kv_heads;
  const int qb = qsl[s];
  const int q_len = qsl[s + 1] - qb;
  if (q_len <= 1 || (int64_t)q_len * G > max_cols) return;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int wq0 = tile * kTokWG + w * kTokW;  // first query token of this wavefront
  if (wq0 >= q_len) return;
  const int n = seq_lens[s];
  const int hq = num_kv_heads * G;
  const int ctx = n - q_len;
  const int tq = wq0 + c / G;
  const bool valid = tq < q_len;
  const int head = h * G + c % G;
  if (n <= 0) {
    if (valid)
      for (int nn = 0; nn < Gm::kN; ++nn)
        for (int i = 0; i < 4; ++i)
          store_elem<DT>(out, ((int64_t)(qb + tq) * hq + head) * D + nn * 16 + 4 * g + i, 0.f);
    return;
  }
  const int lim = ctx + (valid ? tq : q_len - 1);
  WaveState<DT, D> st;
  load_q<DT, D>(st, q + ((int64_t)(qb + (valid ? tq : 0)) * hq + head) * D, valid, g);

  const int wlast = min(wq0 + kTokW, q_len) - 1;
  const int nblk = min(max(ctx + wlast, 0) / kBlock + 1, bt_stride);
  const int32_t* btr = bt + (int64_t)s * bt_stride;
  const int64_t head_off = (int64_t)h * Gm::kTile;
  const int64_t blk_elems = (int64_t)num_kv_heads * Gm::kTile;
  u32x4 kc[Gm::kChunks], vc[Gm::kChunks], kn[Gm::kChunks], vn[Gm::kChunks];
  {
    const int64_t phys = uniform(btr[0]);
    load_tile<DT, D>(kp + phys * blk_elems + head_off, vp + phys * blk_elems + head_off, kc, vc,
                     lane);
  }
  for (int blk = 0; blk < nblk; ++blk) {
    if (blk + 1 < nblk) {
      const int64_t phys = uniform(btr[blk + 1]);
      load_tile<DT, D>(kp + phys * blk_elems + head_off, vp + phys * blk_elems + head_off, kn, vn,
                       lane);
    }
    attend_block<DT, D>(st, kc, vc, blk * kBlock, n, lim, scale_log2, g);
#pragma unroll
    for (int i = 0; i < Gm::kChunks; ++i) {
      kc[i] = kn[i];
      vc[i] = vn[i];
    }
  }
  float lsum = st.l + shfl_xor(st.l, 16);
  lsum += shfl_xor(lsum, 32);
  const float inv = 1.f / lsum;
  if (valid) {
    const int64_t o = ((int64_t)(qb + tq) * hq + head) * D + 4 * g;
#pragma unroll
    for (int nn = 0; nn < Gm::kN; ++nn)
#pragma unroll
      for (int i = 0; i < 4; ++i) store_elem<DT>(out, o + nn * 16 + i, st.acc[nn][i] * inv);
  }
}


// ---------------------------------------------------------------------------
// Large chunks
// ---------------------------------------------------------------------------
constexpr int kPfWaves = 8;
constexpr int kPfThreads = kPfWaves * kWave;
constexpr int kPfBuckets = 64;  // context-length classes of the plan (1024 tokens each)

template <class DT, int D>
struct PfGeo {
  static constexpr int kCT = D <= 128 ? 2 : 1;                      // 16-column tiles per wave
  static constexpr int kCols = kPfWaves * kCT * 16;                 // columns per item
  static constexpr int kTileChunks = kBlock * D * DT::kBytes / 16;  // 16-byte chunks per tile
  static constexpr int kStageChunks = 4 * kTileChunks;              // K, V of two blocks
  static constexpr int kPerThread = kStageChunks / kPfThreads;
  static constexpr int kLdsBytes = 2 * kStageChunks * 16;           // double buffer
  static_assert(kStageChunks % kPfThreads == 0, "whole chunks per thread");
};

struct PfItem {
  int32_t s, qtile, h, pad;
};

// Work list of the tiled kernel: one workgroup of 1024 threads.  Items of one
// (sequence, q-tile) are adjacent (all KV heads); q-tiles are ordered by the
// context their last row sees, longest first, in 1024-token classes.  Also
// resets the queue: queue[0] = next item, queue[1] = number of items.
__global__ __launch_bounds__(1024) void prefill_plan_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int num_seqs,
    int num_kv_heads, int G, int cols, PfItem* __restrict__ items, int32_t* __restrict__ queue,
    int max_items) {
  __shared__ int hist[kPfBuckets], base[kPfBuckets];
  const int tid = threadIdx.x;
  const int qt_tokens = cols / G;
  if (tid < kPfBuckets) hist[tid] = 0;
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
    for (int s = tid; s < num_seqs; s += blockDim.x) {
      const int qb = qsl[s], q_len = qsl[s + 1] - qb, n = seq_lens[s];
      if ((int64_t)q_len * G <= kSmallChunkCols) continue;
      const int ctx = n - q_len;
      const int nqt = (q_len + qt_tokens - 1) / qt_tokens;
      for (int t = 0; t < nqt; ++t) {
        const int vis = max(ctx + min(q_len, (t + 1) * qt_tokens), 0);
        const int b = kPfBuckets - 1 - min(kPfBuckets - 1, vis >> 10);
        const int pos = atomicAdd(&hist[b], num_kv_heads);
        if (pass == 1)
          for (int h = 0; h < num_kv_heads; ++h)
            if (base[b] + pos + h < max_items) items[base[b] + pos + h] = PfItem{s, t, h, 0};
      }
    }
    __syncthreads();
    if (pass == 0 && tid == 0) {
      int run = 0;
      for (int b = 0; b < kPfBuckets; ++b) {
        base[b] = run;
        run += hist[b];
        hist[b] = 0;
      }
      queue[0] = 0;
      queue[1] = min(run, max_items);
    }
    __syncthreads();
  }
}

// four consecutive output elements of one row (fp32 -> storage type, RNE)
template <class DT>
__device__ __forceinline__ void store4(typename DT::T* out, int64_t i, f32x4 v) {
  if constexpr (DT::kBytes == 4) {
    *(f32x4*)(out + i) = v;
  } else {
    uint2 pk;
    if constexpr (__is_same(DT, TBF16)) {
      pk.x = pack2_bf16(v[0], v[1]);
      pk.y = pack2_bf16(v[2], v[3]);
    } else {
      pk.x = pack2_f16(v[0], v[1]);
      pk.y = pack2_f16(v[2], v[3]);
    }
    *(uint2*)(out + i) = pk;
  }
}

template <class DT, int D, int G>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_tiled_kernel(const typename DT::T* __restrict__ q, typename DT::T* __restrict__ out,
                          const typename DT::T* __restrict__ kp,
                          const typename DT::T* __restrict__ vp, const int32_t* __restrict__ bt,
                          int bt_stride, const int32_t* __restrict__ seq_lens,
                          const int32_t* __restrict__ qsl, int num_kv_heads, float scale_log2,
                          const PfItem* __restrict__ items, int32_t* __restrict__ queue) {
  static_assert(DT::kBytes == 2, "16-bit element types");
  typedef Geo<DT, D> Gm;
  typedef PfGeo<DT, D> P;
  constexpr int kCT = P::kCT;
  constexpr int QT = P::kCols / G;  // query tokens per item
  extern __shared__ u32x4 sm_stage[];  // [2][K0, V0, K1, V1][kTileChunks]
  __shared__ int sm_item;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int hq = num_kv_heads * G;
  const int total = queue[1];
  const int64_t blk_elems = (int64_t)num_kv_heads * Gm::kTile;

  for (;;) {
    if (tid == 0) sm_item = atomicAdd(&queue[0], 1);
    __syncthreads();
    const int it = sm_item;
    __syncthreads();
    if (it >= total) break;
    const PfItem item = items[it];
    const int s = item.s, h = item.h;
    const int qb = qsl[s], q_len = qsl[s + 1] - qb, n = seq_lens[s];
    const int ctx = n - q_len;
    const int tq0 = item.qtile * QT, tq_end = min(q_len, tq0 + QT);
    const int32_t* btr = bt + (int64_t)s * bt_stride;
    const int64_t head_off = (int64_t)h * Gm::kTile;

    // this wavefront's columns: col = (w*kCT + ct)*16 + c -> token tq0 + col/G, head h*G + col%G
    u32x4 qv[kCT][Gm::kChunks];
    f32x4 acc[kCT][Gm::kN];
    float m[kCT], l[kCT];
    int lim[kCT];
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      const int col = (w * kCT + ct) * 16 + c;
      const int tq = tq0 + col / G;
      const bool valid = tq < tq_end;
      lim[ct] = valid ? ctx + tq : -1;
      const u32x4* q4 =
          (const u32x4*)(q + ((int64_t)(qb + (valid ? tq : tq0)) * hq + h * G + col % G) * D);
#pragma unroll
      for (int kk = 0; kk < Gm::kChunks; ++kk) qv[ct][kk] = valid ? q4[kk * 4 + g] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int nn = 0; nn < Gm::kN; ++nn) acc[ct][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[ct] = -INFINITY;
      l[ct] = 0.f;
    }
    const int wave_tq = tq0 + (w * kCT * 16) / G;  // first token of this wavefront
    const bool wave_active = wave_tq < tq_end;
    const int wave_min_lim = ctx + wave_tq;
    // blocks the tile's last row can see (a sequence with no tokens sees none)
    const int nvis = n > 0 ? min((ctx + tq_end - 1) / kBlock + 1, bt_stride) : 0;
    const int steps = (nvis + 1) / 2;

    u32x4 stg[P::kPerThread];
    auto fetch_stage = [&](int j) {
#pragma unroll
      for (int k = 0; k < P::kPerThread; ++k) {
        const int idx = tid + k * kPfThreads;
        const int t = idx / P::kTileChunks, ci = idx % P::kTileChunks;
        const int blk = 2 * j + (t >> 1);
        const bool is_v = t & 1;
        u32x4 v = {0, 0, 0, 0};
        if (blk < nvis) {
          const int64_t phys = btr[blk];
          const u32x4* src = (const u32x4*)((is_v ? vp : kp) + phys * blk_elems + head_off);
          v = src[ci];
          if (is_v && blk * kBlock + kBlock > n) {
            // V of slots past the sequence end may be anything: zero it (tokens 4g'..4g'+3)
            const int t0 = blk * kBlock + 4 * ((ci >> 4) & 3);
            const uint32_t m0 = (t0 + 0 < n ? 0x0000ffffu : 0u) | (t0 + 1 < n ? 0xffff0000u : 0u);
            const uint32_t m1 = (t0 + 2 < n ? 0x0000ffffu : 0u) | (t0 + 3 < n ? 0xffff0000u : 0u);
            v.x &= m0;
            v.y &= m1;
            v.z &= m0;
            v.w &= m1;
          }
        }
        stg[k] = v;
      }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
      for (int k = 0; k < P::kPerThread; ++k) sm_stage[buf * P::kStageChunks + tid + k * kPfThreads] = stg[k];
    };
    auto compute = [&](int j, int buf) {
      const u32x4* st = sm_stage + buf * P::kStageChunks;
      const int t0 = 32 * j;
      const bool need_mask = t0 + 31 > wave_min_lim;
      f32x4 sc[2][kCT];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        u32x4 kr[Gm::kChunks];
#pragma unroll
        for (int kk = 0; kk < Gm::kChunks; ++kk) kr[kk] = st[(2 * bb) * P::kTileChunks + kk * kWave + lane];
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          f32x4 acc_s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < Gm::kChunks; ++kk) acc_s = mma_k32(kr[kk], qv[ct][kk], acc_s, DT());
          sc[bb][ct] = acc_s;
        }
      }
      u32x4 pk[kCT];
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = sc[0][ct][i];
          v[4 + i] = sc[1][ct][i];
        }
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int t = t0 + (i >> 2) * 16 + 4 * g + (i & 3);
            v[i] = t <= lim[ct] ? v[i] : -INFINITY;
          }
        }
        float bm = fmaxf(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])),
                         fmaxf(fmaxf(v[4], v[5]), fmaxf(v[6], v[7])));
        bm = fmaxf(bm, shfl_xor(bm, 16));
        bm = fmaxf(bm, shfl_xor(bm, 32));
        const float mn = fmaxf(m[ct], bm * scale_log2);
        const float mu = (mn == -INFINITY) ? 0.f : mn;  // a column with nothing visible yet
        const float alpha = fast_exp2(m[ct] - mu);
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(v[i], scale_log2, -mu));
        l[ct] = l[ct] * alpha + (((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
        m[ct] = mn;
#pragma unroll
        for (int nn = 0; nn < Gm::kN; ++nn) acc[ct][nn] *= alpha;
        if constexpr (__is_same(DT, TBF16)) {
          pk[ct] = u32x4{pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3]), pack2_bf16(p[4], p[5]),
                         pack2_bf16(p[6], p[7])};
        } else {
          pk[ct] = u32x4{pack2_f16(p[0], p[1]), pack2_f16(p[2], p[3]), pack2_f16(p[4], p[5]),
                         pack2_f16(p[6], p[7])};
        }
      }
#pragma unroll
      for (int mm = 0; mm < Gm::kChunks; ++mm) {
        const u32x4 v0 = st[1 * P::kTileChunks + mm * kWave + lane];
        const u32x4 v1 = st[3 * P::kTileChunks + mm * kWave + lane];
        const u32x4 lo = {v0.x, v0.y, v1.x, v1.y};  // dims of slice 2mm: tokens 4g.. of both blocks
        const u32x4 hi = {v0.z, v0.w, v1.z, v1.w};  // slice 2mm+1
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          acc[ct][2 * mm] = mma_k32(lo, pk[ct], acc[ct][2 * mm], DT());
          acc[ct][2 * mm + 1] = mma_k32(hi, pk[ct], acc[ct][2 * mm + 1], DT());
        }
      }
    };

    if (steps > 0) {
      fetch_stage(0);
      store_stage(0);
      __syncthreads();
      for (int j = 0; j < steps; ++j) {
        if (j + 1 < steps) fetch_stage(j + 1);
        if (wave_active) compute(j, j & 1);
        if (j + 1 < steps) store_stage((j + 1) & 1);
        __syncthreads();
      }
    }
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      float lsum = l[ct] + shfl_xor(l[ct], 16);
      lsum += shfl_xor(lsum, 32);
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // nothing visible -> zeros
      if (lim[ct] >= 0 || (n <= 0 && tq0 + ((w * kCT + ct) * 16 + c) / G < tq_end)) {
        const int col = (w * kCT + ct) * 16 + c;
        const int64_t o = ((int64_t)(qb + tq0 + col / G) * hq + h * G + col % G) * D + 4 * g;
#pragma unroll
        for (int nn = 0; nn < Gm::kN; ++nn) store4<DT>(out, o + nn * 16, acc[ct][nn] * inv);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <class DT, int D, int G>
static int small_launch(const AttnArgs& a, int max_cols) {
  typedef typename DT::T T;
  constexpr int kTokWG = kWaves * (16 / G);
  const int64_t max_tok = min((int64_t)a.max_q_len, (int64_t)max_cols / G);
  dim3 grid(a.num_kv_heads * (unsigned)((max_tok + kTokWG - 1) / kTokWG), a.num_seqs);
  hipLaunchKernelGGL((prefill_small_kernel<DT, D, G>), grid, dim3(256), 0, a.stream,
                     (const T*)a.q, (T*)a.out, (const T*)a.kp, (const T*)a.vp, a.bt, a.bt_stride,
                     a.seq_lens, a.qsl, a.num_kv_heads, a.scale_log2, max_cols);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <class DT, int D, int G>
static int tiled_launch(const AttnArgs& a) {
  typedef typename DT::T T;
  typedef PfGeo<DT, D> P;
  static int grid = 0;  // resident workgroups of the persistent kernel (per instantiation)
  if (!grid) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, prefill_tiled_kernel<DT, D, G>,
                                                     kPfThreads, P::kLdsBytes) != hipSuccess)
      return PKV_ERR_HIP;
    grid = cus * (per > 0 ? per : 1);
  }
  PfItem* items = (PfItem*)a.ws_pf;
  int32_t* queue = (int32_t*)((char*)a.ws_pf + a.pf_items * sizeof(PfItem));
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, a.stream, a.seq_lens, a.qsl,
                     a.num_seqs, a.num_kv_heads, G, P::kCols, items, queue, (int)a.pf_items);
  hipLaunchKernelGGL((prefill_tiled_kernel<DT, D, G>), dim3(grid), dim3(kPfThreads), P::kLdsBytes,
                     a.stream, (const T*)a.q, (T*)a.out, (const T*)a.kp, (const T*)a.vp, a.bt,
                     a.bt_stride, a.seq_lens, a.qsl, a.num_kv_heads, a.scale_log2, items, queue);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <class DT, int D>
static int small_g(const AttnArgs& a, int G, int max_cols) {
  switch (G) {
    case 1: return small_launch<DT, D, 1>(a, max_cols);
    case 2: return small_launch<DT, D, 2>(a, max_cols);
    case 4: return small_launch<DT, D, 4>(a, max_cols);
    case 8: return small_launch<DT, D, 8>(a, max_cols);
  }
  return PKV_ERR_UNSUPPORTED;
}

template <class DT>
static int small_d(const AttnArgs& a, int D, int G, int max_cols) {
  switch (D) {
    case 64: return small_g<DT, 64>(a, G, max_cols);
    case 128: return small_g<DT, 128>(a, G, max_cols);
    case 256:
      if constexpr (DT::kBytes == 2) return small_g<DT, 256>(a, G, max_cols);
      break;
  }
  return PKV_ERR_UNSUPPORTED;
}

template <class DT, int D>
static int tiled_g(const AttnArgs& a, int G) {
  switch (G) {
    case 1: return tiled_launch<DT, D, 1>(a);
    case 2: return tiled_launch<DT, D, 2>(a);
    case 4: return tiled_launch<DT, D, 4>(a);
    case 8: return tiled_launch<DT, D, 8>(a);
  }
  return PKV_ERR_UNSUPPORTED;
}

template <class DT>
static int tiled_d(const AttnArgs& a, int D, int G) {
  switch (D) {
    case 64: return tiled_g<DT, 64>(a, G);
    case 128: return tiled_g<DT, 128>(a, G);
    case 256: return tiled_g<DT, 256>(a, G);
  }
  return PKV_ERR_UNSUPPORTED;
}

int launch_prefill_small(const AttnArgs& a, int dtype, int head_dim, int G) {
  // fp32 has no tiled kernel: every chunk takes the per-wavefront kernel
  switch (dtype) {
    case PKV_F32: return small_d<TF32>(a, head_dim, G, 0x7fffffff);
    case PKV_F16: return small_d<TF16>(a, head_dim, G, kSmallChunkCols);
    case PKV_BF16: return small_d<TBF16>(a, head_dim, G, kSmallChunkCols);
  }
  return PKV_ERR_UNSUPPORTED;
}

int launch_prefill_tiled(const AttnArgs& a, int dtype, int head_dim, int G) {
  switch (dtype) {
    case PKV_F32: return PKV_OK;
    case PKV_F16: return tiled_d<TF16>(a, head_dim, G);
    case PKV_BF16: return tiled_d<TBF16>(a, head_dim, G);
  }
  return PKV_ERR_UNSUPPORTED;
}

int64_t prefill_items_bound(int64_t num_seqs, int64_t num_q_tokens, int64_t num_q_heads) {
  // q-tiles of a sequence: ceil(q_len*G/cols) <= q_len*G/cols + 1 with cols >= 128, times the
  // KV heads; chunks hold at least two query tokens
  const int64_t chunks = num_seqs < num_q_tokens / 2 ? num_seqs : num_q_tokens / 2;
  return (num_q_tokens * num_q_heads + 127) / 128 + (chunks + 1) * num_q_heads;
}

int64_t prefill_workspace_bytes(int64_t num_seqs, int64_t num_q_tokens, int64_t num_q_heads) {
  return prefill_items_bound(num_seqs, num_q_tokens, num_q_heads) * (int64_t)sizeof(PfItem) + 64;
}

}  // namespace pkv
