// Prefill chunks for gfx950: query rows with q_len > 1 attend to the whole
// cached context of their sequence plus the chunk's own earlier tokens
// (blog.mckayzhao.com/?p=56, chunked prefill under advanced features; the
// mixed {request_id: num_tokens} batch of the V1 section).  Keys are read block
// by block through the block table, as for decode (same page, section
// "PagedAttention").
//
// Two kernels:
//   * small chunks (q_len * G <= 32 (query token, head) columns, e.g. the
//     verify step of speculative decoding): decode-style, one workgroup per
//     (sequence, KV head) whose wavefronts split the context's blocks;
//   * large chunks: a plan kernel lists (sequence, 256-column query tile, KV
//     head) items, longest context first, and a persistent kernel takes them
//     from a queue.  Per item, K/V tiles of two blocks at a time are staged
//     in LDS (double buffered) and shared by 8 wavefronts of 32 columns; the
//     scores S^T = K.Q^T use 16x16x32 matrix instructions and the product
//     O^T += V^T.P^T runs over 32 tokens at a time, also 16x16x32.
#include "attn_common.h"

namespace pkv {

// ---------------------------------------------------------------------------
// fp32 chunks wider than the small kernel's columns (there is no fp32 tiled
// kernel): grid (num_kv_heads * q_tiles, num_seqs), 4 wavefronts.  Each
// wavefront owns 16/G query tokens x G heads (one 16-column tile) and scans
// every block its last token can see, causal inside the chunk.  Chunks of at
// most min_cols columns are left to the small kernel.
// ---------------------------------------------------------------------------
template <class DT, int D, int G>
__global__ __launch_bounds__(256) void prefill_wave_kernel(
    const typename DT::T* __restrict__ q, typename DT::T* __restrict__ out,
    const typename DT::T* __restrict__ kp, const typename DT::T* __restrict__ vp,
    const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ qsl, int num_kv_heads, float scale_log2, int min_cols) {
  typedef Geo<DT, D> Gm;
  constexpr int kTokW = 16 / G;            // query tokens per wavefront
  constexpr int kTokWG = kWaves * kTokW;   // query tokens per workgroup
  const int s = blockIdx.y;
  const int h = blockIdx.x % num_kv_heads;
  const int tile = blockIdx.x / num_kv_heads;
  const int qb = qsl[s];
  const int q_len = qsl[s + 1] - qb;
  if (q_len <= 1 || (int64_t)q_len * G <= min_cols) return;
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
constexpr int kPfBuckets = 64;     // context-length classes of the plan (1024 tokens each)
constexpr int kPfDepth = 2;        // steps of K/V in flight per thread (register stages)
constexpr int kPfTableMax = 8192;  // block-table entries an item keeps in LDS (131072 tokens)
// The exponentials use a reference max that may lag the true running max by
// up to 2^kPfLag (weights <= 2^8, far from overflow); the accumulators are
// rescaled only when some column's max moves further than that.
constexpr float kPfLag = 8.f;

template <class DT, int D>
struct PfGeo {
  static constexpr int kCT = D <= 128 ? 2 : 1;                      // 16-column tiles per wave
  static constexpr int kSB = D <= 128 ? 4 : 2;                      // KV blocks per pipeline step
  static constexpr int kCols = kPfWaves * kCT * 16;                 // columns per item
  static constexpr int kTileChunks = kBlock * D * DT::kBytes / 16;  // 16-byte chunks per tile
  static constexpr int kStageChunks = 2 * kSB * kTileChunks;        // K and V of a step
  static constexpr int kPerThread = kStageChunks / kPfThreads;
  static constexpr int kLdsBytes = 2 * kStageChunks * 16;           // double buffer
  static_assert(kStageChunks % kPfThreads == 0, "whole chunks per thread");
  static_assert(kSB % 2 == 0 && kPfTableMax % kSB == 0, "whole block pairs per step");
  static_assert(kLdsBytes + kPfTableMax * 4 + 64 <= 160 * 1024, "LDS of one workgroup");
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
    int num_kv_heads, int G, int cols, int small_cols, PfItem* __restrict__ items,
    int32_t* __restrict__ queue, int max_items) {
  __shared__ int hist[kPfBuckets], base[kPfBuckets];
  const int tid = threadIdx.x;
  const int qt_tokens = cols / G;
  if (tid < kPfBuckets) hist[tid] = 0;
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
    for (int s = tid; s < num_seqs; s += blockDim.x) {
      const int qb = qsl[s], q_len = qsl[s + 1] - qb, n = seq_lens[s];
      if ((int64_t)q_len * G <= small_cols) continue;
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

// max over the four lanes c, c+16, c+32, c+48 of a column (row swaps, no LDS)
__device__ __forceinline__ float col_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
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
  constexpr int kSB = P::kSB;
  constexpr int kTC = P::kTileChunks;
  constexpr int QT = P::kCols / G;  // query tokens per item
  // LDS stage: [K of blocks 0..kSB-1][V of block pair 0: slices r=0][r=1][pair 1: r=0][r=1]...
  // A V entry of 16 bytes holds the 8-byte half r of one chunk for the pair's first block,
  // then for its second: exactly one A operand of the 32-token V^T.P^T product.
  extern __shared__ u32x4 sm_stage[];
  __shared__ int sm_item;
  __shared__ int32_t sm_bt[kPfTableMax];  // the item's block-table entries (one segment)
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
    f32x4 accl[kCT];  // row sums of the rounded weights (every element holds the column's sum)
    float m[kCT];     // reference max of each column (log2 domain)
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
      accl[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      m[ct] = -INFINITY;
    }
    const int wave_tq = tq0 + (w * kCT * 16) / G;  // first token of this wavefront
    const bool wave_active = wave_tq < tq_end;
    const int wave_min_lim = ctx + wave_tq;
    // blocks the tile's last row can see (a sequence with no tokens sees none)
    const int nvis = n > 0 ? min((ctx + tq_end - 1) / kBlock + 1, bt_stride) : 0;
    int seg0 = 0;  // first block of the block-table segment held in sm_bt

    // K/V of step j: registers -> LDS buffer j & 1; the next kPfDepth-1 steps are in flight.
    // Thread chunk k of a step is chunk ci of tile t = 2b + (0 for K, 1 for V) of the step's
    // block b.  Loads are unconditional (blocks past the visible range re-read the last one)
    // so that each wait covers exactly one step; masking happens when the step is stored.
    u32x4 stg[kPfDepth][P::kPerThread];
    auto fetch_stage = [&](u32x4 (&dst)[P::kPerThread], int j) {
#pragma unroll
      for (int k = 0; k < P::kPerThread; ++k) {
        const int idx = tid + k * kPfThreads;
        const int t = idx / kTC, ci = idx % kTC;
        const int blk = min(kSB * j + (t >> 1), nvis - 1);
        const int64_t phys = sm_bt[blk - seg0];
        const u32x4* src = (const u32x4*)(((t & 1) ? vp : kp) + phys * blk_elems + head_off);
        dst[k] = src[ci];
      }
    };
    auto store_stage = [&](const u32x4 (&src)[P::kPerThread], int j, int buf) {
      u32x4* st = sm_stage + buf * P::kStageChunks;
#pragma unroll
      for (int k = 0; k < P::kPerThread; ++k) {
        const int idx = tid + k * kPfThreads;
        const int t = idx / kTC, ci = idx % kTC;
        const int b = t >> 1, blk = kSB * j + b;
        u32x4 v = blk < nvis ? src[k] : u32x4{0, 0, 0, 0};
        if (t & 1) {
          if (blk * kBlock + kBlock > n) {
            // V of slots past the sequence end may be anything: zero it (tokens 4g'..4g'+3)
            const int t0 = blk * kBlock + 4 * ((ci >> 4) & 3);
            const uint32_t m0 = (t0 + 0 < n ? 0x0000ffffu : 0u) | (t0 + 1 < n ? 0xffff0000u : 0u);
            const uint32_t m1 = (t0 + 2 < n ? 0x0000ffffu : 0u) | (t0 + 3 < n ? 0xffff0000u : 0u);
            v.x &= m0;
            v.y &= m1;
            v.z &= m0;
            v.w &= m1;
          }
          uint2* v2 = (uint2*)(st + (kSB + 2 * (b >> 1)) * kTC);
          v2[2 * ci + (b & 1)] = uint2{v.x, v.y};
          v2[2 * (kTC + ci) + (b & 1)] = uint2{v.z, v.w};
        } else {
          st[b * kTC + ci] = v;
        }
      }
    };
    auto compute = [&](int j, int buf) {
      const u32x4* st = sm_stage + buf * P::kStageChunks;
      const int t0 = kSB * kBlock * j;
      const bool need_mask = t0 + kSB * kBlock - 1 > wave_min_lim;
      // S^T = K.Q^T: lane 16g+c holds tokens 4g..4g+3 of each block for column c
      f32x4 sc[kSB][kCT];
#pragma unroll
      for (int b = 0; b < kSB; ++b) {
        u32x4 kr[Gm::kChunks];
#pragma unroll
        for (int kk = 0; kk < Gm::kChunks; ++kk) kr[kk] = st[b * kTC + kk * kWave + lane];
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < Gm::kChunks; ++kk) a = mma_k32(kr[kk], qv[ct][kk], a, DT());
          sc[b][ct] = a;
        }
      }
      // column maxima of this step; the reference max moves only when one of them exceeds it
      // by more than kPfLag (a wave-wide decision)
      float bms[kCT];
      bool move = false;
#pragma unroll
      for (int ct = 0; ct < kCT; ++ct) {
        if (need_mask) {
#pragma unroll
          for (int b = 0; b < kSB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t = t0 + b * kBlock + 4 * g + i;
              sc[b][ct][i] = t <= lim[ct] ? sc[b][ct][i] : -INFINITY;
            }
        }
        float bm = -INFINITY;
#pragma unroll
        for (int b = 0; b < kSB; ++b)
          bm = fmaxf(bm, fmaxf(fmaxf(sc[b][ct][0], sc[b][ct][1]), fmaxf(sc[b][ct][2], sc[b][ct][3])));
        bms[ct] = col_max4(bm) * scale_log2;
        move |= bms[ct] > m[ct] + kPfLag;  // also the first visible key of a column (m = -inf)
      }
      if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          const float mn = fmaxf(m[ct], bms[ct]);
          const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m[ct] - mn);
#pragma unroll
          for (int nn = 0; nn < Gm::kN; ++nn) acc[ct][nn] *= alpha;
          accl[ct] *= alpha;
          m[ct] = mn;
        }
      }
      const uint32_t one2 = __is_same(DT, TBF16) ? 0x3F803F80u : 0x3C003C00u;
      const u32x4 ones = {one2, one2, one2, one2};
#pragma unroll
      for (int pp = 0; pp < kSB / 2; ++pp) {
        // weights of the block pair: lane 16g+c holds tokens 4g..4g+3 of both blocks (k = 8g..)
        u32x4 pk[kCT];
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          const float mu = m[ct] == -INFINITY ? 0.f : m[ct];  // nothing visible yet
          float p[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(fmaf(sc[2 * pp][ct][i], scale_log2, -mu));
            p[4 + i] = fast_exp2(fmaf(sc[2 * pp + 1][ct][i], scale_log2, -mu));
          }
          if constexpr (__is_same(DT, TBF16)) {
            pk[ct] = u32x4{pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3]), pack2_bf16(p[4], p[5]),
                           pack2_bf16(p[6], p[7])};
          } else {
            pk[ct] = u32x4{pack2_f16(p[0], p[1]), pack2_f16(p[2], p[3]), pack2_f16(p[4], p[5]),
                           pack2_f16(p[6], p[7])};
          }
        }
        // O^T += V^T . P^T over the pair's 32 tokens, and the row sums against a slice of ones
#pragma unroll
        for (int mm = 0; mm < Gm::kChunks; ++mm) {
          const u32x4 lo = st[(kSB + 2 * pp) * kTC + mm * kWave + lane];      // dim slice 2mm
          const u32x4 hi = st[(kSB + 2 * pp + 1) * kTC + mm * kWave + lane];  // slice 2mm+1
#pragma unroll
          for (int ct = 0; ct < kCT; ++ct) {
            acc[ct][2 * mm] = mma_k32(lo, pk[ct], acc[ct][2 * mm], DT());
            acc[ct][2 * mm + 1] = mma_k32(hi, pk[ct], acc[ct][2 * mm + 1], DT());
          }
        }
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) accl[ct] = mma_k32(ones, pk[ct], accl[ct], DT());
      }
    };

    // the block table goes through LDS in segments of kPfTableMax blocks; steps j in [js, je)
    for (; seg0 < nvis; seg0 += kPfTableMax) {
      const int seg_n = min(kPfTableMax, nvis - seg0);
      for (int i = tid; i < seg_n; i += kPfThreads) sm_bt[i] = btr[seg0 + i];
      __syncthreads();
      const int js = seg0 / kSB, je = (seg0 + seg_n + kSB - 1) / kSB;
      const int jl = je - 1;  // steps past the segment fetch its last step again (unused)
#pragma unroll
      for (int u = 0; u + 1 < kPfDepth; ++u) fetch_stage(stg[u], min(js + u, jl));
      store_stage(stg[0], js, js & 1);
      __syncthreads();
      for (int j0 = js; j0 < je; j0 += kPfDepth) {
#pragma unroll
        for (int u = 0; u < kPfDepth; ++u) {
          const int j = j0 + u;  // K/V of step j: stg[u] and LDS buffer j & 1
          if (j >= je) break;
          fetch_stage(stg[(u + kPfDepth - 1) % kPfDepth], min(j + kPfDepth - 1, jl));
          if (wave_active) compute(j, j & 1);
          if (j + 1 < je) store_stage(stg[(u + 1) % kPfDepth], j + 1, (j + 1) & 1);
          __syncthreads();
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      const float lsum = accl[ct][0];
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // nothing visible -> zeros
      const int col = (w * kCT + ct) * 16 + c;
      if (tq0 + col / G < tq_end && (lim[ct] >= 0 || n <= 0)) {
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
static int wave_launch(const AttnArgs& a) {
  typedef typename DT::T T;
  constexpr int kTokWG = kWaves * (16 / G);
  dim3 grid(a.num_kv_heads * (unsigned)((a.max_q_len + kTokWG - 1) / kTokWG), a.num_seqs);
  hipLaunchKernelGGL((prefill_wave_kernel<DT, D, G>), grid, dim3(256), 0, a.stream, (const T*)a.q,
                     (T*)a.out, (const T*)a.kp, (const T*)a.vp, a.bt, a.bt_stride, a.seq_lens,
                     a.qsl, a.num_kv_heads, a.scale_log2, 16);
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
                     a.num_seqs, a.num_kv_heads, G, P::kCols,
                     small_chunk_max_cols(DT::kBytes == 2 ? PKV_BF16 : PKV_F32, D), items, queue,
                     (int)a.pf_items);
  hipLaunchKernelGGL((prefill_tiled_kernel<DT, D, G>), dim3(grid), dim3(kPfThreads), P::kLdsBytes,
                     a.stream, (const T*)a.q, (T*)a.out, (const T*)a.kp, (const T*)a.vp, a.bt,
                     a.bt_stride, a.seq_lens, a.qsl, a.num_kv_heads, a.scale_log2, items, queue);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <class DT, int D>
static int wave_g(const AttnArgs& a, int G) {
  switch (G) {
    case 1: return wave_launch<DT, D, 1>(a);
    case 2: return wave_launch<DT, D, 2>(a);
    case 4: return wave_launch<DT, D, 4>(a);
    case 8: return wave_launch<DT, D, 8>(a);
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

int launch_prefill_wave(const AttnArgs& a, int dtype, int head_dim, int G) {
  if (dtype != PKV_F32) return PKV_ERR_UNSUPPORTED;
  switch (head_dim) {
    case 64: return wave_g<TF32, 64>(a, G);
    case 128: return wave_g<TF32, 128>(a, G);
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
