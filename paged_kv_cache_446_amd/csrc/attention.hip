// PagedAttention for gfx950: decode (split-K over the paged context, then a
// merge of the partitions) and prefill chunks (causal inside the chunk).
//
// The kernels find every block through the sequence's block table and read K
// and V block by block; the result is that of attention over the same tokens
// stored contiguously (blog.mckayzhao.com/?p=56, section "PagedAttention").
// Decode looks at every earlier token (devpress.csdn.net/amd/
// 6a408ab810ee7a33f2834f35.html, prefill / decode section); a prefill chunk
// of a long prompt sees the cached context plus its own earlier tokens
// (blog page, chunked prefill under advanced features).
//
// Work decomposition.  A wavefront owns a 16-column tile of the score matrix
// S^T = K . Q^T: the columns are (query token, query head) pairs of one KV
// head, so a KV tile is read once for all G = Hq/Hkv heads that share it.
// For every 16-token block: 16x16x32 matrix instructions for S^T, a
// wavefront-shuffle online softmax (running max and sum per column), and
// 16x16x16 matrix instructions for O^T += V^T . P^T, whose P^T operand is the
// S^T result already in place.
//
// Decode splits the context of a sequence into partitions of kPartBlocks
// blocks (1024 tokens).  One workgroup per (sequence, partition, KV head):
// its four wavefronts take every fourth block, streaming K/V tiles with
// non-temporal loads (each tile is read once), merge through LDS, and a
// second kernel merges the partitions of long sequences with the log-sum-exp
// rule.  Workgroup ids are remapped so that the eight KV heads of one
// partition, and neighbouring partitions, run on the same XCD (hardware
// dispatch deals consecutive workgroups round-robin over the eight XCDs).
#include <hip/hip_runtime.h>
#include <math.h>

#include "pkv.h"
#include "pkv_device.h"
#include "pkv_host.h"

namespace pkv {

constexpr int kWaves = 4;        // wavefronts per workgroup
constexpr int kPartBlocks = 64;  // blocks per decode partition (1024 tokens)
constexpr int kPerWave = kPartBlocks / kWaves;  // blocks of a partition per wavefront
constexpr int kXcds = 8;         // accelerator complex dies of an MI355X
static_assert(kPerWave <= 64, "one block-table entry per lane");

typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));

template <class DT, int D>
struct Geo {
  static constexpr int kChunks = D * DT::kBytes / 64;  // 16-byte operand chunks per lane per tile
  static constexpr int kN = D / 16;                    // 16-dim slices of the output
  static constexpr int kTile = kBlock * D;             // elements per (block, head) tile
  static constexpr int kX = 16 / DT::kBytes;           // elements per 16-byte chunk
};

template <class DT, int D>
struct WaveState {
  u32x4 q[Geo<DT, D>::kChunks];  // Q^T operand of this lane's column
  f32x4 acc[Geo<DT, D>::kN];     // O^T: lane 16g+c holds dims 16n+4g..16n+4g+3 of column c
  float m;                       // running max of the column (log2 domain)
  float l;                       // running sum of this lane's 4 tokens per block
};

template <class DT, int D>
__device__ __forceinline__ void load_q(WaveState<DT, D>& st, const typename DT::T* qrow, bool valid,
                                       int g) {
  const u32x4* q4 = (const u32x4*)qrow;
#pragma unroll
  for (int kk = 0; kk < Geo<DT, D>::kChunks; ++kk)
    st.q[kk] = valid ? q4[kk * 4 + g] : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int n = 0; n < Geo<DT, D>::kN; ++n) st.acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
}

// One (block, KV head) tile of K and of V into registers: chunk i*64 + lane of
// each.  kStream marks tiles read exactly once (decode): non-temporal loads
// keep them from displacing reusable lines in the caches.
template <class DT, int D, bool kStream = false>
__device__ __forceinline__ void load_tile(const typename DT::T* kt, const typename DT::T* vt,
                                          u32x4 (&kr)[Geo<DT, D>::kChunks],
                                          u32x4 (&vr)[Geo<DT, D>::kChunks], int lane) {
  const u32x4* k4 = (const u32x4*)kt;
  const u32x4* v4 = (const u32x4*)vt;
#pragma unroll
  for (int i = 0; i < Geo<DT, D>::kChunks; ++i) {
    if constexpr (kStream) {
      kr[i] = __builtin_bit_cast(u32x4, __builtin_nontemporal_load((const u32v4*)(k4 + i * kWave + lane)));
      vr[i] = __builtin_bit_cast(u32x4, __builtin_nontemporal_load((const u32v4*)(v4 + i * kWave + lane)));
    } else {
      kr[i] = k4[i * kWave + lane];
      vr[i] = v4[i * kWave + lane];
    }
  }
}

template <class DT, int D>
struct TileBuf {
  u32x4 k[Geo<DT, D>::kChunks], v[Geo<DT, D>::kChunks];
};

__device__ __forceinline__ float lanef(const u32x4& v, int e) {
  return __uint_as_float(e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w);
}

// One 16-token block: scores, online softmax update, P.V accumulate.
//   tok0  absolute index of the block's first token
//   n     tokens in the sequence (slots >= n hold stale data: never used)
//   lim   last token this lane's column may see (inclusive, < n)
template <class DT, int D>
__device__ __forceinline__ void attend_block(WaveState<DT, D>& st,
                                             const u32x4 (&kr)[Geo<DT, D>::kChunks],
                                             u32x4 (&vr)[Geo<DT, D>::kChunks], int tok0, int n,
                                             int lim, float scale_log2, int g) {
  typedef Geo<DT, D> Gm;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (DT::kBytes == 2) {
#pragma unroll
    for (int kk = 0; kk < Gm::kChunks; ++kk) s = mma_k32(kr[kk], st.q[kk], s, DT());
  } else {
#pragma unroll
    for (int kk = 0; kk < Gm::kChunks; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) s = mma_f32(lanef(kr[kk], e), lanef(st.q[kk], e), s);
  }
  const int t0 = tok0 + 4 * g;
  float sv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = (t0 + i <= lim) ? s[i] * scale_log2 : -INFINITY;
  float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  bm = fmaxf(bm, shfl_xor(bm, 16));
  bm = fmaxf(bm, shfl_xor(bm, 32));
  const float mn = fmaxf(st.m, bm);
  const float mu = (mn == -INFINITY) ? 0.f : mn;  // a column with nothing visible yet
  const float alpha = fast_exp2(st.m - mu);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - mu);
  st.m = mn;
#pragma unroll
  for (int nn = 0; nn < Gm::kN; ++nn) st.acc[nn] *= alpha;

  // slots at or past the sequence end may hold anything (even NaN): select, never multiply
  const bool tail = tok0 + kBlock > n;
  if constexpr (DT::kBytes == 2) {
    uint32_t pd0, pd1;
    if constexpr (__is_same(DT, TBF16)) {
      pd0 = pack2_bf16(p[0], p[1]);
      pd1 = pack2_bf16(p[2], p[3]);
    } else {
      pd0 = pack2_f16(p[0], p[1]);
      pd1 = pack2_f16(p[2], p[3]);
    }
    // the sum uses the rounded weights, so the output is a convex combination of V rows
    float ps;
    if constexpr (__is_same(DT, TBF16)) {
      ps = (bf16_bits_to_f32(pd0 & 0xffffu) + bf16_bits_to_f32(pd0 >> 16)) +
           (bf16_bits_to_f32(pd1 & 0xffffu) + bf16_bits_to_f32(pd1 >> 16));
    } else {
      ps = ((float)__builtin_bit_cast(_Float16, (uint16_t)(pd0 & 0xffffu)) +
            (float)__builtin_bit_cast(_Float16, (uint16_t)(pd0 >> 16))) +
           ((float)__builtin_bit_cast(_Float16, (uint16_t)(pd1 & 0xffffu)) +
            (float)__builtin_bit_cast(_Float16, (uint16_t)(pd1 >> 16)));
    }
    st.l = st.l * alpha + ps;
    if (tail) {
      const uint32_t m0 = (t0 + 0 < n ? 0x0000ffffu : 0u) | (t0 + 1 < n ? 0xffff0000u : 0u);
      const uint32_t m1 = (t0 + 2 < n ? 0x0000ffffu : 0u) | (t0 + 3 < n ? 0xffff0000u : 0u);
#pragma unroll
      for (int i = 0; i < Gm::kChunks; ++i) {
        vr[i].x &= m0;
        vr[i].y &= m1;
        vr[i].z &= m0;
        vr[i].w &= m1;
      }
    }
#pragma unroll
    for (int i = 0; i < Gm::kChunks; ++i) {
      st.acc[2 * i] = mma_k16(vr[i].x, vr[i].y, pd0, pd1, st.acc[2 * i], DT());
      st.acc[2 * i + 1] = mma_k16(vr[i].z, vr[i].w, pd0, pd1, st.acc[2 * i + 1], DT());
    }
  } else {
    st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    if (tail) {
#pragma unroll
      for (int i = 0; i < Gm::kChunks; ++i) {
        vr[i].x = t0 + 0 < n ? vr[i].x : 0u;
        vr[i].y = t0 + 1 < n ? vr[i].y : 0u;
        vr[i].z = t0 + 2 < n ? vr[i].z : 0u;
        vr[i].w = t0 + 3 < n ? vr[i].w : 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < Gm::kChunks; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) st.acc[i] = mma_f32(lanef(vr[i], j), p[j], st.acc[i]);
  }
}

template <class DT>
__device__ __forceinline__ void store_elem(typename DT::T* out, int64_t i, float v) {
  if constexpr (__is_same(DT, TBF16))
    out[i] = (uint16_t)f32_to_bf16_bits(v);
  else
    out[i] = (typename DT::T)v;
}

// ---------------------------------------------------------------------------
// Decode: a 1-D grid over (sequence, partition, KV head), 4 wavefronts each.
// ---------------------------------------------------------------------------

// Waves per SIMD the register allocation must allow: three for the 16-bit
// types up to head_dim 128 (enough K/V bytes in flight per CU), otherwise
// whatever the kernel needs.
template <class DT, int D>
constexpr int decode_occupancy() {
  return (DT::kBytes == 2 && D <= 128) ? 3 : 1;
}

// Workgroup id -> work item.  Dispatch deals consecutive ids round-robin over
// the XCDs; item j = (id % 8) * (grid / 8) + id / 8 gives every XCD one
// contiguous run of items (the host pads the grid to a multiple of 8).
__device__ __forceinline__ int xcd_item(int id, int grid) {
  return (id % kXcds) * (grid / kXcds) + id / kXcds;
}

template <class DT, int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(decode_occupancy<DT, D>())))
void decode_kernel(const typename DT::T* __restrict__ q, typename DT::T* __restrict__ out,
                   const typename DT::T* __restrict__ kp, const typename DT::T* __restrict__ vp,
                   const int32_t* __restrict__ bt, int bt_stride,
                   const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
                   int num_seqs, int num_kv_heads, float scale_log2, int max_parts,
                   float* __restrict__ ws_o, float* __restrict__ ws_ml) {
  typedef Geo<DT, D> Gm;
  const int j = xcd_item(blockIdx.x, gridDim.x);
  const int h = j % num_kv_heads;
  const int sp = j / num_kv_heads;
  const int part = sp % max_parts;
  const int s = sp / max_parts;
  if (s >= num_seqs) return;  // grid padding
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int b0 = part * kPartBlocks;
  const int32_t* btr = bt + (int64_t)s * bt_stride;
  // block-table entries of this wavefront's blocks b0 + w + 4i, one per lane,
  // loaded alongside the sequence metadata (bounded by the table width only)
  int btv = 0;
  {
    const int bi = b0 + w + kWaves * lane;
    if (lane < kPerWave && bi < bt_stride) btv = btr[bi];
  }
  const int qb = qsl[s];
  if (qsl[s + 1] - qb != 1) return;
  const int n = seq_lens[s];
  const int hq = num_kv_heads * G;
  if (n <= 0) {
    if (part == 0)
      for (int e = threadIdx.x; e < G * D; e += blockDim.x)
        store_elem<DT>(out, ((int64_t)qb * hq + h * G) * D + e, 0.f);
    return;
  }
  // a sequence longer than the bounds the host passed is cut at them (never read past them)
  const int nblocks = min((n + kBlock - 1) / kBlock, min(bt_stride, max_parts * kPartBlocks));
  if (b0 >= nblocks) return;
  const int b1 = min(nblocks, b0 + kPartBlocks);
  const int nparts = (nblocks + kPartBlocks - 1) / kPartBlocks;
  const int g = lane >> 4, c = lane & 15;

  WaveState<DT, D> st;
  load_q<DT, D>(st, q + ((int64_t)qb * hq + h * G + (c < G ? c : 0)) * D, c < G, g);

  const int64_t head_off = (int64_t)h * Gm::kTile;
  const int64_t blk_elems = (int64_t)num_kv_heads * Gm::kTile;
  const int nw = (b0 + w < b1) ? (b1 - b0 - w + kWaves - 1) / kWaves : 0;  // blocks of this wave
  auto fetch = [&](TileBuf<DT, D>& tb, int i) {
    const int64_t phys = __builtin_amdgcn_readlane(btv, i);
    load_tile<DT, D, true>(kp + phys * blk_elems + head_off, vp + phys * blk_elems + head_off,
                           tb.k, tb.v, lane);
  };
  auto consume = [&](TileBuf<DT, D>& tb, int i) {
    attend_block<DT, D>(st, tb.k, tb.v, (b0 + w + kWaves * i) * kBlock, n, n - 1, scale_log2, g);
  };
  // two register buffers: the next tile is in flight while this one is used
  TileBuf<DT, D> A, B;
  if (nw > 0) fetch(A, 0);
  for (int i = 0; i < nw; i += 2) {
    if (i + 1 < nw) fetch(B, i + 1);
    consume(A, i);
    if (i + 1 < nw) {
      if (i + 2 < nw) fetch(A, i + 2);
      consume(B, i + 1);
    }
  }

  // merge the four wavefronts through LDS
  __shared__ float sm_m[kWaves][16], sm_l[kWaves][16];
  __shared__ float sm_o[kWaves][G][D];
  float lsum = st.l + shfl_xor(st.l, 16);
  lsum += shfl_xor(lsum, 32);
  if (g == 0) {
    sm_m[w][c] = st.m;
    sm_l[w][c] = lsum;
  }
  if (c < G) {
#pragma unroll
    for (int nn = 0; nn < Gm::kN; ++nn)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[w][c][nn * 16 + 4 * g + i] = st.acc[nn][i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int cc = e / D, d = e - cc * D;
    float M = sm_m[0][cc];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww][cc]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(sm_m[ww][cc] - M);  // wavefronts without blocks: -inf -> 0
      num += f * sm_o[ww][cc][d];
      den += f * sm_l[ww][cc];
    }
    if (nparts == 1) {
      store_elem<DT>(out, ((int64_t)qb * hq + h * G + cc) * D + d, num / den);
    } else {
      const int64_t idx = ((int64_t)s * max_parts + part) * hq + h * G + cc;
      ws_o[idx * D + d] = num / den;
      if (d == 0) {
        ws_ml[2 * idx] = M;
        ws_ml[2 * idx + 1] = den;
      }
    }
  }
}

// Merge of decode partitions, one workgroup per (sequence, KV head):
//   o = sum_p 2^(m_p - M) l_p o_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// The partition weights go through LDS; every output element then sums its
// partitions with independent loads.  Dynamic LDS: max_parts * G floats.
template <class DT, int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    typename DT::T* __restrict__ out, const float* __restrict__ ws_o,
    const float* __restrict__ ws_ml, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ qsl, int num_kv_heads, int max_parts, int bt_stride) {
  extern __shared__ float sm_w[];  // [nparts][G]
  __shared__ float sm_M[G], sm_den[G];
  const int s = blockIdx.x / num_kv_heads, h = blockIdx.x % num_kv_heads;
  const int qb = qsl[s];
  if (qsl[s + 1] - qb != 1) return;
  const int n = seq_lens[s];
  const int nblocks = min((n + kBlock - 1) / kBlock, min(bt_stride, max_parts * kPartBlocks));
  const int nparts = (nblocks + kPartBlocks - 1) / kPartBlocks;
  if (nparts <= 1) return;
  const int hq = num_kv_heads * G;
  const int64_t base = (int64_t)s * max_parts * hq + h * G;  // (partition 0, head h*G)
  for (int t = threadIdx.x; t < nparts * G; t += blockDim.x) {
    const int p = t / G, cc = t - p * G;
    sm_w[t] = ws_ml[2 * (base + (int64_t)p * hq + cc)];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float M = -INFINITY;
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, sm_w[p * G + threadIdx.x]);
    sm_M[threadIdx.x] = M;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < nparts * G; t += blockDim.x) {
    const int p = t / G, cc = t - p * G;
    sm_w[t] = fast_exp2(sm_w[t] - sm_M[cc]) * ws_ml[2 * (base + (int64_t)p * hq + cc) + 1];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float den = 0.f;
    for (int p = 0; p < nparts; ++p) den += sm_w[p * G + threadIdx.x];
    sm_den[threadIdx.x] = den;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int cc = e / D, d = e - cc * D;
    const float* o = ws_o + (base + cc) * D + d;
    const int64_t step = (int64_t)hq * D;  // one partition further
    float num = 0.f;
    int p = 0;
    for (; p + 4 <= nparts; p += 4) {
      const float o0 = o[(p + 0) * step], o1 = o[(p + 1) * step];
      const float o2 = o[(p + 2) * step], o3 = o[(p + 3) * step];
      num += sm_w[(p + 0) * G + cc] * o0;
      num += sm_w[(p + 1) * G + cc] * o1;
      num += sm_w[(p + 2) * G + cc] * o2;
      num += sm_w[(p + 3) * G + cc] * o3;
    }
    for (; p < nparts; ++p) num += sm_w[p * G + cc] * o[p * step];
    store_elem<DT>(out, ((int64_t)qb * hq + h * G + cc) * D + d, num / sm_den[cc]);
  }
}

// ---------------------------------------------------------------------------
// Prefill chunks (q_len > 1): grid (num_kv_heads * q_tiles, num_seqs).  Each
// wavefront owns 16/G query tokens x G heads and scans every block its last
// token can see, causal inside the chunk.
// ---------------------------------------------------------------------------
template <class DT, int D, int G>
__global__ __launch_bounds__(256) void prefill_kernel(
    const typename DT::T* __restrict__ q, typename DT::T* __restrict__ out,
    const typename DT::T* __restrict__ kp, const typename DT::T* __restrict__ vp,
    const int32_t* __restrict__ bt, int bt_stride, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ qsl, int num_kv_heads, float scale_log2) {
  typedef Geo<DT, D> Gm;
  constexpr int kTokW = 16 / G;            // query tokens per wavefront
  constexpr int kTokWG = kWaves * kTokW;   // query tokens per workgroup
  const int s = blockIdx.y;
  const int h = blockIdx.x % num_kv_heads;
  const int tile = blockIdx.x / num_kv_heads;
  const int qb = qsl[s];
  const int q_len = qsl[s + 1] - qb;
  if (q_len <= 1) return;
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
// host side
// ---------------------------------------------------------------------------

struct AttnArgs {
  const void* q;
  void* out;
  const void* kp;
  const void* vp;
  const int32_t* bt;
  int bt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int num_seqs, num_kv_heads, max_q_len, max_parts;
  float scale_log2;
  float* ws_o;
  float* ws_ml;
  hipStream_t stream;
};

template <class DT, int D, int G>
static int launch(const AttnArgs& a) {
  typedef typename DT::T T;
  dim3 blk(256);
  const int64_t items = (int64_t)a.num_kv_heads * a.max_parts * a.num_seqs;
  const int64_t grid = (items + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((decode_kernel<DT, D, G>), dim3((unsigned)grid), blk, 0, a.stream,
                     (const T*)a.q, (T*)a.out, (const T*)a.kp, (const T*)a.vp, a.bt, a.bt_stride,
                     a.seq_lens, a.qsl, a.num_seqs, a.num_kv_heads, a.scale_log2, a.max_parts,
                     a.ws_o, a.ws_ml);
  if (a.max_parts > 1)
    hipLaunchKernelGGL((decode_merge_kernel<DT, D, G>), dim3(a.num_seqs * a.num_kv_heads), blk,
                       (size_t)a.max_parts * G * sizeof(float), a.stream, (T*)a.out, a.ws_o,
                       a.ws_ml, a.seq_lens, a.qsl, a.num_kv_heads, a.max_parts, a.bt_stride);
  if (a.max_q_len > 1) {
    constexpr int kTokWG = kWaves * (16 / G);
    dim3 gp(a.num_kv_heads * ((a.max_q_len + kTokWG - 1) / kTokWG), a.num_seqs);
    hipLaunchKernelGGL((prefill_kernel<DT, D, G>), gp, blk, 0, a.stream, (const T*)a.q, (T*)a.out,
                       (const T*)a.kp, (const T*)a.vp, a.bt, a.bt_stride, a.seq_lens, a.qsl,
                       a.num_kv_heads, a.scale_log2);
  }
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

template <class DT, int D>
static int dispatch_g(const AttnArgs& a, int G) {
  switch (G) {
    case 1: return launch<DT, D, 1>(a);
    case 2: return launch<DT, D, 2>(a);
    case 4: return launch<DT, D, 4>(a);
    case 8: return launch<DT, D, 8>(a);
  }
  return PKV_ERR_UNSUPPORTED;
}

template <class DT>
static int dispatch_d(const AttnArgs& a, int D, int G) {
  switch (D) {
    case 64: return dispatch_g<DT, 64>(a, G);
    case 128: return dispatch_g<DT, 128>(a, G);
    case 256:
      if constexpr (DT::kBytes == 2) return dispatch_g<DT, 256>(a, G);
      break;
  }
  return PKV_ERR_UNSUPPORTED;
}

static int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

static int64_t max_partitions(int32_t max_seq_len) {
  const int64_t nb = ((int64_t)max_seq_len + kBlock - 1) / kBlock;
  const int64_t p = (nb + kPartBlocks - 1) / kPartBlocks;
  return p < 1 ? 1 : p;
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t pkv_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_tokens,
                                                      int32_t max_seq_len, int32_t num_q_heads,
                                                      int32_t head_dim) {
  if (num_seqs < 0 || num_q_tokens < 0 || max_seq_len < 0 || num_q_heads <= 0 || head_dim <= 0)
    return 0;
  const int64_t parts = max_partitions(max_seq_len);
  const int64_t rows = (int64_t)num_seqs * parts * num_q_heads;
  // (m, l) pairs, then the partition outputs, each section 256-byte aligned
  return (size_t)(round256(rows * 2 * 4) + round256(rows * (int64_t)head_dim * 4));
}

extern "C" int pkv_paged_attention(const pkv_cache_t* cache, int32_t layer, void* out,
                                   const void* q, const int32_t* block_tables, int32_t bt_stride,
                                   const int32_t* seq_lens, const int32_t* query_start_loc,
                                   int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len,
                                   int32_t max_seq_len, int32_t num_q_heads, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_cache(cache);
  if (rc != PKV_OK) return rc;
  if (layer < 0 || layer >= cache->num_layers) return PKV_ERR_INVALID_ARGUMENT;
  if (num_seqs < 0 || num_q_tokens < 0 || max_q_len < 0 || max_seq_len < 0 || bt_stride < 0)
    return PKV_ERR_INVALID_ARGUMENT;
  if (num_seqs == 0 || num_q_tokens == 0) return PKV_OK;
  if (num_seqs > 65535 || bt_stride < 1) return PKV_ERR_INVALID_ARGUMENT;
  if (!out || !q || !block_tables || !seq_lens || !query_start_loc)
    return PKV_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(out)) return PKV_ERR_INVALID_ARGUMENT;
  if (max_q_len < 1 || max_q_len > num_q_tokens) return PKV_ERR_INVALID_ARGUMENT;
  if ((int64_t)bt_stride * kBlock < max_seq_len) return PKV_ERR_INVALID_ARGUMENT;
  if (!(scale == scale) || !isfinite(scale)) return PKV_ERR_INVALID_ARGUMENT;
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads) return PKV_ERR_INVALID_ARGUMENT;
  const int G = num_q_heads / cache->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return PKV_ERR_UNSUPPORTED;
  if (cache->dtype == PKV_F32 && cache->head_dim == 256) return PKV_ERR_UNSUPPORTED;
  // decode grid (padded to whole XCD rounds) and the merge's LDS must fit their limits
  if ((int64_t)num_seqs * cache->num_kv_heads * max_partitions(max_seq_len) + kXcds > 0x7fffffff)
    return PKV_ERR_INVALID_ARGUMENT;
  if (max_partitions(max_seq_len) * G * (int64_t)sizeof(float) > 65536) return PKV_ERR_UNSUPPORTED;
  const size_t need = pkv_paged_attention_workspace_bytes(num_seqs, num_q_tokens, max_seq_len,
                                                          num_q_heads, cache->head_dim);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PKV_ERR_WORKSPACE;

  const int64_t layer_elems = (int64_t)layer * cache->num_blocks * cache->num_kv_heads * kBlock *
                              cache->head_dim;
  const int eb = elem_bytes(cache->dtype);
  AttnArgs a;
  a.q = q;
  a.out = out;
  a.kp = (const char*)cache->k_pool + layer_elems * eb;
  a.vp = (const char*)cache->v_pool + layer_elems * eb;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.seq_lens = seq_lens;
  a.qsl = query_start_loc;
  a.num_seqs = num_seqs;
  a.num_kv_heads = cache->num_kv_heads;
  a.max_q_len = max_q_len;
  a.max_parts = (int)max_partitions(max_seq_len);
  a.scale_log2 = scale * 1.4426950408889634f;
  const int64_t rows = (int64_t)num_seqs * a.max_parts * num_q_heads;
  a.ws_ml = (float*)workspace;
  a.ws_o = (float*)((char*)workspace + round256(rows * 2 * 4));
  a.stream = (hipStream_t)stream;
  switch (cache->dtype) {
    case PKV_F32: return dispatch_d<TF32>(a, cache->head_dim, G);
    case PKV_F16: return dispatch_d<TF16>(a, cache->head_dim, G);
    case PKV_BF16: return dispatch_d<TBF16>(a, cache->head_dim, G);
  }
  return PKV_ERR_UNSUPPORTED;
}
