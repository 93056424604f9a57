// Device building blocks shared by the attention kernels of libpkv (decode and
// prefill): tile geometry, the per-wavefront online-softmax state, tile loads
// and the 16-token block step.  Tile layouts are those of include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pkv.h"
#include "pkv_device.h"

namespace pkv {

constexpr int kWaves = 4;  // wavefronts per decode workgroup
constexpr int kXcds = 8;   // accelerator complex dies of an MI355X

// Workgroup id -> index into a list of `live` work units.  Dispatch deals
// consecutive ids round-robin over the XCDs; unit j = (id % 8) * C + id / 8
// with C = ceil(live / 8) gives every XCD one contiguous run of units.  Ids
// whose unit is past the list (the grid is sized for the worst case) come
// last in dispatch order and return at once; returns -1 for them.
__device__ __forceinline__ int xcd_unit(int id, int live) {
  const int per = (live + kXcds - 1) / kXcds;
  const int r = id / kXcds;
  if (r >= per) return -1;
  const int j = (id % kXcds) * per + r;
  return j < live ? j : -1;
}


template <class DT, int D>
struct Geo {
  static constexpr int kChunks = D * DT::kBytes / 64;  // 16-byte operand chunks per lane per tile
  static constexpr int kN = D / 16;                    // 16-dim slices of the output
  static constexpr int kTile = kBlock * D;             // elements per (block, head) tile
  static constexpr int kX = 16 / DT::kBytes;           // elements per 16-byte chunk
};

// The exponentials of a column use a reference max that may lag its running max
// by up to 2^kMaxLag (weights <= 256, far from overflow in fp32 and in the 16-bit
// weight types); (m, l, o) stay consistent with whatever reference they carry.
constexpr float kMaxLag = 8.f;

template <class DT, int D>
struct WaveState {
  u32x4 q[Geo<DT, D>::kChunks];  // Q^T operand of this lane's column
  f32x4 acc[Geo<DT, D>::kN];     // O^T: lane 16g+c holds dims 16n+4g..16n+4g+3 of column c
  float m;                       // reference max of the column (log2 domain)
  float l;                       // running sum of this lane's 4 tokens per block (relative to m)
};

template <class DT, int D>
__device__ __forceinline__ void init_state(WaveState<DT, D>& st) {
#pragma unroll
  for (int n = 0; n < Geo<DT, D>::kN; ++n) st.acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
}

// Q^T operand chunk kk of lane 16g + c: head dims (4kk+g)*x .. +x of the lane's column
template <class DT, int D>
__device__ __forceinline__ void load_q(WaveState<DT, D>& st, const typename DT::T* qrow, bool valid,
                                       int g) {
  const u32x4* q4 = (const u32x4*)qrow;
#pragma unroll
  for (int kk = 0; kk < Geo<DT, D>::kChunks; ++kk)
    st.q[kk] = valid ? q4[kk * 4 + g] : u32x4{0, 0, 0, 0};
  init_state(st);
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

// max over the four lanes c, c+16, c+32, c+48 of a column (row swaps, no LDS)
__device__ __forceinline__ float col_max4(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
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
  const float bm = col_max4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
  // st.m is the reference max of the exponentials: it moves (and the accumulators are
  // rescaled) only when some column's block max exceeds it by more than 2^kMaxLag, a
  // wave-wide decision; the first visible key of a column (st.m = -inf) always moves it
  if (__builtin_amdgcn_ballot_w64(bm > st.m + kMaxLag)) {
    const float mn = fmaxf(st.m, bm);
    const float alpha = mn == -INFINITY ? 1.f : fast_exp2(st.m - mn);
#pragma unroll
    for (int nn = 0; nn < Gm::kN; ++nn) st.acc[nn] *= alpha;
    st.l *= alpha;
    st.m = mn;
  }
  const float mu = st.m == -INFINITY ? 0.f : st.m;  // a column with nothing visible yet
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - mu);

  // slots at or past the sequence end may hold anything (even NaN): select, never multiply
  const bool tail = tok0 + kBlock > n;
  if constexpr (DT::kBytes == 2) {
    uint32_t pd0, pd1, pl0 = 0, pl1 = 0;
    if constexpr (__is_same(DT, TBF16)) {
      pd0 = pack2_bf16(p[0], p[1]);
      pd1 = pack2_bf16(p[2], p[3]);
    } else {
      pd0 = pack2_f16(p[0], p[1]);
      pd1 = pack2_f16(p[2], p[3]);
    }
    // the sum uses the weights as P.V sees them, so the output is a convex
    // combination of V rows.  bf16 keeps 8 significant bits, too few for rows of a
    // few keys with large values: the weights enter P.V as hi + lo, the bf16 value
    // and its bf16 rounding residue, which agree with the fp32 weights to about 16
    // bits, so the sum takes the fp32 weights themselves.
    float ps;
    if constexpr (__is_same(DT, TBF16)) {
      const float h0 = bf16_bits_to_f32(pd0 & 0xffffu), h1 = bf16_bits_to_f32(pd0 >> 16);
      const float h2 = bf16_bits_to_f32(pd1 & 0xffffu), h3 = bf16_bits_to_f32(pd1 >> 16);
      pl0 = pack2_bf16(p[0] - h0, p[1] - h1);
      pl1 = pack2_bf16(p[2] - h2, p[3] - h3);
      ps = (p[0] + p[1]) + (p[2] + p[3]);
    } else {
      ps = ((float)__builtin_bit_cast(_Float16, (uint16_t)(pd0 & 0xffffu)) +
            (float)__builtin_bit_cast(_Float16, (uint16_t)(pd0 >> 16))) +
           ((float)__builtin_bit_cast(_Float16, (uint16_t)(pd1 & 0xffffu)) +
            (float)__builtin_bit_cast(_Float16, (uint16_t)(pd1 >> 16)));
    }
    st.l += ps;
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
      if constexpr (__is_same(DT, TBF16)) {
        st.acc[2 * i] = mma_k16(vr[i].x, vr[i].y, pl0, pl1, st.acc[2 * i], DT());
        st.acc[2 * i + 1] = mma_k16(vr[i].z, vr[i].w, pl0, pl1, st.acc[2 * i + 1], DT());
      }
    }
  } else {
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
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

// Four consecutive outputs (i a multiple of 4), rounded to the output type.
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

// Arguments of one paged_attention call, as the kernels' launchers see them.
struct AttnArgs {
  const void* q;
  void* out;
  const void* kp;
  const void* vp;
  const int32_t* bt;  // block tables, or first blocks of contiguous runs (contiguous != 0)
  int bt_stride;
  int contiguous;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int num_seqs, num_kv_heads, max_q_len, max_parts;
  bool uniform_q;     // every row has max_q_len query tokens (num_q_tokens = num_seqs * max_q_len)
  bool order_by_part; // rows share prefixes of blocks: decode work partition-major
  float scale_log2;
  float* ws_o;
  float* ws_ml;
  void* ws_pf;        // tiled-prefill work lists, queue counters and split partials
  int64_t pf_items;   // items bound (q-tile items; each extra piece takes one more slot)
  int64_t pf_slots;   // partial slots for split items (0: no chunk can exist)
  void* ws_plan;      // decode work lists (decode_plan_kernel)
  hipStream_t stream;
};

// Launchers of the prefill kernels (prefill.hip) for chunks wider than
// small_chunk_max_cols (query token, head) columns; narrower rows take the
// partitioned decode kernel.  Each returns PKV_OK or a PKV_ERR_* status and
// only enqueues work on a.stream.
//   16-bit types: planned work list + LDS-tiled persistent kernel
//   fp32: one wavefront per 16 columns
int launch_prefill_wave(const AttnArgs& a, int dtype, int head_dim, int G);
int launch_prefill_tiled(const AttnArgs& a, int dtype, int head_dim, int G);
// Widest row, in (query token, head) columns, the decode kernel takes: two
// 16-column tiles per wavefront for 16-bit types up to head_dim 128, else one.
inline int small_chunk_max_cols(int dtype, int head_dim) {
  return (dtype != PKV_F32 && head_dim <= 128) ? 32 : 16;
}
// Bounds of the tiled prefill's work items and split partial slots, and the
// workspace bytes they, the merge list and the queue counters take.
int64_t prefill_items_bound(int64_t num_seqs, int64_t num_q_tokens, int64_t num_q_heads);
int64_t prefill_slots_bound(int64_t num_seqs, int64_t num_q_tokens);
int64_t prefill_workspace_bytes(int64_t num_seqs, int64_t num_q_tokens, int64_t num_q_heads,
                                int64_t head_dim);

}  // namespace pkv
