// PagedAttention for gfx950: decode (split-K over the paged context, then a
// merge of the partitions) and the paged_attention entry point, which also
// launches the prefill-chunk kernels of prefill.hip.
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

#include "attn_common.h"
#include "pkv_host.h"

namespace pkv {

constexpr int kPartBlocks = 64;  // blocks per decode partition (1024 tokens)
constexpr int kPerWave = kPartBlocks / kWaves;  // blocks of a partition per wavefront
constexpr int kXcds = 8;         // accelerator complex dies of an MI355X
static_assert(kPerWave <= 64, "one block-table entry per lane");


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

// Work lists of one call, written by decode_plan_kernel: the live decode items
// (sequence, partition) in sequence order, and the sequences whose partitions
// need merging.  plan[0] = number of items, plan[1] = number of merges.
struct DecodePlan {
  int32_t* counts;
  int2* items;     // [num_seqs * max_parts]
  int32_t* merge;  // [num_seqs]
};

// One workgroup of 1024 threads; thread t owns sequences [t*k, t*k + k).
// A decode row (q_len = 1) of a sequence with n > 0 tokens has one item per
// 1024-token partition; an empty sequence has one item (its zero output).
__global__ __launch_bounds__(1024) void decode_plan_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int num_seqs,
    int bt_stride, int max_parts, int32_t* __restrict__ counts, int2* __restrict__ items,
    int32_t* __restrict__ merge) {
  __shared__ int sm_tot[2][1024 / kWave];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int k = (num_seqs + blockDim.x - 1) / blockDim.x;
  const int s0 = tid * k;
  int nit = 0, nmg = 0;
  for (int j = 0; j < k; ++j) {
    const int s = s0 + j;
    if (s >= num_seqs) break;
    if (qsl[s + 1] - qsl[s] != 1) continue;
    const int n = seq_lens[s];
    const int nb = n > 0 ? min((n + kBlock - 1) / kBlock, min(bt_stride, max_parts * kPartBlocks)) : 0;
    const int np = n > 0 ? (nb + kPartBlocks - 1) / kPartBlocks : 1;
    nit += np;
    nmg += np > 1;
  }
  // exclusive prefix of (nit, nmg) over the workgroup: wave scan, then wave totals
  int xi = nit, xm = nmg;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int yi = __shfl_up(xi, off), ym = __shfl_up(xm, off);
    if (lane >= off) {
      xi += yi;
      xm += ym;
    }
  }
  if (lane == kWave - 1) {
    sm_tot[0][w] = xi;
    sm_tot[1][w] = xm;
  }
  __syncthreads();
  int bi = 0, bm = 0, ti = 0, tm = 0;
  for (int ww = 0; ww < (int)(blockDim.x / kWave); ++ww) {
    if (ww < w) {
      bi += sm_tot[0][ww];
      bm += sm_tot[1][ww];
    }
    ti += sm_tot[0][ww];
    tm += sm_tot[1][ww];
  }
  int pi = bi + xi - nit, pm = bm + xm - nmg;
  for (int j = 0; j < k; ++j) {
    const int s = s0 + j;
    if (s >= num_seqs) break;
    if (qsl[s + 1] - qsl[s] != 1) continue;
    const int n = seq_lens[s];
    const int nb = n > 0 ? min((n + kBlock - 1) / kBlock, min(bt_stride, max_parts * kPartBlocks)) : 0;
    const int np = n > 0 ? (nb + kPartBlocks - 1) / kPartBlocks : 1;
    for (int p = 0; p < np; ++p) items[pi + p] = int2{s, p};
    pi += np;
    if (np > 1) merge[pm++] = s;
  }
  if (tid == 0) {
    counts[0] = ti;
    counts[1] = tm;
  }
}

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

template <class DT, int D, int G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(decode_occupancy<DT, D>())))
void decode_kernel(const typename DT::T* __restrict__ q, typename DT::T* __restrict__ out,
                   const typename DT::T* __restrict__ kp, const typename DT::T* __restrict__ vp,
                   const int32_t* __restrict__ bt, int bt_stride,
                   const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
                   int num_kv_heads, float scale_log2, int max_parts,
                   float* __restrict__ ws_o, float* __restrict__ ws_ml, DecodePlan plan,
                   int contiguous) {
  typedef Geo<DT, D> Gm;
  const int j = xcd_unit(blockIdx.x, plan.counts[0] * num_kv_heads);
  if (j < 0) return;
  const int h = j % num_kv_heads;
  const int2 item = plan.items[j / num_kv_heads];
  const int s = item.x, part = item.y;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int b0 = part * kPartBlocks;
  const int32_t* btr = bt + (int64_t)s * bt_stride;
  // block-table entries of this wavefront's blocks b0 + w + 4i, one per lane,
  // loaded alongside the sequence metadata (bounded by the table width only).
  // Contiguous storage (the baseline without paging): bt[s] is the sequence's
  // first block and block i is bt[s] + i.
  int btv = 0;
  {
    const int bi = b0 + w + kWaves * lane;
    if (lane < kPerWave && bi < bt_stride) btv = contiguous ? bt[s] + bi : btr[bi];
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
  // two register buffers, both in flight: each iteration uses a tile and refills its buffer
  // two tiles ahead.  The prologue waits once for Q and the first two tiles; after that
  // every wait covers exactly the tile about to be used, and the refill is kept after the
  // use (a hoisted load would need fresh registers and a copy at the loop edge).
  TileBuf<DT, D> A, B;
  if (nw > 0) fetch(A, 0);
  if (nw > 1) fetch(B, 1);
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero
  int i = 0;
  for (; i + 3 < nw; i += 2) {
    consume(A, i);
    __builtin_amdgcn_sched_barrier(0);
    fetch(A, i + 2);
    consume(B, i + 1);
    __builtin_amdgcn_sched_barrier(0);
    fetch(B, i + 3);
  }
  if (i < nw) consume(A, i);
  if (i + 2 < nw) fetch(A, i + 2);
  if (i + 1 < nw) consume(B, i + 1);
  if (i + 2 < nw) consume(A, i + 2);

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
// Every thread owns outputs of one query head and loads the (m, l, o) of all
// partitions at once, kMergeBatch partitions per round, so a merge costs one
// memory round trip after the sequence metadata (C3-like contexts: one round).
constexpr int kMergeBatch = 8;

template <class DT, int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    typename DT::T* __restrict__ out, const float* __restrict__ ws_o,
    const float* __restrict__ ws_ml, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ qsl, int num_kv_heads, int max_parts, int bt_stride,
    DecodePlan plan) {
  const int j = xcd_unit(blockIdx.x, plan.counts[1] * num_kv_heads);
  if (j < 0) return;
  const int s = plan.merge[j / num_kv_heads], h = j % num_kv_heads;
  const int qb = qsl[s];
  if (qsl[s + 1] - qb != 1) return;
  const int n = seq_lens[s];
  const int nblocks = min((n + kBlock - 1) / kBlock, min(bt_stride, max_parts * kPartBlocks));
  const int nparts = (nblocks + kPartBlocks - 1) / kPartBlocks;
  if (nparts <= 1) return;
  const int hq = num_kv_heads * G;
  const int64_t base = (int64_t)s * max_parts * hq + h * G;  // (partition 0, head h*G)
  for (int e = threadIdx.x; e < G * D; e += blockDim.x) {
    const int cc = e / D, d = e - cc * D;
    const int64_t row0 = base + cc;  // this head's row in partition 0; + p*hq for partition p
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int p0 = 0; p0 < nparts; p0 += kMergeBatch) {
      float mp[kMergeBatch], lp[kMergeBatch], op[kMergeBatch];
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const int p = min(p0 + k, nparts - 1);  // past the end: re-read the last (weight 0)
        const int64_t row = row0 + (int64_t)p * hq;
        mp[k] = ws_ml[2 * row];
        lp[k] = ws_ml[2 * row + 1];
        op[k] = ws_o[row * D + d];
      }
      float bm = M;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) bm = fmaxf(bm, mp[k]);
      const float f0 = fast_exp2(M - bm);  // M = -inf on the first round: 0
      num *= f0;
      den *= f0;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const float f = p0 + k < nparts ? fast_exp2(mp[k] - bm) * lp[k] : 0.f;
        num += f * op[k];
        den += f;
      }
      M = bm;
    }
    store_elem<DT>(out, ((int64_t)qb * hq + h * G + cc) * D + d, num / den);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------


template <class DT, int D, int G>
static int launch(const AttnArgs& a) {
  typedef typename DT::T T;
  dim3 blk(256);
  DecodePlan plan;
  plan.counts = (int32_t*)a.ws_plan;
  plan.items = (int2*)((char*)a.ws_plan + 256);
  plan.merge = (int32_t*)((char*)plan.items + (size_t)a.num_seqs * a.max_parts * sizeof(int2));
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, a.stream, a.seq_lens, a.qsl,
                     a.num_seqs, a.bt_stride, a.max_parts, plan.counts, plan.items, plan.merge);
  // grids sized for every sequence in every partition; the plan's counts cut them short
  const int64_t units = (int64_t)a.num_kv_heads * a.max_parts * a.num_seqs;
  const int64_t grid = (units + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((decode_kernel<DT, D, G>), dim3((unsigned)grid), blk, 0, a.stream,
                     (const T*)a.q, (T*)a.out, (const T*)a.kp, (const T*)a.vp, a.bt, a.bt_stride,
                     a.seq_lens, a.qsl, a.num_kv_heads, a.scale_log2, a.max_parts, a.ws_o,
                     a.ws_ml, plan, a.contiguous);
  if (a.max_parts > 1) {
    const int64_t mgrid = ((int64_t)a.num_seqs * a.num_kv_heads + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((decode_merge_kernel<DT, D, G>), dim3((unsigned)mgrid), blk, 0, a.stream,
                       (T*)a.out, a.ws_o, a.ws_ml, a.seq_lens, a.qsl, a.num_kv_heads,
                       a.max_parts, a.bt_stride, plan);
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

static int64_t decode_plan_bytes(int64_t num_seqs, int64_t max_parts) {
  return round256(256 + num_seqs * max_parts * (int64_t)sizeof(int2) + num_seqs * 4);
}

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
  // decode (m, l) pairs, decode partition outputs, prefill work list, decode plan; each
  // section 256-byte aligned
  return (size_t)(round256(rows * 2 * 4) + round256(rows * (int64_t)head_dim * 4) +
                  round256(prefill_workspace_bytes(num_seqs, num_q_tokens, num_q_heads)) +
                  decode_plan_bytes(num_seqs, parts));
}

static int attention_impl(const pkv_cache_t* cache, int32_t layer, void* out, const void* q,
                          const int32_t* block_tables, int32_t bt_stride, int contiguous,
                          const int32_t* seq_lens, const int32_t* query_start_loc,
                          int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len,
                          int32_t max_seq_len, int32_t num_q_heads, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
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
  // the decode grid (padded to whole XCD rounds) must fit its limit
  if ((int64_t)num_seqs * cache->num_kv_heads * max_partitions(max_seq_len) + kXcds > 0x7fffffff)
    return PKV_ERR_INVALID_ARGUMENT;
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
  a.contiguous = contiguous;
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
  a.ws_pf = (char*)workspace + round256(rows * 2 * 4) + round256(rows * (int64_t)cache->head_dim * 4);
  a.pf_items = prefill_items_bound(num_seqs, num_q_tokens, num_q_heads);
  a.ws_plan = (char*)a.ws_pf + round256(prefill_workspace_bytes(num_seqs, num_q_tokens, num_q_heads));
  a.stream = (hipStream_t)stream;
  // decode rows (q_len = 1), then prefill chunks: small ones per wavefront, large ones tiled
  switch (cache->dtype) {
    case PKV_F32: rc = dispatch_d<TF32>(a, cache->head_dim, G); break;
    case PKV_F16: rc = dispatch_d<TF16>(a, cache->head_dim, G); break;
    case PKV_BF16: rc = dispatch_d<TBF16>(a, cache->head_dim, G); break;
    default: return PKV_ERR_UNSUPPORTED;
  }
  if (rc != PKV_OK || max_q_len <= 1) return rc;
  rc = launch_prefill_small(a, cache->dtype, cache->head_dim, G);
  if (rc != PKV_OK || (int64_t)max_q_len * G <= kSmallChunkCols) return rc;
  return launch_prefill_tiled(a, cache->dtype, cache->head_dim, G);
}

extern "C" int pkv_paged_attention(const pkv_cache_t* cache, int32_t layer, void* out,
                                   const void* q, const int32_t* block_tables, int32_t bt_stride,
                                   const int32_t* seq_lens, const int32_t* query_start_loc,
                                   int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len,
                                   int32_t max_seq_len, int32_t num_q_heads, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return attention_impl(cache, layer, out, q, block_tables, bt_stride, 0, seq_lens,
                        query_start_loc, num_seqs, num_q_tokens, max_q_len, max_seq_len,
                        num_q_heads, scale, workspace, workspace_bytes, stream);
}

extern "C" int pkv_contiguous_attention(const pkv_cache_t* cache, int32_t layer, void* out,
                                        const void* q, const int32_t* first_block,
                                        const int32_t* seq_lens, const int32_t* query_start_loc,
                                        int32_t num_seqs, int32_t num_q_tokens,
                                        int32_t max_seq_len, int32_t num_q_heads, float scale,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  // decode rows only: the same kernels, the blocks of a sequence addressed as one run
  const int32_t run = (int32_t)(((int64_t)max_seq_len + kBlock - 1) / kBlock);
  return attention_impl(cache, layer, out, q, first_block, run > 0 ? run : 1, 1, seq_lens,
                        query_start_loc, num_seqs, num_q_tokens, 1, max_seq_len, num_q_heads,
                        scale, workspace, workspace_bytes, stream);
}
