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
// Decode splits the context of a sequence into partitions of 1024, 2048, 3072 or
// 4096 tokens, a size a plan kernel chooses per call from the lengths of the whole
// batch (1024 when rows share blocks).  Short chunks (a few query tokens, e.g. the
// k+1 tokens that verify a speculative draft) take the same kernel with their
// q_len * G columns in one or two column tiles, so K/V are read once per row.
// One workgroup per work unit (sequence, partition, KV head): its four wavefronts
// take every fourth block, streaming K/V tiles with non-temporal loads (each tile
// is read once), merge through LDS, and a second kernel merges the partitions of
// long sequences with the log-sum-exp rule.  Work items are listed longest first
// and dealt to the XCDs in rounds (hardware dispatch deals consecutive workgroups
// round-robin over the eight XCDs), or partition-major when rows share blocks, so
// that the rows reading one tile run together on one XCD.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "attn_common.h"
#include "pkv_host.h"

namespace pkv {

constexpr int kPartBlocks = 64;  // blocks of the shortest decode partition (1024 tokens)
constexpr int kOddRounds = 10;   // dealing cycle: odd XCDs take 10 items per 11 of an even one
constexpr int kPartChoices = 4;  // partitions of 1, 2, 3 or 4 x kPartBlocks blocks
constexpr int kPartMax = kPartChoices * kPartBlocks;
constexpr int kPlanLevels = 2048;  // partition indices the plan orders items by (2M tokens)

// ---------------------------------------------------------------------------
// Decode and short chunks: a 1-D grid over (item, KV head), 4 wavefronts each.
// A row of q_len query tokens has q_len * G (token, head) columns per KV head;
// the kernel instantiation with CT column tiles takes the rows with
// (CT-1)*16 < q_len * G <= CT*16, so a decode row (q_len = 1) fills G columns
// of one tile and a speculative-decoding verify row of k+1 tokens fills
// (k+1) * G columns (blog page, advanced features, speculative decoding).
// ---------------------------------------------------------------------------

// Waves per SIMD the register allocation must allow: three for one column
// tile of a 16-bit type up to head_dim 128 (enough K/V bytes in flight per
// CU), two for two tiles, otherwise whatever the kernel needs.
template <class DT, int D, int CT>
constexpr int decode_occupancy() {
  return (DT::kBytes == 2 && D <= 128) ? (CT == 1 ? 3 : 2) : 1;
}

// Work of one decode workgroup, as decode_plan_kernel writes it: sequence s,
// KV head h, blocks [b0, b1) (partition part of the row), the row's first query
// row qb, its query tokens and sequence length, and the workspace row of
// (this partition, token 0, head h*G) if the row is split over partitions
// (wrow < 0 otherwise).  One 48-byte record per item.
struct alignas(16) DecodeItem {
  int32_t s, h, b0, b1, qb, q_len, n, part;
  int64_t wrow, unused;
};

// Work lists of one call, written by decode_plan_kernel: the items of one-tile
// rows (class 1) and of two-tile rows (class 2), with h = 0, longest first
// (blocks per item in bins of 4, descending), or partition-major when the caller says that
// rows share prefixes of blocks (PKV_ATTN_SHARED_PREFIXES): partition 0 of every
// row, then partition 1 of every row that has one, and so on.  The order within
// one length or partition index is not kept.
//   Longest first: the items are dealt to the eight XCDs in rounds of eight, in
//   alternating directions, with the KV heads of an item together, so every XCD
//   takes its share of the long items first and the short ones fill the gaps at
//   the end (list scheduling, longest processing time first).
//   Partition-major: rows that share blocks read them at about the same time, so
//   an XCD's L2 serves most of those reads; workgroup units are (KV head, item)
//   pairs dealt to the eight XCDs in contiguous runs (xcd_unit).
// A sequence split over several partitions owns a run of workspace rows from some
// base r: row r + (p * q_len + t) * Hq + head holds partition p's result for query
// token t; one merge entry per (split sequence, query token).
// One merge: the output query row, the partition count, the workspace row of
// (partition 0, this token, head 0) and the rows between partitions.
struct MergeEntry {
  int32_t qrow, nparts, unused0, unused1;
  int64_t row0, pstride;
};

struct DecodePlan {
  int32_t* counts;    // [0] class-1 items, [1] merges, [2] class-2 items;
                      // nullptr: no plan, every row is one item (single-partition batches)
  DecodeItem* items;  // [2][cap]
  MergeEntry* merge;  // [num_seqs * 32]
  int num_seqs;
  int cap;            // num_seqs * max_parts
  int by_part;        // partition-major lists, units (KV head, item) in XCD runs;
                      // otherwise longest first, dealt to the XCDs in rounds of 8 items
};

// Blocks per partition of a row: pb for decode rows, the size the plan chose for
// the call; a multi-token row uses pb << shift, with the shift the plan chose so
// that the split rows fit the workspace.
__device__ __forceinline__ int part_blocks(int q_len, int pb, int shift) {
  return q_len > 1 ? pb << shift : pb;
}

// Column-tile class of a row: 1 or 2, or 0 for rows left to the prefill kernels
// (and rows with no query token, or more than the call's max_q_len).
__device__ __forceinline__ int row_class(int q_len, int max_q, int G, int max_cols) {
  const int64_t cols = (int64_t)q_len * G;
  if (q_len < 1 || q_len > max_q || cols > max_cols) return 0;
  return cols <= 16 ? 1 : 2;
}

// Fixed cost of one decode workgroup (launch, metadata, Q, merge through LDS) in
// the plan's time unit, one 16-token block step of a wavefront.
constexpr int kUnitCost = 2;
// An HBM write of split partials among the K/V reads costs about as much time as
// reading this many times its bytes (measured on the GQA decode workload).
constexpr int kPartialWeight = 11;
// Length bins of decode items: ceil(blocks / 4) - 1, the block steps of each wavefront
// of the workgroup minus one (items of the longest partition in the last bin).
constexpr int kSizeBins = kPartMax / kWaves;
static_assert(kSizeBins == kWave, "one length bin per lane");

__device__ __forceinline__ int size_bin(int blocks) {
  return blocks > 0 ? min((blocks + kWaves - 1) / kWaves, kSizeBins) - 1 : 0;
}

// One workgroup of 1024 threads; thread t owns sequences [t*k, t*k + k).  A
// small row of a sequence with n > 0 tokens has one item per partition; an
// empty sequence has one item (its zero output).  A split row has one merge
// entry per query token.  budget: workspace rows for split rows
// (each row is head_dim floats).
//
// Partition size.  The decode workgroups are list-scheduled, longest first, onto
// `slots` resident workgroups.  For each size of 1 to kPartChoices times
// kPartBlocks blocks the plan estimates the finish time in block steps: the ideal
// sum over (item, KV head) units of kUnitCost + ceil(blocks / 4) divided by
// slots; at least j + 1 times the (j * slots + 1)-th longest unit for j >= 0,
// since some workgroup runs j + 1 of the j * slots + 1 longest; plus the split
// partials' bytes weighed as kPartialWeight times K/V bytes.  The smallest
// estimate wins (ties: the larger partition, fewer partials).  Rows that share
// blocks (PKV_ATTN_SHARED_PREFIXES) keep kPartBlocks: their reads come mostly
// from L2, and more, shorter partitions read together serve more of them from
// there.  The partition size sets the rounding order of a row's sums, so it is
// the one way the batch and the hint reach a row's output bits (within the
// tolerance of the arithmetic: the result is the same attention).
//
// The partition shift of multi-token rows starts at 0 and grows until the split
// rows fit; this terminates, since once a partition spans max_parts * 1024
// tokens no multi-token row is split, and decode rows alone need at most
// num_seqs * max_parts * hq rows.
//
// Lists are counting-sorted by key: the length bin, longest first (the same
// per-bin counts the estimate used, while no multi-token row changed its
// partition size), or the partition index (partition-major).  Merge entries and
// workspace rows are handed out by atomic counters, in no particular order.
__global__ __launch_bounds__(1024) void decode_plan_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int num_seqs,
    int bt_stride, int max_parts, int max_q, int G, int max_cols, int hq, long long budget,
    int num_kv_heads, int slots, int row_bytes, int step_bytes, DecodePlan plan) {
  __shared__ int sm_hist[2][kPartChoices][kSizeBins];     // items per class, size, length bin
  __shared__ unsigned long long sm_pbytes[kPartChoices];  // split partials' bytes, per size
  __shared__ float sm_est[kPartChoices];
  __shared__ int sm_lvl[2][kPlanLevels];  // items per list key and class, then cursors
  __shared__ int sm_cnt[4];               // class-1 items, class-2 items, merge entries, cursor
  __shared__ unsigned long long sm_rows[2];  // workspace rows of split rows; cursor
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int k = (num_seqs + blockDim.x - 1) / blockDim.x;
  const int s0 = tid * k;
  auto blocks = [&](int n) {
    return n > 0 ? min((n + kBlock - 1) / kBlock, min(bt_stride, max_parts * kPartBlocks)) : 0;
  };
  // One row per thread (up to 1024 rows): the row's metadata is loaded once.
  int c_qb = 0, c_qe = 0, c_n = 0;
  if (k == 1 && s0 < num_seqs) {
    c_qb = qsl[s0];
    c_qe = qsl[s0 + 1];
    c_n = seq_lens[s0];
  }
  auto qb_of = [&](int s) { return k == 1 ? c_qb : qsl[s]; };
  auto qlen_of = [&](int s) { return k == 1 ? c_qe - c_qb : qsl[s + 1] - qsl[s]; };
  auto n_of = [&](int s) { return k == 1 ? c_n : seq_lens[s]; };
  const bool by_part = plan.by_part;
  const bool choose = max_parts > 1 && !by_part;
  for (int i = tid; i < 2 * kPartChoices * kSizeBins; i += blockDim.x) (&sm_hist[0][0][0])[i] = 0;
  if (by_part)
    for (int i = tid; i < 2 * max_parts; i += blockDim.x) sm_lvl[i / max_parts][i % max_parts] = 0;
  if (tid < kPartChoices) sm_pbytes[tid] = 0;
  if (tid < 4) sm_cnt[tid] = 0;
  if (tid < 2) sm_rows[tid] = 0;
  __syncthreads();

  // 1. items per class, partition size and length bin; split partials' bytes per size
  if (choose) {
    unsigned long long pbytes[kPartChoices] = {};
    for (int j = 0; j < k; ++j) {
      const int s = s0 + j;
      if (s >= num_seqs) break;
      const int q_len = qlen_of(s);
      const int cls = row_class(q_len, max_q, G, max_cols);
      if (!cls) continue;
      const int nb = blocks(n_of(s));
#pragma unroll
      for (int c = 0; c < kPartChoices; ++c) {
        const int pb = (c + 1) * kPartBlocks, f = nb / pb, rem = nb - f * pb;
        if (f) atomicAdd(&sm_hist[cls - 1][c][size_bin(pb)], f);
        if (rem || !nb) atomicAdd(&sm_hist[cls - 1][c][size_bin(rem)], 1);
        if (f + (rem > 0) > 1) pbytes[c] += (unsigned long long)(f + (rem > 0)) * q_len * hq * row_bytes;
      }
    }
#pragma unroll
    for (int c = 0; c < kPartChoices; ++c)
      if (pbytes[c]) atomicAdd(&sm_pbytes[c], pbytes[c]);
  }
  __syncthreads();

  // 2. the estimate of each size: wavefront c for size c, lane i for length bin i
  if (choose) {
    if (w < kPartChoices) {
      const long long cnt = (long long)(sm_hist[0][w][lane] + sm_hist[1][w][lane]) * num_kv_heads;
      const int t = kUnitCost + lane + 1;
      long long work = cnt * t;  // summed over the wavefront below
      long long suf = cnt;       // inclusive suffix sum: units in this bin and longer ones
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const long long y = __shfl_down(suf, off);
        if (lane + off < kWave) suf += y;
      }
      const long long above = suf - cnt;  // units in longer bins
      float bound = 0.f;
      if (cnt > 0) {
        const long long jhi = (suf - 1) / slots;  // largest j with j * slots + 1 <= suf
        if (jhi * slots >= above) bound = (float)((jhi + 1) * t);
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) {
        work += __shfl_xor(work, off);
        bound = fmaxf(bound, __shfl_xor(bound, off));
      }
      const float est = fmaxf(bound, (float)work / slots +
                                         (float)sm_pbytes[w] * kPartialWeight / ((float)step_bytes * slots));
      if (lane == 0) sm_est[w] = est;
    }
  } else if (tid < kPartChoices) {
    // one partition spans every row, or rows share blocks: kPartBlocks
    sm_est[tid] = tid ? INFINITY : 0.f;
  }
  __syncthreads();
  int pb0 = kPartBlocks;  // the smallest estimate; ties: the larger partition
  {
    float e = sm_est[0];
#pragma unroll
    for (int c = 1; c < kPartChoices; ++c)
      if (sm_est[c] <= e) {
        e = sm_est[c];
        pb0 = (c + 1) * kPartBlocks;
      }
  }

  // 3. totals: items of each class, merge entries, workspace rows (and the shift)
  int shift = 0;
  for (;; ++shift) {
    int n1 = 0, n2 = 0, nmg = 0;
    unsigned long long nrow = 0;
    for (int j = 0; j < k; ++j) {
      const int s = s0 + j;
      if (s >= num_seqs) break;
      const int q_len = qlen_of(s);
      const int cls = row_class(q_len, max_q, G, max_cols);
      if (!cls) continue;
      const int n = n_of(s), pb = part_blocks(q_len, pb0, shift);
      const int np = n > 0 ? (blocks(n) + pb - 1) / pb : 1;
      (cls == 1 ? n1 : n2) += np;
      if (np > 1) {
        nmg += q_len;
        nrow += (unsigned long long)np * q_len * hq;
      }
    }
    if (n1) atomicAdd(&sm_cnt[0], n1);
    if (n2) atomicAdd(&sm_cnt[1], n2);
    if (nmg) atomicAdd(&sm_cnt[2], nmg);
    if (nrow) atomicAdd(&sm_rows[0], nrow);
    __syncthreads();
    if ((long long)sm_rows[0] <= budget || (pb0 << shift) >= max_parts * kPartBlocks) break;
    __syncthreads();  // every thread has read the total before it is cleared
    if (tid < 3) sm_cnt[tid] = 0;
    if (tid == 0) sm_rows[0] = 0;
    __syncthreads();
  }

  // 4. list keys and their starts.  Longest first with unchanged partition sizes: the
  //    counts of step 1 (one key per lane); otherwise counted here
  const bool from_hist = choose && shift == 0;
  const int ci = pb0 / kPartBlocks - 1;
  const int levels = by_part ? max_parts : kSizeBins;
  auto key = [&](int p, int nb, int pb) {
    return by_part ? p : kSizeBins - 1 - size_bin(min(nb, (p + 1) * pb) - p * pb);
  };
  if (!from_hist) {
    if (!by_part)
      for (int i = tid; i < 2 * kSizeBins; i += blockDim.x) sm_lvl[i / kSizeBins][i % kSizeBins] = 0;
    __syncthreads();
    for (int j = 0; j < k; ++j) {
      const int s = s0 + j;
      if (s >= num_seqs) break;
      const int q_len = qlen_of(s);
      const int cls = row_class(q_len, max_q, G, max_cols);
      if (!cls) continue;
      const int n = n_of(s), nb = blocks(n), pb = part_blocks(q_len, pb0, shift);
      const int np = n > 0 ? (nb + pb - 1) / pb : 1;
      for (int p = 0; p < np; ++p) atomicAdd(&sm_lvl[cls - 1][key(p, nb, pb)], 1);
    }
    __syncthreads();
  }
  if (w < 2) {  // exclusive scan over the keys of class w + 1: lane i owns a run of keys
    const int per = (levels + kWave - 1) / kWave;
    const int v0 = min(lane * per, levels), v1 = min(v0 + per, levels);
    int sum = 0;
    if (from_hist)
      sum = sm_hist[w][ci][kSizeBins - 1 - lane];
    else
      for (int v = v0; v < v1; ++v) sum += sm_lvl[w][v];
    int x = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    int run = x - sum;
    if (from_hist) {
      sm_lvl[w][lane] = run;
    } else {
      for (int v = v0; v < v1; ++v) {
        const int c = sm_lvl[w][v];
        sm_lvl[w][v] = run;
        run += c;
      }
    }
  }
  __syncthreads();

  // 5. items at their keys' cursors; merge entries and workspace rows of split rows
  for (int j = 0; j < k; ++j) {
    const int s = s0 + j;
    if (s >= num_seqs) break;
    const int q_len = qlen_of(s);
    const int cls = row_class(q_len, max_q, G, max_cols);
    if (!cls) continue;
    const int n = n_of(s), nb = blocks(n), pb = part_blocks(q_len, pb0, shift);
    const int np = n > 0 ? (nb + pb - 1) / pb : 1;
    const int qb = qb_of(s);
    long long pr = -1;
    if (np > 1) {
      pr = (long long)atomicAdd(&sm_rows[1], (unsigned long long)np * q_len * hq);
      const int pm = atomicAdd(&sm_cnt[3], q_len);
      for (int t = 0; t < q_len; ++t)
        plan.merge[pm + t] =
            MergeEntry{qb + t, np, 0, 0, pr + (long long)t * hq, (long long)q_len * hq};
    }
    DecodeItem* list = plan.items + (cls == 1 ? 0 : (int64_t)plan.cap);
    for (int p = 0; p < np; ++p)
      list[atomicAdd(&sm_lvl[cls - 1][key(p, nb, pb)], 1)] =
          DecodeItem{s, 0, p * pb, min(nb, (p + 1) * pb), qb, q_len, n, p,
                     np > 1 ? pr + (long long)p * q_len * hq : -1, 0};
  }
  if (tid == 0) {
    plan.counts[0] = sm_cnt[0];
    plan.counts[1] = sm_cnt[2];
    plan.counts[2] = sm_cnt[1];
  }
}

// One work unit (item, KV head) of the decode kernel: the item's blocks of one row
// for the G query heads of KV head it.h, merged over the four wavefronts through LDS.
template <class DT, int D, int G, int CT>
__device__ __forceinline__ void decode_unit(
    const DecodeItem& it, const typename DT::T* __restrict__ q, typename DT::T* __restrict__ out,
    const typename DT::T* __restrict__ kp, const typename DT::T* __restrict__ vp,
    const int32_t* __restrict__ bt, int bt_stride, int num_kv_heads, float scale_log2,
    int max_parts, float* __restrict__ ws_o, float* __restrict__ ws_ml, int contiguous) {
  typedef Geo<DT, D> Gm;
  const int s = it.s, h = it.h, b0 = it.b0, qb = it.qb, q_len = it.q_len, n = it.n;
  const int cols = q_len * G;
  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);
  const int32_t* btr = bt + (int64_t)s * bt_stride;
  // block-table entries of this wavefront's first blocks b0 + w + 4i, one per lane
  // (bounded by the item and the table width).  Contiguous storage (the baseline
  // without paging): bt[s] is the sequence's first block and block i is bt[s] + i.
  auto table = [&](int i) {  // entry of this wavefront's block i (relative), or 0
    const int bi = b0 + w + kWaves * i;
    return (bi < it.b1 && bi < bt_stride) ? (contiguous ? bt[s] + bi : btr[bi]) : 0;
  };
  int btv = table(lane);
  const int hq = num_kv_heads * G;
  if (n <= 0) {
    if (it.part == 0)
      for (int e = threadIdx.x; e < cols * D; e += blockDim.x)
        store_elem<DT>(out, ((int64_t)(qb + e / D / G) * hq + h * G + (e / D) % G) * D + e % D, 0.f);
    return;
  }
  // a sequence longer than the bounds the host passed is cut at them (never read past them)
  const int nblocks = min((n + kBlock - 1) / kBlock, min(bt_stride, max_parts * kPartBlocks));
  const int b1 = min(nblocks, it.b1);
  if (b0 >= b1) return;
  const bool split = it.wrow >= 0;  // the row has other partitions
  const int ctx = n - q_len;
  const int g = lane >> 4, c = lane & 15;

  WaveState<DT, D> st[CT];
  int lim[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = ct * 16 + c, tq = col / G;
    const bool valid = col < cols;
    lim[ct] = valid ? ctx + tq : -1;  // a column past the row sees nothing
    load_q<DT, D>(st[ct], q + ((int64_t)(qb + (valid ? tq : 0)) * hq + h * G + col % G) * D, valid, g);
  }

  const int64_t head_off = (int64_t)h * Gm::kTile;
  const int64_t blk_elems = (int64_t)num_kv_heads * Gm::kTile;
  const int nw = (b0 + w < b1) ? (b1 - b0 - w + kWaves - 1) / kWaves : 0;  // blocks of this wave
  for (int i0 = 0; i0 < nw; i0 += kWave) {
    if (i0 > 0) btv = table(i0 + lane);
    const int cnt = min(kWave, nw - i0);
    auto fetch = [&](TileBuf<DT, D>& tb, int i) {
      const int64_t phys = __builtin_amdgcn_readlane(btv, i);
      load_tile<DT, D, true>(kp + phys * blk_elems + head_off, vp + phys * blk_elems + head_off,
                             tb.k, tb.v, lane);
    };
    auto consume = [&](TileBuf<DT, D>& tb, int i) {
      const int tok0 = (b0 + w + kWaves * (i0 + i)) * kBlock;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        attend_block<DT, D>(st[ct], tb.k, tb.v, tok0, n, lim[ct], scale_log2, g);
    };
    // two register buffers, both in flight: each iteration uses a tile and refills its
    // buffer two tiles ahead.  The prologue waits once for Q and the first two tiles;
    // after that every wait covers exactly the tile about to be used, and the refill is
    // kept after the use (a hoisted load would need fresh registers and a copy at the
    // loop edge).
    TileBuf<DT, D> A, B;
    fetch(A, 0);
    if (cnt > 1) fetch(B, 1);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt, expcnt and lgkmcnt all zero
    int i = 0;
    for (; i + 3 < cnt; i += 2) {
      consume(A, i);
      __builtin_amdgcn_sched_barrier(0);
      fetch(A, i + 2);
      consume(B, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      fetch(B, i + 3);
    }
    if (i < cnt) consume(A, i);
    if (i + 2 < cnt) fetch(A, i + 2);
    if (i + 1 < cnt) consume(B, i + 1);
    if (i + 2 < cnt) consume(A, i + 2);
  }

  // merge the four wavefronts through LDS
  __shared__ float sm_m[kWaves][CT * 16], sm_l[kWaves][CT * 16];
  __shared__ float sm_o[kWaves][CT * 16][D];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = ct * 16 + c;
    float lsum = st[ct].l + shfl_xor(st[ct].l, 16);
    lsum += shfl_xor(lsum, 32);
    if (g == 0) {
      sm_m[w][col] = st[ct].m;
      sm_l[w][col] = lsum;
    }
    if (col < cols) {
#pragma unroll
      for (int nn = 0; nn < Gm::kN; ++nn)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm_o[w][col][nn * 16 + 4 * g + r] = st[ct].acc[nn][r];
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < cols * D; e += blockDim.x) {
    const int col = e / D, d = e - col * D;
    float M = sm_m[0][col];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, sm_m[ww][col]);
    // a partition that starts inside a multi-token row hides it from the row's
    // earlier tokens: such a column has M = -inf and leaves (o, m, l) = (0, -inf, 0)
    const float Mu = M == -INFINITY ? 0.f : M;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = fast_exp2(sm_m[ww][col] - Mu);  // wavefronts without blocks: -inf -> 0
      num += f * sm_o[ww][col][d];
      den += f * sm_l[ww][col];
    }
    const float o = den > 0.f ? num / den : 0.f;
    const int64_t qrow = (int64_t)(col / G) * hq + col % G;  // from (token 0, head h*G)
    if (!split) {
      store_elem<DT>(out, ((int64_t)qb * hq + h * G + qrow) * D + d, o);
    } else {
      const int64_t idx = it.wrow + qrow;
      ws_o[idx * D + d] = o;
      if (d == 0) {
        ws_ml[2 * idx] = M;
        ws_ml[2 * idx + 1] = den;
      }
    }
  }
}

template <class DT, int D, int G, int CT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(decode_occupancy<DT, D, CT>())))
void decode_kernel(const typename DT::T* __restrict__ q, typename DT::T* __restrict__ out,
                   const typename DT::T* __restrict__ kp, const typename DT::T* __restrict__ vp,
                   const int32_t* __restrict__ bt, int bt_stride,
                   const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl,
                   int num_kv_heads, float scale_log2, int max_parts, int max_q,
                   float* __restrict__ ws_o, float* __restrict__ ws_ml, DecodePlan plan,
                   int contiguous) {
  // The work item's fields are held in scalar registers: read with readfirstlane in
  // the planned loop, pinned by an empty asm where the unplanned path loads them (so
  // that its metadata loads issue together, in one round trip).
  DecodeItem it;
  if (plan.counts) {
    // planned lists: workgroup b takes units v = b, b + grid, b + 2 grid, ... (grid a
    // multiple of 8, so every unit of a workgroup maps to the same XCD), in list order
    // on that XCD, until the list ends
    const int live = plan.counts[CT == 1 ? 0 : 2];
    for (int v = blockIdx.x;; v += gridDim.x) {
      int i, h;
      if (plan.by_part) {
        // head-major units in XCD runs: the rows reading one (block, head) tile run together
        const int j = xcd_unit(v, live * num_kv_heads);
        if (j < 0) return;
        i = j % live;
        h = j / live;
      } else {
        // longest first: the r-th unit of XCD x is KV head r % H of the XCD's item r / H.
        // The list is dealt in rounds of 8 items, item x of a round to XCD x, counted from
        // the other end in odd rounds (so no XCD takes the longest item of every round).
        // The odd-numbered XCDs stream K/V about 10% slower than the even ones, so after
        // every kOddRounds rounds one round of 4 items goes to the even XCDs alone: per
        // cycle of kOddRounds * 8 + 4 items an even XCD takes kOddRounds + 1, an odd one
        // kOddRounds.  Past the list: done.
        const int x = v % kXcds, r = v / kXcds;
        const int rd = r / num_kv_heads;
        const int per = (x & 1) ? kOddRounds : kOddRounds + 1;  // this XCD's items per cycle
        const int cyc = rd / per, k = rd - cyc * per;
        const int base = cyc * (kOddRounds * kXcds + kXcds / 2);
        i = k < kOddRounds ? base + k * kXcds + ((k & 1) ? kXcds - 1 - x : x)
                           : base + kOddRounds * kXcds + x / 2;
        h = r % num_kv_heads;
        if (i >= live) return;
      }
      if (v != (int)blockIdx.x) __syncthreads();  // the last unit's LDS has been read
      // one item per workgroup: the loop hides from the compiler that it is uniform
      const DecodeItem& src = plan.items[(CT == 1 ? 0 : (int64_t)plan.cap) + uniform(i)];
      it.s = uniform(src.s);
      it.b0 = uniform(src.b0);
      it.b1 = uniform(src.b1);
      it.qb = uniform(src.qb);
      it.q_len = uniform(src.q_len);
      it.n = uniform(src.n);
      it.part = uniform(src.part);
      it.wrow = ((int64_t)uniform((int)(src.wrow >> 32)) << 32) | (uint32_t)uniform((int)src.wrow);
      it.h = uniform(h);
      if (it.wrow >= 0) it.wrow += it.h * G;
      decode_unit<DT, D, G, CT>(it, q, out, kp, vp, bt, bt_stride, num_kv_heads, scale_log2,
                                max_parts, ws_o, ws_ml, contiguous);
    }
  } else {  // one partition per row: every sequence is an item
    const int j = xcd_unit(blockIdx.x, plan.num_seqs * num_kv_heads);
    if (j < 0) return;
    const int s = j / num_kv_heads;
    int q0 = qsl[s], q1 = qsl[s + 1], n = seq_lens[s];
    asm volatile("" : "+s"(q0), "+s"(q1), "+s"(n));
    it = DecodeItem{s, j % num_kv_heads, 0, kPartBlocks, q0, q1 - q0, n, 0, -1, 0};
    const int cols = it.q_len * G;
    if (it.q_len < 1 || it.q_len > max_q || cols > CT * 16 || cols <= (CT - 1) * 16) return;
    decode_unit<DT, D, G, CT>(it, q, out, kp, vp, bt, bt_stride, num_kv_heads, scale_log2,
                              max_parts, ws_o, ws_ml, contiguous);
  }
}

// Merge of the partitions of split rows, one workgroup per (merge entry = split
// sequence and query token, KV head):
//   o = sum_p 2^(m_p - M) l_p o_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// A thread owns four consecutive outputs of one query head and loads the (m, l)
// pair and the four partial outputs of kMergeBatch partitions at once, so a
// merge costs one memory round trip after its entry (contexts up to 8192
// tokens: one round).
constexpr int kMergeBatch = 8;

template <class DT, int D, int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    typename DT::T* __restrict__ out, const float* __restrict__ ws_o,
    const float* __restrict__ ws_ml, int num_kv_heads, DecodePlan plan) {
  const int j = xcd_unit(blockIdx.x, plan.counts[1] * num_kv_heads);
  if (j < 0) return;
  const MergeEntry me = plan.merge[j / num_kv_heads];
  const int h = j % num_kv_heads;
  const int hq = num_kv_heads * G;
  constexpr int kQuads = D / 4;
  for (int u = threadIdx.x; u < G * kQuads; u += blockDim.x) {
    const int cc = u / kQuads, d = (u - cc * kQuads) * 4;
    const int64_t row0 = me.row0 + h * G + cc;  // partition 0; + p * pstride for partition p
    float M = -INFINITY, den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < me.nparts; p0 += kMergeBatch) {
      float2 ml[kMergeBatch];
      f32x4 op[kMergeBatch];
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const int p = min(p0 + k, me.nparts - 1);  // past the end: re-read the last (weight 0)
        const int64_t row = row0 + p * me.pstride;
        ml[k] = *(const float2*)(ws_ml + 2 * row);
        op[k] = *(const f32x4*)(ws_o + row * D + d);
      }
      float bm = M;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) bm = fmaxf(bm, ml[k].x);
      const float f0 = fast_exp2(M - bm);  // M = -inf on the first round: 0
      num *= f0;
      den *= f0;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        // hidden partitions (m = -inf, l = 0) weigh 0; partition 0 is never hidden
        const float f = p0 + k < me.nparts ? fast_exp2(ml[k].x - bm) * ml[k].y : 0.f;
        num += f * op[k];
        den += f;
      }
      M = bm;
    }
    store4<DT>(out, ((int64_t)me.qrow * hq + h * G + cc) * D + d, num / den);
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static int64_t round256(int64_t b) { return (b + 255) / 256 * 256; }

// counts, the item records of two classes, merge entries (up to 32 query tokens per
// sequence)
static int64_t plan_item_bytes(int64_t num_seqs, int64_t max_parts) {
  return round256(256 + 2 * num_seqs * max_parts * (int64_t)sizeof(DecodeItem));
}
static int64_t decode_plan_bytes(int64_t num_seqs, int64_t max_parts) {
  return plan_item_bytes(num_seqs, max_parts) + round256(num_seqs * 32 * (int64_t)sizeof(MergeEntry));
}

// Workspace rows (head_dim floats each) for the partial results of split rows:
// twice what a decode-only batch can need, so that short multi-token rows split
// too (the plan enlarges their partitions when they would not fit).
static int64_t split_rows(int64_t num_seqs, int64_t max_parts, int64_t num_q_heads) {
  return 2 * num_seqs * max_parts * num_q_heads;
}

// Compute units of the current device (queried once per device; 256 on an MI355X,
// fewer in a partitioned mode), or 0 if the runtime cannot say.
static int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= 64) return 0;
  if (!cached[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return 0;
    cached[dev] = cus;
  }
  return cached[dev];
}

// Workgroups of a planned decode launch per resident slot: enough that every unit of
// a usual batch has its own workgroup (dealt by the hardware as slots free up), few
// enough that the workgroups past the list (the grid is sized before the list is
// known) cost little.
constexpr int kDecodeOversub = 8;

template <class DT, int D, int G, int CT>
static int launch_ct(const AttnArgs& a, const DecodePlan& plan, int slots) {
  typedef typename DT::T T;
  // unplanned: one workgroup per (row, KV head); planned: every sequence in every
  // partition at most, and at most kDecodeOversub per slot (workgroups then loop over
  // units); the plan's counts cut the lists short
  const int64_t units = (int64_t)a.max_parts * a.num_seqs * a.num_kv_heads;
  int64_t grid = (units + kXcds - 1) / kXcds * kXcds;
  if (plan.counts) {
    const int64_t cap = ((int64_t)slots * kDecodeOversub + kXcds - 1) / kXcds * kXcds;
    if (grid > cap) grid = cap;
  }
  hipLaunchKernelGGL((decode_kernel<DT, D, G, CT>), dim3((unsigned)grid), dim3(256), 0, a.stream,
                     (const T*)a.q, (T*)a.out, (const T*)a.kp, (const T*)a.vp, a.bt, a.bt_stride,
                     a.seq_lens, a.qsl, a.num_kv_heads, a.scale_log2, a.max_parts, a.max_q_len,
                     a.ws_o, a.ws_ml, plan, a.contiguous);
  return PKV_OK;
}

template <class DT, int D, int G>
static int launch(const AttnArgs& a) {
  typedef typename DT::T T;
  constexpr int kMaxCols = (DT::kBytes == 2 && D <= 128) ? 32 : 16;
  DecodePlan plan;
  plan.num_seqs = a.num_seqs;
  plan.cap = a.num_seqs * a.max_parts;
  // partition-major needs one list key per partition index
  plan.by_part = a.order_by_part && a.max_parts <= kPlanLevels ? 1 : 0;
  plan.counts = nullptr;
  plan.items = nullptr;
  plan.merge = nullptr;
  // a class no row can be in is not launched: two-tile rows need max_q_len * G > 16,
  // and rows of one q_len are all in the same class
  const int64_t widest = (int64_t)a.max_q_len * G;
  const bool two_only = a.uniform_q && widest > 16;
  // resident decode workgroups the plan balances over: those of the one-tile kernel,
  // unless every row takes two tiles
  const int cus = device_cus();
  if (cus <= 0) return PKV_ERR_HIP;
  const int slots = cus * (two_only ? decode_occupancy<DT, D, 2>() : decode_occupancy<DT, D, 1>());
  if (a.max_parts > 1) {
    // sequences may span several partitions: list the live (sequence, partition) items
    plan.counts = (int32_t*)a.ws_plan;
    plan.items = (DecodeItem*)((char*)a.ws_plan + 256);
    char* mp = (char*)a.ws_plan + plan_item_bytes(a.num_seqs, a.max_parts);
    plan.merge = (MergeEntry*)mp;
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(1024), 0, a.stream, a.seq_lens, a.qsl,
                       a.num_seqs, a.bt_stride, a.max_parts, a.max_q_len, G, kMaxCols,
                       a.num_kv_heads * G,
                       (long long)split_rows(a.num_seqs, a.max_parts, a.num_kv_heads * G),
                       a.num_kv_heads, slots,
                       (D + 2) * 4, kWaves * 2 * kBlock * D * DT::kBytes, plan);
  }
  if (!two_only && launch_ct<DT, D, G, 1>(a, plan, cus * decode_occupancy<DT, D, 1>()) != PKV_OK)
    return PKV_ERR_HIP;
  if constexpr (kMaxCols > 16)
    if (widest > 16 && launch_ct<DT, D, G, 2>(a, plan, cus * decode_occupancy<DT, D, 2>()) != PKV_OK)
      return PKV_ERR_HIP;
  if (a.max_parts > 1) {
    // merge entries: at most one per query token of the rows this kernel takes
    const int64_t qmax = a.max_q_len < kMaxCols / G ? a.max_q_len : kMaxCols / G;
    const int64_t mgrid = ((int64_t)a.num_seqs * qmax * a.num_kv_heads + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((decode_merge_kernel<DT, D, G>), dim3((unsigned)mgrid), dim3(256), 0,
                       a.stream, (T*)a.out, a.ws_o, a.ws_ml, a.num_kv_heads, plan);
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
  const int64_t rows = split_rows(num_seqs, parts, num_q_heads);
  // split rows' (m, l) pairs and partition outputs, prefill work list, decode plan; each
  // section 256-byte aligned
  return (size_t)(round256(rows * 2 * 4) + round256(rows * (int64_t)head_dim * 4) +
                  round256(prefill_workspace_bytes(num_seqs, num_q_tokens, num_q_heads, head_dim)) +
                  decode_plan_bytes(num_seqs, parts));
}

static int attention_impl(const pkv_cache_t* cache, int32_t layer, void* out, const void* q,
                          const int32_t* block_tables, int32_t bt_stride, int contiguous,
                          const int32_t* seq_lens, const int32_t* query_start_loc,
                          int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len,
                          int32_t max_seq_len, int32_t num_q_heads, float scale, void* workspace,
                          size_t workspace_bytes, uint32_t flags, void* stream) {
  int rc = check_cache(cache);
  if (flags & ~PKV_ATTN_SHARED_PREFIXES) return PKV_ERR_INVALID_ARGUMENT;
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
  // the decode and merge grids (padded to whole XCD rounds) must fit their limit
  const int64_t per_seq = max_partitions(max_seq_len) > 32 ? max_partitions(max_seq_len) : 32;
  if ((int64_t)num_seqs * cache->num_kv_heads * per_seq + kXcds > 0x7fffffff)
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
  a.uniform_q = (int64_t)num_seqs * max_q_len == num_q_tokens;
  a.order_by_part = (flags & PKV_ATTN_SHARED_PREFIXES) != 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  const int64_t rows = split_rows(num_seqs, a.max_parts, num_q_heads);
  a.ws_ml = (float*)workspace;
  a.ws_o = (float*)((char*)workspace + round256(rows * 2 * 4));
  a.ws_pf = (char*)workspace + round256(rows * 2 * 4) + round256(rows * (int64_t)cache->head_dim * 4);
  a.pf_items = prefill_items_bound(num_seqs, num_q_tokens, num_q_heads);
  a.pf_slots = prefill_slots_bound(num_seqs, num_q_tokens);
  a.ws_plan = (char*)a.ws_pf + round256(prefill_workspace_bytes(num_seqs, num_q_tokens, num_q_heads,
                                                                cache->head_dim));
  a.stream = (hipStream_t)stream;
  // decode rows and short chunks (q_len * G <= small_cols) in the partitioned kernel,
  // then longer chunks: tiled (fp32: one wavefront per 16 columns)
  const int small_cols = small_chunk_max_cols(cache->dtype, cache->head_dim);
  if (!(a.uniform_q && (int64_t)max_q_len * G > small_cols)) {  // some row may be short
    switch (cache->dtype) {
      case PKV_F32: rc = dispatch_d<TF32>(a, cache->head_dim, G); break;
      case PKV_F16: rc = dispatch_d<TF16>(a, cache->head_dim, G); break;
      case PKV_BF16: rc = dispatch_d<TBF16>(a, cache->head_dim, G); break;
      default: return PKV_ERR_UNSUPPORTED;
    }
  }
  if (rc != PKV_OK || (int64_t)max_q_len * G <= small_cols) return rc;
  if (cache->dtype == PKV_F32) return launch_prefill_wave(a, cache->dtype, cache->head_dim, G);
  return launch_prefill_tiled(a, cache->dtype, cache->head_dim, G);
}

extern "C" int pkv_paged_attention(const pkv_cache_t* cache, int32_t layer, void* out,
                                   const void* q, const int32_t* block_tables, int32_t bt_stride,
                                   const int32_t* seq_lens, const int32_t* query_start_loc,
                                   int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len,
                                   int32_t max_seq_len, int32_t num_q_heads, float scale,
                                   void* workspace, size_t workspace_bytes, uint32_t flags,
                                   void* stream) {
  return attention_impl(cache, layer, out, q, block_tables, bt_stride, 0, seq_lens,
                        query_start_loc, num_seqs, num_q_tokens, max_q_len, max_seq_len,
                        num_q_heads, scale, workspace, workspace_bytes, flags, stream);
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
                        scale, workspace, workspace_bytes, 0, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free paged_attention: the workspace is a static device array.
// ---------------------------------------------------------------------------
namespace pkv {

// One copy per GPU the library runs on, held until the process ends.  In host
// code the name stands in for the variable and is not a device address: host code
// uses only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[PKV_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_addr[kMaxDevices];

// Device address of the current GPU's scratch array, looked up on the first call
// on that GPU and kept.
static int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return PKV_OK;
}

}  // namespace pkv

extern "C" int pkv_paged_attention_no_alloc(const pkv_cache_t* cache, int32_t layer, void* out,
                                            const void* q, const int32_t* block_tables,
                                            int32_t bt_stride, const int32_t* seq_lens,
                                            const int32_t* query_start_loc, int32_t num_seqs,
                                            int32_t num_q_tokens, int32_t max_q_len,
                                            int32_t max_seq_len, int32_t num_q_heads, float scale,
                                            uint32_t flags, void* stream) {
  if (!cache) return PKV_ERR_INVALID_ARGUMENT;
  // every section of the workspace is written by the call's own kernels before it is
  // read (plan counts, work lists, the prefill queue, partials): nothing to clear
  const size_t need = pkv_paged_attention_workspace_bytes(num_seqs, num_q_tokens, max_seq_len,
                                                          num_q_heads, cache->head_dim);
  if (need > PKV_STATIC_WORKSPACE_BYTES) return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != PKV_OK) return rc;
  return attention_impl(cache, layer, out, q, block_tables, bt_stride, 0, seq_lens,
                        query_start_loc, num_seqs, num_q_tokens, max_q_len, max_seq_len,
                        num_q_heads, scale, ws, PKV_STATIC_WORKSPACE_BYTES, flags, stream);
}
