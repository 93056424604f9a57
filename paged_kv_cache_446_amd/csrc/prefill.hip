// Prefill chunks for gfx950: query rows with q_len > 1 attend to the whole
// cached context of their sequence plus the chunk's own earlier tokens
// (blog.mckayzhao.com/?p=56, chunked prefill under advanced features; the
// mixed {request_id: num_tokens} batch of the V1 section).  Keys are read block
// by block through the block table, as for decode (same page, section
// "PagedAttention").  Chunks of at most 32 (token, head) columns per KV head
// take the partitioned decode kernel (attention.hip); this file holds the rest.
//
//   * 16-bit types: a plan kernel lists (sequence, 256-column query tile, KV
//     head, block range) items, longest first, and a persistent kernel takes
//     them from a queue, die by die when the list is long (the query tiles
//     reading one context then share a die's L2).  Per item, K/V tiles of
//     several blocks at a time are staged in LDS (double buffered) and shared
//     by 8 wavefronts of 32 columns; the scores S^T = K.Q^T use 16x16x32
//     matrix instructions and the product O^T += V^T.P^T runs over 32 tokens
//     at a time, also 16x16x32.
//     When a few long items would leave most of the chip idle, the plan cuts
//     their context into pieces of about one workgroup's share of the work;
//     pieces write fp32 partials (max, sum, normalised output) and a merge
//     kernel combines them with the log-sum-exp rule, as decode does.
//   * fp32: one wavefront per 16 columns.
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
constexpr int kPfTableMax = 4096;  // block-table entries an item keeps in LDS (65536 tokens)
// The exponentials use a reference max that may lag the true running max by
// up to 2^kPfLag (weights <= 2^8, far from overflow); the accumulators are
// rescaled only when some column's max moves further than that.
constexpr float kPfLag = 8.f;

template <class DT, int D>
struct PfGeo {
  static constexpr int kCT = D <= 128 ? 2 : 1;                      // 16-column tiles per wave
  static constexpr int kSB = D <= 128 ? 4 : 2;                      // KV blocks per compute step
  static constexpr int kSS = D <= 128 ? 2 : 1;                      // compute steps per LDS stage
  static constexpr int kStageB = kSB * kSS;                         // KV blocks per LDS stage
  static constexpr int kCols = kPfWaves * kCT * 16;                 // columns per item
  static constexpr int kTileChunks = kBlock * D * DT::kBytes / 16;  // 16-byte chunks per tile
  static constexpr int kStageChunks = 2 * kStageB * kTileChunks;    // K and V of a stage
  static constexpr int kPerThread = kStageChunks / kPfThreads;
  static constexpr int kLdsBytes = 2 * kStageChunks * 16;           // double buffer
  static_assert(kStageChunks % kPfThreads == 0, "whole chunks per thread");
  static_assert(kSB % 2 == 0 && kPfTableMax % kStageB == 0, "whole block pairs per step");
  static_assert(kLdsBytes + kPfTableMax * 4 + 64 <= 160 * 1024, "LDS of one workgroup");
};

// A piece of a (sequence, query tile, KV head): blocks [kb0, kb1) of the visible
// context.  slot < 0: the piece is the whole context and writes the output;
// otherwise it writes partials to slot (kPfSlotCols columns of (m, l, o)).
struct PfItem {
  int32_t s, qtile, h, kb0, kb1, slot, pad0, pad1;
};
// One split (sequence, query tile, KV head): its np pieces hold slots slot0 ..
// slot0 + np - 1, piece p covering the context blocks after those of piece p-1.
struct PfMerge {
  int32_t s, qb, q_len, qtile, h, np, slot0, pad;
};

constexpr int kPfSlotCols = 256;      // columns of a partial slot (the widest item)
constexpr int kPfSplitWorkers = 256;  // workers the split rule balances over (at most)
constexpr int kPfMaxSlots = kPfSplitWorkers;  // partial slots of one call
constexpr int kPfMinPiece = 64;       // blocks of the shortest piece (1024 tokens)

// Byte offsets of the tiled prefill's workspace: items (the q-tile items plus one
// per extra piece), the plan's (sequence, q-tile) list, merges, queue counters,
// partial outputs and (m, l) pairs.
struct PfLayout {
  int64_t items, tiles, merges, queue, part_o, part_ml, total;
  PfLayout(int64_t n_items, int64_t slots, int64_t head_dim) {
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    items = 0;
    tiles = up((n_items + slots) * (int64_t)sizeof(PfItem));  // (sequence, q-tile) list
    merges = tiles + up(n_items * (int64_t)sizeof(int2));
    queue = merges + up((slots / 2 + 1) * (int64_t)sizeof(PfMerge));
    part_o = queue + 256;
    part_ml = part_o + up(slots * kPfSlotCols * head_dim * 4);
    total = part_ml + up(slots * kPfSlotCols * 8);
  }
};

// Queue counters of the tiled kernel (ints at the workspace's queue offset): the
// next-item counter of each die, the number of items and the number of merges.
constexpr int kPfQNext = 0;
constexpr int kPfQTotal = kXcds;
constexpr int kPfQMerges = kXcds + 1;

// Work list of the tiled kernel: one workgroup of 1024 threads.  Every
// (sequence, q-tile) of a chunk wider than small_cols columns has one item per
// KV head, the KV heads of a q-tile side by side; items are ordered by the
// context they read, longest first, in 1024-token classes.  The (sequence,
// q-tile) pairs are first listed flat (a scan over the sequences), so that the
// threads share them evenly however they are spread over sequences.  All
// q-tiles of a sequence take the class of its whole context, so that the lanes
// holding them reserve one range together: its q-tiles sit next to each other,
// listed last q-tile (the longest) first.
// The tiled kernel's workgroups on die d take items d, d + 8, d + 16, ... first.
// A (sequence, q-tile, piece) lists its KV heads rotated by (sequence + piece),
// so that with Hkv a multiple of 8 the q-tiles of one (sequence, KV head,
// piece), which read nearly the same blocks, all fall to one die and run there
// at about the same time, sharing its L2, while each die still sees every KV
// head.
//
// Splitting: with W the blocks all items read (over KV heads too) and P the
// workers, an item of b blocks is cut into np = floor(b P / W) pieces (at least
// one, each at least kPfMinPiece blocks and a whole number of pipeline steps of
// sb blocks): items of more than one worker's share are split, and the pieces
// of all split items number at most P, so one round of workers takes them and
// max_slots >= P partial slots suffice.  Pieces keep the class of their own
// length.  Also resets the queue counters.
__global__ __launch_bounds__(1024) void prefill_plan_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int num_seqs,
    int num_kv_heads, int G, int cols, int small_cols, int bt_stride, int sb, int workers,
    int max_slots, PfItem* __restrict__ items, int2* __restrict__ tiles,
    PfMerge* __restrict__ merges, int32_t* __restrict__ queue, int max_items) {
  __shared__ int hist[kPfBuckets], base[kPfBuckets];
  __shared__ int sm_tot[1024 / kWave];
  __shared__ unsigned long long sm_work;
  __shared__ int sm_slot, sm_merge;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nwaves = blockDim.x / kWave;
  const int qt_tokens = cols / G;
  if (tid < kPfBuckets) hist[tid] = 0;
  if (tid == 0) {
    sm_work = 0;
    sm_slot = 0;
    sm_merge = 0;
  }
  // 1. q-tiles per sequence, an exclusive scan over the sequences (thread t owns
  //    sequences [t k, t k + k)), and the flat (sequence, q-tile) list
  const int k = (num_seqs + blockDim.x - 1) / blockDim.x;
  const int s0 = tid * k;
  auto ntiles = [&](int s) {
    const int q_len = qsl[s + 1] - qsl[s];
    return (int64_t)q_len * G <= small_cols ? 0 : (q_len + qt_tokens - 1) / qt_tokens;
  };
  int mine = 0;
  for (int j = 0; j < k && s0 + j < num_seqs; ++j) mine += ntiles(s0 + j);
  int x = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) sm_tot[w] = x;
  __syncthreads();
  int before = 0, total = 0;
  for (int ww = 0; ww < nwaves; ++ww) {
    before += ww < w ? sm_tot[ww] : 0;
    total += sm_tot[ww];
  }
  int pos = before + x - mine;
  for (int j = 0; j < k && s0 + j < num_seqs; ++j) {
    const int nt = ntiles(s0 + j);
    for (int t = 0; t < nt; ++t) tiles[pos + t] = int2{s0 + j, nt - 1 - t};  // longest first
    pos += nt;
  }
  __syncthreads();  // the list is visible to the whole workgroup
  // blocks q-tile t of sequence s reads (the blocks its last row sees)
  auto vis_blocks = [&](int s, int t) {
    const int q_len = qsl[s + 1] - qsl[s], n = seq_lens[s];
    const int vis = n - q_len + min(q_len, (t + 1) * qt_tokens);
    return (n > 0 && vis > 0) ? min((vis - 1) / kBlock + 1, bt_stride) : 0;
  };
  // 2. the work W
  {
    unsigned long long wk = 0;
    for (int i = tid; i < total; i += blockDim.x) {
      const int2 st = tiles[i];
      wk += (unsigned long long)vis_blocks(st.x, st.y) * num_kv_heads;
    }
    if (wk) atomicAdd(&sm_work, wk);
  }
  __syncthreads();
  const long long W = (long long)sm_work;
  const bool split = max_slots >= workers && workers > 0 && W > 0;
  // 3. pieces: counted in pass 0, written in pass 1
  for (int pass = 0; pass < 2; ++pass) {
    for (int i = tid; i < total; i += blockDim.x) {
      const int2 st = tiles[i];
      const int s = st.x, t = st.y;
      const int vb = vis_blocks(s, t);
      int np = 1, pl = vb;  // np pieces of pl blocks
      if (split) {
        const long long want = min((long long)vb * workers / W, (long long)vb / kPfMinPiece);
        if (want > 1) {
          pl = ((vb + (int)want - 1) / (int)want + sb - 1) / sb * sb;
          np = (vb + pl - 1) / pl;
        }
      }
      int slot0 = -1;
      if (pass == 1 && np > 1) {
        slot0 = atomicAdd(&sm_slot, np * num_kv_heads);
        const int mi = atomicAdd(&sm_merge, num_kv_heads);
        const int qb = qsl[s], q_len = qsl[s + 1] - qb;
        for (int h = 0; h < num_kv_heads; ++h)
          merges[mi + h] = PfMerge{s, qb, q_len, t, h, np, slot0 + h * np, 0};
      }
      const int n = seq_lens[s];
      const int vb_seq = n > 0 ? min((n - 1) / kBlock + 1, bt_stride) : 0;  // the last q-tile's
      for (int p = 0; p < np; ++p) {
        const int kb0 = p * pl, kb1 = min(vb, kb0 + pl);
        const int len = np > 1 ? kb1 - kb0 : vb_seq;
        const int b = kPfBuckets - 1 - min(kPfBuckets - 1, (len * kBlock) >> 10);
        const int at = atomicAdd(&hist[b], num_kv_heads);
        if (pass == 1) {
          const int rot = (s + p) % num_kv_heads;  // same for every q-tile of (s, piece p)
          for (int h = 0; h < num_kv_heads; ++h) {
            const int at_h = base[b] + at + (h + rot) % num_kv_heads;
            if (at_h < max_items)
              items[at_h] = PfItem{s, t, h, kb0, kb1, np > 1 ? slot0 + h * np + p : -1, 0, 0};
          }
        }
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
      for (int d = 0; d < kXcds; ++d) queue[kPfQNext + d] = 0;
      queue[kPfQTotal] = min(run, max_items);
    }
    __syncthreads();
  }
  if (tid == 0) queue[kPfQMerges] = sm_merge;
}

template <class DT, int D, int G>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_tiled_kernel(const typename DT::T* __restrict__ q, typename DT::T* __restrict__ out,
                          const typename DT::T* __restrict__ kp,
                          const typename DT::T* __restrict__ vp, const int32_t* __restrict__ bt,
                          int bt_stride, const int32_t* __restrict__ seq_lens,
                          const int32_t* __restrict__ qsl, int num_kv_heads, float scale_log2,
                          const PfItem* __restrict__ items, int32_t* __restrict__ queue,
                          float* __restrict__ part_o, float2* __restrict__ part_ml) {
  static_assert(DT::kBytes == 2, "16-bit element types");
  typedef Geo<DT, D> Gm;
  typedef PfGeo<DT, D> P;
  constexpr int kCT = P::kCT;
  constexpr int kSB = P::kSB;
  constexpr int kStageB = P::kStageB;
  constexpr int kTC = P::kTileChunks;
  constexpr int QT = P::kCols / G;  // query tokens per item
  // LDS stage: [K of blocks 0..kStageB-1][V of block pair 0: slices r=0][r=1][pair 1: ...]...
  // A V entry of 16 bytes holds the 8-byte half r of one chunk for the pair's first block,
  // then for its second: exactly one A operand of the 32-token V^T.P^T product.
  extern __shared__ u32x4 sm_stage[];
  __shared__ int sm_item;
  __shared__ int32_t sm_bt[kPfTableMax];  // the item's block-table entries (one segment)
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int hq = num_kv_heads * G;
  const int total = queue[kPfQTotal];
  const int64_t blk_elems = (int64_t)num_kv_heads * Gm::kTile;
  // With at least two rounds of items, workgroups (dealt to the dies round-robin) take their
  // die's share of the list (items die, die + 8, ...) first, then the other dies' shares in
  // turn; with fewer, every workgroup starts at once and nothing is gained by keeping the
  // q-tiles of one context on one die (they then read the same lines at the same moment),
  // so all take the list in order.  Thread 0 only.
  const bool by_die = total >= 2 * (int)gridDim.x;
  const int die = by_die ? blockIdx.x % kXcds : 0;
  int tried = 0;

  for (;;) {
    if (tid == 0) {
      int got = -1;
      for (; tried < kXcds; ++tried) {
        const int d = (die + tried) % kXcds;
        const int k = atomicAdd(&queue[kPfQNext + d], 1);
        const int i = by_die ? k * kXcds + d : k;
        if (i < total) {
          got = i;
          break;
        }
        if (!by_die) tried = kXcds - 1;  // the one list is done
      }
      sm_item = got;
    }
    __syncthreads();
    const int it = sm_item;
    __syncthreads();
    if (it < 0) break;
    const PfItem item = items[it];
    const int s = item.s, h = item.h, kb0 = item.kb0, kb1 = item.kb1;
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
    // this item reads blocks [kb0, kb1) of those the tile's last row can see; a piece
    // boundary other than the last block falls on a whole step
    int seg0 = kb0;  // first block of the block-table segment held in sm_bt

    // K/V of stage j: registers -> LDS buffer j & 1, a compute step's blocks at a time: the
    // part for compute step ss of stage j + 1 is loaded while step ss of stage j computes,
    // then stored into the other buffer.  Thread chunk k of a stage is chunk ci of tile
    // t = 2b + (0 for K, 1 for V) of the stage's block b; part ss holds chunks
    // k = ss * kPH .. ss * kPH + kPH - 1, the tiles of blocks ss * kSB .. ss * kSB + kSB - 1.
    // Loads are unconditional (blocks past the visible range re-read the last one) so that
    // each wait covers exactly one part; masking happens when the part is stored.
    constexpr int kPH = P::kPerThread / P::kSS;
    u32x4 stg[kPH];
    auto fetch_part = [&](int j, int ss) {
#pragma unroll
      for (int k = 0; k < kPH; ++k) {
        const int idx = tid + (ss * kPH + k) * kPfThreads;
        const int t = idx / kTC, ci = idx % kTC;
        const int blk = min(kStageB * j + (t >> 1), kb1 - 1);
        const int64_t phys = sm_bt[blk - seg0];
        const u32x4* src = (const u32x4*)(((t & 1) ? vp : kp) + phys * blk_elems + head_off);
        stg[k] = src[ci];
      }
    };
    auto store_part = [&](int j, int ss, int buf) {
      u32x4* st = sm_stage + buf * P::kStageChunks;
#pragma unroll
      for (int k = 0; k < kPH; ++k) {
        const int idx = tid + (ss * kPH + k) * kPfThreads;
        const int t = idx / kTC, ci = idx % kTC;
        const int b = t >> 1, blk = kStageB * j + b;
        u32x4 v = blk < kb1 ? stg[k] : u32x4{0, 0, 0, 0};
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
          uint2* v2 = (uint2*)(st + (kStageB + 2 * (b >> 1)) * kTC);
          v2[2 * ci + (b & 1)] = uint2{v.x, v.y};
          v2[2 * (kTC + ci) + (b & 1)] = uint2{v.z, v.w};
        } else {
          st[b * kTC + ci] = v;
        }
      }
    };
    // compute step ss of stage j: the stage's blocks ss * kSB .. ss * kSB + kSB - 1
    auto compute = [&](int j, int buf, int ss) {
      const u32x4* st = sm_stage + buf * P::kStageChunks + ss * kSB * kTC;  // its K tiles
      const u32x4* sv = sm_stage + buf * P::kStageChunks + (kStageB + ss * kSB) * kTC;  // V
      const int t0 = (kStageB * j + kSB * ss) * kBlock;
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
      // the reference max moves only when some column's max over this step exceeds it by
      // more than kPfLag (a wave-wide decision); a lane's own max decides it (x * scale rounds
      // monotonically, so some lane's scaled max exceeds the bound exactly when the column's
      // does), and the column maxima are reduced across lanes only when it moves
      float bml[kCT];
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
        bml[ct] = bm;
        move |= bm * scale_log2 > m[ct] + kPfLag;  // also the first visible key (m = -inf)
      }
      if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
        for (int ct = 0; ct < kCT; ++ct) {
          const float mn = fmaxf(m[ct], col_max4(bml[ct]) * scale_log2);
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
          const u32x4 lo = sv[(2 * pp) * kTC + mm * kWave + lane];      // dim slice 2mm
          const u32x4 hi = sv[(2 * pp + 1) * kTC + mm * kWave + lane];  // slice 2mm+1
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
    for (; seg0 < kb1; seg0 += kPfTableMax) {
      const int seg_n = min(kPfTableMax, kb1 - seg0);
      for (int i = tid; i < seg_n; i += kPfThreads) sm_bt[i] = btr[seg0 + i];
      __syncthreads();
      const int js = seg0 / kStageB, je = (seg0 + seg_n + kStageB - 1) / kStageB;
      const int jl = je - 1;  // stages past the segment fetch its last stage again (unused)
#pragma unroll
      for (int ss = 0; ss < P::kSS; ++ss) {
        fetch_part(js, ss);
        store_part(js, ss, js & 1);
      }
      __syncthreads();
      for (int j = js; j < je; ++j) {
#pragma unroll
        for (int ss = 0; ss < P::kSS; ++ss) {
          fetch_part(min(j + 1, jl), ss);
          if (wave_active) compute(j, j & 1, ss);
          if (j + 1 < je) store_part(j + 1, ss, (j + 1) & 1);
        }
        __syncthreads();
      }
    }
#pragma unroll
    for (int ct = 0; ct < kCT; ++ct) {
      const float lsum = accl[ct][0];
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;  // nothing visible -> zeros
      const int col = (w * kCT + ct) * 16 + c;
      if (item.slot < 0) {
        if (tq0 + col / G < tq_end && (lim[ct] >= 0 || n <= 0)) {
          const int64_t o = ((int64_t)(qb + tq0 + col / G) * hq + h * G + col % G) * D + 4 * g;
#pragma unroll
          for (int nn = 0; nn < Gm::kN; ++nn) store4<DT>(out, o + nn * 16, acc[ct][nn] * inv);
        }
      } else if (tq0 + col / G < tq_end) {
        // a piece: (m, l, o) of the column over this piece's keys; a column that sees
        // none of them leaves (-inf, 0, 0), which the merge weighs 0
        const int64_t row = (int64_t)item.slot * kPfSlotCols + col;
#pragma unroll
        for (int nn = 0; nn < Gm::kN; ++nn)
          *(f32x4*)(part_o + row * D + nn * 16 + 4 * g) = acc[ct][nn] * inv;
        if (g == 0) part_ml[row] = float2{lsum > 0.f ? m[ct] : -INFINITY, lsum};
      }
    }
  }
}

// Merge of split items, one workgroup per (entry of the plan's merge list,
// group of kMergeCols columns):
//   o = sum_p 2^(m_p - M) l_p o_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// A thread owns four consecutive dims of one column and loads eight pieces at
// a time.
constexpr int kMergeCols = 32;
template <class DT, int D, int G>
__global__ __launch_bounds__(256) void prefill_merge_kernel(
    typename DT::T* __restrict__ out, const float* __restrict__ part_o,
    const float2* __restrict__ part_ml, int num_kv_heads, const PfMerge* __restrict__ merges,
    const int32_t* __restrict__ queue) {
  constexpr int kBatch = 8;
  constexpr int QT = PfGeo<DT, D>::kCols / G;  // query tokens per q-tile
  constexpr int kQuads = D / 4;
  constexpr int kGroups = kPfSlotCols / kMergeCols;
  const int j = xcd_unit(blockIdx.x, queue[kPfQMerges] * kGroups);
  if (j < 0) return;
  const PfMerge mg = merges[j / kGroups];
  const int c0 = (j % kGroups) * kMergeCols;
  const int hq = num_kv_heads * G;
  const int tq0 = mg.qtile * QT;
  const int ncols = min((min(mg.q_len, tq0 + QT) - tq0) * G - c0, kMergeCols);
  for (int u = threadIdx.x; u < ncols * kQuads; u += blockDim.x) {
    const int col = c0 + u / kQuads, d = (u % kQuads) * 4;
    float M = -INFINITY, den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < mg.np; p0 += kBatch) {
      float2 ml[kBatch];
      f32x4 op[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int p = min(p0 + k, mg.np - 1);  // past the end: re-read the last (weight 0)
        const int64_t row = (int64_t)(mg.slot0 + p) * kPfSlotCols + col;
        ml[k] = part_ml[row];
        op[k] = *(const f32x4*)(part_o + row * D + d);
      }
      float bm = M;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) bm = fmaxf(bm, ml[k].x);
      const float bmu = bm == -INFINITY ? 0.f : bm;  // no key seen yet in any piece
      const float f0 = fast_exp2(M - bmu);
      num *= f0;
      den *= f0;
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        // pieces that hide the column (m = -inf, l = 0) weigh 0
        const float f = p0 + k < mg.np ? fast_exp2(ml[k].x - bmu) * ml[k].y : 0.f;
        num += f * op[k];
        den += f;
      }
      M = bm;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    store4<DT>(out, ((int64_t)(mg.qb + tq0 + col / G) * hq + mg.h * G + col % G) * D + d, num * inv);
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
  const PfLayout L(a.pf_items, a.pf_slots, D);
  PfItem* items = (PfItem*)((char*)a.ws_pf + L.items);
  int2* tiles = (int2*)((char*)a.ws_pf + L.tiles);
  PfMerge* merges = (PfMerge*)((char*)a.ws_pf + L.merges);
  int32_t* queue = (int32_t*)((char*)a.ws_pf + L.queue);
  float* part_o = (float*)((char*)a.ws_pf + L.part_o);
  float2* part_ml = (float2*)((char*)a.ws_pf + L.part_ml);
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(1024), 0, a.stream, a.seq_lens, a.qsl,
                     a.num_seqs, a.num_kv_heads, G, P::kCols,
                     small_chunk_max_cols(DT::kBytes == 2 ? PKV_BF16 : PKV_F32, D), a.bt_stride,
                     P::kStageB, grid < kPfSplitWorkers ? grid : kPfSplitWorkers, (int)a.pf_slots,
                     items, tiles, merges, queue, (int)(a.pf_items + a.pf_slots));
  hipLaunchKernelGGL((prefill_tiled_kernel<DT, D, G>), dim3(grid), dim3(kPfThreads), P::kLdsBytes,
                     a.stream, (const T*)a.q, (T*)a.out, (const T*)a.kp, (const T*)a.vp, a.bt,
                     a.bt_stride, a.seq_lens, a.qsl, a.num_kv_heads, a.scale_log2, items, queue,
                     part_o, part_ml);
  if (a.pf_slots >= 2) {  // split items, if the plan made any: at most pf_slots / 2 merges
    const int64_t mgrid = (a.pf_slots / 2 * (kPfSlotCols / kMergeCols) + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((prefill_merge_kernel<DT, D, G>), dim3((unsigned)mgrid), dim3(256), 0,
                       a.stream, (T*)a.out, part_o, part_ml, a.num_kv_heads, merges, queue);
  }
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

int64_t prefill_slots_bound(int64_t num_seqs, int64_t num_q_tokens) {
  // every row has a query token, so a batch without more tokens than rows has no chunk
  return num_q_tokens > num_seqs ? kPfMaxSlots : 0;
}

int64_t prefill_workspace_bytes(int64_t num_seqs, int64_t num_q_tokens, int64_t num_q_heads,
                                int64_t head_dim) {
  const PfLayout L(prefill_items_bound(num_seqs, num_q_tokens, num_q_heads),
                   prefill_slots_bound(num_seqs, num_q_tokens), head_dim);
  return L.total;
}

}  // namespace pkv
