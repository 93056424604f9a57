/*
 * pkv.h -- paged KV cache and PagedAttention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpkv.  Every call returns an int status (PKV_OK = 0, negative on
 * error); nothing crosses the ABI as a C++ exception and the library never
 * prints.  The caller owns every device buffer (pools, inputs, outputs,
 * metadata, workspace).  Device calls only enqueue work on the caller's HIP
 * stream (passed as void*; NULL means the default stream): they neither
 * allocate nor synchronize, and the caller keeps every buffer alive until the
 * stream has passed the call.  Host-visible scalars are checked before any
 * launch; device-resident metadata (tables, lengths, slots, pairs) is a
 * documented precondition and is not read by the host.
 *
 * What the operations are comes from these pages:
 *   [blog]    blog.mckayzhao.com/?p=56 ("vLLM" essay)
 *   [devpress] devpress.csdn.net/amd/6a408ab810ee7a33f2834f35.html (explainer)
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PKV_OK 0
#define PKV_ERR_INVALID_ARGUMENT (-1) /* a host-visible argument is out of range */
#define PKV_ERR_UNSUPPORTED (-2)      /* dtype / head_dim / group size not built */
#define PKV_ERR_OUT_OF_BLOCKS (-3)    /* the free pool cannot satisfy the request */
#define PKV_ERR_REFCOUNT (-4)         /* reference count would leave its range */
#define PKV_ERR_WORKSPACE (-5)        /* workspace missing or too small */
#define PKV_ERR_HIP (-6)              /* a HIP runtime call failed */

/* Static string for a status code (never NULL). */
const char* pkv_status_string(int status);

/* ---- element types ------------------------------------------------------- */
#define PKV_F32 0
#define PKV_F16 1
#define PKV_BF16 2

/* Tokens per KV block: the pages' default block size ([blog] "PagedAttention"). */
#define PKV_BLOCK_SIZE 16

/*
 * Block pool descriptor.  The KV cache is a pool of equal blocks, each holding
 * the K and V entries of 16 tokens; any block can serve any sequence, which
 * reaches its blocks through a block table ([blog] "PagedAttention";
 * [devpress] "PagedAttention: core idea").
 *
 * k_pool and v_pool are device buffers, each laid out as
 *     [num_layers][num_blocks][num_kv_heads][tile]
 * A tile holds the 16 tokens x head_dim elements of one block and one KV head
 * (16 * head_dim * element_bytes bytes, contiguous).  With x = 16 / element
 * bytes (elements per 16-byte chunk) and x4 = x / 4, element (t, d) of a tile,
 * t in [0,16), d in [0,head_dim), sits at
 *     K tile: ((d / x) * 16 + t) * x + d % x
 *     V tile: (((m * 4 + g) * 16 + c) * x4 + r) * 4 + j
 *             where t = 4g + j, d = 16n + c, m = n / x4, r = n % x4
 * (integer division).  K keeps each 16-byte run of head dims of the 16 tokens
 * together; V keeps four consecutive tokens of each head dim together.  Both
 * are the operand order of gfx950's matrix instructions, so attention reads
 * every tile as four fully coalesced 1 KiB wave loads (bf16, head_dim 128).
 * Slot s (see kv_cache_write) is block s / 16, token position s % 16.
 */
typedef struct pkv_cache {
  void* k_pool;
  void* v_pool;
  int32_t num_layers;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* PKV_F32, PKV_F16 or PKV_BF16 */
} pkv_cache_t;

/* Bytes of ONE pool (K or V) described by `cache`; 0 if the shape is invalid. */
size_t pkv_pool_bytes(const pkv_cache_t* cache);

/*
 * Supported shapes: dtype f32/f16/bf16; head_dim 64, 128 or 256; query heads
 * per KV head (group) 1, 2, 4 or 8.  Anything else is PKV_ERR_UNSUPPORTED.
 */

/* ---- device calls -------------------------------------------------------- */

/*
 * kv_cache_write: append the K and V entries of new tokens to the cache.  Each
 * token processed in prefill or decode adds one entry ([devpress], prefill /
 * decode / KV cache section: the cache grows by one note per token).
 *   k_new, v_new   device, [num_tokens][num_kv_heads][head_dim], pool dtype;
 *                  k_new 16-byte aligned, v_new aligned to its element
 *   slot_mapping   device int64 [num_tokens]; token i goes to block
 *                  slot/16, position slot%16; a negative slot, or one at or past
 *                  num_blocks * 16, is skipped
 *   layer          which layer of the pools to write
 * Bytes are copied unchanged (no arithmetic); bytes of slots the call does not
 * name keep their values.  Four consecutive tokens that fill positions 4g..4g+3
 * of one block (the tokens of a prefill chunk) have their V written as whole
 * 16-byte chunks; other tokens' V is written element by element.  Two tokens of one call must not share a slot (the
 * allocator never hands out a slot twice).  num_tokens = 0 is a no-op; above
 * 2^30 tokens, or with more than 65535 KV heads, the call returns
 * PKV_ERR_UNSUPPORTED (split the write).
 */
int pkv_kv_cache_write(const pkv_cache_t* cache, int32_t layer, const void* k_new,
                       const void* v_new, const int64_t* slot_mapping, int32_t num_tokens,
                       void* stream);

/*
 * copy_blocks: copy-on-write copies.  A sequence about to modify a shared
 * block first gets a copy and modifies that; the original block is left
 * unchanged ([blog], copy-on-write section).
 *   pairs   device int32 [num_pairs][2] = (src, dst) physical block ids; a pair
 *           naming a block outside [0, num_blocks) is skipped
 * Copies K and V, every KV head and every layer, bit for bit.  A dst must not
 * appear twice, nor also as a src, in one call.  num_pairs = 0 is a no-op.
 */
int pkv_copy_blocks(const pkv_cache_t* cache, const int32_t* pairs, int32_t num_pairs,
                    void* stream);

/* ---- measurement only (not part of the hot path) -------------------------- */
/*
 * Read `bytes` of device
 * memory at buf once, as a plain stream (16-byte non-temporal loads, several in
 * flight per thread), on `stream`.  The time it takes is the practical HBM read
 * rate the attention kernels are compared with, beside the nominal peak.
 *   buf, sink  device pointers, 16-byte aligned; sink: 16 bytes the kernel may
 *              write (a fold of the data), owned by the caller
 *   bytes      a multiple of 16; 0 is a no-op
 * Asynchronous; PKV_ERR_INVALID_ARGUMENT on misalignment or a NULL pointer.
 */
int pkv_calib_stream_read(const void* buf, size_t bytes, void* sink, void* stream);

/*
 * paged_attention: softmax attention for a batch of sequences whose K/V live
 * in the block pool.  The kernel finds every block through the block table
 * and reads K and V block by block; the result equals attention over the same
 * tokens stored contiguously ([blog] "PagedAttention").
 *   q              device [num_q_tokens][num_q_heads][head_dim], pool dtype
 *   out            device, same shape and dtype; written with round-to-nearest-even
 *   block_tables   device int32 [num_seqs][bt_stride]; entry j of row s is the
 *                  physical block of tokens 16j..16j+15 of sequence s
 *   seq_lens       device int32 [num_seqs]: tokens in the cache for each
 *                  sequence, INCLUDING this step's tokens (written before)
 *   query_start_loc device int32 [num_seqs + 1]: sequence s owns query rows
 *                  qsl[s] .. qsl[s+1]-1.  A sequence with q_len = qsl[s+1]-qsl[s]
 *                  query rows is a decode (q_len = 1) or a prefill chunk
 *                  (q_len > 1): row i sits at position seq_len - q_len + i and
 *                  sees keys 0 .. seq_len - q_len + i (causal inside the chunk,
 *                  the whole cached context before it).  This is the mixed
 *                  batch the pages describe as one {request_id: num_tokens}
 *                  schedule ([blog] "V1"; chunked prefill under advanced
 *                  features).
 *   max_q_len, max_seq_len   host-known upper bounds over the batch
 *   scale          softmax scale applied to q.k (usually 1/sqrt(head_dim))
 *   workspace      device scratch of at least pkv_paged_attention_workspace_bytes()
 *   flags          0, or PKV_ATTN_SHARED_PREFIXES (below)
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).  Preconditions
 * (not checked on the device): 1 <= q_len <= seq_len <= max_seq_len,
 * q_len <= max_q_len, ceil(seq_len/16) <= bt_stride, table entries < num_blocks.
 * A sequence with seq_len = 0 and q_len >= 1 yields zeros.
 * Accumulation is fp32.  The output is bitwise reproducible run to run and
 * independent of where blocks sit in the pool.  Long decode rows are split into
 * partitions of 1024 to 4096 tokens, a size the call chooses from the lengths of
 * the whole batch (and 1024 under PKV_ATTN_SHARED_PREFIXES); the size sets the
 * order of a row's fp32 sums, so the batch around a row, and that flag, can move
 * its output by rounding (within the tolerance of the arithmetic), never more.
 */
int pkv_paged_attention(const pkv_cache_t* cache, int32_t layer, void* out, const void* q,
                        const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                        const int32_t* query_start_loc, int32_t num_seqs, int32_t num_q_tokens,
                        int32_t max_q_len, int32_t max_seq_len, int32_t num_q_heads, float scale,
                        void* workspace, size_t workspace_bytes, uint32_t flags, void* stream);

/* flags of pkv_paged_attention (any other bit: PKV_ERR_INVALID_ARGUMENT).
 * PKV_ATTN_SHARED_PREFIXES: rows share prefixes of blocks (parallel samples or
 *   beam candidates that point at the same blocks, prefix-cache hits; [blog]
 *   copy-on-write section).  A hint about speed: the work is then ordered so
 *   that rows read shared blocks at about the same time, in 1024-token partitions
 *   (pkv_ba_num_shared() > 0 tells a caller that some block has several users).
 *   Results change by rounding at most (see the partition size above). */
#define PKV_ATTN_SHARED_PREFIXES 1u

/*
 * contiguous_attention: the baseline the pages compare paging against -- every
 * sequence's K/V stored as one contiguous run of blocks, reached without a block
 * table ([blog] "PagedAttention": paged reads give the same result as contiguous
 * storage at a per-kernel cost).  Decode rows only.
 *   first_block    device int32 [num_seqs]: block j of sequence s is first_block[s] + j
 *   other arguments as for pkv_paged_attention (max_q_len is 1)
 * Same kernels and arithmetic as pkv_paged_attention: on a pool whose sequences
 * occupy consecutive blocks the two give identical bits.  Rows of sequences with
 * q_len != 1 are not written.  Preconditions (not checked on the device):
 * first_block[s] + ceil(seq_len/16) <= num_blocks.  Workspace as for
 * pkv_paged_attention_workspace_bytes(num_seqs, num_q_tokens, max_seq_len, ...).
 */
int pkv_contiguous_attention(const pkv_cache_t* cache, int32_t layer, void* out, const void* q,
                             const int32_t* first_block, const int32_t* seq_lens,
                             const int32_t* query_start_loc, int32_t num_seqs,
                             int32_t num_q_tokens, int32_t max_seq_len, int32_t num_q_heads,
                             float scale, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes pkv_paged_attention needs for these bounds (0 on bad input). */
size_t pkv_paged_attention_workspace_bytes(int32_t num_seqs, int32_t num_q_tokens,
                                           int32_t max_seq_len, int32_t num_q_heads,
                                           int32_t head_dim);

/*
 * paged_attention for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid allocation.  Same
 * arguments, kernels and results as pkv_paged_attention, without the workspace
 * arguments: the workspace is a static device array of PKV_STATIC_WORKSPACE_BYTES
 * inside the library, one per GPU, held from the library's load on that GPU until
 * the process ends.  The call allocates nothing and frees nothing.
 *   PKV_ERR_WORKSPACE if pkv_paged_attention_workspace_bytes() for these bounds
 *   exceeds PKV_STATIC_WORKSPACE_BYTES (256 MiB: every workload of up to 256 rows
 *   of 8,192 tokens at 32 query heads, or a mixed batch of 16 prefill chunks over
 *   32,768-token contexts plus 128 decodes, fits).
 * Every call on one GPU uses that GPU's one array: calls that overlap on a GPU
 * (on different streams, or from different threads) race and must not be issued;
 * calls in one stream are ordered and safe.  The array keeps the last call's
 * contents; nothing in it needs to start at zero.
 */
#define PKV_STATIC_WORKSPACE_BYTES ((size_t)256 << 20)
int pkv_paged_attention_no_alloc(const pkv_cache_t* cache, int32_t layer, void* out,
                                 const void* q, const int32_t* block_tables, int32_t bt_stride,
                                 const int32_t* seq_lens, const int32_t* query_start_loc,
                                 int32_t num_seqs, int32_t num_q_tokens, int32_t max_q_len,
                                 int32_t max_seq_len, int32_t num_q_heads, float scale,
                                 uint32_t flags, void* stream);

/* ---- host block allocator (plain C, no GPU use) -------------------------- */
/*
 * A pool of equal blocks handed out on demand: a sequence gets a new block
 * when its last block is full, and any free block will do ([devpress]
 * "PagedAttention: core idea", steps one and two).  N tokens use ceil(N/16)
 * blocks, wasting at most 15 slots in the last block ([blog]
 * "PagedAttention").  Blocks carry reference counts so that several
 * sequences can point at one block; a sequence about to modify a shared
 * block copies it first ([blog], copy-on-write section).  A finished
 * sequence returns all its blocks ([devpress], core idea).
 *
 * Policy (the pages leave it open): the free pool is a FIFO queue seeded
 * with free_order (or 0..num_blocks-1); allocation takes the front, a block
 * whose count reaches zero goes to the back.  Handles are opaque, owned by
 * the library until pkv_ba_destroy, and not thread-safe.
 */
typedef struct pkv_ba pkv_ba_t;

/* free_order: host int32 [num_blocks] permutation of 0..num_blocks-1, or NULL.
 * block_size must be PKV_BLOCK_SIZE. */
int pkv_ba_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                  pkv_ba_t** out);
void pkv_ba_destroy(pkv_ba_t* ba);
/* Take a free block; its count becomes 1.  PKV_ERR_OUT_OF_BLOCKS if none. */
int pkv_ba_alloc(pkv_ba_t* ba, int32_t* block);
/* Count + 1 of an allocated block (PKV_ERR_REFCOUNT if it is free). */
int pkv_ba_incref(pkv_ba_t* ba, int32_t block);
/* Count - 1; at zero the block returns to the free pool (PKV_ERR_REFCOUNT if free). */
int pkv_ba_decref(pkv_ba_t* ba, int32_t block);
int pkv_ba_refcount(const pkv_ba_t* ba, int32_t block, int32_t* count);
int32_t pkv_ba_num_free(const pkv_ba_t* ba);
int32_t pkv_ba_num_blocks(const pkv_ba_t* ba);
/* ceil(n / block_size), or -1 if n < 0 or block_size <= 0. */
int64_t pkv_blocks_for_tokens(int64_t n, int32_t block_size);

/*
 * Append n_new tokens to a sequence described by (table[cap], *nblk,
 * *seq_len); *nblk must equal ceil(*seq_len/16).  Writes n_new int64 slots.
 * If the first new token lands in a partially filled last block shared with
 * another sequence (count > 1), that block is copied first: a new block is
 * allocated, the old one's count drops by one, the table points at the copy,
 * and (src, dst) is written to cow_pair[0..1] with *n_cow = 1 (else 0); the
 * caller must run pkv_copy_blocks on that pair before writing the slots.
 * New blocks follow in logical order.  All or nothing: on any error nothing
 * changes.  Errors: PKV_ERR_OUT_OF_BLOCKS, PKV_ERR_INVALID_ARGUMENT (table
 * too small, inconsistent state, last entry not a block id), PKV_ERR_REFCOUNT
 * (the last block is free).  Only the last existing entry is read, so a call
 * costs O(new blocks), not O(context); the whole table is checked by
 * pkv_seq_fork, pkv_seq_reorder and pkv_seq_free.
 */
int pkv_seq_append_slots(pkv_ba_t* ba, int32_t* table, int32_t cap, int32_t* nblk,
                         int32_t* seq_len, int32_t n_new, int64_t* slots_out, int32_t* cow_pair,
                         int32_t* n_cow);

/*
 * The same for a batch: sequence s uses tables[s * cap ...], nblk[s],
 * seq_lens[s] and appends n_new[s] tokens; slots go out back to back in
 * sequence order, copy-on-write pairs to cow_pairs (room for num_seqs pairs),
 * their number to *n_cow.  Sequences are processed in order; on an error at
 * sequence k, sequences 0..k-1 keep their appends, sequence k is unchanged,
 * and *n_done = k.
 */
int pkv_batch_append_slots(pkv_ba_t* ba, int32_t* tables, int32_t cap, int32_t* nblk,
                           int32_t* seq_lens, const int32_t* n_new, int32_t num_seqs,
                           int64_t* slots_out, int32_t* cow_pairs, int32_t* n_cow,
                           int32_t* n_done);

/* Copy-on-write of logical block j ahead of a modification: if its count is
 * above one, allocate a copy, point table[j] at it, drop one count of the
 * original and report (src, dst) in pair (*n_cow = 1); otherwise *n_cow = 0. */
int pkv_seq_make_writable(pkv_ba_t* ba, int32_t* table, int32_t nblk, int32_t j, int32_t* pair,
                          int32_t* n_cow);

/* A child sequence sharing every block of the parent (each count + 1);
 * dst_table receives the nblk entries.  All or nothing. */
int pkv_seq_fork(pkv_ba_t* ba, const int32_t* src_table, int32_t nblk, int32_t* dst_table);

/* A finished sequence: drop one count of each block in logical order; blocks
 * reaching zero return to the free pool.  All or nothing. */
int pkv_seq_free(pkv_ba_t* ba, const int32_t* table, int32_t nblk);

/* ---- prefix cache (host) --------------------------------------------------- */
/*
 * Hash-based automatic prefix caching: a request whose prompt begins with the
 * same tokens as an earlier one reuses the earlier request's full KV blocks
 * instead of recomputing them ([blog] advanced features and V1: prefix caching
 * by hash, on by default; [devpress] sharing section: prompt caching).
 *
 * A full block caches the K/V of one exact prompt prefix (the K/V of a token
 * depend on every token before it).  It is sealed with the 16 token ids it
 * holds and its parent: the cached block of the prefix before it (-1 for a
 * prompt's first block).  A sealed block stays in the cache while it is in use
 * and after its count drops to zero; the free pool hands out the block
 * released longest ago first, and a cached block taken that way leaves the
 * cache together with every block cached below it (their prefixes begin with
 * the evicted one).  The contents of a sealed block must not change, and a
 * block appears at most once in a table.
 */

/* Chained 64-bit hash of one block's 16 token ids after a parent hash (0 for
 * the first block).  Lookups locate candidates with it and then compare the
 * parent block and the token ids exactly; a parent is always a live cached
 * prefix, so a hash collision cannot produce a wrong hit. */
uint64_t pkv_prefix_hash(uint64_t parent_hash, const int32_t* tokens16);

/* Start a new sequence from the cache: walk the full blocks of its prompt
 * tokens[0..num_tokens) in order and take each cached block that continues the
 * chain (count + 1; a free cached block leaves the free pool), stopping at the
 * first miss or at cap blocks.  table[0..*nblk) receives the blocks; the
 * sequence then holds *nblk * 16 cached tokens and appends the rest with
 * pkv_seq_append_slots.  Never allocates, so it cannot run out of blocks. */
int pkv_seq_cache_lookup(pkv_ba_t* ba, const int32_t* tokens, int32_t num_tokens, int32_t* table,
                         int32_t cap, int32_t* nblk);

/* Register the full blocks of a sequence (table[0..nblk) holding
 * tokens[0..num_tokens)) in the cache once their K/V are written.  Blocks
 * already cached must hold the same prefix (PKV_ERR_INVALID_ARGUMENT
 * otherwise, and nothing changes); a block whose prefix is cached in another
 * block stays out of the cache, and the next block is cached after that other
 * block. */
int pkv_seq_cache_seal(pkv_ba_t* ba, const int32_t* tokens, int32_t num_tokens,
                       const int32_t* table, int32_t nblk);

/*
 * Beam reorder: after a beam-search step the surviving candidates continue some
 * of the old rows, several children per parent or none ([blog] beam search: the
 * candidates share their beginning; [devpress] "how memory is shared").  In
 * place, for num_rows rows of tables [num_rows][cap], nblk and seq_lens: new row
 * i becomes a copy of old row parents[i].  Every block of a parent gains one user
 * per child (in child order), then every block of every old row loses one (in row
 * order; a block left without users joins the free queue).  The next append to a
 * row whose last block is shared and partly filled copies that block
 * (pkv_seq_append_slots, copy-on-write).
 *   parents  int32 [num_rows], each in [0, num_rows)
 *   work     int32 scratch of num_rows * cap entries, owned by the caller
 * Checks everything first: on an error nothing changes (PKV_ERR_INVALID_ARGUMENT,
 * or PKV_ERR_REFCOUNT if a count would overflow or names a free block).
 */
int pkv_seq_reorder(pkv_ba_t* ba, int32_t* tables, int32_t cap, int32_t* nblk, int32_t* seq_lens,
                    int32_t num_rows, const int32_t* parents, int32_t* work);

/* Blocks currently in the cache (in use or free). */
int32_t pkv_ba_num_cached(const pkv_ba_t* ba);

/* Blocks with a reference count of two or more: blocks that several sequences
 * share after a fork or a prefix-cache hit ([devpress] "how memory is shared").
 * -1 for a NULL handle. */
int32_t pkv_ba_num_shared(const pkv_ba_t* ba);

/* ---- host checks of kernel metadata (plain C, no GPU use) ---------------- */
/*
 * The kernels trust the metadata they are given (they only skip slots and block
 * ids outside the pool).  These calls check the rules of the block scheme on
 * HOST copies of that metadata, for callers that want a check before a launch
 * (tests, debugging).  Each returns PKV_OK, or PKV_ERR_INVALID_ARGUMENT and
 * writes the index of the first offending entry to *bad (-1 when the sizes or
 * pointers themselves are wrong); bad may be NULL.  Nothing is modified.
 *
 * pkv_check_slot_mapping: for kv_cache_write.  Every slot is negative (a
 *   padding token) or below num_blocks * 16, and no slot is named twice: a
 *   slot holds one token ([devpress] prefill / decode / KV cache section).
 *   *bad is the earliest token with a slot out of the pool or a slot that an
 *   earlier token already names.
 */
int pkv_check_slot_mapping(const int64_t* slots, int32_t num_tokens, int32_t num_blocks,
                           int32_t* bad);
/* pkv_check_copy_pairs: for copy_blocks.  pairs [num_pairs][2] = (src, dst):
 *   both in [0, num_blocks), src != dst, no dst named twice, and no dst that is
 *   also a src of the call (a copy goes to a new private block, [blog]
 *   copy-on-write section).  *bad is the earliest pair that breaks a rule. */
int pkv_check_copy_pairs(const int32_t* pairs, int32_t num_pairs, int32_t num_blocks,
                         int32_t* bad);
/* pkv_check_batch: for paged_attention, the preconditions it states: per
 *   sequence 1 <= q_len <= max_q_len, 0 <= seq_len <= max_seq_len, q_len <=
 *   seq_len unless seq_len = 0, ceil(seq_len / 16) <= bt_stride and each of those
 *   table entries in [0, num_blocks); query_start_loc[0] >= 0 and
 *   query_start_loc[num_seqs] <= num_q_tokens (else *bad = -1).  *bad is the
 *   earliest sequence that breaks a rule. */
int pkv_check_batch(const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                    const int32_t* query_start_loc, int32_t num_seqs, int32_t num_q_tokens,
                    int32_t max_q_len, int32_t max_seq_len, int32_t num_blocks, int32_t* bad);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
