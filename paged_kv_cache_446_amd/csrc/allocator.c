/*
 * Host block allocator with reference counts (plain C99, no GPU use).
 *
 * The KV cache is a pool of equal blocks handed out on demand: a sequence gets
 * a new block when its last block fills, any free block will do, and a
 * finished sequence returns every block (devpress.csdn.net/amd/
 * 6a408ab810ee7a33f2834f35.html, section "PagedAttention: core idea").  N
 * tokens need ceil(N/16) blocks (blog.mckayzhao.com/?p=56, section
 * "PagedAttention").  Shared blocks carry reference counts and are copied
 * before a sequence modifies them (same blog page, copy-on-write section).
 *
 * Free pool: a FIFO ring of block ids.  Allocation pops the front; a block
 * whose count reaches zero is pushed at the back.
 */
#include <stdlib.h>
#include <string.h>

#include "pkv.h"

struct pkv_ba {
  int32_t num_blocks;
  int32_t* ref;  /* [num_blocks] reference counts, 0 = free */
  int32_t* ring; /* [num_blocks] free queue storage */
  int32_t head;  /* index of the front element */
  int32_t count; /* number of free blocks */
};

static int32_t ring_pop_front(pkv_ba_t* ba) {
  int32_t b = ba->ring[ba->head];
  ba->head = (ba->head + 1) % ba->num_blocks;
  ba->count--;
  return b;
}

static void ring_push_back(pkv_ba_t* ba, int32_t b) {
  ba->ring[(ba->head + ba->count) % ba->num_blocks] = b;
  ba->count++;
}

/* undo the newest push_back (the block must be at the back) */
static void ring_pop_back(pkv_ba_t* ba) { ba->count--; }

int64_t pkv_blocks_for_tokens(int64_t n, int32_t block_size) {
  if (n < 0 || block_size <= 0) return -1;
  return (n + block_size - 1) / block_size;
}

int pkv_ba_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                  pkv_ba_t** out) {
  if (!out) return PKV_ERR_INVALID_ARGUMENT;
  *out = NULL;
  if (num_blocks <= 0 || block_size != PKV_BLOCK_SIZE) return PKV_ERR_INVALID_ARGUMENT;
  pkv_ba_t* ba = (pkv_ba_t*)calloc(1, sizeof(pkv_ba_t));
  if (!ba) return PKV_ERR_INVALID_ARGUMENT;
  ba->ref = (int32_t*)calloc((size_t)num_blocks, sizeof(int32_t));
  ba->ring = (int32_t*)malloc((size_t)num_blocks * sizeof(int32_t));
  if (!ba->ref || !ba->ring) {
    pkv_ba_destroy(ba);
    return PKV_ERR_INVALID_ARGUMENT;
  }
  ba->num_blocks = num_blocks;
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = free_order ? free_order[i] : i;
    /* free_order must be a permutation: use ref[] as the seen-set */
    if (b < 0 || b >= num_blocks || ba->ref[b]) {
      pkv_ba_destroy(ba);
      return PKV_ERR_INVALID_ARGUMENT;
    }
    ba->ref[b] = 1;
    ba->ring[i] = b;
  }
  memset(ba->ref, 0, (size_t)num_blocks * sizeof(int32_t));
  ba->head = 0;
  ba->count = num_blocks;
  *out = ba;
  return PKV_OK;
}

void pkv_ba_destroy(pkv_ba_t* ba) {
  if (!ba) return;
  free(ba->ref);
  free(ba->ring);
  free(ba);
}

static int valid_id(const pkv_ba_t* ba, int32_t b) { return b >= 0 && b < ba->num_blocks; }

int pkv_ba_alloc(pkv_ba_t* ba, int32_t* block) {
  if (!ba || !block) return PKV_ERR_INVALID_ARGUMENT;
  if (ba->count == 0) return PKV_ERR_OUT_OF_BLOCKS;
  int32_t b = ring_pop_front(ba);
  ba->ref[b] = 1;
  *block = b;
  return PKV_OK;
}

int pkv_ba_incref(pkv_ba_t* ba, int32_t block) {
  if (!ba || !valid_id(ba, block)) return PKV_ERR_INVALID_ARGUMENT;
  if (ba->ref[block] <= 0) return PKV_ERR_REFCOUNT;
  if (ba->ref[block] == INT32_MAX) return PKV_ERR_REFCOUNT;
  ba->ref[block]++;
  return PKV_OK;
}

int pkv_ba_decref(pkv_ba_t* ba, int32_t block) {
  if (!ba || !valid_id(ba, block)) return PKV_ERR_INVALID_ARGUMENT;
  if (ba->ref[block] <= 0) return PKV_ERR_REFCOUNT;
  if (--ba->ref[block] == 0) ring_push_back(ba, block);
  return PKV_OK;
}

int pkv_ba_refcount(const pkv_ba_t* ba, int32_t block, int32_t* count) {
  if (!ba || !count || !valid_id(ba, block)) return PKV_ERR_INVALID_ARGUMENT;
  *count = ba->ref[block];
  return PKV_OK;
}

int32_t pkv_ba_num_free(const pkv_ba_t* ba) { return ba ? ba->count : -1; }

int32_t pkv_ba_num_blocks(const pkv_ba_t* ba) { return ba ? ba->num_blocks : -1; }

/* every entry of table[0..nblk) must name an allocated block */
static int check_table(const pkv_ba_t* ba, const int32_t* table, int32_t nblk) {
  for (int32_t j = 0; j < nblk; ++j) {
    if (!valid_id(ba, table[j])) return PKV_ERR_INVALID_ARGUMENT;
    if (ba->ref[table[j]] <= 0) return PKV_ERR_REFCOUNT;
  }
  return PKV_OK;
}

int pkv_seq_append_slots(pkv_ba_t* ba, int32_t* table, int32_t cap, int32_t* nblk,
                         int32_t* seq_len, int32_t n_new, int64_t* slots_out, int32_t* cow_pair,
                         int32_t* n_cow) {
  if (!ba || !table || !nblk || !seq_len || !n_cow || (n_new > 0 && !slots_out) || !cow_pair)
    return PKV_ERR_INVALID_ARGUMENT;
  const int64_t len = *seq_len;
  const int32_t nb = *nblk;
  if (n_new < 0 || len < 0 || cap < 0 || nb != pkv_blocks_for_tokens(len, PKV_BLOCK_SIZE))
    return PKV_ERR_INVALID_ARGUMENT;
  if (len + n_new > INT32_MAX) return PKV_ERR_INVALID_ARGUMENT;
  const int64_t need_blocks = pkv_blocks_for_tokens(len + n_new, PKV_BLOCK_SIZE);
  if (need_blocks > cap) return PKV_ERR_INVALID_ARGUMENT;
  int rc = check_table(ba, table, nb);
  if (rc != PKV_OK) return rc;
  const int cow = n_new > 0 && (len % PKV_BLOCK_SIZE) != 0 && ba->ref[table[nb - 1]] > 1;
  if (need_blocks - nb + cow > ba->count) return PKV_ERR_OUT_OF_BLOCKS;
  *n_cow = 0;
  if (cow) {
    int32_t src = table[nb - 1], dst;
    pkv_ba_alloc(ba, &dst);
    pkv_ba_decref(ba, src); /* count > 1, so it stays allocated */
    table[nb - 1] = dst;
    cow_pair[0] = src;
    cow_pair[1] = dst;
    *n_cow = 1;
  }
  for (int64_t j = nb; j < need_blocks; ++j) pkv_ba_alloc(ba, &table[j]);
  for (int32_t i = 0; i < n_new; ++i) {
    const int64_t p = len + i;
    slots_out[i] = (int64_t)table[p / PKV_BLOCK_SIZE] * PKV_BLOCK_SIZE + p % PKV_BLOCK_SIZE;
  }
  *nblk = (int32_t)need_blocks;
  *seq_len = (int32_t)(len + n_new);
  return PKV_OK;
}

int pkv_batch_append_slots(pkv_ba_t* ba, int32_t* tables, int32_t cap, int32_t* nblk,
                           int32_t* seq_lens, const int32_t* n_new, int32_t num_seqs,
                           int64_t* slots_out, int32_t* cow_pairs, int32_t* n_cow,
                           int32_t* n_done) {
  if (!ba || !tables || !nblk || !seq_lens || !n_new || !cow_pairs || !n_cow || !n_done ||
      num_seqs < 0 || cap < 0)
    return PKV_ERR_INVALID_ARGUMENT;
  *n_cow = 0;
  *n_done = 0;
  int64_t off = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t one = 0;
    int rc = pkv_seq_append_slots(ba, tables + (int64_t)s * cap, cap, &nblk[s], &seq_lens[s],
                                  n_new[s], slots_out ? slots_out + off : NULL,
                                  cow_pairs + 2 * (int64_t)(*n_cow), &one);
    if (rc != PKV_OK) return rc;
    *n_cow += one;
    off += n_new[s];
    *n_done = s + 1;
  }
  return PKV_OK;
}

int pkv_seq_make_writable(pkv_ba_t* ba, int32_t* table, int32_t nblk, int32_t j, int32_t* pair,
                          int32_t* n_cow) {
  if (!ba || !table || !pair || !n_cow || j < 0 || j >= nblk) return PKV_ERR_INVALID_ARGUMENT;
  const int32_t src = table[j];
  if (!valid_id(ba, src)) return PKV_ERR_INVALID_ARGUMENT;
  if (ba->ref[src] <= 0) return PKV_ERR_REFCOUNT;
  *n_cow = 0;
  if (ba->ref[src] == 1) return PKV_OK;
  if (ba->count == 0) return PKV_ERR_OUT_OF_BLOCKS;
  int32_t dst;
  pkv_ba_alloc(ba, &dst);
  pkv_ba_decref(ba, src);
  table[j] = dst;
  pair[0] = src;
  pair[1] = dst;
  *n_cow = 1;
  return PKV_OK;
}

int pkv_seq_fork(pkv_ba_t* ba, const int32_t* src_table, int32_t nblk, int32_t* dst_table) {
  if (!ba || !src_table || !dst_table || nblk < 0) return PKV_ERR_INVALID_ARGUMENT;
  int rc = check_table(ba, src_table, nblk);
  if (rc != PKV_OK) return rc;
  for (int32_t j = 0; j < nblk; ++j)
    if (ba->ref[src_table[j]] == INT32_MAX) return PKV_ERR_REFCOUNT;
  for (int32_t j = 0; j < nblk; ++j) {
    ba->ref[src_table[j]]++;
    dst_table[j] = src_table[j];
  }
  return PKV_OK;
}

int pkv_seq_free(pkv_ba_t* ba, const int32_t* table, int32_t nblk) {
  if (!ba || !table || nblk < 0) return PKV_ERR_INVALID_ARGUMENT;
  for (int32_t j = 0; j < nblk; ++j)
    if (!valid_id(ba, table[j])) return PKV_ERR_INVALID_ARGUMENT;
  int32_t j = 0;
  int rc = PKV_OK;
  for (; j < nblk; ++j) {
    rc = pkv_ba_decref(ba, table[j]);
    if (rc != PKV_OK) break;
  }
  if (rc == PKV_OK) return PKV_OK;
  /* undo, newest first: a block that reached zero is the newest push */
  while (--j >= 0) {
    const int32_t b = table[j];
    if (ba->ref[b] == 0) ring_pop_back(ba);
    ba->ref[b]++;
  }
  return rc;
}
