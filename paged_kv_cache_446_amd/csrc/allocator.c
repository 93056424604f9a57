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
 * Free pool: a FIFO queue of block ids (a doubly linked list over block ids, so
 * that a cached block can leave it from the middle).  Allocation pops the
 * front; a block whose count reaches zero is pushed at the back, so the front
 * is the block released longest ago.
 *
 * Prefix cache (hash-based automatic prefix caching: blog page, advanced
 * features and V1 sections; devpress page, sharing section, prompt caching):
 * a full block caches the K/V of one exact prompt prefix.  It is sealed with
 * the 16 token ids it holds and its parent: the cached block of the prefix
 * before it (-1 for a prompt's first block).  Sealed blocks form a forest in
 * which a block's parent is always sealed: when allocation takes a sealed block
 * from the front of the free queue (least recently released first), the block
 * and everything sealed below it leave the cache together.  A lookup walks a
 * new prompt's full blocks, locating each candidate by a chained 64-bit hash
 * and accepting it only if its parent is the block found one step earlier and
 * its token ids are equal; a parent id names a live cached prefix, so a hit is
 * exact whatever the hash does.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "pkv.h"

struct pkv_ba {
  int32_t num_blocks;
  int32_t* ref;  /* [num_blocks] reference counts, 0 = free */
  int32_t* next; /* [num_blocks] free queue links (-1 = none) */
  int32_t* prev;
  int32_t head, tail; /* front and back of the free queue (-1 if empty) */
  int32_t count;      /* number of free blocks */
  int32_t num_shared; /* blocks with a count of 2 or more */
  /* prefix cache */
  uint8_t* sealed;   /* [num_blocks] 1 if the block is in the cache */
  uint64_t* hash;    /* [num_blocks] chained hash of the block's tokens */
  int32_t* parent;   /* [num_blocks] cached block of the prefix before, -1 for the first */
  int32_t* first_child, *next_sib, *prev_sib; /* [num_blocks] sealed children of a sealed block */
  int32_t* tokens;   /* [num_blocks][16] token ids */
  int32_t* slot;     /* [hcap] open-addressing table of sealed block ids; -1 empty, -2 deleted */
  int64_t hcap;      /* power of two >= 2 * num_blocks */
  int32_t num_sealed;
  int64_t num_deleted; /* deleted slots (the table is rebuilt when they pile up) */
};

static void q_remove(pkv_ba_t* ba, int32_t b) {
  const int32_t p = ba->prev[b], n = ba->next[b];
  if (p >= 0) ba->next[p] = n; else ba->head = n;
  if (n >= 0) ba->prev[n] = p; else ba->tail = p;
  ba->next[b] = ba->prev[b] = -1;
  ba->count--;
}

static void unseal(pkv_ba_t* ba, int32_t b);

static int32_t q_pop_front(pkv_ba_t* ba) {
  const int32_t b = ba->head;
  q_remove(ba, b);
  if (ba->sealed[b]) unseal(ba, b); /* the least recently released cached block is evicted */
  return b;
}

static void q_push_back(pkv_ba_t* ba, int32_t b) {
  ba->prev[b] = ba->tail;
  ba->next[b] = -1;
  if (ba->tail >= 0) ba->next[ba->tail] = b; else ba->head = b;
  ba->tail = b;
  ba->count++;
}

/* undo the newest push_back (the block must be at the back) */
static void q_pop_back(pkv_ba_t* ba) { q_remove(ba, ba->tail); }

/* ---- prefix-cache hash table ------------------------------------------------ */

/* the splitmix64 output function (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", 2014) as a 64-bit mixer */
static uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t pkv_prefix_hash(uint64_t parent_hash, const int32_t* tokens) {
  uint64_t h = mix64(parent_hash ^ 0x243F6A8885A308D3ull);
  for (int i = 0; i < PKV_BLOCK_SIZE; ++i) h = mix64(h ^ (uint32_t)tokens[i]);
  return h;
}

/* sealed block equal to (h, parent, tokens), or -1 */
static int32_t find_sealed(const pkv_ba_t* ba, uint64_t h, int32_t parent, const int32_t* tokens) {
  for (int64_t i = (int64_t)(h & (uint64_t)(ba->hcap - 1)), k = 0; k < ba->hcap;
       i = (i + 1) & (ba->hcap - 1), ++k) {
    const int32_t b = ba->slot[i];
    if (b == -1) return -1;
    if (b >= 0 && ba->hash[b] == h && ba->parent[b] == parent &&
        memcmp(ba->tokens + (int64_t)b * PKV_BLOCK_SIZE, tokens, PKV_BLOCK_SIZE * sizeof(int32_t)) == 0)
      return b;
  }
  return -1;
}

static void slot_insert(pkv_ba_t* ba, int32_t b) {
  int64_t i = (int64_t)(ba->hash[b] & (uint64_t)(ba->hcap - 1));
  while (ba->slot[i] >= 0) i = (i + 1) & (ba->hcap - 1);
  if (ba->slot[i] == -2) ba->num_deleted--;
  ba->slot[i] = b;
}

/* rebuild the table without deleted slots (keeps probe sequences short) */
static void rehash(pkv_ba_t* ba) {
  for (int64_t i = 0; i < ba->hcap; ++i) ba->slot[i] = -1;
  ba->num_deleted = 0;
  for (int32_t b = 0; b < ba->num_blocks; ++b)
    if (ba->sealed[b]) slot_insert(ba, b);
}

/* parent: a sealed block or -1 */
static void seal(pkv_ba_t* ba, int32_t b, uint64_t h, int32_t parent, const int32_t* tokens) {
  if (4 * (ba->num_sealed + 1 + ba->num_deleted) > 3 * ba->hcap) rehash(ba);
  ba->hash[b] = h;
  slot_insert(ba, b);
  ba->sealed[b] = 1;
  ba->parent[b] = parent;
  ba->first_child[b] = -1;
  ba->prev_sib[b] = -1;
  ba->next_sib[b] = parent >= 0 ? ba->first_child[parent] : -1;
  if (ba->next_sib[b] >= 0) ba->prev_sib[ba->next_sib[b]] = b;
  if (parent >= 0) ba->first_child[parent] = b;
  memcpy(ba->tokens + (int64_t)b * PKV_BLOCK_SIZE, tokens, PKV_BLOCK_SIZE * sizeof(int32_t));
  ba->num_sealed++;
}

static void drop_from_table(pkv_ba_t* ba, int32_t b) {
  int64_t i = (int64_t)(ba->hash[b] & (uint64_t)(ba->hcap - 1));
  while (ba->slot[i] != b) i = (i + 1) & (ba->hcap - 1);
  ba->slot[i] = -2;
  ba->num_deleted++;
  ba->sealed[b] = 0;
  ba->num_sealed--;
}

/* Remove a sealed block and every block sealed below it from the cache: their
 * prefixes begin with the evicted one, which a lookup can no longer walk. */
static void unseal(pkv_ba_t* ba, int32_t root) {
  const int32_t p = ba->parent[root];
  if (p >= 0) { /* unlink root from its parent's children */
    const int32_t pv = ba->prev_sib[root], nx = ba->next_sib[root];
    if (pv >= 0) ba->next_sib[pv] = nx; else ba->first_child[p] = nx;
    if (nx >= 0) ba->prev_sib[nx] = pv;
  }
  /* pre-order walk of the subtree; the links below root are read, not changed (an
   * unsealed block's links are reset when it is sealed again) */
  int32_t b = root;
  for (;;) {
    drop_from_table(ba, b);
    if (ba->first_child[b] >= 0) {
      b = ba->first_child[b];
      continue;
    }
    while (b != root && ba->next_sib[b] < 0) b = ba->parent[b];
    if (b == root) break;
    b = ba->next_sib[b];
  }
}

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
  const size_t nb = (size_t)num_blocks;
  ba->hcap = 2;
  while (ba->hcap < 2 * (int64_t)num_blocks) ba->hcap *= 2;
  ba->ref = (int32_t*)calloc(nb, sizeof(int32_t));
  ba->next = (int32_t*)malloc(nb * sizeof(int32_t));
  ba->prev = (int32_t*)malloc(nb * sizeof(int32_t));
  ba->sealed = (uint8_t*)calloc(nb, 1);
  ba->hash = (uint64_t*)calloc(nb, sizeof(uint64_t));
  ba->parent = (int32_t*)calloc(nb, sizeof(int32_t));
  ba->first_child = (int32_t*)calloc(nb, sizeof(int32_t));
  ba->next_sib = (int32_t*)calloc(nb, sizeof(int32_t));
  ba->prev_sib = (int32_t*)calloc(nb, sizeof(int32_t));
  ba->tokens = (int32_t*)calloc(nb * PKV_BLOCK_SIZE, sizeof(int32_t));
  ba->slot = (int32_t*)malloc((size_t)ba->hcap * sizeof(int32_t));
  if (!ba->ref || !ba->next || !ba->prev || !ba->sealed || !ba->hash || !ba->parent ||
      !ba->first_child || !ba->next_sib || !ba->prev_sib || !ba->tokens || !ba->slot) {
    pkv_ba_destroy(ba);
    return PKV_ERR_INVALID_ARGUMENT;
  }
  for (int64_t i = 0; i < ba->hcap; ++i) ba->slot[i] = -1;
  ba->num_blocks = num_blocks;
  ba->head = ba->tail = -1;
  for (int32_t i = 0; i < num_blocks; ++i) {
    int32_t b = free_order ? free_order[i] : i;
    /* free_order must be a permutation: use ref[] as the seen-set */
    if (b < 0 || b >= num_blocks || ba->ref[b]) {
      pkv_ba_destroy(ba);
      return PKV_ERR_INVALID_ARGUMENT;
    }
    ba->ref[b] = 1;
    q_push_back(ba, b);
  }
  memset(ba->ref, 0, nb * sizeof(int32_t));
  *out = ba;
  return PKV_OK;
}

void pkv_ba_destroy(pkv_ba_t* ba) {
  if (!ba) return;
  free(ba->ref);
  free(ba->next);
  free(ba->prev);
  free(ba->sealed);
  free(ba->hash);
  free(ba->parent);
  free(ba->first_child);
  free(ba->next_sib);
  free(ba->prev_sib);
  free(ba->tokens);
  free(ba->slot);
  free(ba);
}

static int valid_id(const pkv_ba_t* ba, int32_t b) { return b >= 0 && b < ba->num_blocks; }

/* every count change of an allocated block goes through these two */
static void ref_inc(pkv_ba_t* ba, int32_t b) {
  if (++ba->ref[b] == 2) ba->num_shared++;
}
static void ref_dec(pkv_ba_t* ba, int32_t b) {
  if (ba->ref[b]-- == 2) ba->num_shared--;
}

int pkv_ba_alloc(pkv_ba_t* ba, int32_t* block) {
  if (!ba || !block) return PKV_ERR_INVALID_ARGUMENT;
  if (ba->count == 0) return PKV_ERR_OUT_OF_BLOCKS;
  int32_t b = q_pop_front(ba);
  ba->ref[b] = 1;
  *block = b;
  return PKV_OK;
}

int pkv_ba_incref(pkv_ba_t* ba, int32_t block) {
  if (!ba || !valid_id(ba, block)) return PKV_ERR_INVALID_ARGUMENT;
  if (ba->ref[block] <= 0) return PKV_ERR_REFCOUNT;
  if (ba->ref[block] == INT32_MAX) return PKV_ERR_REFCOUNT;
  ref_inc(ba, block);
  return PKV_OK;
}

int pkv_ba_decref(pkv_ba_t* ba, int32_t block) {
  if (!ba || !valid_id(ba, block)) return PKV_ERR_INVALID_ARGUMENT;
  if (ba->ref[block] <= 0) return PKV_ERR_REFCOUNT;
  ref_dec(ba, block);
  if (ba->ref[block] == 0) q_push_back(ba, block);
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
  /* one pass without early exits (the common case: all good); on a bad entry the
   * ordered walk below names the error of the first one */
  if (nblk > 0 && ba->num_blocks > 0) {
    int bad = 0;
    for (int32_t j = 0; j < nblk; ++j) {
      const int32_t b = table[j];
      const int ok = (uint32_t)b < (uint32_t)ba->num_blocks;
      bad |= !ok | (ba->ref[ok ? b : 0] <= 0);
    }
    if (!bad) return PKV_OK;
  }
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
  /* the one existing entry this call reads (it may write into or copy that block); the
   * rest of the table is checked by the calls that walk it (fork, reorder, free) */
  int rc = check_table(ba, table + (nb > 0 ? nb - 1 : 0), nb > 0 ? 1 : 0);
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
    ref_inc(ba, src_table[j]);
    dst_table[j] = src_table[j];
  }
  return PKV_OK;
}

int pkv_seq_reorder(pkv_ba_t* ba, int32_t* tables, int32_t cap, int32_t* nblk, int32_t* seq_lens,
                    int32_t num_rows, const int32_t* parents, int32_t* work) {
  if (!ba || num_rows < 0 || cap < 0 || (num_rows > 0 && (!tables || !nblk || !seq_lens ||
                                                          !parents || !work)))
    return PKV_ERR_INVALID_ARGUMENT;
  /* check everything first: nothing changes on an error */
  for (int32_t r = 0; r < num_rows; ++r) {
    if (nblk[r] < 0 || nblk[r] > cap || seq_lens[r] < 0 ||
        nblk[r] != pkv_blocks_for_tokens(seq_lens[r], PKV_BLOCK_SIZE))
      return PKV_ERR_INVALID_ARGUMENT;
    if (parents[r] < 0 || parents[r] >= num_rows) return PKV_ERR_INVALID_ARGUMENT;
    int rc = check_table(ba, tables + (int64_t)r * cap, nblk[r]);
    if (rc != PKV_OK) return rc;
  }
  /* Child i and old row i often hold the same blocks in the same columns (their
   * shared beginning): such a block gains and loses one user, stays allocated (child
   * i keeps it) and ends with its old count, so both steps are skipped for the first
   * same[i] columns, where the two rows agree.  What is left runs in the same order
   * as the full walk -- gains in child order, then losses in row order -- so the
   * final counts and the order of freed blocks are those of the full walk.  same[]
   * lives in work until step 3 (cap >= 1 whenever a row holds a block). */
  int32_t* same = work;
  if (cap == 0) return PKV_OK; /* no row holds a block, every row keeps its length 0 */
  for (int32_t i = 0; i < num_rows; ++i) {
    const int32_t* ti = tables + (int64_t)i * cap;
    const int32_t* tp = tables + (int64_t)parents[i] * cap;
    const int32_t n = nblk[i] < nblk[parents[i]] ? nblk[i] : nblk[parents[i]];
    int32_t j = 0;
    if (parents[i] == i) j = n;
    else
      while (j < n && ti[j] == tp[j]) ++j;
    same[i] = j;
  }
  /* every remaining gain: the counts must not overflow */
  for (int32_t i = 0; i < num_rows; ++i) {
    const int32_t* t = tables + (int64_t)parents[i] * cap;
    for (int32_t j = same[i]; j < nblk[parents[i]]; ++j)
      if (ba->ref[t[j]] > INT32_MAX - num_rows) return PKV_ERR_REFCOUNT;
  }
  /* 1. the children take their parents' blocks, in child order */
  for (int32_t i = 0; i < num_rows; ++i) {
    const int32_t* t = tables + (int64_t)parents[i] * cap;
    for (int32_t j = same[i], n = nblk[parents[i]]; j < n; ++j) ref_inc(ba, t[j]);
  }
  /* 2. the old rows let go, in row order (blocks left without users join the free
   *    queue in that order) */
  for (int32_t r = 0; r < num_rows; ++r) {
    const int32_t* t = tables + (int64_t)r * cap;
    for (int32_t j = same[r], n = nblk[r]; j < n; ++j) {
      const int32_t blk = t[j];
      ref_dec(ba, blk);
      if (ba->ref[blk] == 0) q_push_back(ba, blk);
    }
  }
  /* 3. the new rows: copies of their parents (tables through work, then lengths) */
  memcpy(work, tables, (size_t)num_rows * (size_t)cap * sizeof(int32_t));
  for (int32_t i = 0; i < num_rows; ++i)
    if (parents[i] != i)
      memcpy(tables + (int64_t)i * cap, work + (int64_t)parents[i] * cap,
             (size_t)cap * sizeof(int32_t));
  for (int32_t i = 0; i < num_rows; ++i) work[i] = nblk[parents[i]];
  for (int32_t i = 0; i < num_rows; ++i) nblk[i] = work[i];
  for (int32_t i = 0; i < num_rows; ++i) work[i] = seq_lens[parents[i]];
  for (int32_t i = 0; i < num_rows; ++i) seq_lens[i] = work[i];
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
    if (ba->ref[b] == 0) q_pop_back(ba);
    ref_inc(ba, b);
  }
  return rc;
}

/* ---- prefix cache ------------------------------------------------------------ */

int pkv_seq_cache_lookup(pkv_ba_t* ba, const int32_t* tokens, int32_t num_tokens, int32_t* table,
                         int32_t cap, int32_t* nblk) {
  if (!ba || !table || !nblk || num_tokens < 0 || cap < 0 || (num_tokens > 0 && !tokens))
    return PKV_ERR_INVALID_ARGUMENT;
  const int32_t full = num_tokens / PKV_BLOCK_SIZE;
  const int32_t limit = full < cap ? full : cap;
  uint64_t h = 0;
  int32_t j = 0;
  for (; j < limit; ++j) {
    const int32_t* tk = tokens + (int64_t)j * PKV_BLOCK_SIZE;
    h = pkv_prefix_hash(h, tk);
    const int32_t b = find_sealed(ba, h, j ? table[j - 1] : -1, tk);
    if (b < 0 || ba->ref[b] == INT32_MAX) break;
    if (ba->ref[b] == 0) q_remove(ba, b); /* a cached block back from the free queue */
    ref_inc(ba, b);
    table[j] = b;
  }
  *nblk = j;
  return PKV_OK;
}

int pkv_seq_cache_seal(pkv_ba_t* ba, const int32_t* tokens, int32_t num_tokens,
                       const int32_t* table, int32_t nblk) {
  if (!ba || !table || num_tokens < 0 || nblk < 0 || (num_tokens > 0 && !tokens))
    return PKV_ERR_INVALID_ARGUMENT;
  const int32_t full = num_tokens / PKV_BLOCK_SIZE;
  const int32_t n = full < nblk ? full : nblk;
  int rc = check_table(ba, table, n);
  if (rc != PKV_OK) return rc;
  /* Both passes walk the prompt's prefixes; `cur` is the cached block of the prefix
   * before block j: table[j - 1] if it is (or will be) sealed, else the block that
   * already caches the same prefix.  Verify first, then seal: all or nothing. */
  uint64_t h = 0;
  int32_t cur = -1;
  for (int32_t j = 0; j < n; ++j) {
    const int32_t* tk = tokens + (int64_t)j * PKV_BLOCK_SIZE;
    const int32_t b = table[j];
    h = pkv_prefix_hash(h, tk);
    if (ba->sealed[b]) {
      if (ba->hash[b] != h || ba->parent[b] != cur ||
          memcmp(ba->tokens + (int64_t)b * PKV_BLOCK_SIZE, tk, PKV_BLOCK_SIZE * sizeof(int32_t)))
        return PKV_ERR_INVALID_ARGUMENT; /* a cached block must keep its contents */
      cur = b;
    } else {
      const int32_t f = find_sealed(ba, h, cur, tk);
      cur = f >= 0 ? f : b;
    }
  }
  h = 0;
  cur = -1;
  for (int32_t j = 0; j < n; ++j) {
    const int32_t* tk = tokens + (int64_t)j * PKV_BLOCK_SIZE;
    const int32_t b = table[j];
    h = pkv_prefix_hash(h, tk);
    if (ba->sealed[b]) {
      cur = b;
      continue;
    }
    const int32_t f = find_sealed(ba, h, cur, tk);
    if (f >= 0) { /* the same prefix is cached in another block already */
      cur = f;
      continue;
    }
    seal(ba, b, h, cur, tk);
    cur = b;
  }
  return PKV_OK;
}

int32_t pkv_ba_num_cached(const pkv_ba_t* ba) { return ba ? ba->num_sealed : -1; }

int32_t pkv_ba_num_shared(const pkv_ba_t* ba) { return ba ? ba->num_shared : -1; }
