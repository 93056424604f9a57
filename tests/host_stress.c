/* Seeded stress of libpkv's host code (block allocator, prefix cache, beam
 * reorder, metadata checks), built by gcc under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  No GPU: only the plain-C part of the library is
 * compiled in.
 *
 * A stream of random operations (prompts from a few families of recombining
 * 16-token blocks, decode appends, batch appends, forks, copy-on-write, beam
 * reorders, frees) runs against one pool.  Next to the allocator the driver
 * keeps its own model of what each physical slot holds: a fingerprint of the
 * whole token prefix that the slot's K/V were computed from (the K/V of a
 * token depend on every token before it).  After every operation it checks:
 *   - each block's reference count equals the number of table entries naming
 *     it, and the free count equals the number of blocks nobody names;
 *   - no table names a block twice;
 *   - every slot a live sequence reads holds that sequence's prefix (so a
 *     prefix-cache hit or a copy-on-write never hands over another prefix's
 *     K/V, and no write lands in a block another sequence reads);
 *   - the slot maps, copy pairs and batch metadata it produced pass the host
 *     checks, and planted faults in them do not.
 * Prints "ok <ops>" and exits 0, or prints the failure and exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pkv.h"

#define NB 160   /* blocks in the pool */
#define CAP 40   /* table entries per sequence */
#define MAXS 24  /* sequences alive at once */
#define MAXT (CAP * PKV_BLOCK_SIZE)

typedef struct {
  int live;
  int32_t table[CAP];
  int32_t nblk, len;
  int32_t tok[MAXT];
  uint64_t fp[MAXT]; /* fingerprint of tok[0..i] */
} seq_t;

static seq_t seqs[MAXS];
static uint64_t slot_fp[NB * PKV_BLOCK_SIZE]; /* what each slot holds (0: nothing yet) */
static uint64_t rng_s;
static long ops, hits, cows;

static uint64_t rnd(void) { /* xorshift64* */
  rng_s ^= rng_s >> 12;
  rng_s ^= rng_s << 25;
  rng_s ^= rng_s >> 27;
  return rng_s * 2685821657736338717ULL;
}
static int rn(int n) { return (int)(rnd() % (uint64_t)n); }

static uint64_t fp_next(uint64_t prev, int32_t token) { /* FNV-1a over the prefix */
  uint64_t h = prev ? prev : 1469598103934665603ULL;
  for (int i = 0; i < 4; ++i) {
    h ^= (uint64_t)((uint32_t)token >> (8 * i) & 0xFF);
    h *= 1099511628211ULL;
  }
  return h | 1; /* never 0 */
}

#define FAIL(...)                                           \
  do {                                                      \
    fprintf(stderr, "op %ld: ", ops);                       \
    fprintf(stderr, __VA_ARGS__);                           \
    fprintf(stderr, "\n");                                  \
    exit(1);                                                \
  } while (0)

#define OK(call)                                                         \
  do {                                                                   \
    int rc_ = (call);                                                    \
    if (rc_ != PKV_OK) FAIL("%s returned %d (line %d)", #call, rc_, __LINE__); \
  } while (0)

static void set_tokens(seq_t* s, int from, int to) { /* fingerprints of tok[from..to) */
  for (int i = from; i < to; ++i) s->fp[i] = fp_next(i ? s->fp[i - 1] : 0, s->tok[i]);
}

static void write_slots(const seq_t* s, const int64_t* slots, int first, int n) {
  for (int i = 0; i < n; ++i) {
    if (slots[i] < 0 || slots[i] >= NB * PKV_BLOCK_SIZE) FAIL("slot %lld out of the pool", (long long)slots[i]);
    slot_fp[slots[i]] = s->fp[first + i];
  }
}

static void copy_block(int32_t src, int32_t dst) {
  ++cows;
  memcpy(&slot_fp[dst * PKV_BLOCK_SIZE], &slot_fp[src * PKV_BLOCK_SIZE], sizeof(uint64_t) * PKV_BLOCK_SIZE);
}

static void check_pairs(const int32_t* pairs, int32_t n) {
  int32_t bad;
  OK(pkv_check_copy_pairs(pairs, n, NB, &bad));
  if (n > 0) { /* planted: the first pair copied onto itself */
    int32_t p2[2] = {pairs[0], pairs[0]};
    if (pkv_check_copy_pairs(p2, 1, NB, &bad) != PKV_ERR_INVALID_ARGUMENT || bad != 0)
      FAIL("a self copy passed the pair check");
  }
}

static void check_slots(const int64_t* slots, int32_t n) {
  int32_t bad;
  OK(pkv_check_slot_mapping(slots, n, NB, &bad));
  if (n > 1) { /* planted: the last token repeats the first one's slot */
    int64_t* dup = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
    memcpy(dup, slots, sizeof(int64_t) * (size_t)n);
    dup[n - 1] = dup[0];
    if (pkv_check_slot_mapping(dup, n, NB, &bad) != PKV_ERR_INVALID_ARGUMENT || bad != n - 1)
      FAIL("a shared slot passed the slot check (bad=%d)", bad);
    free(dup);
  }
}

static void check_all(pkv_ba_t* ba) {
  static int32_t users[NB];
  memset(users, 0, sizeof(users));
  int32_t tabs[MAXS * CAP], lens[MAXS], qsl[MAXS + 1];
  int32_t n = 0;
  qsl[0] = 0;
  for (int i = 0; i < MAXS; ++i) {
    seq_t* s = &seqs[i];
    if (!s->live) continue;
    if (s->nblk != (int32_t)pkv_blocks_for_tokens(s->len, PKV_BLOCK_SIZE))
      FAIL("seq %d: %d blocks for %d tokens", i, s->nblk, s->len);
    for (int j = 0; j < s->nblk; ++j) {
      const int32_t b = s->table[j];
      if (b < 0 || b >= NB) FAIL("seq %d: entry %d = %d", i, j, b);
      ++users[b];
      for (int k = 0; k < j; ++k)
        if (s->table[k] == b) FAIL("seq %d names block %d twice", i, b);
    }
    for (int t = 0; t < s->len; ++t) {
      const int64_t slot = (int64_t)s->table[t / PKV_BLOCK_SIZE] * PKV_BLOCK_SIZE + t % PKV_BLOCK_SIZE;
      if (slot_fp[slot] != s->fp[t]) FAIL("seq %d token %d: slot %lld holds another prefix", i, t, (long long)slot);
    }
    if (s->len > 0) {
      memcpy(&tabs[n * CAP], s->table, sizeof(s->table));
      lens[n] = s->len;
      qsl[n + 1] = qsl[n] + 1;
      ++n;
    }
  }
  int32_t free_blocks = 0;
  for (int32_t b = 0; b < NB; ++b) {
    int32_t c;
    OK(pkv_ba_refcount(ba, b, &c));
    if (c != users[b]) FAIL("block %d: count %d, %d users", b, c, users[b]);
    free_blocks += users[b] == 0;
  }
  if (pkv_ba_num_free(ba) != free_blocks) FAIL("%d free, expected %d", pkv_ba_num_free(ba), free_blocks);
  int32_t bad;
  OK(pkv_check_batch(tabs, CAP, lens, qsl, n, n, 1, MAXT, NB, &bad));
  if (n > 0) { /* planted: a table entry past the pool */
    const int32_t keep = tabs[0];
    tabs[0] = NB;
    if (pkv_check_batch(tabs, CAP, lens, qsl, n, n, 1, MAXT, NB, &bad) != PKV_ERR_INVALID_ARGUMENT || bad != 0)
      FAIL("a table entry past the pool passed the batch check");
    tabs[0] = keep;
  }
}

static int free_slot(void) {
  for (int i = 0; i < MAXS; ++i)
    if (!seqs[i].live) return i;
  return -1;
}
static int live_slot(void) {
  int idx[MAXS], n = 0;
  for (int i = 0; i < MAXS; ++i)
    if (seqs[i].live) idx[n++] = i;
  return n ? idx[rn(n)] : -1;
}

static void release(pkv_ba_t* ba, int i) {
  OK(pkv_seq_free(ba, seqs[i].table, seqs[i].nblk));
  seqs[i].live = 0;
}

/* append n tokens (already in tok[len..len+n)) through the allocator; 0 if out of blocks */
static int append(pkv_ba_t* ba, seq_t* s, int n) {
  int64_t slots[MAXT];
  int32_t pair[2], ncow;
  int32_t nblk = s->nblk, len = s->len;
  const int rc = pkv_seq_append_slots(ba, s->table, CAP, &nblk, &len, n, slots, pair, &ncow);
  if (rc == PKV_ERR_OUT_OF_BLOCKS) return 0;
  OK(rc);
  if (ncow) {
    check_pairs(pair, 1);
    copy_block(pair[0], pair[1]);
  }
  check_slots(slots, n);
  set_tokens(s, s->len, s->len + n);
  write_slots(s, slots, s->len, n);
  s->nblk = nblk;
  s->len = len;
  return 1;
}

static void op_prompt(pkv_ba_t* ba) {
  const int i = free_slot();
  if (i < 0) return;
  seq_t* s = &seqs[i];
  const int nb = 1 + rn(CAP / 2);
  const int n = (nb - 1) * PKV_BLOCK_SIZE + 1 + rn(PKV_BLOCK_SIZE);
  const int fam = rn(3);
  for (int j = 0; j < nb; ++j) { /* blocks drawn from a small alphabet: prefixes recombine */
    const int pick = fam == 0 ? j % 4 : fam == 1 ? rn(3) : (j < 2 ? rn(2) : 7 + rn(2));
    for (int t = 0; t < PKV_BLOCK_SIZE && j * PKV_BLOCK_SIZE + t < n; ++t)
      s->tok[j * PKV_BLOCK_SIZE + t] = pick * 100 + t;
  }
  set_tokens(s, 0, n);
  OK(pkv_seq_cache_lookup(ba, s->tok, n, s->table, CAP, &s->nblk));
  hits += s->nblk;
  s->len = s->nblk * PKV_BLOCK_SIZE;
  s->live = 1;
  for (int t = 0; t < s->len; ++t) { /* a hit must hold exactly this prompt's prefix */
    const int64_t slot = (int64_t)s->table[t / PKV_BLOCK_SIZE] * PKV_BLOCK_SIZE + t % PKV_BLOCK_SIZE;
    if (slot_fp[slot] != s->fp[t]) FAIL("cache hit on block %d holds another prefix", s->table[t / PKV_BLOCK_SIZE]);
  }
  if (n > s->len && !append(ba, s, n - s->len)) {
    release(ba, i);
    return;
  }
  OK(pkv_seq_cache_seal(ba, s->tok, s->len, s->table, s->nblk));
}

static void op_decode(pkv_ba_t* ba) {
  const int i = live_slot();
  if (i < 0) return;
  seq_t* s = &seqs[i];
  int n = 1 + rn(20);
  if (s->len + n > MAXT) n = MAXT - s->len;
  if (n <= 0) {
    release(ba, i);
    return;
  }
  for (int t = 0; t < n; ++t) s->tok[s->len + t] = 5000 + rn(50);
  if (!append(ba, s, n)) return;
  if (rn(3) == 0) OK(pkv_seq_cache_seal(ba, s->tok, s->len, s->table, s->nblk));
}

static void op_fork(pkv_ba_t* ba) {
  const int i = live_slot(), k = free_slot();
  if (i < 0 || k < 0) return;
  OK(pkv_seq_fork(ba, seqs[i].table, seqs[i].nblk, seqs[k].table));
  seqs[k].nblk = seqs[i].nblk;
  seqs[k].len = seqs[i].len;
  memcpy(seqs[k].tok, seqs[i].tok, sizeof(int32_t) * (size_t)seqs[i].len);
  memcpy(seqs[k].fp, seqs[i].fp, sizeof(uint64_t) * (size_t)seqs[i].len);
  seqs[k].live = 1;
}

static void op_make_writable(pkv_ba_t* ba) {
  const int i = live_slot();
  if (i < 0 || seqs[i].nblk == 0) return;
  seq_t* s = &seqs[i];
  int32_t pair[2], ncow;
  const int rc = pkv_seq_make_writable(ba, s->table, s->nblk, rn(s->nblk), pair, &ncow);
  if (rc == PKV_ERR_OUT_OF_BLOCKS) return;
  OK(rc);
  if (ncow) {
    check_pairs(pair, 1);
    copy_block(pair[0], pair[1]);
  }
}

static void op_batch(pkv_ba_t* ba) {
  int idx[MAXS], n = 0;
  for (int i = 0; i < MAXS; ++i)
    if (seqs[i].live && seqs[i].len + 2 <= MAXT) idx[n++] = i;
  if (!n) return;
  static int32_t tabs[MAXS * CAP];
  int32_t nblk[MAXS], lens[MAXS], nnew[MAXS], pairs[2 * MAXS], ncow, ndone;
  int64_t slots[2 * MAXS];
  int total = 0;
  for (int k = 0; k < n; ++k) {
    seq_t* s = &seqs[idx[k]];
    memcpy(&tabs[k * CAP], s->table, sizeof(s->table));
    nblk[k] = s->nblk;
    lens[k] = s->len;
    nnew[k] = 1 + rn(2);
    for (int t = 0; t < nnew[k]; ++t) s->tok[s->len + t] = 9000 + rn(9);
    total += nnew[k];
  }
  const int rc = pkv_batch_append_slots(ba, tabs, CAP, nblk, lens, nnew, n, slots, pairs, &ncow, &ndone);
  if (rc != PKV_OK && rc != PKV_ERR_OUT_OF_BLOCKS) FAIL("batch append returned %d", rc);
  if (rc == PKV_OK && ndone != n) FAIL("batch append did %d of %d", ndone, n);
  check_pairs(pairs, ncow);
  for (int c = 0; c < ncow; ++c) copy_block(pairs[2 * c], pairs[2 * c + 1]);
  int off = 0;
  for (int k = 0; k < ndone; ++k) {
    seq_t* s = &seqs[idx[k]];
    set_tokens(s, s->len, s->len + nnew[k]);
    write_slots(s, slots + off, s->len, nnew[k]);
    off += nnew[k];
    memcpy(s->table, &tabs[k * CAP], sizeof(s->table));
    s->nblk = nblk[k];
    s->len = lens[k];
  }
  check_slots(slots, off);
  (void)total;
}

static void op_reorder(pkv_ba_t* ba) {
  int idx[MAXS], n = 0;
  for (int i = 0; i < MAXS; ++i)
    if (seqs[i].live) idx[n++] = i;
  if (n < 2) return;
  static int32_t tabs[MAXS * CAP], work[MAXS * CAP];
  static seq_t old[MAXS];
  int32_t nblk[MAXS], lens[MAXS], parents[MAXS];
  for (int k = 0; k < n; ++k) {
    old[k] = seqs[idx[k]];
    memcpy(&tabs[k * CAP], old[k].table, sizeof(old[k].table));
    nblk[k] = old[k].nblk;
    lens[k] = old[k].len;
    parents[k] = rn(3) ? rn(n) : k;
  }
  OK(pkv_seq_reorder(ba, tabs, CAP, nblk, lens, n, parents, work));
  for (int k = 0; k < n; ++k) {
    seq_t* s = &seqs[idx[k]];
    *s = old[parents[k]];
    if (memcmp(s->table, &tabs[k * CAP], sizeof(int32_t) * (size_t)nblk[k]) || s->nblk != nblk[k] ||
        s->len != lens[k])
      FAIL("row %d is not a copy of row %d", k, parents[k]);
  }
}

static void op_errors(pkv_ba_t* ba) {
  /* argument errors change nothing */
  int32_t c, t[2] = {0, NB};
  if (pkv_ba_refcount(ba, NB, &c) != PKV_ERR_INVALID_ARGUMENT) FAIL("refcount of block NB");
  if (pkv_seq_free(ba, t, 2) == PKV_OK) FAIL("free of a table naming block NB");
  for (int32_t b = 0; b < NB; ++b) {
    OK(pkv_ba_refcount(ba, b, &c));
    if (c == 0) {
      if (pkv_ba_decref(ba, b) != PKV_ERR_REFCOUNT) FAIL("decref of free block %d", b);
      break;
    }
  }
}

int main(int argc, char** argv) {
  const unsigned long seed = argc > 1 ? strtoul(argv[1], NULL, 10) : 1;
  const long n_ops = argc > 2 ? strtol(argv[2], NULL, 10) : 4000;
  rng_s = 0x9E3779B97F4A7C15ULL ^ (seed * 0xD1B54A32D192ED03ULL);
  if (!rng_s) rng_s = 1;
  int32_t order[NB];
  for (int i = 0; i < NB; ++i) order[i] = i;
  for (int i = NB - 1; i > 0; --i) { /* seeded free order */
    const int j = rn(i + 1), x = order[i];
    order[i] = order[j];
    order[j] = x;
  }
  pkv_ba_t* ba = NULL;
  OK(pkv_ba_create(NB, PKV_BLOCK_SIZE, order, &ba));
  for (ops = 0; ops < n_ops; ++ops) {
    const int r = rn(100);
    if (r < 25) op_prompt(ba);
    else if (r < 50) op_decode(ba);
    else if (r < 58) op_fork(ba);
    else if (r < 64) op_make_writable(ba);
    else if (r < 76) op_batch(ba);
    else if (r < 82) op_reorder(ba);
    else if (r < 84) op_errors(ba);
    else {
      const int i = live_slot();
      if (i >= 0) release(ba, i);
    }
    check_all(ba);
  }
  for (int i = 0; i < MAXS; ++i)
    if (seqs[i].live) release(ba, i);
  check_all(ba);
  if (pkv_ba_num_free(ba) != NB) FAIL("%d of %d blocks free at the end", pkv_ba_num_free(ba), NB);
  pkv_ba_destroy(ba);
  printf("ok ops=%ld hits=%ld cows=%ld\n", ops, hits, cows);
  return 0;
}
