/* Host checks of the metadata the kernels trust (plain C, no GPU use).
 *
 * The block scheme rests on a few rules: a token's slot names one position of
 * one block of the pool and no two tokens of a write share it; a copy-on-write
 * pair copies a shared block into a different, private one
 * (blog.mckayzhao.com/?p=56, copy-on-write section); a block table maps every
 * logical block of a sequence to a physical block of the pool
 * (devpress.csdn.net/amd/6a408ab810ee7a33f2834f35.html, core idea).  The
 * kernels do not check these on the device (beyond skipping ids outside the
 * pool); these functions check them on host copies of the metadata.
 */
#include <stdlib.h>

#include "pkv.h"

static void set_bad(int32_t* bad, int32_t i) {
  if (bad) *bad = i;
}

typedef struct {
  int64_t slot;
  int32_t token;
} slot_use;

static int cmp_use(const void* a, const void* b) {  // by slot, then token
  const slot_use *x = (const slot_use*)a, *y = (const slot_use*)b;
  if (x->slot != y->slot) return (x->slot > y->slot) - (x->slot < y->slot);
  return (x->token > y->token) - (x->token < y->token);
}

static int cmp_i32(const void* a, const void* b) {
  const int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

int pkv_check_slot_mapping(const int64_t* slots, int32_t num_tokens, int32_t num_blocks,
                           int32_t* bad) {
  set_bad(bad, -1);
  if (num_tokens < 0 || num_blocks < 0 || (num_tokens > 0 && !slots))
    return PKV_ERR_INVALID_ARGUMENT;
  const int64_t cap = (int64_t)num_blocks * PKV_BLOCK_SIZE;
  slot_use* use = (slot_use*)malloc(sizeof(slot_use) * (size_t)(num_tokens > 0 ? num_tokens : 1));
  if (!use) return PKV_ERR_INVALID_ARGUMENT;
  int32_t n = 0, first = -1;  // first: the earliest token that breaks a rule
  for (int32_t i = 0; i < num_tokens; ++i) {
    if (slots[i] < 0) continue;  // padding token
    if (slots[i] >= cap) {
      if (first < 0) first = i;
      continue;
    }
    use[n].slot = slots[i];
    use[n++].token = i;
  }
  qsort(use, (size_t)n, sizeof(slot_use), cmp_use);
  for (int32_t k = 1; k < n; ++k)  // the later tokens of a shared slot
    if (use[k].slot == use[k - 1].slot && (first < 0 || use[k].token < first)) first = use[k].token;
  free(use);
  if (first < 0) return PKV_OK;
  set_bad(bad, first);
  return PKV_ERR_INVALID_ARGUMENT;
}

int pkv_check_copy_pairs(const int32_t* pairs, int32_t num_pairs, int32_t num_blocks,
                         int32_t* bad) {
  set_bad(bad, -1);
  if (num_pairs < 0 || num_blocks < 0 || (num_pairs > 0 && !pairs)) return PKV_ERR_INVALID_ARGUMENT;
  int32_t first = -1;  // the earliest pair that breaks a rule
  for (int32_t p = 0; p < num_pairs && first < 0; ++p) {
    const int32_t s = pairs[2 * p], d = pairs[2 * p + 1];
    if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks || s == d) first = p;
  }
  size_t n = (size_t)(num_pairs > 0 ? num_pairs : 1);
  slot_use* use = (slot_use*)malloc(sizeof(slot_use) * n);  // (dst, pair)
  int32_t* dst = (int32_t*)malloc(sizeof(int32_t) * n);
  if (!use || !dst) {
    free(use);
    free(dst);
    return PKV_ERR_INVALID_ARGUMENT;
  }
  for (int32_t p = 0; p < num_pairs; ++p) {
    use[p].slot = pairs[2 * p + 1];
    use[p].token = p;
    dst[p] = pairs[2 * p + 1];
  }
  qsort(use, (size_t)num_pairs, sizeof(slot_use), cmp_use);
  qsort(dst, (size_t)num_pairs, sizeof(int32_t), cmp_i32);
  for (int32_t k = 1; k < num_pairs; ++k)  // the later pairs naming a dst named before
    if (use[k].slot == use[k - 1].slot && (first < 0 || use[k].token < first)) first = use[k].token;
  // a dst that is also some pair's src (the copy order would then matter)
  for (int32_t p = 0; p < num_pairs && (first < 0 || p < first); ++p)
    if (bsearch(&pairs[2 * p], dst, (size_t)num_pairs, sizeof(int32_t), cmp_i32)) first = p;
  free(use);
  free(dst);
  if (first < 0) return PKV_OK;
  set_bad(bad, first);
  return PKV_ERR_INVALID_ARGUMENT;
}

int pkv_check_batch(const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
                    const int32_t* query_start_loc, int32_t num_seqs, int32_t num_q_tokens,
                    int32_t max_q_len, int32_t max_seq_len, int32_t num_blocks, int32_t* bad) {
  set_bad(bad, -1);
  if (num_seqs < 0 || num_q_tokens < 0 || bt_stride < 0 || num_blocks < 0 ||
      (num_seqs > 0 && (!block_tables || !seq_lens || !query_start_loc)))
    return PKV_ERR_INVALID_ARGUMENT;
  if (num_seqs > 0 && (query_start_loc[0] < 0 || query_start_loc[num_seqs] > num_q_tokens))
    return PKV_ERR_INVALID_ARGUMENT;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t q_len = query_start_loc[s + 1] - query_start_loc[s];
    const int32_t len = seq_lens[s];
    const int64_t nblk = pkv_blocks_for_tokens(len < 0 ? 0 : len, PKV_BLOCK_SIZE);
    int ok = q_len >= 1 && q_len <= max_q_len && len >= 0 && len <= max_seq_len &&
             (len == 0 || q_len <= len) && nblk <= bt_stride;
    for (int64_t j = 0; ok && j < nblk; ++j) {
      const int32_t b = block_tables[(int64_t)s * bt_stride + j];
      ok = b >= 0 && b < num_blocks;
    }
    if (!ok) {
      set_bad(bad, s);
      return PKV_ERR_INVALID_ARGUMENT;
    }
  }
  return PKV_OK;
}
