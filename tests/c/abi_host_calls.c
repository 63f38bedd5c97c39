/* A plain C99 caller of the library's host entry points: builds against
 * include/lazy_attn.h and links liblazyattn.so with no C++ or Python in
 * between.  No device is needed (only host-side entry points are called). */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lazy_attn.h"

static int fails = 0;
#define CHECK(cond, ...)          \
  do {                            \
    if (!(cond)) {                \
      printf("FAIL: " __VA_ARGS__); \
      printf("\n");               \
      ++fails;                    \
    }                             \
  } while (0)

int main(void) {
  la_params p;
  memset(&p, 0, sizeof p);
  p.num_q_heads = 8;
  p.num_kv_heads = 2;
  p.head_dim = 128;
  p.block_size = 16;
  p.num_blocks = 10;
  p.dtype = LA_BF16;
  p.scale = 0.088f;
  p.max_pos = 256;

  /* cos/sin table: row 0 is (cos 0, sin 0) = (1, 0) */
  float* table = (float*)malloc(sizeof(float) * 256 * 128);
  CHECK(lazy_attn_rope_table(1e4, 128, 256, table) == LA_OK, "rope_table");
  CHECK(table[0] == 1.0f && table[64] == 0.0f, "rope_table row 0");

  /* two requests share document blocks {1, 2} (20 tokens) at offsets 0 and 40 */
  int64_t req_seg_start[3] = {0, 1, 3};
  int64_t seg_start[3] = {0, 40, 0};
  int64_t seg_len[3] = {20, 20, 16};
  uint8_t seg_new[3] = {0, 0, 0};
  int64_t seg_blk_start[4] = {0, 2, 4, 5};
  int64_t seg_blocks[5] = {1, 2, 1, 2, 7};
  req_seg_start[2] = 3;
  uint64_t words[8];
  int32_t rbs[3], maxb = 0;
  la_status st = lazy_attn_pack_segments(&p, 2, req_seg_start, seg_start, seg_len, seg_new,
                                         seg_blk_start, seg_blocks, words, 8, rbs, &maxb);
  CHECK(st == LA_OK, "pack_segments: %s", lazy_attn_last_error());
  CHECK(rbs[0] == 0 && rbs[1] == 2 && rbs[2] == 5 && maxb == 3, "pack_segments rows");
  CHECK((words[0] & 0xFFFFFFFFu) == 1 && ((words[3] >> 32) & 0xFFFFFFu) == 56,
        "pack_segments words");

  int32_t q_pos[2] = {20, 60};
  st = lazy_attn_validate_table(&p, 2, words, rbs, q_pos, NULL, maxb, 0);
  CHECK(st == LA_OK, "validate_table: %s", lazy_attn_last_error());
  words[1] = (words[1] & ~(uint64_t)0xFFFFFFFFu) | 10u; /* block id == num_blocks */
  st = lazy_attn_validate_table(&p, 2, words, rbs, q_pos, NULL, maxb, 0);
  CHECK(st == LA_ERR_INVALID_ARG, "validate_table accepted a bad block id");
  CHECK(strstr(lazy_attn_last_error(), "block id") != NULL, "error text: %s",
        lazy_attn_last_error());
  CHECK(strcmp(lazy_attn_status_string(LA_ERR_INVALID_ARG), "INVALID_ARG") == 0 ||
            strstr(lazy_attn_status_string(LA_ERR_INVALID_ARG), "INVALID") != NULL,
        "status_string");

  /* shared-decode plan: sizes first, then the blob */
  la_shared_plan_info info;
  st = lazy_attn_plan_shared_decode(&p, 2, req_seg_start, seg_start, seg_len, seg_new,
                                    seg_blk_start, seg_blocks, 0, &info, NULL, 0);
  CHECK(st == LA_OK, "plan sizes: %s", lazy_attn_last_error());
  /* the shared document is one item with two members; request 1's private
     block is its own run */
  CHECK(info.n_items == 2 && info.n_members == 3 && info.n_words == 3,
        "plan sizes %d items %d members %d words", info.n_items, info.n_members, info.n_words);
  void* blob = malloc((size_t)info.plan_bytes);
  st = lazy_attn_plan_shared_decode(&p, 2, req_seg_start, seg_start, seg_len, seg_new,
                                    seg_blk_start, seg_blocks, 0, &info, blob, info.plan_bytes);
  CHECK(st == LA_OK, "plan blob: %s", lazy_attn_last_error());

  size_t ws = 0;
  CHECK(lazy_attn_decode_workspace_size(&p, 2, maxb, &ws) == LA_OK, "workspace_size");

  /* cache simulator: a trace of one document at two positions hits once when
     the cache is position-agnostic, never when it keys on the position */
  int64_t docs[2] = {5, 5};
  int32_t pos[2] = {0, 1};
  int64_t hits = -1;
  CHECK(lazy_attn_cache_simulate(2, docs, pos, 2, 4, LA_CACHE_POSITION_AGNOSTIC, LA_EVICT_LRU,
                                 &hits) == LA_OK && hits == 1, "agnostic hits %lld", (long long)hits);
  CHECK(lazy_attn_cache_simulate(2, docs, pos, 2, 4, LA_CACHE_POSITION_AWARE, LA_EVICT_LRU,
                                 &hits) == LA_OK && hits == 0, "aware hits %lld", (long long)hits);

  free(blob);
  free(table);
  printf(fails ? "FAILED %d\n" : "OK\n", fails);
  return fails ? 1 : 0;
}
