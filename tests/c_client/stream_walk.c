/* A plain C client of libswattn (no Python, no torch): walks a 540p-shaped stream of
 * 1000 chunks through a metadata-only cache and checks, after every commit, the slot
 * table against the closed form of the bounded cache ("Vidu S2 vs PixVerse R2" blog,
 * section "Choice 3: bounded memory": the first S blocks are permanent sinks, a
 * window keeps the W most recent blocks, older ones are dropped) and the S1 time
 * bases (slot l starts at l * F).  Also checks a few error paths.  Exit status 0 on
 * success; the first mismatch is printed. */
#include <stdio.h>
#include <string.h>

#include "swattn.h"

#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      fprintf(stderr, __VA_ARGS__);           \
      fprintf(stderr, " [%s]\n", sw_last_error()); \
      return 1;                               \
    }                                         \
  } while (0)

int main(void) {
  sw_cache_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.n_heads = 24;
  cfg.head_dim = 128;
  cfg.frames_per_block = 3;
  cfg.lat_h = 34;
  cfg.lat_w = 60;
  cfg.n_sink = 1;
  cfg.n_window = 3;
  cfg.dtype = SW_BF16;
  cfg.rope_theta = 10000.0;
  cfg.policy = SW_ROPE_S1_RELOCATE;
  cfg.tile = 128;

  size_t bytes = 0;
  CHECK(sw_cache_required_bytes(&cfg, &bytes) == SW_OK && bytes > 0, "required_bytes failed");
  sw_cache* c = NULL;
  CHECK(sw_cache_create(&cfg, NULL, 0, NULL, &c) == SW_OK, "create failed");
  CHECK(sw_cache_evict(c) == SW_ERR_STATE, "evict on an empty window must fail");

  static char dummy[16]; /* metadata-only: pointers are only checked for NULL */
  const int S = cfg.n_sink, W = cfg.n_window, F = cfg.frames_per_block;
  for (int64_t n = 0; n < 1000; ++n) {
    CHECK(sw_cache_append_block(c, SW_KV_CURRENT, dummy, dummy, n) == SW_OK, "stage %lld", (long long)n);
    const int n_sink = n < S ? (int)n : S;
    const int n_win = n - S > 0 ? (n - S < W ? (int)(n - S) : W) : 0;
    sw_slot_info info[16];
    int32_t cnt = 0;
    CHECK(sw_cache_inspect(c, info, 16, &cnt) == SW_OK, "inspect");
    CHECK(cnt == n_sink + n_win + 1, "chunk %lld: %d slots, expected %d", (long long)n, cnt, n_sink + n_win + 1);
    for (int l = 0; l < cnt; ++l) {
      const int64_t want_block = l < n_sink ? l : (l < n_sink + n_win ? n - n_win + (l - n_sink) : n);
      const int want_role = l < n_sink ? 0 : (l < n_sink + n_win ? 1 : 2);
      CHECK(info[l].block_id == want_block && info[l].role == want_role && info[l].time_base == l * F,
            "chunk %lld slot %d: block %lld role %d base %d", (long long)n, l, (long long)info[l].block_id,
            info[l].role, info[l].time_base);
    }
    if (n >= S && n_win == W) {
      CHECK(sw_cache_append_block(c, SW_KV_CLEAN, NULL, NULL, n) == SW_ERR_CAPACITY,
            "commit into a full window must fail");
      CHECK(sw_cache_evict(c) == SW_OK, "evict at chunk %lld", (long long)n);
    }
    CHECK(sw_cache_append_block(c, SW_KV_CLEAN, NULL, NULL, n) == SW_OK, "commit %lld", (long long)n);
    CHECK(sw_cache_append_block(c, SW_KV_CLEAN, NULL, NULL, n) == SW_ERR_STATE, "double commit must fail");
  }
  CHECK(sw_chunk_attend(c, dummy, SW_STEP_FINAL, NULL, 0, dummy, NULL) == SW_ERR_STATE,
        "a metadata-only cache cannot launch");
  CHECK(sw_cache_destroy(c) == SW_OK, "destroy");
  printf("c client: 1000 chunks ok\n");
  return 0;
}
