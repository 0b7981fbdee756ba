/* Host-side validation of the C ABI under AddressSanitizer.
 *
 * Linked against a host-only build of the library (no device code, so nothing
 * here can launch a kernel or touch a GPU), instrumented with
 * -fsanitize=address.  Every call below must be answered on the host: sizes
 * for valid configurations, and for invalid arguments the documented status
 * with a message from llama_last_error.  ASan aborts the run on any heap,
 * stack or global overrun in that host code.  Prints one summary line and
 * exits 0 when every check holds. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "llama_block.h"

static int n_checks = 0, n_failed = 0;

static void check(int ok, const char* what) {
  ++n_checks;
  if (!ok) {
    ++n_failed;
    fprintf(stderr, "FAILED: %s (last error: %s)\n", what, llama_last_error());
  }
}

/* a refused call: the expected status and a non-empty message */
static void refused(llama_status st, llama_status want, const char* what) {
  check(st == want && strlen(llama_last_error()) > 0, what);
}

static llama_block_config base_cfg(void) {
  llama_block_config c;
  memset(&c, 0, sizeof c);
  c.dim = 4096;
  c.n_heads = 32;
  c.n_kv_heads = 32;
  c.ffn_dim = 11008;
  c.norm_eps = 1e-5f;
  c.rope_theta = 1e4f;
  c.act_dtype = LLAMA_BF16;
  c.weight_format = LLAMA_W_DENSE;
  c.group_size = 64;
  c.max_seq = 4097;
  return c;
}

static llama_kvcache_config base_kv(void) {
  llama_kvcache_config k;
  k.n_layers = 1;
  k.max_batch = 16;
  k.max_seq = 4160;
  k.n_kv_heads = 32;
  k.head_dim = 128;
  k.page_size = 64;
  k.dtype = LLAMA_BF16;
  return k;
}

int main(void) {
  /* ---- valid configurations: weight, scratch and cache sizes */
  llama_block_config good[5];
  good[0] = base_cfg();                                    /* 7B-shaped */
  good[1] = base_cfg();                                    /* 13B-shaped */
  good[1].dim = 5120, good[1].n_heads = 40, good[1].n_kv_heads = 40, good[1].ffn_dim = 13824;
  good[2] = base_cfg();                                    /* 70B-shaped, grouped heads */
  good[2].dim = 8192, good[2].n_heads = 64, good[2].n_kv_heads = 8, good[2].ffn_dim = 28672;
  good[3] = good[1];                                       /* 4-bit weights */
  good[3].weight_format = LLAMA_W_Q4;
  good[4] = base_cfg();                                    /* tiny fp32, sliding window */
  good[4].dim = 256, good[4].n_heads = 4, good[4].n_kv_heads = 2, good[4].ffn_dim = 688;
  good[4].act_dtype = LLAMA_F32, good[4].sliding_window = 37;
  for (int i = 0; i < 5; ++i) {
    check(llama_block_weight_bytes(&good[i]) > 0, "weight bytes of a valid config");
    const int tok[4] = {1, 97, 2048, 4096}, bat[4] = {1, 3, 16, 64};
    for (int t = 0; t < 4; ++t)
      for (int b = 0; b < 4; ++b)
        check(llama_scratch_bytes(&good[i], tok[t], bat[b], 4160) > 0, "scratch bytes of a valid call shape");
  }
  check(llama_scratch_bytes(&good[0], 4096, 16, 4160) >= llama_scratch_bytes(&good[0], 64, 16, 4160),
        "scratch grows with the token count");
  llama_block_config big = good[2];
  big.max_seq = 131072;
  check(llama_block_weight_bytes(&big) > llama_block_weight_bytes(&good[2]), "a longer rotation table");
  llama_kvcache_config kv = base_kv();
  check(llama_kvcache_bytes(&kv) >= (size_t)2 * 16 * 4160 * 32 * 128 * 2, "cache holds K and V");
  check(llama_head_scratch_bytes(4, 5120, 32000) > 0, "head scratch");

  /* ---- invalid configurations: 0 bytes, and create refuses them */
  llama_block_config bad[9];
  for (int i = 0; i < 9; ++i) bad[i] = base_cfg();
  bad[0].n_kv_heads = 5;                 /* heads not a multiple of kv heads */
  bad[1].sliding_window = -1;
  bad[2].dim = 4000;                     /* dim not a multiple of heads */
  bad[3].norm_eps = 0.0f;
  bad[4].rope_theta = 0.0f;
  bad[5].act_dtype = 7;
  bad[6].weight_format = 3;
  bad[7].max_seq = 0;
  bad[8].dim = -4096;
  llama_block* blk = NULL;
  llama_block_weights w;
  memset(&w, 0, sizeof w);
  for (int i = 0; i < 9; ++i) {
    check(llama_block_weight_bytes(&bad[i]) == 0, "weight bytes of an invalid config");
    check(llama_scratch_bytes(&bad[i], 64, 1, 128) == 0, "scratch bytes of an invalid config");
    refused(llama_block_create(&bad[i], &w, NULL, 0, NULL, &blk), LLAMA_ERR_INVALID_ARG, "create, invalid config");
  }
  llama_block_config uns = base_cfg();
  uns.dim = 3072;                        /* head_dim 96 in bf16 */
  refused(llama_block_create(&uns, &w, NULL, 0, NULL, &blk), LLAMA_ERR_UNSUPPORTED, "create, head_dim 96");
  refused(llama_block_create(NULL, &w, NULL, 0, NULL, &blk), LLAMA_ERR_INVALID_ARG, "create, NULL config");
  check(blk == NULL, "no handle from a refused create");

  /* ---- cache configurations */
  llama_kvcache* cache = NULL;
  llama_kvcache_config kb = base_kv();
  kb.page_size = 48;                     /* not a multiple of 64 */
  check(llama_kvcache_bytes(&kb) == 0, "cache bytes, page size 48");
  refused(llama_kvcache_alloc(&kb, NULL, 0, NULL, &cache), LLAMA_ERR_UNSUPPORTED, "cache alloc, page size 48");
  kb = base_kv();
  kb.n_layers = 0;
  refused(llama_kvcache_alloc(&kb, NULL, 0, NULL, &cache), LLAMA_ERR_INVALID_ARG, "cache alloc, no layers");
  refused(llama_kvcache_alloc(NULL, NULL, 0, NULL, &cache), LLAMA_ERR_INVALID_ARG, "cache alloc, NULL config");
  int32_t lens[4] = {0, 0, 0, 0};
  refused(llama_kvcache_set_lens(NULL, 0, lens, 4, NULL), LLAMA_ERR_INVALID_ARG, "set lens, NULL cache");
  refused(llama_kvcache_get_lens(NULL, 0, lens, 4), LLAMA_ERR_INVALID_ARG, "get lens, NULL cache");
  refused(llama_kvcache_set_block_table(NULL, lens, NULL), LLAMA_ERR_INVALID_ARG, "block table, NULL cache");

  /* ---- block calls with missing handles or buffers */
  char buf[256];
  refused(llama_block_prefill(NULL, NULL, 0, buf, buf, 1, 8, buf, sizeof buf, NULL), LLAMA_ERR_INVALID_ARG,
          "prefill, NULL block");
  const int32_t seq_lens[2] = {3, 0};
  refused(llama_block_prefill_ragged(NULL, NULL, 0, buf, buf, 2, seq_lens, buf, sizeof buf, NULL),
          LLAMA_ERR_INVALID_ARG, "ragged prefill, NULL block");
  refused(llama_block_decode(NULL, NULL, 0, buf, buf, 1, buf, sizeof buf, NULL), LLAMA_ERR_INVALID_ARG,
          "decode, NULL block");
  refused(llama_block_decode_noalloc(NULL, NULL, 0, buf, buf, 1, NULL), LLAMA_ERR_INVALID_ARG,
          "no-allocation decode, NULL block");
  refused(llama_block_set_diag(NULL, 1), LLAMA_ERR_INVALID_ARG, "diag, NULL block");
  refused(llama_block_profile_start(NULL, 4, 0xffu), LLAMA_ERR_INVALID_ARG, "profile, NULL block");

  /* ---- stack ends */
  refused(llama_embed(NULL, 32000, 4096, LLAMA_BF16, (const int32_t*)buf, 4, buf, NULL), LLAMA_ERR_INVALID_ARG,
          "embed, NULL table");
  refused(llama_embed(buf, 0, 4096, LLAMA_BF16, (const int32_t*)buf, 4, buf, NULL), LLAMA_ERR_INVALID_ARG,
          "embed, empty vocabulary");
  llama_linear head;
  memset(&head, 0, sizeof head);
  refused(llama_lm_head_argmax(&head, LLAMA_W_DENSE, 64, LLAMA_BF16, buf, 1e-5f, buf, 1, 4096, 32000, NULL,
                               (int32_t*)buf, buf, sizeof buf, NULL),
          LLAMA_ERR_INVALID_ARG, "head, NULL weight");
  const float* lg = (const float*)buf;
  refused(llama_sample(NULL, 1, 32000, 0.8f, 0.9f, lg, (int32_t*)buf, NULL), LLAMA_ERR_INVALID_ARG,
          "sample, NULL logits");
  refused(llama_sample(lg, 1, 32000, NAN, 0.9f, lg, (int32_t*)buf, NULL), LLAMA_ERR_INVALID_ARG,
          "sample, NaN temperature");
  refused(llama_sample(lg, 1, 32000, 0.8f, 1.5f, lg, (int32_t*)buf, NULL), LLAMA_ERR_INVALID_ARG,
          "sample, top_p above 1");
  refused(llama_sample(lg, 0, 32000, 0.8f, 0.9f, lg, (int32_t*)buf, NULL), LLAMA_ERR_INVALID_ARG,
          "sample, no rows");
  llama_stack* st = NULL;
  refused(llama_stack_create(NULL, 40, buf, 32000, buf, &head, &st), LLAMA_ERR_INVALID_ARG,
          "stack, NULL blocks");
  refused(llama_stack_set_sampling(NULL, 0.8f, 0.9f, lg), LLAMA_ERR_INVALID_ARG, "sampling, NULL stack");
  check(llama_stack_scratch_bytes(NULL, 512, 640) == 0, "stack scratch, NULL stack");
  llama_block_destroy(NULL);
  llama_kvcache_free(NULL);
  llama_stack_destroy(NULL);

  printf("ABI host checks: %d of %d passed\n", n_checks - n_failed, n_checks);
  return n_failed == 0 ? 0 : 1;
}
