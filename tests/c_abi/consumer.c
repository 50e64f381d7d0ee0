/* A plain C consumer of libkpool.so: the header compiles as ISO C11 with
 * every warning an error, and the library answers its host-only entry
 * points (version, sizes, status strings, argument validation) without a
 * GPU. Prints one line per check; exits non-zero on the first failure.
 * Built and run by tests/test_c_abi.py. */
#include <stdio.h>
#include <string.h>

#include "kpool.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);       \
      return 1;                                                       \
    }                                                                 \
    printf("ok: %s\n", #cond);                                        \
  } while (0)

int main(void) {
  kpool_params p;
  static _Alignas(256) char fake[256];
  size_t ws;
  memset(&p, 0, sizeof p);
  p.num_docs = 1;
  p.total_tokens = 65536;
  p.max_seqlen = 65536;
  p.num_heads = 32;
  p.head_dim = 128;
  p.kpool = 4;
  p.index_topk = 2048;
  p.always_select_tail = 1;
  p.query_chunk = 4096;

  CHECK(kpool_abi_version() == KPOOL_ABI_VERSION);
  CHECK(kpool_logits_ld(&p) == 16384);
  CHECK(kpool_query_chunk_rows(&p) == 4096);
  ws = kpool_workspace_bytes(&p);
  CHECK(ws >= (size_t)4096 * 16384 * 4);
  CHECK(kpool_fused_max_ksel(&p) == 1184);
  CHECK(kpool_fused_workspace_bytes(&p) == 0); /* no logits tile */
  CHECK(kpool_decode_noalloc_max_bytes() == ((size_t)32 << 20));
  CHECK(strcmp(kpool_status_string(KPOOL_OK), "ok") == 0);
  CHECK(strcmp(kpool_status_string(KPOOL_E_WORKSPACE), "workspace too small") == 0);

  /* validation happens before any launch: these calls touch no device */
  CHECK(kpool_indexer_topk(NULL, fake, (const float*)fake, fake, (const int32_t*)fake,
                           (const int32_t*)fake, fake, ws, (int32_t*)fake, NULL, NULL) ==
        KPOOL_E_INVALID);
  CHECK(strlen(kpool_last_error()) > 0);
  p.num_heads = 48;
  CHECK(kpool_indexer_topk(&p, fake, (const float*)fake, fake, (const int32_t*)fake,
                           (const int32_t*)fake, fake, ws, (int32_t*)fake, NULL, NULL) ==
        KPOOL_E_UNSUPPORTED);
  p.num_heads = 32;
  CHECK(kpool_indexer_topk(&p, fake, (const float*)fake, fake, (const int32_t*)fake,
                           (const int32_t*)fake, fake, ws - 1, (int32_t*)fake, NULL, NULL) ==
        KPOOL_E_WORKSPACE);
  {
    /* the indexer's launches: nine at 64K with 4096-row chunks */
    int32_t info[6 * 9];
    CHECK(kpool_indexer_launches(&p, NULL, 0) == 9);
    CHECK(kpool_indexer_launches(&p, info, 9) == 9);
    CHECK(info[0] == 61440 && info[1] == 65536 && info[2] == 16384 && info[3] == info[4]);
    CHECK(info[6 + 3] == 0 && info[6 + 4] == 4096 && info[6 + 5] == 1024);
    CHECK(kpool_indexer_scoring(&p, 9, fake, (const float*)fake, fake, (const int32_t*)fake,
                                (const int32_t*)fake, fake, ws, 0, NULL) == KPOOL_E_INVALID);
    CHECK(kpool_indexer_selection(&p, -1, (const int32_t*)fake, (const int32_t*)fake, fake, ws,
                                  (int32_t*)fake, NULL, NULL) == KPOOL_E_INVALID);
  }
  CHECK(kpool_fp8_quantize(fake, -1, (uint8_t*)fake, (float*)fake, NULL) == KPOOL_E_INVALID);
  {
    kpool_mla_params mp;
    memset(&mp, 0, sizeof mp);
    mp.num_tokens = 4;
    mp.num_heads = 64;
    mp.kv_rows = 16;
    mp.width = 8;
    mp.dim_qk = 512;
    mp.dim_v = 512;
    mp.sm_scale = 0.0625f;
    mp.num_heads = 96;
    CHECK(kpool_sparse_mla_fwd(&mp, fake, fake, (const int32_t*)fake, fake, (float*)fake, NULL) ==
          KPOOL_E_UNSUPPORTED);
    mp.num_heads = 64;
    mp.dim_v = 448;
    CHECK(kpool_sparse_mla_fwd(&mp, fake, fake, (const int32_t*)fake, fake, (float*)fake, NULL) ==
          KPOOL_E_UNSUPPORTED);
    mp.dim_v = 512;
    mp.width = -1;
    CHECK(kpool_sparse_mla_fwd(&mp, fake, fake, (const int32_t*)fake, fake, (float*)fake, NULL) ==
          KPOOL_E_INVALID);
    mp.width = 8;
    CHECK(kpool_sparse_mla_fwd(&mp, fake + 2, fake, (const int32_t*)fake, fake, (float*)fake,
                               NULL) == KPOOL_E_INVALID);
    mp.num_tokens = 0;
    CHECK(kpool_sparse_mla_fwd(&mp, NULL, NULL, NULL, NULL, NULL, NULL) == KPOOL_OK);
  }
  CHECK(kpool_check_cu_seqlens((const int32_t*)fake, -1, 8, 8, (int32_t*)fake, NULL) ==
        KPOOL_E_INVALID);
  CHECK(kpool_check_cu_seqlens(NULL, 1, 8, 8, (int32_t*)fake, NULL) == KPOOL_E_INVALID);
  CHECK((KPOOL_CU_FIRST_NOT_ZERO | KPOOL_CU_DECREASING | KPOOL_CU_TOO_LONG |
         KPOOL_CU_LAST_NOT_TOTAL) == 15);
  printf("all checks passed\n");
  return 0;
}
