// Host-side argument handling of libkpool under AddressSanitizer and
// UndefinedBehaviorSanitizer: the C-ABI layer (api.cpp) is built with both
// sanitizers on its host code and linked into this program with the
// unchanged kernels. Every call below fails validation (null, misaligned or
// inconsistent arguments, unsupported shapes, extreme sizes), so no kernel
// is launched; the sanitizers check the size arithmetic, the message
// formatting and the thread-local error string on the way. Exits non-zero
// on the first unexpected status. Built and run on a host without a GPU by
// tests/test_host_sanitizers.py.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>

#include "kpool.h"

static int failures = 0;

#define EXPECT(call, status)                                                        \
  do {                                                                              \
    const kpool_status got_ = (call);                                               \
    if (got_ != (status)) {                                                         \
      std::fprintf(stderr, "line %d: %s -> %d, expected %d (%s)\n", __LINE__, #call, \
                   (int)got_, (int)(status), kpool_last_error());                   \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

static kpool_params base() {
  kpool_params p;
  std::memset(&p, 0, sizeof p);
  p.num_docs = 1;
  p.total_tokens = 65536;
  p.max_seqlen = 65536;
  p.num_heads = 32;
  p.head_dim = 128;
  p.kpool = 4;
  p.index_topk = 2048;
  p.always_select_tail = 1;
  p.query_chunk = 4096;
  return p;
}

int main() {
  alignas(256) static char buf[1024];
  void* F = buf;                                 // aligned, never dereferenced
  void* M = buf + 4;                             // 4-byte aligned only
  const float* Ff = reinterpret_cast<const float*>(buf);
  const int32_t* Fi = reinterpret_cast<const int32_t*>(buf);
  int32_t* Fo = reinterpret_cast<int32_t*>(buf);
  kpool_params p = base();
  const size_t ws = kpool_workspace_bytes(&p);
  if (ws < (size_t)4096 * 16384 * 4) { std::fprintf(stderr, "workspace %zu\n", ws); ++failures; }

  // sizes at the edges of int32 arithmetic
  kpool_params big = base();
  big.total_tokens = 0x7fffffff;
  big.max_seqlen = 4 * 65536;
  big.query_chunk = 0x7fffffff;
  if (kpool_workspace_bytes(&big) == 0) { std::fprintf(stderr, "big workspace 0\n"); ++failures; }
  big.max_seqlen = 0x7fffffff;                   // too many pools per document
  if (kpool_workspace_bytes(&big) != 0) { std::fprintf(stderr, "oversized accepted\n"); ++failures; }
  kpool_params neg = base();
  neg.index_topk = 0x7fffffff;
  EXPECT(kpool_indexer_topk(&neg, F, Ff, F, Fi, Fi, F, ws, Fo, nullptr, nullptr),
         KPOOL_E_UNSUPPORTED);
  neg = base();
  neg.kpool = -5;
  EXPECT(kpool_compress(&neg, F, F, Ff, Fi, Fo, F, nullptr), KPOOL_E_UNSUPPORTED);
  neg = base();
  neg.scale = -1.f;
  EXPECT(kpool_indexer_topk(&neg, F, Ff, F, Fi, Fi, F, ws, Fo, nullptr, nullptr),
         KPOOL_E_INVALID);
  neg.scale = __builtin_nanf("");
  EXPECT(kpool_indexer_topk(&neg, F, Ff, F, Fi, Fi, F, ws, Fo, nullptr, nullptr),
         KPOOL_E_INVALID);

  // pointers: null, misaligned, workspace
  EXPECT(kpool_indexer_topk(nullptr, F, Ff, F, Fi, Fi, F, ws, Fo, nullptr, nullptr),
         KPOOL_E_INVALID);
  EXPECT(kpool_indexer_topk(&p, nullptr, Ff, F, Fi, Fi, F, ws, Fo, nullptr, nullptr),
         KPOOL_E_INVALID);
  EXPECT(kpool_indexer_topk(&p, M, Ff, F, Fi, Fi, F, ws, Fo, nullptr, nullptr), KPOOL_E_INVALID);
  EXPECT(kpool_indexer_topk(&p, F, Ff, F, Fi, Fi, F, ws - 1, Fo, nullptr, nullptr),
         KPOOL_E_WORKSPACE);
  EXPECT(kpool_compress(&p, F, F, reinterpret_cast<const float*>(M), Fi, Fo, F, nullptr),
         KPOOL_E_INVALID);
  EXPECT(kpool_logits(&p, F, Ff, F, Fi, Fi, 5, 3, F, ws, reinterpret_cast<float*>(F), 1, nullptr),
         KPOOL_E_INVALID);
  EXPECT(kpool_logits(&p, F, Ff, F, Fi, Fi, 0, 16, F, ws, reinterpret_cast<float*>(F), 64,
                      nullptr),
         KPOOL_E_INVALID);
  EXPECT(kpool_select(&p, Ff, -1, 3, Fi, Fi, Fo, nullptr), KPOOL_E_INVALID);
  EXPECT(kpool_select_expand(&p, Ff, 0, 3, Fi, Fi, nullptr, reinterpret_cast<int32_t*>(M),
                             nullptr),
         KPOOL_E_INVALID);
  EXPECT(kpool_expand(&p, Fi, Fi, Fi, nullptr, nullptr), KPOOL_E_INVALID);
  EXPECT(kpool_fp8_quantize(F, -7, reinterpret_cast<uint8_t*>(F), reinterpret_cast<float*>(F),
                            nullptr),
         KPOOL_E_INVALID);
  kpool_params f = base();
  f.index_topk = 4 * 5000;                      // beyond the fused kernel's list
  EXPECT(kpool_indexer_topk_fused(&f, F, Ff, F, Fi, Fi, nullptr, 0, Fo, nullptr, nullptr),
         KPOOL_E_UNSUPPORTED);

  // the indexer's launch plan (host arithmetic only) and its staged entry
  // points' checks; chunk bounds near 2^31 must not overflow
  {
    int32_t info[6 * 9];
    if (kpool_indexer_launches(&p, info, 9) != 9 || info[0] != 61440 || info[2] != 16384 ||
        info[6 + 4] != 4096) {
      std::fprintf(stderr, "64K plan\n");
      ++failures;
    }
    kpool_params huge = base();
    huge.total_tokens = 0x7fffffff;
    huge.max_seqlen = 4 * 65536;
    huge.query_chunk = (1 << 30) + 1;          // the second chunk ends past 2^31
    int32_t hi[12];
    if (kpool_indexer_launches(&huge, hi, 2) != 2 || hi[1] != 0x7fffffff || hi[6] != 0 ||
        hi[7] != (1 << 30) + 1) {
      std::fprintf(stderr, "plan near 2^31\n");
      ++failures;
    }
    EXPECT(kpool_indexer_scoring(&p, 9, F, Ff, F, Fi, Fi, F, ws, 0, nullptr), KPOOL_E_INVALID);
    EXPECT(kpool_indexer_scoring(&p, -1, F, Ff, F, Fi, Fi, F, ws, 0, nullptr), KPOOL_E_INVALID);
    EXPECT(kpool_indexer_scoring(&p, 0, F, Ff, F, Fi, Fi, F, ws, 1, nullptr), KPOOL_E_INVALID);
    EXPECT(kpool_indexer_scoring(&p, 0, F, Ff, F, Fi, Fi, F, ws - 1, 0, nullptr),
           KPOOL_E_WORKSPACE);
    EXPECT(kpool_indexer_selection(&p, 9, Fi, Fi, F, ws, Fo, nullptr, nullptr), KPOOL_E_INVALID);
    EXPECT(kpool_indexer_selection(&p, 0, Fi, Fi, F, ws, reinterpret_cast<int32_t*>(M), nullptr,
                                   nullptr),
           KPOOL_E_INVALID);
    EXPECT(kpool_indexer_scoring(&huge, 2, F, Ff, F, Fi, Fi, F, ws, 0, nullptr), KPOOL_E_INVALID);
  }

  // serving entry points
  kpool_params d = base();
  d.num_docs = 64;
  d.total_tokens = 0;
  const size_t dws = kpool_decode_workspace_bytes(&d);
  EXPECT(kpool_decode_topk(&d, F, Ff, F, 100, nullptr, Fi, Fi, nullptr, F, dws - 1, Fo, nullptr,
                           nullptr),
         KPOOL_E_WORKSPACE);
  EXPECT(kpool_decode_topk(&d, F, Ff, F, -1, nullptr, Fi, Fi, nullptr, F, dws, Fo, nullptr,
                           nullptr),
         KPOOL_E_INVALID);
  d.num_docs = 1 << 20;                         // scores beyond the built-in scratch
  EXPECT(kpool_decode_topk_noalloc(&d, F, Ff, F, 100, nullptr, Fi, Fi, nullptr, Fo, nullptr,
                                   nullptr),
         KPOOL_E_WORKSPACE);
  EXPECT(kpool_compress_pools(&d, F, F, Ff, 0x7fffffff, Fi, 10, F, nullptr, nullptr),
         KPOOL_E_UNSUPPORTED);

  // the error string is per thread
  std::thread other([&] {
    EXPECT(kpool_expand(nullptr, Fi, Fi, Fi, Fo, nullptr), KPOOL_E_INVALID);
  });
  other.join();
  if (std::strlen(kpool_last_error()) == 0) { std::fprintf(stderr, "empty error\n"); ++failures; }
  for (int s = -1; s <= 5; ++s) (void)std::strlen(kpool_status_string((kpool_status)s));

  std::printf(failures ? "FAILED %d\n" : "all sanitized checks passed\n", failures);
  return failures ? 1 : 0;
}
