// C ABI of libkpool.so: argument checks, workspace layout and the query-chunk
// loop of the KPool indexer. The operations themselves are documented in
// include/kpool.h; this file only validates and enqueues kernels.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "kpool.h"
#include "kpool_internal.h"

namespace {

// A roctx range around the host side of one phase (its validation and
// launches), so a profiler's marker trace shows compress, each chunk's
// scoring and selection, and the serving calls by name. Without a profiler
// attached the calls return at once.
struct Range {
  explicit Range(const char* name) { roctxRangePushA(name); }
  ~Range() { roctxRangePop(); }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

thread_local std::string g_last_error;

kpool_status fail(kpool_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

kpool_status ok() {
  g_last_error.clear();
  return KPOOL_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Default query chunk: as many rows as fit a logits tile of this many bytes
// (4096 rows of 16384 pools at a 64K context; the whole batch for short ones).
constexpr size_t kDefaultTileBytes = size_t(256) << 20;

struct Derived {
  int B, T, H, D, kpool, topk, k_sel, width, max_pools, qc, tail, fp8;
  bool fused;                      // the indexer scores and selects in one kernel
  int64_t ld;
  float scale;
  size_t off_logits, off_qc, off_qs, off_kc, off_ks, total;
};

kpool_status derive(const kpool_params* p, Derived* d, bool need_heads) {
  if (!p) return fail(KPOOL_E_INVALID, "params is null");
  d->B = p->num_docs;
  d->T = p->total_tokens;
  d->H = p->num_heads;
  d->D = p->head_dim;
  d->kpool = p->kpool;
  d->topk = p->index_topk;
  d->tail = p->always_select_tail;
  d->fp8 = p->use_fp8;
  if (d->B < 1) return fail(KPOOL_E_INVALID, "num_docs must be >= 1 (got %d)", d->B);
  if (d->T < 0) return fail(KPOOL_E_INVALID, "total_tokens must be >= 0 (got %d)", d->T);
  if (p->max_seqlen < 0 || p->max_seqlen > d->T)
    return fail(KPOOL_E_INVALID, "max_seqlen must be in [0, total_tokens] (got %d, T = %d)",
                p->max_seqlen, d->T);
  if (d->kpool < 1 || d->kpool > 64)
    return fail(KPOOL_E_UNSUPPORTED, "kpool must be in [1, 64] (got %d)", d->kpool);
  if (d->D != 64 && d->D != 128)
    return fail(KPOOL_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->D);
  if (d->tail != 0 && d->tail != 1)
    return fail(KPOOL_E_INVALID, "always_select_tail must be 0 or 1");
  if (d->fp8 != 0 && d->fp8 != 1) return fail(KPOOL_E_INVALID, "use_fp8 must be 0 or 1");
  if (need_heads) {
    if (d->H != 4 && d->H != 8 && d->H != 16 && d->H != 32 && d->H != 64)
      return fail(KPOOL_E_UNSUPPORTED, "num_heads must be 4, 8, 16, 32 or 64 (got %d)", d->H);
    if (d->topk < d->kpool)
      return fail(KPOOL_E_INVALID, "index_topk (%d) must be >= kpool (%d)", d->topk, d->kpool);
    if (d->topk > (1 << 24)) return fail(KPOOL_E_UNSUPPORTED, "index_topk too large");
    if (d->fp8 && d->D != 128)
      return fail(KPOOL_E_UNSUPPORTED, "the FP8 path needs head_dim == 128 (got %d)", d->D);
    if (p->query_chunk < 0) return fail(KPOOL_E_INVALID, "query_chunk must be >= 0");
    if (!(p->scale >= 0.f) || p->scale > 1e30f)
      return fail(KPOOL_E_INVALID, "scale must be finite and >= 0 (0 = head_dim^-1/2)");
  }
  d->k_sel = d->topk / d->kpool;
  d->width = d->topk + d->kpool;
  d->max_pools = p->max_seqlen / d->kpool;
  if (need_heads && d->max_pools > kpool::kMaxSelectPools)
    return fail(KPOOL_E_UNSUPPORTED, "max_seqlen / kpool = %d exceeds %d pools per document",
                d->max_pools, kpool::kMaxSelectPools);
  d->ld = (int64_t)round_up((size_t)std::max(d->max_pools, 1), 64);
  d->scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)d->D);
  const int64_t qc = p->query_chunk > 0
                       ? (int64_t)p->query_chunk
                       : (int64_t)(kDefaultTileBytes / ((size_t)d->ld * sizeof(float)));
  d->qc = (int)std::max<int64_t>(1, std::min<int64_t>(qc, std::max(d->T, 1)));
  d->fused = need_heads && kpool::logits_select_supported(d->H, d->D, d->fp8, d->k_sel);
  // workspace layout (256-byte aligned pieces): the FP8 codes and scales of
  // q and of the pooled keys, then the logits tile of the two-kernel path
  size_t off = 0;
  d->off_qc = d->off_qs = d->off_kc = d->off_ks = off;
  if (d->fp8) {
    const size_t qrows = (size_t)d->T * d->H, krows = (size_t)(d->T / d->kpool);
    d->off_qc = off;
    off = round_up(off + qrows * 128, 256);
    d->off_qs = off;
    off = round_up(off + qrows * 4, 256);
    d->off_kc = off;
    off = round_up(off + krows * 128, 256);
    d->off_ks = off;
    off = round_up(off + krows * 4, 256);
  }
  d->off_logits = off;
  off = round_up(off + (size_t)d->qc * d->ld * 4, 256);
  d->total = d->T > 0 ? off : 0;
  return KPOOL_OK;
}

// The indexer's scoring launches. Chunk c is query rows [c qc, min(T, (c + 1)
// qc)); a row t has at most (t + 1) / kpool causal pools, so the chunk's
// scores fit a row stride of min(max_pools, c1 / kpool) rounded up to 64.
// Two chunks share a launch when both fit the logits tile (qc x ld floats)
// at their own strides: the longest chunk left goes with the shortest, its
// rows first. Each CU then takes a long and a short block and the dispatcher
// evens them out, so whole blocks suffice (one start-up per block instead of
// two pieces of a long block), and there are about half as many launches.
// Every score is computed as in a launch of its own chunk.
struct ChunkLaunch {
  int c_long, c_short;             // chunk indices; c_short = -1: none
  int64_t ld_long, ld_short;       // their tile row strides (floats)
};

// first row and row count of chunk c (64-bit: T and the chunk may both be
// close to 2^31)
int64_t chunk_begin(const Derived& d, int c) { return (int64_t)c * d.qc; }
int64_t chunk_rows(const Derived& d, int c) {
  return std::min<int64_t>(d.T, chunk_begin(d, c) + d.qc) - chunk_begin(d, c);
}

int64_t chunk_ld(const Derived& d, int c) {
  const int64_t c1 = chunk_begin(d, c) + chunk_rows(d, c);
  const int64_t bound = std::min<int64_t>(d.max_pools, c1 / d.kpool);
  return (int64_t)round_up((size_t)std::max<int64_t>(bound, 1), 64);
}

// The plan is walked, never stored (a batch of 2^31 tokens in 1-row chunks
// has 2^31 launches): each step takes the longest chunk left and, when it
// fits, the shortest.
struct PlanWalk {
  int lo, hi;
  explicit PlanWalk(const Derived& d) : lo(0), hi(d.T > 0 ? (int)((d.T - 1) / d.qc) : -1) {}
  bool next(const Derived& d, ChunkLaunch& L) {
    if (lo > hi) return false;
    const int64_t cap = (int64_t)d.qc * d.ld;
    const int64_t ldh = chunk_ld(d, hi), ldl = chunk_ld(d, lo);
    if (lo < hi && chunk_rows(d, hi) * ldh + chunk_rows(d, lo) * ldl <= cap) {
      L = ChunkLaunch{hi, lo, ldh, ldl};
      ++lo;
    } else {
      L = ChunkLaunch{hi, -1, ldh, 0};
    }
    --hi;
    return true;
  }
};

int64_t plan_count(const Derived& d) {
  PlanWalk w(d);
  ChunkLaunch L;
  int64_t n = 0;
  while (w.next(d, L)) ++n;
  return n;
}

// launch i of the plan (0 <= i < plan_count(d))
ChunkLaunch plan_at(const Derived& d, int64_t i) {
  PlanWalk w(d);
  ChunkLaunch L{};
  for (int64_t k = 0; k <= i && w.next(d, L); ++k) {
  }
  return L;
}

kpool_status check_ptr(const void* ptr, size_t align, const char* name) {
  if (!ptr) return fail(KPOOL_E_INVALID, "%s is null", name);
  if (!aligned(ptr, align)) return fail(KPOOL_E_INVALID, "%s is not %zu-byte aligned", name, align);
  return KPOOL_OK;
}

#define CHECK(expr)                       \
  do {                                    \
    kpool_status s_ = (expr);             \
    if (s_ != KPOOL_OK) return s_;        \
  } while (0)

kpool_status after_launch() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KPOOL_E_LAUNCH, "HIP launch error: %s", hipGetErrorString(e));
  return ok();
}

kpool::LogitsArgs logits_args(const Derived& d, const void* q, const float* w, const void* pooled,
                              const int32_t* cu, const int32_t* cuP, uint8_t* ws) {
  kpool::LogitsArgs a{};
  a.q = d.fp8 ? (const void*)(ws + d.off_qc) : q;
  a.q_scale = d.fp8 ? reinterpret_cast<const float*>(ws + d.off_qs) : nullptr;
  a.w = w;
  a.keys = d.fp8 ? (const void*)(ws + d.off_kc) : pooled;
  a.k_scale = d.fp8 ? reinterpret_cast<const float*>(ws + d.off_ks) : nullptr;
  a.cu = cu;
  a.cu_pools = cuP;
  a.B = d.B; a.T = d.T; a.H = d.H; a.D = d.D; a.kpool = d.kpool;
  a.max_pools = d.max_pools; a.k_sel = d.k_sel; a.scale = d.scale;
  a.ld = d.ld;
  a.fp8 = d.fp8;
  return a;
}

void quantize_q(const Derived& d, const void* q, int q_begin, int q_end, uint8_t* ws,
                hipStream_t st) {
  const size_t qrow0 = (size_t)q_begin * d.H;
  const int qrows = (q_end - q_begin) * d.H;
  if (qrows <= 0) return;
  kpool::launch_fp8_quantize(reinterpret_cast<const uint16_t*>(q) + qrow0 * 128, qrows, nullptr,
                             ws + d.off_qc + qrow0 * 128,
                             reinterpret_cast<float*>(ws + d.off_qs) + qrow0, st);
}

void quantize_inputs(const Derived& d, const void* q, const void* pooled, const int32_t* cuP,
                     int q_begin, int q_end, uint8_t* ws, hipStream_t st) {
  quantize_q(d, q, q_begin, q_end, ws, st);
  kpool::launch_fp8_quantize(reinterpret_cast<const uint16_t*>(pooled), d.T / d.kpool,
                             cuP + d.B, ws + d.off_kc, reinterpret_cast<float*>(ws + d.off_ks), st);
}

// The rows of one scoring launch of the indexer: range a at the start of the
// tile, range b (possibly empty) right after a's rows.
struct LaunchRows {
  int a0, a1, b0, b1;
  int64_t lda, ldb;
};

LaunchRows launch_rows(const Derived& d, const ChunkLaunch& L) {
  LaunchRows R{};
  R.a0 = (int)chunk_begin(d, L.c_long);
  R.a1 = (int)(chunk_begin(d, L.c_long) + chunk_rows(d, L.c_long));
  R.lda = L.ld_long;
  if (L.c_short >= 0) {
    R.b0 = (int)chunk_begin(d, L.c_short);
    R.b1 = (int)(chunk_begin(d, L.c_short) + chunk_rows(d, L.c_short));
    R.ldb = L.ld_short;
  }
  return R;
}

// The scoring kernel of one indexer launch into the workspace tile.
void enqueue_scoring(const Derived& d, const LaunchRows& R, kpool::LogitsArgs a, uint8_t* ws,
                     hipStream_t st) {
  float* const tile = reinterpret_cast<float*>(ws + d.off_logits);
  a.skip_select_all = 1;
  a.q_begin = R.a0;
  a.q_end = R.a1;
  a.out = tile;
  a.ld = R.lda;
  a.q_begin2 = R.b0;
  a.q_end2 = R.b1;
  a.out2 = tile + (size_t)(R.a1 - R.a0) * R.lda;
  a.ld2 = R.ldb;
  kpool::launch_logits(a, st);
}

// The selection + expansion kernels of one indexer launch, from the tile.
void enqueue_selection(const Derived& d, const LaunchRows& R, const uint8_t* ws,
                       const int32_t* cu, const int32_t* cuP, int32_t* out_tok,
                       int32_t* out_ids, hipStream_t st) {
  const float* const tile = reinterpret_cast<const float*>(ws + d.off_logits);
  auto select = [&](const float* scores, int64_t ld, int c0, int c1) {
    kpool::launch_select(scores, ld, c0, c1, cu, cuP, d.B, d.T, d.kpool, d.k_sel, d.width,
                         d.tail, d.max_pools, out_ids ? out_ids + (size_t)c0 * d.k_sel : nullptr,
                         out_tok + (size_t)c0 * d.width, st);
  };
  if (R.b1 > R.b0)
    kpool::launch_select2(tile, R.lda, R.a0, R.a1, tile + (size_t)(R.a1 - R.a0) * R.lda, R.ldb,
                          R.b0, R.b1, cu, cuP, d.B, d.T, d.kpool, d.k_sel, d.width, d.tail,
                          d.max_pools, out_ids, out_tok, st);
  else
    select(tile, R.lda, R.a0, R.a1);
}

// Parameters of a decode call: num_docs = B sequences, max_seqlen bounds
// every sequence length; total_tokens and query_chunk are not used.
struct DecodeDerived {
  int B, H, D, kpool, k_sel, width, max_pools, tail, fp8;
  int64_t ld;
  float scale;
  size_t total;                    // workspace: the scores
};

kpool_status derive_decode(const kpool_params* p, DecodeDerived* d) {
  if (!p) return fail(KPOOL_E_INVALID, "params is null");
  d->B = p->num_docs;
  d->H = p->num_heads;
  d->D = p->head_dim;
  d->kpool = p->kpool;
  d->tail = p->always_select_tail;
  if (d->B < 1) return fail(KPOOL_E_INVALID, "num_docs (sequences) must be >= 1 (got %d)", d->B);
  if (p->max_seqlen < 0) return fail(KPOOL_E_INVALID, "max_seqlen must be >= 0");
  if (d->kpool < 1 || d->kpool > 64)
    return fail(KPOOL_E_UNSUPPORTED, "kpool must be in [1, 64] (got %d)", d->kpool);
  if (d->D != 64 && d->D != 128)
    return fail(KPOOL_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->D);
  if (d->H != 4 && d->H != 8 && d->H != 16 && d->H != 32 && d->H != 64)
    return fail(KPOOL_E_UNSUPPORTED, "num_heads must be 4, 8, 16, 32 or 64 (got %d)", d->H);
  if (d->tail != 0 && d->tail != 1)
    return fail(KPOOL_E_INVALID, "always_select_tail must be 0 or 1");
  d->fp8 = p->use_fp8;
  if (d->fp8 != 0 && d->fp8 != 1) return fail(KPOOL_E_INVALID, "use_fp8 must be 0 or 1");
  if (d->fp8 && d->D != 128)
    return fail(KPOOL_E_UNSUPPORTED, "the FP8 path needs head_dim == 128 (got %d)", d->D);
  if (p->index_topk < d->kpool)
    return fail(KPOOL_E_INVALID, "index_topk (%d) must be >= kpool (%d)", p->index_topk, d->kpool);
  if (p->index_topk > (1 << 24)) return fail(KPOOL_E_UNSUPPORTED, "index_topk too large");
  if (!(p->scale >= 0.f) || p->scale > 1e30f)
    return fail(KPOOL_E_INVALID, "scale must be finite and >= 0 (0 = head_dim^-1/2)");
  d->k_sel = p->index_topk / d->kpool;
  d->width = p->index_topk + d->kpool;
  d->max_pools = p->max_seqlen / d->kpool;
  if (d->max_pools > kpool::kMaxSelectPools)
    return fail(KPOOL_E_UNSUPPORTED, "max_seqlen / kpool = %d exceeds %d pools per sequence",
                d->max_pools, kpool::kMaxSelectPools);
  d->ld = (int64_t)round_up((size_t)std::max(d->max_pools, 1), 64);
  d->scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)d->D);
  d->total = round_up((size_t)d->B * d->ld * 4, 256);
  return KPOOL_OK;
}

// Checks shared by the two indexer entry points; `need` is the workspace
// the entry point uses.
kpool_status check_indexer_args(const Derived& d, const void* q, const float* w,
                                const void* pooled, const int32_t* cu_seqlens,
                                const int32_t* cu_pools, const void* workspace,
                                size_t workspace_bytes, size_t need,
                                const int32_t* out_token_idx, const int32_t* out_pool_idx) {
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(w, 4, "w"));
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(cu_pools, 4, "cu_pools"));
  CHECK(check_ptr(out_token_idx, 16, "out_token_idx"));
  if (out_pool_idx) CHECK(check_ptr(out_pool_idx, 4, "out_pool_idx"));
  if (d.T / d.kpool > 0) CHECK(check_ptr(pooled, 16, "pooled"));
  if (need > 0) {
    CHECK(check_ptr(workspace, 256, "workspace"));
    if (workspace_bytes < need)
      return fail(KPOOL_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  }
  return KPOOL_OK;
}

}  // namespace

extern "C" {

int kpool_abi_version(void) { return KPOOL_ABI_VERSION; }

size_t kpool_workspace_bytes(const kpool_params* p) {
  Derived d;
  if (derive(p, &d, true) != KPOOL_OK) return 0;
  return d.total;
}

int64_t kpool_logits_ld(const kpool_params* p) {
  Derived d;
  if (derive(p, &d, true) != KPOOL_OK) return 0;
  return d.ld;
}

int32_t kpool_query_chunk_rows(const kpool_params* p) {
  Derived d;
  if (derive(p, &d, true) != KPOOL_OK) return 0;
  return d.T > 0 ? d.qc : 0;
}

kpool_status kpool_compress(const kpool_params* p, const void* k, const void* gate,
                            const float* ape, const int32_t* cu_seqlens, int32_t* cu_pools,
                            void* pooled, void* stream) {
  Range range("kpool_compress");
  Derived d;
  CHECK(derive(p, &d, false));
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(cu_pools, 4, "cu_pools"));
  if (d.T / d.kpool > 0) {
    CHECK(check_ptr(k, 16, "k"));
    CHECK(check_ptr(gate, 16, "gate"));
    CHECK(check_ptr(ape, 16, "ape"));
    CHECK(check_ptr(pooled, 16, "pooled"));
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  kpool::launch_compress(reinterpret_cast<const uint16_t*>(k),
                         reinterpret_cast<const uint16_t*>(gate), ape, cu_seqlens, cu_pools, d.B,
                         d.T, d.D, d.kpool, reinterpret_cast<uint16_t*>(pooled), st);
  return after_launch();
}

kpool_status kpool_indexer_topk(const kpool_params* p, const void* q, const float* w,
                                const void* pooled, const int32_t* cu_seqlens,
                                const int32_t* cu_pools, void* workspace,
                                size_t workspace_bytes, int32_t* out_token_idx,
                                int32_t* out_pool_idx, void* stream) {
  Range range("kpool_indexer_topk");
  Derived d;
  CHECK(derive(p, &d, true));
  if (d.T == 0) return ok();
  CHECK(check_indexer_args(d, q, w, pooled, cu_seqlens, cu_pools, workspace, workspace_bytes,
                           d.total, out_token_idx, out_pool_idx));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  (void)hipGetLastError();
  if (d.fp8) {
    Range r("kpool.fp8_quantize");
    quantize_inputs(d, q, pooled, cu_pools, 0, d.T, ws, st);
  }
  const kpool::LogitsArgs a = logits_args(d, q, w, pooled, cu_seqlens, cu_pools, ws);
  PlanWalk walk(d);
  ChunkLaunch L;
  while (walk.next(d, L)) {
    const LaunchRows R = launch_rows(d, L);
    {
      Range r("kpool.logits");
      enqueue_scoring(d, R, a, ws, st);
    }
    Range r("kpool.select_expand");
    enqueue_selection(d, R, ws, cu_seqlens, cu_pools, out_token_idx, out_pool_idx, st);
  }
  return after_launch();
}

int32_t kpool_indexer_launches(const kpool_params* p, int32_t* info, int32_t max_launches) {
  Derived d;
  if (derive(p, &d, true) != KPOOL_OK) return 0;
  PlanWalk walk(d);
  ChunkLaunch L;
  int64_t n = 0;
  while (walk.next(d, L)) {
    if (info && n < max_launches) {
      const LaunchRows R = launch_rows(d, L);
      int32_t* o = info + 6 * (size_t)n;
      o[0] = R.a0; o[1] = R.a1; o[2] = (int32_t)R.lda;
      o[3] = R.b0; o[4] = R.b1; o[5] = (int32_t)R.ldb;
    }
    ++n;
  }
  return (int32_t)std::min<int64_t>(n, 0x7fffffff);
}

kpool_status kpool_indexer_scoring(const kpool_params* p, int32_t launch, const void* q,
                                   const float* w, const void* pooled,
                                   const int32_t* cu_seqlens, const int32_t* cu_pools,
                                   void* workspace, size_t workspace_bytes, int32_t flags,
                                   void* stream) {
  Derived d;
  CHECK(derive(p, &d, true));
  if (flags & ~KPOOL_LOGITS_INPUTS_QUANTIZED)
    return fail(KPOOL_E_INVALID, "unknown scoring flags 0x%x", flags);
  const int64_t nl = plan_count(d);
  if (launch < 0 || launch >= nl)
    return fail(KPOOL_E_INVALID, "launch %d outside [0, %lld)", launch, (long long)nl);
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(w, 4, "w"));
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(cu_pools, 4, "cu_pools"));
  if (d.T / d.kpool > 0) CHECK(check_ptr(pooled, 16, "pooled"));
  CHECK(check_ptr(workspace, 256, "workspace"));
  if (workspace_bytes < d.total)
    return fail(KPOOL_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, d.total);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  const LaunchRows R = launch_rows(d, plan_at(d, launch));
  (void)hipGetLastError();
  if (d.fp8 && !(flags & KPOOL_LOGITS_INPUTS_QUANTIZED)) {
    quantize_inputs(d, q, pooled, cu_pools, R.a0, R.a1, ws, st);
    quantize_q(d, q, R.b0, R.b1, ws, st);
  }
  Range r("kpool.logits");
  enqueue_scoring(d, R, logits_args(d, q, w, pooled, cu_seqlens, cu_pools, ws), ws, st);
  return after_launch();
}

kpool_status kpool_indexer_selection(const kpool_params* p, int32_t launch,
                                     const int32_t* cu_seqlens, const int32_t* cu_pools,
                                     const void* workspace, size_t workspace_bytes,
                                     int32_t* out_token_idx, int32_t* out_pool_idx,
                                     void* stream) {
  Derived d;
  CHECK(derive(p, &d, true));
  const int64_t nl = plan_count(d);
  if (launch < 0 || launch >= nl)
    return fail(KPOOL_E_INVALID, "launch %d outside [0, %lld)", launch, (long long)nl);
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(cu_pools, 4, "cu_pools"));
  CHECK(check_ptr(out_token_idx, 16, "out_token_idx"));
  if (out_pool_idx) CHECK(check_ptr(out_pool_idx, 4, "out_pool_idx"));
  CHECK(check_ptr(workspace, 256, "workspace"));
  if (workspace_bytes < d.total)
    return fail(KPOOL_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, d.total);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  Range r("kpool.select_expand");
  enqueue_selection(d, launch_rows(d, plan_at(d, launch)), reinterpret_cast<const uint8_t*>(workspace),
                    cu_seqlens, cu_pools, out_token_idx, out_pool_idx, st);
  return after_launch();
}

int32_t kpool_fused_max_ksel(const kpool_params* p) {
  if (!p) return 0;
  const int H = p->num_heads, D = p->head_dim, fp8 = p->use_fp8;
  if (H != 4 && H != 8 && H != 16 && H != 32 && H != 64) return 0;
  if ((D != 64 && D != 128) || (fp8 != 0 && fp8 != 1) || (fp8 && D != 128)) return 0;
  return kpool::logits_select_max_ksel(H, D, fp8);
}

size_t kpool_fused_workspace_bytes(const kpool_params* p) {
  Derived d;
  if (derive(p, &d, true) != KPOOL_OK || !d.fused || d.T == 0) return 0;
  return d.off_logits;             // the FP8 codes and scales; no tile
}

kpool_status kpool_indexer_topk_fused(const kpool_params* p, const void* q, const float* w,
                                      const void* pooled, const int32_t* cu_seqlens,
                                      const int32_t* cu_pools, void* workspace,
                                      size_t workspace_bytes, int32_t* out_token_idx,
                                      int32_t* out_pool_idx, void* stream) {
  Range range("kpool_indexer_topk_fused");
  Derived d;
  CHECK(derive(p, &d, true));
  if (!d.fused)
    return fail(KPOOL_E_UNSUPPORTED,
                "K_sel = %d does not fit the fused kernel's per-query candidate list at H = %d, "
                "D = %d%s (kpool_indexer_topk takes any K_sel)",
                d.k_sel, d.H, d.D, d.fp8 ? ", FP8" : "");
  if (d.T == 0) return ok();
  CHECK(check_indexer_args(d, q, w, pooled, cu_seqlens, cu_pools, workspace, workspace_bytes,
                           d.off_logits, out_token_idx, out_pool_idx));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  (void)hipGetLastError();
  if (d.fp8) quantize_inputs(d, q, pooled, cu_pools, 0, d.T, ws, st);
  kpool::LogitsArgs a = logits_args(d, q, w, pooled, cu_seqlens, cu_pools, ws);
  a.skip_select_all = 1;
  a.width = d.width;
  a.tail_on = d.tail;
  // one launch per query chunk (no tile, so no two-chunk launches); nothing
  // but the token rows (and pool ids) is written
  for (int64_t c0 = 0; c0 < d.T; c0 += d.qc) {
    const int64_t c1 = std::min<int64_t>(d.T, c0 + d.qc);
    a.q_begin = (int)c0;
    a.q_end = (int)c1;
    a.out_tok = out_token_idx + (size_t)c0 * d.width;
    a.out_ids = out_pool_idx ? out_pool_idx + (size_t)c0 * d.k_sel : nullptr;
    kpool::launch_logits_select(a, st);
  }
  return after_launch();
}

kpool_status kpool_logits(const kpool_params* p, const void* q, const float* w,
                          const void* pooled, const int32_t* cu_seqlens,
                          const int32_t* cu_pools, int32_t q_begin, int32_t q_end,
                          void* workspace, size_t workspace_bytes, float* out, int32_t flags,
                          void* stream) {
  Derived d;
  CHECK(derive(p, &d, true));
  if (flags & ~(KPOOL_LOGITS_FILL_MASKED | KPOOL_LOGITS_SKIP_ALL_SELECTED |
                KPOOL_LOGITS_INPUTS_QUANTIZED))
    return fail(KPOOL_E_INVALID, "unknown logits flags 0x%x", flags);
  if (q_begin < 0 || q_end < q_begin || q_end > d.T)
    return fail(KPOOL_E_INVALID, "query rows [%d, %d) outside [0, %d]", q_begin, q_end, d.T);
  if (q_end == q_begin) return ok();
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(w, 4, "w"));
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(cu_pools, 4, "cu_pools"));
  CHECK(check_ptr(out, 16, "out"));
  if (d.T / d.kpool > 0) CHECK(check_ptr(pooled, 16, "pooled"));
  if (d.fp8) {                     // the codes and scales; no tile
    CHECK(check_ptr(workspace, 256, "workspace"));
    if (workspace_bytes < d.off_logits)
      return fail(KPOOL_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                  d.off_logits);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  (void)hipGetLastError();
  if (d.fp8 && !(flags & KPOOL_LOGITS_INPUTS_QUANTIZED))
    quantize_inputs(d, q, pooled, cu_pools, q_begin, q_end, ws, st);
  kpool::LogitsArgs a = logits_args(d, q, w, pooled, cu_seqlens, cu_pools, ws);
  a.out = out;
  a.q_begin = q_begin;
  a.q_end = q_end;
  a.fill_masked = (flags & KPOOL_LOGITS_FILL_MASKED) ? 1 : 0;
  a.skip_select_all = (flags & KPOOL_LOGITS_SKIP_ALL_SELECTED) ? 1 : 0;
  kpool::launch_logits(a, st);
  return after_launch();
}

kpool_status kpool_select(const kpool_params* p, const float* logits, int32_t q_begin,
                          int32_t q_end, const int32_t* cu_seqlens, const int32_t* cu_pools,
                          int32_t* out_pool_idx, void* stream) {
  Derived d;
  CHECK(derive(p, &d, true));
  if (q_begin < 0 || q_end < q_begin || q_end > d.T)
    return fail(KPOOL_E_INVALID, "query rows [%d, %d) outside [0, %d]", q_begin, q_end, d.T);
  if (q_end == q_begin) return ok();
  CHECK(check_ptr(logits, 16, "logits"));
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(cu_pools, 4, "cu_pools"));
  CHECK(check_ptr(out_pool_idx, 4, "out_pool_idx"));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  kpool::launch_select(logits, d.ld, q_begin, q_end, cu_seqlens, cu_pools, d.B, d.T, d.kpool,
                       d.k_sel, d.width, d.tail, d.max_pools, out_pool_idx, nullptr, st);
  return after_launch();
}

kpool_status kpool_select_expand(const kpool_params* p, const float* logits, int32_t q_begin,
                                 int32_t q_end, const int32_t* cu_seqlens,
                                 const int32_t* cu_pools, int32_t* out_pool_idx,
                                 int32_t* out_token_idx, void* stream) {
  Derived d;
  CHECK(derive(p, &d, true));
  if (q_begin < 0 || q_end < q_begin || q_end > d.T)
    return fail(KPOOL_E_INVALID, "query rows [%d, %d) outside [0, %d]", q_begin, q_end, d.T);
  if (q_end == q_begin) return ok();
  CHECK(check_ptr(logits, 16, "logits"));
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(cu_pools, 4, "cu_pools"));
  CHECK(check_ptr(out_token_idx, 16, "out_token_idx"));
  if (out_pool_idx) CHECK(check_ptr(out_pool_idx, 4, "out_pool_idx"));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  kpool::launch_select(logits, d.ld, q_begin, q_end, cu_seqlens, cu_pools, d.B, d.T, d.kpool,
                       d.k_sel, d.width, d.tail, d.max_pools, out_pool_idx, out_token_idx, st);
  return after_launch();
}

kpool_status kpool_expand(const kpool_params* p, const int32_t* pool_idx,
                          const int32_t* cu_seqlens, const int32_t* cu_pools,
                          int32_t* out_token_idx, void* stream) {
  Derived d;
  CHECK(derive(p, &d, true));
  if (d.T == 0) return ok();
  CHECK(check_ptr(pool_idx, 4, "pool_idx"));
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(cu_pools, 4, "cu_pools"));
  CHECK(check_ptr(out_token_idx, 16, "out_token_idx"));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  kpool::launch_expand(pool_idx, 0, d.T, cu_seqlens, cu_pools, d.B, d.T, d.kpool, d.k_sel,
                       d.width, d.tail, d.max_pools, out_token_idx, st);
  return after_launch();
}

size_t kpool_decode_workspace_bytes(const kpool_params* p) {
  DecodeDerived d;
  if (derive_decode(p, &d) != KPOOL_OK) return 0;
  return d.total;
}

}  // extern "C"

namespace {

// Argument checks of the decode entry points, workspace aside.
kpool_status check_decode_args(const DecodeDerived& d, const void* q, const float* w,
                               const void* pooled, int32_t pooled_rows,
                               const float* pooled_scale, const int32_t* pool_start,
                               const int32_t* seq_lens, const int32_t* token_base,
                               const int32_t* out_token_idx, const int32_t* out_pool_idx) {
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(w, 4, "w"));
  CHECK(check_ptr(pool_start, 4, "pool_start"));
  CHECK(check_ptr(seq_lens, 4, "seq_lens"));
  if (token_base) CHECK(check_ptr(token_base, 4, "token_base"));
  CHECK(check_ptr(out_token_idx, 16, "out_token_idx"));
  if (out_pool_idx) CHECK(check_ptr(out_pool_idx, 4, "out_pool_idx"));
  if (pooled_rows < 0) return fail(KPOOL_E_INVALID, "pooled_rows must be >= 0 (got %d)", pooled_rows);
  if (d.max_pools > 0 && pooled_rows > 0) {
    CHECK(check_ptr(pooled, 16, "pooled"));
    if (d.fp8) CHECK(check_ptr(pooled_scale, 4, "pooled_scale"));
  }
  return KPOOL_OK;
}

// The two launches of a decode step; `scores` holds B rows of d.ld floats.
kpool_status run_decode(const DecodeDerived& d, const void* q, const float* w,
                        const void* pooled, int32_t pooled_rows, const float* pooled_scale,
                        const int32_t* pool_start, const int32_t* seq_lens,
                        const int32_t* token_base, float* scores, int32_t* out_token_idx,
                        int32_t* out_pool_idx, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  kpool::DecodeLogitsArgs a{};
  a.q = q;                       // BF16; the FP8 kernel quantises its rows itself
  if (d.fp8) a.k_scale = pooled_scale;
  a.fp8 = d.fp8;
  a.w = w;
  a.keys = pooled;
  a.pooled_rows = pooled_rows;
  a.pool_start = pool_start;
  a.seq_lens = seq_lens;
  a.B = d.B; a.H = d.H; a.D = d.D; a.kpool = d.kpool; a.max_pools = d.max_pools;
  a.scale = d.scale;
  a.out = scores;
  a.ld = d.ld;
  kpool::launch_decode_logits(a, st);
  kpool::launch_select_decode(scores, d.ld, d.B, seq_lens, pool_start, token_base, d.kpool,
                              d.k_sel, d.width, d.tail, d.max_pools, out_pool_idx, out_token_idx,
                              st);
  return after_launch();
}

// Scratch of kpool_decode_topk_noalloc: the scores of one decode step live in
// this array, so that entry point allocates nothing. Each device holds its
// own copy, from the library's load until the process ends; its address on a
// device comes from hipGetSymbolAddress with that device current (the
// array's name in host code is only a stand-in and is never used as an
// address).
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per
// device); null with a message on failure.
kpool_status scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KPOOL_E_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KPOOL_E_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(KPOOL_E_LAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KPOOL_OK;
}

}  // namespace

extern "C" {

kpool_status kpool_decode_topk(const kpool_params* p, const void* q, const float* w,
                               const void* pooled, int32_t pooled_rows,
                               const float* pooled_scale, const int32_t* pool_start,
                               const int32_t* seq_lens, const int32_t* token_base,
                               void* workspace, size_t workspace_bytes,
                               int32_t* out_token_idx, int32_t* out_pool_idx, void* stream) {
  Range range("kpool_decode_topk");
  DecodeDerived d;
  CHECK(derive_decode(p, &d));
  CHECK(check_decode_args(d, q, w, pooled, pooled_rows, pooled_scale, pool_start, seq_lens,
                          token_base, out_token_idx, out_pool_idx));
  CHECK(check_ptr(workspace, 256, "workspace"));
  if (workspace_bytes < d.total)
    return fail(KPOOL_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, d.total);
  return run_decode(d, q, w, pooled, pooled_rows, pooled_scale, pool_start, seq_lens, token_base,
                    reinterpret_cast<float*>(workspace), out_token_idx, out_pool_idx, stream);
}

size_t kpool_decode_noalloc_max_bytes(void) { return kScratchBytes; }

size_t kpool_proj_workspace_bytes(const kpool_proj_params* pp) {
  if (!pp || pp->hidden <= 0) return 0;
  return round_up((size_t)128 * pp->hidden * 2, 256);
}

kpool_status kpool_indexer_projections(const kpool_proj_params* pp, const void* x, const void* qr,
                                       const void* wq_b, const void* wk,
                                       const float* k_norm_weight, const float* k_norm_bias,
                                       const void* wg, const float* ww, void* workspace,
                                       size_t workspace_bytes, void* q_out, void* k_out,
                                       void* gate_out, float* w_out, void* stream) {
  Range range("kpool_indexer_projections");
  if (!pp) return fail(KPOOL_E_INVALID, "params is null");
  const int T = pp->num_tokens, hidden = pp->hidden, qlr = pp->q_lora_rank, H = pp->num_heads;
  if (T < 0) return fail(KPOOL_E_INVALID, "num_tokens must be >= 0 (got %d)", T);
  if (pp->head_dim != 128)
    return fail(KPOOL_E_UNSUPPORTED, "the projections need head_dim == 128 (got %d)", pp->head_dim);
  if (H != 4 && H != 8 && H != 16 && H != 32)
    return fail(KPOOL_E_UNSUPPORTED, "the projections take num_heads 4, 8, 16 or 32 (got %d)", H);
  if (hidden <= 0 || hidden % 64 != 0 || qlr <= 0 || qlr % 64 != 0)
    return fail(KPOOL_E_UNSUPPORTED, "hidden (%d) and q_lora_rank (%d) must be positive "
                "multiples of 64", hidden, qlr);
  if (!(pp->eps >= 0.f) || pp->eps > 1.f)
    return fail(KPOOL_E_INVALID, "eps must be in [0, 1] (0 = 1e-6)");
  if (T == 0) return ok();
  CHECK(check_ptr(x, 16, "x"));
  CHECK(check_ptr(qr, 16, "qr"));
  CHECK(check_ptr(wq_b, 16, "wq_b"));
  CHECK(check_ptr(wk, 16, "wk"));
  CHECK(check_ptr(k_norm_weight, 4, "k_norm_weight"));
  CHECK(check_ptr(k_norm_bias, 4, "k_norm_bias"));
  CHECK(check_ptr(wg, 16, "wg"));
  CHECK(check_ptr(ww, 4, "ww"));
  CHECK(check_ptr(q_out, 16, "q_out"));
  CHECK(check_ptr(k_out, 16, "k_out"));
  CHECK(check_ptr(gate_out, 16, "gate_out"));
  CHECK(check_ptr(w_out, 4, "w_out"));
  const size_t need = kpool_proj_workspace_bytes(pp);
  CHECK(check_ptr(workspace, 256, "workspace"));
  if (workspace_bytes < need)
    return fail(KPOOL_E_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  kpool::ProjArgs a{};
  a.x = reinterpret_cast<const uint16_t*>(x);
  a.qr = reinterpret_cast<const uint16_t*>(qr);
  a.wq_b = reinterpret_cast<const uint16_t*>(wq_b);
  a.wk = reinterpret_cast<const uint16_t*>(wk);
  a.ln_w = k_norm_weight;
  a.ln_b = k_norm_bias;
  a.wg = reinterpret_cast<const uint16_t*>(wg);
  a.ww = ww;
  a.w3 = reinterpret_cast<uint16_t*>(workspace);
  a.T = T; a.hidden = hidden; a.q_lora = qlr; a.H = H;
  a.eps = pp->eps > 0.f ? pp->eps : 1e-6f;
  a.q = reinterpret_cast<uint16_t*>(q_out);
  a.k = reinterpret_cast<uint16_t*>(k_out);
  a.gate = reinterpret_cast<uint16_t*>(gate_out);
  a.w = w_out;
  (void)hipGetLastError();
  kpool::launch_indexer_projections(a, reinterpret_cast<hipStream_t>(stream));
  return after_launch();
}

kpool_status kpool_check_cu_seqlens(const int32_t* cu_seqlens, int32_t num_docs,
                                    int32_t total_tokens, int32_t max_seqlen, int32_t* flags_out,
                                    void* stream) {
  Range range("kpool_check_cu_seqlens");
  static_assert(kpool::kCuFirstNotZero == KPOOL_CU_FIRST_NOT_ZERO &&
                    kpool::kCuDecreasing == KPOOL_CU_DECREASING &&
                    kpool::kCuTooLong == KPOOL_CU_TOO_LONG &&
                    kpool::kCuLastNotTotal == KPOOL_CU_LAST_NOT_TOTAL,
                "violation bits");
  if (num_docs < 0 || total_tokens < 0 || max_seqlen < 0)
    return fail(KPOOL_E_INVALID, "num_docs (%d), total_tokens (%d) and max_seqlen (%d) must be >= 0",
                num_docs, total_tokens, max_seqlen);
  CHECK(check_ptr(cu_seqlens, 4, "cu_seqlens"));
  CHECK(check_ptr(flags_out, 4, "flags_out"));
  (void)hipGetLastError();
  hipError_t e = kpool::launch_check_cu_seqlens(cu_seqlens, num_docs, total_tokens, max_seqlen,
                                                flags_out, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KPOOL_E_LAUNCH, "HIP launch error: %s", hipGetErrorString(e));
  return ok();
}

kpool_status kpool_sparse_mla_fwd(const kpool_mla_params* mp, const void* q, const void* kv,
                                  const int32_t* indices, void* out, float* lse, void* stream) {
  Range range("kpool_sparse_mla_fwd");
  if (!mp) return fail(KPOOL_E_INVALID, "params is null");
  const int T = mp->num_tokens, H = mp->num_heads, N = mp->kv_rows, W = mp->width;
  if (T < 0 || N < 0 || W < 0)
    return fail(KPOOL_E_INVALID, "num_tokens (%d), kv_rows (%d) and width (%d) must be >= 0", T,
                N, W);
  if (H <= 0 || H % 64 != 0)
    return fail(KPOOL_E_UNSUPPORTED, "num_heads must be a positive multiple of 64 (got %d)", H);
  if (W > 4096)
    return fail(KPOOL_E_UNSUPPORTED, "width must be <= 4096 entries per query (got %d)", W);
  if (mp->dim_qk != 512 || mp->dim_v != 512)
    return fail(KPOOL_E_UNSUPPORTED, "dim_qk and dim_v must be 512 (got %d, %d)", mp->dim_qk,
                mp->dim_v);
  if (!std::isfinite(mp->sm_scale) || !(mp->sm_scale > 0.f))
    return fail(KPOOL_E_INVALID, "sm_scale must be finite and > 0");
  if ((int64_t)T * (H / 64) > (1ll << 31) - 8)
    return fail(KPOOL_E_UNSUPPORTED, "num_tokens * num_heads / 64 is too large for one launch");
  if (T == 0) return ok();
  CHECK(check_ptr(q, 16, "q"));
  CHECK(check_ptr(out, 16, "out"));
  CHECK(check_ptr(lse, 4, "lse"));
  if (N > 0) CHECK(check_ptr(kv, 16, "kv"));
  if (W > 0) CHECK(check_ptr(indices, 4, "indices"));
  kpool::MlaArgs a{};
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.kv = reinterpret_cast<const uint16_t*>(kv);
  a.idx = indices;
  a.out = reinterpret_cast<uint16_t*>(out);
  a.lse = lse;
  a.T = T; a.H = H; a.N = N; a.W = W;
  a.scale2 = (float)((double)mp->sm_scale * 1.4426950408889634);
  (void)hipGetLastError();
  hipError_t e = kpool::launch_sparse_mla(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KPOOL_E_LAUNCH, "HIP launch error: %s", hipGetErrorString(e));
  return after_launch();
}

kpool_status kpool_decode_topk_noalloc(const kpool_params* p, const void* q, const float* w,
                                       const void* pooled, int32_t pooled_rows,
                                       const float* pooled_scale, const int32_t* pool_start,
                                       const int32_t* seq_lens, const int32_t* token_base,
                                       int32_t* out_token_idx, int32_t* out_pool_idx,
                                       void* stream) {
  Range range("kpool_decode_topk_noalloc");
  DecodeDerived d;
  CHECK(derive_decode(p, &d));
  if (d.total > kScratchBytes)
    return fail(KPOOL_E_WORKSPACE,
                "the scores of %d sequences of up to %d pools need %zu bytes; the built-in "
                "scratch holds %zu (num_docs * kpool_logits_ld * 4)",
                d.B, d.max_pools, d.total, kScratchBytes);
  CHECK(check_decode_args(d, q, w, pooled, pooled_rows, pooled_scale, pool_start, seq_lens,
                          token_base, out_token_idx, out_pool_idx));
  void* ws = nullptr;
  CHECK(scratch_on_current_device(&ws));
  return run_decode(d, q, w, pooled, pooled_rows, pooled_scale, pool_start, seq_lens, token_base,
                    reinterpret_cast<float*>(ws), out_token_idx, out_pool_idx, stream);
}

kpool_status kpool_compress_pools(const kpool_params* p, const void* k, const void* gate,
                                  const float* ape, int32_t num_pools, const int32_t* dst_rows,
                                  int32_t pooled_rows, void* pooled, float* pooled_scale,
                                  void* stream) {
  Range range("kpool_compress_pools");
  if (!p) return fail(KPOOL_E_INVALID, "params is null");
  const int D = p->head_dim, kp = p->kpool;
  if (p->use_fp8 != 0 && p->use_fp8 != 1) return fail(KPOOL_E_INVALID, "use_fp8 must be 0 or 1");
  if (p->use_fp8 && D != 128)
    return fail(KPOOL_E_UNSUPPORTED, "the FP8 path needs head_dim == 128 (got %d)", D);
  if (kp < 1 || kp > 64) return fail(KPOOL_E_UNSUPPORTED, "kpool must be in [1, 64] (got %d)", kp);
  if (D != 64 && D != 128) return fail(KPOOL_E_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", D);
  if (num_pools < 0) return fail(KPOOL_E_INVALID, "num_pools must be >= 0 (got %d)", num_pools);
  if (pooled_rows < 0) return fail(KPOOL_E_INVALID, "pooled_rows must be >= 0 (got %d)", pooled_rows);
  if ((int64_t)num_pools * kp > INT32_MAX) return fail(KPOOL_E_UNSUPPORTED, "too many tokens");
  if (num_pools == 0) return ok();
  CHECK(check_ptr(k, 16, "k"));
  CHECK(check_ptr(gate, 16, "gate"));
  CHECK(check_ptr(ape, 16, "ape"));
  CHECK(check_ptr(dst_rows, 4, "dst_rows"));
  CHECK(check_ptr(pooled, 16, "pooled"));
  if (p->use_fp8) CHECK(check_ptr(pooled_scale, 4, "pooled_scale"));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  kpool::launch_compress_pools(reinterpret_cast<const uint16_t*>(k),
                               reinterpret_cast<const uint16_t*>(gate), ape, num_pools, D, kp,
                               dst_rows, pooled_rows, reinterpret_cast<uint16_t*>(pooled),
                               p->use_fp8 ? pooled_scale : nullptr, st);
  return after_launch();
}

kpool_status kpool_fp8_quantize(const void* x, int32_t rows, uint8_t* codes, float* row_scale,
                                void* stream) {
  if (rows < 0) return fail(KPOOL_E_INVALID, "rows must be >= 0 (got %d)", rows);
  if (rows == 0) return ok();
  CHECK(check_ptr(x, 16, "x"));
  CHECK(check_ptr(codes, 16, "codes"));
  CHECK(check_ptr(row_scale, 4, "row_scale"));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  kpool::launch_fp8_quantize(reinterpret_cast<const uint16_t*>(x), rows, nullptr, codes, row_scale,
                             st);
  return after_launch();
}

const char* kpool_status_string(kpool_status s) {
  // a C caller may pass any int: read it as one (an out-of-range value
  // loaded as the enum type would be undefined in C++)
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case KPOOL_OK: return "ok";
    case KPOOL_E_INVALID: return "invalid argument";
    case KPOOL_E_UNSUPPORTED: return "unsupported shape";
    case KPOOL_E_WORKSPACE: return "workspace too small";
    case KPOOL_E_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* kpool_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
