// Host-side launchers of the KPool kernels (internal to libkpool.so). Every
// launcher assumes its arguments were validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kpool {

// Key compression; also writes cu_pools (the per-document pool offsets).
void launch_compress(const uint16_t* k, const uint16_t* gate, const float* ape,
                     const int32_t* cu, int32_t* cu_pools, int B, int T, int D, int kpool,
                     uint16_t* pooled, hipStream_t st);

// FP8 input path over `rows` rows of 128 BF16 values. When rows_dev is not
// null, rows at or beyond *rows_dev are skipped (the count lives on the
// device, e.g. cu_pools[B]).
void launch_fp8_quantize(const uint16_t* x, int rows, const int32_t* rows_dev,
                         uint8_t* codes, float* row_scale, hipStream_t st);

struct LogitsArgs {
  const void* q;            // BF16 [T, H, D] or E4M3 codes [T, H, 128]
  const float* q_scale;     // FP8 path: FP32 [T, H] row scales, else null
  const float* w;           // FP32 [T, H]
  const void* keys;         // BF16 [T/kpool, D] or E4M3 codes [T/kpool, 128]
  const float* k_scale;     // FP8 path: FP32 [T/kpool] row scales, else null
  const int32_t* cu;
  const int32_t* cu_pools;
  int B, T, H, D, kpool, max_pools, k_sel;
  float scale;
  int q_begin, q_end;       // global query rows of this launch
  float* out;               // FP32 [q_end - q_begin, ld]
  int64_t ld;
  // a second row range in the same launch, scored into out2 with row stride
  // ld2 (none when q_end2 <= q_begin2; fill_masked covers the first range
  // only). Its blocks are dispatched after the first range's, so the range
  // with the longer rows goes first.
  int q_begin2, q_end2;
  float* out2;
  int64_t ld2;
  int fill_masked;          // 1: write -inf in columns n_c .. ld-1
  int skip_select_all;      // 1: leave rows with n_c <= k_sel unwritten
  int fp8;
  int pieces;               // set by the launcher: workgroups per query block
  // fused selection (launch_logits_select): every row's chosen pools go
  // straight to its token row; no logits tile
  int32_t* out_tok;         // [q_end - q_begin, width]
  int32_t* out_ids;         // [q_end - q_begin, k_sel] global pool ids, or null
  int width, tail_on;
};
void launch_logits(const LogitsArgs& a, hipStream_t st);

// Scoring, pool top-k, expansion and tail of rows q_begin .. q_end-1 in one
// kernel: each workgroup keeps a running top-k_sel of every query's scores
// in LDS while it sweeps the pools, so no score leaves the chip. Returns
// false (and launches nothing) for shapes whose per-query LDS list cannot
// hold k_sel entries with room to spare; the caller then takes the tile path.
bool logits_select_supported(int H, int D, int fp8, int k_sel);
int logits_select_max_ksel(int H, int D, int fp8);
void launch_logits_select(const LogitsArgs& a, hipStream_t st);

// Pool top-k of rows q_begin .. q_end-1 from a logits tile; writes the pool
// ids (out_ids, may be null) and/or the expanded token rows with the tail
// (out_tok, may be null), both indexed by row - q_begin.
void launch_select(const float* logits, int64_t ld, int q_begin, int q_end,
                   const int32_t* cu, const int32_t* cu_pools, int B, int T, int kpool,
                   int k_sel, int width, int tail_on, int max_pools, int32_t* out_ids,
                   int32_t* out_tok, hipStream_t st);

// The same on two row ranges in one launch (out_ids / out_tok indexed by the
// global row t).
void launch_select2(const float* logits, int64_t ld, int q_begin, int q_end,
                    const float* logits2, int64_t ld2, int q_begin2, int q_end2,
                    const int32_t* cu, const int32_t* cu_pools, int B, int T, int kpool,
                    int k_sel, int width, int tail_on, int max_pools, int32_t* out_ids,
                    int32_t* out_tok, hipStream_t st);

void launch_expand(const int32_t* pool_ids, int q_begin, int q_end, const int32_t* cu,
                   const int32_t* cu_pools, int B, int T, int kpool, int k_sel, int width,
                   int tail, int max_pools, int32_t* out, hipStream_t st);

// Decode: one query per sequence b (its token seq_lens[b] - 1) against the
// sequence's floor(seq_lens[b] / kpool) cached pools at pooled rows
// pool_start[b] ...; scores to out [B, ld].
struct DecodeLogitsArgs {
  const void* q;               // BF16 [B, H, D] (the FP8 kernel quantises the rows)
  const float* w;              // FP32 [B, H]
  const void* keys;            // BF16 [pooled_rows, D], or E4M3 codes [pooled_rows, 128]
  const float* k_scale;        // FP8: FP32 [pooled_rows] row scales, else null
  int pooled_rows;             // reads are clamped into this many rows
  int fp8;
  const int32_t* pool_start;   // [B]
  const int32_t* seq_lens;     // [B]
  int B, H, D, kpool, max_pools;
  float scale;
  float* out;                  // FP32 [B, ld]
  int64_t ld;
  int pieces;                  // set by the launcher
};
void launch_decode_logits(const DecodeLogitsArgs& a, hipStream_t st);

// Selection + expansion of decode rows: row r is the query of sequence r
// (length seq_lens[r], pools at pool_start[r], token ids from token_base[r],
// or 0 when token_base is null).
void launch_select_decode(const float* scores, int64_t ld, int B, const int32_t* seq_lens,
                          const int32_t* pool_start, const int32_t* token_base, int kpool,
                          int k_sel, int width, int tail_on, int max_pools, int32_t* out_ids,
                          int32_t* out_tok, hipStream_t st);

// Compression of N complete pools given their slot tokens: pool n is tokens
// n kpool .. n kpool + kpool - 1 of k / gate, written to pooled row
// dst_rows[n] (rows outside [0, dst_cap) are skipped). With row_scale (D =
// 128), the rows are E4M3 codes of the FP8 input path instead (pooled viewed
// as uint8 [dst_cap, 128]) and their scales go to row_scale.
void launch_compress_pools(const uint16_t* k, const uint16_t* gate, const float* ape, int N,
                           int D, int kpool, const int32_t* dst_rows, int dst_cap,
                           uint16_t* pooled, float* row_scale, hipStream_t st);

// The indexer projections (head_dim 128): q = qr wq_b^T, k = LayerNorm(x
// wk^T), gate = x wg^T (BF16), w = x ww^T (FP32); w3 is device scratch of
// 128 x hidden BF16 for the split of ww.
struct ProjArgs {
  const uint16_t* x;        // BF16 [T, hidden]
  const uint16_t* qr;       // BF16 [T, q_lora]
  const uint16_t* wq_b;     // BF16 [H*128, q_lora]
  const uint16_t* wk;       // BF16 [128, hidden]
  const float* ln_w;        // FP32 [128]
  const float* ln_b;        // FP32 [128]
  const uint16_t* wg;       // BF16 [128, hidden]
  const float* ww;          // FP32 [H, hidden]
  uint16_t* w3;             // scratch BF16 [128, hidden]
  int T, hidden, q_lora, H;
  float eps;
  uint16_t* q;              // BF16 [T, H*128]
  uint16_t* k;              // BF16 [T, 128]
  uint16_t* gate;           // BF16 [T, 128]
  float* w;                 // FP32 [T, H]
};
void launch_indexer_projections(const ProjArgs& p, hipStream_t st);

// Sparse attention of the NoPE absorbed MLA (latent width 512, key = value).
struct MlaArgs {
  const uint16_t* q;        // BF16 [T, H, 512]
  const uint16_t* kv;       // BF16 [N, 512]
  const int32_t* idx;       // int32 [T, W]
  uint16_t* out;            // BF16 [T, H, 512]
  float* lse;               // FP32 [T, H]
  int T, H, N, W;
  float scale2;             // sm_scale * log2(e)
};
int mla_lds_bytes();
hipError_t launch_sparse_mla(const MlaArgs& m, hipStream_t st);

// Violation bits of the cu_seqlens check (the values of the header's
// KPOOL_CU_* constants).
constexpr int kCuFirstNotZero = 1, kCuDecreasing = 2, kCuTooLong = 4, kCuLastNotTotal = 8;
hipError_t launch_check_cu_seqlens(const int32_t* cu, int B, int T, int max_seqlen, int32_t* out,
                                   hipStream_t stream);

// Largest max_pools the selection kernel handles (its LDS bitmap has one bit
// per pool of a row).
constexpr int kMaxSelectPools = 65536;

}  // namespace kpool
