/*
 * kpool.h -- C ABI of the KPool DSA indexer on AMD MI355X (gfx950).
 *
 * The indexer picks, for every query of a packed (THD) batch, the earlier
 * tokens its sparse attention will read. The method is the KPool indexer of
 * GLM-5.3-Flash as described on three pull-request pages, cited here by title
 * and section:
 *   [MLM] Megatron-LM PR #7054 "GLM5.3 Flash (KDA + mHC + KPool DSA) support +
 *         FP8", section "3. KPool DSA indexer + NoPE";
 *   [SKY] SkyRL PR #2179 "GLM-5.3-Flash (glm5_next) support", the commit
 *         that adopts the k-pool indexer and "Limitations / follow-ups";
 *   [XT]  xtuner PR #2108 "Add GLM-5.3-Flash F5: NoPE DSA + KPool indexer +
 *         clamped SwiGLU", "Summary" and the F5 commit message.
 *
 * Notation. B documents, cu_seqlens cu[0..B] (int32, cu[0] = 0, cu[B] = T,
 * non-decreasing). Document b holds tokens cu[b] .. cu[b+1]-1, length L_b.
 * P_b = floor(L_b / kpool) complete pools; cu_pools cuP[b] = sum_{b'<b} P_b';
 * P = cuP[B]. For token t of document b, i = t - cu[b] is its position,
 * n_c(t) = floor((i + 1) / kpool) its causal pools (pools whose tokens are all
 * at or before t), K_sel = index_topk / kpool (integer division), W =
 * index_topk + kpool the output row width, and tail(t) = (i + 1) mod kpool
 * when always_select_tail is set, else 0. max_pools = floor(max_seqlen / kpool).
 *
 * Memory. Every pointer is device memory owned by the caller unless stated
 * otherwise. The library never allocates, frees or synchronises: work is
 * enqueued on `stream` (a hipStream_t passed as void*; NULL = the null
 * stream) and the caller synchronises. BF16 tensors are passed as raw 16-bit
 * words. Outputs are overwritten in full, padding included.
 *
 * Errors. Every entry point checks its arguments before enqueuing anything;
 * on failure it enqueues nothing, leaves the outputs untouched and returns a
 * status, with a description in kpool_last_error() (per calling thread). A
 * launch failure reported by the HIP runtime returns KPOOL_E_LAUNCH.
 * Pointers must be 16-byte aligned, except the int32 and FP32 arrays
 * cu_seqlens, cu_pools, w, row_scale, pooled_scale, dst_rows, pool_start,
 * seq_lens, token_base and out_pool_idx, which need 4-byte alignment (ape,
 * read 16 bytes at a time, needs 16). The contents of cu_seqlens are a
 * precondition that the host cannot see: for contents that break it, outputs are
 * unspecified, but every kernel keeps its reads and writes inside the
 * documented extents of the buffers.
 */
#ifndef KPOOL_H_
#define KPOOL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KPOOL_ABI_VERSION 1

typedef enum {
  KPOOL_OK = 0,
  KPOOL_E_INVALID = 1,      /* null / misaligned pointer, inconsistent sizes   */
  KPOOL_E_UNSUPPORTED = 2,  /* a valid shape this library has no kernel for    */
  KPOOL_E_WORKSPACE = 3,    /* workspace smaller than kpool_workspace_bytes()  */
  KPOOL_E_LAUNCH = 4        /* the HIP runtime reported an error               */
} kpool_status;

typedef struct {
  int32_t num_docs;           /* B >= 1                                            */
  int32_t total_tokens;       /* T >= 0, equals cu_seqlens[B]                      */
  int32_t max_seqlen;         /* >= every L_b; sets max_pools and the tile width   */
  int32_t num_heads;          /* H in {4, 8, 16, 32, 64}                           */
  int32_t head_dim;           /* D in {64, 128}; the FP8 path needs D == 128       */
  int32_t kpool;              /* 1 .. 64                                           */
  int32_t index_topk;         /* >= kpool                                          */
  int32_t always_select_tail; /* 0 / 1                                             */
  int32_t use_fp8;            /* 0 / 1: FP8 input path                             */
  int32_t query_chunk;        /* query rows per logits tile; 0 = as many as fit a  */
                              /* 256 MiB tile (kpool_query_chunk_rows)             */
  float   scale;              /* score scale inside the ReLU; 0 = head_dim^-1/2    */
} kpool_params;

/* KPOOL_ABI_VERSION of the built library. */
int kpool_abi_version(void);

/* Bytes of device workspace kpool_indexer_topk and kpool_logits need for
 * these parameters (0 when T == 0). The workspace holds, with use_fp8, the
 * E4M3 codes and row scales of q and of the pooled keys, then the FP32
 * logits tile of kpool_query_chunk_rows x kpool_logits_ld floats. It is
 * also enough for kpool_indexer_topk_fused. */
size_t kpool_workspace_bytes(const kpool_params* p);

/* Row stride, in floats, of the logits tiles of kpool_logits / kpool_select:
 * max_pools rounded up to a multiple of 64. */
int64_t kpool_logits_ld(const kpool_params* p);

/* Query rows per logits tile of kpool_indexer_topk: query_chunk when
 * it is set, else floor(256 MiB / (4 * kpool_logits_ld(p))), capped at T
 * (0 when T == 0 or the parameters are invalid). */
int32_t kpool_query_chunk_rows(const kpool_params* p);

/* Step 1, key compression ([MLM] section 3; [SKY] k-pool commit). For each
 * document b, pool p < P_b and dimension d, with slot tokens
 * t_s = cu[b] + p*kpool + s:
 *   a_s = gate[t_s, d] + ape[s, d]                (FP32)
 *   pooled[cuP[b] + p, d] = BF16( sum_s softmax_s(a)[s] * k[t_s, d] )
 * with FP32 accumulation and round-to-nearest-even to BF16. Pools restart at
 * every document; a document's last L_b mod kpool tokens form no pool.
 *   k, gate     BF16 [T, D] row-major
 *   ape         FP32 [kpool, D]
 *   cu_seqlens  int32 [B + 1]
 *   cu_pools    out int32 [B + 1] (cuP)
 *   pooled      out BF16 [floor(T / kpool), D]; rows P.. are not written
 * Uses params: num_docs, total_tokens, head_dim, kpool. */
kpool_status kpool_compress(const kpool_params* p, const void* k, const void* gate,
                            const float* ape, const int32_t* cu_seqlens,
                            int32_t* cu_pools, void* pooled, void* stream);

/* Steps 2-4 for every query of the batch ([MLM] section 3; [SKY] limitations;
 * [XT] summary and F5 commit):
 *   score[t, p] = sum_h w[t, h] * ReLU(scale * q[t, h, :] . pooled[p, :])
 * over the causal pools p = cuP[b] .. cuP[b] + n_c(t) - 1 of t's document;
 * the min(K_sel, n_c(t)) best pools (ties to the lower pool id) are expanded,
 * in ascending pool order, to their kpool tokens, followed by the tail(t)
 * tokens cu[b] + n_c(t)*kpool .. t, then -1 up to width W. Query rows go
 * kpool_query_chunk_rows at a time (a chunk) through a logits tile in the
 * workspace ([XT] summary: chunking bounds the tile): the launches that
 * kpool_indexer_launches lists, each the scoring kernel of kpool_logits over
 * one chunk, or over a long and a short chunk that fit the tile together at
 * their own row strides, then the selection + expansion kernel of
 * kpool_select_expand on each of its chunks.
 * With use_fp8 the q rows (t, h) and the pooled rows first go through the FP8
 * input path of kpool_fp8_quantize and are scored from their E4M3 codes and
 * power-of-two scales.
 *   q          BF16 [T, H, D]
 *   w          FP32 [T, H]
 *   pooled     BF16 [floor(T / kpool), D] as written by kpool_compress
 *   cu_pools   int32 [B + 1] as written by kpool_compress
 *   workspace  at least kpool_workspace_bytes(p) bytes, 256-byte aligned
 *   out_token_idx  out int32 [T, W]: global token indices, ascending, -1 pad
 *   out_pool_idx   out int32 [T, K_sel] (may be NULL): global pool ids,
 *                  ascending, -1 pad */
kpool_status kpool_indexer_topk(const kpool_params* p, const void* q, const float* w,
                                const void* pooled, const int32_t* cu_seqlens,
                                const int32_t* cu_pools, void* workspace,
                                size_t workspace_bytes, int32_t* out_token_idx,
                                int32_t* out_pool_idx, void* stream);

/* kpool_indexer_topk one launch at a time, for callers that interleave other
 * work with the chunks or time the two kernels apart.
 *
 * kpool_indexer_launches returns the number of scoring launches the indexer
 * makes (0 when T == 0 or the parameters are invalid) and, when info is not
 * NULL, writes the first min(count, max_launches) of them as six int32 each:
 *   {a0, a1, lda, b0, b1, ldb}
 * launch i scores query rows a0 .. a1-1 into the workspace's logits tile
 * with row stride lda floats, then rows b0 .. b1-1 (none when b0 == b1)
 * right after them with row stride ldb. Every row stride is at least the
 * largest causal pool count of its rows, rounded up to 64 (a row t has at
 * most (t + 1) / kpool pools); the two ranges fit the tile together. Every
 * query row belongs to exactly one range of one launch.
 *
 * kpool_indexer_scoring enqueues launch i's scoring kernel (rows with
 * n_c(t) <= K_sel are left unwritten, as the indexer does). With use_fp8 it
 * first quantises the launch's q rows and all pooled keys into the
 * workspace, unless flags holds KPOOL_LOGITS_INPUTS_QUANTIZED (the workspace
 * already holds them; no other flag is accepted).
 * kpool_indexer_selection enqueues the selection + expansion of launch i's
 * rows from the tile; it writes rows a0 .. a1-1 and b0 .. b1-1 of
 * out_token_idx [T, W] (16-byte aligned) and, if not NULL, of out_pool_idx
 * [T, K_sel]. Scoring then selection of every launch, in any launch order
 * but each selection after its own scoring and before the next scoring,
 * writes what kpool_indexer_topk writes. Arguments as for
 * kpool_indexer_topk; both return KPOOL_E_INVALID for a launch index outside
 * [0, count). */
int32_t kpool_indexer_launches(const kpool_params* p, int32_t* info, int32_t max_launches);
kpool_status kpool_indexer_scoring(const kpool_params* p, int32_t launch, const void* q,
                                   const float* w, const void* pooled,
                                   const int32_t* cu_seqlens, const int32_t* cu_pools,
                                   void* workspace, size_t workspace_bytes, int32_t flags,
                                   void* stream);
kpool_status kpool_indexer_selection(const kpool_params* p, int32_t launch,
                                     const int32_t* cu_seqlens, const int32_t* cu_pools,
                                     const void* workspace, size_t workspace_bytes,
                                     int32_t* out_token_idx, int32_t* out_pool_idx,
                                     void* stream);

/* Steps 2-4 in one kernel per query chunk, with the same arguments and the
 * same output as kpool_indexer_topk, bit for bit ([MLM] section 3 names a
 * fused scoring + top-k + expansion op). Each workgroup keeps a running top
 * K_sel of each of its queries' scores in LDS while the pools stream past
 * (exact selection when a candidate list fills, then a higher entry
 * threshold), so no score is written to memory. Needs K_sel to fit the
 * per-query candidate list: K_sel <= kpool_fused_max_ksel(p) (1184 at
 * H = 32, D = 128; 1344 with use_fp8; fewer with fewer heads, whose
 * workgroups hold more queries). Otherwise it returns KPOOL_E_UNSUPPORTED
 * and enqueues nothing. The
 * workspace holds only the FP8 codes and scales:
 * kpool_fused_workspace_bytes(p) bytes (0 without use_fp8, and 0 when the
 * shape is unsupported; the pointer may then be NULL). */
int32_t kpool_fused_max_ksel(const kpool_params* p);      /* uses H, D, use_fp8 */
size_t kpool_fused_workspace_bytes(const kpool_params* p);
kpool_status kpool_indexer_topk_fused(const kpool_params* p, const void* q, const float* w,
                                      const void* pooled, const int32_t* cu_seqlens,
                                      const int32_t* cu_pools, void* workspace,
                                      size_t workspace_bytes, int32_t* out_token_idx,
                                      int32_t* out_pool_idx, void* stream);

/* Step 2 alone, for query rows q_begin .. q_end-1 (0 <= q_begin <= q_end <= T):
 *   out[r, j] = score of row t = q_begin + r against doc-local pool j of t's
 *               document, for j < n_c(t)
 * (row stride ld = kpool_logits_ld(p) floats). Same scoring as
 * kpool_indexer_topk, including the FP8 path (whose quantised q rows and keys
 * are written to the workspace first). flags:
 *   KPOOL_LOGITS_FILL_MASKED  also write -inf in columns n_c(t) .. ld-1
 *   KPOOL_LOGITS_SKIP_ALL_SELECTED  rows whose n_c(t) <= K_sel may be left
 *       unwritten (their selection takes every pool); this is the launch
 *       kpool_indexer_topk makes for each query chunk.
 *   KPOOL_LOGITS_INPUTS_QUANTIZED  (use_fp8 only) the workspace already
 *       holds the E4M3 codes and scales of q rows q_begin .. q_end-1 and of
 *       the pooled keys, as an earlier kpool_logits or kpool_indexer_topk
 *       call with the same parameters, inputs and workspace left them; the
 *       quantisation is skipped and only the scoring kernel runs.
 * Columns and rows not covered by the flags are left untouched. */
#define KPOOL_LOGITS_FILL_MASKED 1
#define KPOOL_LOGITS_SKIP_ALL_SELECTED 2
#define KPOOL_LOGITS_INPUTS_QUANTIZED 4
kpool_status kpool_logits(const kpool_params* p, const void* q, const float* w,
                          const void* pooled, const int32_t* cu_seqlens,
                          const int32_t* cu_pools, int32_t q_begin, int32_t q_end,
                          void* workspace, size_t workspace_bytes, float* out,
                          int32_t flags, void* stream);

/* Step 3 alone: for rows r of a logits tile laid out as kpool_logits writes it
 * (row stride kpool_logits_ld(p)), the min(K_sel, n_c(t)) largest scores of
 * columns 0 .. n_c(t)-1, t = q_begin + r; larger score first, equal scores to
 * the lower column, NaN ranks as -inf. Writes global pool ids cuP[b] + j in
 * ascending order, -1 padded, to out_pool_idx [q_end - q_begin, K_sel]. */
kpool_status kpool_select(const kpool_params* p, const float* logits, int32_t q_begin,
                          int32_t q_end, const int32_t* cu_seqlens,
                          const int32_t* cu_pools, int32_t* out_pool_idx, void* stream);

/* Steps 3 and 4 together, as kpool_indexer_topk runs them on each query
 * chunk: the selection of kpool_select on rows q_begin .. q_end-1 of a
 * logits tile, written directly as token rows (the expansion and tail of
 * kpool_expand) to out_token_idx [q_end - q_begin, W] and, when
 * out_pool_idx is not NULL, as pool ids to out_pool_idx
 * [q_end - q_begin, K_sel]. out_token_idx must be 16-byte aligned. */
kpool_status kpool_select_expand(const kpool_params* p, const float* logits, int32_t q_begin,
                                 int32_t q_end, const int32_t* cu_seqlens,
                                 const int32_t* cu_pools, int32_t* out_pool_idx,
                                 int32_t* out_token_idx, void* stream);

/* Step 4 alone, for every query t: expands the pool ids of row t of pool_idx
 * [T, K_sel] (global ids, ascending, -1 padded, min(K_sel, n_c(t)) valid) to
 * kpool consecutive tokens each and appends the tail:
 *   out[t, j] = cu[b] + (id - cuP[b])*kpool + (j mod kpool),
 *               id = pool_idx[t, j / kpool],           j < kpool*n_sel
 *   then the tail(t) tokens cu[b] + n_c(t)*kpool .. t, then -1 to width W. */
kpool_status kpool_expand(const kpool_params* p, const int32_t* pool_idx,
                          const int32_t* cu_seqlens, const int32_t* cu_pools,
                          int32_t* out_token_idx, void* stream);

/* FP8 input path ([MLM] section 3) for `rows` rows of 128 BF16 values:
 *   y = BF16( FWHT_128(x) * FP32(128^-1/2) )   FP32 butterflies, stages
 *        h = 1, 2, ..., 64, (a, b) -> (a + b, a - b), Sylvester order
 *   e = min{ e integer : max|y| <= 448 * 2^e } (0 for an all-zero row)
 *   codes = E4M3 (OCP e4m3fn, round to nearest even, subnormals kept) of
 *           y * 2^-e;  row_scale = 2^e
 *   x      BF16 [rows, 128];  codes out uint8 [rows, 128];
 *   row_scale out FP32 [rows]. */
kpool_status kpool_fp8_quantize(const void* x, int32_t rows, uint8_t* codes,
                                float* row_scale, void* stream);

/* ---- Serving: one query per sequence, pooled keys kept in a cache -------
 * ([MLM] sections 3 and 4: the indexer of the serving path scores pools of
 * keys compressed as tokens arrive, with an FP8 key store.) A sequence of L
 * tokens holds its floor(L / kpool) complete pools in the caller's cache of
 * pooled rows; its query is its token L - 1, whose indexer row is the one
 * kpool_indexer_topk computes for the last token of a document of L tokens.
 * The cache holds BF16 rows [pooled_rows, D], or with use_fp8 the E4M3 codes
 * [pooled_rows, 128] (uint8) and power-of-two scales [pooled_rows] (FP32)
 * that kpool_fp8_quantize gives the BF16 rows.
 *
 * kpool_compress_pools: step 1 for pools that have just completed, given by
 * their slot tokens. Pool n of the call is tokens n*kpool .. n*kpool+kpool-1
 * of k and gate; its pooled key (the same arithmetic as kpool_compress) goes
 * to row dst_rows[n] of the cache (with use_fp8: its codes and scale, the
 * FP8 input path applied to the BF16 pooled row); rows outside
 * [0, pooled_rows) are skipped.
 *   k, gate    BF16 [num_pools * kpool, D]
 *   ape        FP32 [kpool, D]
 *   dst_rows   int32 [num_pools]
 *   pooled     BF16 [pooled_rows, D], or uint8 codes [pooled_rows, 128]
 *   pooled_scale  FP32 [pooled_rows] with use_fp8, else ignored (may be NULL)
 * Uses params: head_dim, kpool, use_fp8 (which needs head_dim == 128). */
kpool_status kpool_compress_pools(const kpool_params* p, const void* k, const void* gate,
                                  const float* ape, int32_t num_pools, const int32_t* dst_rows,
                                  int32_t pooled_rows, void* pooled, float* pooled_scale,
                                  void* stream);

/* Bytes of workspace kpool_decode_topk needs (0 for invalid parameters):
 * the scores of every sequence, B rows of kpool_logits_ld floats. */
size_t kpool_decode_workspace_bytes(const kpool_params* p);

/* Steps 2-4 for B = num_docs sequences, one query each. Sequence b has
 * L_b = seq_lens[b] tokens (0 <= L_b <= max_seqlen; 0: an all -1 row); its
 * n_c = floor(L_b / kpool) complete pools are pooled rows pool_start[b] ..
 * pool_start[b] + n_c - 1, and its token ids start at token_base[b] (0 when
 * token_base is NULL). Row b of the outputs:
 *   score[j] = sum_h w[b, h] * ReLU(scale * q[b, h, :] . pooled[pool_start[b] + j, :])
 *   for j < n_c; the min(K_sel, n_c) best (ties to the lower j), expanded
 *   in ascending order to token_base[b] + j*kpool + s, s < kpool; then the
 *   tail token_base[b] + n_c*kpool .. token_base[b] + L_b - 1 (when
 *   always_select_tail); then -1 to width W.
 *   q           BF16 [B, H, D]
 *   w           FP32 [B, H]
 *   pooled      the cache, BF16 [pooled_rows, D] or (use_fp8) E4M3 codes
 *               [pooled_rows, 128]; reads are kept inside it, and the rows
 *               named above must lie in it for a meaningful result
 *   pooled_scale  FP32 [pooled_rows] with use_fp8 (may be NULL otherwise)
 *   pool_start, seq_lens  int32 [B];  token_base  int32 [B] or NULL
 *   workspace   at least kpool_decode_workspace_bytes(p) bytes, 256-byte aligned
 *   out_token_idx  out int32 [B, W];  out_pool_idx  out int32 [B, K_sel]
 *               (may be NULL): pool_start[b] + j, ascending, -1 pad
 * With use_fp8 the q rows (b, h) go through the FP8 input path (inside the
 * scoring kernel) and are scored from their codes against the cached key
 * codes, as kpool_indexer_topk's FP8 path scores them.
 * Uses params: num_docs (= B), max_seqlen (a bound on every L_b), num_heads,
 * head_dim, kpool, index_topk, always_select_tail, use_fp8 (head_dim 128),
 * scale; total_tokens and query_chunk are not used.
 * Lengths above max_seqlen are scored over their first floor(max_seqlen /
 * kpool) pools. */
kpool_status kpool_decode_topk(const kpool_params* p, const void* q, const float* w,
                               const void* pooled, int32_t pooled_rows,
                               const float* pooled_scale, const int32_t* pool_start,
                               const int32_t* seq_lens, const int32_t* token_base,
                               void* workspace, size_t workspace_bytes,
                               int32_t* out_token_idx, int32_t* out_pool_idx, void* stream);

/* ---- The indexer projections -------------------------------------------
 * ([MLM] section 4, the DSA indexer's forward and its precision split;
 * section 3, the per-token compression gate.) The four inputs of the
 * indexer for T tokens, from the layer input x and the query latent qr:
 *   q    = BF16(qr wq_b^T)                  [T, H*D], read as [T, H, D]
 *   k    = BF16(LayerNorm(BF16(x wk^T)))    [T, D]   (k_norm, FP32 inside)
 *   gate = BF16(x wg^T)                     [T, D]   (compression gate logits)
 *   w    = x ww^T in FP32                   [T, H]   (head weights)
 * with FP32 accumulation and round-to-nearest-even. LayerNorm over the D
 * values of a row: (v - mean) / sqrt(var + eps) * k_norm_weight +
 * k_norm_bias, var the mean squared deviation. No rotary embedding (the
 * NoPE indexer) and no activation rotation. The gate is read as a linear
 * map of x (the pages name the parameter, not its shape).
 *   x   BF16 [T, hidden];  qr BF16 [T, q_lora_rank]
 *   wq_b BF16 [H*D, q_lora_rank];  wk, wg BF16 [D, hidden] (row = output)
 *   k_norm_weight, k_norm_bias FP32 [D];  ww FP32 [H, hidden]
 *   workspace  kpool_proj_workspace_bytes(pp) bytes, 256-byte aligned
 *   q_out, k_out, gate_out  BF16 outputs;  w_out FP32 [T, H]
 * Needs head_dim == 128, num_heads in {4, 8, 16, 32}, hidden and
 * q_lora_rank multiples of 64. */
typedef struct {
  int32_t num_tokens;       /* T >= 0                                        */
  int32_t hidden;           /* width of x                                    */
  int32_t q_lora_rank;      /* width of qr                                   */
  int32_t num_heads;        /* H                                             */
  int32_t head_dim;         /* D (128)                                       */
  float   eps;              /* LayerNorm epsilon; 0 = 1e-6                   */
} kpool_proj_params;
size_t kpool_proj_workspace_bytes(const kpool_proj_params* pp);
kpool_status kpool_indexer_projections(const kpool_proj_params* pp, const void* x, const void* qr,
                                       const void* wq_b, const void* wk,
                                       const float* k_norm_weight, const float* k_norm_bias,
                                       const void* wg, const float* ww, void* workspace,
                                       size_t workspace_bytes, void* q_out, void* k_out,
                                       void* gate_out, float* w_out, void* stream);

/* ---- Debug check of the document offsets -------------------------------
 * ([MLM] section 3: pools restart at every document of the packed batch, so
 * cu_seqlens decides every pool's tokens.) The entry points that take
 * cu_seqlens assume, without checking its device-resident contents, that
 * cu_seqlens[0] = 0, that it never decreases, that no document is longer
 * than max_seqlen and that cu_seqlens[num_docs] = total_tokens. This call
 * checks exactly that on the device and writes, to the device int32
 * *flags_out, the OR of KPOOL_CU_* bits for the violations found (0 = the
 * offsets are valid). It reads cu_seqlens[0 .. num_docs] and writes
 * *flags_out only (no prior clearing needed); one small launch on `stream`.
 * KPOOL_E_INVALID for num_docs < 0, total_tokens < 0, max_seqlen < 0, or a
 * null or misaligned (4-byte) pointer. */
#define KPOOL_CU_FIRST_NOT_ZERO 1
#define KPOOL_CU_DECREASING 2
#define KPOOL_CU_TOO_LONG 4
#define KPOOL_CU_LAST_NOT_TOTAL 8
kpool_status kpool_check_cu_seqlens(const int32_t* cu_seqlens, int32_t num_docs,
                                    int32_t total_tokens, int32_t max_seqlen, int32_t* flags_out,
                                    void* stream);

/* ---- Sparse attention over the selected rows (the indices' consumer) ----
 * ([XT] "Summary": the sparse MLA backend runs FlashMLA's forward over the
 * indexer's int32 indices, with heads in multiples of 64; [XT] LSE fix
 * commit: the saved LSE is the natural logarithm; [MLM] section 3: NoPE, the
 * absorbed query has no positional slice.) For query token t and head h:
 *   s_j      = sm_scale * <q[t, h, :], kv[j, :]>   for each listed row j
 *   out[t,h] = sum_j softmax(s)_j * kv[j, :]        BF16 (round to nearest even)
 *   lse[t,h] = ln sum_j exp(s_j)                    FP32
 * kv holds one latent row per token, shared by every head, which is both
 * the key and the value (dim_qk = dim_v = 512). An entry of indices outside
 * [0, kv_rows) -- such as the indexer's -1 padding -- is unused; any other
 * entry is one softmax term (a row listed twice counts twice). A query with
 * no used entry gets out = 0 and lse = -inf. Scores and sums in FP32 from
 * BF16 products; the softmax weights are rounded to BF16 for the weighted
 * sum of the rows.
 *   q        BF16 [num_tokens, num_heads, 512], 16-byte aligned
 *   kv       BF16 [kv_rows, 512], 16-byte aligned
 *   indices  int32 [num_tokens, width] (e.g. kpool_indexer_topk's
 *            out_token_idx with width = index_topk + kpool), 4-byte aligned
 *   out      BF16 [num_tokens, num_heads, 512], 16-byte aligned
 *   lse      FP32 [num_tokens, num_heads], 4-byte aligned
 * Device pointers, owned by the caller; nothing is allocated. Needs
 * num_heads a positive multiple of 64, dim_qk = dim_v = 512 and width <=
 * 4096, else KPOOL_E_UNSUPPORTED; negative sizes or an sm_scale that is not finite
 * and positive give KPOOL_E_INVALID. Nothing is enqueued on an error. */
typedef struct {
  int32_t num_tokens;       /* T >= 0                                        */
  int32_t num_heads;        /* H, a positive multiple of 64                  */
  int32_t kv_rows;          /* N >= 0 rows in kv                             */
  int32_t width;            /* 0 <= W <= 4096 entries per query in indices  */
  int32_t dim_qk;           /* 512                                           */
  int32_t dim_v;            /* 512                                           */
  float   sm_scale;         /* score scale, finite and > 0                   */
} kpool_mla_params;
kpool_status kpool_sparse_mla_fwd(const kpool_mla_params* mp, const void* q, const void* kv,
                                  const int32_t* indices, void* out, float* lse, void* stream);

/* ---- For callers that cannot allocate ----------------------------------
 * For code that must not call hipMalloc (work captured in a HIP graph, tight
 * serving loops, hosts that forbid allocation): kpool_decode_topk with its
 * scores kept in a scratch array built into the library instead of a caller
 * workspace. The array holds kpool_decode_noalloc_max_bytes() bytes (32 MiB)
 * on each device the library runs on, from load until the process ends; a
 * call needs num_docs * kpool_logits_ld * 4 bytes of it (for example 512
 * sequences of up to 64K tokens at kpool 4) and fails with
 * KPOOL_E_WORKSPACE, enqueuing nothing, when that is more. The call
 * allocates no memory. Every call on one device uses the same array: calls
 * that overlap on one device (on different streams, or from several host
 * threads) race and their outputs are unspecified; calls ordered on one
 * stream are safe. Arguments and outputs are those of kpool_decode_topk. */
size_t kpool_decode_noalloc_max_bytes(void);
kpool_status kpool_decode_topk_noalloc(const kpool_params* p, const void* q, const float* w,
                                       const void* pooled, int32_t pooled_rows,
                                       const float* pooled_scale, const int32_t* pool_start,
                                       const int32_t* seq_lens, const int32_t* token_base,
                                       int32_t* out_token_idx, int32_t* out_pool_idx,
                                       void* stream);

/* Static description of a status code. */
const char* kpool_status_string(kpool_status s);

/* Detail of the last failure of the calling thread ("" if none). */
const char* kpool_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KPOOL_H_ */
