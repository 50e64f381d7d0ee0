// Step 2 of the KPool indexer: pool scores of a chunk of query rows.
//
//   score[t, j] = sum_h w[t, h] * ReLU(scale * q[t, h, :] . pooled[cuP[b] + j, :])
//
// for the causal pools j < n_c(t) of t's document. Megatron-LM PR #7054,
// section "3. KPool DSA indexer + NoPE" (top-k over pools, FP32 head weights);
// xtuner PR #2108, F5 commit (the DSA indexer score with head_dim^-1/2 inside
// the ReLU, which ReLU's positive homogeneity lets us fold into w) and
// "Summary" (the logits tile is bounded by query chunking).
//
// A dense contraction on MFMA: M = (query, head) rows, N = pools, K = D. A
// wave keeps MT row tiles of 32 (query, head) rows of q in registers for the
// whole launch (A operand) and sweeps the document's causal pools; a
// workgroup of NW waves shares each 64-pool tile of keys through LDS (B
// operand, rows padded by 16 bytes so the 16-byte lane reads of one pass hit
// distinct banks). The epilogue stays in registers: each lane holds 16 rows of
// one pool column of a 32 x 32 accumulator, multiplies by w' = w * scale,
// clamps at 0 and sums the heads of each query, then adds the other half-wave.
//
// bf16: v_mfma_f32_32x32x16_bf16. fp8: v_mfma_f32_32x32x64_f8f6f4 on E4M3
// codes; the row scales of q fold into w' and the key scales multiply the
// head sum (both are powers of two, so this is exact up to FP32 rounding).
//
// The K index is permuted identically for A and B (lane half g takes a
// contiguous slice of D), which leaves every dot product unchanged and lets a
// lane read one contiguous run of q and of each key row.

#include <algorithm>
#include <type_traits>

#include "kpool_device.h"
#include "kpool_internal.h"

namespace kpool {

// FP8 MFMA K: v_mfma_f32_32x32x64_f8f6f4 takes 64 K values per instruction.
constexpr int kFp8K = 64;

constexpr int kLogitsWaves = 8;
constexpr int kPoolTile = 64;                 // pools per LDS stage (two 32-wide MFMA units)
constexpr int kUnits = kPoolTile / 32;

template <int H, int D, bool FP8>
struct LogitsCfg {
  static constexpr int MT = 2;                       // 32-row tiles per wave
  static constexpr int QPW = 32 * MT / H;            // queries per wave (H <= 32)
  static constexpr int QPB = kLogitsWaves * (QPW > 0 ? QPW : 1);   // queries per workgroup
  static constexpr int ROWB = FP8 ? D : 2 * D;       // bytes per key row
  static constexpr int CPR = ROWB / 16;              // 16-byte chunks per key row
  static constexpr int TILE_BYTES = kPoolTile * ROWB;
  static constexpr int LPW = TILE_BYTES / (1024 * kLogitsWaves);   // 1 KB loads per wave
  static constexpr int A_BYTES = 32 * MT * ROWB;     // q rows of one wave
  static constexpr int KSTEP = FP8 ? kFp8K : 16;     // K per MFMA
  static constexpr int NSTEP = D / KSTEP;            // MFMAs per 32 x 32 tile
  static_assert(LPW >= 1 && LPW * 1024 * kLogitsWaves == TILE_BYTES, "tile split");
};

// LDS tile layout: key row r (0..63) occupies ROWB contiguous bytes; its
// 16-byte chunk c sits at chunk position c ^ f(r). A 16-byte lane read is
// served 16 lanes (256 bytes) per pass; the lanes of a pass read 16
// consecutive rows at one chunk, and f spreads them over 16 bank groups:
// 256-byte rows use f(r) = r & 15; 128-byte rows pair rows (r, r + 1) in one
// 256-byte line and use f(r) = (r >> 1) & 7.
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  return CPR == 16 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7));
}

// One gfx950 global_load_lds_dwordx4: lane l copies 16 bytes from src to
// block + 16 l, block being a 1 KB LDS block of this wave. Issued as inline
// asm (M0 saved and restored) so the compiler does not track it: its
// conservative tracking would wait for every outstanding store before each
// tile; the kernel waits for exactly the copies it needs instead (see step).
__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* block) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)block);
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(dst), "v"(src)
      : "memory");
}

// The same with 4 bytes per lane (global_load_lds_dword): lane l copies
// src to block + 4 l, block being a 256-byte LDS block of this wave.
__device__ __forceinline__ void dma4(const float* src, float* block) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)block);
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dword %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(dst), "v"(src)
      : "memory");
}

// Issue this wave's share of a key tile straight into LDS. Rows past the
// causal range read the last causal row instead: their scores are never
// stored. On the FP8 path wave 0 also copies the tile's 64 key scales, so
// the epilogue reads them from LDS: a global load there would make the
// compiler's wait for it also wait for the next tile's copy, which was issued
// before it (vector-memory operations complete in order).
template <int H, int D, bool FP8>
__device__ __forceinline__ void load_key_tile(const uint8_t* __restrict__ keys, int pool0, int j0,
                                              int maxnc, uint8_t* lds, int wid, int lane,
                                              const float* __restrict__ kscale = nullptr,
                                              float* sbuf = nullptr) {
  using C = LogitsCfg<H, D, FP8>;
  if constexpr (FP8) {
    if (wid == 0) {
      const int jr = j0 + lane < maxnc ? j0 + lane : maxnc - 1;
      dma4(kscale + pool0 + jr, sbuf);
    }
  }
#pragma unroll
  for (int i = 0; i < C::LPW; ++i) {
    const int L = (wid * C::LPW + i) * 64 + lane;     // LDS chunk index
    const int r = L / C::CPR, pos = L % C::CPR;
    const int c = swz<C::CPR>(r, pos);
    const int jr = j0 + r < maxnc ? j0 + r : maxnc - 1;
    dma16(keys + (size_t)(pool0 + jr) * C::ROWB + c * 16, lds + (wid * C::LPW + i) * 1024);
  }
}

// Issue this wave's 64 rows of q (contiguous in memory from row0) into its
// LDS staging block, one coalesced 1 KB copy per instruction, with the key
// tiles' chunk swizzle so that the fragment reads are conflict-free. Rows
// past row_last (queries past the launch) read row_last instead; their
// fragments are zeroed after the read.
template <int H, int D, bool FP8>
__device__ __forceinline__ void load_q_rows(const uint8_t* __restrict__ q, size_t row0,
                                            size_t row_last, uint8_t* lds, int lane) {
  using C = LogitsCfg<H, D, FP8>;
#pragma unroll
  for (int i = 0; i < C::A_BYTES / 1024; ++i) {
    const int L = i * 64 + lane;
    const int r = L / C::CPR, pos = L % C::CPR;
    const int c = swz<C::CPR>(r, pos);
    const size_t row = row0 + r < row_last ? row0 + r : row_last;
    dma16(q + row * C::ROWB + c * 16, lds + i * 1024);
  }
}

// ReLU as an integer max on the encoding: non-negative floats (and +0) are
// non-negative integers, negative floats and -0 are negative integers. One
// VALU op and no NaN canonicalisation, unlike fmaxf.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0), leaving expcnt / lgkmcnt unconstrained
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

// s_waitcnt vmcnt(N): wait until at most N vector-memory instructions of this
// wave are outstanding. They complete in issue order, so this waits for
// everything issued before the last N. The counter field holds at most 63;
// a larger N waits for 63, which only waits for more.
template <int N>
__device__ __forceinline__ void wait_vmem_leave() {
  static_assert(N >= 0, "vmcnt range");
  constexpr int M = N < 63 ? N : 63;
  __builtin_amdgcn_s_waitcnt(0x0f70 | (M & 15) | ((M >> 4) << 14));
}

// Output slots of one lane per 32-pool unit: the queries whose score for pool
// column n of the unit this lane stores.
template <int H>
struct OutSlots {
  static constexpr int MT = 2;
  static constexpr int N = H == 4 ? MT * 4 : (H == 64 ? 1 : MT * (32 / H) / 2);
  // query (within the wave) of slot k for half-wave g
  __device__ static int query(int k, int g) {
    if constexpr (H == 4) return (k >> 2) * 8 + 2 * (k & 3) + g;   // k = mt * 4 + J
    else if constexpr (H == 64) return 0;
    else return 2 * k + g;
  }
};

// Fused selection: LDS left for the per-query candidate lists once the two
// key tiles and the small per-query arrays are placed, and the entries each
// list holds (6 bytes each: the score's bits and a 16-bit pool index).
template <int H, int D, bool FP8>
struct SelCfg {
  using C = LogitsCfg<H, D, FP8>;
  static constexpr int SMALL = C::QPB * 4 * 8 + 1280 + 32 * 6 + (FP8 ? 512 : 0);
  static constexpr int BUDGET = 160 * 1024 - 2 * C::TILE_BYTES - SMALL;
  // at most 24 entries per lane while a list is ranked (its keys stay in
  // registers beside the operands the sweep holds)
  static constexpr int CAP_LDS = (BUDGET / (C::QPB * 6)) & ~7;
  static constexpr int CAP = CAP_LDS < 1536 ? CAP_LDS : 1536;
  // a wave asks for a shrink once one of its lists has passed TRIGGER. From
  // the last check a list passed (count <= TRIGGER), or from a shrink (count
  // <= k_sel + slack), to the next shrink two step starts after a failed
  // check, a list takes at most two steps of two 32-pool units and its run's
  // last unit: 160 entries; a unit's stores reach 31 positions past its count.
  // So TRIGGER + 160 <= CAP and k_sel + slack + 160 <= CAP.
  static constexpr int TRIGGER = CAP - 160;
};

__device__ __forceinline__ float key_to_f32(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Top-k shrink of one candidate list of cnt > k entries, whole wave.
// Entries are in ascending pool order (the sweep appends them in that
// order), so "equal scores to the lower pool" is "equal scores to the
// earlier entry". A threshold key theta with at least k keys >= theta is
// found by bisection over the bits where the list's smallest and largest
// keys differ; counts come from ballots (scalar popcounts), so each step is
// one vector compare per slot. The bisection stops once k to k + slack keys
// reach the candidate; with slack 0 (the final selection) it ends either
// there or at the k-th largest key. The list is compacted in place, order
// kept: every entry above theta, and entries equal to theta up to a total
// of k + slack when they fit, else only the first k - #(above) of them. So
// the kept entries include the exact top k. Returns theta (a later entry, of
// a higher pool, can belong to the top k only if its key exceeds theta) and
// the number kept.
template <int CAP>
__device__ __forceinline__ uint32_t list_select(uint32_t* __restrict__ lval,
                                                uint16_t* __restrict__ lidx, int cnt, int k,
                                                int slack, int lane, int& kept_out) {
  constexpr int SL = (CAP + 63) / 64;
  static_assert(SL <= 64, "list slots per lane");
  uint32_t kv[SL];
  uint64_t vmask = 0u;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int s = 0; s < SL; ++s) {
    const int e = s * 64 + lane;
    const bool valid = e < cnt;
    const uint32_t key = valid ? f32_order_key(__uint_as_float(lval[valid ? e : 0])) : 0u;
    kv[s] = key;                                      // invalid slots hold 0 (below every key)
    vmask |= valid ? (1ull << s) : 0ull;
    kmin = valid && key < kmin ? key : kmin;
    kmax = valid && key > kmax ? key : kmax;
  }
  kmin = wave_min(kmin);
  kmax = wave_max(kmax);
  // #(keys >= c) over the list, wave-uniform (for c >= 1 invalid slots never count)
  auto count_ge = [&](uint32_t c) {
    int n = 0;
#pragma unroll
    for (int s = 0; s < SL; ++s) n += __popcll(__ballot(kv[s] >= c));
    return n;
  };
  // theta lies in [kmin, kmax], so it shares their common leading bits
  const int free_bits = kmin == kmax ? 0 : 32 - __clz(kmin ^ kmax);
  uint32_t th = free_bits >= 32 ? 0u : (kmin >> free_bits) << free_bits;
  int n_ge = cnt;                                     // #(keys >= th)
  for (int b = free_bits - 1; b >= 0; --b) {
    const uint32_t cand = th | (1u << b);
    const int c = count_ge(cand);
    if (c >= k) {
      th = cand;
      n_ge = c;
      if (c <= k + slack) break;
    }
  }
  int above = 0;
#pragma unroll
  for (int s = 0; s < SL; ++s) above += __popcll(__ballot(((vmask >> s) & 1u) && kv[s] > th));
  const int keep_eq = (n_ge <= k + slack ? n_ge : k) - above;
  // compaction: slot s writes only positions below 64 (s + 1), so the pool
  // indices of a later batch of slots can be read before this batch writes
  int eq_seen = 0, kept = 0;
  constexpr int BATCH = 8;
#pragma unroll
  for (int s0 = 0; s0 < SL; s0 += BATCH) {
    uint32_t ix[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int s = s0 + j;
      if (s < SL) {
        const int e = s * 64 + lane;
        ix[j] = lidx[((vmask >> s) & 1u) ? e : 0];
      }
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int s = s0 + j;
      if (s < SL) {
        const bool valid = (vmask >> s) & 1u;
        const bool eq = valid && kv[s] == th;
        const uint64_t mq = __ballot(eq);
        const bool keep = valid && (kv[s] > th || (eq && eq_seen + popc_lt(mq) < keep_eq));
        eq_seen += __popcll(mq);
        const uint64_t mk = __ballot(keep);
        if (keep) {
          const int pos = kept + popc_lt(mk);
          lval[pos] = __float_as_uint(key_to_f32(kv[s]));
          lidx[pos] = (uint16_t)ix[j];
        }
        kept += __popcll(mk);
      }
    }
  }
  kept_out = kept;
  return th;
}

template <int H, int D, bool FP8, bool SEL>
__global__ __launch_bounds__(64 * kLogitsWaves) void logits_kernel(LogitsArgs a) {
  using C = LogitsCfg<H, D, FP8>;
  using S = OutSlots<H>;
  using SC = SelCfg<H, D, FP8>;
  constexpr int MT = C::MT, QPB = C::QPB;
  constexpr int QPW = QPB / kLogitsWaves;
  static_assert(H >= 4 && H <= 64 && (H & (H - 1)) == 0, "H in {4, 8, 16, 32, 64}");

  // two key-tile buffers; the second one is larger and first serves as the
  // staging area of the q rows, read into registers before any key tile
  // goes there
  // staging: the q rows of every wave, then the head weights of every wave
  // (64 FP32 per wave) and, on the FP8 path, the q row scales
  constexpr int W_OFF = kLogitsWaves * C::A_BYTES;
  constexpr int QS_OFF = W_OFF + kLogitsWaves * 256;
  constexpr int STAGE_USED = QS_OFF + (FP8 ? kLogitsWaves * 256 : 0);
  // fused selection: after tile1, one candidate list per query, scores
  // (FP32 bits) [QPB][CAP] then pool indices (uint16) [QPB][CAP]; the q
  // staging overlaps them (it is read into registers before any entry is
  // written)
  constexpr int CAP = SEL ? SC::CAP : 0;
  constexpr int LIST_OFF = 2 * C::TILE_BYTES;
  // (plus 32 entries that take the stores of half-waves holding no query:
  // the second half at 64 heads)
  constexpr int LIST_ENTRIES = QPB * CAP + 32;
  constexpr int LIST_BYTES = LIST_ENTRIES * 6;
  constexpr int TILES_USED = SEL ? 2 * C::TILE_BYTES + LIST_BYTES : 2 * C::TILE_BYTES;
  constexpr int STAGE_END = C::TILE_BYTES + STAGE_USED;
  constexpr int LDS_BYTES = TILES_USED > STAGE_END ? TILES_USED : STAGE_END;
  static_assert(LDS_BYTES + 1024 <= 160 * 1024, "LDS budget");
  static_assert(!SEL || CAP >= 64, "candidate list capacity");
  // one LDS object with tile0 first, so every tile0 read and most tile1
  // reads fold their address into the 16-bit instruction offset
  __shared__ __attribute__((aligned(1024))) uint8_t lds_tiles[LDS_BYTES];
  uint8_t* const tile0 = lds_tiles;
  uint8_t* const tile1 = lds_tiles + C::TILE_BYTES;
  uint32_t* const lval = reinterpret_cast<uint32_t*>(lds_tiles + LIST_OFF);
  uint16_t* const lidx = reinterpret_cast<uint16_t*>(lds_tiles + LIST_OFF + LIST_ENTRIES * 4);
  __shared__ int q_doc[QPB], q_nc[QPB];
  __shared__ int q_start[SEL ? QPB : 1], q_pool0[SEL ? QPB : 1];
  __shared__ __attribute__((aligned(256))) float kscale_lds[2][FP8 ? 64 : 1];   // per tile buffer
  // step at which every wave shrinks its lists, by the step's parity: a
  // request for step s + 1 is written during step s, while step s's own
  // slot is still being read
  __shared__ int s_req[2];
  __shared__ int run_doc[QPB], run_nc[QPB], run_pool0[QPB];
  constexpr int QW = (QPB + 63) / 64;                // waves holding one query per lane
  __shared__ int run_cnt[QW];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  // workgroup -> (query block, piece of its pool range). Consecutive
  // workgroups go to consecutive XCDs; the pieces of one block are 8 apart, so
  // they land on the same XCD at about the same time and read its q rows
  // through one L2. The largest blocks (latest queries, most causal pools)
  // are dispatched first: those of the first row range, then those of the
  // second (a launch with two ranges puts the range with the longer rows
  // first).
  // Only the first range is split into pieces; the second range's blocks
  // follow the first range's workgroups, one each.
  const int nqb1 = (a.q_end - a.q_begin + QPB - 1) / QPB;
  const int nqb2 = a.q_end2 > a.q_begin2 ? (a.q_end2 - a.q_begin2 + QPB - 1) / QPB : 0;
  const int nwg1 = (nqb1 + 7) / 8 * 8 * a.pieces;
  int bi, piece = 0, npieces = 1;
  if ((int)blockIdx.x < nwg1) {
    const int grp = (int)blockIdx.x / (8 * a.pieces), r8 = (int)blockIdx.x % (8 * a.pieces);
    piece = r8 / 8;
    npieces = a.pieces;
    bi = grp * 8 + r8 % 8;
    if (bi >= nqb1) return;                  // padding of the last group
  } else {
    bi = nqb1 + ((int)blockIdx.x - nwg1);
    if (bi >= nqb1 + nqb2) return;
  }
  // this block's row range: its first row, its end, and where its scores go
  const bool second = bi >= nqb1;
  const int q_begin = second ? a.q_begin2 : a.q_begin;
  const int q_end = second ? a.q_end2 : a.q_end;
  float* const out_base = second ? a.out2 : a.out;
  const int64_t ld = second ? a.ld2 : a.ld;
  const int qblk = second ? nqb2 - 1 - (bi - nqb1) : nqb1 - 1 - bi;
  const int t0 = q_begin + qblk * QPB;
  const uint8_t* keys = reinterpret_cast<const uint8_t*>(a.keys);

  // document, causal range and pool offset of each query: a few dependent
  // loads, done before the q rows are requested so they do not queue behind
  int my_doc = -1, my_nc = 0, my_pool0 = 0, my_start = 0;
  if (tid < QPB) {
    const int t = t0 + tid;
    if (t < q_end) {
      const QueryInfo qi = query_info(a.cu, a.cu_pools, a.B, a.T, a.kpool, a.max_pools, t);
      my_doc = qi.doc;
      my_nc = qi.n_c;
      my_pool0 = qi.pool0;
      my_start = qi.start;
    }
    q_doc[tid] = my_doc;
    q_nc[tid] = my_nc;
    if constexpr (SEL) {
      q_start[tid] = my_start;
      q_pool0[tid] = my_pool0;
    }
  }
  if (tid == 0) s_req[0] = s_req[1] = -1;
  __syncthreads();
  // Runs of queries in one document. Queries are in token order, so each
  // document's queries are consecutive and the last one of a run has the
  // widest causal range; run r goes to slot r of the run_* arrays.
  const bool run_end = tid < QPB && my_doc >= 0 && (tid == QPB - 1 || q_doc[tid + 1] != my_doc);
  const uint64_t end_mask = __ballot(run_end);
  if (wid < QW && lane == 0) run_cnt[wid] = __popcll(end_mask);
  __syncthreads();
  int n_runs = 0, runs_before = 0;
#pragma unroll
  for (int w = 0; w < QW; ++w) {
    n_runs += run_cnt[w];
    runs_before += w < wid ? run_cnt[w] : 0;
  }
  if (run_end) {
    const int r = runs_before + popc_lt(end_mask);
    run_doc[r] = my_doc;
    run_nc[r] = my_nc;
    run_pool0[r] = my_pool0;
  }
  __syncthreads();

  // this workgroup's work in run r: the widest causal range of its queries,
  // the document's first pool, and its share [jt_lo, jt_hi) of the tiles
  struct DocWork { int maxnc, pool0, jt_lo, jt_hi; };
  auto run_work = [&](int r) {
    DocWork d{run_nc[r], run_pool0[r], 0, 0};
    if (d.maxnc == 0 || (a.skip_select_all && d.maxnc <= a.k_sel)) return d;
    const int ntiles = (d.maxnc + kPoolTile - 1) / kPoolTile;
    d.jt_lo = ntiles * piece / npieces;
    d.jt_hi = ntiles * (piece + 1) / npieces;
    return d;
  };
  int r_first = n_runs;
  for (int r = 0; r < n_runs; ++r) {
    const DocWork d = run_work(r);
    if (d.jt_lo < d.jt_hi) { r_first = r; break; }
  }
  const bool any_work = r_first < n_runs;    // (uniform)
  if (!SEL && !any_work) return;             // nothing to score

  // fused selection, per output slot k of this lane (query S::query(k, g) of
  // the wave): entries in the list, the threshold a new score must exceed
  // (open: no threshold yet, every score enters), the list's first entry
  int cnt_r[S::N];
  float thr_r[S::N];
  bool open_r[S::N];
  int lbase[S::N];
#pragma unroll
  for (int k = 0; k < S::N; ++k) {
    cnt_r[k] = 0;
    thr_r[k] = 0.f;
    open_r[k] = true;
    lbase[k] = (H == 64 && g == 1) ? QPB * CAP : (wid * QPW + S::query(k, g)) * CAP;
  }
  int stepno = 0;
  // a shrink may keep up to k_sel + slack entries (when the bisection finds
  // such a threshold first): at most CAP - 160, the bound the trigger
  // assumes for a list just shrunk
  const int slack = min(64, CAP - 160 - a.k_sel);
  int pending = -1;                         // the step at which a shrink was asked for
  const int gneg = g ? -1 : 0;
  // every list of the wave above k_sel entries -> its exact top k_sel
  auto shrink_wave = [&]() {
#pragma unroll 1
    for (int qq = 0; qq < QPW; ++qq) {
      const int kq = qq >> 1, gq = qq & 1;     // the slot and half-wave holding query qq
      int c = cnt_r[0];
#pragma unroll
      for (int k = 1; k < S::N; ++k) c = k == kq ? cnt_r[k] : c;
      c = __builtin_amdgcn_readlane(c, gq * 32);
      // a list that a shrink could not cut below k_sel + slack is left as it
      // is (its threshold must not drop)
      if (c <= a.k_sel + slack) continue;
      const int base = (wid * QPW + qq) * CAP;
      int kept;
      const uint32_t th = list_select<(SEL ? CAP : 64)>(lval + base, lidx + base, c, a.k_sel,
                                                        slack, lane, kept);
      const float tf = key_to_f32(th);
#pragma unroll
      for (int k = 0; k < S::N; ++k) {
        if (k == kq && g == gq) {
          cnt_r[k] = kept;
          thr_r[k] = tf;
          open_r[k] = false;
        }
      }
    }
  };
  // at the end of step s, a wave with a list past the trigger asks every
  // wave to shrink at the start of step s + 2: the request is read at the
  // start of step s + 1, after the barrier that orders it, and acted on one
  // step later, so no wave waits for that read
  auto request_check = [&]() {
    bool over = false;
#pragma unroll
    for (int k = 0; k < S::N; ++k) over |= cnt_r[k] > SC::TRIGGER;
    // (none when the next step shrinks already: that covers every list)
    if (__ballot(over) && pending != stepno + 1) {
      if (lane == 0) s_req[(stepno + 1) & 1] = stepno + 2;
    }
  };

  if (any_work) {
  {
    // the first key tile and the q rows are in flight together
    const DocWork d = run_work(r_first);
    load_key_tile<H, D, FP8>(keys, d.pool0, d.jt_lo * kPoolTile, d.maxnc, tile0, wid, lane,
                             a.k_scale, kscale_lds[0]);
  }
  {
    const size_t row0 = (size_t)(t0 + wid * QPW) * H, row_last = (size_t)q_end * H - 1;
    load_q_rows<H, D, FP8>(reinterpret_cast<const uint8_t*>(a.q), row0, row_last,
                           tile1 + wid * C::A_BYTES, lane);
    // the wave's 64 head weights (rows past the launch read row_last)
    const size_t wr = row0 + lane < row_last ? row0 + lane : row_last;
    dma4(a.w + wr, reinterpret_cast<float*>(tile1 + W_OFF) + wid * 64);
    if constexpr (FP8) dma4(a.q_scale + wr, reinterpret_cast<float*>(tile1 + QS_OFF) + wid * 64);
  }

  // LDS byte offset, within a 32-row block, of each 16-byte chunk this lane
  // reads as an MFMA operand (row n, half g of D, swizzled). The swizzle
  // depends only on the row's low bits, so the same offsets serve every 32-key
  // unit of both tiles and both 32-row blocks of q; they are kept in registers
  // (the asm hides them from rematerialisation) and a block's base folds into
  // the read's immediate.
  constexpr int NCH = C::CPR / 2;
  uint32_t boff[NCH];
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    boff[u] = (uint32_t)(n * C::ROWB + swz<C::CPR>(n, g * NCH + u) * 16);
    asm volatile("" : "+v"(boff[u]));
  }

  // ---- A operand: this wave's (query, head) rows, held for the whole launch.
  // Row m of tile mt is flat row mt * 32 + m of the wave: query flat / H,
  // head flat % H. Lane (n, g) holds row n, K slice [g D/2, (g + 1) D/2).
  using Frag = typename std::conditional<FP8, i32x8_t, bf16x8_t>::type;
  Frag afrag[MT][C::NSTEP];
  float wq[MT][16];          // w' of the 16 accumulator rows this lane holds
  // the q rows, head weights (and the first key tile) have arrived in LDS
  wait_vmem_all();
  __syncthreads();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      // accumulator rows 8 J + 4 g .. + 3 of tile mt: four consecutive rows
      // of the wave, one 16-byte read (the same address for a half-wave)
      const int fr = mt * 32 + J * 8 + g * 4;
      const float4 w4 = *reinterpret_cast<const float4*>(tile1 + W_OFF + (wid * 64 + fr) * 4);
      float4 s4 = make_float4(1.f, 1.f, 1.f, 1.f);
      if constexpr (FP8) s4 = *reinterpret_cast<const float4*>(tile1 + QS_OFF + (wid * 64 + fr) * 4);
      const bool ok = t0 + wid * QPW + fr / H < q_end;   // the four rows share a query
      wq[mt][J * 4 + 0] = ok ? w4.x * a.scale * s4.x : 0.f;
      wq[mt][J * 4 + 1] = ok ? w4.y * a.scale * s4.y : 0.f;
      wq[mt][J * 4 + 2] = ok ? w4.z * a.scale * s4.z : 0.f;
      wq[mt][J * 4 + 3] = ok ? w4.w * a.scale * s4.w : 0.f;
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const bool ok = t0 + wid * QPW + (mt * 32 + n) / H < q_end;
    const uint8_t* blk = tile1 + wid * C::A_BYTES + mt * 32 * C::ROWB;
#pragma unroll
    for (int s = 0; s < C::NSTEP; ++s) {
      if constexpr (FP8) {
        uint4 lo4 = *reinterpret_cast<const uint4*>(blk + boff[2 * s]);
        uint4 hi4 = *reinterpret_cast<const uint4*>(blk + boff[2 * s + 1]);
        if (!ok) lo4 = hi4 = make_uint4(0, 0, 0, 0);
        i32x8_t f = {(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                     (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
        afrag[mt][s] = f;
      } else {
        uint4 v = *reinterpret_cast<const uint4*>(blk + boff[s]);
        if (!ok) v = make_uint4(0, 0, 0, 0);
        afrag[mt][s] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
  }

  // ---- scores leave through a buffer resource over this workgroup's rows;
  // a masked lane stores at offset num_records, which the hardware drops
  const int wg_rows = min(QPB, q_end - t0);
  const uint32_t nrec = (uint32_t)((size_t)wg_rows * ld * 4);
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      out_base + (size_t)(t0 - q_begin) * ld, 0, (int)nrec, 0x00020000);

  for (int r = r_first; r < n_runs; ++r) {
    const DocWork dw = run_work(r);
    const int b = run_doc[r];
    if (dw.jt_lo >= dw.jt_hi) continue;
    const int maxnc = dw.maxnc, pool0 = dw.pool0, jt_lo = dw.jt_lo, jt_hi = dw.jt_hi;

    // per output slot: causal limit (0 for other documents) and row offset
    uint32_t lim[S::N], roff[S::N];
#pragma unroll
    for (int k = 0; k < S::N; ++k) {
      const int qb = wid * QPW + S::query(k, g);
      const bool mine = q_doc[qb] == b && (H != 64 || g == 0);
      lim[k] = mine ? (uint32_t)q_nc[qb] : 0u;
      roff[k] = (uint32_t)((size_t)qb * ld * 4);
    }

    // epilogue of one 32-pool unit whose first column is cbase (negative:
    // nothing to store): w' * ReLU, sum over heads, causal mask, store
    auto epilogue = [&](const f32x16_t (&acc)[MT], int cbase, float kscale) {
      const int col = cbase + n;
      // the lane's rows of one query form one multiply-add chain (one VALU
      // op per row after the ReLU; the chain's latency hides behind MFMAs)
      float outv[S::N];
      if constexpr (H == 4) {
        // rows 8J + 4g .. + 3 are query 2J + g of the tile: complete per lane
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int J = 0; J < 4; ++J) {
            float s4 = wq[mt][J * 4] * relu(acc[mt][J * 4]);
#pragma unroll
            for (int jj = 1; jj < 4; ++jj) s4 += wq[mt][J * 4 + jj] * relu(acc[mt][J * 4 + jj]);
            outv[mt * 4 + J] = s4;
          }
      } else if constexpr (H == 64) {
        // both row tiles hold the same query; add the two half-waves
        float s = wq[0][0] * relu(acc[0][0]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = (mt == 0 ? 1 : 0); j < 16; ++j) s += wq[mt][j] * relu(acc[mt][j]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s),
                                                         false, false);
        outv[0] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      } else {
        constexpr int QPT = 32 / H;                      // queries per 32-row tile
        constexpr int RPQ = 16 / QPT;                    // this lane's rows per query
        float tot[MT * QPT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int qq = 0; qq < QPT; ++qq) {
            float s = wq[mt][qq * RPQ] * relu(acc[mt][qq * RPQ]);
#pragma unroll
            for (int j = qq * RPQ + 1; j < (qq + 1) * RPQ; ++j) s += wq[mt][j] * relu(acc[mt][j]);
            tot[mt * QPT + qq] = s;
          }
        // pair queries 2i and 2i+1: after the swap the low half-wave holds
        // the full sum of query 2i and the high half-wave that of 2i+1
#pragma unroll
        for (int i = 0; i < S::N; ++i) {
          const auto sw = __builtin_amdgcn_permlane32_swap(
              __float_as_uint(tot[2 * i]), __float_as_uint(tot[2 * i + 1]), false, false);
          outv[i] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
      }
#pragma unroll
      for (int k = 0; k < S::N; ++k) {
        const bool ok = (uint32_t)col < lim[k];
        const float sv = outv[k] * kscale;
        if constexpr (SEL) {
          // the score enters the query's list when it exceeds the threshold
          // (NaN never does once there is one). The lanes of one slot's
          // query are one half-wave: the a entering scores take list
          // positions cnt .. cnt + a - 1 in lane order, and the other lanes
          // of the half write into cnt + a .. cnt + 31, past the list's end
          // (room the shrink protocol keeps free), so every lane stores and
          // the epilogue stays one branch-free block beside the MFMAs
          const bool app = ok & (open_r[k] | (sv > thr_r[k]));
          const uint64_t m = __ballot(app);
          const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
          const int lo_cnt = __popc(lo), hi_cnt = __popc(hi);
          // entering lanes below this one in its half, and in its half
          const int below =
              (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u)) - (lo_cnt & gneg);
          const int a_cnt = lo_cnt + ((hi_cnt - lo_cnt) & gneg);
          const int pos = cnt_r[k] + (app ? below : a_cnt + (n - below));
          lval[lbase[k] + pos] = __float_as_uint(sv);
          lidx[lbase[k] + pos] = (uint16_t)col;
          cnt_r[k] += a_cnt;
        } else {
          const uint32_t off = ok ? roff[k] + (uint32_t)col * 4u : nrec;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sv), orsrc, (int)off, 0, 0);
        }
      }
    };

    // MFMAs of one 32-pool unit (key rows 32 np .. 32 np + 31 of tile tb)
    auto mma = [&](f32x16_t (&acc)[MT], const uint8_t* __restrict__ tb, int np) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mt][j] = 0.f;
      const uint8_t* unit = tb + np * 32 * C::ROWB;     // constant: folds into the offset
#pragma unroll
      for (int s = 0; s < C::NSTEP; ++s) {
        if constexpr (FP8) {
          const uint4 lo4 = *reinterpret_cast<const uint4*>(unit + boff[2 * s]);
          const uint4 hi4 = *reinterpret_cast<const uint4*>(unit + boff[2 * s + 1]);
          i32x8_t bf = {(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                        (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afrag[mt][s], bf, acc[mt], 0,
                                                                      0, 0, 0, 0, 0);
        } else {
          const uint4 v = *reinterpret_cast<const uint4*>(unit + boff[s]);
          const bf16x8_t bf = __builtin_bit_cast(bf16x8_t, v);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[mt][s], bf, acc[mt], 0, 0, 0);
        }
      }
    };

    // interleave the MFMAs of one unit with the epilogue VALU work of the
    // previous unit so the matrix core and the vector ALU work together
    // (measured on gfx950: for BF16 the LDS read is best placed after its
    // slot's MFMA, for FP8 before it)
    auto interleave = [&]() {
#pragma unroll
      for (int i = 0; i < C::NSTEP * MT; ++i) {
        if constexpr (FP8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      // MFMA
        if constexpr (!FP8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);                      // VALU
      }
    };

    f32x16_t accA[MT], accB[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) accB[mt][j] = 0.f;
    // first column of the unit held in accB; kNoUnit: none (its columns are
    // negative, so every lane's store is masked)
    constexpr int kNoUnit = -(1 << 30);
    int prev = kNoUnit;
    float ks_prev = 1.f;   // FP8: key scale of this lane's column in accB's unit

    if (r != r_first) {  // (the first run's first tile is already on its way)
      __syncthreads();   // both LDS buffers are free
      load_key_tile<H, D, FP8>(keys, pool0, jt_lo * kPoolTile, maxnc, tile0, wid, lane,
                               a.k_scale, kscale_lds[0]);
    }

    // Tiles alternate between tile0 and tile1; the body is instantiated once
    // per buffer so each LDS read names a fixed buffer.
    // The DMA of tile jt was issued at the start of the previous step, before
    // that step's kUnits * S::N output stores: waiting until only those
    // stores are outstanding covers the DMA without waiting for the stores.
    // The fused selection issues no stores in a step, so it waits for
    // everything (the DMA).
    static_assert(kUnits == 2, "one pair of 32-pool units per tile");
    auto step = [&](const int jt, const uint8_t* __restrict__ tb, uint8_t* __restrict__ nb,
                    const int buf) {
      if (SEL || jt == jt_lo) wait_vmem_all();
      else wait_vmem_leave<kUnits * S::N>();
      __syncthreads();   // tile jt is in LDS; tile jt - 1 is no longer read
      // FP8: this tile's key scales of the lane's two columns, read before
      // the next copy may overwrite the other buffer's
      float ks0 = 1.f, ks1 = 1.f;
      if constexpr (FP8) {
        ks0 = kscale_lds[buf][n];
        ks1 = kscale_lds[buf][32 + n];
      }
      const int j0 = jt * kPoolTile;
      if (jt + 1 < jt_hi)
        load_key_tile<H, D, FP8>(keys, pool0, j0 + kPoolTile, maxnc, nb, wid, lane, a.k_scale,
                                 kscale_lds[buf ^ 1]);
      if constexpr (SEL) {
        if (pending == stepno) shrink_wave();         // every wave at the same step
        pending = s_req[stepno & 1];
      }
      // FP8: a wave still in the step's first unit outranks one in the
      // second, so the two waves of a SIMD reach the next barrier closer
      // together (measured: -4 % per FP8 step; the BF16 path is 2-4 %
      // slower with either order, so it keeps equal priority)
      if constexpr (FP8 && !SEL) __builtin_amdgcn_s_setprio(1);
      mma(accA, tb, 0);
      epilogue(accB, prev, ks_prev);
      interleave();
      if constexpr (FP8 && !SEL) __builtin_amdgcn_s_setprio(0);
      mma(accB, tb, 1);
      epilogue(accA, j0, ks0);
      interleave();
      prev = j0 + 32;
      ks_prev = ks1;
      if constexpr (SEL) {
        request_check();
        ++stepno;
      }
    };
    for (int jt = jt_lo; jt < jt_hi; jt += 2) {
      step(jt, tile0, tile1, 0);
      if (jt + 1 < jt_hi) step(jt + 1, tile1, tile0, 1);
    }
    epilogue(accB, prev, ks_prev);
    if constexpr (SEL) request_check();
  }
  }  // any_work

  if constexpr (SEL) {
    // ---- token rows of the wave's queries: the exact top k_sel of each
    // list (ascending pools), or every causal pool when n_c <= k_sel; then
    // the tail tokens and -1 padding
    const bool vec4 = a.kpool == 4 && (a.width & 3) == 0;
#pragma unroll 1
    for (int qq = 0; qq < QPW; ++qq) {
      const int qb = wid * QPW + qq;
      const int t = t0 + qb;
      if (t >= q_end) break;
      const int n_c = q_nc[qb];
      const int start = q_start[qb];
      const int n_sel = n_c < a.k_sel ? n_c : a.k_sel;
      const int base = qb * CAP;
      if (n_c > a.k_sel) {
        const int kq = qq >> 1, gq = qq & 1;
        int c = cnt_r[0];
#pragma unroll
        for (int k = 1; k < S::N; ++k) c = k == kq ? cnt_r[k] : c;
        c = __builtin_amdgcn_readlane(c, gq * 32);
        int kept;
        if (c > a.k_sel)
          list_select<(SEL ? CAP : 64)>(lval + base, lidx + base, c, a.k_sel, 0, lane, kept);
      }
      const int tail = a.tail_on ? (t - start + 1) % a.kpool : 0;
      const int row = t - q_begin;
      int32_t* otok = a.out_tok + (size_t)row * a.width;
      if (a.out_ids) {
        int32_t* oid = a.out_ids + (size_t)row * a.k_sel;
        const int pool0 = q_pool0[qb];
        for (int j = lane; j < a.k_sel; j += 64)
          oid[j] = j < n_sel ? pool0 + (n_c > a.k_sel ? (int)lidx[base + j] : j) : -1;
      }
      const int from = n_sel * a.kpool;              // tail and padding start here
      const int tail_base = start + n_c * a.kpool;
      if (vec4) {
        for (int j = lane; j < n_sel; j += 64) {
          const int pb = start + 4 * (n_c > a.k_sel ? (int)lidx[base + j] : j);
          *reinterpret_cast<int4*>(otok + 4 * j) = make_int4(pb, pb + 1, pb + 2, pb + 3);
        }
        for (int gi = (from >> 2) + lane; gi < (a.width >> 2); gi += 64) {
          int e[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int jj = gi * 4 + c - from;
            e[c] = jj < tail ? tail_base + jj : -1;
          }
          *reinterpret_cast<int4*>(otok + gi * 4) = make_int4(e[0], e[1], e[2], e[3]);
        }
      } else {
        for (int j = lane; j < from; j += 64) {
          const int e = j / a.kpool;
          const int p = n_c > a.k_sel ? (int)lidx[base + e] : e;
          otok[j] = start + p * a.kpool + (j - e * a.kpool);
        }
        for (int j = from + lane; j < a.width; j += 64) {
          const int jj = j - from;
          otok[j] = jj < tail ? tail_base + jj : -1;
        }
      }
    }
  }
}

__global__ void fill_kernel(float* __restrict__ out, size_t count, float v) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < count; i += stride) out[i] = v;
}

template <int H, int D, bool FP8, bool SEL>
static void launch_hdf(LogitsArgs a, hipStream_t st) {
  constexpr int QPB = LogitsCfg<H, D, FP8>::QPB;
  const int nqb1 = (a.q_end - a.q_begin + QPB - 1) / QPB;
  const int nqb2 = a.q_end2 > a.q_begin2 ? (a.q_end2 - a.q_begin2 + QPB - 1) / QPB : 0;
  // Each query block is one workgroup of a CU, and its work grows with its
  // queries' causal range, so one workgroup per block leaves CUs idle while
  // the longest rows finish. Long rows are split into two pieces of the pool
  // range: the dispatcher hands the next (smaller) piece to whichever CU
  // frees first. Each piece pays the start-up again (about 8 us to bring in
  // its q rows), so this pays only for long sweeps: measured on the 64K
  // context (16384 pools, BF16) it gains about 1 %, and it loses at 8192
  // pools on the FP8 path, whose sweep is half as long per pool. The fused
  // selection keeps each query's candidates in its workgroup, so it takes
  // whole blocks. A launch of two row ranges (short rows after long ones)
  // has its own mix of block sizes to balance with and takes whole blocks.
  const long sweep = (long)a.max_pools * (FP8 ? 1 : 2);
  a.pieces = (!SEL && nqb2 == 0 && sweep >= 32768) ? 2 : 1;
  const int nwg = (nqb1 + 7) / 8 * 8 * a.pieces + nqb2;
  logits_kernel<H, D, FP8, SEL><<<nwg, 64 * kLogitsWaves, 0, st>>>(a);
}

template <int D, bool FP8, bool SEL>
static void launch_df(const LogitsArgs& a, hipStream_t st) {
  switch (a.H) {
    case 4: launch_hdf<4, D, FP8, SEL>(a, st); break;
    case 8: launch_hdf<8, D, FP8, SEL>(a, st); break;
    case 16: launch_hdf<16, D, FP8, SEL>(a, st); break;
    case 32: launch_hdf<32, D, FP8, SEL>(a, st); break;
    default: launch_hdf<64, D, FP8, SEL>(a, st); break;
  }
}

void launch_logits(const LogitsArgs& a, hipStream_t st) {
  const int rows = a.q_end - a.q_begin;
  if (rows <= 0 && a.q_end2 <= a.q_begin2) return;
  if (a.fill_masked && rows > 0) {
    const size_t count = (size_t)rows * a.ld;
    const int blocks = (int)std::min<size_t>((count + 255) / 256, 8192);
    fill_kernel<<<blocks, 256, 0, st>>>(a.out, count, -INFINITY);
  }
  if (a.fp8) launch_df<128, true, false>(a, st);
  else if (a.D == 128) launch_df<128, false, false>(a, st);
  else launch_df<64, false, false>(a, st);
}

template <int D, bool FP8>
static int sel_capacity(int H) {
  switch (H) {
    case 4: return SelCfg<4, D, FP8>::CAP;
    case 8: return SelCfg<8, D, FP8>::CAP;
    case 16: return SelCfg<16, D, FP8>::CAP;
    case 32: return SelCfg<32, D, FP8>::CAP;
    default: return SelCfg<64, D, FP8>::CAP;
  }
}

int logits_select_max_ksel(int H, int D, int fp8) {
  const int cap = fp8 ? sel_capacity<128, true>(H)
                      : (D == 128 ? sel_capacity<128, false>(H) : sel_capacity<64, false>(H));
  // a list just shrunk holds at least k_sel entries and takes up to 160 more
  // before the next shrink
  return cap - 160 > 0 ? cap - 160 : 0;
}

bool logits_select_supported(int H, int D, int fp8, int k_sel) {
  return k_sel >= 1 && k_sel <= logits_select_max_ksel(H, D, fp8);
}

void launch_logits_select(const LogitsArgs& a, hipStream_t st) {
  if (a.q_end <= a.q_begin) return;
  if (a.fp8) launch_df<128, true, true>(a, st);
  else if (a.D == 128) launch_df<128, false, true>(a, st);
  else launch_df<64, false, true>(a, st);
}

}  // namespace kpool
