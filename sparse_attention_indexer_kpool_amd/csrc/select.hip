// Steps 3 and 4 of the KPool indexer for one chunk of query rows: per-query
// pool top-k and, when asked, expansion of the chosen pools to token indices
// with the tail appended.
//
// Megatron-LM PR #7054, section "3. KPool DSA indexer + NoPE": the indexer's
// top-k runs over pools and keeps index_topk // kpool of them; the chosen
// pools expand back to token indices and, with always_select_tail, each
// query keeps its incomplete causal pool. SkyRL PR #2179 ("Limitations /
// follow-ups") gives the order: score pools, expand to tokens, append the
// tail pool. xtuner PR #2108 (selector fix commit) names a radix-select row
// selector as the production alternative to a full sort; this kernel is an
// exact selection written for gfx950.
//
// One workgroup per query row (a launch may cover two row ranges, each with
// its own scores and row stride: the indexer selects both chunks of a
// two-chunk scoring launch at once); HBM-bound: each causal score is read
// once with coalesced 16-byte loads and stays in registers. Selection order: larger
// score first, equal scores to the lower pool index, NaN ranks as -inf.
//
//   1. The row is loaded (slots past n_c hold NaN).
//   2. A sample of the row (one value in eight) is histogrammed over 1024
//      bins linear in the value between the sample's min and max; its upper
//      tail gives a level L below which, with a wide margin, no chosen value
//      lies.
//   3. Every value >= L is appended to a list in LDS (one segment per wave,
//      a ballot prefix per lane). The list size is exact, so L is verified:
//      if fewer than K_sel values reach L, or a segment overflows, the row
//      takes the general path below.
//   4. On the short list: a value-linear histogram finds the bin b* holding
//      the K_sel-th value (bins are monotone in the value: FP32 subtraction,
//      multiplication and truncation all preserve order), the few values of
//      b* are ranked against each other, and that gives the exact threshold
//      element (tau, idx_tau). An element is chosen iff it ranks at or above
//      it.
//   5. Chosen pools set bits of an LDS bitmap over the row; one prefix sum of
//      per-thread bit counts turns the bitmap into ascending output slots.
//      Each chosen pool writes its global id (optional) and, when token rows
//      are asked for, its kpool token ids (one 16-byte store for kpool = 4);
//      the tail tokens and the -1 padding follow.
//
// Short rows (at most three float4 groups per thread, 3072 pools with 256
// threads) skip steps 2 and 3: every value is its own list entry, held in
// registers, and one histogram of the whole row takes the place of the
// sample's and the list's, so the row crosses seven workgroup barriers
// instead of eleven (64K step: selection 0.68 -> 0.64 ms; allowing four
// groups measured the same, six and eight slower).
//
// General path (non-finite or constant rows, an unlucky sample): repeated
// histogram rounds over order-preserving 32-bit keys (NaN -> -inf, -0 -> +0),
// bins a right shift of key - min, then over the pool index once all
// remaining keys tie; it re-reads the row from memory. Rows with
// n_c <= K_sel select every causal pool and read no logits.

#include "kpool_device.h"
#include "kpool_internal.h"

namespace kpool {

constexpr int kBins = 1024;         // value-linear bins
// List entries per lane of a wave segment. The 256-thread shapes take six:
// those of up to 10 groups, whose registers allow eight workgroups per CU,
// then also fit eight in the CU's 160 KB of LDS (19.6 KB each instead of
// 23.7 KB), and the longer ones lose nothing (64K step, selection 0.711 ->
// 0.676 ms). The wider shapes keep eight: a wave's segment holds its share
// of the sampled level's margin, and a segment that overflows sends the row
// to the slow general path.
__host__ __device__ constexpr int list_per_lane(int nt) {
  return nt == 256 ? 6 : 8;
}
constexpr int kLogKeyBins = 10;     // key-space bins of the general path
constexpr int kKeyBins = 1 << kLogKeyBins;

// Makes the compiler forget what it knows about the values, so per-element
// results of one phase are recomputed in the next instead of being held in
// registers across a barrier.
template <int E>
__device__ __forceinline__ void forget(float (&v)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) asm volatile("" : "+v"(v[e]));
}

template <int NT, int G>
struct SelectShared {
  static constexpr int NW = NT / 64;
  static constexpr int WORDS = NT * G / 8;       // bitmap words: 4 G NT bits
  uint32_t hist[kBins + 1];
  float red_f[2][NW];
  uint32_t red_u[2][NW];
  int red_n[NW];                                 // sample counts (kept apart from wave_tot)
  int wave_tot[NW];
  int res[3];                                    // b*, count above b*, count in b*
  uint32_t cand_key[NT];
  int cand_idx[NT];
  int cand_cnt;
  int seg_cnt[NW];
  uint32_t th_key;
  int th_idx;
  uint32_t bitmap[WORDS];
};

// Suffix scan of sh.hist[0 .. NBINS): the bin b* with (count above b*) < k <=
// (count above b*) + hist[b*]. Results land in sh.res; ends with a barrier.
template <int NT, int G, int NBINS>
__device__ __forceinline__ void find_bin(SelectShared<NT, G>& sh, int k) {
  constexpr int NW = NT / 64;
  constexpr int BPT = (NBINS + NT - 1) / NT;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int own = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int b = tid * BPT + j;
    own += b < NBINS ? (int)sh.hist[b] : 0;
  }
  const int suf = wave_suffix_sum(own);
  if (lane == 0) sh.wave_tot[wid] = suf;
  __syncthreads();
  int above = suf - own;
#pragma unroll
  for (int w = 0; w < NW; ++w) above += w > wid ? sh.wave_tot[w] : 0;
  if (above < k && k <= above + own) {
    int acc = above;
    for (int j = BPT - 1; j >= 0; --j) {
      const int b = tid * BPT + j;
      const int h = b < NBINS ? (int)sh.hist[b] : 0;
      if (acc + h >= k) { sh.res[0] = b; sh.res[1] = acc; sh.res[2] = h; break; }
      acc += h;
    }
  }
  __syncthreads();
}

// Value-linear bin over [lo, lo + kBins / inv]; NaN lands in bin 0 (fmaxf
// returns the non-NaN operand).
__device__ __forceinline__ int vbin(float x, float lo, float inv) {
  return (int)fminf(fmaxf((x - lo) * inv, 0.f), (float)(kBins - 1));
}

// The threshold element among the c_in candidates of bin b* (sh.cand_key,
// sh.cand_idx): the one of rank k_in - 1 by larger key first, equal keys to
// the lower index. Every wave ranks the few candidates itself (lane l takes
// candidates l, l + 64, ...), so the result needs no barrier to reach the
// other waves. Returns (key, index).
template <int NT, int G>
__device__ __forceinline__ uint2 threshold_of(const SelectShared<NT, G>& sh, int c_in, int k_in,
                                             int lane) {
  uint32_t tk = 0u;
  int ti = 0;
  for (int c0 = 0; c0 < c_in; c0 += 64) {
    const int ci = c0 + lane;
    bool hit = false;
    uint32_t mk = 0u;
    int mi = 0;
    if (ci < c_in) {
      mk = sh.cand_key[ci];
      mi = sh.cand_idx[ci];
      int rank = 0;
      for (int q = 0; q < c_in; ++q) {
        const uint32_t okey = sh.cand_key[q];
        rank += (okey > mk) || (okey == mk && sh.cand_idx[q] < mi);
      }
      hit = rank == k_in - 1;
    }
    const uint64_t hm = __ballot(hit);
    if (hm) {
      const int src = __ffsll((unsigned long long)hm) - 1;
      tk = (uint32_t)__builtin_amdgcn_readlane((int)mk, src);
      ti = __builtin_amdgcn_readlane(mi, src);
    }
  }
  return make_uint2(tk, (uint32_t)ti);
}

// A short row (at most GL float4 groups per thread) without the sample, the
// level and the list: its values stay in registers, one value-linear
// histogram of the whole row over [min, max] finds the bin b* of the
// K_sel-th value, b*'s few values are ranked exactly, and the chosen set
// their bitmap bits. Loads the row itself, clears the histogram, bitmap and
// counters, and ends with a barrier. Returns false when the row needs the
// general path (fewer than K_sel non-NaN values, infinities, a constant row,
// a crowded bin).
template <int NT, int G, int GL>
__device__ __forceinline__ bool lean_row(SelectShared<NT, G>& sh, const float* __restrict__ row,
                                         int ld, int n_c, int k_sel, int nwords) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int ng = (n_c + 4 * NT - 1) / (4 * NT);
  const uint8_t* rowb = reinterpret_cast<const uint8_t*>(row);
  auto idx_of = [&](int g, int c) { return (g * NT + tid) * 4 + c; };
  float4 raw[GL];
#pragma unroll
  for (int g = 0; g < GL; ++g) {
    if (g < ng) {
      const int off = min(g * NT * 16 + tid * 16, (ld - 4) * 4);
      raw[g] = *reinterpret_cast<const float4*>(rowb + off);
    } else {
      raw[g] = make_float4(NAN, NAN, NAN, NAN);
    }
  }
  float u[4 * GL];
#pragma unroll
  for (int g = 0; g < GL; ++g) {
    u[4 * g + 0] = raw[g].x; u[4 * g + 1] = raw[g].y; u[4 * g + 2] = raw[g].z; u[4 * g + 3] = raw[g].w;
#pragma unroll
    for (int c = 0; c < 4; ++c) u[4 * g + c] = idx_of(g, c) < n_c ? u[4 * g + c] : NAN;
  }
  forget(u);
  float mn = INFINITY, mx = -INFINITY;
  int ns = 0;
#pragma unroll
  for (int e = 0; e < 4 * GL; ++e) {
    mn = fminf(mn, u[e]);
    mx = fmaxf(mx, u[e]);
    ns += u[e] == u[e];
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  ns = wave_sum(ns);
  if (lane == 0) { sh.red_f[0][wid] = mn; sh.red_f[1][wid] = mx; sh.red_n[wid] = ns; }
  for (int j = tid; j <= kBins; j += NT) sh.hist[j] = 0u;
  for (int j = tid; j < nwords; j += NT) sh.bitmap[j] = 0u;
  if (tid == 0) { sh.cand_cnt = 0; sh.res[0] = sh.res[1] = sh.res[2] = 0; }
  __syncthreads();
  mn = sh.red_f[0][0]; mx = sh.red_f[1][0];
  int S = sh.red_n[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    mn = fminf(mn, sh.red_f[0][w]);
    mx = fmaxf(mx, sh.red_f[1][w]);
    S += sh.red_n[w];
  }
  const float range = mx - mn;
  bool fast = S >= k_sel && (range > 0.f) && (range <= 3.0e38f);
  if (fast) {
    const float inv = (float)kBins / range;
#pragma unroll
    for (int e = 0; e < 4 * GL; ++e)
      if (u[e] == u[e]) atomicAdd(&sh.hist[vbin(u[e], mn, inv)], 1u);
    __syncthreads();
    find_bin<NT, G, kBins>(sh, k_sel);
    const int bstar = sh.res[0];
    const int k_in = k_sel - sh.res[1];
    const int c_in = sh.res[2];
    if (c_in > NT) {
      fast = false;                                    // crowded bin: general path
    } else {
      forget(u);
#pragma unroll
      for (int g = 0; g < GL; ++g) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float x = u[4 * g + c];
          if (x == x && vbin(x, mn, inv) == bstar) {
            const int slot = atomicAdd(&sh.cand_cnt, 1);
            sh.cand_key[slot] = f32_order_key(x);
            sh.cand_idx[slot] = idx_of(g, c);
          }
        }
      }
      __syncthreads();
      const uint2 th = threshold_of<NT, G>(sh, c_in, k_in, lane);
      forget(u);
#pragma unroll
      for (int g = 0; g < GL; ++g) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float x = u[4 * g + c];
          const int ix = idx_of(g, c);
          if (x == x) {
            const uint32_t kx = f32_order_key(x);
            if (kx > th.x || (kx == th.x && ix <= (int)th.y)) atomicOr(&sh.bitmap[ix >> 5], 1u << (ix & 31));
          }
        }
      }
    }
  }
  __syncthreads();
  return fast;
}

struct SelectArgs {
  const float* logits;
  int64_t ld;
  int q_begin, q_end;
  const int32_t* cu;
  const int32_t* cu_pools;
  int B, T, kpool, k_sel, width, tail_on, max_pools, list_cap;
  int32_t* out_ids;     // [rows, K_sel] global pool ids, or null
  int32_t* out_tok;     // [rows, width] token ids with the tail, or null
  // a second row range after the first (none when q_end2 <= q_begin2)
  const float* logits2;
  int64_t ld2;
  int q_begin2, q_end2;
  int32_t* out_ids2;
  int32_t* out_tok2;
  // decode rows (dec_len not null): row r is the last token of a sequence of
  // dec_len[r] tokens whose pools start at row dec_pool0[r] and whose token
  // ids start at dec_base[r] (0 when dec_base is null)
  const int32_t* dec_len;
  const int32_t* dec_pool0;
  const int32_t* dec_base;
};

// Row facts of decode row r, in the form query_info gives a prefill row.
__device__ __forceinline__ QueryInfo decode_info(const SelectArgs& a, int r) {
  QueryInfo qi;
  const int L = max(a.dec_len[r], 0);
  qi.doc = r;
  qi.start = a.dec_base ? a.dec_base[r] : 0;
  qi.pool0 = a.dec_pool0[r];
  qi.i = L - 1;
  qi.n_c = min(L / a.kpool, a.max_pools);
  return qi;
}

template <int NT, int G, bool VEC4>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  constexpr int NW = NT / 64;
  constexpr int E = 4 * G;                       // values per thread
  constexpr int LPL = list_per_lane(NT);
  using Sh = SelectShared<NT, G>;
  __shared__ Sh sh;
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  uint2* list = reinterpret_cast<uint2*>(dyn);      // list_cap (value bits, index) pairs
  const int rows1 = a.q_end - a.q_begin;
  const bool second = (int)blockIdx.x >= rows1;
  const float* __restrict__ logits = second ? a.logits2 : a.logits;
  const int64_t ld = second ? a.ld2 : a.ld;
  const int k_sel = a.k_sel, kpool = a.kpool, list_cap = a.list_cap;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int r = second ? (int)blockIdx.x - rows1 : (int)blockIdx.x;
  const int t = (second ? a.q_begin2 : a.q_begin) + r;
  if (t >= (second ? a.q_end2 : a.q_end)) return;
  const QueryInfo qi = a.dec_len ? decode_info(a, r)
                                 : query_info(a.cu, a.cu_pools, a.B, a.T, kpool, a.max_pools, t);
  const int n_c = qi.n_c;
  const int n_sel = n_c < k_sel ? n_c : k_sel;
  const int tail = a.tail_on ? (qi.i + 1) % kpool : 0;
  const int tail_base = qi.start + n_c * kpool;
  int32_t* const ids_base = second ? a.out_ids2 : a.out_ids;
  int32_t* const tok_base = second ? a.out_tok2 : a.out_tok;
  int32_t* oid = ids_base ? ids_base + (size_t)r * k_sel : nullptr;
  int32_t* otok = tok_base ? tok_base + (size_t)r * a.width : nullptr;

  // token slots from n_sel * kpool on: the tail tokens, then -1
  auto write_tail = [&]() {
    if (!otok) return;
    const int from = n_sel * kpool;
    if (VEC4) {
      for (int gi = (from >> 2) + tid; gi < (a.width >> 2); gi += NT) {
        int e[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int jj = gi * 4 + c - from;
          e[c] = jj < tail ? tail_base + jj : -1;
        }
        *reinterpret_cast<int4*>(otok + gi * 4) = make_int4(e[0], e[1], e[2], e[3]);
      }
    } else {
      for (int j = from + tid; j < a.width; j += NT) {
        const int jj = j - from;
        otok[j] = jj < tail ? tail_base + jj : -1;
      }
    }
  };
  // doc-local pool p is the pos-th chosen pool
  auto emit = [&](int pos, int p) {
    if (oid) oid[pos] = qi.pool0 + p;
    if (otok) {
      const int base = qi.start + p * kpool;
      if (VEC4) {
        *reinterpret_cast<int4*>(otok + pos * 4) = make_int4(base, base + 1, base + 2, base + 3);
      } else {
        for (int c = 0; c < kpool; ++c) otok[pos * kpool + c] = base + c;
      }
    }
  };

  if (n_c <= k_sel) {
    // every causal pool: ids pool0 .., tokens start .. start + n_c kpool + tail - 1
    if (oid)
      for (int j = tid; j < k_sel; j += NT) oid[j] = j < n_c ? qi.pool0 + j : -1;
    if (otok) {
      const int nt = n_c * kpool + tail;
      if (VEC4) {
        for (int gi = tid; gi < (a.width >> 2); gi += NT) {
          int e[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) e[c] = gi * 4 + c < nt ? qi.start + gi * 4 + c : -1;
          *reinterpret_cast<int4*>(otok + gi * 4) = make_int4(e[0], e[1], e[2], e[3]);
        }
      } else {
        for (int j = tid; j < a.width; j += NT) otok[j] = j < nt ? qi.start + j : -1;
      }
    }
    return;
  }
  const int ng = (n_c + 4 * NT - 1) / (4 * NT);      // groups holding valid values
  const int nwords = (n_c + 31) >> 5;
  auto idx_of = [&](int g, int c) { return (g * NT + tid) * 4 + c; };

  // Short rows (at most GL groups per thread) take the lean path, the others
  // the sampled level and the list.
  constexpr int GL = G < 3 ? G : 3;
  const float* row = logits + (size_t)r * ld;
  bool fast;
  if (ng <= GL) {
    fast = lean_row<NT, G, GL>(sh, row, (int)ld, n_c, k_sel, nwords);
  } else {
    // ---- 1. load the row. All loads are issued before any value is used, so a
    // wave keeps its loads in flight together. Groups below ng - 1 are full and
    // load through a uniform base; the last group clamps its addresses into the
    // row and masks slots past n_c to NaN (which never reaches the level below
    // and ranks as -inf).
    const uint8_t* rowb = reinterpret_cast<const uint8_t*>(row);
    const int lastg = ng - 1;
    float4 raw[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g < lastg) {
        raw[g] = *reinterpret_cast<const float4*>(rowb + g * NT * 16 + tid * 16);
      } else if (g == lastg) {
        const int off = min(g * NT * 16 + tid * 16, ((int)ld - 4) * 4);
        raw[g] = *reinterpret_cast<const float4*>(rowb + off);
      } else {
        raw[g] = make_float4(NAN, NAN, NAN, NAN);
      }
    }
    float v[E];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      v[4 * g + 0] = raw[g].x; v[4 * g + 1] = raw[g].y; v[4 * g + 2] = raw[g].z; v[4 * g + 3] = raw[g].w;
      if (g == lastg) {
        const int base = (g * NT + tid) * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[4 * g + c] = base + c < n_c ? v[4 * g + c] : NAN;
      }
    }
    forget(v);

    // ---- 2. sample: value (g, (g / 2) mod 4) of every even group g, its
    // min / max, and a value-linear histogram of it
    float smn = INFINITY, smx = -INFINITY;
    int ns = 0;
#pragma unroll
    for (int g = 0; g < G; g += 2) {
      if (g < ng) {
        const float x = v[4 * g + ((g >> 1) & 3)];
        smn = fminf(smn, x);
        smx = fmaxf(smx, x);
        ns += x == x;
      }
    }
    smn = wave_min(smn);
    smx = wave_max(smx);
    ns = wave_sum(ns);
    if (lane == 0) { sh.red_f[0][wid] = smn; sh.red_f[1][wid] = smx; sh.red_n[wid] = ns; }
    for (int j = tid; j <= kBins; j += NT) sh.hist[j] = 0u;
    for (int j = tid; j < nwords; j += NT) sh.bitmap[j] = 0u;
    if (tid == 0) { sh.cand_cnt = 0; sh.res[0] = sh.res[1] = sh.res[2] = 0; }
    __syncthreads();
    smn = sh.red_f[0][0]; smx = sh.red_f[1][0];
    int S = sh.red_n[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      smn = fminf(smn, sh.red_f[0][w]);
      smx = fmaxf(smx, sh.red_f[1][w]);
      S += sh.red_n[w];
    }
    const float srange = smx - smn;
    fast = S > 0 && (srange > 0.f) && (srange <= 3.0e38f);   // finite, not constant

    if (fast) {
      const float inv = (float)kBins / srange;
#pragma unroll
      for (int g = 0; g < G; g += 2) {
        if (g < ng) {
          const float x = v[4 * g + ((g >> 1) & 3)];
          if (x == x) atomicAdd(&sh.hist[vbin(x, smn, inv)], 1u);
        }
      }
      __syncthreads();
      // sample rank of the level: a 25 % margin over the expected count of
      // chosen values in the sample plus four standard deviations
      const float expect = (float)k_sel * (float)S / (float)n_c;
      int m = (int)ceilf(1.25f * expect + 4.f * sqrtf(expect) + 4.f);
      m = m < S ? m : S;
      find_bin<NT, G, kBins>(sh, m > 0 ? m : 1);
      const float L = smn + (float)sh.res[0] * (srange / (float)kBins);

      // ---- 3. compact every value >= L into the LDS list. Each wave appends
      // to its own segment of seg_cap entries: a ballot gives each lane its
      // prefix, the running count stays scalar, and a (value, index) pair is one
      // 8-byte LDS write. A wave that overflows its segment keeps writing into
      // the segment's last slot; its count records the overflow.
      const int seg_cap = list_cap / NW;                 // at most 64 * LPL
      uint2* seg = list + wid * seg_cap;
      int running = 0;
      forget(v);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g < ng) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const bool keep = v[4 * g + c] >= L;
            const uint64_t m = __ballot(keep);
            // entries past the segment's end all land in its last slot; the
            // count still records the overflow, which sends the row to the
            // general path
            if (keep) {
              const int pos = min(running + popc_lt(m), seg_cap - 1);
              seg[pos] = make_uint2(__float_as_uint(v[4 * g + c]), (uint32_t)idx_of(g, c));
            }
            running += __popcll(m);
          }
        }
      }
      if (lane == 0) sh.seg_cnt[wid] = running;
      for (int j = tid; j <= kBins; j += NT) sh.hist[j] = 0u;
      __syncthreads();
      int total = 0;
      bool overflow = false;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = sh.seg_cnt[w];
        overflow |= c > seg_cap;
        total += c;
      }
      if (overflow || total < k_sel) {
        fast = false;                                    // the level missed: general path
      } else {
        // ---- 4. exact threshold on the list. Each wave takes its own segment
        // into registers once (lane l holds entries l, l + 64, ...); min / max,
        // histogram, candidate gather and marking all work from there.
        float ev[LPL];
        int ei[LPL];
#pragma unroll
        for (int i = 0; i < LPL; ++i) {
          const int j = lane + 64 * i;
          const uint2 e = seg[j < running ? j : 0];
          ev[i] = j < running ? __uint_as_float(e.x) : NAN;   // list values are never NaN
          ei[i] = (int)e.y;
        }
        // histogram range: every list value is >= L, and all but the few
        // above the sample's maximum are <= smx (those land in the top bin,
        // which keeps the bins monotone); no reduction over the list needed
        const float lmn = L, lmx = smx;
        const float lrange = lmx - lmn;
        if (!(lrange > 0.f) || !(lrange <= 3.0e38f)) {
          fast = false;                                  // ties or infinities: general path
        } else {
          const float linv = (float)kBins / lrange;
#pragma unroll
          for (int i = 0; i < LPL; ++i)
            if (ev[i] == ev[i]) atomicAdd(&sh.hist[vbin(ev[i], lmn, linv)], 1u);
          __syncthreads();
          find_bin<NT, G, kBins>(sh, k_sel);
          const int bstar = sh.res[0];
          const int k_in = k_sel - sh.res[1];
          const int c_in = sh.res[2];
          if (c_in > NT) {
            fast = false;                                // crowded bin: general path
          } else {
#pragma unroll
            for (int i = 0; i < LPL; ++i) {
              if (ev[i] == ev[i] && vbin(ev[i], lmn, linv) == bstar) {
                const int slot = atomicAdd(&sh.cand_cnt, 1);
                sh.cand_key[slot] = f32_order_key(ev[i]);
                sh.cand_idx[slot] = ei[i];
              }
            }
            __syncthreads();
            const uint2 th = threshold_of<NT, G>(sh, c_in, k_in, lane);
            const uint32_t tk = th.x;
            const int ti = (int)th.y;
            // ---- 5a. chosen list entries set their bitmap bits
#pragma unroll
            for (int i = 0; i < LPL; ++i) {
              if (ev[i] == ev[i]) {
                const uint32_t kx = f32_order_key(ev[i]);
                if (kx > tk || (kx == tk && ei[i] <= ti)) atomicOr(&sh.bitmap[ei[i] >> 5], 1u << (ei[i] & 31));
              }
            }
          }
        }
      }
      __syncthreads();
    }
  }

  if (!fast) {
    // ---- general path: histogram rounds over keys, then over the index. It
    // is rare, so it re-reads the row instead of holding keys in registers.
    auto value_at = [&](int e) -> float {
      const int ix = idx_of(e >> 2, e & 3);
      return ix < n_c ? row[ix] : NAN;
    };
    uint64_t cand = 0, sel = 0;
#pragma unroll 1
    for (int e = 0; e < E; ++e) cand |= (uint64_t)(idx_of(e >> 2, e & 3) < n_c) << e;
    int k = k_sel, c_cnt = n_c, mode = 0;
#pragma unroll 1
    while (true) {
      if (c_cnt == k) { sel |= cand; break; }
      if (c_cnt <= NT) {
        if (tid == 0) sh.cand_cnt = 0;
        __syncthreads();
#pragma unroll 1
        for (int e = 0; e < E; ++e) {
          if ((cand >> e) & 1ull) {
            const int slot = atomicAdd(&sh.cand_cnt, 1);
            sh.cand_key[slot] = f32_order_key(value_at(e));
            sh.cand_idx[slot] = idx_of(e >> 2, e & 3);
          }
        }
        __syncthreads();
        if (tid < c_cnt) {
          const uint32_t mk = sh.cand_key[tid];
          const int mi = sh.cand_idx[tid];
          int rank = 0;
          for (int q = 0; q < c_cnt; ++q) {
            const uint32_t okey = sh.cand_key[q];
            rank += (okey > mk) || (okey == mk && sh.cand_idx[q] < mi);
          }
          if (rank == k - 1) { sh.th_key = mk; sh.th_idx = mi; }
        }
        __syncthreads();
        const uint32_t tk = sh.th_key;
        const int ti = sh.th_idx;
#pragma unroll 1
        for (int e = 0; e < E; ++e) {
          if ((cand >> e) & 1ull) {
            const uint32_t ke = f32_order_key(value_at(e));
            const int ix = idx_of(e >> 2, e & 3);
            if (ke > tk || (ke == tk && ix <= ti)) sel |= 1ull << e;
          }
        }
        break;
      }
      uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll 1
      for (int e = 0; e < E; ++e) {
        if ((cand >> e) & 1ull) {
          const uint32_t ck = mode ? ~(uint32_t)idx_of(e >> 2, e & 3) : f32_order_key(value_at(e));
          lo = ck < lo ? ck : lo;
          hi = ck > hi ? ck : hi;
        }
      }
      lo = wave_min(lo);
      hi = wave_max(hi);
      if (lane == 0) { sh.red_u[0][wid] = lo; sh.red_u[1][wid] = hi; }
      for (int j = tid; j <= kKeyBins; j += NT) sh.hist[j] = 0u;
      __syncthreads();
      lo = sh.red_u[0][0]; hi = sh.red_u[1][0];
      for (int w = 1; w < NW; ++w) {
        lo = sh.red_u[0][w] < lo ? sh.red_u[0][w] : lo;
        hi = sh.red_u[1][w] > hi ? sh.red_u[1][w] : hi;
      }
      if (lo == hi) {          // every remaining key ties: continue on the index
        mode = 1;
        __syncthreads();
        continue;
      }
      const int bits = 32 - __clz(hi - lo);
      const int shift = bits > kLogKeyBins ? bits - kLogKeyBins : 0;
#pragma unroll 1
      for (int e = 0; e < E; ++e) {
        if ((cand >> e) & 1ull) {
          const uint32_t ck = mode ? ~(uint32_t)idx_of(e >> 2, e & 3) : f32_order_key(value_at(e));
          atomicAdd(&sh.hist[(ck - lo) >> shift], 1u);
        }
      }
      __syncthreads();
      find_bin<NT, G, kKeyBins>(sh, k);
      const uint32_t bstar = (uint32_t)sh.res[0];
      const int n_above = sh.res[1];
      const int n_in = sh.res[2];
#pragma unroll 1
      for (int e = 0; e < E; ++e) {
        if ((cand >> e) & 1ull) {
          const uint32_t ck = mode ? ~(uint32_t)idx_of(e >> 2, e & 3) : f32_order_key(value_at(e));
          const uint32_t b = (ck - lo) >> shift;
          if (b > bstar) sel |= 1ull << e;
          if (b != bstar) cand &= ~(1ull << e);
        }
      }
      k -= n_above;
      c_cnt = n_in;
      __syncthreads();
    }
#pragma unroll 1
    for (int e = 0; e < E; ++e) {
      if ((sel >> e) & 1ull) {
        const int ix = idx_of(e >> 2, e & 3);
        atomicOr(&sh.bitmap[ix >> 5], 1u << (ix & 31));
      }
    }
    __syncthreads();
  }

  // ---- 5b. bitmap -> ascending pool ids: thread tid owns words
  // [tid * wpt, (tid + 1) * wpt); a block prefix sum of bit counts places them
  const int wpt = (nwords + NT - 1) / NT;
  int cnt = 0;
  for (int i = 0; i < wpt; ++i) {
    const int w = tid * wpt + i;
    if (w < nwords) cnt += __popc(sh.bitmap[w]);
  }
  const int incl = wave_prefix_sum(cnt);
  if (lane == 63) sh.wave_tot[wid] = incl;
  __syncthreads();
  int pos = incl - cnt;
#pragma unroll
  for (int w = 0; w < NW; ++w) pos += w < wid ? sh.wave_tot[w] : 0;
  for (int i = 0; i < wpt; ++i) {
    const int w = tid * wpt + i;
    uint32_t m = w < nwords ? sh.bitmap[w] : 0u;
    while (m) {
      const int bit = __ffs(m) - 1;
      if (pos < k_sel) emit(pos, w * 32 + bit);
      ++pos;
      m &= m - 1;
    }
  }
  write_tail();
}

// LDS list capacity: one segment of 64 * list_per_lane entries per wave. The
// sampled level keeps about 1.25 K_sel plus a few sample standard deviations
// in all, spread evenly over the waves; rows whose share overflows a segment
// take the general path.
// A wave of a G-group row holds at most 4 G values, so short rows need less.
static int list_capacity(int nt, int g) {
  const int lpl = list_per_lane(nt);
  return (nt / 64) * 64 * (4 * g < lpl ? 4 * g : lpl);
}

template <int NT, int G>
static void launch_sel(SelectArgs a, hipStream_t st) {
  a.list_cap = list_capacity(NT, G);
  const size_t lds = (size_t)a.list_cap * 8;
  if (a.kpool == 4 && (a.width & 3) == 0)
    select_kernel<NT, G, true><<<(a.q_end - a.q_begin) + max(a.q_end2 - a.q_begin2, 0), NT, lds, st>>>(a);
  else
    select_kernel<NT, G, false><<<(a.q_end - a.q_begin) + max(a.q_end2 - a.q_begin2, 0), NT, lds, st>>>(a);
}

static void launch_select_args(SelectArgs& a, hipStream_t st) {
  const int max_pools = a.max_pools;
  if (max_pools <= 1024) launch_sel<256, 1>(a, st);
  else if (max_pools <= 2048) launch_sel<256, 2>(a, st);
  else if (max_pools <= 4096) launch_sel<256, 4>(a, st);
  else if (max_pools <= 8192) launch_sel<256, 8>(a, st);
  else if (max_pools <= 10240) launch_sel<256, 10>(a, st);
  else if (max_pools <= 12288) launch_sel<256, 12>(a, st);
  else if (max_pools <= 14336) launch_sel<256, 14>(a, st);
  else if (max_pools <= 16384) launch_sel<256, 16>(a, st);
  else if (max_pools <= 32768) launch_sel<512, 16>(a, st);
  else launch_sel<1024, 16>(a, st);
}

void launch_select(const float* logits, int64_t ld, int q_begin, int q_end,
                   const int32_t* cu, const int32_t* cu_pools, int B, int T, int kpool,
                   int k_sel, int width, int tail_on, int max_pools, int32_t* out_ids,
                   int32_t* out_tok, hipStream_t st) {
  if (q_end <= q_begin) return;
  SelectArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.q_begin = q_begin;
  a.q_end = q_end;
  a.cu = cu;
  a.cu_pools = cu_pools;
  a.B = B;
  a.T = T;
  a.kpool = kpool;
  a.k_sel = k_sel;
  a.width = width;
  a.tail_on = tail_on;
  // n_c(t) <= (t + 1) / kpool <= q_end / kpool whatever the documents are,
  // so a chunk of early rows takes the variant sized for its longest row
  // (fewer registers, more rows in flight per CU)
  const int bound = q_end / kpool;
  if (bound < max_pools) max_pools = bound < 1 ? 1 : bound;
  a.max_pools = max_pools;
  a.out_ids = out_ids;
  a.out_tok = out_tok;
  launch_select_args(a, st);
}

void launch_select2(const float* logits, int64_t ld, int q_begin, int q_end,
                    const float* logits2, int64_t ld2, int q_begin2, int q_end2,
                    const int32_t* cu, const int32_t* cu_pools, int B, int T, int kpool,
                    int k_sel, int width, int tail_on, int max_pools, int32_t* out_ids,
                    int32_t* out_tok, hipStream_t st) {
  if (q_end <= q_begin) return;
  SelectArgs a{};
  a.logits = logits;
  a.ld = ld;
  a.q_begin = q_begin;
  a.q_end = q_end;
  a.logits2 = logits2;
  a.ld2 = ld2;
  a.q_begin2 = q_begin2;
  a.q_end2 = q_end2;
  a.cu = cu;
  a.cu_pools = cu_pools;
  a.B = B;
  a.T = T;
  a.kpool = kpool;
  a.k_sel = k_sel;
  a.width = width;
  a.tail_on = tail_on;
  const int bound = max(q_end, q_end2) / kpool;
  if (bound < max_pools) max_pools = bound < 1 ? 1 : bound;
  a.max_pools = max_pools;
  a.out_ids = out_ids ? out_ids + (size_t)q_begin * k_sel : nullptr;
  a.out_tok = out_tok + (size_t)q_begin * width;
  a.out_ids2 = out_ids ? out_ids + (size_t)q_begin2 * k_sel : nullptr;
  a.out_tok2 = out_tok + (size_t)q_begin2 * width;
  launch_select_args(a, st);
}

void launch_select_decode(const float* scores, int64_t ld, int B, const int32_t* seq_lens,
                          const int32_t* pool_start, const int32_t* token_base, int kpool,
                          int k_sel, int width, int tail_on, int max_pools, int32_t* out_ids,
                          int32_t* out_tok, hipStream_t st) {
  if (B <= 0) return;
  SelectArgs a{};
  a.logits = scores;
  a.ld = ld;
  a.q_begin = 0;
  a.q_end = B;
  a.B = B;
  a.kpool = kpool;
  a.k_sel = k_sel;
  a.width = width;
  a.tail_on = tail_on;
  a.max_pools = max_pools < 1 ? 1 : max_pools;
  a.out_ids = out_ids;
  a.out_tok = out_tok;
  a.dec_len = seq_lens;
  a.dec_pool0 = pool_start;
  a.dec_base = token_base;
  // A decode batch can have fewer rows than the GPU has CUs; then the time is
  // one row's latency, which 1024 threads per row shorten
  if (B <= 512) {
    const int mp = a.max_pools;
    if (mp <= 4096) launch_sel<1024, 1>(a, st);
    else if (mp <= 8192) launch_sel<1024, 2>(a, st);
    else if (mp <= 16384) launch_sel<1024, 4>(a, st);
    else if (mp <= 32768) launch_sel<1024, 8>(a, st);
    else launch_sel<1024, 16>(a, st);
    return;
  }
  launch_select_args(a, st);
}

}  // namespace kpool
