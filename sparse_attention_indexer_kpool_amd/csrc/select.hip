// Step 3 of the KPool indexer: per-query pool top-k.
//
// Megatron-LM PR #7054, section "3. KPool DSA indexer + NoPE": the indexer's
// top-k runs over pools and keeps index_topk // kpool of them. xtuner PR #2108
// (selector fix commit) names a radix-select row selector as the production
// alternative to a full sort; this kernel is an exact histogram selection
// written for gfx950.
//
// One workgroup of 256 (or 1024) threads per query row; HBM-bound: each causal
// score is read once with coalesced 16-byte loads and stays in registers.
//
//   1. min / max of the row (invalid tail slots hold NaN, which min / max skip
//      and which ranks as -inf).
//   2. One histogram of 1024 bins that are linear in the value,
//      bin = trunc((x - min) * 1024 / (max - min)) clamped to [0, 1023]. FP32
//      subtraction, multiplication and truncation are monotone, so bins
//      follow the order of the values exactly; equal values share a bin and a
//      larger bin means a larger value. Linear bins spread typical score
//      distributions thinly, which keeps LDS atomic collisions rare.
//   3. The bin b* holding the k-th largest value, found by a suffix scan of
//      the histogram.
//   4. The few candidates of b* are gathered to LDS and ranked against each
//      other (larger value first, ties to the lower index), which gives the
//      exact threshold element (tau, idx_tau).
//   5. An element is chosen iff x > tau, or x == tau and idx <= idx_tau. The
//      chosen pool ids are written in ascending order: per-wave ballot counts
//      of every 1024-element group are scanned once, then each lane writes at
//      its prefix.
//
// Rows whose values are not all finite, whose values are all equal or whose
// threshold bin is crowded fall back to a general path: repeated histogram
// rounds over order-preserving 32-bit keys (NaN -> -inf, -0 -> +0) with bins
// that are a right shift of key - min, then over the pool index once all
// remaining keys tie. Rows with n_c <= K_sel select every causal pool and read
// no logits.

#include "kpool_device.h"
#include "kpool_internal.h"

namespace kpool {

// Makes the compiler forget what it knows about the values, so per-element
// results of one phase (bins, ballots) are recomputed in the next instead of
// being held in registers across a barrier.
template <int E>
__device__ __forceinline__ void forget(float (&v)[E]) {
#pragma unroll
  for (int e = 0; e < E; ++e) asm volatile("" : "+v"(v[e]));
}

constexpr int kFastBins = 1024;     // value-linear bins of the first round
constexpr int kLogKeyBins = 10;     // key-space bins of the general path
constexpr int kKeyBins = 1 << kLogKeyBins;

template <int NT>
struct SelectShared {
  static constexpr int NW = NT / 64;
  uint32_t hist[kFastBins + 1];       // + one bin for non-candidates
  float red_f[2][NW];
  uint32_t red_u[2][NW];
  int wave_tot[NW];
  int res[3];                         // b*, count above b*, count in b*
  float cand_val[NT];
  uint32_t cand_key[NT];
  int cand_idx[NT];
  int cand_cnt;
  float th_val;
  uint32_t th_key;
  int th_idx;
  int grp[64 * NW];
};

// Suffix scan of the histogram: the bin b* with (count above b*) < k <=
// (count above b*) + hist[b*]. Results land in sh.res; ends with a barrier.
template <int NT, int NBINS>
__device__ __forceinline__ void find_bin(SelectShared<NT>& sh, int k) {
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

template <int NT, int G>
__global__ __launch_bounds__(NT) void select_kernel(
    const float* __restrict__ logits, int64_t ld, int q_begin, int q_end,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_pools, int B, int T,
    int kpool, int k_sel, int max_pools, int32_t* __restrict__ out_ids) {
  constexpr int NW = NT / 64;
  constexpr int E = 4 * G;                    // values per thread
  static_assert(E <= 64 && G * NW <= 64 * NW, "sizes");
  __shared__ SelectShared<NT> sh;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  const int r = blockIdx.x;
  const int t = q_begin + r;
  if (t >= q_end) return;
  const QueryInfo qi = query_info(cu, cu_pools, B, T, kpool, max_pools, t);
  const int n_c = qi.n_c;
  int32_t* o = out_ids + (size_t)r * k_sel;
  if (n_c <= k_sel) {
    for (int j = tid; j < k_sel; j += NT) o[j] = j < n_c ? qi.pool0 + j : -1;
    return;
  }
  const int ng = (n_c + 4 * NT - 1) / (4 * NT);      // groups holding valid values
  auto idx_of = [&](int g, int c) { return (g * NT + tid) * 4 + c; };

  // ---- 1. load (invalid slots = NaN) and the row's min / max
  // Groups below ng are loaded by every lane (uniform branch); a lane whose
  // slots lie past n_c reads an in-row address (clamped to the row's last 16
  // bytes) and masks the values to NaN without branching.
  const float* row = logits + (size_t)r * ld;
  float v[E];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float4 f = make_float4(NAN, NAN, NAN, NAN);
    if (g < ng) {
      const int base = (g * NT + tid) * 4;
      const int addr = base < (int)ld - 4 ? base : (int)ld - 4;
      f = *reinterpret_cast<const float4*>(row + addr);
      f.x = base + 0 < n_c ? f.x : NAN;
      f.y = base + 1 < n_c ? f.y : NAN;
      f.z = base + 2 < n_c ? f.z : NAN;
      f.w = base + 3 < n_c ? f.w : NAN;
    }
    v[4 * g + 0] = f.x; v[4 * g + 1] = f.y; v[4 * g + 2] = f.z; v[4 * g + 3] = f.w;
  }
  forget(v);
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) { mn = fminf(mn, v[e]); mx = fmaxf(mx, v[e]); }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) { sh.red_f[0][wid] = mn; sh.red_f[1][wid] = mx; }
  for (int j = tid; j <= kFastBins; j += NT) sh.hist[j] = 0u;
  __syncthreads();
  mn = sh.red_f[0][0]; mx = sh.red_f[1][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) { mn = fminf(mn, sh.red_f[0][w]); mx = fmaxf(mx, sh.red_f[1][w]); }
  const float range = mx - mn;
  bool fast = (range > 0.f) && (range <= 3.0e38f);    // finite, not all equal, no overflow

  float tau = 0.f;
  int idx_tau = 0;
  if (fast) {
    // ---- 2. value-linear histogram (NaN and invalid slots land in bin 0)
    const float inv = (float)kFastBins / range;
    auto bin_of = [&](float x) {
      // fmaxf returns 0 for a NaN argument, so NaN lands in bin 0
      return (int)fminf(fmaxf((x - mn) * inv, 0.f), (float)(kFastBins - 1));
    };
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g < ng) {
#pragma unroll
        for (int c = 0; c < 4; ++c) atomicAdd(&sh.hist[bin_of(v[4 * g + c])], 1u);
      }
    }
    __syncthreads();
    forget(v);
    if (tid == 0) sh.hist[0] -= (uint32_t)(ng * 4 * NT - n_c);   // drop the invalid slots
    __syncthreads();
    // ---- 3. threshold bin
    find_bin<NT, kFastBins>(sh, k_sel);
    const int bstar = sh.res[0];
    const int k_in = k_sel - sh.res[1];              // still to take from b*
    const int c_in = sh.res[2];
    if (c_in > NT) {
      fast = false;                                  // crowded bin: general path
    } else {
      // ---- 4. gather b* and rank its candidates
      if (tid == 0) sh.cand_cnt = 0;
      __syncthreads();
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (g < ng) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float x = v[4 * g + c];
            const int ix = idx_of(g, c);
            // invalid slots are NaN and sit in bin 0
            if (bin_of(x) == bstar && (bstar != 0 || ix < n_c)) {
              const int slot = atomicAdd(&sh.cand_cnt, 1);
              sh.cand_key[slot] = f32_order_key(x);
              sh.cand_idx[slot] = ix;
            }
          }
        }
      }
      __syncthreads();
      if (tid < c_in) {
        const uint32_t mk = sh.cand_key[tid];
        const int mi = sh.cand_idx[tid];
        int rank = 0;
        for (int m = 0; m < c_in; ++m) {
          const uint32_t okey = sh.cand_key[m];
          rank += (okey > mk) || (okey == mk && sh.cand_idx[m] < mi);
        }
        if (rank == k_in - 1) { sh.th_key = mk; sh.th_idx = mi; }
      }
      __syncthreads();
      const uint32_t tk = sh.th_key;
      idx_tau = sh.th_idx;
      // back from key to value; a NaN threshold ranks as -inf (key of -inf)
      const uint32_t u = (tk & 0x80000000u) ? (tk & 0x7fffffffu) : ~tk;
      tau = __uint_as_float(u);
      if (!(fabsf(tau) <= 3.402823466e38f)) fast = false;   // +-inf threshold: general path
    }
    __syncthreads();
  }

  uint64_t sel = 0;    // bit e: value e is chosen (general path only)
  if (!fast) {
    // ---- general path: histogram rounds over keys, then over the index. It
    // is rare, so it re-reads the row instead of holding keys in registers.
    auto value_at = [&](int e) -> float {
      const int ix = idx_of(e >> 2, e & 3);
      return ix < n_c ? row[ix] : NAN;
    };
    uint64_t cand = 0;
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
          for (int m = 0; m < c_cnt; ++m) {
            const uint32_t okey = sh.cand_key[m];
            rank += (okey > mk) || (okey == mk && sh.cand_idx[m] < mi);
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
      find_bin<NT, kKeyBins>(sh, k);
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
  }

  // ---- 5. write the chosen pools in ascending order
  forget(v);
  auto chosen = [&](int g, int c) -> bool {
    if (!fast) return (sel >> (4 * g + c)) & 1ull;
    const float x = v[4 * g + c];
    return x > tau || (x == tau && idx_of(g, c) <= idx_tau);
  };
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g < ng) {
      int tot = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) tot += __popcll(__ballot(chosen(g, c)));
      if (lane == 0) sh.grp[g * NW + wid] = tot;
    }
  }
  __syncthreads();
  forget(v);
  if (wid == 0) {
    int carry = 0;
    for (int base = 0; base < ng * NW; base += 64) {
      const int j = base + lane;
      const int x = j < ng * NW ? sh.grp[j] : 0;
      const int incl = wave_prefix_sum(x);
      if (j < ng * NW) sh.grp[j] = carry + incl - x;
      carry += __shfl(incl, 63, 64);
    }
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g < ng) {
      int pos = sh.grp[g * NW + wid];
      uint64_t m[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) m[c] = __ballot(chosen(g, c));
      if ((m[0] | m[1] | m[2] | m[3]) == 0ull) continue;
#pragma unroll
      for (int c = 0; c < 4; ++c) pos += popc_lt(m[c]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if ((m[c] >> lane) & 1ull) {
          if (pos < k_sel) o[pos] = qi.pool0 + idx_of(g, c);
          ++pos;
        }
      }
    }
  }
}

template <int NT, int G>
static void launch_sel(const float* logits, int64_t ld, int q_begin, int q_end,
                       const int32_t* cu, const int32_t* cu_pools, int B, int T, int kpool,
                       int k_sel, int max_pools, int32_t* out_ids, hipStream_t st) {
  select_kernel<NT, G><<<q_end - q_begin, NT, 0, st>>>(
      logits, ld, q_begin, q_end, cu, cu_pools, B, T, kpool, k_sel, max_pools, out_ids);
}

void launch_select(const float* logits, int64_t ld, int q_begin, int q_end,
                   const int32_t* cu, const int32_t* cu_pools, int B, int T, int kpool,
                   int k_sel, int max_pools, int32_t* out_ids, hipStream_t st) {
  if (q_end <= q_begin) return;
#define KP_SEL(NT, G) launch_sel<NT, G>(logits, ld, q_begin, q_end, cu, cu_pools, B, T, kpool, k_sel, max_pools, out_ids, st)
  if (max_pools <= 1024) KP_SEL(256, 1);
  else if (max_pools <= 2048) KP_SEL(256, 2);
  else if (max_pools <= 4096) KP_SEL(256, 4);
  else if (max_pools <= 8192) KP_SEL(256, 8);
  else if (max_pools <= 16384) KP_SEL(256, 16);
  else if (max_pools <= 32768) KP_SEL(512, 16);
  else KP_SEL(1024, 16);
#undef KP_SEL
}

}  // namespace kpool
