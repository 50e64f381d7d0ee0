// Device-side helpers shared by the KPool kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kpool {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
  return __uint_as_float(h16 << 16);
}

// FP32 -> BF16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Document of token t: the largest b in [0, B) with cu[b] <= t. For
// non-decreasing cu this is the document that holds t; for any contents the
// result stays in [0, B).
__device__ __forceinline__ int doc_of(const int32_t* __restrict__ cu, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Row facts of query t, clamped so that every derived index stays inside
// the buffers even when cu_seqlens breaks its precondition.
struct QueryInfo {
  int doc;      // b
  int start;    // cu[b]
  int pool0;    // cuP[b]
  int n_c;      // causal pools, <= max_pools and <= pools of the document
  int i;        // position in the document
};

__device__ __forceinline__ QueryInfo query_info(const int32_t* __restrict__ cu,
                                                const int32_t* __restrict__ cuP, int B,
                                                int T, int kpool, int max_pools, int t) {
  QueryInfo r;
  r.doc = doc_of(cu, B, t);
  r.start = clampi(cu[r.doc], 0, t);
  int pool_cap = T / kpool;
  r.pool0 = clampi(cuP[r.doc], 0, pool_cap);
  int pools_doc = clampi(cuP[r.doc + 1] - r.pool0, 0, pool_cap - r.pool0);
  r.i = t - r.start;
  int nc = (r.i + 1) / kpool;
  nc = nc < max_pools ? nc : max_pools;
  r.n_c = nc < pools_doc ? nc : pools_doc;
  return r;
}

// Order-preserving map of FP32 to uint32 (larger float -> larger key). NaN
// maps to the key of -inf and -0 to the key of +0, so keys compare exactly as
// the floats do with NaN ranked as -inf.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) u = 0xff800000u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanemask_lt() { return (1ull << __lane_id()) - 1ull; }

__device__ __forceinline__ int popc_lt(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Cross-lane helpers on DPP (data-parallel primitives: a VALU operand read
// from another lane of the same row of 16, or broadcast across rows), which
// cost a few cycles each instead of an LDS permute.

template <typename T>
__device__ __forceinline__ int bits_of(T v) { return __builtin_bit_cast(int, v); }
template <typename T>
__device__ __forceinline__ T from_bits(int b) { return __builtin_bit_cast(T, b); }

// Value of lane l ^ m (m = 1, 2, 4 or 8; a constant once loops unroll)
// within each row of 16 lanes: a DPP quad_perm swap for 1 and 2, and a
// ds_swizzle in bit mode (source lane (l & 31) ^ m) for 4 and 8, which
// measured faster than the two DPP moves those masks would need.
__device__ __forceinline__ float xor_lane16(float v, int m) {
  const int x = bits_of(v);
  switch (m) {
    case 1: return from_bits<float>(__builtin_amdgcn_update_dpp(x, x, 0xb1, 0xf, 0xf, false));
    case 2: return from_bits<float>(__builtin_amdgcn_update_dpp(x, x, 0x4e, 0xf, 0xf, false));
    case 4: return from_bits<float>(__builtin_amdgcn_ds_swizzle(x, (4 << 10) | 0x1f));
    default: return from_bits<float>(__builtin_amdgcn_ds_swizzle(x, (8 << 10) | 0x1f));
  }
}

// Reduction over the 64 lanes with an idempotent op (min or max); the result
// is wave-uniform. Quad swaps and row mirrors reduce each row of 16 lanes,
// row_bcast:15 / row_bcast:31 fold the rows into lane 63, read back with
// readlane. Rows a broadcast skips keep their value (op(x, x) = x).
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce_idem(T v, Op op) {
  static_assert(sizeof(T) == 4, "32-bit values");
  int x = bits_of(v);
  x = bits_of(op(from_bits<T>(x), from_bits<T>(__builtin_amdgcn_update_dpp(x, x, 0xb1, 0xf, 0xf, false))));
  x = bits_of(op(from_bits<T>(x), from_bits<T>(__builtin_amdgcn_update_dpp(x, x, 0x4e, 0xf, 0xf, false))));
  x = bits_of(op(from_bits<T>(x), from_bits<T>(__builtin_amdgcn_update_dpp(x, x, 0x141, 0xf, 0xf, false))));
  x = bits_of(op(from_bits<T>(x), from_bits<T>(__builtin_amdgcn_update_dpp(x, x, 0x140, 0xf, 0xf, false))));
  x = bits_of(op(from_bits<T>(x), from_bits<T>(__builtin_amdgcn_update_dpp(x, x, 0x142, 0xa, 0xf, false))));
  x = bits_of(op(from_bits<T>(x), from_bits<T>(__builtin_amdgcn_update_dpp(x, x, 0x143, 0xc, 0xf, false))));
  return from_bits<T>(__builtin_amdgcn_readlane(x, 63));
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  return wave_reduce_idem(v, [](T a, T b) { return a > b ? a : b; });
}

template <typename T>
__device__ __forceinline__ T wave_min(T v) {
  return wave_reduce_idem(v, [](T a, T b) { return a < b ? a : b; });
}

// Inclusive prefix sum over the lanes of a wave: row_shr 1, 2, 4, 8 build
// the sum within each row of 16 (lanes shifted in from outside the row read
// 0), row_bcast:15 adds row 0's total to row 1 (and row 2's to row 3),
// row_bcast:31 adds rows 0-1 to rows 2-3.
__device__ __forceinline__ int wave_prefix_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

// Sum over the wave (wave-uniform).
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_prefix_sum(v), 63);
}

// Inclusive suffix sum over the lanes of a wave (lane l gets sum of l..63).
__device__ __forceinline__ int wave_suffix_sum(int v) {
  const int incl = wave_prefix_sum(v);
  return __builtin_amdgcn_readlane(incl, 63) - incl + v;
}

}  // namespace kpool
