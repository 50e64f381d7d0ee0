// Step 1 of the KPool indexer: pool offsets per document and key compression.
//
// Megatron-LM PR #7054, section "3. KPool DSA indexer + NoPE": keys are pooled
// kpool tokens at a time; per dimension, a softmax over the pool's slots of
// (per-token gate logit + per-slot position bias) weights the slot keys, with
// FP32 accumulation and a BF16 result; in a packed batch every document
// starts its own pools. SkyRL PR #2179 (the commit adopting the k-pool
// indexer) describes the same weighting of the keys.
//
// HBM-bound. Each thread owns 8 dimensions (16 bytes) of one pool: it reads
// kpool 16-byte slices of k and of the gate and writes one 16-byte slice of
// the pooled key, so a wave moves whole 256-byte rows for D = 128.

#include "kpool_device.h"
#include "kpool_internal.h"
#include "fp8_row.h"

namespace kpool {

// cu_pools[b] = sum over b' < b of floor(L_b' / kpool). One workgroup; a
// running carry walks the documents 1024 at a time. Negative lengths (a
// broken cu_seqlens) count as zero pools.
__global__ __launch_bounds__(1024) void cu_pools_kernel(const int32_t* __restrict__ cu,
                                                        int B, int kpool,
                                                        int32_t* __restrict__ cu_pools) {
  __shared__ int wave_tot[16];
  __shared__ int carry_s;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  if (tid == 0) { carry_s = 0; cu_pools[0] = 0; }
  __syncthreads();
  for (int base = 0; base < B; base += 1024) {
    int b = base + tid;
    int cnt = 0;
    if (b < B) {
      int len = cu[b + 1] - cu[b];
      cnt = len > 0 ? len / kpool : 0;
    }
    int incl = wave_prefix_sum(cnt);
    if (lane == 63) wave_tot[wid] = incl;
    __syncthreads();
    int add = carry_s;
    for (int j = 0; j < wid; ++j) add += wave_tot[j];
    if (b < B) cu_pools[b + 1] = add + incl;
    __syncthreads();
    if (tid == 1023) carry_s = add + incl;
    __syncthreads();
  }
}

// Two FP32 values -> packed BF16 pair (low half first), round to nearest
// even by gfx950's conversion instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Documents whose pool offsets the compress kernel computes itself (one
// prefix over the documents per workgroup, in LDS); beyond this a separate
// cu_pools launch comes first.
constexpr int kFusedDocs = 1024;

// KP = kpool when it is a compile-time constant, 0 for a runtime kpool.
// FUSED: the workgroup derives cu_pools from cu_seqlens (B <= kFusedDocs)
// and workgroup 0 writes it; otherwise cu_pools is an input.
// SCATTER: the T tokens are T / kpool complete pools given back to back (one
// document); pool p goes to pooled row dst_rows[p], skipped when that row is
// outside [0, dst_cap); cu and cu_pools are not used.
// FP8OUT (with SCATTER, D = 128): the BF16 pooled row goes on through the FP8
// input path; its E4M3 codes are written to row dst_rows[p] of `pooled`
// viewed as uint8 [dst_cap, 128] and its scale to row_scale[dst_rows[p]].
template <int D, int KP, bool FUSED, bool SCATTER = false, bool FP8OUT = false>
__global__ __launch_bounds__(256) void compress_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ gate,
    const float* __restrict__ ape, const int32_t* __restrict__ cu,
    int32_t* __restrict__ cu_pools, int B, int T, int kpool_rt,
    uint16_t* __restrict__ pooled, const int32_t* __restrict__ dst_rows = nullptr,
    int dst_cap = 0, float* __restrict__ row_scale = nullptr) {
  static_assert(!FP8OUT || (SCATTER && D == 128), "FP8 output: scattered pools, D = 128");
  constexpr int TPP = D / 8;                  // threads per pool
  constexpr int PPB = 256 / TPP;              // pools per workgroup
  const int kpool = KP > 0 ? KP : kpool_rt;
  const int pool_cap = T / kpool;
  const int tid = threadIdx.x;

  __shared__ int s_cup[FUSED ? kFusedDocs + 1 : 1];
  __shared__ int s_wsum[4];
  const int32_t* cup = cu_pools;
  // the pool starting at token t0 -> pooled row p (16 bytes of it per thread)
  auto pool_body = [&](int p, int t0) {
    const int d0 = (tid % TPP) * 8;
    auto lo_hi = [](uint32_t w, int half) { return bf16_bits_to_f32((w >> (16 * half)) & 0xffffu); };
    float z[8], acc[8], m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { z[e] = 0.f; acc[e] = 0.f; m[e] = -INFINITY; }
    if constexpr (KP > 0) {
      // all slot slices of the pool in registers: one read of gate and k.
      // The gate slices and the position bias are requested first and the
      // key slices last, so the softmax weights (which need only the gate)
      // are computed while the key slices are still on their way: the
      // compiler's wait for the last gate load leaves the key loads
      // outstanding (vector-memory loads complete in issue order). The
      // memory clobber and the scheduling barrier keep every load issued
      // before the first use; left alone, the scheduler sinks the k loads to
      // their uses and each then waits a full memory round trip of its own.
      uint4 g4[KP], k4[KP];
      float4 ap[KP][2];
#pragma unroll
      for (int s = 0; s < KP; ++s)
        g4[s] = *reinterpret_cast<const uint4*>(gate + (size_t)(t0 + s) * D + d0);
#pragma unroll
      for (int s = 0; s < KP; ++s) {
        ap[s][0] = *reinterpret_cast<const float4*>(ape + s * D + d0);
        ap[s][1] = *reinterpret_cast<const float4*>(ape + s * D + d0 + 4);
      }
#pragma unroll
      for (int s = 0; s < KP; ++s)
        k4[s] = *reinterpret_cast<const uint4*>(k + (size_t)(t0 + s) * D + d0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      float a[KP][8];
#pragma unroll
      for (int s = 0; s < KP; ++s) {
        const float4 a0 = ap[s][0];
        const float4 a1 = ap[s][1];
        const uint32_t gw[4] = {g4[s].x, g4[s].y, g4[s].z, g4[s].w};
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          a[s][e] = lo_hi(gw[e >> 1], e & 1) + av[e];        // slot logit, FP32
          m[e] = fmaxf(m[e], a[s][e]);
        }
      }
      // the weights, before any key slice is touched
#pragma unroll
      for (int s = 0; s < KP; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // hardware exp2 of the argument times log2(e): a few FP32 ulps
          // from the exact exponential, far inside the BF16 result's ulp
          a[s][e] = __expf(a[s][e] - m[e]);
          z[e] += a[s][e];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < KP; ++s) {
        const uint32_t kw[4] = {k4[s].x, k4[s].y, k4[s].z, k4[s].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += a[s][e] * lo_hi(kw[e >> 1], e & 1);
      }
    } else {
      // runtime kpool: pass 1 finds the per-dimension maximum, pass 2 the
      // weights, their sum and the weighted keys
      for (int ss = 0; ss < kpool; ++ss) {
        const uint4 g4 = *reinterpret_cast<const uint4*>(gate + (size_t)(t0 + ss) * D + d0);
        const float4 a0 = *reinterpret_cast<const float4*>(ape + ss * D + d0);
        const float4 a1 = *reinterpret_cast<const float4*>(ape + ss * D + d0 + 4);
        const uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w};
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], lo_hi(gw[e >> 1], e & 1) + av[e]);
      }
      for (int ss = 0; ss < kpool; ++ss) {
        const uint4 g4 = *reinterpret_cast<const uint4*>(gate + (size_t)(t0 + ss) * D + d0);
        const uint4 k4 = *reinterpret_cast<const uint4*>(k + (size_t)(t0 + ss) * D + d0);
        const float4 a0 = *reinterpret_cast<const float4*>(ape + ss * D + d0);
        const float4 a1 = *reinterpret_cast<const float4*>(ape + ss * D + d0 + 4);
        const uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w};
        const uint32_t kw[4] = {k4.x, k4.y, k4.z, k4.w};
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ex = __expf((lo_hi(gw[e >> 1], e & 1) + av[e]) - m[e]);
          z[e] += ex;
          acc[e] += ex * lo_hi(kw[e >> 1], e & 1);
        }
      }
    }
    uint32_t outw[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      // z >= 1 (the largest slot contributes exp(0)); the hardware
      // reciprocal is within 1 FP32 ulp
      outw[e >> 1] = pack_bf16x2(acc[e] * __builtin_amdgcn_rcpf(z[e]),
                                 acc[e + 1] * __builtin_amdgcn_rcpf(z[e + 1]));
    }
    if constexpr (FP8OUT) {
      // the 16 lanes of the pool hold its row, 8 BF16 values each, in the
      // layout of the FP8 quantiser
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32((outw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      uint32_t packed[2];
      const int l = tid % TPP;
      const int ex = fp8_row_codes(v, l, packed);
      uint8_t* codes = reinterpret_cast<uint8_t*>(pooled);
      *reinterpret_cast<uint2*>(codes + (size_t)p * 128 + l * 8) = make_uint2(packed[0], packed[1]);
      if (l == 0) row_scale[p] = ldexpf(1.0f, ex);
    } else {
      *reinterpret_cast<uint4*>(pooled + (size_t)p * D + d0) =
          make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
  };
  if constexpr (SCATTER) {
    const int p = blockIdx.x * PPB + tid / TPP;
    if (p >= pool_cap) return;
    const int row = dst_rows[p];
    if (row < 0 || row >= dst_cap) return;
    pool_body(row, p * kpool);
    return;
  }
  if (FUSED && B == 1) {
    // one document: cu = {0, T} by the interface's precondition, so pool p
    // starts at token p kpool and nothing has to be read before the slices
    if (blockIdx.x == 0 && tid == 0) { cu_pools[0] = 0; cu_pools[1] = pool_cap; }
    const int p = blockIdx.x * PPB + tid / TPP;
    if (p >= pool_cap) return;
    pool_body(p, p * kpool);
    return;
  }
  if constexpr (FUSED) {
    // cuP[b + 1] = sum over b' <= b of floor(L_b' / kpool): thread tid owns
    // documents tid * per .. tid * per + per - 1; a block prefix sum of the
    // per-thread totals places them (negative lengths count as zero pools)
    const int per = (B + 255) >> 8;           // <= 4
    int cnt[4], tsum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = tid * per + j;
      int c = 0;
      if (j < per && b < B) {
        const int len = cu[b + 1] - cu[b];
        c = len > 0 ? len / kpool : 0;
      }
      cnt[j] = c;
      tsum += c;
    }
    const int lane = tid & 63, wid = tid >> 6;
    const int incl = wave_prefix_sum(tsum);
    if (lane == 63) s_wsum[wid] = incl;
    __syncthreads();
    int run = incl - tsum;
    for (int w = 0; w < wid; ++w) run += s_wsum[w];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = tid * per + j;
      if (j < per && b < B) {
        run += cnt[j];
        s_cup[b + 1] = run;
      }
    }
    if (tid == 0) s_cup[0] = 0;
    __syncthreads();
    if (blockIdx.x == 0)
      for (int b = tid; b <= B; b += 256) cu_pools[b] = s_cup[b];
    cup = s_cup;
  }

  const int total = clampi(cup[B], 0, pool_cap);
  const int p = blockIdx.x * PPB + tid / TPP;
  if (p >= total) return;

  // Document of pool p: the first pool of the wave is looked up by binary
  // search, the rest of the wave walks forward past the few boundaries it
  // can cross.
  const int p_first = __builtin_amdgcn_readfirstlane(p);
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cup[mid] <= p_first) lo = mid; else hi = mid - 1;
  }
  int b = lo;
  while (b + 1 < B && cup[b + 1] <= p) ++b;
  const int local = p - cup[b];
  const int t0 = clampi(cu[b] + local * kpool, 0, T - kpool);

  pool_body(p, t0);
}

template <int D, bool FUSED>
static void launch_compress_df(const uint16_t* k, const uint16_t* gate, const float* ape,
                               const int32_t* cu, int32_t* cu_pools, int B, int T, int kpool,
                               uint16_t* pooled, hipStream_t st) {
  constexpr int PPB = 256 / (D / 8);
  const int pool_cap = T / kpool;
  dim3 grid((pool_cap + PPB - 1) / PPB), block(256);
#define KP_C(KPV) compress_kernel<D, KPV, FUSED><<<grid, block, 0, st>>>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled)
  switch (kpool) {
    case 1: KP_C(1); break;
    case 2: KP_C(2); break;
    case 4: KP_C(4); break;
    case 8: KP_C(8); break;
    default: KP_C(0); break;
  }
#undef KP_C
}

void launch_compress(const uint16_t* k, const uint16_t* gate, const float* ape,
                     const int32_t* cu, int32_t* cu_pools, int B, int T, int D, int kpool,
                     uint16_t* pooled, hipStream_t st) {
  const bool fused = B <= kFusedDocs;
  if (T / kpool <= 0) {                       // no pools: only the offsets
    cu_pools_kernel<<<1, 1024, 0, st>>>(cu, B, kpool, cu_pools);
    return;
  }
  if (!fused) cu_pools_kernel<<<1, 1024, 0, st>>>(cu, B, kpool, cu_pools);
  if (D == 128) {
    if (fused) launch_compress_df<128, true>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled, st);
    else launch_compress_df<128, false>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled, st);
  } else {
    if (fused) launch_compress_df<64, true>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled, st);
    else launch_compress_df<64, false>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled, st);
  }
}

void launch_compress_pools(const uint16_t* k, const uint16_t* gate, const float* ape, int N,
                           int D, int kpool, const int32_t* dst_rows, int dst_cap,
                           uint16_t* pooled, float* row_scale, hipStream_t st) {
  if (N <= 0) return;
  const int T = N * kpool;
  const int ppb = 256 / (D / 8);
  const dim3 grid((N + ppb - 1) / ppb), block(256);
#define KP_S(DV, KPV, F8)                                                                \
  compress_kernel<DV, KPV, true, true, F8><<<grid, block, 0, st>>>(                      \
      k, gate, ape, nullptr, nullptr, 1, T, kpool, pooled, dst_rows, dst_cap, row_scale)
#define KP_SD(DV, F8)                   \
  switch (kpool) {                      \
    case 1: KP_S(DV, 1, F8); break;     \
    case 2: KP_S(DV, 2, F8); break;     \
    case 4: KP_S(DV, 4, F8); break;     \
    case 8: KP_S(DV, 8, F8); break;     \
    default: KP_S(DV, 0, F8); break;    \
  }
  if (row_scale) { KP_SD(128, true) }
  else if (D == 128) { KP_SD(128, false) }
  else { KP_SD(64, false) }
#undef KP_SD
#undef KP_S
}

}  // namespace kpool
