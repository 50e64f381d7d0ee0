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

// KP = kpool when it is a compile-time constant, 0 for a runtime kpool.
template <int D, int KP>
__global__ __launch_bounds__(256) void compress_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ gate,
    const float* __restrict__ ape, const int32_t* __restrict__ cu,
    const int32_t* __restrict__ cu_pools, int B, int T, int kpool_rt,
    uint16_t* __restrict__ pooled) {
  constexpr int TPP = D / 8;                  // threads per pool
  constexpr int PPB = 256 / TPP;              // pools per workgroup
  const int kpool = KP > 0 ? KP : kpool_rt;
  const int pool_cap = T / kpool;
  const int total = clampi(cu_pools[B], 0, pool_cap);
  const int p = blockIdx.x * PPB + threadIdx.x / TPP;
  if (p >= total) return;
  const int d0 = (threadIdx.x % TPP) * 8;

  // Document of pool p: the first pool of the wave is looked up by binary
  // search, the rest of the wave walks forward past the few boundaries it
  // can cross.
  const int p_first = __builtin_amdgcn_readfirstlane(p);
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_pools[mid] <= p_first) lo = mid; else hi = mid - 1;
  }
  int b = lo;
  while (b + 1 < B && cu_pools[b + 1] <= p) ++b;
  const int local = p - cu_pools[b];
  const int t0 = clampi(cu[b] + local * kpool, 0, T - kpool);

  float m[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m[e] = -INFINITY;
  // pass 1: the per-dimension maximum of the slot logits
#pragma unroll
  for (int s = 0; s < (KP > 0 ? KP : 1); ++s) {
    for (int ss = s; ss < (KP > 0 ? s + 1 : kpool); ++ss) {
      const uint4 g4 = *reinterpret_cast<const uint4*>(gate + (size_t)(t0 + ss) * D + d0);
      const float4 a0 = *reinterpret_cast<const float4*>(ape + ss * D + d0);
      const float4 a1 = *reinterpret_cast<const float4*>(ape + ss * D + d0 + 4);
      const uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w};
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float g = bf16_bits_to_f32((gw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
        m[e] = fmaxf(m[e], g + av[e]);
      }
    }
  }
  // pass 2: weights, their sum and the weighted keys, all in FP32
  float z[8], acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { z[e] = 0.f; acc[e] = 0.f; }
#pragma unroll
  for (int s = 0; s < (KP > 0 ? KP : 1); ++s) {
    for (int ss = s; ss < (KP > 0 ? s + 1 : kpool); ++ss) {
      const uint4 g4 = *reinterpret_cast<const uint4*>(gate + (size_t)(t0 + ss) * D + d0);
      const uint4 k4 = *reinterpret_cast<const uint4*>(k + (size_t)(t0 + ss) * D + d0);
      const float4 a0 = *reinterpret_cast<const float4*>(ape + ss * D + d0);
      const float4 a1 = *reinterpret_cast<const float4*>(ape + ss * D + d0 + 4);
      const uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w};
      const uint32_t kw[4] = {k4.x, k4.y, k4.z, k4.w};
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float g = bf16_bits_to_f32((gw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
        float kv = bf16_bits_to_f32((kw[e >> 1] >> (16 * (e & 1))) & 0xffffu);
        float ex = expf((g + av[e]) - m[e]);
        z[e] += ex;
        acc[e] += ex * kv;
      }
    }
  }
  uint32_t outw[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    uint32_t lo16 = f32_to_bf16_bits(acc[e] / z[e]);
    uint32_t hi16 = f32_to_bf16_bits(acc[e + 1] / z[e + 1]);
    outw[e >> 1] = lo16 | (hi16 << 16);
  }
  *reinterpret_cast<uint4*>(pooled + (size_t)p * D + d0) =
      make_uint4(outw[0], outw[1], outw[2], outw[3]);
}

template <int D>
static void launch_compress_d(const uint16_t* k, const uint16_t* gate, const float* ape,
                              const int32_t* cu, const int32_t* cu_pools, int B, int T,
                              int kpool, uint16_t* pooled, hipStream_t st) {
  constexpr int PPB = 256 / (D / 8);
  const int pool_cap = T / kpool;
  if (pool_cap <= 0) return;
  dim3 grid((pool_cap + PPB - 1) / PPB), block(256);
  switch (kpool) {
    case 1: compress_kernel<D, 1><<<grid, block, 0, st>>>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled); break;
    case 2: compress_kernel<D, 2><<<grid, block, 0, st>>>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled); break;
    case 4: compress_kernel<D, 4><<<grid, block, 0, st>>>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled); break;
    case 8: compress_kernel<D, 8><<<grid, block, 0, st>>>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled); break;
    default: compress_kernel<D, 0><<<grid, block, 0, st>>>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled); break;
  }
}

void launch_cu_pools(const int32_t* cu, int B, int kpool, int32_t* cu_pools, hipStream_t st) {
  cu_pools_kernel<<<1, 1024, 0, st>>>(cu, B, kpool, cu_pools);
}

void launch_compress(const uint16_t* k, const uint16_t* gate, const float* ape,
                     const int32_t* cu, const int32_t* cu_pools, int B, int T, int D,
                     int kpool, uint16_t* pooled, hipStream_t st) {
  if (D == 128) launch_compress_d<128>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled, st);
  else launch_compress_d<64>(k, gate, ape, cu, cu_pools, B, T, kpool, pooled, st);
}

}  // namespace kpool
