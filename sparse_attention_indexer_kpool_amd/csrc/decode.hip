// Decode step of the KPool indexer: one new query per sequence, scored against
// that sequence's cached pooled keys.
//
// Megatron-LM PR #7054, section "3. KPool DSA indexer + NoPE": the indexer
// scores pools, keeps index_topk // kpool of them and expands them to tokens,
// always adding the query's incomplete pool; the same section and section "4.
// DSA indexer FP8 precision split" place that indexer in serving, where a
// sequence grows one token per step and its pooled keys are kept in a cache.
// The query of a sequence of L tokens is its token L - 1, so its causal pools
// are the floor(L / kpool) complete pools of the cache and its tail the last
// L mod kpool tokens: the row the prefill indexer computes for that token.
//
//   score[b, j] = sum_h w[b, h] * ReLU(scale * q[b, h, :] . pooled[start_b + j, :])
//
// HBM-bound: every causal pooled key of every sequence is read once (2 D
// bytes per pool, or D bytes of E4M3 codes and a 4-byte scale); the
// arithmetic is 2 H D FLOP per pool, a few percent of what the matrix cores
// could do in that time. Still a contraction, so it runs on them:
// v_mfma_f32_32x32x16_bf16 for a BF16 cache, v_mfma_f32_32x32x64_f8f6f4 on
// E4M3 codes for an FP8 cache (the q rows quantised first, inside the
// kernel; their scales fold into w', and each key's scale multiplies its
// head sum, as in the prefill kernel). The A operand is the sequence's H head rows of q (zero rows up to
// a multiple of 32), held in registers; the B operand is a block of 32 keys,
// each lane pair reading adjacent bytes of a key row per step. The epilogue
// multiplies each lane's 16 head rows by w' = w * scale, clamps at 0, sums
// them and adds the other half-wave's 16 rows.

#include <type_traits>

#include "fp8_row.h"
#include "kpool_device.h"
#include "kpool_internal.h"

namespace kpool {

constexpr int kDecWaves = 4;                       // waves per workgroup
constexpr int kDecBlocksPerWave = 4;               // 32-pool blocks per wave
constexpr int kDecPoolsPerGroup = 32 * kDecWaves * kDecBlocksPerWave;   // 512

// Bytes of MFMA step s held by lane half g of a row (the same map for A and
// B, so the dot products are unchanged whatever order K is taken in): step s
// covers K values KSTEP s .. KSTEP s + KSTEP - 1 and lane half g the g-th
// half of them, so the two lanes of a pair read adjacent bytes of a row and
// one load instruction touches 32 rows' cache lines. (Giving each lane one
// contiguous half of the row instead touches 64 lines per instruction:
// 229 against 212 us for 256 sequences of 64K tokens, BF16.)
template <bool FP8>
__device__ __forceinline__ int koff_bytes(int s, int g) {
  return FP8 ? 64 * s + 32 * g : 32 * s + 16 * g;
}

template <int H, int D, bool FP8>
__global__ __launch_bounds__(64 * kDecWaves) void decode_logits_kernel(DecodeLogitsArgs a) {
  constexpr int MT = H > 32 ? H / 32 : 1;          // 32-row tiles of heads
  constexpr int KSTEP = FP8 ? 64 : 16;             // K per MFMA
  constexpr int NSTEP = D / KSTEP;                 // MFMAs per 32 x 32 tile
  constexpr int ROWB = FP8 ? D : 2 * D;            // bytes per q or key row
  constexpr int CH = FP8 ? 2 : 1;                  // 16-byte chunks per lane and step
  using Frag = typename std::conditional<FP8, i32x8_t, bf16x8_t>::type;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = (int)blockIdx.x / a.pieces;
  const int piece = (int)blockIdx.x % a.pieces;
  const int L = max(a.seq_lens[b], 0);
  const int n_c = min(L / a.kpool, a.max_pools);
  if (piece * kDecPoolsPerGroup >= n_c) return;   // the whole workgroup: nothing to score
  const int p_lo = piece * kDecPoolsPerGroup + 32 * wid;   // this wave's first pool
  const int n = lane & 31, g = lane >> 5;
  const int pool0 = a.pool_start[b];
  const uint8_t* __restrict__ kb = reinterpret_cast<const uint8_t*>(a.keys);

  // FP8: the workgroup first takes the sequence's H BF16 q rows through the
  // FP8 input path (16 lanes per row, the quantiser's layout and arithmetic)
  // into LDS; the A fragments and row scales are read from there. Every
  // workgroup of the sequence repeats this (H rows, a few hundred VALU
  // operations per lane) instead of a separate launch writing the codes.
  __shared__ __attribute__((aligned(16))) uint8_t q_codes[FP8 ? H * 128 : 16];
  __shared__ float q_scales[FP8 ? H : 1];
  if constexpr (FP8) {
    const int grp = threadIdx.x >> 4, l = threadIdx.x & 15;
    const uint16_t* __restrict__ qsrc = reinterpret_cast<const uint16_t*>(a.q);
    for (int r = grp; r < H; r += 64 * kDecWaves / 16) {   // uniform per 16-lane group
      const uint4 in = *reinterpret_cast<const uint4*>(qsrc + ((size_t)b * H + r) * 128 + l * 8);
      const uint32_t wv[4] = {in.x, in.y, in.z, in.w};
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu);
      uint32_t packed[2];
      const int ex = fp8_row_codes(v, l, packed);
      *reinterpret_cast<uint2*>(q_codes + r * 128 + l * 8) = make_uint2(packed[0], packed[1]);
      if (l == 0) q_scales[r] = ldexpf(1.0f, ex);
    }
    __syncthreads();
  }
  if (p_lo >= n_c) return;                         // nothing for this wave (no barrier below)
  const uint8_t* __restrict__ qb = FP8 ? q_codes : reinterpret_cast<const uint8_t*>(a.q);

  auto to_frag = [](const uint4 (&c)[CH]) -> Frag {
    if constexpr (FP8) {
      const i32x8_t f = {(int)c[0].x, (int)c[0].y, (int)c[0].z, (int)c[0].w,
                         (int)c[CH - 1].x, (int)c[CH - 1].y, (int)c[CH - 1].z, (int)c[CH - 1].w};
      return f;
    } else {
      return __builtin_bit_cast(bf16x8_t, c[0]);
    }
  };

  // A: head rows of q[b]; lane (n, g) holds row n of each tile, the bytes
  // koff_bytes(s, g) .. of step s
  Frag afrag[MT][NSTEP];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = mt * 32 + n;
    const uint8_t* qrow = FP8 ? qb + (head < H ? head : 0) * ROWB
                              : qb + ((size_t)b * H + (head < H ? head : 0)) * ROWB;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      uint4 c[CH];
#pragma unroll
      for (int h = 0; h < CH; ++h)
        c[h] = head < H ? *reinterpret_cast<const uint4*>(qrow + koff_bytes<FP8>(s, g) + 16 * h)
                        : make_uint4(0, 0, 0, 0);
      afrag[mt][s] = to_frag(c);
    }
  }
  // w' of this lane's accumulator rows (element v of a 32 x 32 accumulator is
  // row 8 (v / 4) + 4 g + (v mod 4)); FP8: times the q row's scale
  float wq[MT][16];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int head = mt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      float wv = 0.f;
      if (head < H) {
        wv = a.w[(size_t)b * H + head] * a.scale;
        if constexpr (FP8) wv *= q_scales[head];
      }
      wq[mt][v] = wv;
    }

  // B of block i: key row p_lo + 32 kDecWaves i + n, clamped into the causal
  // range (clamped columns are never stored) and into the cache
  auto key_row = [&](int i) {
    const int p = min(p_lo + 32 * kDecWaves * i + n, n_c - 1);
    return clampi(pool0 + p, 0, a.pooled_rows - 1);
  };
  auto load_b = [&](int i, uint4 (&bf)[NSTEP][CH]) {
    const uint8_t* krow = kb + (size_t)key_row(i) * ROWB;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s)
#pragma unroll
      for (int h = 0; h < CH; ++h)
        bf[s][h] = *reinterpret_cast<const uint4*>(krow + koff_bytes<FP8>(s, g) + 16 * h);
  };
  float* __restrict__ out = a.out + (size_t)b * a.ld;
  uint4 bfr[2][NSTEP][CH];
  load_b(0, bfr[0]);
#pragma unroll
  for (int i = 0; i < kDecBlocksPerWave; ++i) {
    const int c0 = p_lo + 32 * kDecWaves * i;      // first column of block i
    if (c0 >= n_c) break;
    // the next block's keys are requested before this block's MFMAs; the
    // memory clobber and the scheduling barrier keep those loads here
    if (i + 1 < kDecBlocksPerWave && c0 + 32 * kDecWaves < n_c) load_b(i + 1, bfr[(i + 1) & 1]);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    f32x16_t acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][v] = 0.f;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const Frag bf = to_frag(bfr[i & 1][s]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (FP8)
          acc[mt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afrag[mt][s], bf, acc[mt], 0, 0,
                                                                    0, 0, 0, 0);
        else
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afrag[mt][s], bf, acc[mt], 0, 0, 0);
      }
    }
    // w' * ReLU over this lane's head rows (ReLU as an integer max: FP32
    // values of either sign order like their bit patterns against +0)
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        sum += wq[mt][v] * __int_as_float(max(__float_as_int(acc[mt][v]), 0));
    // add the other half-wave's rows of the same column
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(sum), __float_as_uint(sum),
                                                     false, false);
    float score = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    if constexpr (FP8) score *= a.k_scale[key_row(i)];     // the key's power-of-two scale
    if (g == 0 && c0 + n < n_c) out[c0 + n] = score;
  }
}

template <int H, int D, bool FP8>
static void launch_hd(const DecodeLogitsArgs& a0, hipStream_t st) {
  DecodeLogitsArgs a = a0;
  a.pieces = (a.max_pools + kDecPoolsPerGroup - 1) / kDecPoolsPerGroup;
  if (a.pieces < 1) a.pieces = 1;
  decode_logits_kernel<H, D, FP8><<<a.B * a.pieces, 64 * kDecWaves, 0, st>>>(a);
}

template <int D, bool FP8>
static void launch_d(const DecodeLogitsArgs& a, hipStream_t st) {
  switch (a.H) {
    case 4: launch_hd<4, D, FP8>(a, st); break;
    case 8: launch_hd<8, D, FP8>(a, st); break;
    case 16: launch_hd<16, D, FP8>(a, st); break;
    case 32: launch_hd<32, D, FP8>(a, st); break;
    default: launch_hd<64, D, FP8>(a, st); break;
  }
}

void launch_decode_logits(const DecodeLogitsArgs& a, hipStream_t st) {
  if (a.B <= 0 || a.max_pools <= 0 || a.pooled_rows <= 0) return;
  if (a.fp8) launch_d<128, true>(a, st);
  else if (a.D == 128) launch_d<128, false>(a, st);
  else launch_d<64, false>(a, st);
}

}  // namespace kpool
