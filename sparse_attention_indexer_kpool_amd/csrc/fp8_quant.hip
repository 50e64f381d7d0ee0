// FP8 input path of the KPool indexer (Megatron-LM PR #7054, section "3. KPool
// DSA indexer + NoPE", FP8 option): q rows and pooled-key rows are rotated by
// a Hadamard transform in FP32, rounded to BF16, and stored as E4M3 codes
// under a power-of-two scale per row, matching the serving indexer's input
// precision.
//
// Readings: 128-point orthonormal Sylvester Hadamard evaluated as butterfly
// stages h = 1, 2, ..., 64 with (a, b) -> (a + b, a - b); scale 2^e with the
// smallest integer e such that max|y| <= 448 * 2^e (e = 0 for a zero row);
// OCP E4M3 (e4m3fn), round to nearest even, subnormals kept.
//
// HBM-bound: 256 bytes in and 128 + 4 bytes out per row. Sixteen lanes own a
// row, eight values per lane; stages h < 8 stay in a lane, stages h >= 8
// exchange with lane l ^ (h / 8). Every value goes through the same FP32
// operations in the same order as the stage definition, so codes are exact.

#include "kpool_device.h"
#include "kpool_internal.h"

#pragma clang fp contract(off)

namespace kpool {

// E4M3 (e4m3fn) code of x, round to nearest even. |x| <= 448 for finite
// rows; NaN gives 0x7f and larger magnitudes saturate to 448 (broken input
// only).
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a <= 448.0f)) return sign | (a != a ? 0x7fu : 0x7eu);
  if (a < 0x1p-6f) {
    // subnormal range: multiples of 2^-9; rintf rounds halves to even
    return sign | (uint32_t)rintf(a * 512.0f);
  }
  const int E = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;   // -6 .. 8
  const float n = rintf(ldexpf(a, 3 - E));                          // 8 .. 16
  return sign | (uint32_t)(((E + 7) << 3) + ((int)n - 8));
}

__global__ __launch_bounds__(256) void fp8_quantize_kernel(
    const uint16_t* __restrict__ x, int rows, const int32_t* __restrict__ rows_dev,
    uint8_t* __restrict__ codes, float* __restrict__ row_scale) {
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  int limit = rows;
  if (rows_dev) {
    const int rd = *rows_dev;
    limit = rd < limit ? (rd > 0 ? rd : 0) : limit;
  }
  // whole 16-lane groups leave together, so the shuffles below see live lanes
  if (row >= limit) return;

  const uint4 in = *reinterpret_cast<const uint4*>(x + (size_t)row * 128 + l * 8);
  const uint32_t wv[4] = {in.x, in.y, in.z, in.w};
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu);

  // stages h = 1, 2, 4 inside the lane
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((e & h) == 0) {
        const float a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
    }
  }
  // stages h = 8, 16, 32, 64 across lanes l and l ^ (h / 8)
#pragma unroll
  for (int s = 1; s < 16; s <<= 1) {
    const bool upper = (l & s) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float other = __shfl_xor(v[e], s, 16);
      v[e] = upper ? (other - v[e]) : (v[e] + other);
    }
  }
  const float norm = 0.08838834764831845f;   // FP32(128^-1/2)
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = bf16_bits_to_f32(f32_to_bf16_bits(v[e] * norm));
    amax = fmaxf(amax, fabsf(v[e]));
  }
#pragma unroll
  for (int s = 1; s < 16; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 16));

  int ex = 0;
  if (amax > 0.f && amax <= 3.402823466e38f) {
    int fe;
    const float f = frexpf(amax, &fe);      // amax = f * 2^fe, f in [0.5, 1)
    ex = fe - 9 + (f > 0.875f ? 1 : 0);
  }
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) packed[e >> 2] |= e4m3_rne(ldexpf(v[e], -ex)) << (8 * (e & 3));
  *reinterpret_cast<uint2*>(codes + (size_t)row * 128 + l * 8) = make_uint2(packed[0], packed[1]);
  if (l == 0) row_scale[row] = ldexpf(1.0f, ex);
}

void launch_fp8_quantize(const uint16_t* x, int rows, const int32_t* rows_dev,
                         uint8_t* codes, float* row_scale, hipStream_t st) {
  if (rows <= 0) return;
  fp8_quantize_kernel<<<(rows + 15) / 16, 256, 0, st>>>(x, rows, rows_dev, codes, row_scale);
}

}  // namespace kpool
