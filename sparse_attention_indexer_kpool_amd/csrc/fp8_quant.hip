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
// BF16 and E4M3 rounding use gfx950's conversion instructions
// (v_cvt_pk_bf16_f32, v_cvt_pk_fp8_f32), both round to nearest even; they
// were checked bit for bit against the definitions over every BF16 input in
// the E4M3 range, all E4M3 rounding midpoints and 2 M FP32 values with ties.
//
// HBM-bound: 256 bytes in and 128 + 4 bytes out per row. Sixteen lanes own a
// row, eight values per lane, and take four rows in turn (their loads are
// issued together); stages h < 8 stay in a lane, stages h >= 8 exchange with
// lane l ^ (h / 8) through DPP and ds_swizzle lane permutations (neither
// touches LDS memory). Every value goes through the same FP32 operations in
// the same order as the stage definition, so codes are exact.

#include "kpool_device.h"
#include "kpool_internal.h"
#include "fp8_row.h"

#pragma clang fp contract(off)

namespace kpool {

constexpr int kQuantRows = 4;   // rows per 16-lane group

__global__ __launch_bounds__(256) void fp8_quantize_kernel(
    const uint16_t* __restrict__ x, int rows, const int32_t* __restrict__ rows_dev,
    uint8_t* __restrict__ codes, float* __restrict__ row_scale) {
  const int row0 = (blockIdx.x * 16 + (threadIdx.x >> 4)) * kQuantRows;
  const int l = threadIdx.x & 15;
  int limit = rows;
  if (rows_dev) {
    const int rd = *rows_dev;
    limit = rd < limit ? (rd > 0 ? rd : 0) : limit;
  }
  // whole 16-lane groups leave together, so the shuffles below see live lanes
  if (row0 >= limit) return;

  // the group's rows are loaded before any is transformed, so a lane keeps
  // kQuantRows 16-byte loads in flight
  uint4 in[kQuantRows];
#pragma unroll
  for (int r = 0; r < kQuantRows; ++r)
    in[r] = row0 + r < limit ? *reinterpret_cast<const uint4*>(x + (size_t)(row0 + r) * 128 + l * 8)
                             : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int r = 0; r < kQuantRows; ++r) {
    const int row = row0 + r;
    const uint32_t wv[4] = {in[r].x, in[r].y, in[r].z, in[r].w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf16_bits_to_f32((wv[e >> 1] >> (16 * (e & 1))) & 0xffffu);

    uint32_t packed[2];
    const int ex = fp8_row_codes(v, l, packed);
    if (row < limit) {
      *reinterpret_cast<uint2*>(codes + (size_t)row * 128 + l * 8) = make_uint2(packed[0], packed[1]);
      if (l == 0) row_scale[row] = ldexpf(1.0f, ex);
    }
  }
}

void launch_fp8_quantize(const uint16_t* x, int rows, const int32_t* rows_dev,
                         uint8_t* codes, float* row_scale, hipStream_t st) {
  if (rows <= 0) return;
  constexpr int RPB = 16 * kQuantRows;   // rows per workgroup
  fp8_quantize_kernel<<<(rows + RPB - 1) / RPB, 256, 0, st>>>(x, rows, rows_dev, codes, row_scale);
}

}  // namespace kpool
