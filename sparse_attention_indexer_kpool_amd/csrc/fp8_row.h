// FP8 input path of one 128-wide row held by 16 lanes (8 values each, lane
// l holding elements 8 l .. 8 l + 7): the FP32 Hadamard transform, the
// 128^-1/2 scaling rounded to BF16, the power-of-two row exponent and the
// E4M3 codes. Used by the quantiser and by the compression of pools into an
// FP8 cache, so both give the same codes for the same BF16 row.
//
// Megatron-LM PR #7054, sections "3. KPool DSA indexer + NoPE" and "4. DSA
// indexer FP8 precision split": the serving indexer's q and pooled keys go
// through a Hadamard rotation, BF16 and E4M3 with a power-of-two row scale.
#pragma once

#include "kpool_device.h"

namespace kpool {

// v: the row's values (BF16 values in FP32), overwritten with the rotated
// BF16 values; the 16 lanes of the row must be active together. Returns the
// row exponent e (row scale 2^e) and the eight E4M3 codes in packed.
__device__ __forceinline__ int fp8_row_codes(float (&v)[8], int l, uint32_t (&packed)[2]) {
#pragma clang fp contract(off)
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
  // stages h = 8, 16, 32, 64 across lanes l and l ^ (h / 8): the lower
  // lane keeps v + other, the upper one other - v, both as one
  // fma(+-1, v, other), which rounds exactly as the addition or
  // subtraction does
#pragma unroll
  for (int s = 1; s < 16; s <<= 1) {
    const float sgn = (l & s) != 0 ? -1.f : 1.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float other = xor_lane16(v[e], s);
      v[e] = fmaf(sgn, v[e], other);
    }
  }
  const float norm = 0.08838834764831845f;   // FP32(128^-1/2)
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = (float)(__bf16)(v[e] * norm);      // v_cvt_pk_bf16_f32: round to nearest even
    amax = fmaxf(amax, fabsf(v[e]));
  }
#pragma unroll
  for (int s = 1; s < 16; s <<= 1) amax = fmaxf(amax, xor_lane16(amax, s));

  int ex = 0;
  if (amax > 0.f && amax <= 3.402823466e38f) {
    int fe;
    const float f = frexpf(amax, &fe);      // amax = f * 2^fe, f in [0.5, 1)
    ex = fe - 9 + (f > 0.875f ? 1 : 0);
  }
  // v_cvt_pk_fp8_f32: OCP E4M3, round to nearest even, subnormals kept;
  // |v 2^-ex| <= 448 by the choice of ex, so nothing saturates
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * h], -ex), ldexpf(v[4 * h + 1], -ex), 0,
                                            false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * h + 2], -ex), ldexpf(v[4 * h + 3], -ex), w,
                                        true);
    packed[h] = (uint32_t)w;
  }
  return ex;
}

}  // namespace kpool
