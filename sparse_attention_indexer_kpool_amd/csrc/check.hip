// Device-side check of a packed batch's document offsets, the precondition
// every entry point that takes cu_seqlens states (Megatron-LM PR #7054,
// section "3. KPool DSA indexer + NoPE": pools restart at every document of
// the packed batch, so the offsets decide every pool's tokens).
// One workgroup reads cu_seqlens[0 .. B] once (grid-stride over the
// documents) and writes one int32 of violation bits; nothing else is read
// or written, and the flags word needs no clearing beforehand.

#include "kpool_device.h"
#include "kpool_internal.h"

namespace kpool {

namespace {

__global__ __launch_bounds__(256) void check_cu_kernel(const int32_t* __restrict__ cu, int B, int T,
                                                        int max_seqlen, int32_t* __restrict__ out) {
  __shared__ int red[4];
  int bits = 0;
  if (threadIdx.x == 0) {
    if (cu[0] != 0) bits |= kCuFirstNotZero;
    if (cu[B] != T) bits |= kCuLastNotTotal;
  }
  for (int b = threadIdx.x; b < B; b += 256) {
    const int lo = cu[b], hi = cu[b + 1];
    if (hi < lo) bits |= kCuDecreasing;
    else if ((int64_t)hi - lo > max_seqlen) bits |= kCuTooLong;
  }
  // OR over the workgroup
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) bits |= __shfl_xor(bits, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = bits;
  __syncthreads();
  if (threadIdx.x == 0) out[0] = red[0] | red[1] | red[2] | red[3];
}

}  // namespace

hipError_t launch_check_cu_seqlens(const int32_t* cu, int B, int T, int max_seqlen, int32_t* out,
                                   hipStream_t stream) {
  hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, stream, cu, B, T, max_seqlen, out);
  return hipGetLastError();
}

}  // namespace kpool
