// The indexer projections that feed the KPool path: per token,
//   q    = linear_wq_b(qr)                       BF16 [T, H, D]
//   k    = k_norm(linear_wk(x))                   BF16 [T, D] (LayerNorm, FP32)
//   gate = index_kpool_compress_gate(x)           BF16 [T, D]
//   w    = linear_weights_proj(x)                 FP32 [T, H]
// Megatron-LM PR #7054, section "4. DSA indexer FP8 precision split" (the
// indexer's forward: q from linear_wq_b of the query latent; the k path
// linear_wk then k_norm; the head-weight projection kept in FP32) and section
// "3. KPool DSA indexer + NoPE" (the per-token compression gate, BF16). The
// gate is read as a linear map of x to D logits; no rotary embedding (NoPE)
// and no activation rotation.
//
// Two MFMA GEMM kernels, C[M, N] = A[M, K] B[N, K]^T with BF16 operands and
// FP32 accumulation, both operands copied straight into LDS with
// global_load_lds_dwordx4 in 64-wide K steps (double buffered; each lane's
// byte offsets are fixed for the whole K loop and only the scalar base
// moves, so the copies take no vector ALU work), the fragments of the next
// 16-wide K sub-step read while the current one's MFMAs run.
// - The x side (k, gate, head weights: 384 columns) in 128 x 128 tiles whose
//   epilogue depends on the 128-column block: a BF16 store (gate), a
//   LayerNorm of whole 128-value rows (k), or the FP32 head weights. Those
//   come from the same BF16 MFMA: the FP32 matrix W is split exactly into
//   three BF16 matrices, W = hi + mid + lo (each the BF16 rounding of what
//   the previous ones leave, so the remainder is below 2^-24 |W|), and the
//   three products, each exact in FP32 (BF16 x BF16), are summed in FP32.
// - q (H x 128 columns, most of the FLOPs) in 256 x 256 tiles with BF16
//   stores.

#include "kpool_device.h"
#include "kpool_internal.h"

namespace kpool {

namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kGemmThreads = 256;               // 4 waves, 2 x 2 over the tile
constexpr int kTileBytes = kBM * kBK * 2;        // one operand tile, BF16
constexpr int kCPR = kBK * 2 / 16;               // 16-byte chunks per tile row (8)

// chunk c of tile row r sits at position c ^ f(r): 128-byte rows pair up in
// a 256-byte line, so f(r) = (r >> 1) & 7 spreads the 16 rows a read pass
// touches at one chunk over distinct banks
__device__ __forceinline__ int swz8(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// global_load_lds_dwordx4 with an SGPR base and a per-lane 32-bit byte
// offset: lane l copies 16 bytes from base + voff to LDS address dst + 16 l
__device__ __forceinline__ void dma_sv(const void* base_, uint32_t voff, uint32_t dst_) {
  const uint64_t b64 = (uint64_t)(uintptr_t)base_;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  const void* base = (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  const uint32_t dst = __builtin_amdgcn_readfirstlane(dst_);
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(dst), "v"(voff), "s"(base)
      : "memory");
}

// This wave's 4 chunks of a 128 x 64 operand tile: byte offsets from the
// tile's first row at K column 0 (rows past `rows` read the last row)
__device__ __forceinline__ void tile_offsets(int64_t ld, int rows, int row0, int wid, int lane,
                                             uint32_t (&off)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int L = (wid * 4 + i) * 64 + lane;
    const int r = L / kCPR, pos = L % kCPR;
    const int c = swz8(r, pos);
    const int rr = (row0 + r < rows ? row0 + r : rows - 1) - row0;
    off[i] = (uint32_t)(((int64_t)rr * ld + c * 8) * 2);
  }
}

// Two FP32 values -> packed BF16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_round_f(float x) {
  return __uint_as_float(pack_bf16x2(x, 0.f) << 16);
}

}  // namespace

// Epilogue of a 128-column block.
enum ProjEpi : int { EPI_STORE_BF16 = 0, EPI_LAYERNORM = 1, EPI_SUM3_F32 = 2 };

struct GemmBlock {                 // one 128-column block of the output
  const uint16_t* b;               // BF16 [128, K]: this block's rows of B
  int b_rows;                      // rows of b that exist (the rest read its last row)
  int epi;
  void* out;                       // see the epilogues
  int64_t ldo;                     // row stride of out, elements
  int out_col0;                    // first output column of this block
};

struct GemmArgs {
  const uint16_t* a;               // BF16 [M, K]
  int M, K;
  int nblk;                        // column blocks (N / 128)
  GemmBlock blk[3];                // column block -> its B rows and epilogue
  const float* ln_w;               // LayerNorm weight, bias [128] (EPI_LAYERNORM)
  const float* ln_b;
  float eps;
  int heads;                       // H (EPI_SUM3_F32: columns h, 32 + h, 64 + h)
};

constexpr int kLDC = kBN + 4;                    // epilogue tile row stride, floats
constexpr int kGemmLds = 4 * kTileBytes > kBM * kLDC * 4 ? 4 * kTileBytes : kBM * kLDC * 4;

__global__ __launch_bounds__(kGemmThreads) void proj_gemm_kernel(GemmArgs g) {
  // operand tiles A0 B0 A1 B1; after the K loop, the FP32 output block
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kGemmLds];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int n = lane & 31, hg = lane >> 5;
  // block -> (row block, column block): groups of kGroupM row blocks take
  // every column block before the next group starts, and workgroups are
  // dealt to the 8 XCDs in turn, so an XCD's L2 holds its group's rows of A
  // and a quarter of the column blocks of B while they are used
  constexpr int kGroupM = 8;
  const int per_group = kGroupM * g.nblk;
  const int grp = (int)blockIdx.x / per_group, within = (int)blockIdx.x % per_group;
  const int mb = grp * kGroupM + within / g.nblk, nb = within % g.nblk;
  const int row0 = mb * kBM;
  if (row0 >= g.M) return;                 // padding of the last group (uniform)
  const GemmBlock blk = g.blk[nb];
  const int KT = g.K / kBK;

  // fragment offsets (the same swizzle for A and B): row n of a 32-row
  // block, chunk hg * 4 + s for K step s
  uint32_t off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) off[s] = (uint32_t)(n * 128 + swz8(n, hg * 4 + s) * 16);

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  uint32_t aoff[4], bof[4];
  tile_offsets(g.K, g.M, row0, wid, lane, aoff);
  tile_offsets(g.K, blk.b_rows, 0, wid, lane, bof);
  const uint16_t* const abase = g.a + (size_t)row0 * g.K;
  const uint16_t* const bbase = blk.b;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  auto issue = [&](int kt) {
    const uint32_t dA = lds0 + (kt & 1) * 2 * kTileBytes + wid * 4 * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_sv(abase + kt * kBK, aoff[i], dA + i * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_sv(bbase + kt * kBK, bof[i], dA + kTileBytes + i * 1024);
  };
  issue(0);
  bf16x8_t af[2][2], bfr[2][2];
  for (int kt = 0; kt < KT; ++kt) {
    wait_vmem_all();
    __syncthreads();               // stage kt is in LDS; stage kt - 1 is no longer read
    const uint8_t* As = lds + (kt & 1) * 2 * kTileBytes;
    const uint8_t* Bs = As + kTileBytes;
    if (kt + 1 < KT) issue(kt + 1);
    auto rd = [&](int s, int b) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[b][i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                    As + (wm * 64 + i * 32) * 128 + off[s]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[b][j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                     Bs + (wn * 64 + j * 32) * 128 + off[s]));
    };
    rd(0, 0);
    // falling wave priority over the K step's sub-steps: a wave behind the
    // other wave of its SIMD outranks it, so both reach the next barrier
    // together (measured: -4 % for the projections)
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s == 1) __builtin_amdgcn_s_setprio(2);
      if (s == 2) __builtin_amdgcn_s_setprio(1);
      if (s == 3) __builtin_amdgcn_s_setprio(0);
      if (s + 1 < 4) rd(s + 1, (s + 1) & 1);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][i], bfr[s & 1][j],
                                                              acc[i][j], 0, 0, 0);
    }
  }

  // accumulator element e of tile (i, j): row wm*64 + i*32 + 8*(e/4) + 4*hg +
  // e%4, column wn*64 + j*32 + n (of the 128 x 128 block)
  if (blk.epi == EPI_STORE_BF16) {
    uint16_t* out = reinterpret_cast<uint16_t*>(blk.out);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = row0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * hg + (e & 3);
        if (r < g.M) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int c = blk.out_col0 + wn * 64 + j * 32 + n;
            out[(size_t)r * blk.ldo + c] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.f) & 0xffffu);
          }
        }
      }
    return;
  }

  // the other epilogues need whole rows: the block goes to LDS as FP32
  // [128][128] (the operand buffers are free once every wave is past its
  // last MFMA), rows padded by 4 floats against bank conflicts
  constexpr int LDC = kLDC;
  float* ct = reinterpret_cast<float*>(lds);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = wm * 64 + i * 32 + 8 * (e >> 2) + 4 * hg + (e & 3);
#pragma unroll
      for (int j = 0; j < 2; ++j) ct[r * LDC + wn * 64 + j * 32 + n] = acc[i][j][e];
    }
  __syncthreads();

  if (blk.epi == EPI_LAYERNORM) {
    // two threads per row, 64 columns each: the linear layer's BF16 output,
    // then mean and variance over the 128 values in FP32, normalise, scale
    // and shift, BF16
    // (three passes over the row in LDS, so no thread holds its 64 values
    // in registers: the kernel keeps two waves per SIMD)
    const int r = tid >> 1, half = tid & 1;
    const float* src = ct + r * LDC + half * 64;
    float s = 0.f;
#pragma unroll 4
    for (int c = 0; c < 64; c += 4) {
      const float4 f = *reinterpret_cast<const float4*>(src + c);
      s += bf16_round_f(f.x); s += bf16_round_f(f.y);
      s += bf16_round_f(f.z); s += bf16_round_f(f.w);
    }
    s += __shfl_xor(s, 1);
    const float mean = s / 128.f;
    float q = 0.f;
#pragma unroll 4
    for (int c = 0; c < 64; c += 4) {
      const float4 f = *reinterpret_cast<const float4*>(src + c);
      const float d0 = bf16_round_f(f.x) - mean, d1 = bf16_round_f(f.y) - mean;
      const float d2 = bf16_round_f(f.z) - mean, d3 = bf16_round_f(f.w) - mean;
      q += d0 * d0; q += d1 * d1; q += d2 * d2; q += d3 * d3;
    }
    q += __shfl_xor(q, 1);
    const float inv = 1.f / sqrtf(q / 128.f + g.eps);
    const int gr = row0 + r;
    if (gr < g.M) {
      uint16_t* out = reinterpret_cast<uint16_t*>(blk.out) + (size_t)gr * blk.ldo + half * 64;
#pragma unroll 2
      for (int c = 0; c < 64; c += 8) {
        const float4 f0 = *reinterpret_cast<const float4*>(src + c);
        const float4 f1 = *reinterpret_cast<const float4*>(src + c + 4);
        const float v[8] = {bf16_round_f(f0.x), bf16_round_f(f0.y), bf16_round_f(f0.z),
                            bf16_round_f(f0.w), bf16_round_f(f1.x), bf16_round_f(f1.y),
                            bf16_round_f(f1.z), bf16_round_f(f1.w)};
        uint32_t w4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c0 = half * 64 + c + 2 * u;
          const float y0 = (v[2 * u] - mean) * inv * g.ln_w[c0] + g.ln_b[c0];
          const float y1 = (v[2 * u + 1] - mean) * inv * g.ln_w[c0 + 1] + g.ln_b[c0 + 1];
          w4[u] = pack_bf16x2(y0, y1);
        }
        *reinterpret_cast<uint4*>(out + c) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
    return;
  }

  // EPI_SUM3_F32: w[t, h] = hi + (mid + lo), columns h, 32 + h, 64 + h
  for (int idx = tid; idx < kBM * g.heads; idx += kGemmThreads) {
    const int r = idx / g.heads, h = idx % g.heads;
    const int gr = row0 + r;
    if (gr < g.M) {
      const float* rowp = ct + r * LDC;
      reinterpret_cast<float*>(blk.out)[(size_t)gr * blk.ldo + h] =
          rowp[h] + (rowp[32 + h] + rowp[64 + h]);
    }
  }
}

// W [H, K] FP32 -> three BF16 matrices stacked in one [128, K] block: rows
// h, 32 + h, 64 + h hold hi, mid, lo of row h (hi = BF16(W), mid =
// BF16(W - hi), lo = BF16(W - hi - mid); both differences are exact in
// FP32); the other rows are zero.
__global__ void split3_kernel(const float* __restrict__ w, int H, int K, uint16_t* __restrict__ out) {
  const int64_t total = (int64_t)128 * K;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int row = (int)(i / K), col = (int)(i % K);
    const int part = row / 32, h = row % 32;
    uint16_t v = 0;
    if (part < 3 && h < H) {
      const float x = w[(size_t)h * K + col];
      const float hi = bf16_round_f(x);
      const float r1 = x - hi;
      const float mid = bf16_round_f(r1);
      const float lo = bf16_round_f(r1 - mid);
      const float pick = part == 0 ? hi : (part == 1 ? mid : lo);
      v = (uint16_t)(__float_as_uint(pick) >> 16);
    }
    out[i] = v;
  }
}

// The query projection alone: C[M, N] = A[M, K] B[N, K]^T stored as BF16,
// N a multiple of 256. Tiles of 256 x 256 with 8 waves, each wave 128 rows x
// 64 columns (4 x 2 MFMA blocks): a K sub-step reads 6 fragments for 8
// MFMAs, against 4 for 4 in the 128 x 128 kernel, and a K step copies 64 KB
// of operands for twice the FLOPs per byte; these two bound the smaller
// tile through LDS and L2 bandwidth. The output goes through LDS so that
// every store is a 16-byte piece of a 128-byte row run.
constexpr int kWM = 256, kWN = 256;
constexpr int kWThreads = 512;
constexpr int kWTile = kWM * kBK * 2;            // one operand tile, 32 KB

struct WideArgs {
  const uint16_t* a;               // BF16 [M, K]
  const uint16_t* b;               // BF16 [N, K]
  uint16_t* c;                     // BF16 [M, N]
  int M, N, K;
};

// This wave's 4 chunks of a 256 x 64 tile (rows past `rows` read the last row)
__device__ __forceinline__ void wide_offsets(int64_t ld, int rows, int row0, int wid, int lane,
                                             uint32_t (&off)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int L = (wid * 4 + i) * 64 + lane;
    const int r = L / kCPR, pos = L % kCPR;
    const int c = swz8(r, pos);
    const int rr = (row0 + r < rows ? row0 + r : rows - 1) - row0;
    off[i] = (uint32_t)(((int64_t)rr * ld + c * 8) * 2);
  }
}

__global__ __launch_bounds__(kWThreads) void proj_gemm_wide_kernel(WideArgs g) {
  // two stages of (A tile, B tile); after the K loop, the BF16 output
  // sub-tiles of the eight waves (16 KB each)
  __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * kWTile];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 2, wn = wid & 3;           // 2 x 4 waves: 128 rows x 64 columns each
  const int n = lane & 31, hg = lane >> 5;
  // groups of 8 row blocks take every column block in turn (the L2 of an
  // XCD keeps its group's rows of A while the column blocks go by)
  const int nblk = g.N / kWN;
  const int per_group = 8 * nblk;
  const int grp = (int)blockIdx.x / per_group, within = (int)blockIdx.x % per_group;
  const int mb = grp * 8 + within / nblk, nb = within % nblk;
  const int row0 = mb * kWM, col0 = nb * kWN;
  if (row0 >= g.M) return;                          // padding of the last group (uniform)
  const int KT = g.K / kBK;

  uint32_t off[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) off[s] = (uint32_t)(n * 128 + swz8(n, hg * 4 + s) * 16);

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  uint32_t aoff[4], bof[4];
  wide_offsets(g.K, g.M, row0, wid, lane, aoff);
  wide_offsets(g.K, g.N, col0, wid, lane, bof);
  const uint16_t* const abase = g.a + (size_t)row0 * g.K;
  const uint16_t* const bbase = g.b + (size_t)col0 * g.K;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
  auto issue = [&](int kt) {
    const uint32_t dA = lds0 + (kt & 1) * 2 * kWTile + wid * 4 * 1024;
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_sv(abase + kt * kBK, aoff[i], dA + i * 1024);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_sv(bbase + kt * kBK, bof[i], dA + kWTile + i * 1024);
  };
  issue(0);
  bf16x8_t af[2][4], bfr[2][2];
  for (int kt = 0; kt < KT; ++kt) {
    wait_vmem_all();
    __syncthreads();               // stage kt is in LDS; stage kt - 1 is no longer read
    const uint8_t* As = lds + (kt & 1) * 2 * kWTile;
    const uint8_t* Bs = As + kWTile;
    if (kt + 1 < KT) issue(kt + 1);
    auto rd = [&](int s, int b) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[b][i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                    As + (wm * 128 + i * 32) * 128 + off[s]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[b][j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                     Bs + (wn * 64 + j * 32) * 128 + off[s]));
    };
    rd(0, 0);
    // falling wave priority over the K step's sub-steps: a wave behind the
    // other wave of its SIMD outranks it, so both reach the next barrier
    // together (measured: -4 % for the projections)
    __builtin_amdgcn_s_setprio(3);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s == 1) __builtin_amdgcn_s_setprio(2);
      if (s == 2) __builtin_amdgcn_s_setprio(1);
      if (s == 3) __builtin_amdgcn_s_setprio(0);
      if (s + 1 < 4) rd(s + 1, (s + 1) & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s & 1][i], bfr[s & 1][j],
                                                              acc[i][j], 0, 0, 0);
    }
  }

  // the wave's 128 x 64 results as BF16 into its 16 KB of LDS (row stride
  // 128 bytes), then out as 16-byte pieces: 8 lanes per 128-byte row run.
  // Accumulator element e of block (i, j): row i*32 + 8*(e/4) + 4*hg + e%4,
  // column j*32 + n of the wave's sub-tile.
  __syncthreads();                 // every wave is past its last fragment read
  uint16_t* st = reinterpret_cast<uint16_t*>(lds + wid * 16384);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = i * 32 + 8 * (e >> 2) + 4 * hg + (e & 3);
        st[r * 64 + j * 32 + n] = (uint16_t)(pack_bf16x2(acc[i][j][e], 0.f) & 0xffffu);
      }
  __builtin_amdgcn_s_waitcnt(0xc07f);          // this wave's LDS writes are done (lgkmcnt 0)
  __builtin_amdgcn_wave_barrier();
  const int orow0 = row0 + wm * 128, ocol0 = col0 + wn * 64;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int r = k * 8 + (lane >> 3), c = (lane & 7) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(st + r * 64 + c);
    if (orow0 + r < g.M)
      *reinterpret_cast<uint4*>(g.c + (size_t)(orow0 + r) * g.N + ocol0 + c) = v;
  }
}

// workgroups for M rows and nblk column blocks, whole groups of 8 row blocks
static int gemm_grid(int M, int nblk) {
  const int mblk = (M + kBM - 1) / kBM;
  return (mblk + 7) / 8 * 8 * nblk;
}

void launch_indexer_projections(const ProjArgs& p, hipStream_t st) {
  // x-side: k (LayerNorm), gate, the FP32 head weights
  {
    split3_kernel<<<256, 256, 0, st>>>(p.ww, p.H, p.hidden, p.w3);
    GemmArgs g{};
    g.a = p.x;
    g.M = p.T;
    g.K = p.hidden;
    g.ln_w = p.ln_w;
    g.ln_b = p.ln_b;
    g.eps = p.eps;
    g.heads = p.H;
    g.blk[0] = GemmBlock{p.wk, 128, EPI_LAYERNORM, p.k, 128, 0};
    g.blk[1] = GemmBlock{p.wg, 128, EPI_STORE_BF16, p.gate, 128, 0};
    g.blk[2] = GemmBlock{p.w3, 128, EPI_SUM3_F32, p.w, p.H, 0};
    g.nblk = 3;
    proj_gemm_kernel<<<gemm_grid(p.T, g.nblk), kGemmThreads, 0, st>>>(g);
  }
  // q: the query latent times wq_b, H*D columns (a multiple of 512)
  {
    WideArgs g{p.qr, p.wq_b, p.q, p.T, p.H * 128, p.q_lora};
    const int mblk = (p.T + kWM - 1) / kWM;
    const int grid = (mblk + 7) / 8 * 8 * (g.N / kWN);
    proj_gemm_wide_kernel<<<grid, kWThreads, 0, st>>>(g);
  }
}

}  // namespace kpool
