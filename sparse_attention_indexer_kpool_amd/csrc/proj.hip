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
// One MFMA GEMM, C[M, N] = A[M, K] B[N, K]^T with BF16 operands and FP32
// accumulation, in 128 x 128 tiles of a 64-wide K step, both operands copied
// straight into LDS with global_load_lds_dwordx4 (double buffered). The
// epilogue depends on the 128-column block: a BF16 store (q, gate), a
// LayerNorm of whole 128-value rows (k), or the FP32 head weights. Those
// come from the same BF16 MFMA: the FP32 matrix W is split exactly into
// three BF16 matrices, W = hi + mid + lo (each the BF16 rounding of what the
// previous ones leave, so the remainder is below 2^-24 |W|), and the three
// products, each exact in FP32 (BF16 x BF16), are summed in FP32.

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

__device__ __forceinline__ void dma16(const void* src, uint8_t* block) {
  const uint32_t dst = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)block);
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(dst), "v"(src)
      : "memory");
}

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// This wave's share (4 of 16 1-KB blocks) of a 128 x 64 tile of rows
// row0 .. row0 + 127 (rows past `rows` read the last row), K columns k0 ..
// k0 + 63 of a row-major [rows, ld] BF16 matrix.
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ m, int64_t ld, int rows,
                                          int row0, int k0, uint8_t* lds, int wid, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int L = (wid * 4 + i) * 64 + lane;       // chunk index in the tile
    const int r = L / kCPR, pos = L % kCPR;
    const int c = swz8(r, pos);
    const int gr = row0 + r < rows ? row0 + r : rows - 1;
    dma16(m + (size_t)gr * ld + k0 + c * 8, lds + (wid * 4 + i) * 1024);
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
  GemmBlock blk[32];               // blockIdx.y -> block (N / 128 of them)
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

  load_tile(g.a, g.K, g.M, row0, 0, lds, wid, lane);
  load_tile(blk.b, g.K, blk.b_rows, 0, 0, lds + kTileBytes, wid, lane);
  for (int kt = 0; kt < KT; ++kt) {
    wait_vmem_all();
    __syncthreads();               // stage kt is in LDS; stage kt - 1 is no longer read
    const uint8_t* As = lds + (kt & 1) * 2 * kTileBytes;
    const uint8_t* Bs = As + kTileBytes;
    if (kt + 1 < KT) {
      uint8_t* nA = lds + ((kt + 1) & 1) * 2 * kTileBytes;
      load_tile(g.a, g.K, g.M, row0, (kt + 1) * kBK, nA, wid, lane);
      load_tile(blk.b, g.K, blk.b_rows, 0, (kt + 1) * kBK, nA + kTileBytes, wid, lane);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                 As + (wm * 64 + i * 32) * 128 + off[s]));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                                  Bs + (wn * 64 + j * 32) * 128 + off[s]));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
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
    const int r = tid >> 1, half = tid & 1;
    const float* src = ct + r * LDC + half * 64;
    float v[64];
#pragma unroll
    for (int c = 0; c < 64; c += 4) {
      const float4 f = *reinterpret_cast<const float4*>(src + c);
      v[c] = bf16_round_f(f.x); v[c + 1] = bf16_round_f(f.y);
      v[c + 2] = bf16_round_f(f.z); v[c + 3] = bf16_round_f(f.w);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < 64; ++c) s += v[c];
    s += __shfl_xor(s, 1);
    const float mean = s / 128.f;
    float q = 0.f;
#pragma unroll
    for (int c = 0; c < 64; ++c) {
      const float d = v[c] - mean;
      q += d * d;
    }
    q += __shfl_xor(q, 1);
    const float inv = 1.f / sqrtf(q / 128.f + g.eps);
    const int gr = row0 + r;
    if (gr < g.M) {
      uint16_t* out = reinterpret_cast<uint16_t*>(blk.out) + (size_t)gr * blk.ldo + half * 64;
#pragma unroll
      for (int c = 0; c < 64; c += 8) {
        uint32_t w4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c0 = half * 64 + c + 2 * u;
          const float y0 = (v[c + 2 * u] - mean) * inv * g.ln_w[c0] + g.ln_b[c0];
          const float y1 = (v[c + 2 * u + 1] - mean) * inv * g.ln_w[c0 + 1] + g.ln_b[c0 + 1];
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
  // q: the query latent times wq_b, H*D columns in blocks of 128
  {
    const int N = p.H * 128;
    for (int n0 = 0; n0 < N; n0 += 32 * kBN) {
      GemmArgs g{};
      g.a = p.qr;
      g.M = p.T;
      g.K = p.q_lora;
      const int nb = (N - n0) / kBN < 32 ? (N - n0) / kBN : 32;
      for (int b = 0; b < nb; ++b) {
        const int c0 = n0 + b * kBN;
        g.blk[b] = GemmBlock{p.wq_b + (size_t)c0 * p.q_lora, 128, EPI_STORE_BF16, p.q, N, c0};
      }
      g.nblk = nb;
      proj_gemm_kernel<<<gemm_grid(p.T, nb), kGemmThreads, 0, st>>>(g);
    }
  }
}

}  // namespace kpool
