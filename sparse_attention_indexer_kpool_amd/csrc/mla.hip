// Sparse attention of the NoPE absorbed MLA over the indexer's token rows:
// for query token t and head h,
//   s_j    = sm_scale * <q[t, h, :], kv[j, :]>          j over the listed rows
//   o[t,h] = sum_j softmax(s)_j kv[j, :d_v]              (BF16 out)
//   lse    = ln sum_j exp(s_j)                           (FP32 out)
// xtuner PR #2108, "Summary" (the sparse MLA backend runs FlashMLA's forward
// over the int32 indices, heads in multiples of 64, the head/value widths no
// longer fixed at 576) and the LSE fix commit (natural-log LSE); Megatron-LM
// PR #7054, section "3. KPool DSA indexer + NoPE" (NoPE: the absorbed query
// has no positional slice, so the latent row is both key and value).
// Entries outside [0, kv_rows) -- the indexer's -1 padding -- are unused; a
// row listed twice counts twice; a query with no used entry gets o = 0 and
// lse = -inf.
//
// One workgroup per (token, group of 64 heads), four waves. Wave w owns heads
// 32*(w & 1) .. +31 of the group and latent dims 256*(w >> 1) .. +255:
//   * The listed rows come in blocks of 32. Each block is copied straight
//     from HBM/L2 into LDS (global_load_lds_dwordx4, one 1 KB row per wave
//     instruction, double buffered) as a row-major [32][512] BF16 tile whose
//     16-byte chunks are XOR-swizzled per row.
//   * Scores: S^T (32 rows x 32 heads) = K . Q^T over the wave's 256 dims
//     (v_mfma_f32_32x32x16_bf16, K from LDS, Q^T held in registers); the
//     partner wave (other dim half, same heads) adds its half through LDS.
//   * Online softmax in base 2 per head (a head is one MFMA column, so its
//     running max, sum and rescale live in one lane pair).
//   * O^T (256 dims x 32 heads) += V^T . P^T: V^T comes from the same
//     row-major tile through the LDS transpose read (ds_read_b64_tr_b16);
//     P^T is the score accumulator itself, rounded to BF16, because the
//     transpose read is addressed so that its key order matches the order
//     of the score rows in the accumulator.
// Each gathered byte feeds 64 heads x 4 FLOPs: with the dims split two ways
// and the heads two ways, every LDS byte of the tile is read by two waves.

#include "kpool_device.h"
#include "kpool_internal.h"

namespace kpool {

namespace {

constexpr int kD = 512;                 // latent width (key = value)
constexpr int kHG = 64;                 // heads per workgroup
constexpr int kBlk = 32;                // listed rows per block
constexpr int kRowBytes = kD * 2;       // 1 KB
constexpr int kTile = kBlk * kRowBytes; // 32 KB
constexpr int kStages = 4;              // tile buffers: three blocks in flight
constexpr int kXchg = 4 * 16 * 64 * 4;  // partial scores of the four waves
constexpr int kMaxWidth = 4096;         // list entries staged in LDS
constexpr int kMlaLds = kStages * kTile + kXchg + kMaxWidth * 4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// chunk c (16 bytes) of tile row r sits at chunk position
// c ^ f(r) ^ 8 ((c >> 1) & 1). f maps the 16 rows of an aligned group onto
// 0..15, so 16 rows read at one chunk hit 16 distinct positions. f also gives
// the 4 rows of an aligned quadruple distinct values of f >> 1, so a
// transpose read (4 rows x 2 adjacent chunks per 16 lanes) covers 8
// distinct positions of one aligned 8-chunk half of a 256-byte bank window.
// The extra flip of bit 3 by bit 1 of c sends the 16 lanes next to them,
// which read chunks c + 2 and c + 3 of the same rows, to the other half.
__device__ __forceinline__ int swz(int r) {
  return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8);
}

// One 1 KB row: lane l copies 16 bytes from row_base + voff(l) to LDS
// address dst + 16 l (row_base and dst are wave-uniform, voff a 32-bit byte
// offset).
__device__ __forceinline__ void dma_row(const void* row_base, uint32_t voff, uint32_t dst) {
  uint32_t m0_saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(m0_saved)
      : "s"(dst), "v"(voff), "s"(row_base)
      : "memory");
}

// s_waitcnt vmcnt(N) with expcnt and lgkmcnt left unconstrained
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ i16x4 lds_tr4(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4 __attribute__((address_space(3)))*)(
          (__attribute__((address_space(3))) uint8_t*)p));
}

struct MlaKernelArgs {
  const uint16_t* q;       // [T, H, 512]
  const uint16_t* kv;      // [N, 512]
  const int32_t* idx;      // [T, W]
  uint16_t* out;           // [T, H, 512]
  float* lse;              // [T, H]
  int T, H, N, W, groups;  // groups = H / 64
  int64_t total;           // T * groups
  int64_t per_xcd;         // ceil(total / 8)
  float scale2;            // sm_scale * log2(e)
};

// Copy block `blk` (listed entries 32*blk .. +31) of this query into `tile`:
// wave w copies rows 8w .. 8w+7, one 1 KB row per instruction. `ids` holds
// entry 32*blk + (lane & 31) of the list (-1 past the end); an unused entry
// copies row 0 (its score is masked).
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ kv, int ids, int N,
                                           uint32_t tile_lds, int wid) {
  // the lane id, produced here (opaque to the compiler): the eight source
  // offsets below are recomputed (one XOR each) instead of being kept live
  // across the loop
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  const int ids_ok = (ids >= 0 && ids < N) ? ids : 0;   // one clamp for all 32 rows
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wid * 8 + j;                       // wave-uniform
    const int tok = __builtin_amdgcn_readlane(ids_ok, r);
    const int c0 = ln ^ swz(r);                      // global chunk for LDS position `lane`
    const uint32_t c = (uint32_t)(c0 ^ (((c0 >> 1) & 1) << 3));
    dma_row(kv + (size_t)tok * kD, c << 4, tile_lds + r * kRowBytes);
  }
}

__global__ __launch_bounds__(256, 1) void mla_fwd_kernel(MlaKernelArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* tiles = smem;                                   // kStages x 32 KB
  float* xchg = (float*)(smem + kStages * kTile);          // [4 waves][16 regs][64 lanes]
  int* ids_lds = (int*)(smem + kStages * kTile + kXchg);   // the query's list

  // blocks are dealt to the 8 XCDs in turn: give each XCD a contiguous run of
  // (token, head group) items, so the rows that neighbouring tokens share
  // stay in that XCD's L2
  const int64_t id = blockIdx.x;
  const int64_t item = (id & 7) * a.per_xcd + (id >> 3);
  if (item >= a.total) return;
  const int t = (int)(item / a.groups);
  const int hg = (int)(item % a.groups);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t tiles_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int hp = wid & 1, fh = wid >> 1;
  const int32_t* __restrict__ idx_row = a.idx + (size_t)t * a.W;

  // ---- stage the list in LDS; used length = one past its last entry in [0, N)
  int last = -1;
  for (int e = tid; e < a.W; e += 256) {
    const int v = idx_row[e];
    ids_lds[e] = v;
    if (v >= 0 && v < a.N) last = e;
  }
  last = wave_max(last);
  int* red = (int*)xchg;
  if (lane == 0) red[wid] = last;
  __syncthreads();
  last = max(max(red[0], red[1]), max(red[2], red[3]));
  __syncthreads();
  const int nblk = (last + kBlk) / kBlk;           // 0 when nothing is used

  // entry 32*blk + (lane & 31) of the list, -1 past its end
  auto ids_of = [&](int blk) {
    const int e = blk * kBlk + (lane & 31);
    return e < a.W ? ids_lds[e] : -1;
  };

#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < nblk) load_block(a.kv, ids_of(p), a.N, tiles_lds + p * kTile, wid);

  // ---- Q^T fragments: head 64hg + 32hp + (lane & 31), dims 256fh + 16ks + 8(lane >> 5) + 0..7
  bf16x8 qf[16];
  {
    const uint16_t* qrow = a.q + ((size_t)t * a.H + hg * kHG + hp * 32 + (lane & 31)) * kD +
                           fh * 256 + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * ks));
  }
  // the first blocks and Q have landed: no wait for Q remains inside the loop,
  // where it would also hold back the copies of later blocks
  wait_vmcnt<0>();
  // Q^T stays in accumulation registers (an MFMA reads its B operand from
  // there directly), leaving the vector registers to the LDS fragments
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) asm volatile("" : "+a"(qf[ks]));

  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int h = lane >> 5;

  // per-lane LDS byte offsets inside a tile
  //   K (A operand of S^T = K.Q^T): row lane & 31, dims 256fh + 16ks + 8h .. +7
  const int krow = (lane & 31) * kRowBytes;
  const int ku = swz(lane & 31) ^ h;    // chunk 2ks + h sits at 2ks ^ ku ^ 8 (ks & 1)
  //   V^T (A operand of O^T = V^T.P^T) by transpose reads: rows r0 and r0 + 8
  //   (r0 = 16 st + 4h + (i >> 2)), dims 256fh + 32mt + 16(b & 1) + 4(i & 3) ..
  const int tb = lane >> 4, ti = lane & 15;
  const int tsub = (ti & 1) * 8;

  auto kfrags = [&](uint32_t tile_off, bf16x8 (&kf)[16]) {
    const uint8_t* trow = tiles + tile_off + krow;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      kf[ks] = __builtin_bit_cast(
          bf16x8, *(const u32x4*)(trow + ((fh * 32 + ((2 * ks) ^ ku ^ ((ks & 1) << 3))) << 4)));
  };
  // S = this wave's partial + the partner's (same heads, other dim half);
  // both waves add the same two numbers, so both hold identical scores
  float* mine = xchg + wid * 1024;
  const float* other = xchg + (wid ^ 2) * 1024;
  auto put_partial = [&](const f32x16& sp) {
#pragma unroll
    for (int r = 0; r < 16; ++r) mine[r * 64 + lane] = sp[r];
  };
  auto add_partner = [&](f32x16& sp) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sp[r] = sp[r] + other[r * 64 + lane];
  };

  // Unused rows of block b become -inf; returns the block's largest score
  // in base-2 units (scale2 > 0 keeps the order), -inf if none is used.
  auto prep = [&](f32x16& sc, int b) {
    const int idc = ids_of(b);
    const uint32_t used_mask = (uint32_t)__ballot(idc >= 0 && idc < a.N);
    if (used_mask != 0xffffffffu) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * h + (r & 3);
        sc[r] = ((used_mask >> row) & 1u) ? sc[r] : -INFINITY;
      }
    }
    float mxs = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                      fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mxs = fmaxf(mxs, fmaxf(fmaxf(fmaxf(sc[8], sc[9]), fmaxf(sc[10], sc[11])),
                           fmaxf(fmaxf(sc[12], sc[13]), fmaxf(sc[14], sc[15]))));
    mxs = fmaxf(mxs, __shfl_xor(mxs, 32));
    return mxs * a.scale2;
  };

  // Software pipeline over blocks: iteration blk holds the full scores of
  // block blk (s_cur, with its max mx_cur); it runs the weights of blk
  // interleaved with the score products of block blk + 1, then
  // O^T += V^T P^T of blk, then exchanges the partial scores of blk + 1.
  // Register r of a score accumulator holds row 8(r/4) + 4h + r%4 (the
  // 32 x 32 MFMA output layout). The base-2 reference point m_run moves only
  // when a score passes it by more than 8 (weights stay <= 2^8); when it
  // moves with a non-zero accumulator the inner loop stops, the accumulator
  // is rescaled outside it, and the loop resumes at the same block.
  f32x16 s_cur = f32x16{};
  float mx_cur = -INFINITY;
  if (nblk > 0) {
    __syncthreads();                                   // the first blocks are in LDS
    bf16x8 kf[16];
    kfrags(0, kf);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks)
      s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s_cur, 0, 0, 0);
    put_partial(s_cur);
    __syncthreads();
    add_partner(s_cur);
    mx_cur = prep(s_cur, 0);
  }

  int blk = 0;
  for (;;) {
    // nothing the compiler loaded is pending when the inner loop starts, so
    // it places no wait inside the loop (a wait there would also hold back
    // the copies of later blocks)
    wait_vmcnt<0>();
    for (; blk < nblk; ++blk) {
      const bool move = mx_cur > (m_run == -INFINITY ? -INFINITY : m_run + 8.f);
      if (__any(move && m_run != -INFINITY)) break;   // rare: rescale below
      m_run = move ? mx_cur : m_run;                   // first used block: nothing to rescale
      const bool nxt = blk + 1 < nblk;                 // uniform
      if (nxt) {
        // block blk + 1 has landed once at most the copies of block blk + 2
        // (8 per wave, issued later, completing in order) are outstanding
        if (blk + 2 < nblk) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        __syncthreads();   // block blk + 1 is in LDS; block blk - 1 is no longer read
        if (blk + kStages - 1 < nblk)
          load_block(a.kv, ids_of(blk + kStages - 1), a.N,
                     tiles_lds + (uint32_t)((blk + kStages - 1) % kStages) * kTile, wid);
      }
      const uint32_t tcur = (uint32_t)(blk % kStages) * kTile;
      const uint32_t tnxt = (uint32_t)((blk + 1) % kStages) * kTile;

      // ---- the weights of this block beside the score products of the next
      // one (K fragments of the next block: stale data after the last block,
      // whose products are discarded), with the V^T reads of this block
      // spread over the same steps. Each step is fenced so that the issue
      // order is exactly: one product, the weight of one score, two reads.
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
      const uint8_t* vt = tiles + tcur;
      const int vc = fh * 32 + 2 * (tb & 1) + ((ti & 3) >> 1);   // chunk of dim tile 0
      auto vread = [&](int j) -> i16x4 {                         // j = 4 mt + 2 st + half
        const int mt = j >> 2, st = (j >> 1) & 1, hf = j & 1;
        const int rr = 16 * st + 4 * h + (ti >> 2) + 8 * hf;
        return lds_tr4(vt + rr * kRowBytes + (((vc + 4 * mt) ^ swz(rr) ^ ((tb & 1) << 3)) << 4) +
                       tsub);
      };
      const uint8_t* krd = tiles + tnxt + krow;
      auto kread = [&](int ks) -> bf16x8 {
        return __builtin_bit_cast(
            bf16x8, *(const u32x4*)(krd + ((fh * 32 + ((2 * ks) ^ ku ^ ((ks & 1) << 3))) << 4)));
      };
      auto vfrag = [&](const i16x4& lo, const i16x4& hi) -> bf16x8 {
        return __builtin_bit_cast(
            bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3],
                                                               hi[0], hi[1], hi[2], hi[3]});
      };
      bf16x8 kf[16];
      i16x4 vr[32];
      f32x16 s_nxt = f32x16{};
      float psum = 0.f;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) kf[ks] = kread(ks);
#pragma unroll
      for (int j = 0; j < 4; ++j) vr[j] = vread(j);
      __builtin_amdgcn_sched_barrier(0);
      // steps k = 0..15: product k, weight of score k, then the K fragment
      // eight steps ahead (k < 8) or two V^T reads of dim tiles 0..3 (k >= 8)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        s_nxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], qf[k], s_nxt, 0, 0, 0);
        s_cur[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(s_cur[k], a.scale2, neg_m));
        psum += s_cur[k];
        if (k < 8) {
          kf[k + 8] = kread(k + 8);
        } else if (k < 14) {
          vr[4 + 2 * (k - 8)] = vread(4 + 2 * (k - 8));
          vr[5 + 2 * (k - 8)] = vread(5 + 2 * (k - 8));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 pb[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4 w;
        w.x = pack_bf16x2(s_cur[8 * st + 0], s_cur[8 * st + 1]);
        w.y = pack_bf16x2(s_cur[8 * st + 2], s_cur[8 * st + 3]);
        w.z = pack_bf16x2(s_cur[8 * st + 4], s_cur[8 * st + 5]);
        w.w = pack_bf16x2(s_cur[8 * st + 6], s_cur[8 * st + 7]);
        pb[st] = __builtin_bit_cast(bf16x8, w);
      }
      psum += __shfl_xor(psum, 32);
      l_run += psum;
      __builtin_amdgcn_sched_barrier(0);
      // ---- O^T += V^T P^T: dim tiles 0..3 while tiles 4..7 are read
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int mt = q >> 1, st = q & 1;
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            vfrag(vr[4 * mt + 2 * st], vr[4 * mt + 2 * st + 1]), pb[st], acc[mt], 0, 0, 0);
        vr[16 + 2 * q] = vread(16 + 2 * q);
        vr[17 + 2 * q] = vread(17 + 2 * q);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int q = 8; q < 16; ++q) {
        const int mt = q >> 1, st = q & 1;
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            vfrag(vr[4 * mt + 2 * st], vr[4 * mt + 2 * st + 1]), pb[st], acc[mt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- exchange the next block's partial scores
      if (nxt) {
        put_partial(s_nxt);
        __syncthreads();
        add_partner(s_nxt);
        s_cur = s_nxt;
        mx_cur = prep(s_cur, blk + 1);
      }
    }
    if (blk >= nblk) break;
    // the reference point of some heads moves by more than 8 at block blk
    const bool move = mx_cur > m_run + 8.f;
    const float m_new = move ? mx_cur : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] *= alpha;
    m_run = m_new;
  }

  // ---- o = O / l (BF16), lse = ln 2 * (m + log2 l)
  const int head = hg * kHG + hp * 32 + (lane & 31);
  const bool any = l_run > 0.f;
  const float inv = any ? 1.f / l_run : 0.f;
  uint16_t* orow = a.out + ((size_t)t * a.H + head) * kD + fh * 256 + 4 * h;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 w;
      w.x = pack_bf16x2(acc[mt][4 * g + 0] * inv, acc[mt][4 * g + 1] * inv);
      w.y = pack_bf16x2(acc[mt][4 * g + 2] * inv, acc[mt][4 * g + 3] * inv);
      *(uint2*)(orow + mt * 32 + 8 * g) = w;
    }
  }
  if (fh == 0 && h == 0)
    a.lse[(size_t)t * a.H + head] =
        any ? (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace

int mla_lds_bytes() { return kMlaLds; }

hipError_t launch_sparse_mla(const MlaArgs& m, hipStream_t stream) {
  MlaKernelArgs a;
  a.q = m.q;
  a.kv = m.kv;
  a.idx = m.idx;
  a.out = m.out;
  a.lse = m.lse;
  a.T = m.T;
  a.H = m.H;
  a.N = m.N;
  a.W = m.W;
  a.groups = m.H / kHG;
  a.total = (int64_t)m.T * a.groups;
  a.per_xcd = (a.total + 7) / 8;
  a.scale2 = m.scale2;
  if (a.total == 0) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)mla_fwd_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kMlaLds);
  if (e != hipSuccess) return e;
  const int64_t grid = 8 * a.per_xcd;
  hipLaunchKernelGGL(mla_fwd_kernel, dim3((unsigned)grid), dim3(256), kMlaLds, stream, a);
  return hipGetLastError();
}

}  // namespace kpool
