// Step 4 of the KPool indexer: expansion of the chosen pools to token indices
// and the always-select-tail append.
//
// Megatron-LM PR #7054, section "3. KPool DSA indexer + NoPE": the top pools
// are expanded back to token indices and, with always_select_tail, each query
// also keeps its incomplete causal pool so that short prefixes stay fully
// visible. SkyRL PR #2179 ("Limitations / follow-ups") gives the order:
// score pools, expand them to tokens, append the query's tail pool.
//
// HBM-bound and write-dominated: per row it reads K_sel pool ids (4 bytes
// each) and writes W = index_topk + kpool token ids. One wave per row; the
// row's document facts are wave-uniform. For kpool == 4 a lane turns one pool
// id into one 16-byte store of four consecutive tokens.

#include "kpool_device.h"
#include "kpool_internal.h"

namespace kpool {

constexpr int kExpandWaves = 4;

template <bool VEC4>
__global__ __launch_bounds__(64 * kExpandWaves) void expand_kernel(
    const int32_t* __restrict__ pool_ids, int q_begin, int q_end,
    const int32_t* __restrict__ cu, const int32_t* __restrict__ cu_pools, int B, int T,
    int kpool, int k_sel, int width, int tail_on, int max_pools,
    int32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * kExpandWaves + (threadIdx.x >> 6);
  const int t = q_begin + r;
  if (t >= q_end) return;
  const QueryInfo qi = query_info(cu, cu_pools, B, T, kpool, max_pools, t);
  const int n_sel = qi.n_c < k_sel ? qi.n_c : k_sel;
  const int tail = tail_on ? (qi.i + 1) % kpool : 0;
  const int n_pool_tok = n_sel * kpool;
  const int tail_base = qi.start + qi.n_c * kpool;
  const int32_t* ids = pool_ids + (size_t)r * k_sel;
  int32_t* o = out + (size_t)r * width;
  if (VEC4) {
    // kpool == 4 and width % 4 == 0: group j of four outputs is pool slot j
    // while j < n_sel, else tail / padding. A lane requests the ids of KU
    // groups before it stores any, so their loads are in flight together
    // (streaming stores were tried here and were slower).
    constexpr int KU = 8;      // measured best of 2 .. 16 on 64K rows of 2052
    typedef int i32x4v __attribute__((ext_vector_type(4)));
    const int groups = width >> 2;
    for (int j0 = lane; j0 < groups; j0 += 64 * KU) {
      int idv[KU];
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int j = j0 + 64 * u;
        idv[u] = j < n_sel ? ids[j] : 0;
      }
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int j = j0 + 64 * u;
        if (j >= groups) break;
        i32x4v v;
        if (j < n_sel) {
          const int base = qi.start + (idv[u] - qi.pool0) * 4;
          v = i32x4v{base, base + 1, base + 2, base + 3};
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int jj = j * 4 + c - n_pool_tok;
            v[c] = jj < tail ? tail_base + jj : -1;
          }
        }
        *reinterpret_cast<i32x4v*>(o + j * 4) = v;
      }
    }
  } else {
    for (int j = lane; j < width; j += 64) {
      int v;
      if (j < n_pool_tok) {
        int slot = j / kpool;
        v = qi.start + (ids[slot] - qi.pool0) * kpool + (j - slot * kpool);
      } else {
        int jj = j - n_pool_tok;
        v = jj < tail ? tail_base + jj : -1;
      }
      o[j] = v;
    }
  }
}

void launch_expand(const int32_t* pool_ids, int q_begin, int q_end, const int32_t* cu,
                   const int32_t* cu_pools, int B, int T, int kpool, int k_sel, int width,
                   int tail, int max_pools, int32_t* out, hipStream_t st) {
  const int rows = q_end - q_begin;
  if (rows <= 0) return;
  dim3 grid((rows + kExpandWaves - 1) / kExpandWaves), block(64 * kExpandWaves);
  if (kpool == 4 && (width & 3) == 0)
    expand_kernel<true><<<grid, block, 0, st>>>(pool_ids, q_begin, q_end, cu, cu_pools, B, T,
                                                kpool, k_sel, width, tail, max_pools, out);
  else
    expand_kernel<false><<<grid, block, 0, st>>>(pool_ids, q_begin, q_end, cu, cu_pools, B, T,
                                                 kpool, k_sel, width, tail, max_pools, out);
}

}  // namespace kpool
