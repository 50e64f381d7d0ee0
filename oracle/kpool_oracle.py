"""Plain, slow CPU oracle of the KPool DSA indexer -- test infrastructure only.

Only tests/, `__graft_entry__.smoke()` and the CPU-baseline leg of bench.py may
use this module. It shares no code with the HIP library: no kernels, headers,
helpers, tables or constants. The indexer is NumPy in FP32 (the pages fix FP32
accumulation for the pooling); the sparse attention that consumes its indices
is NumPy in FP64. Both are evaluated in the order the pages describe, with no
blocking or fusion. BF16 and E4M3 rounding are written out from their
definitions.

Sources (three web pages; cited by title and section):
  [MLM]  Megatron-LM PR #7054, "GLM5.3 Flash (KDA + mHC + KPool DSA) support +
         FP8", section "3. KPool DSA indexer + NoPE" and section "Testing".
  [SKY]  SkyRL PR #2179, "GLM-5.3-Flash (glm5_next) support", the commit that
         points megatron-core at the k-pool indexer, and "Limitations /
         follow-ups".
  [XT]   xtuner PR #2108, "Add GLM-5.3-Flash F5: NoPE DSA + KPool indexer +
         clamped SwiGLU", "Summary" and the F5 commit message.

Readings of points the pages leave open (each one is also listed in the design
notes of the repository):
  * A pool is causal for query t when every one of its tokens is at or before
    t: doc-local pools p < n_c = floor((i + 1) / kpool), i = t - cu[b]. The
    "incomplete causal pool" is the partial pool holding tokens
    n_c*kpool .. i (0 to kpool-1 tokens).
  * An incomplete pool at the end of a document is not compressed.
  * The position bias is indexed by the slot within the pool: ape[s, d].
  * Softmax is max-subtracted and normalised by division, in FP32.
  * The score scale D^-1/2 sits inside the ReLU.
  * Top-k ties go to the lower pool index; NaN scores rank as -inf.
  * Selected count is min(index_topk // kpool, n_c).
  * Output rows: the chosen pools' tokens in ascending pool order, then the
    tail tokens, then -1 up to width index_topk + kpool. Token and pool ids
    are global in the packed (THD) layout.
  * FP8 input path: 128-point Sylvester Hadamard (stages h = 1, 2, ..., 64,
    butterfly (a, b) -> (a + b, a - b)) in FP32, times FP32(128^-1/2), rounded
    to BF16; row exponent e = min{e : amax <= 448 * 2^e} (0 for an all-zero
    row); codes = OCP E4M3 (e4m3fn, max 448, subnormals kept) of y * 2^-e,
    round to nearest even. The keys are quantised after pooling.
  * Sparse attention (the consumer): one latent row per token shared by all
    heads serves as key (all d_qk components) and value (the first d_v); the
    score is sm_scale * <q, row> with sm_scale an input; an entry outside
    [0, N) is unused, every other entry is one softmax term; lse is the
    natural logarithm; a query with no used entry gets o = 0, lse = -inf.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round FP32 values to BF16 (round to nearest, ties to even); the result
    is returned as FP32 holding the BF16 value. BF16 keeps the top 16 bits of
    the FP32 encoding, so rounding adds half an ulp of the dropped 16 bits,
    plus one when the kept part is odd, and truncates."""
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)
    out = r.astype(np.uint32).view(F32)
    return np.where(np.isnan(x), F32(np.nan), out).astype(F32)


def e4m3_decode_table() -> np.ndarray:
    """Values of the 127 non-negative finite OCP E4M3 (e4m3fn) codes 0..126:
    exponent field e = code >> 3 (bias 7), mantissa m = code & 7; e == 0 is
    subnormal m * 2^-9, otherwise (1 + m/8) * 2^(e - 7). Code 127 is NaN."""
    codes = np.arange(127)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_E4M3 = e4m3_decode_table()


def e4m3_encode(x) -> np.ndarray:
    """Encode finite values with |x| <= 448 as E4M3 codes (uint8), rounding to
    the nearest representable value with ties to the even mantissa.

    The spacing of representable values is 2^(E - 3) inside binade
    [2^E, 2^(E + 1)) for E >= -6 and 2^-9 below 2^-6 (subnormals). Dividing by
    that spacing is exact in FP64 and np.rint rounds halves to even, which is
    the even mantissa because the mantissa field and the quotient share parity.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > 448.0):
        raise ValueError("e4m3_encode expects finite |x| <= 448")
    a = np.abs(x)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    E = ex - 1                               # floor(log2(a)) for a > 0
    spacing = np.where(a >= 2.0 ** -6, np.ldexp(1.0, E - 3), 2.0 ** -9)
    val = np.rint(a / spacing) * spacing
    code = np.searchsorted(_E4M3, val)
    assert np.all(_E4M3[code] == val)
    sign = np.signbit(x).astype(np.uint8) << 7       # the sign is kept, also on zero
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    mag = _E4M3[np.minimum(c & 0x7F, 126)]
    return np.where(c & 0x80, -mag, mag)


def pow2_row_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e; 0 when amax == 0."""
    amax = float(amax)
    if amax == 0.0:
        return 0
    e = int(np.ceil(np.log2(amax / 448.0)))
    while amax > np.ldexp(448.0, e):
        e += 1
    while amax <= np.ldexp(448.0, e - 1):
        e -= 1
    return e


def fwht128(x) -> np.ndarray:
    """Unnormalised 128-point Walsh-Hadamard transform of each row, in FP32,
    Sylvester (natural) order: stages h = 1, 2, 4, ..., 64; in every block of
    2h entries, entry j < h and entry j + h become (a + b, a - b)."""
    y = np.array(x, dtype=F32, copy=True)
    R, n = y.shape
    assert n == 128
    h = 1
    while h < n:
        blocks = y.reshape(R, n // (2 * h), 2, h)
        a = blocks[:, :, 0, :]
        b = blocks[:, :, 1, :]
        y = np.stack([a + b, a - b], axis=2).reshape(R, n)
        h *= 2
    return y


def fp8_quantize_rows(x):
    """FP8 input path of [MLM] section 3 (a Hadamard rotation in FP32, a BF16
    rounding, then E4M3 codes under a power-of-two scale per row), applied to
    rows of 128 BF16 values.

    Returns (codes uint8 [R, 128], exponents int [R], dequantised FP32 [R, 128]
    = decode(code) * 2^e). The row scale is 2^e."""
    x = np.asarray(x, dtype=F32)
    R = x.shape[0]
    y = bf16_round(fwht128(x) * F32(1.0 / np.sqrt(128.0)))
    amax = np.abs(y).max(axis=1) if R else np.zeros(0, F32)
    exps = np.array([pow2_row_exponent(a) for a in amax], dtype=np.int64)
    scaled = y.astype(np.float64) * np.ldexp(1.0, -exps)[:, None]
    codes = e4m3_encode(scaled)
    deq = (e4m3_decode(codes) * np.ldexp(1.0, exps)[:, None]).astype(F32)
    return codes, exps, deq


# ---------------------------------------------------------------------------
# Packed-THD bookkeeping
# ---------------------------------------------------------------------------

def cu_pools_of(cu_seqlens, kpool: int) -> np.ndarray:
    """Pool offsets per document: complete pools floor(L_b / kpool), summed.
    In a packed batch the pooling starts afresh at every document start
    ([MLM] section 3)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    counts = (cu[1:] - cu[:-1]) // kpool
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def doc_of(t: int, cu_seqlens) -> int:
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return int(np.searchsorted(cu, t, side="right") - 1)


def causal_pools(i: int, kpool: int) -> int:
    """Number of complete pools whose tokens all lie at or before doc-local
    position i."""
    return (i + 1) // kpool


# ---------------------------------------------------------------------------
# Step 1: key compression ([MLM] section 3; [SKY] k-pool commit)
# ---------------------------------------------------------------------------

def compress(k, gate, ape, cu_seqlens, kpool: int):
    """Pooled keys: for each document, each complete pool and each dimension
    d, a per-dimension softmax over the pool's slots of (gate logit + slot
    bias) weights the slot keys; FP32 arithmetic, BF16 result.

    k, gate: [T, D] (BF16 values held as FP32); ape: [kpool, D] FP32.
    Returns (pooled FP32 [P, D] holding BF16 values, cu_pools int64 [B + 1])."""
    k = np.asarray(k, dtype=F32)
    gate = np.asarray(gate, dtype=F32)
    ape = np.asarray(ape, dtype=F32)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cuP = cu_pools_of(cu, kpool)
    D = k.shape[1]
    pooled = np.zeros((int(cuP[-1]), D), dtype=F32)
    for b in range(len(cu) - 1):
        n = int(cuP[b + 1] - cuP[b])
        if n == 0:
            continue
        start = int(cu[b])
        ks = k[start:start + n * kpool].reshape(n, kpool, D)
        gs = gate[start:start + n * kpool].reshape(n, kpool, D)
        a = gs + ape[None, :, :]                       # [n, kpool, D]
        m = a[:, 0, :]
        for s in range(1, kpool):
            m = np.maximum(m, a[:, s, :])
        e = np.exp(a - m[:, None, :]).astype(F32)
        Z = e[:, 0, :]
        for s in range(1, kpool):
            Z = Z + e[:, s, :]
        pi = e / Z[:, None, :]
        acc = pi[:, 0, :] * ks[:, 0, :]
        for s in range(1, kpool):
            acc = acc + pi[:, s, :] * ks[:, s, :]
        pooled[int(cuP[b]):int(cuP[b]) + n] = bf16_round(acc)
    return pooled, cuP


# ---------------------------------------------------------------------------
# Step 2: pool scores ([MLM] section 3: the top-k is taken over pools; [XT] F5
# commit: the indexer score, with head_dim^-1/2 inside the ReLU)
# ---------------------------------------------------------------------------

def row_scores(q_t, w_t, keys, scale: float) -> np.ndarray:
    """score[p] = sum_h w[h] * ReLU(scale * q[h] . key[p]) for the given keys
    (the query's causal pools). q_t: [H, D]; w_t: [H]; keys: [n, D]."""
    q_t = np.asarray(q_t, dtype=F32)
    w_t = np.asarray(w_t, dtype=F32)
    keys = np.asarray(keys, dtype=F32)
    n = keys.shape[0]
    out = np.zeros(n, dtype=F32)
    if n == 0:
        return out
    dots = (q_t @ keys.T).astype(F32)                  # [H, n], FP32
    sc = F32(scale)
    for h in range(q_t.shape[0]):
        out = out + w_t[h] * np.maximum(F32(0.0), sc * dots[h])
    return out.astype(F32)


# ---------------------------------------------------------------------------
# Step 3: pool top-k ([MLM] section 3: top index_topk // kpool pools)
# ---------------------------------------------------------------------------

def select_pools(scores, k_sel: int) -> np.ndarray:
    """Doc-local indices of the min(k_sel, n) highest-scoring pools, in
    ascending order. Larger score first, equal scores to the lower index; NaN
    ranks as -inf."""
    s = np.asarray(scores, dtype=F32)
    n = s.shape[0]
    n_sel = min(k_sel, n)
    s = np.where(np.isnan(s), F32(-np.inf), s)
    order = np.lexsort((np.arange(n), -s))              # score desc, index asc
    return np.sort(order[:n_sel]).astype(np.int64)


# ---------------------------------------------------------------------------
# Step 4: expansion + tail ([MLM] section 3; [SKY] "Limitations / follow-ups":
# score pools, expand the chosen ones to tokens, then add the query's tail)
# ---------------------------------------------------------------------------

def expand_row(t: int, cu_seqlens, cu_pools, pool_ids_global, kpool: int,
               index_topk: int, tail_on: bool) -> np.ndarray:
    """Token row of query t: each chosen pool's kpool consecutive tokens in
    ascending pool order, then the tail tokens n_c*kpool .. i of the query's
    document, then -1 up to width index_topk + kpool."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cuP = np.asarray(cu_pools, dtype=np.int64)
    b = doc_of(t, cu)
    i = t - int(cu[b])
    row = []
    for gid in pool_ids_global:
        p = int(gid) - int(cuP[b])
        row.extend(int(cu[b]) + p * kpool + s for s in range(kpool))
    if tail_on:
        n_c = causal_pools(i, kpool)
        row.extend(range(int(cu[b]) + n_c * kpool, t + 1))
    W = index_topk + kpool
    assert len(row) <= W
    return np.array(row + [-1] * (W - len(row)), dtype=np.int32)


# ---------------------------------------------------------------------------
# The whole path
# ---------------------------------------------------------------------------

def indexer_topk(q, w, pooled, cu_seqlens, kpool: int, index_topk: int,
                 tail_on: bool, scale: float = 0.0, rows=None, fp8: bool = False,
                 return_scores: bool = False):
    """Token indices [R, index_topk + kpool] and global pool ids
    [R, index_topk // kpool] (-1 padded) for the query rows `rows` (default:
    all). q: [T, H, D]; w: [T, H] FP32; pooled: [P, D] (BF16 values).

    With fp8, q rows (t, h) and pooled rows are replaced by their dequantised
    FP8 values before scoring."""
    q = np.asarray(q, dtype=F32)
    w = np.asarray(w, dtype=F32)
    pooled = np.asarray(pooled, dtype=F32)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    cuP = cu_pools_of(cu, kpool)
    T, H, D = q.shape
    if scale == 0.0:
        scale = float(F32(1.0 / np.sqrt(D)))
    rows = list(range(T)) if rows is None else [int(r) for r in rows]
    k_sel = index_topk // kpool
    W = index_topk + kpool
    if fp8:
        _, _, keys_all = fp8_quantize_rows(pooled)
    else:
        keys_all = pooled
    tok = np.full((len(rows), W), -1, dtype=np.int32)
    pid = np.full((len(rows), k_sel), -1, dtype=np.int32)
    all_scores = []
    for r, t in enumerate(rows):
        b = doc_of(t, cu)
        i = t - int(cu[b])
        n_c = causal_pools(i, kpool)
        keys = keys_all[int(cuP[b]):int(cuP[b]) + n_c]
        q_t = q[t]
        if fp8:
            _, _, q_t = fp8_quantize_rows(q_t)
        sc = row_scores(q_t, w[t], keys, scale)
        if return_scores:
            all_scores.append(sc)
        chosen = select_pools(sc, k_sel) + int(cuP[b])
        pid[r, :len(chosen)] = chosen
        tok[r] = expand_row(t, cu, cuP, chosen, kpool, index_topk, tail_on)
    if return_scores:
        return tok, pid, all_scores
    return tok, pid


# ---------------------------------------------------------------------------
# Serving: one query per sequence over its cached pools ([MLM] sections 3
# and 4: the serving indexer scores the pools of a growing sequence)
# ---------------------------------------------------------------------------

def decode_topk(q, w, pooled, pool_start, seq_lens, kpool: int, index_topk: int,
                tail_on: bool, scale: float = 0.0, token_base=None, fp8: bool = False):
    """Token rows [B, index_topk + kpool] and pool ids [B, index_topk //
    kpool] for B sequences, one query each: sequence b has L_b = seq_lens[b]
    tokens, its query is token L_b - 1, and its floor(L_b / kpool) complete
    pools are pooled rows pool_start[b] onwards. Row b is the row
    indexer_topk gives the last token of a document of L_b tokens (pool ids
    offset by pool_start[b], token ids by token_base[b]); L_b = 0 gives a row
    of -1. q: [B, H, D]; w: [B, H] FP32; pooled: [P, D] (BF16 values). With
    fp8, q rows (b, h) and the pooled rows are replaced by their dequantised
    FP8 values before scoring, as in indexer_topk."""
    q = np.asarray(q, dtype=F32)
    w = np.asarray(w, dtype=F32)
    pooled = np.asarray(pooled, dtype=F32)
    B, H, D = q.shape
    if scale == 0.0:
        scale = float(F32(1.0 / np.sqrt(D)))
    k_sel = index_topk // kpool
    W = index_topk + kpool
    tok = np.full((B, W), -1, dtype=np.int32)
    pid = np.full((B, k_sel), -1, dtype=np.int32)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        base = 0 if token_base is None else int(token_base[b])
        n_c = causal_pools(L - 1, kpool)
        keys = pooled[int(pool_start[b]):int(pool_start[b]) + n_c]
        q_b = q[b]
        if fp8:
            _, _, keys = fp8_quantize_rows(keys)
            _, _, q_b = fp8_quantize_rows(q_b)
        chosen = select_pools(row_scores(q_b, w[b], keys, scale), k_sel)
        pid[b, :len(chosen)] = chosen + int(pool_start[b])
        # the expansion of the last token of a one-document batch [0, L)
        row = expand_row(L - 1, [0, L], [0, L // kpool], chosen, kpool, index_topk, tail_on)
        tok[b] = np.where(row >= 0, row + base, -1)
    return tok, pid



# ---------------------------------------------------------------------------
# The indexer projections feeding the path ([MLM] section 4, the DSA indexer
# precision split and its forward fragment: q from linear_wq_b of the query
# latent, k = k_norm(linear_wk(x)), the head weights from linear_weights_proj
# kept in FP32; [MLM] section 3: the per-token compression gate). Readings:
# the compression gate is a linear map of the same input x to D gate logits
# per token (BF16, like linear_wk); a linear layer's BF16 output is its FP32
# product rounded to BF16, and k_norm is a LayerNorm over the D values of a
# row, evaluated in FP32 on the BF16 output of linear_wk. No rotary embedding
# (the NoPE indexer) and no activation rotation.
# ---------------------------------------------------------------------------

def linear_bf16(a, w):
    """A BF16 linear layer: a [T, K] @ w[N, K]^T with FP32 products and sums,
    rounded to BF16 (returned as FP32 holding BF16 values)."""
    a = np.asarray(a, dtype=F32)
    w = np.asarray(w, dtype=F32)
    return bf16_round((a @ w.T).astype(F32))


def layer_norm(v, gamma, beta, eps: float):
    """LayerNorm of each row of v over its last axis, in FP32: (v - mean) /
    sqrt(var + eps) * gamma + beta, var the mean squared deviation."""
    v = np.asarray(v, dtype=F32)
    mean = (v.sum(axis=1, dtype=F32) / F32(v.shape[1])).astype(F32)
    dev = (v - mean[:, None]).astype(F32)
    var = ((dev * dev).sum(axis=1, dtype=F32) / F32(v.shape[1])).astype(F32)
    inv = (F32(1.0) / np.sqrt(var + F32(eps))).astype(F32)
    return (dev * inv[:, None] * np.asarray(gamma, F32)[None, :]
            + np.asarray(beta, F32)[None, :]).astype(F32)


def indexer_projections(x, qr, wq_b, wk, k_norm_weight, k_norm_bias, wg, ww,
                        num_heads: int, head_dim: int, eps: float = 1e-6):
    """The four inputs of the indexer for T tokens.
      x   [T, hidden] (BF16 values), qr [T, q_lora_rank] (BF16 values)
      wq_b [H*D, q_lora_rank], wk [D, hidden], wg [D, hidden] (BF16 values)
      k_norm_weight, k_norm_bias [D] (FP32); ww [H, hidden] (FP32)
    Returns q [T, H, D] (BF16 values), k [T, D] (BF16 values), gate [T, D]
    (BF16 values) and w [T, H] (FP32)."""
    T = np.asarray(x).shape[0]
    q = linear_bf16(qr, wq_b).reshape(T, num_heads, head_dim)
    k = bf16_round(layer_norm(linear_bf16(x, wk), k_norm_weight, k_norm_bias, eps))
    gate = linear_bf16(x, wg)
    w = (np.asarray(x, dtype=F32) @ np.asarray(ww, dtype=F32).T).astype(F32)
    return q, k, gate, w


# ---------------------------------------------------------------------------
# The consumer of the indices: sparse attention of the NoPE absorbed MLA.
# [XT] Summary: a new sparse MLA backend runs FlashMLA's forward over the
# indexer's int32 token indices; its heads must come in multiples of 64, and
# its (head_dim, value_dim) pair is no longer fixed at 576. [MLM] section 3:
# with NoPE the absorbed query has no positional slice. [XT] LSE fix commit:
# the saved softmax LSE is the natural logarithm.
# Readings: in the absorbed form every head attends to one shared latent row
# per token; with no positional slice that row is both the key (all d_qk
# components) and the value (its first d_v components). The score is
# sm_scale * <q, row>; sm_scale is an input, since the pages give no value.
# A listed entry outside [0, N) -- the indexer's -1 padding -- is unused;
# every other entry is one term of the softmax (a row listed twice counts
# twice). A query with no used entry gets o = 0 and lse = -inf.
# Evaluated in FP64 from the BF16 inputs.
# ---------------------------------------------------------------------------

def sparse_mla_forward(q, kv, indices, sm_scale: float, d_v: int | None = None):
    """q [T, H, d_qk], kv [N, d_qk], indices [T, W] integers.
    Returns o [T, H, d_v] and lse [T, H] (natural log), both FP64."""
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    indices = np.asarray(indices)
    T, H, d_qk = q.shape
    N = kv.shape[0]
    if d_v is None:
        d_v = d_qk
    o = np.zeros((T, H, d_v))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        sel = [int(j) for j in indices[t] if 0 <= int(j) < N]
        if not sel:
            continue
        rows = kv[sel]                              # [n, d_qk]
        s = sm_scale * (q[t] @ rows.T)              # [H, n]
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        l = e.sum(axis=1)
        o[t] = (e @ rows[:, :d_v]) / l[:, None]
        lse[t] = m + np.log(l)
    return o, lse
