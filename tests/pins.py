"""Pins of the CPU oracle: checks against what the pages and mathematics fix,
not against the oracle itself. Each pin takes the oracle module as an argument
so that test_oracle_mutations.py can run the same pins against an oracle with
a planted mistake and see them fail.

The pages (cited by title and section):
  Megatron-LM PR #7054 "GLM5.3 Flash (KDA + mHC + KPool DSA) support + FP8",
    section "3. KPool DSA indexer + NoPE" (pooling, pool top-k, expansion,
    always-select-tail, packed restart, FP8 input path) and "Testing"
    (full causal prefix kept under the pool budget; FP8 emulation against an
    explicit Hadamard matrix).
  SkyRL PR #2179, k-pool commit (below the budget every pool is selectable)
    and "Limitations / follow-ups" (score, expand, append the tail).
  xtuner PR #2108 F5 commit message (ReLU homogeneity lets head_dim^-1/2 move
    from the ReLU argument into the head weight), Summary (the sparse MLA
    forward over the indices) and the LSE fix commit (natural-log LSE).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import brute_force as bf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32 = np.float32


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16_ulp(x):
    """Spacing of BF16 values at |x| (8 significant bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    a = np.maximum(a, 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(int) - 7)


def assert_within_bf16_ulps(got, ref, n=1, floor=None):
    """|got - ref| <= n BF16 ulps (of the larger of the two), plus an optional
    absolute floor per element (the FP32 evaluation error bound of a sum that
    cancels, see pooled_fp32_floor)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    lim = n * np.maximum(bf16_ulp(ref), bf16_ulp(got))
    if floor is not None:
        lim = lim + floor
    bad = err > lim
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} values beyond {n} BF16 ulp; first at {tuple(i)}: "
                             f"got {got[tuple(i)]} ref {ref[tuple(i)]} limit {lim[tuple(i)]}")


def pooled_fp32_floor(k, gate, ape, cu_seqlens, kpool):
    """Per (pool, dim) absolute error bound of evaluating the pooled key in
    FP32: the slot weights carry a few ulps from exp, the sum and the division,
    the weighted sum adds one rounding per slot, so each side is within
    (2 kpool + 8) * 2^-24 * sum_s |pi_s k_s| of the exact value; two sides that
    err in opposite directions differ by twice that. When the slot terms cancel
    this bound exceeds one BF16 ulp of the result."""
    k = np.asarray(k, np.float64)
    a = np.asarray(gate, np.float64)
    ape = np.asarray(ape, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    rows = []
    for b in range(len(cu) - 1):
        n = int((cu[b + 1] - cu[b]) // kpool)
        if n == 0:
            continue
        s = int(cu[b])
        ks = k[s:s + n * kpool].reshape(n, kpool, -1)
        lg = a[s:s + n * kpool].reshape(n, kpool, -1) + ape[None]
        e = np.exp(lg - lg.max(axis=1, keepdims=True))
        pi = e / e.sum(axis=1, keepdims=True)
        rows.append(np.abs(pi * ks).sum(axis=1))
    if not rows:
        return np.zeros((0, k.shape[1]))
    return 2.0 * (2 * kpool + 8) * 2.0 ** -24 * np.concatenate(rows)


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(*shape, generator=g)).to(torch.bfloat16).float().numpy()


# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

def pin_bf16_round_matches_library(o):
    """BF16 RNE equals torch's float32 -> bfloat16 conversion."""
    g = torch.Generator().manual_seed(1)
    x = torch.cat([torch.randn(20000, generator=g) * 10.0 ** e for e in range(-30, 31, 6)])
    # exact halfway cases: low 16 bits = 0x8000, both parities of bit 16
    u = torch.randint(0, 2 ** 15, (4096,), generator=g, dtype=torch.int32) * 2 ** 17
    halves = (u | 0x8000).view(torch.float32)
    halves_odd = ((u + 2 ** 16) | 0x8000).view(torch.float32)
    x = torch.cat([x, halves, halves_odd])
    x = x[torch.isfinite(x)]
    ref = x.to(torch.bfloat16).float().numpy()
    got = o.bf16_round(x.numpy())
    assert np.array_equal(ref.view(np.uint32), got.view(np.uint32))


def pin_e4m3_exhaustive(o):
    """E4M3 codes equal torch's float8_e4m3fn cast for every finite BF16 value
    with |x| <= 448 (the cast is an independent RNE implementation)."""
    b = torch.arange(0, 65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    x = b.float()
    x = x[torch.isfinite(x) & (x.abs() <= 448)]
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = o.e4m3_encode(x.numpy())
    assert np.array_equal(ref, got)
    # decoding gives the value torch reads back
    dec = torch.from_numpy(got).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(o.e4m3_decode(got).astype(F32), dec)


def pin_pow2_exponent(o):
    """Closed forms of the smallest e with amax <= 448 * 2^e."""
    cases = {448.0: 0, 449.0: 1, 896.0: 1, 897.0: 2, 224.0: -1, 1.0: -8,
             0.875: -9, 0.876: -8, 2.0 ** -20: -28, 0.0: 0}
    for amax, e in cases.items():
        assert o.pow2_row_exponent(amax) == e, (amax, e, o.pow2_row_exponent(amax))


def pin_fwht_matches_matrix(o):
    """The FWHT equals multiplication by the explicit Sylvester Hadamard matrix
    (scipy) within FP32 rounding, and applying it twice gives 128 x."""
    from scipy.linalg import hadamard
    x = rnd((64, 128), 3)
    Hm = hadamard(128).astype(np.float64)
    ref = x.astype(np.float64) @ Hm.T
    got = o.fwht128(x).astype(np.float64)
    assert np.allclose(got, ref, rtol=0, atol=1e-4 * np.abs(x).sum(axis=1).max())
    twice = o.fwht128(o.fwht128(x)).astype(np.float64)
    assert np.allclose(twice, 128.0 * x, rtol=0, atol=1e-3)


def pin_fp8_golden(o):
    g = load_golden("fp8_rows.json")
    for row in g["rows"]:
        x = np.zeros((1, 128), F32)
        for j, v in row["x_nonzero"].items():
            x[0, int(j)] = v
        codes, exps, deq = o.fp8_quantize_rows(x)
        assert int(exps[0]) == row["exponent"]
        for key, val in row["codes"].items():
            sl = {"all": slice(None), "even": slice(0, None, 2), "odd": slice(1, None, 2)}[key]
            assert np.all(codes[0, sl] == val), (key, codes[0, sl][:4])
        for key, val in row["dequant"].items():
            sl = {"all": slice(None), "even": slice(0, None, 2), "odd": slice(1, None, 2)}[key]
            assert np.all(deq[0, sl] == F32(val))


def pin_fp8_error_bound(o):
    """Dequantised rows stay within the E4M3 half-step of the rotated BF16 row
    (relative 2^-4 of each value, or half the subnormal step 2^-10 * 2^e), and
    the rotation preserves dot products: deq(Hq) . deq(Hk) ~ q . k."""
    x = rnd((256, 128), 4)
    codes, exps, deq = o.fp8_quantize_rows(x)
    from scipy.linalg import hadamard
    y = (x.astype(np.float64) @ hadamard(128).T) / math.sqrt(128.0)
    scale = np.ldexp(1.0, exps)[:, None]
    lim = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10 * scale) + np.abs(y) * 2.0 ** -8
    assert np.all(np.abs(deq - y) <= lim * 1.0001)
    amax = np.abs(y).max(axis=1)          # FP64 rotation; BF16 rounding moves it < 2^-8
    assert np.all(amax <= 448.0 * scale[:, 0] * (1 + 2.0 ** -7))
    assert np.all(amax > 224.0 * scale[:, 0] * (1 - 2.0 ** -7))
    dots_ref = (x[:128].astype(np.float64) * x[128:]).sum(1)
    dots = (deq[:128].astype(np.float64) * deq[128:]).sum(1)
    norms = np.linalg.norm(x[:128], axis=1) * np.linalg.norm(x[128:], axis=1)
    assert np.all(np.abs(dots - dots_ref) <= 2.0 ** -4 * norms)   # Cauchy-Schwarz on the error


# ---------------------------------------------------------------------------
# Compression
# ---------------------------------------------------------------------------

def pin_compress_kpool1_identity(o):
    """One slot: the softmax weight is exactly 1, so pooled == k."""
    k, gate = rnd((37, 64), 5), rnd((37, 64), 6)
    ape = rnd((1, 64), 7, 0.1)
    pooled, cuP = o.compress(k, gate, ape, [0, 20, 37], 1)
    assert np.array_equal(pooled, k) and list(cuP) == [0, 20, 37]


def pin_compress_uniform_mean(o):
    """Equal logits in every slot: weights are exactly 1/kpool, so the pooled
    key is the BF16 mean of the slot keys (exact scaling by 1/4)."""
    k = rnd((64, 32), 8)
    gate = np.repeat(rnd((16, 32), 9), 4, axis=0)      # same logit in all 4 slots
    ape = np.zeros((4, 32), F32)
    pooled, _ = o.compress(k, gate, ape, [0, 64], 4)
    kk = torch.from_numpy(k).reshape(16, 4, 32)
    s = ((kk[:, 0] + kk[:, 1]) + kk[:, 2]) + kk[:, 3]
    ref = (s * 0.25).to(torch.bfloat16).float().numpy()
    assert np.array_equal(pooled, ref)


def pin_compress_closed_form_kpool2(o):
    """Two slots: weights are the logistic sigmoid of the logit difference,
    pooled = sig(a0 - a1) k0 + sig(a1 - a0) k1 (FP64), within 1 BF16 ulp.
    The slot bias is asymmetric so a transposed or misindexed bias shows."""
    k = rnd((40, 16), 10)
    gate = rnd((40, 16), 11, 2.0)
    ape = rnd((2, 16), 12, 1.0)
    pooled, _ = o.compress(k, gate, ape, [0, 40], 2)
    a0 = gate[0::2].astype(np.float64) + ape[0]
    a1 = gate[1::2].astype(np.float64) + ape[1]
    s0 = 1.0 / (1.0 + np.exp(a1 - a0))
    ref = s0 * k[0::2] + (1.0 - s0) * k[1::2]
    assert_within_bf16_ulps(pooled, ref, 1)


def pin_compress_dominant_slot(o):
    """A slot whose logit exceeds the others by >= 100 takes weight 1 in FP32:
    pooled equals that slot's key bit-exactly, for every slot position."""
    for dom in range(4):
        k = rnd((32, 16), 13 + dom)
        gate = rnd((32, 16), 20 + dom)
        gate[dom::4] += 200.0
        ape = rnd((4, 16), 30, 0.1)
        pooled, _ = o.compress(k, gate, ape, [0, 32], 4)
        assert np.array_equal(pooled, k[dom::4]), dom


def pin_compress_convex(o):
    """Pooled values lie between the smallest and largest slot key, per dim."""
    k = rnd((128, 32), 40)
    pooled, _ = o.compress(k, rnd((128, 32), 41, 3.0), rnd((4, 32), 42, 0.5), [0, 128], 4)
    kk = k.reshape(32, 4, 32)
    assert np.all(pooled >= kk.min(1)) and np.all(pooled <= kk.max(1))


def pin_compress_packed_restart(o):
    """Packed documents pool independently: pools never straddle a document
    start, incomplete end-of-document pools are dropped, and the packed result
    equals each document compressed alone."""
    lens = [7, 1, 12, 0, 9]
    T = sum(lens)
    k, gate, ape = rnd((T, 16), 50), rnd((T, 16), 51), rnd((4, 16), 52, 0.1)
    cu = np.concatenate([[0], np.cumsum(lens)])
    pooled, cuP = o.compress(k, gate, ape, cu, 4)
    assert list(cuP) == [0, 1, 1, 4, 4, 6]
    parts = []
    for b, L in enumerate(lens):
        s = cu[b]
        p, _ = o.compress(k[s:s + L], gate[s:s + L], ape, [0, L], 4)
        parts.append(p)
    assert np.array_equal(pooled, np.concatenate(parts))


def pin_compress_brute_fp64(o):
    """FP64 brute force on tiny packed inputs, every kpool in {1, 2, 3, 4}."""
    for kp in (1, 2, 3, 4):
        lens = [9, 6, 13]
        T = sum(lens)
        k, gate = rnd((T, 8), 60 + kp), rnd((T, 8), 70 + kp, 2.0)
        ape = rnd((kp, 8), 80 + kp, 0.5)
        cu = np.concatenate([[0], np.cumsum(lens)])
        pooled, _ = o.compress(k, gate, ape, cu, kp)
        ref = np.array(bf.brute_pooled(k, gate, ape, lens, kp))
        assert_within_bf16_ulps(pooled, ref, 1, pooled_fp32_floor(k, gate, ape, cu, kp) / 2)


def pin_compress_slot_shift_invariance(o):
    """Adding one constant to every slot's logit of a pool (per dimension)
    leaves the softmax, hence the pooled key, unchanged (to 1 BF16 ulp)."""
    k, gate, ape = rnd((64, 16), 90), rnd((64, 16), 91), rnd((4, 16), 92, 0.2)
    shift = np.repeat(rnd((16, 16), 93, 3.0), 4, axis=0)
    p0, _ = o.compress(k, gate, ape, [0, 64], 4)
    p1, _ = o.compress(k, (gate + shift).astype(F32), ape, [0, 64], 4)
    assert_within_bf16_ulps(p1, p0, 1)


# ---------------------------------------------------------------------------
# Scores, selection, expansion
# ---------------------------------------------------------------------------

def pin_scores_onehot_golden(o):
    g = load_golden("scores_onehot.json")
    q = np.array(g["q"], F32)
    w = np.array(g["w"], F32)
    keys = np.array(g["keys"], F32)
    s = o.row_scores(q, w, keys, 1.0 / math.sqrt(g["D"]))
    assert np.array_equal(s, np.array(g["scores"], F32)), s
    assert list(o.select_pools(s, 2)) == g["top2_pools"]


def pin_scores_odd_in_w(o):
    """The score is linear in the head weights: negating w negates every score
    exactly (a mistake that put w inside the ReLU would break this)."""
    q = rnd((8, 64), 100).reshape(8, 64)
    keys = rnd((30, 64), 101)
    w = rnd((8,), 102)
    s1 = o.row_scores(q, w, keys, 0.125)
    s2 = o.row_scores(q, -w, keys, 0.125)
    assert np.array_equal(s1, -s2) and np.any(s1 != 0)


def pin_scores_single_head_relu(o):
    """One head with w = 1: score = ReLU(scale * q . k) (FP64 reference), and a
    key orthogonal to q scores exactly 0."""
    q = rnd((1, 32), 110)
    keys = rnd((50, 32), 111)
    keys[7] = 0.0
    s = o.row_scores(q, np.ones(1, F32), keys, 0.25)
    ref = np.maximum(0.0, 0.25 * (keys.astype(np.float64) @ q[0].astype(np.float64)))
    assert np.allclose(s, ref, rtol=1e-5, atol=1e-6) and s[7] == 0.0


def pin_relu_homogeneity(o):
    """Moving the scale D^-1/2 out of the ReLU into w changes nothing: bit-exact
    for D = 64 (scale 2^-3), within FP32 rounding for D = 128, and the chosen
    pools are identical."""
    for D, exact in ((64, True), (128, False)):
        H = 8
        q = rnd((H, D), 120 + D)
        keys = rnd((300, D), 121 + D)
        w = rnd((H,), 122 + D)
        sc = float(F32(1.0 / math.sqrt(D)))
        inside = o.row_scores(q, w, keys, sc)
        folded = o.row_scores(q, (w * F32(sc)).astype(F32), keys, 1.0)
        if exact:
            assert np.array_equal(inside, folded)
        else:
            assert np.allclose(inside, folded, rtol=1e-5, atol=1e-6)
        assert np.array_equal(o.select_pools(inside, 40), o.select_pools(folded, 40))


def pin_select_matches_sort(o):
    """Selection equals a full sort by (score desc, index asc), including ties,
    -inf and NaN (ranked as -inf)."""
    g = torch.Generator().manual_seed(130)
    for n, k in ((1, 1), (5, 3), (100, 16), (1000, 256), (64, 64), (10, 20)):
        s = torch.randint(-4, 5, (n,), generator=g).float().numpy() * 0.5
        if n > 10:
            s[3] = np.nan
            s[4] = -np.inf
            s[5] = np.inf
        key = [(-(-np.inf if np.isnan(v) else v), j) for j, v in enumerate(s)]
        ref = sorted(j for _, j in sorted(key)[:min(k, n)])
        assert list(o.select_pools(s.astype(F32), k)) == ref
    # NaN ranks as -inf and then loses or wins the tie by index
    assert list(o.select_pools(np.array([np.nan, -np.inf, 1.0], F32), 2)) == [0, 2]
    assert list(o.select_pools(np.array([-np.inf, np.nan, 1.0], F32), 2)) == [0, 2]


def pin_select_kpool1_matches_topk(o):
    """With kpool = 1 the method is token-level DSA top-k; on tie-free scores
    the chosen set equals torch.topk of the token-level scores."""
    T, H, D, topk = 200, 4, 16, 32
    q = rnd((T, H, D), 140)
    k = rnd((T, D), 141)
    w = rnd((T, H), 142)
    ape = np.zeros((1, D), F32)
    pooled, _ = o.compress(k, rnd((T, D), 143), ape, [0, T], 1)
    tok, pid = o.indexer_topk(q, w, pooled, [0, T], 1, topk, True)
    qt = torch.from_numpy(q).double()
    kt = torch.from_numpy(k).double()
    sc = torch.einsum("thd,sd->ths", qt, kt) * (1.0 / math.sqrt(D))
    full = (torch.from_numpy(w).double()[:, :, None] * sc.clamp_min(0)).sum(1)
    for t in range(T):
        n = t + 1
        ref = sorted(torch.topk(full[t, :n], min(topk, n)).indices.tolist())
        got = sorted(int(x) for x in pid[t] if x >= 0)
        if got != ref:      # FP32 vs FP64 may swap pools tied to ~1e-6
            kth = float(torch.topk(full[t, :n], min(topk, n)).values[-1])
            for j in set(got) ^ set(ref):
                assert abs(float(full[t, j]) - kth) <= 1e-5 * max(abs(kth), 1e-3), (t, j)
        else:
            assert [int(x) for x in tok[t] if x >= 0] == ref


def pin_expand_golden(o):
    g = load_golden("expand_two_docs.json")
    cu = g["cu_seqlens"]
    kp, topk = g["kpool"], g["index_topk"]
    cuP = o.cu_pools_of(cu, kp)
    for mode, tail in (("tail_on", True), ("tail_off", False)):
        for t in range(cu[-1]):
            b = o.doc_of(t, cu)
            i = t - cu[b]
            n_c = o.causal_pools(i, kp)
            scores = np.array(g["scores"].get(str(t), [0.0] * n_c), F32)
            assert len(scores) == n_c
            chosen = o.select_pools(scores, topk // kp) + cuP[b]
            if mode == "tail_on":
                exp_ids = [x for x in g["tail_on"]["pool_ids"][t] if x >= 0]
                assert list(chosen) == exp_ids, t
            row = o.expand_row(t, cu, cuP, chosen, kp, topk, tail)
            assert list(row) == g[mode]["tokens"][t], (mode, t, row)


def _tiny_case(seed, lens, H, D, kp, with_ties=False):
    T = sum(lens)
    q, k, gate = rnd((T, H, D), seed), rnd((T, D), seed + 1), rnd((T, D), seed + 2)
    w = rnd((T, H), seed + 3) / math.sqrt(H)
    ape = rnd((kp, D), seed + 4, 0.1)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return q, k, gate, w.astype(F32), ape, cu


def pin_end_to_end_brute(o):
    """FP64 brute force (explicit token sets, full sort, tail = visible tokens
    no causal pool covers) on tiny packed inputs, kpool in {1, 2, 4}, tail on
    and off. Pooled keys agree to 1 BF16 ulp; scores to 1e-5 relative; the
    chosen sets agree except where the brute-force scores are within 1e-4
    relative of the k-th score; token rows follow the chosen sets exactly."""
    for kp in (1, 2, 4):
        for tail in (True, False):
            lens = [23, 5, 36]
            H, D, topk = 3, 8, 8
            q, k, gate, w, ape, cu = _tiny_case(200 + kp, lens, H, D, kp)
            pooled, cuP = o.compress(k, gate, ape, cu, kp)
            keys64 = bf.brute_pooled(k, gate, ape, lens, kp)
            assert_within_bf16_ulps(pooled, np.array(keys64).reshape(pooled.shape), 1)
            sc = float(F32(1.0 / math.sqrt(D)))
            tok, pid, scores = o.indexer_topk(q, w, pooled, cu, kp, topk, tail, sc,
                                              return_scores=True)
            btok, bpid, bsc = bf.brute_rows(q, w, pooled.tolist(), lens, kp, topk, tail, sc)
            for t in range(sum(lens)):
                b = o.doc_of(t, cu)
                ids = sorted(bsc[t])
                ref_s = np.array([bsc[t][g] for g in ids])
                assert [g - int(cuP[b]) for g in ids] == list(range(len(ids)))
                assert np.allclose(scores[t], ref_s, rtol=1e-5, atol=1e-6)
                got = set(int(x) for x in pid[t] if x >= 0)
                ref = set(x for x in bpid[t] if x >= 0)
                if got != ref:
                    kth = sorted(ref_s, reverse=True)[topk // kp - 1]
                    for gid in got ^ ref:
                        assert abs(bsc[t][gid] - kth) <= 1e-4 * abs(kth), (t, gid)
                else:
                    assert list(tok[t]) == btok[t], (kp, tail, t)


def pin_prefix_visibility(o):
    """With the tail on, a query whose document prefix has at most
    index_topk + kpool - 1 tokens sees exactly every token of its document up
    to itself, whatever the weights (the 'full causal prefix under the pool
    budget' property of the pages' test suite)."""
    lens = [40, 17, 70]
    H, D, kp, topk = 2, 8, 4, 32
    q, k, gate, w, ape, cu = _tiny_case(300, lens, H, D, kp)
    pooled, _ = o.compress(k, gate, ape, cu, kp)
    tok, _ = o.indexer_topk(q, w, pooled, cu, kp, topk, True)
    for t in range(sum(lens)):
        b = o.doc_of(t, cu)
        i = t - int(cu[b])
        row = [int(x) for x in tok[t] if x >= 0]
        if i + 1 <= topk + kp - 1:
            assert row == list(range(int(cu[b]), t + 1)), t


def pin_counts_and_restart(o):
    """Row structure: kpool * min(K_sel, n_c) + tail valid entries, strictly
    ascending, inside the query's document and at or before the query; each
    chosen pool contributes kpool consecutive tokens starting on a pool
    boundary of that document."""
    lens = [61, 3, 90, 8]
    H, D, kp, topk = 2, 8, 4, 16
    q, k, gate, w, ape, cu = _tiny_case(400, lens, H, D, kp)
    pooled, cuP = o.compress(k, gate, ape, cu, kp)
    tok, pid = o.indexer_topk(q, w, pooled, cu, kp, topk, True)
    for t in range(sum(lens)):
        b = o.doc_of(t, cu)
        lo = int(cu[b])
        i = t - lo
        n_c = (i + 1) // kp
        row = [int(x) for x in tok[t] if x >= 0]
        assert all(x == -1 for x in tok[t][len(row):])
        assert len(row) == kp * min(topk // kp, n_c) + (i + 1) % kp
        assert row == sorted(set(row)) and all(lo <= x <= t for x in row)
        ids = [int(x) for x in pid[t] if x >= 0]
        assert len(ids) == min(topk // kp, n_c)
        assert all(cuP[b] <= g < cuP[b] + n_c for g in ids)
        for j, g in enumerate(ids):
            start = lo + (g - int(cuP[b])) * kp
            assert row[j * kp:(j + 1) * kp] == list(range(start, start + kp))


def pin_packed_equals_per_document(o):
    """The packed result equals each document run alone, shifted by its token
    and pool offsets."""
    lens = [50, 21, 66]
    H, D, kp, topk = 2, 8, 4, 16
    q, k, gate, w, ape, cu = _tiny_case(500, lens, H, D, kp)
    pooled, cuP = o.compress(k, gate, ape, cu, kp)
    tok, pid = o.indexer_topk(q, w, pooled, cu, kp, topk, True)
    for b, L in enumerate(lens):
        s = int(cu[b])
        pb, _ = o.compress(k[s:s + L], gate[s:s + L], ape, [0, L], kp)
        tb, ib = o.indexer_topk(q[s:s + L], w[s:s + L], pb, [0, L], kp, topk, True)
        assert np.array_equal(np.where(tb >= 0, tb + s, -1), tok[s:s + L])
        assert np.array_equal(np.where(ib >= 0, ib + int(cuP[b]), -1), pid[s:s + L])


def pin_row_subsets(o):
    """Any subset of query rows gives the same rows as the full run."""
    lens = [80]
    q, k, gate, w, ape, cu = _tiny_case(600, lens, 2, 8, 4)
    pooled, _ = o.compress(k, gate, ape, cu, 4)
    tok, pid = o.indexer_topk(q, w, pooled, cu, 4, 16, True)
    rows = [79, 3, 40, 41, 0]
    t2, p2 = o.indexer_topk(q, w, pooled, cu, 4, 16, True, rows=rows)
    assert np.array_equal(t2, tok[rows]) and np.array_equal(p2, pid[rows])


def pin_positive_rescale(o):
    """Scaling w by c > 0 leaves the chosen pools unchanged."""
    lens = [120]
    q, k, gate, w, ape, cu = _tiny_case(700, lens, 4, 16, 4)
    pooled, _ = o.compress(k, gate, ape, cu, 4)
    _, p1 = o.indexer_topk(q, w, pooled, cu, 4, 32, True)
    _, p2 = o.indexer_topk(q, (w * F32(4.0)).astype(F32), pooled, cu, 4, 32, True)
    assert np.array_equal(p1, p2)


def pin_fp8_end_to_end_library(o):
    """FP8 path end to end against a route built from library routines: the
    explicit Sylvester matrix (scipy), torch's BF16 and float8_e4m3fn casts and
    the closed-form power-of-two exponent. Scores agree to 2e-3 relative and
    the chosen sets agree away from near-ties; the result also differs from the
    BF16 path (the quantisation is really applied)."""
    from scipy.linalg import hadamard
    lens = [300]
    H, D, kp, topk = 4, 128, 4, 32
    q, k, gate, w, ape, cu = _tiny_case(800, lens, H, D, kp)
    pooled, cuP = o.compress(k, gate, ape, cu, kp)
    Hm = torch.from_numpy(hadamard(128).astype(np.float32)) * np.float32(1.0 / math.sqrt(128.0))

    def lib_quant(x):
        y = (torch.from_numpy(np.ascontiguousarray(x, dtype=F32)) @ Hm.T).to(torch.bfloat16).float()
        amax = y.abs().amax(1)
        e = torch.where(amax > 0, torch.ceil(torch.log2(amax / 448.0)), torch.zeros_like(amax))
        s = torch.pow(2.0, e)[:, None]
        return ((y / s).to(torch.float8_e4m3fn).float() * s).numpy()

    keys = lib_quant(pooled)
    rows = list(range(0, 300, 7)) + [299]
    tok, pid, scores = o.indexer_topk(q, w, pooled, cu, kp, topk, True, rows=rows,
                                      fp8=True, return_scores=True)
    _, pid_bf16 = o.indexer_topk(q, w, pooled, cu, kp, topk, True, rows=rows)
    sc = np.float32(1.0 / math.sqrt(D))
    changed = 0
    for r, t in enumerate(rows):
        n_c = (t + 1) // kp
        qd = lib_quant(q[t])
        d = qd.astype(np.float64) @ keys[:n_c].T.astype(np.float64)
        ref = (w[t].astype(np.float64)[:, None] * np.maximum(0.0, sc * d)).sum(0)
        lim = 2e-3 * np.maximum(np.abs(ref), 0.01 * np.abs(ref).max(initial=0.0))
        assert np.all(np.abs(scores[r] - ref) <= lim + 1e-6), t
        got = set(int(x) for x in pid[r] if x >= 0)
        want = set(np.argsort(-ref, kind="stable")[:min(topk // kp, n_c)].tolist())
        if got != want:
            kth = np.sort(ref)[::-1][topk // kp - 1]
            for j in got ^ want:
                assert abs(ref[j] - kth) <= 1e-3 * abs(kth), (t, j)
        changed += int(not np.array_equal(pid[r], pid_bf16[r]))
    assert changed > 0


def pin_decode_is_last_token_row(o):
    """Serving: the decode row of a sequence of L tokens equals the prefill
    row of the last token of a document of L tokens, with the sequence's
    pools anywhere in a shared cache (pool ids offset by its start) and its
    token ids offset by its base; L = 0 gives a row of -1. Lengths cross
    every case: no pool, fewer pools than K_sel, more, ragged tails; kpool
    1, 3, 4; tail on and off."""
    H, D = 3, 8
    lens = [0, 1, 3, 4, 5, 37, 64, 90, 23]
    for kp in (1, 3, 4):
        for tail in (True, False):
            topk = 4 * kp
            B = len(lens)
            q_rows, w_rows, cache, starts, per_doc = [], [], [], [], []
            cursor = 5                                    # the cache starts with unrelated rows
            cache.append(rnd((5, D), 950).astype(F32))
            for b, L in enumerate(lens):
                q, k, gate, w, ape, cu = _tiny_case(900 + 10 * b + kp, [max(L, 1)], H, D, kp)
                pb, _ = o.compress(k[:L], gate[:L], ape, [0, L], kp)
                starts.append(cursor)
                cache.append(pb)
                cursor += len(pb)
                cache.append(rnd((2, D), 960 + b).astype(F32))   # a gap between sequences
                cursor += 2
                q_rows.append(q[max(L, 1) - 1])
                w_rows.append(w[max(L, 1) - 1])
                if L > 0:
                    tok, pid = o.indexer_topk(q[:L], w[:L], pb, [0, L], kp, topk, tail,
                                              rows=[L - 1])
                else:
                    tok = np.full((1, topk + kp), -1, np.int32)
                    pid = np.full((1, topk // kp), -1, np.int32)
                per_doc.append((tok[0], pid[0]))
            pooled = np.concatenate(cache).astype(F32)
            base = [1000 * b + 7 for b in range(B)]
            dtok, dpid = o.decode_topk(np.stack(q_rows), np.stack(w_rows), pooled, starts, lens,
                                       kp, topk, tail, token_base=base)
            for b in range(B):
                tok, pid = per_doc[b]
                assert np.array_equal(dtok[b], np.where(tok >= 0, tok + base[b], -1)), (kp, tail, b)
                assert np.array_equal(dpid[b], np.where(pid >= 0, pid + starts[b], -1)), (kp, tail, b)


def pin_decode_fp8_is_last_token_row(o):
    """The FP8 decode row (q and cached keys through the FP8 input path)
    equals the FP8 prefill row of the sequence's last token."""
    H, D, kp, topk = 2, 128, 4, 16
    lens = [0, 7, 40, 131]
    q_rows, w_rows, cache, starts, per_doc = [], [], [], [], []
    cursor = 0
    for b, L in enumerate(lens):
        q, k, gate, w, ape, cu = _tiny_case(970 + b, [max(L, 1)], H, D, kp)
        pb, _ = o.compress(k[:L], gate[:L], ape, [0, L], kp)
        starts.append(cursor)
        cache.append(pb)
        cursor += len(pb)
        q_rows.append(q[max(L, 1) - 1])
        w_rows.append(w[max(L, 1) - 1])
        if L > 0:
            tok, pid = o.indexer_topk(q[:L], w[:L], pb, [0, L], kp, topk, True, rows=[L - 1],
                                      fp8=True)
        else:
            tok = np.full((1, topk + kp), -1, np.int32)
            pid = np.full((1, topk // kp), -1, np.int32)
        per_doc.append((tok[0], pid[0]))
    pooled = np.concatenate(cache).astype(F32)
    dtok, dpid = o.decode_topk(np.stack(q_rows), np.stack(w_rows), pooled, starts, lens, kp,
                               topk, True, fp8=True)
    for b in range(len(lens)):
        tok, pid = per_doc[b]
        assert np.array_equal(dtok[b], tok), b
        assert np.array_equal(dpid[b], np.where(pid >= 0, pid + starts[b], -1)), b


# ---------------------------------------------------------------------------
# the indexer projections
# ---------------------------------------------------------------------------

def _proj_case(seed, T=24, hidden=192, qlr=96, H=4, D=32):
    g = torch.Generator().manual_seed(seed)
    bf = lambda *sh, s=1.0: (s * torch.randn(*sh, generator=g)).to(torch.bfloat16).float().numpy()
    x, qr = bf(T, hidden), bf(T, qlr)
    wq_b, wk, wg = bf(H * D, qlr, s=qlr ** -0.5), bf(D, hidden, s=hidden ** -0.5), bf(D, hidden, s=hidden ** -0.5)
    gamma = (1.0 + 0.1 * torch.randn(D, generator=g)).numpy().astype(np.float32)
    beta = (0.1 * torch.randn(D, generator=g)).numpy().astype(np.float32)
    ww = (hidden ** -0.5 * torch.randn(H, hidden, generator=g)).numpy().astype(np.float32)
    return x, qr, wq_b, wk, gamma, beta, wg, ww, H, D


def pin_linear_bf16_matches_library(o):
    """A BF16 linear layer: the FP64 product rounded to BF16 by torch, within
    one BF16 ulp (FP32 accumulation can cross a rounding boundary) plus the
    FP32 dot-product bound; most elements equal."""
    x, qr, wq_b, wk, gamma, beta, wg, ww, H, D = _proj_case(1)
    got = o.linear_bf16(x, wk)
    exact = torch.from_numpy(x).double() @ torch.from_numpy(wk).double().T
    ref = exact.to(torch.bfloat16).double().numpy()
    bound = 2 * x.shape[1] * 2.0 ** -24 * (np.abs(x) @ np.abs(wk).T)
    assert_within_bf16_ulps(got, ref, 1, bound)
    assert np.mean(got == ref) > 0.97


def pin_layer_norm_matches_library(o):
    """LayerNorm vs torch's layer_norm in FP64 (weight and bias), within FP32
    rounding; with weight 1 and bias 0 each row has mean 0 and variance
    var / (var + eps)."""
    g = torch.Generator().manual_seed(2)
    v = (3.0 * torch.randn(40, 64, generator=g) + 1.5).numpy().astype(np.float32)
    gamma = (1.0 + 0.2 * torch.randn(64, generator=g)).numpy().astype(np.float32)
    beta = (0.3 * torch.randn(64, generator=g)).numpy().astype(np.float32)
    got = o.layer_norm(v, gamma, beta, 1e-6)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(v).double(), (64,),
                                         torch.from_numpy(gamma).double(),
                                         torch.from_numpy(beta).double(), 1e-6).numpy()
    assert np.allclose(got, ref, rtol=1e-5, atol=1e-5)
    plain = o.layer_norm(v, np.ones(64, np.float32), np.zeros(64, np.float32), 1e-2)
    var = v.astype(np.float64).var(axis=1)
    assert np.allclose(plain.mean(axis=1), 0.0, atol=1e-5)
    assert np.allclose(plain.astype(np.float64).var(axis=1), var / (var + 1e-2), rtol=1e-4)
    # a constant row normalises to the bias exactly (the deviation is 0)
    const = o.layer_norm(np.full((1, 64), 7.25, np.float32), gamma, beta, 1e-6)
    assert np.array_equal(const[0], beta)


def pin_projections_onehot(o):
    """x = e_i: the gate is column i of wg, the head weights column i of ww
    (FP32, exact), k the LayerNorm of column i of wk (FP64 closed form, then
    BF16); q = e_j of the query latent gives column j of wq_b per head."""
    x, qr, wq_b, wk, gamma, beta, wg, ww, H, D = _proj_case(3)
    T, hidden = x.shape
    xs = np.zeros_like(x)
    xs[np.arange(T), np.arange(T) % hidden] = 1.0
    qs = np.zeros_like(qr)
    qs[np.arange(T), (3 * np.arange(T)) % qr.shape[1]] = 1.0
    q, k, gate, w = o.indexer_projections(xs, qs, wq_b, wk, gamma, beta, wg, ww, H, D)
    for t in range(T):
        i, j = t % hidden, (3 * t) % qr.shape[1]
        assert np.array_equal(gate[t], wg[:, i])
        assert np.array_equal(w[t], ww[:, i])
        col = wk[:, i].astype(np.float64)
        ln = (col - col.mean()) / np.sqrt(col.var() + 1e-6) * gamma + beta
        assert np.allclose(k[t], ln, rtol=2 ** -7, atol=1e-6)
        assert np.array_equal(q[t].reshape(-1), wq_b[:, j])
        assert np.array_equal(q[t, 1], wq_b[D:2 * D, j])


def pin_k_path_golden(o):
    """k = BF16(LayerNorm(BF16(x wk^T))): an FP64 evaluation of the same
    steps (the linear output rounded to BF16 before the norm) agrees on
    almost every element and within one BF16 ulp everywhere."""
    x, qr, wq_b, wk, gamma, beta, wg, ww, H, D = _proj_case(4, T=64)
    _, k, _, _ = o.indexer_projections(x, qr, wq_b, wk, gamma, beta, wg, ww, H, D)
    lin = (torch.from_numpy(x).double() @ torch.from_numpy(wk).double().T).to(torch.bfloat16).double()
    ln = torch.nn.functional.layer_norm(lin, (D,), torch.from_numpy(gamma).double(),
                                        torch.from_numpy(beta).double(), 1e-6)
    ref = ln.to(torch.bfloat16).double().numpy()
    assert_within_bf16_ulps(k, ref, 1)
    assert np.mean(k == ref) > 0.98


def pin_head_weights_fp32(o):
    """The head weights stay in FP32: FP64 product within the FP32
    dot-product bound, and not rounded to BF16."""
    x, qr, wq_b, wk, gamma, beta, wg, ww, H, D = _proj_case(5)
    _, _, _, w = o.indexer_projections(x, qr, wq_b, wk, gamma, beta, wg, ww, H, D)
    ref = x.astype(np.float64) @ ww.astype(np.float64).T
    bound = 2 * x.shape[1] * 2.0 ** -24 * (np.abs(x).astype(np.float64) @ np.abs(ww).T)
    assert np.all(np.abs(w - ref) <= bound)
    assert np.mean(o.bf16_round(w) != w) > 0.9


# ---------------------------------------------------------------------------
# Sparse attention of the NoPE absorbed MLA over the selected token rows
# (xtuner PR #2108, Summary: the FlashMLA forward consumes the int32 indices;
# the LSE fix commit: the saved LSE is the natural logarithm).
# ---------------------------------------------------------------------------

def _mla_case(seed, T=7, H=4, N=23, d=16, W=9):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, H, d))
    kv = r.standard_normal((N, d))
    idx = r.integers(0, N, size=(T, W))
    idx[r.random((T, W)) < 0.25] = -1
    return q, kv, idx


def _sdpa_rows(q_t, rows, sm_scale, d_v):
    """torch's scaled_dot_product_attention (FP64, CPU) of one query's heads
    over the given key/value rows; a library routine, not the oracle."""
    qt = torch.from_numpy(np.ascontiguousarray(q_t))[None, :, None, :]          # [1, H, 1, d]
    k = torch.from_numpy(np.ascontiguousarray(rows))[None, None].expand(1, q_t.shape[0], -1, -1)
    v = torch.from_numpy(np.ascontiguousarray(rows[:, :d_v]))[None, None].expand(1, q_t.shape[0], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, k, v, scale=sm_scale)
    return out[0, :, 0, :].numpy()


def pin_mla_matches_sdpa(o):
    """Each query equals torch's attention over the rows its valid entries
    list (repeats included), for d_v = d_qk and for d_v < d_qk (the value is
    the leading part of the latent row)."""
    for d_v in (16, 10):
        q, kv, idx = _mla_case(1)
        idx[2, :3] = idx[2, 3]                 # a row listed several times
        got, _ = o.sparse_mla_forward(q, kv, idx, 0.37, d_v=d_v)
        for t in range(q.shape[0]):
            sel = [int(j) for j in idx[t] if 0 <= j < kv.shape[0]]
            ref = _sdpa_rows(q[t], kv[sel], 0.37, d_v) if sel else np.zeros((q.shape[1], d_v))
            assert np.allclose(got[t], ref, rtol=1e-12, atol=1e-12)


def pin_mla_causal_dense(o):
    """Listing tokens 0..t (then -1 padding) for query t is causal attention
    over the whole sequence: torch's is_causal path, FP64."""
    T, H, d = 11, 3, 8
    r = np.random.default_rng(2)
    q = r.standard_normal((T, H, d))
    kv = r.standard_normal((T, d))
    idx = np.full((T, T), -1)
    for t in range(T):
        idx[t, :t + 1] = np.arange(t + 1)
    got, _ = o.sparse_mla_forward(q, kv, idx, 0.5)
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]                      # [1, H, T, d]
    k = torch.from_numpy(kv)[None, None].expand(1, H, T, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, k, k, is_causal=True, scale=0.5)
    assert np.allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def pin_mla_closed_forms(o):
    """One valid entry: o is that row, lse its score. q = 0: o is the mean of
    the listed rows (a repeat counts twice) and lse = ln n. No valid entry
    (-1 and out-of-range ids): o = 0, lse = -inf."""
    r = np.random.default_rng(3)
    N, H, d = 6, 2, 5
    kv = r.standard_normal((N, d))
    q = r.standard_normal((4, H, d))
    q[1] = 0.0
    q[3] = 0.0
    idx = np.array([[-1, 4, -1, 17],        # one valid entry (17 >= N is unused)
                    [0, 2, 2, 5],            # q = 0: weights 1, 2, 1 over rows 0, 2, 5
                    [-1, -1, -1, N],         # nothing valid
                    [3, 3, 3, 3]])           # q = 0, one row four times
    out, lse = o.sparse_mla_forward(q, kv, idx, 0.8)
    assert np.allclose(out[0], np.broadcast_to(kv[4], (H, d)), rtol=1e-14, atol=1e-14)
    assert np.allclose(lse[0], 0.8 * (q[0] @ kv[4]), rtol=1e-14, atol=1e-14)
    assert np.allclose(out[1], np.broadcast_to((kv[0] + 2 * kv[2] + kv[5]) / 4, (H, d)), atol=1e-14)
    assert np.allclose(lse[1], math.log(4.0), atol=1e-14)
    assert np.all(out[2] == 0.0) and np.all(np.isneginf(lse[2]))
    assert np.allclose(out[3], np.broadcast_to(kv[3], (H, d)), atol=1e-14)
    assert np.allclose(lse[3], math.log(4.0), atol=1e-14)


def pin_mla_lse_natural_log(o):
    """Two listed rows with scores a and b: lse = ln(e^a + e^b) (natural log,
    not log2), and o = sum_j exp(s_j - lse) v_j."""
    kv = np.array([[1.0, 0.0, 2.0], [0.0, 1.0, -1.0]])
    q = np.array([[[0.7, -0.3, 0.2]]])
    a, b = 0.9 * (0.7 + 0.4), 0.9 * (-0.3 - 0.2)
    out, lse = o.sparse_mla_forward(q, kv, np.array([[1, 0]]), 0.9)
    assert abs(lse[0, 0] - math.log(math.exp(a) + math.exp(b))) < 1e-14
    ref = math.exp(a - lse[0, 0]) * kv[0] + math.exp(b - lse[0, 0]) * kv[1]
    assert np.allclose(out[0, 0], ref, atol=1e-14)


def pin_mla_order_invariance(o):
    """Shuffling a query's entries, or moving its -1 padding, changes
    nothing beyond rounding (the softmax is a sum over the listed rows)."""
    q, kv, idx = _mla_case(4, W=12)
    ref_o, ref_l = o.sparse_mla_forward(q, kv, idx, 0.25)
    r = np.random.default_rng(5)
    shuf = np.stack([r.permutation(row) for row in idx])
    got_o, got_l = o.sparse_mla_forward(q, kv, shuf, 0.25)
    assert np.allclose(got_o, ref_o, rtol=1e-12, atol=1e-12)
    assert np.allclose(got_l, ref_l, rtol=1e-12, atol=1e-12)


def pin_mla_brute_loops(o):
    """Scalar loops with math.exp on a tiny case (no arrays, no library
    attention)."""
    q, kv, idx = _mla_case(6, T=3, H=2, N=5, d=3, W=4)
    out, lse = o.sparse_mla_forward(q, kv, idx, 1.3)
    for t in range(3):
        sel = [int(j) for j in idx[t] if 0 <= j < 5]
        for h in range(2):
            if not sel:
                assert lse[t, h] == -math.inf and all(out[t, h] == 0.0)
                continue
            s = [1.3 * sum(q[t, h, c] * kv[j, c] for c in range(3)) for j in sel]
            z = sum(math.exp(x) for x in s)
            assert abs(lse[t, h] - math.log(z)) < 1e-12
            for c in range(3):
                v = sum(math.exp(x) * kv[j, c] for x, j in zip(s, sel)) / z
                assert abs(out[t, h, c] - v) < 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
