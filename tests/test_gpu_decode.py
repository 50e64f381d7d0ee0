"""GPU parity of the serving entry points, through the C ABI, against the CPU
oracle on the same seeded inputs:
  compress_pools  pooled rows of pools given by their slot tokens, written to
                  scattered cache rows: within 1 BF16 ulp (plus the FP32
                  cancellation floor) of oracle.compress of the same slot
                  tokens, and bit-identical to the rows kpool_compress writes
                  for them; rows outside the cache are skipped
  decode_topk     pool sets vs the oracle's decode rows (oracle scores from the
                  same cached keys): equal except pools within 1e-3 relative of
                  the k-th score; token rows equal the oracle's expansion of the
                  GPU's pool ids exactly; the last token of every document of a
                  packed batch gets the prefill indexer's row
  FP8 cache       compress_pools codes and scales bit-identical to the
                  oracle's FP8 input path (oracle.fp8_quantize_rows) applied to
                  the BF16 pooled rows of the same pools, and, on every pool
                  whose BF16 row equals the oracle's, to the oracle's whole chain
                  (oracle.compress, then oracle.fp8_quantize_rows); FP8 decode vs the
                  oracle's FP8 decode (q and keys through the oracle's own FP8
                  input path) and vs the FP8 prefill row of each last token
"""
import numpy as np
import pytest
import torch

import oracle
import pins
import workloads as wlm
from gpu_common import DEV, Dev, log, oracle_inputs, sets_match_up_to_ties

import sparse_attention_indexer_kpool_amd as kp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kp.lib()


def _dparams(lens, H, D, kpool, topk, tail=True, fp8=False):
    return kp.Params(num_docs=len(lens), total_tokens=0, max_seqlen=max(max(lens), 0),
                     num_heads=H, head_dim=D, kpool=kpool, index_topk=topk,
                     always_select_tail=int(tail), use_fp8=int(fp8))


def _fp8_cache(pooled_bf16_dev):
    """E4M3 codes and scales of BF16 cache rows, by the library's quantiser
    (its codes are checked bit for bit against the oracle elsewhere)."""
    rows = pooled_bf16_dev.shape[0]
    codes = torch.empty(rows, 128, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, dtype=torch.float32, device=DEV)
    kp.kpool_fp8_quantize(pooled_bf16_dev.contiguous(), rows, codes, scales)
    return codes, scales


def _run_decode(p, di, pooled_dev=None, pooled_scale=None):
    ws = torch.empty(max(kp.kpool_decode_workspace_bytes(p), 256), dtype=torch.uint8, device=DEV)
    tok = torch.full((di.B, p.width), -12345, dtype=torch.int32, device=DEV)
    pid = torch.full((di.B, p.k_sel), -12345, dtype=torch.int32, device=DEV)
    if pooled_dev is None:
        pooled_dev = di.pooled.to(DEV)
    kp.kpool_decode_topk(p, di.q.to(DEV), di.w.to(DEV), pooled_dev,
                         di.pool_start.to(DEV), di.seq_lens.to(DEV), ws, tok, pid,
                         token_base=di.token_base.to(DEV), pooled_scale=pooled_scale)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), pid.cpu().numpy()


def _check_decode(p, di, tok, pid, fp8=False):
    q = di.q.float().numpy()
    w = di.w.numpy()
    pooled = di.pooled.float().numpy()
    sc = float(np.float32(1.0 / np.sqrt(p.head_dim)))
    exact = 0
    for b in range(di.B):
        L = int(di.seq_lens[b])
        s0 = int(di.pool_start[b])
        base = int(di.token_base[b])
        if L == 0:
            assert np.all(tok[b] == -1) and np.all(pid[b] == -1), b
            continue
        n_c = L // p.kpool
        keys, q_b = pooled[s0:s0 + n_c], q[b]
        if fp8:
            _, _, keys = oracle.fp8_quantize_rows(keys)
            _, _, q_b = oracle.fp8_quantize_rows(q_b)
        scores = oracle.row_scores(q_b, w[b], keys, sc)
        ref_local = oracle.select_pools(scores, p.k_sel)
        ref = np.full(p.k_sel, -1, np.int64)
        ref[:len(ref_local)] = ref_local + s0
        okk, why = sets_match_up_to_ties(pid[b], ref, scores, s0, p.k_sel)
        assert okk, f"sequence {b} (L = {L}): {why}"
        exact += int(np.array_equal(pid[b], ref))
        gids = [int(x) for x in pid[b] if x >= 0]
        assert gids == sorted(gids)
        row = oracle.expand_row(L - 1, [0, L], [0, n_c], [g - s0 for g in gids], p.kpool,
                                p.index_topk, bool(p.always_select_tail))
        assert np.array_equal(tok[b], np.where(row >= 0, row + base, -1)), f"sequence {b}"
    log(f"  {exact}/{di.B} rows identical to the oracle's pool set")


@pytest.mark.parametrize("lens,H,D,kpool,topk,tail", [
    ([0, 1, 3, 4, 2047, 2048, 2051, 4098, 9000, 20001, 65536], 32, 128, 4, 2048, True),
    ([0, 2, 3, 300, 301, 902, 5000, 12345], 4, 64, 3, 300, False),
    ([1, 63, 64, 65, 1000, 4096], 64, 128, 1, 64, True),
    ([17, 130, 131, 1024, 3000], 8, 128, 2, 256, True),
    ([2044, 2048, 2055, 4096, 4100, 8191], 16, 64, 4, 512, True),
    ([40, 4095, 4096, 4103], 32, 128, 8, 1024, True),
], ids=["h32_k4", "h4_d64_k3_notail", "h64_k1", "h8_k2", "h16_d64_piece_edges", "k8"])
def test_decode_matches_oracle(lens, H, D, kpool, topk, tail):
    p = _dparams(lens, H, D, kpool, topk, tail)
    di = wlm.make_decode_inputs(lens, H, D, kpool, seed=len(lens) + H + kpool)
    log(f"decode {len(lens)} sequences, H {H} D {D} kpool {kpool} topk {topk}")
    tok, pid = _run_decode(p, di)
    _check_decode(p, di, tok, pid)


def test_decode_64_sequences_at_64k():
    """The serving shape of the benchmark: 64 sequences of 64K tokens
    (16384 cached pools each), sampled rows checked against the oracle."""
    lens = [65536 - 37 * b for b in range(64)]
    p = _dparams(lens, 32, 128, 4, 2048)
    di = wlm.make_decode_inputs(lens, 32, 128, 4, seed=64)
    tok, pid = _run_decode(p, di)
    pick = [0, 1, 17, 40, 63]
    sub = wlm.DecodeInputs(q=di.q[pick], w=di.w[pick], pooled=di.pooled,
                           pool_start=di.pool_start[pick], seq_lens=di.seq_lens[pick],
                           token_base=di.token_base[pick], kpool=4)
    _check_decode(p, sub, tok[pick], pid[pick])


def test_decode_is_prefill_last_token_row():
    """Decode over the pooled keys kpool_compress wrote for a packed batch
    (pool_start = the documents' pool offsets, token_base = their first
    tokens) gives, for each document's last token, the prefill indexer's pool
    set (up to near-ties: the two kernels sum in different orders) and, where
    the sets agree, its token row."""
    d = Dev(wlm.make_inputs(wlm.workload(2)))
    d.compress()
    tok_pf, pid_pf = d.indexer()
    inp = d.inp
    cu = inp.cu_seqlens.numpy().astype(np.int64)
    cuP = d.cu_pools.cpu().numpy().astype(np.int64)
    B = len(inp.doc_lengths)
    last = [int(cu[b + 1]) - 1 for b in range(B)]
    lens = list(inp.doc_lengths)
    di = wlm.DecodeInputs(q=inp.q[last].contiguous(), w=inp.w[last].contiguous(),
                          pooled=d.pooled.cpu(), pool_start=torch.tensor(cuP[:B], dtype=torch.int32),
                          seq_lens=torch.tensor(lens, dtype=torch.int32),
                          token_base=torch.tensor(cu[:B], dtype=torch.int32), kpool=inp.wl.kpool)
    p = _dparams(lens, inp.wl.H, inp.wl.D, inp.wl.kpool, inp.wl.index_topk)
    tok, pid = _run_decode(p, di)
    q, _, _, w, _, _ = oracle_inputs(inp)
    pooled = d.pooled.float().cpu().numpy()
    sc = float(np.float32(1.0 / np.sqrt(inp.wl.D)))
    for b, t in enumerate(last):
        n_c = lens[b] // inp.wl.kpool
        scores = oracle.row_scores(q[t], w[t], pooled[cuP[b]:cuP[b] + n_c], sc)
        okk, why = sets_match_up_to_ties(pid[b], pid_pf[t], scores, int(cuP[b]), p.k_sel)
        assert okk, f"document {b}: {why}"
        if np.array_equal(pid[b], pid_pf[t]):
            assert np.array_equal(tok[b], tok_pf[t]), f"document {b}"


@pytest.mark.parametrize("kpool,D", [(4, 128), (3, 64), (1, 128), (8, 64)])
def test_compress_pools_matches_compress(kpool, D):
    wl = wlm.custom("pools", T=1000, H=4, D=D, kpool=kpool, index_topk=64)
    d = Dev(wlm.make_inputs(wl))
    pooled_ref, _ = d.compress()
    P = pooled_ref.shape[0]
    g = torch.Generator().manual_seed(kpool * 100 + D)
    pick = torch.randperm(P, generator=g)[: P // 2]
    N = len(pick)
    cap = P + 10
    dst = torch.randperm(cap, generator=g)[:N].to(torch.int32)
    dst[3] = -1                                # skipped
    dst[7] = cap                               # skipped
    tok_idx = (pick[:, None] * kpool + torch.arange(kpool)[None, :]).reshape(-1)
    k_slots = d.inp.k[tok_idx].contiguous().to(DEV)
    g_slots = d.inp.gate[tok_idx].contiguous().to(DEV)
    cache = torch.full((cap, D), 0x7F7F, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    p = kp.Params(num_docs=1, total_tokens=1000, max_seqlen=1000, num_heads=4, head_dim=D,
                  kpool=kpool, index_topk=64)
    kp.kpool_compress_pools(p, k_slots, g_slots, d.ape, N, dst.to(DEV), cache)
    torch.cuda.synchronize()
    got = cache.view(torch.int16).cpu().numpy()
    ref_bits = d.pooled.view(torch.int16).cpu().numpy()
    # the oracle on the same slot tokens: one document of N * kpool tokens
    ks_np, gs_np = d.inp.k[tok_idx].float().numpy(), d.inp.gate[tok_idx].float().numpy()
    ape_np = d.inp.ape.numpy()
    cu1 = np.array([0, N * kpool], np.int64)
    ref_orc, _ = oracle.compress(ks_np, gs_np, ape_np, cu1, kpool)
    floor = pins.pooled_fp32_floor(ks_np, gs_np, ape_np, cu1, kpool)
    ok_rows = [n for n in range(N) if 0 <= int(dst[n]) < cap]
    got_rows = cache[dst[ok_rows].long().to(DEV)].float().cpu().numpy()
    pins.assert_within_bf16_ulps(got_rows, ref_orc[ok_rows], 1, floor[ok_rows])
    written = set()
    for n in ok_rows:
        r = int(dst[n])
        assert np.array_equal(got[r], ref_bits[int(pick[n])]), n
        written.add(r)
    untouched = [r for r in range(cap) if r not in written]
    assert np.all(got[untouched] == 0x7F7F)


@pytest.mark.parametrize("lens,H,kpool,topk", [
    ([0, 1, 5, 2047, 2051, 9000, 65536], 32, 4, 2048),
    ([3, 300, 4097], 4, 3, 300),
    ([64, 65, 2000], 64, 1, 64),
], ids=["h32_k4", "h4_k3", "h64_k1"])
def test_decode_fp8_matches_oracle(lens, H, kpool, topk):
    p = _dparams(lens, H, 128, kpool, topk, fp8=True)
    di = wlm.make_decode_inputs(lens, H, 128, kpool, seed=17 + H)
    codes, scales = _fp8_cache(di.pooled.to(DEV))
    log(f"decode fp8 {len(lens)} sequences, H {H} kpool {kpool} topk {topk}")
    tok, pid = _run_decode(p, di, codes, scales)
    _check_decode(p, di, tok, pid, fp8=True)


def test_decode_fp8_is_prefill_last_token_row():
    """FP8 decode over the codes of the pooled keys kpool_compress wrote for
    a packed batch gives each document's last token the FP8 prefill row (up
    to near-ties)."""
    wl = wlm.custom("fp8_docs", doc_lengths=[700, 1300, 2501], H=32, D=128, kpool=4,
                    index_topk=512, fp8=True, heavy_frac=0.05)
    d = Dev(wlm.make_inputs(wl))
    d.compress()
    tok_pf, pid_pf = d.indexer()
    inp = d.inp
    cu = inp.cu_seqlens.numpy().astype(np.int64)
    cuP = d.cu_pools.cpu().numpy().astype(np.int64)
    B = len(inp.doc_lengths)
    last = [int(cu[b + 1]) - 1 for b in range(B)]
    lens = list(inp.doc_lengths)
    P = int(cuP[B])
    codes, scales = _fp8_cache(d.pooled[:P])
    di = wlm.DecodeInputs(q=inp.q[last].contiguous(), w=inp.w[last].contiguous(),
                          pooled=d.pooled[:P].cpu(), pool_start=torch.tensor(cuP[:B], dtype=torch.int32),
                          seq_lens=torch.tensor(lens, dtype=torch.int32),
                          token_base=torch.tensor(cu[:B], dtype=torch.int32), kpool=4)
    p = _dparams(lens, 32, 128, 4, 512, fp8=True)
    tok, pid = _run_decode(p, di, codes, scales)
    q, _, _, w, _, _ = oracle_inputs(inp)
    _, _, keys_all = oracle.fp8_quantize_rows(d.pooled[:P].float().cpu().numpy())
    sc = float(np.float32(1.0 / np.sqrt(128)))
    for b, t in enumerate(last):
        n_c = lens[b] // 4
        _, _, q_t = oracle.fp8_quantize_rows(q[t])
        scores = oracle.row_scores(q_t, w[t], keys_all[cuP[b]:cuP[b] + n_c], sc)
        okk, why = sets_match_up_to_ties(pid[b], pid_pf[t], scores, int(cuP[b]), p.k_sel)
        assert okk, f"document {b}: {why}"
        if np.array_equal(pid[b], pid_pf[t]):
            assert np.array_equal(tok[b], tok_pf[t]), f"document {b}"


@pytest.mark.parametrize("kpool", [4, 3])
def test_compress_pools_fp8_matches_quantised_compress(kpool):
    wl = wlm.custom("pools8", T=1200, H=4, D=128, kpool=kpool, index_topk=64)
    d = Dev(wlm.make_inputs(wl))
    d.compress()
    P = int(d.cu_pools[-1].item())
    ref_codes, ref_scales = _fp8_cache(d.pooled[:P])
    g = torch.Generator().manual_seed(kpool)
    pick = torch.randperm(P, generator=g)[: P // 2]
    N = len(pick)
    cap = P + 7
    dst = torch.randperm(cap, generator=g)[:N].to(torch.int32)
    dst[1] = cap                               # skipped
    tok_idx = (pick[:, None] * kpool + torch.arange(kpool)[None, :]).reshape(-1)
    k_slots = d.inp.k[tok_idx].contiguous().to(DEV)
    g_slots = d.inp.gate[tok_idx].contiguous().to(DEV)
    codes = torch.full((cap, 128), 0xA5, dtype=torch.uint8, device=DEV)
    scales = torch.full((cap,), -3.0, dtype=torch.float32, device=DEV)
    p = kp.Params(num_docs=1, total_tokens=1200, max_seqlen=1200, num_heads=4, head_dim=128,
                  kpool=kpool, index_topk=64, use_fp8=1)
    kp.kpool_compress_pools(p, k_slots, g_slots, d.ape, N, dst.to(DEV), codes, pooled_scale=scales)
    # the same pools in BF16, through the same entry point
    bf_p = kp.Params(num_docs=1, total_tokens=1200, max_seqlen=1200, num_heads=4, head_dim=128,
                     kpool=kpool, index_topk=64, use_fp8=0)
    bf_cache = torch.zeros((cap, 128), dtype=torch.bfloat16, device=DEV)
    kp.kpool_compress_pools(bf_p, k_slots, g_slots, d.ape, N, dst.to(DEV), bf_cache)
    torch.cuda.synchronize()
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    rc, rs = ref_codes.cpu().numpy(), ref_scales.cpu().numpy()
    ok_rows = [n for n in range(N) if 0 <= int(dst[n]) < cap]
    rows_ok = dst[ok_rows].long()
    # (1) the oracle's FP8 input path on the BF16 pooled rows of the same pools
    gpu_bf = bf_cache[rows_ok.to(DEV)].float().cpu().numpy()
    o_codes, o_exps, _ = oracle.fp8_quantize_rows(gpu_bf)
    assert np.array_equal(got_c[rows_ok.numpy()], o_codes)
    assert np.array_equal(got_s[rows_ok.numpy()], np.ldexp(1.0, o_exps).astype(np.float32))
    # (2) the oracle's whole chain (compress, then the FP8 input path) on
    # every pool whose BF16 row equals the oracle's
    ks_np, gs_np = d.inp.k[tok_idx].float().numpy(), d.inp.gate[tok_idx].float().numpy()
    orc_bf, _ = oracle.compress(ks_np, gs_np, d.inp.ape.numpy(), np.array([0, N * kpool]), kpool)
    orc_bf = orc_bf[ok_rows]
    same = np.all(orc_bf == gpu_bf, axis=1)
    c2, e2, _ = oracle.fp8_quantize_rows(orc_bf[same])
    assert np.array_equal(got_c[rows_ok.numpy()[same]], c2)
    assert np.array_equal(got_s[rows_ok.numpy()[same]], np.ldexp(1.0, e2).astype(np.float32))
    log(f"  FP8 cache rows: {int(same.sum())}/{len(ok_rows)} pools through the oracle's whole chain")
    assert same.mean() > 0.5
    written = set()
    for n in ok_rows:
        r = int(dst[n])
        assert np.array_equal(got_c[r], rc[int(pick[n])]), n
        assert got_s[r] == rs[int(pick[n])], n
        written.add(r)
    untouched = [r for r in range(cap) if r not in written]
    assert np.all(got_c[untouched] == 0xA5) and np.all(got_s[untouched] == -3.0)

