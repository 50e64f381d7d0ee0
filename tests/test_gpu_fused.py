"""kpool_indexer_topk_fused against kpool_indexer_topk, through the C ABI.

The fused entry point scores and selects in one kernel: while the pools
stream past, each workgroup keeps a running top-K_sel of every query's scores
in LDS, so no score is written. kpool_indexer_topk writes a logits tile per
query chunk (the scoring kernel of kpool_logits) and then selects and expands
it (the kernel of kpool_select_expand); both stages are held to the oracle
elsewhere. Both paths compute every score with the same arithmetic and
select exactly (larger score first, equal scores to the lower pool, NaN as
-inf), so their token rows and pool ids must agree bit for bit: on the
workloads, and on inputs built to stress the running selection: all-equal
scores, NaN and infinite scores, K_sel at the largest the candidate list
takes (frequent shrinks, the final unit of a row right after a shrink
request), every head count, BF16 and FP8.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wlm
from gpu_common import DEV, Dev, log, oracle_inputs, sets_match_up_to_ties

import sparse_attention_indexer_kpool_amd as kp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kp.lib()


def _fused(d, p):
    T = d.inp.T
    n = kp.kpool_fused_workspace_bytes(p)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=DEV) if n else None
    tok = torch.full((T, p.width), -12345, dtype=torch.int32, device=DEV)
    pid = torch.full((T, p.k_sel), -12345, dtype=torch.int32, device=DEV)
    kp.kpool_indexer_topk_fused(p, d.q, d.w, d.pooled, d.cu, d.cu_pools, ws, tok, pid)
    torch.cuda.synchronize()
    return tok, pid


def _tile_path(d, p):
    """kpool_indexer_topk: the logits tile per query chunk, then selection +
    expansion of each tile."""
    T = d.inp.T
    ws = torch.empty(max(kp.kpool_workspace_bytes(p), 256), dtype=torch.uint8, device=DEV)
    tok = torch.full((T, p.width), -777, dtype=torch.int32, device=DEV)
    pid = torch.full((T, p.k_sel), -777, dtype=torch.int32, device=DEV)
    kp.kpool_indexer_topk(p, d.q, d.w, d.pooled, d.cu, d.cu_pools, ws, tok, pid)
    torch.cuda.synchronize()
    return tok, pid


def _compare(d, p):
    assert p.k_sel <= kp.kpool_fused_max_ksel(p)
    tf, pf = _fused(d, p)
    tt, pt = _tile_path(d, p)
    if not torch.equal(pf, pt):
        bad = (pf != pt).any(dim=1).nonzero().flatten()[:5].tolist()
        raise AssertionError(f"pool ids differ on rows {bad}")
    assert torch.equal(tf, tt), "token rows differ"
    return tf, pf


_cache = {}


def _dev(wl):
    if wl.name not in _cache:
        log(f"inputs {wl.name}")
        d = Dev(wlm.make_inputs(wl))
        d.compress()
        _cache.clear()
        _cache[wl.name] = d
    return _cache[wl.name]


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_fused_equals_tile_path_workloads(idx):
    wl = wlm.workload(idx)
    d = _dev(wl)
    log(f"fused vs tile path {wl.name}")
    _compare(d, d.p)


def _largest_fused_topk(fields):
    """index_topk with the largest K_sel the fused kernel takes."""
    p = kp.Params(num_docs=1, total_tokens=1, max_seqlen=1, num_heads=fields["H"],
                  head_dim=fields["D"], use_fp8=int(fields.get("fp8", False)))
    ksel = kp.kpool_fused_max_ksel(p)
    assert ksel > 0
    return ksel * fields["kpool"]


SHAPES = [
    # (name, fields): K_sel at the largest the candidate list takes for each
    # head count, many pools per row, so the lists shrink every step or two
    ("h32_d128_k4", dict(T=16384, H=32, D=128, kpool=4)),
    ("h16_d128_k1", dict(T=8192, H=16, D=128, kpool=1)),
    ("h64_d64_k2", dict(T=8192, H=64, D=64, kpool=2)),
    ("h8_d128_k4_notail", dict(T=8192, H=8, D=128, kpool=4, tail=False)),
    ("h4_d64_k4", dict(T=8192, H=4, D=64, kpool=4)),
    ("h32_fp8_k4", dict(T=16384, H=32, D=128, kpool=4, fp8=True, heavy_frac=0.05)),
    ("h32_d128_k3_docs", dict(doc_lengths=[5000, 1, 0, 3001, 7, 2048 * 3 + 2], H=32, D=128,
                              kpool=3)),
]


@pytest.mark.parametrize("name,fields", SHAPES, ids=[s[0] for s in SHAPES])
def test_fused_equals_tile_path_at_list_capacity(name, fields):
    topk = _largest_fused_topk(fields)
    wl = wlm.custom(name, index_topk=topk, **fields)
    d = _dev(wl)
    log(f"fused vs tile path {name}: K_sel {topk // fields['kpool']}")
    _compare(d, d.p)
    # one more pool per row is beyond the list: refused, nothing written
    p2 = kp.Params(**{**d.p.__dict__, "index_topk": topk + fields["kpool"]})
    tok = torch.full((d.inp.T, p2.width), -5, dtype=torch.int32, device=DEV)
    with pytest.raises(kp.KPoolError) as e:
        kp.kpool_indexer_topk_fused(p2, d.q, d.w, d.pooled, d.cu, d.cu_pools, None, tok)
    assert e.value.status == kp.KPOOL_E_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((tok == -5).all())


def test_fused_ties_nan_inf():
    """All-equal scores (q rows of zeros: every score is +-0, so the lowest
    pools win), NaN and infinite scores (infinite q entries), zero head
    weights, on 8192 tokens at K_sel 512."""
    wl = wlm.custom("ties_nan_inf", T=8192, H=32, D=128, kpool=4, index_topk=2048)
    inp = wlm.make_inputs(wl)
    g = torch.Generator().manual_seed(3)
    rows = torch.randperm(8192 - 2100, generator=g)[:300] + 2100
    zero_rows, inf_rows, w0_rows = rows[:100], rows[100:200], rows[200:]
    inp.q[zero_rows] = 0
    q = inp.q.float()
    q[inf_rows, :, 5] = float("inf")
    q[inf_rows[::2], 3, 9] = float("-inf")
    inp.q = q.to(torch.bfloat16)
    inp.w[w0_rows] = 0.0
    d = Dev(inp)
    d.compress()
    tok, pid = _compare(d, d.p)
    pid = pid.cpu().numpy()
    for t in zero_rows.tolist()[:10]:
        assert np.array_equal(pid[t], np.arange(512)), f"row {t}: ties go to the lowest pools"


@pytest.mark.parametrize("idx,n", [(0, 256), (1, 192), (2, 192), (3, 96), (4, 64)])
def test_fused_end_to_end_against_oracle(idx, n):
    """The fused entry point against the oracle directly (oracle scores from
    the GPU's pooled keys): pool sets equal except pools within 1e-3 of the
    k-th score, token rows equal the oracle's expansion of the GPU's ids."""
    wl = wlm.workload(idx)
    d = _dev(wl)
    p = d.p
    tok, pid = _fused(d, p)
    tok, pid = tok.cpu().numpy(), pid.cpu().numpy()
    q, _, _, w, _, cu = oracle_inputs(d.inp)
    pooled = d.pooled.float().cpu().numpy()
    cuP = oracle.cu_pools_of(cu, p.kpool)
    rows = sorted(set(wlm.strided_rows(d.inp.T, n)) | {max(c - 1, 0) for c in cu[1:].tolist()})
    rows = [r for r in rows if r < d.inp.T]
    _, opid, osc = oracle.indexer_topk(q, w, pooled[:int(cuP[-1])], cu, p.kpool, p.index_topk,
                                       bool(p.always_select_tail), rows=rows,
                                       fp8=bool(wl.fp8), return_scores=True)
    exact = 0
    for r, t in enumerate(rows):
        b = oracle.doc_of(t, cu)
        okk, why = sets_match_up_to_ties(pid[t], opid[r], osc[r], int(cuP[b]), p.k_sel)
        assert okk, f"row {t}: {why}"
        exact += int(np.array_equal(pid[t], opid[r]))
        gids = [x for x in pid[t] if x >= 0]
        assert gids == sorted(gids)
        assert np.array_equal(tok[t], oracle.expand_row(t, cu, cuP, gids, p.kpool, p.index_topk,
                                                        bool(p.always_select_tail))), f"row {t}"
    log(f"  fused {wl.name}: {exact}/{len(rows)} rows identical to the oracle's pool set")
