"""The indexer's launches one at a time (kpool_indexer_launches,
kpool_indexer_scoring, kpool_indexer_selection) on the GPU:
  * scoring then selection of every launch, in reverse launch order, writes
    exactly what kpool_indexer_topk writes (token rows and pool ids);
  * a launch that scores two chunks (a long one, then a short one at its own
    row stride) writes, for every row that needs a selection, the same FP32
    scores bit for bit as kpool_logits over that chunk alone.
The scores themselves are checked against the oracle in test_gpu_parity.py;
the selection here is the same kernel on the same scores."""
import numpy as np
import pytest
import torch

import workloads as wlm
from gpu_common import DEV, Dev, log, params_for

import sparse_attention_indexer_kpool_amd as kp

pytestmark = pytest.mark.gpu

CASES = [
    # many chunks of uneven causal width: several two-chunk launches, a ragged last chunk
    wlm.custom("docs_qc1500_h32", doc_lengths=[9000, 3, 4100, 2600], H=32, D=128, kpool=4,
               index_topk=256, query_chunk=1500),
    wlm.custom("one_doc_qc1024_h16_k2", doc_lengths=[7000], H=16, D=128, kpool=2,
               index_topk=512, query_chunk=1024, tail=False),
    wlm.custom("fp8_qc2048_h32", doc_lengths=[11000, 1500], H=32, D=128, kpool=4,
               index_topk=512, query_chunk=2048, fp8=True),
    wlm.custom("docs_qc700_h64_d64", doc_lengths=[3000, 2000, 17], H=64, D=64, kpool=4,
               index_topk=128, query_chunk=700),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kp.lib()


_cache = {}


def dev(wl):
    if wl.name not in _cache:
        log(f"inputs {wl.name}")
        d = Dev(wlm.make_inputs(wl))
        d.compress()
        _cache[wl.name] = d
    return _cache[wl.name]


@pytest.mark.parametrize("wl", CASES + [2, 4], ids=lambda w: w if isinstance(w, int) else w.name)
def test_staged_launches_equal_indexer(wl):
    d = dev(wlm.workload(wl) if isinstance(wl, int) else wl)
    p, T = d.p, d.inp.T
    launches = kp.kpool_indexer_launches(p)
    log(f"{d.inp.wl.name}: {len(launches)} launches, "
        f"{sum(1 for x in launches if x[4] > x[3])} with two chunks")
    ref_tok, ref_pid = d.indexer()
    ws = d.workspace()
    tok = torch.full((T, p.width), -12345, dtype=torch.int32, device=DEV)
    pid = torch.full((T, p.k_sel), -12345, dtype=torch.int32, device=DEV)
    for i in reversed(range(len(launches))):
        kp.kpool_indexer_scoring(p, i, d.q, d.w, d.pooled, d.cu, d.cu_pools, ws)
        kp.kpool_indexer_selection(p, i, d.cu, d.cu_pools, ws, tok, pid)
    torch.cuda.synchronize()
    assert np.array_equal(tok.cpu().numpy(), ref_tok)
    assert np.array_equal(pid.cpu().numpy(), ref_pid)


def _n_c(inp, rows):
    cu = inp.cu_seqlens.numpy().astype(np.int64)
    b = np.searchsorted(cu, rows, side="right") - 1
    return (rows - cu[b] + 1) // inp.wl.kpool


def _tile_offset(p, T):
    """Byte offset of the logits tile in the workspace: after the FP8 codes
    and row scales of q and of the pooled keys (each piece 256-byte aligned)
    on the FP8 path, at 0 otherwise (the layout include/kpool.h states)."""
    if not p.use_fp8:
        return 0
    up = lambda x: (x + 255) // 256 * 256
    qrows, krows = T * p.num_heads, T // p.kpool
    return up(up(up(up(qrows * 128) + qrows * 4) + krows * 128) + krows * 4)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_two_chunk_launch_scores_match_single_chunk(wl):
    d = dev(wl)
    p, inp = d.p, d.inp
    launches = kp.kpool_indexer_launches(p)
    two = [i for i, x in enumerate(launches) if x[4] > x[3]]
    assert two, "the case must have a launch of two chunks"
    ws = d.workspace()
    for i in two:
        a0, a1, lda, b0, b1, ldb = launches[i]
        off0 = _tile_offset(p, inp.T)
        ws[off0:].fill_(0x7F)
        kp.kpool_indexer_scoring(p, i, d.q, d.w, d.pooled, d.cu, d.cu_pools, ws)
        torch.cuda.synchronize()
        tile = ws[off0:].view(torch.float32)
        for (r0, r1, ld, off) in ((a0, a1, lda, 0), (b0, b1, ldb, (a1 - a0) * lda)):
            got = tile[off:off + (r1 - r0) * ld].view(r1 - r0, ld).cpu().numpy()
            ref = d.logits(r0, r1).cpu().numpy()
            rows = np.arange(r0, r1)
            nc = _n_c(inp, rows)
            assert nc.max() <= ld
            for r in np.nonzero(nc > p.k_sel)[0]:
                n = int(nc[r])
                assert np.array_equal(got[r, :n].view(np.int32), ref[r, :n].view(np.int32)), \
                    f"launch {i}: row {r0 + r}"
        log(f"{wl.name}: launch {i} rows [{a0},{a1}) ld {lda} + [{b0},{b1}) ld {ldb} match")
