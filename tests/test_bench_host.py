"""Host-side logic of bench.py (CPU only): the causal counts behind the
FLOP and byte figures of the bench line, the one-GPU guard and the lookup
of the committed logits traffic.

The counts follow the path's definitions: query i of a document (0-based)
has n_c = floor((i + 1) / kpool) causal pools, and a row needs selection
when n_c > K_sel. The closed form of the sum over a document of L = q kpool
+ r tokens is kpool q (q - 1) / 2 + q (r + 1)."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _closed_form_sum(L, kpool):
    q, r = divmod(L, kpool)
    return kpool * q * (q - 1) // 2 + q * (r + 1)


def _brute(doc_lengths, kpool, k_sel):
    tot = need = rows = 0
    for L in doc_lengths:
        for i in range(L):
            nc = (i + 1) // kpool
            tot += nc
            if nc > k_sel:
                need += nc
                rows += 1
    return tot, need, rows


@pytest.mark.parametrize("docs,kpool,k_sel", [
    ([256], 4, 16), ([4096], 4, 512), ([2641, 2501, 1405, 615], 4, 512),
    ([7, 1, 0, 13], 3, 1), ([100], 1, 10), ([5], 8, 2),
])
def test_causal_counts_brute_force(docs, kpool, k_sel):
    assert bench.causal_counts(docs, kpool, k_sel) == _brute(docs, kpool, k_sel)


@pytest.mark.parametrize("L,kpool,k_sel,rows", [
    (256, 4, 16, 189), (4096, 4, 512, 2045), (65536, 4, 512, 63485), (32768, 4, 512, 30717),
])
def test_causal_counts_closed_forms(L, kpool, k_sel, rows):
    tot, need, got_rows = bench.causal_counts([L], kpool, k_sel)
    assert tot == _closed_form_sum(L, kpool)
    # rows needing selection: i + 1 >= kpool (K_sel + 1)
    assert got_rows == rows == max(0, L - kpool * (k_sel + 1) + 1)
    # the rows left out hold n_c = 0 .. K_sel, each value kpool times (the
    # last run may be cut short by the document's end)
    i = np.arange(L)
    nc = (i + 1) // kpool
    assert need == tot - int(nc[nc <= k_sel].sum())


def test_64k_flops_figure():
    """The 64K workload's scoring FLOPs, 2 H D over the causal pairs of the
    rows that need selection (the rows whose pools are all chosen are not
    scored)."""
    tot, need, rows = bench.causal_counts([65536], 4, 512)
    assert tot == 536_854_528
    assert 2 * 32 * 128 * need == 4_393_608_937_472


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_logits_traffic_lookup():
    assert bench.logits_traffic("no_such_workload") is None
    digest = bench.logits_source_digest()
    assert len(digest) == 64 and int(digest, 16) >= 0
