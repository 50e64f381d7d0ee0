"""GPU parity of the indexer projections (kpool_indexer_projections) through
the C ABI, against the oracle on the same seeded inputs:
  q, gate  BF16 linear layers: within 1 BF16 ulp plus the FP32 dot-product
           bound 2 K 2^-24 sum |a b| (both sides accumulate in FP32, in
           different orders, and may round across a BF16 boundary)
  w        FP32: within 2 hidden 2^-24 sum |x w| (the GPU's products of the
           exact three-way BF16 split of w are exact; its FP32 sums differ in
           order from the oracle's)
  k        LayerNorm of the BF16 linear output: within 1 BF16 ulp plus
           |k_norm_weight| * 3 delta / sigma per row, delta the largest
           linear-output difference the two sides can have (1 BF16 ulp plus
           the dot-product bound), sigma the row's standard deviation
Small shapes are checked on every row; the bench shape on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import pins
import workloads as wlm
from gpu_common import DEV, log

import sparse_attention_indexer_kpool_amd as kp

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kp.lib()


def _run(pi, T, hidden, qlr, H, eps=1e-6):
    pp = kp.ProjParams(num_tokens=T, hidden=hidden, q_lora_rank=qlr, num_heads=H, head_dim=128,
                       eps=eps)
    ws = torch.empty(max(kp.kpool_proj_workspace_bytes(pp), 256), dtype=torch.uint8, device=DEV)
    q = torch.full((T, H * 128), 7.0, dtype=torch.bfloat16, device=DEV)
    k = torch.full((T, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    gate = torch.full((T, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    w = torch.full((T, H), 7.0, dtype=torch.float32, device=DEV)
    d = lambda t: t.to(DEV).contiguous()
    kp.kpool_indexer_projections(pp, d(pi.x), d(pi.qr), d(pi.wq_b), d(pi.wk), d(pi.k_norm_weight),
                                 d(pi.k_norm_bias), d(pi.wg), d(pi.ww), ws, q, k, gate, w)
    torch.cuda.synchronize()
    return q, k, gate, w


def _check(pi, rows, q, k, gate, w, eps=1e-6):
    x = pi.x[rows].float().numpy()
    qr = pi.qr[rows].float().numpy()
    wq_b, wk, wg = pi.wq_b.float().numpy(), pi.wk.float().numpy(), pi.wg.float().numpy()
    lw, lb, ww = pi.k_norm_weight.numpy(), pi.k_norm_bias.numpy(), pi.ww.numpy()
    H, D = pi.H, pi.D
    oq, ok_, og, ow = oracle.indexer_projections(x, qr, wq_b, wk, lw, lb, wg, ww, H, D, eps)
    sel = torch.tensor(rows, dtype=torch.long, device=DEV)
    gq = q[sel].float().cpu().numpy().reshape(len(rows), H, D)
    gk, gg = k[sel].float().cpu().numpy(), gate[sel].float().cpu().numpy()
    gw = w[sel].cpu().numpy()
    ax, aq = np.abs(x).astype(np.float64), np.abs(qr).astype(np.float64)
    dot = lambda a, b: 2.0 * a.shape[1] * 2.0 ** -24 * (a @ np.abs(b).T.astype(np.float64))
    pins.assert_within_bf16_ulps(gq.reshape(len(rows), -1), oq.reshape(len(rows), -1), 1,
                                 dot(aq, wq_b))
    pins.assert_within_bf16_ulps(gg, og, 1, dot(ax, wg))
    assert np.all(np.abs(gw.astype(np.float64) - ow) <= dot(ax, ww) + 1e-30), "head weights"
    # k: the linear outputs of the two sides differ by at most delta per row
    lin = oracle.linear_bf16(x, wk).astype(np.float64)
    delta = (pins.bf16_ulp(lin) + dot(ax, wk)).max(axis=1)
    sigma = np.sqrt(lin.var(axis=1) + eps)
    lim = np.abs(lw)[None, :] * (3.0 * delta / sigma)[:, None]
    pins.assert_within_bf16_ulps(gk, ok_, 1, lim)
    exact = [float(np.mean(a == b)) for a, b in ((gq, oq), (gk, ok_), (gg, og))]
    log(f"  rows {len(rows)}: identical fraction q {exact[0]:.4f} k {exact[1]:.4f} "
        f"gate {exact[2]:.4f}")


@pytest.mark.parametrize("T,hidden,qlr,H", [
    (1, 64, 64, 4), (127, 256, 192, 8), (300, 512, 128, 32), (129, 128, 64, 16),
], ids=["T1", "T127_h8", "T300_h32", "T129_h16"])
def test_projections_small_all_rows(T, hidden, qlr, H):
    pi = wlm.make_proj_inputs(T, hidden, qlr, H, seed=T + H)
    q, k, gate, w = _run(pi, T, hidden, qlr, H)
    _check(pi, list(range(T)), q, k, gate, w)


def test_projections_bench_shape_sampled():
    """The bench shape (65536 tokens, hidden 4096, query latent 1536, 32
    heads) on sampled rows, including both ends and a 128-row tile edge."""
    T, hidden, qlr, H = 65536, 4096, 1536, 32
    pi = wlm.make_proj_inputs(T, hidden, qlr, H, seed=11)
    q, k, gate, w = _run(pi, T, hidden, qlr, H)
    rows = sorted(set(wlm.strided_rows(T, 48)) | {0, 127, 128, T - 1})
    _check(pi, rows, q, k, gate, w)


def test_projections_feed_the_indexer():
    """The projections' outputs drive compression and the indexer: the
    result equals the indexer run on the oracle's projections wherever the
    two agree bit for bit (spot check of the layouts: q is [T, H, D], k and
    gate [T, D], w [T, H])."""
    T, hidden, qlr, H = 2048, 256, 128, 32
    pi = wlm.make_proj_inputs(T, hidden, qlr, H, seed=5)
    q, k, gate, w = _run(pi, T, hidden, qlr, H)
    assert q.shape == (T, H * 128) and k.shape == (T, 128) and w.shape == (T, H)
    p = kp.Params(num_docs=1, total_tokens=T, max_seqlen=T, num_heads=H, head_dim=128, kpool=4,
                  index_topk=512)
    cu = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    cup = torch.empty(2, dtype=torch.int32, device=DEV)
    pooled = torch.empty(T // 4, 128, dtype=torch.bfloat16, device=DEV)
    ape = torch.zeros(4, 128, dtype=torch.float32, device=DEV)
    kp.kpool_compress(p, k, gate, ape, cu, cup, pooled)
    ws = torch.empty(max(kp.kpool_workspace_bytes(p), 256), dtype=torch.uint8, device=DEV)
    tok = torch.empty(T, p.width, dtype=torch.int32, device=DEV)
    kp.kpool_indexer_topk(p, q.view(T, H, 128), w, pooled, cu, cup, ws, tok, None)
    torch.cuda.synchronize()
    t = tok.cpu().numpy()
    assert np.all(t[T - 1][:512] >= 0)
    assert t[T - 1][-1] == -1 or t[T - 1][-1] == T - 1
