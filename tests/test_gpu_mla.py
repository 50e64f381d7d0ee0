"""Sparse NoPE-MLA forward (kpool_sparse_mla_fwd, through the C ABI) against
the FP64 oracle, element by element (xtuner PR #2108, Summary: FlashMLA's
forward over the indexer's int32 indices; the LSE fix commit: natural-log
LSE).

Tolerance, from the kernel's arithmetic (BF16 inputs, so every product is
exact in FP32):
  * a score is an FP32 sum of 512 products: |ds| <= sm_scale * 512 * 2^-24 *
    sum_d |q_d kv_d| (plus 2^-23 |s| for the scale), which moves each
    normalised weight by at most a factor exp(2 |ds|_max);
  * the weights are rounded to BF16 (2^-9 relative) for the weighted sum,
    whose FP32 accumulation over n rows adds n * 2^-24 relative, both
    relative to A = sum_j p_j |kv_j| (p the normalised weights);
  * the output is rounded to BF16 (2^-9 |o|).
So |o - o_ref| <= (2^-9 + n 2^-24 + 2 ds_max) A + 2^-9 |o_ref|, and
|lse - lse_ref| <= ds_max + n 2^-24 + 2^-22 |lse_ref|. The tests allow twice
each bound (the first-order terms above drop products of small terms)."""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_kpool_amd as kp
import workloads as wlm
from gpu_common import DEV, log

pytestmark = pytest.mark.gpu


def run_gpu(q, kv, idx, sm_scale, fill=True):
    T, H, _ = q.shape
    N, W = kv.shape[0], idx.shape[1]
    out = torch.full((T, H, 512), 7.0 if fill else 0.0, dtype=torch.bfloat16, device=DEV)
    lse = torch.full((T, H), 12345.0, dtype=torch.float32, device=DEV)
    mp = kp.MlaParams(num_tokens=T, num_heads=H, kv_rows=N, width=W, sm_scale=sm_scale)
    kp.kpool_sparse_mla_fwd(mp, q, kv if N > 0 else None, idx if W > 0 else None, out, lse)
    torch.cuda.synchronize()
    return out, lse


def bounds(q_rows, kv, idx_rows, sm_scale, o_ref, lse_ref):
    """Per-element tolerances of the docstring for the given query rows."""
    T, H, d = q_rows.shape
    N = kv.shape[0]
    tol_o = np.zeros_like(o_ref)
    tol_l = np.zeros_like(lse_ref)
    for t in range(T):
        sel = [int(j) for j in idx_rows[t] if 0 <= j < N]
        if not sel:
            continue
        rows = kv[sel]
        s = sm_scale * (q_rows[t] @ rows.T)                             # [H, n]
        mag = abs(sm_scale) * (np.abs(q_rows[t]) @ np.abs(rows).T)
        ds = 512 * 2.0 ** -24 * mag.max(axis=1) + 2.0 ** -23 * np.abs(s).max(axis=1)
        p = np.exp(s - lse_ref[t][:, None])
        A = p @ np.abs(rows)                                            # [H, d]
        n = len(sel)
        tol_o[t] = 2 * ((2.0 ** -9 + n * 2.0 ** -24 + 2 * ds[:, None]) * A
                        + 2.0 ** -9 * np.abs(o_ref[t]))
        tol_l[t] = 2 * (ds + n * 2.0 ** -24 + 2.0 ** -22 * np.abs(lse_ref[t]))
    return tol_o, tol_l


def check_rows(rows, q, kv, idx, sm_scale, out, lse, what):
    q_np = q[rows].float().cpu().numpy().astype(np.float64)
    kv_np = kv.float().cpu().numpy().astype(np.float64)
    idx_np = idx[rows].cpu().numpy()
    o_ref, l_ref = oracle.sparse_mla_forward(q_np, kv_np, idx_np, sm_scale)
    got_o = out[rows].float().cpu().numpy().astype(np.float64)
    got_l = lse[rows].cpu().numpy().astype(np.float64)
    tol_o, tol_l = bounds(q_np, kv_np, idx_np, sm_scale, o_ref, l_ref)
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(got_l), empty), f"{what}: -inf lse pattern differs"
    assert np.all(got_o[empty] == 0.0), f"{what}: rows with no used entry must be zero"
    err_o = np.abs(got_o - o_ref)
    bad = err_o > tol_o
    assert not bad.any(), (f"{what}: {bad.sum()} outputs outside the bound; worst "
                           f"{(err_o / np.maximum(tol_o, 1e-300)).max():.3g}x")
    fin = ~empty
    err_l = np.abs(got_l[fin] - l_ref[fin])
    assert np.all(err_l <= tol_l[fin]), f"{what}: lse off by {err_l.max():.3g}"
    return float((err_o / np.maximum(tol_o, 1e-300)).max()) if err_o.size else 0.0


def dev_inputs(m: wlm.MlaInputs):
    return m.q.to(DEV), m.kv.to(DEV), m.indices.to(DEV)


@pytest.mark.parametrize("T,H,N,W,scale,qs", [
    (37, 64, 100, 70, 1 / math.sqrt(512), 1.0),     # 3 blocks, ragged last block of 6
    (9, 128, 64, 33, 1 / math.sqrt(192), 1.0),      # two head groups, 2 blocks (1 + 1 entry)
    (16, 64, 300, 96, 0.2, 3.0),                    # peaky softmax: the reference max moves
    (5, 64, 40, 1, 0.05, 1.0),                      # one entry per query
])
def test_mla_small_every_row(T, H, N, W, scale, qs):
    log(f"mla small T={T} H={H} N={N} W={W}")
    m = wlm.make_mla_inputs(T, H, N, W, seed=T + W, out_of_range_frac=0.05, q_scale=qs)
    q, kv, idx = dev_inputs(m)
    out, lse = run_gpu(q, kv, idx, scale)
    worst = check_rows(list(range(T)), q, kv, idx, scale, out, lse, f"T{T}H{H}W{W}")
    log(f"worst error / bound {worst:.3f}")


def test_mla_running_max_moves_every_block():
    """Scores that grow along the list by more than the rescale threshold per
    block: the accumulator is rescaled at every block."""
    T, H, N, W = 3, 64, 256, 256
    r = np.random.default_rng(7)
    u = r.standard_normal(512)
    u /= np.linalg.norm(u)
    kv = np.stack([(0.15 * j) * u + 0.01 * r.standard_normal(512) for j in range(N)])
    q = np.broadcast_to(u * 4.0, (T, H, 512)).copy() + 0.01 * r.standard_normal((T, H, 512))
    idx = np.stack([np.arange(W), np.arange(W)[::-1], r.permutation(W)]).astype(np.int32)
    qd = torch.from_numpy(q).to(torch.bfloat16).to(DEV)
    kvd = torch.from_numpy(kv).to(torch.bfloat16).to(DEV)
    idxd = torch.from_numpy(idx).to(DEV)
    out, lse = run_gpu(qd, kvd, idxd, 1.0)
    check_rows([0, 1, 2], qd, kvd, idxd, 1.0, out, lse, "growing scores")


def test_mla_edge_cases():
    """No entries (W = 0), no rows (N = 0), all-unused rows, one used entry in
    the last block of a long list, one row repeated, and T = 0."""
    H = 64
    m = wlm.make_mla_inputs(6, H, 50, 100, seed=3)
    q, kv, idx = dev_inputs(m)
    idx[0] = -1                                     # nothing used
    idx[1] = -1
    idx[1, 99] = 17                                 # one used entry, last block
    idx[2] = 23                                     # one row, 100 times
    idx[3, :] = 50 + torch.arange(100, dtype=torch.int32, device=DEV)   # all out of range
    out, lse = run_gpu(q, kv, idx, 0.1)
    check_rows(list(range(6)), q, kv, idx, 0.1, out, lse, "edge rows")
    # W = 0: every query empty
    out0, lse0 = run_gpu(q, kv, idx[:, :0].contiguous(), 0.1)
    assert torch.all(out0 == 0) and torch.all(torch.isneginf(lse0))
    # N = 0: every entry out of range
    out1, lse1 = run_gpu(q, kv[:0], idx, 0.1)
    assert torch.all(out1 == 0) and torch.all(torch.isneginf(lse1))
    # T = 0: nothing enqueued, nothing written
    mp = kp.MlaParams(num_tokens=0, num_heads=H, kv_rows=50, width=100, sm_scale=0.1)
    kp.kpool_sparse_mla_fwd(mp, None, None, None, None, None)


def test_mla_rejects_bad_shapes():
    q = torch.zeros(2, 32, 512, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kp.KPoolError):
        kp.kpool_sparse_mla_fwd(kp.MlaParams(2, 32, 4, 4, 0.1), q, q, None, q, q)
    with pytest.raises(kp.KPoolError):
        kp.kpool_sparse_mla_fwd(kp.MlaParams(2, 64, 4, 4, 0.1, dim_qk=576), q, q, None, q, q)
    with pytest.raises(kp.KPoolError):
        kp.kpool_sparse_mla_fwd(kp.MlaParams(2, 64, 4, 4, float("nan")), q, q, None, q, q)


def test_mla_bench_shape_sampled():
    """The measured configuration (64K queries, 64 heads, 2052 entries per
    query: index_topk 2048 plus kpool 4) in the launch the benchmark times;
    64 strided rows (and the last) against the oracle."""
    T, H, W = 65536, 64, 2052
    log("mla bench shape: drawing inputs on the device")
    m = wlm.make_mla_inputs_device(T, H, T, W, DEV, seed=5)
    scale = 1 / math.sqrt(192)
    out, lse = run_gpu(m.q, m.kv, m.indices, scale)
    rows = wlm.strided_rows(T, 64)
    worst = check_rows(rows, m.q, m.kv, m.indices, scale, out, lse, "T65536")
    log(f"bench shape: worst error / bound {worst:.3f}")
