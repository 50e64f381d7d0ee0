"""The decode entry point that allocates nothing (kpool_decode_topk_noalloc),
through the C ABI: its outputs equal kpool_decode_topk's (same kernels, the
scores in the library's built-in scratch instead of a caller workspace) on two
calls in a row, the second with a smaller batch, and a batch whose scores do
not fit the scratch is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wlm

import sparse_attention_indexer_kpool_amd as kp

DEV = "cuda:0"


def _params(lens, H, D, kpool, topk, fp8=False):
    return kp.Params(num_docs=len(lens), total_tokens=0, max_seqlen=max(lens), num_heads=H,
                     head_dim=D, kpool=kpool, index_topk=topk, always_select_tail=1,
                     use_fp8=int(fp8))


def _both(p, di, fp8=False):
    """(token rows, pool ids) of kpool_decode_topk and of the no-alloc entry."""
    q, w = di.q.to(DEV), di.w.to(DEV)
    pooled, scales = di.pooled.to(DEV), None
    if fp8:
        rows = pooled.shape[0]
        codes = torch.empty(rows, 128, dtype=torch.uint8, device=DEV)
        scales = torch.empty(rows, dtype=torch.float32, device=DEV)
        kp.kpool_fp8_quantize(pooled, rows, codes, scales)
        pooled = codes
    ps, sl, tb = di.pool_start.to(DEV), di.seq_lens.to(DEV), di.token_base.to(DEV)
    ws = torch.empty(max(kp.kpool_decode_workspace_bytes(p), 256), dtype=torch.uint8, device=DEV)
    tok_a = torch.full((di.B, p.width), -7, dtype=torch.int32, device=DEV)
    pid_a = torch.full((di.B, p.k_sel), -7, dtype=torch.int32, device=DEV)
    kp.kpool_decode_topk(p, q, w, pooled, ps, sl, ws, tok_a, pid_a, token_base=tb,
                         pooled_scale=scales)
    tok_b = torch.full((di.B, p.width), -9, dtype=torch.int32, device=DEV)
    pid_b = torch.full((di.B, p.k_sel), -9, dtype=torch.int32, device=DEV)
    kp.kpool_decode_topk_noalloc(p, q, w, pooled, ps, sl, tok_b, pid_b, token_base=tb,
                                 pooled_scale=scales)
    torch.cuda.synchronize()
    return (tok_a.cpu().numpy(), pid_a.cpu().numpy(), tok_b.cpu().numpy(), pid_b.cpu().numpy())


@pytest.mark.gpu
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_noalloc_matches_decode_twice(fp8):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    # first call: 48 sequences up to 64K tokens (12 MiB of scores in the scratch)
    big = [65536 - 1021 * b for b in range(48)]
    p1 = _params(big, 32, 128, 4, 2048, fp8)
    assert kp.kpool_decode_workspace_bytes(p1) <= kp.kpool_decode_noalloc_max_bytes()
    di1 = wlm.make_decode_inputs(big, 32, 128, 4, seed=11)
    ta, pa, tb, pb = _both(p1, di1, fp8)
    assert np.array_equal(ta, tb) and np.array_equal(pa, pb)
    assert np.all(pa[:, 0] >= 0)
    # second call: fewer, shorter sequences, other shapes; the scratch still
    # holds the first call's scores, which must not leak into these rows
    small = [0, 1, 5, 2047, 2051, 9000]
    p2 = _params(small, 16, 128, 4, 512, fp8)
    di2 = wlm.make_decode_inputs(small, 16, 128, 4, seed=12)
    ta, pa, tb, pb = _both(p2, di2, fp8)
    assert np.array_equal(ta, tb) and np.array_equal(pa, pb)
    assert np.all(tb[0] == -1)


def _no_gpu_visible():
    return torch.cuda.device_count() == 0


@pytest.mark.skipif(not _no_gpu_visible(), reason="fake-pointer calls run only without a GPU")
def test_noalloc_refuses_what_does_not_fit():
    """More scores than the scratch holds: refused during validation (so no
    HIP call is made; the pointers are never dereferenced)."""
    cap = kp.kpool_decode_noalloc_max_bytes()
    assert cap == 32 << 20
    fake = 1 << 20
    p = kp.Params(num_docs=1024, total_tokens=0, max_seqlen=65536, num_heads=32, head_dim=128,
                  kpool=4, index_topk=2048)
    assert kp.kpool_decode_workspace_bytes(p) > cap
    st = kp.lib().kpool_decode_topk_noalloc(ctypes.byref(p.c()), fake, fake, fake, 100, None,
                                            fake, fake, None, fake, None, None)
    assert st == kp.KPOOL_E_WORKSPACE
    assert "scratch" in kp.kpool_last_error()
    # bad arguments of a batch that fits are refused as kpool_decode_topk refuses them
    p2 = kp.Params(num_docs=8, total_tokens=0, max_seqlen=65536, num_heads=32, head_dim=128,
                   kpool=4, index_topk=2048)
    st = kp.lib().kpool_decode_topk_noalloc(ctypes.byref(p2.c()), fake, fake, fake, 100, None,
                                            fake, None, None, fake, None, None)
    assert st == kp.KPOOL_E_INVALID and "seq_lens" in kp.kpool_last_error()
