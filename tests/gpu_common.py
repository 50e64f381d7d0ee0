"""Helpers of the GPU parity tests: seeded inputs on the device, calls through
the C ABI (via the ctypes binding), and comparisons with the CPU oracle."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import sparse_attention_indexer_kpool_amd as kp
import workloads as wlm

DEV = "cuda:0"


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def params_for(inp: wlm.Inputs, query_chunk=None, use_fp8=None, tail=None) -> kp.Params:
    wl = inp.wl
    return kp.Params(
        num_docs=len(inp.doc_lengths), total_tokens=inp.T, max_seqlen=inp.max_seqlen,
        num_heads=wl.H, head_dim=wl.D, kpool=wl.kpool, index_topk=wl.index_topk,
        always_select_tail=int(wl.tail if tail is None else tail),
        use_fp8=int(wl.fp8 if use_fp8 is None else use_fp8),
        query_chunk=wl.query_chunk if query_chunk is None else query_chunk)


class Dev:
    """Device copies of one workload's inputs plus the compressed keys."""

    def __init__(self, inp: wlm.Inputs):
        self.inp = inp
        self.p = params_for(inp)
        self.q = inp.q.to(DEV).contiguous()
        self.k = inp.k.to(DEV).contiguous()
        self.gate = inp.gate.to(DEV).contiguous()
        self.w = inp.w.to(DEV).contiguous()
        self.ape = inp.ape.to(DEV).contiguous()
        self.cu = inp.cu_seqlens.to(DEV).contiguous()
        T, D, kpool = inp.T, inp.wl.D, inp.wl.kpool
        self.cu_pools = torch.full((len(inp.doc_lengths) + 1,), -7, dtype=torch.int32, device=DEV)
        self.pooled = torch.full((max(T // kpool, 1), D), 0x7F7F, dtype=torch.int16,
                                 device=DEV).view(torch.bfloat16)

    def compress(self):
        kp.kpool_compress(self.p, self.k, self.gate, self.ape, self.cu, self.cu_pools, self.pooled)
        torch.cuda.synchronize()
        P = int(self.cu_pools[-1].item())
        return self.pooled[:P].float().cpu().numpy(), self.cu_pools.cpu().numpy()

    def workspace(self, p=None):
        n = kp.kpool_workspace_bytes(p or self.p)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=DEV)

    def indexer(self, p=None, with_pool_idx=True):
        p = p or self.p
        T = self.inp.T
        ws = self.workspace(p)
        tok = torch.full((T, p.width), -12345, dtype=torch.int32, device=DEV)
        pid = torch.full((T, p.k_sel), -12345, dtype=torch.int32, device=DEV) if with_pool_idx else None
        kp.kpool_indexer_topk(p, self.q, self.w, self.pooled, self.cu, self.cu_pools, ws, tok, pid)
        torch.cuda.synchronize()
        return tok.cpu().numpy(), (pid.cpu().numpy() if pid is not None else None)

    def logits(self, q_begin, q_end, p=None):
        p = p or self.p
        ld = kp.kpool_logits_ld(p)
        out = torch.full((q_end - q_begin, ld), 12345.0, dtype=torch.float32, device=DEV)
        ws = self.workspace(p)
        kp.kpool_logits(p, self.q, self.w, self.pooled, self.cu, self.cu_pools, q_begin, q_end,
                        ws, out)
        torch.cuda.synchronize()
        return out


def oracle_inputs(inp: wlm.Inputs):
    return (inp.q.float().numpy(), inp.k.float().numpy(), inp.gate.float().numpy(),
            inp.w.numpy(), inp.ape.numpy(), inp.cu_seqlens.numpy().astype(np.int64))


def scores_close(got, ref, sabs=None, head_dim=128):
    """|g - o| <= 2e-3 * |o| + 2 * gamma_D * sabs elementwise.
    sabs[j] = sum_h |w_h| * scale * sum_d |q_hd k_jd| is the magnitude scale
    of the score's terms; gamma_D = D * 2^-24 is the textbook rounding-error
    bound of an FP32 dot product of length D, applied to each side (it also
    covers the FP32 sum over the H <= D heads). It matters only where the
    heads cancel."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return True, 0.0
    lim = 2e-3 * np.abs(ref) + 1e-30
    if sabs is not None:
        lim = lim + 2.0 * head_dim * 2.0 ** -24 * np.asarray(sabs, np.float64)
    err = np.abs(got - ref) / lim
    return bool(np.all(err <= 1.0)), float(err.max())


def term_scale(q_t, w_t, keys, scale):
    """sum_h |w_h| * scale * sum_d |q_hd| |k_jd| for each key row j."""
    qa = np.abs(np.asarray(q_t, np.float64))
    ka = np.abs(np.asarray(keys, np.float64))
    return (np.abs(np.asarray(w_t, np.float64))[:, None] * scale * (qa @ ka.T)).sum(0)


def sets_match_up_to_ties(got_ids, ref_ids, ref_scores, pool0, k_sel, rel=1e-3):
    """Chosen pool sets agree except pools whose oracle score lies within rel
    of the oracle's k-th score (scores indexed by doc-local pool)."""
    got = set(int(x) for x in got_ids if x >= 0)
    ref = set(int(x) for x in ref_ids if x >= 0)
    if got == ref:
        return True, ""
    n = len(ref_scores)
    kth = np.sort(np.asarray(ref_scores, np.float64))[::-1][min(k_sel, n) - 1]
    for gid in got ^ ref:
        s = float(ref_scores[gid - pool0])
        if abs(s - kth) > rel * abs(kth):
            return False, f"pool {gid} score {s} vs k-th {kth}"
    return len(got) == len(ref), "size mismatch"
