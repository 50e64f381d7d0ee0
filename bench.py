"""Benchmark of the KPool indexer hot path on one MI355X.

One step = the whole path over one batch: kpool_compress + kpool_indexer_topk
(logits, pool top-k and tail + expansion for every query chunk). Inputs are
seeded synthetic tensors already resident in HBM when timing starts.

Prints ONE JSON line: throughput in queries/s (tokens of the batch / step
time), the roofline of the dominant kernel (the MFMA logits kernel, timed live
with HIP events on the launch stream, priced against the BF16 or FP8 dense
MFMA peak), per-phase achieved rates, and the CPU oracle timed on this host on
a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|IDX]
"""
from __future__ import annotations

import argparse
import math
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads as wlm  # noqa: E402

METRIC = "KPool indexer queries/s at 64K ctx; logits TFLOP/s as % of MFMA peak"
# MI355X dense peaks: 256 CUs at 2.4 GHz, 4096 BF16 (8192 FP8) MFMA FLOP per
# CU per clock (published as 2.5 and 5.0 PFLOP/s); HBM3E 8 TB/s.
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12      # 2516.6
PEAK_FP8_TFLOPS = 2 * PEAK_BF16_TFLOPS            # 5033.2
PEAK_HBM_GBS = 8000.0


class TimingEvent:
    """A HIP event for timing a few kernels between two records, created
    through the HIP runtime with hipEventDisableSystemFence: recording it
    then skips the system-scope cache writeback and invalidation that a
    default event does, which the HIP runtime documents as making timings of
    the commands between events more accurate. (Recorded between every
    launch of a 64K step, default events added about 6 us to each launch
    against the kernel trace; these about half of that.) Same interface as
    torch.cuda.Event: record() on torch's current stream, elapsed_time() in
    ms once the device is synchronized."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            h = ctypes.CDLL("libamdhip64.so")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = h
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        stream = self._ct.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = self._hip.hipEventRecord(self.h, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end) -> float:
        ms = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.h:
            self._hip.hipEventDestroy(self.h)


def logits_source_digest() -> str:
    """SHA-256 of what the logits kernel is built from: logits.hip, the
    shared device helpers and its argument struct (the rest of the launcher
    header declares other kernels)."""
    import re
    csrc = os.path.join(ROOT, "sparse_attention_indexer_kpool_amd", "csrc")
    read = lambda f: open(os.path.join(csrc, f), "rb").read()
    args = re.search(rb"struct LogitsArgs \{.*?\};", read("kpool_internal.h"), re.S)
    return hashlib.sha256(read("logits.hip") + read("kpool_device.h") +
                          (args.group(0) if args else b"")).hexdigest()


def logits_traffic(wl_name: str):
    """HBM bytes per logits launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (profiles/logits_kernel_traffic_<workload>.txt), scaled
    by a copy kernel of known size. None when no such file exists or when the
    logits kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"logits_kernel_traffic_{wl_name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if logits_source_digest() != kv.get("source_sha256"):
        return None
    return int(float(kv["hbm_bytes_per_launch"]))


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def causal_counts(doc_lengths, kpool, k_sel):
    """(sum of n_c over all queries, sum of n_c over queries that need
    selection, number of such queries)."""
    tot = need = rows = 0
    for L in doc_lengths:
        i = np.arange(L, dtype=np.int64)
        nc = (i + 1) // kpool
        tot += int(nc.sum())
        m = nc > k_sel
        need += int(nc[m].sum())
        rows += int(m.sum())
    return tot, need, rows


class Path:
    def __init__(self, inp: wlm.Inputs, dev="cuda:0"):
        import sparse_attention_indexer_kpool_amd as kp
        self.kp = kp
        wl = inp.wl
        self.inp = inp
        self.p = kp.Params(num_docs=len(inp.doc_lengths), total_tokens=inp.T,
                           max_seqlen=inp.max_seqlen, num_heads=wl.H, head_dim=wl.D,
                           kpool=wl.kpool, index_topk=wl.index_topk,
                           always_select_tail=int(wl.tail), use_fp8=int(wl.fp8),
                           query_chunk=wl.query_chunk)
        T = inp.T
        self.q = inp.q.to(dev)
        self.k = inp.k.to(dev)
        self.gate = inp.gate.to(dev)
        self.w = inp.w.to(dev)
        self.ape = inp.ape.to(dev)
        self.cu = inp.cu_seqlens.to(dev)
        self.cu_pools = torch.zeros(len(inp.doc_lengths) + 1, dtype=torch.int32, device=dev)
        self.pooled = torch.zeros(max(T // wl.kpool, 1), wl.D, dtype=torch.bfloat16, device=dev)
        self.ws = torch.empty(max(kp.kpool_workspace_bytes(self.p), 256), dtype=torch.uint8,
                              device=dev)
        self.tok = torch.empty(T, self.p.width, dtype=torch.int32, device=dev)
        self.qc = kp.kpool_query_chunk_rows(self.p)
        self.ld = kp.kpool_logits_ld(self.p)

    def step(self):
        kp = self.kp
        kp.kpool_compress(self.p, self.k, self.gate, self.ape, self.cu, self.cu_pools, self.pooled)
        kp.kpool_indexer_topk(self.p, self.q, self.w, self.pooled, self.cu, self.cu_pools,
                              self.ws, self.tok, None)

    def fused_indexer(self):
        """kpool_indexer_topk_fused: scoring, selection and expansion in one
        kernel per query chunk (plus the FP8 quantiser on the FP8 path)."""
        self.kp.kpool_indexer_topk_fused(self.p, self.q, self.w, self.pooled, self.cu,
                                         self.cu_pools, self.ws, self.tok, None)

    def fused_step(self):
        kp = self.kp
        kp.kpool_compress(self.p, self.k, self.gate, self.ape, self.cu, self.cu_pools, self.pooled)
        self.fused_indexer()

    # --- phases timed on their own (same launches as inside a step) --------
    def time_compress_cold(self, n_copies=16, replays=10):
        """Device time (ms) of one kpool_compress launch on inputs that no
        cache holds, as inside a step: n_copies copies of k and gate (more
        bytes than the GPU's last-level cache) are taken in turn, and the
        launches are captured in one HIP graph, so no host launch gap sits
        between them (the kernel runs for a few microseconds, less than a
        Python call takes)."""
        kp = self.kp
        ks = [self.k.clone() for _ in range(n_copies)]
        gs = [self.gate.clone() for _ in range(n_copies)]
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_copies):
                kp.kpool_compress(self.p, ks[i], gs[i], self.ape, self.cu, self.cu_pools,
                                  self.pooled)
        graph.replay()
        torch.cuda.synchronize()
        ms = time_region(graph.replay, replays, warm=1)
        del graph, ks, gs
        return ms / n_copies

    def indexer_phases(self, reps):
        """Device ms per step of the indexer's scoring kernels and of its
        selection + expansion kernels: the step's own launches
        (kpool_indexer_scoring, then kpool_indexer_selection, launch by
        launch), each kernel group bracketed by HIP events (TimingEvent, no
        system fence) on the launch stream; one untimed pass first. On the FP8 path the workspace already
        holds the quantised q and keys of the last step, so only the scoring
        kernel runs."""
        kp = self.kp
        launches = kp.kpool_indexer_launches(self.p)
        flags = kp.KPOOL_LOGITS_INPUTS_QUANTIZED if self.p.use_fp8 else 0
        ev = [[TimingEvent() for _ in range(3)] for _ in launches]
        t_score = t_select = 0.0
        for r in range(reps + 1):
            for i, e in enumerate(ev):
                e[0].record()
                kp.kpool_indexer_scoring(self.p, i, self.q, self.w, self.pooled, self.cu,
                                         self.cu_pools, self.ws, flags)
                e[1].record()
                kp.kpool_indexer_selection(self.p, i, self.cu, self.cu_pools, self.ws, self.tok)
                e[2].record()
            torch.cuda.synchronize()
            if r:
                t_score += sum(e[0].elapsed_time(e[1]) for e in ev)
                t_select += sum(e[1].elapsed_time(e[2]) for e in ev)
        return t_score / reps, t_select / reps, len(launches)

    def phase_fp8_quant(self, bufs):
        """The FP8 input path over every q row (t, h) and every pooled key."""
        qc, qs, kc, ks, P = bufs
        rows = self.inp.T * self.p.num_heads
        self.kp.kpool_fp8_quantize(self.q.view(rows, 128), rows, qc, qs)
        self.kp.kpool_fp8_quantize(self.pooled[:P], P, kc, ks)

    def phase_select(self, logits, ids, reps):
        """Device ms of the kpool_select stage entry (pool ids only) over every
        chunk: each chunk's scores come first from kpool_logits (untimed),
        then the selection kernel alone between HIP events."""
        kp = self.kp
        flags = kp.KPOOL_LOGITS_SKIP_ALL_SELECTED
        if self.p.use_fp8:
            flags |= kp.KPOOL_LOGITS_INPUTS_QUANTIZED
        chunks = [(c0, min(self.inp.T, c0 + self.qc)) for c0 in range(0, self.inp.T, self.qc)]
        ev = [[TimingEvent() for _ in range(2)] for _ in chunks]
        t = 0.0
        for r in range(reps + 1):
            for (c0, c1), e in zip(chunks, ev):
                kp.kpool_logits(self.p, self.q, self.w, self.pooled, self.cu, self.cu_pools, c0,
                                c1, self.ws, logits[:c1 - c0], flags=flags)
                e[0].record()
                kp.kpool_select(self.p, logits[:c1 - c0], c0, c1, self.cu, self.cu_pools,
                                ids[c0:c1])
                e[1].record()
            torch.cuda.synchronize()
            if r:
                t += sum(a.elapsed_time(b) for a, b in ev)
        return t / reps

    def phase_expand(self, ids):
        self.kp.kpool_expand(self.p, ids, self.cu, self.cu_pools, self.tok)


def time_region(fn, reps, warm=1):
    """Average ms of fn over reps after `warm` untimed calls, HIP events on
    torch's current stream (the stream every launch of the library goes
    to)."""
    for _ in range(warm):
        fn()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def cpu_baseline(inp: wlm.Inputs, n_rows: int):
    """The oracle as it stands on this host's cores: compress in full, then
    scoring, selection and expansion of n_rows strided query rows."""
    import oracle
    wl = inp.wl
    q = inp.q.float().numpy()
    k = inp.k.float().numpy()
    gate = inp.gate.float().numpy()
    w = inp.w.numpy()
    ape = inp.ape.numpy()
    cu = inp.cu_seqlens.numpy().astype(np.int64)
    t0 = time.perf_counter()
    pooled, _ = oracle.compress(k, gate, ape, cu, wl.kpool)
    t1 = time.perf_counter()
    rows = wlm.strided_rows(inp.T, n_rows)
    oracle.indexer_topk(q, w, pooled, cu, wl.kpool, wl.index_topk, wl.tail, rows=rows, fp8=wl.fp8)
    t2 = time.perf_counter()
    # per-query cost: the sampled rows plus their share of the compression
    per_query = (t2 - t1) / len(rows) + (t1 - t0) / inp.T
    threads = torch.get_num_threads()
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        pass
    return {"value": round(1.0 / per_query, 2), "unit": "queries/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{wl.name}: compress of all {inp.T} tokens ({t1 - t0:.2f} s) + scoring, "
                      f"top-k and expansion of {len(rows)} strided query rows ({t2 - t1:.2f} s); "
                      f"NumPy FP32 on {os.cpu_count()} host CPUs"}


def decode_bench(reps: int, B: int = 64, L: int = 65536, fp8: bool = False):
    """The serving step: kpool_decode_topk for B sequences of L tokens each
    (one query per sequence over L / 4 cached pooled keys), H = 32, D = 128,
    kpool = 4, index_topk = 2048; with fp8 the cache holds E4M3 codes and
    scales. Returns the JSON object of its line."""
    import sparse_attention_indexer_kpool_amd as kp
    H, D, KP, TOPK = 32, 128, 4, 2048
    di = wlm.make_decode_inputs([L] * B, H, D, KP, seed=7)
    p = kp.Params(num_docs=B, total_tokens=0, max_seqlen=L, num_heads=H, head_dim=D, kpool=KP,
                  index_topk=TOPK, always_select_tail=1, use_fp8=int(fp8))
    dev = "cuda:0"
    q, w, pooled = di.q.to(dev), di.w.to(dev), di.pooled.to(dev)
    scales = None
    if fp8:
        rows = pooled.shape[0]
        codes = torch.empty(rows, 128, dtype=torch.uint8, device=dev)
        scales = torch.empty(rows, dtype=torch.float32, device=dev)
        kp.kpool_fp8_quantize(pooled, rows, codes, scales)
        pooled = codes
    ps, sl, tb = di.pool_start.to(dev), di.seq_lens.to(dev), di.token_base.to(dev)
    ws = torch.empty(kp.kpool_decode_workspace_bytes(p), dtype=torch.uint8, device=dev)
    tok = torch.empty(B, p.width, dtype=torch.int32, device=dev)
    run = lambda: kp.kpool_decode_topk(p, q, w, pooled, ps, sl, ws, tok, token_base=tb,
                                       pooled_scale=scales)
    ms = time_region(run, reps, warm=2)
    n_c = L // KP
    if fp8:   # key codes + scale, scores written and read; q (quantised in the kernel) and w
        by = B * n_c * (D + 4 + 4 + 4) + B * H * (2 * D + 4) + 4 * B * p.width
    else:
        by = B * n_c * (2 * D + 4 + 4) + B * H * (2 * D + 4) + 4 * B * p.width
    return {"workload": f"decode{'_fp8' if fp8 else ''}_B{B}_L{L}_H{H}_D{D}", "ms": round(ms, 4),
            "queries_per_s": round(B / (ms * 1e-3), 1),
            "hbm": {"bytes": by, "GB/s": round(by / (ms * 1e-3) / 1e9, 1),
                    "frac": round(by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "note": "keys read once, scores written and read once, token rows written"}


def projections_bench(reps: int, T: int = 65536, hidden: int = 4096, q_lora: int = 1536,
                      H: int = 32):
    """kpool_indexer_projections at T tokens (stand-in sizes: the pages give
    neither the hidden size nor the query latent width). Returns the JSON
    object of its line."""
    import sparse_attention_indexer_kpool_amd as kp
    pi = wlm.make_proj_inputs(T, hidden, q_lora, H, seed=11)
    dev = "cuda:0"
    d = lambda t: t.to(dev).contiguous()
    pp = kp.ProjParams(num_tokens=T, hidden=hidden, q_lora_rank=q_lora, num_heads=H, head_dim=128)
    ws = torch.empty(kp.kpool_proj_workspace_bytes(pp), dtype=torch.uint8, device=dev)
    q = torch.empty(T, H * 128, dtype=torch.bfloat16, device=dev)
    k = torch.empty(T, 128, dtype=torch.bfloat16, device=dev)
    g = torch.empty_like(k)
    w = torch.empty(T, H, dtype=torch.float32, device=dev)
    args = [d(pi.x), d(pi.qr), d(pi.wq_b), d(pi.wk), d(pi.k_norm_weight), d(pi.k_norm_bias),
            d(pi.wg), d(pi.ww)]
    run = lambda: kp.kpool_indexer_projections(pp, *args, ws, q, k, g, w)
    ms = time_region(run, reps, warm=2)
    # algorithmic MFMA work: q, k and the gate, and the head weights as three
    # BF16 products (FP32 weights split exactly into three BF16 parts)
    flops = 2.0 * T * (q_lora * H * 128 + hidden * (128 + 128 + 3 * H))
    del pi, args, q, k, g, w, ws
    torch.cuda.empty_cache()
    return {"entry": "kpool_indexer_projections",
            "workload": f"proj_T{T}_hidden{hidden}_qlora{q_lora}_H{H}_D128", "ms": round(ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(flops / (ms * 1e-3) / 1e12, 2),
                         "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                         "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "note": "hidden and q_lora_rank are stand-in sizes"}


def sparse_mla_bench(reps: int, T: int = 65536, H: int = 64, W: int = 2052):
    """kpool_sparse_mla_fwd over T query tokens, H heads and W listed rows
    each (index_topk 2048 + kpool 4, the indexer's row width), latent width
    512, rows drawn uniformly from each token's causal prefix. Returns the
    JSON object of its line."""
    import sparse_attention_indexer_kpool_amd as kp
    dev = "cuda:0"
    m = wlm.make_mla_inputs_device(T, H, T, W, dev, seed=5)
    out = torch.empty(T, H, 512, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(T, H, dtype=torch.float32, device=dev)
    mp = kp.MlaParams(num_tokens=T, num_heads=H, kv_rows=T, width=W, sm_scale=1 / math.sqrt(192))
    used = int(((m.indices >= 0) & (m.indices < T)).sum().item())
    run = lambda: kp.kpool_sparse_mla_fwd(mp, m.q, m.kv, m.indices, out, lse)
    ms = time_region(run, reps, warm=2)
    # algorithmic work: per used entry and head, 512 multiply-adds for the
    # score and 512 for the weighted row
    flops = used * H * 512 * 4.0
    gathered = used * 1024.0 + 2 * T * H * 512 * 2 + T * W * 4
    del m, out, lse
    torch.cuda.empty_cache()
    tf = flops / (ms * 1e-3) / 1e12
    return {"entry": "kpool_sparse_mla_fwd",
            "workload": f"sparse_mla_T{T}_H{H}_W{W}_D512", "ms": round(ms, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2),
                         "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)},
            "bytes_touched": gathered,
            "note": "rows gathered per query: 1 KB each, mostly from L2/MALL; "
                    "rows drawn uniformly from the causal prefix"}


def measure_workload(wl, steps: int, warmup: int):
    """One workload: the whole step timed over `steps` steps after `warmup`
    untimed ones, then each phase alone with the same launches. Returns
    (inputs, ms per step, the line's figures for this workload)."""
    log(f"inputs {wl.name}")
    inp = wlm.make_inputs(wl)
    path = Path(inp)
    T = inp.T
    tot_nc, need_nc, need_rows = causal_counts(inp.doc_lengths, wl.kpool, wl.k_sel)

    log(f"{wl.name}: warmup {warmup}")
    for _ in range(warmup):
        path.step()
    torch.cuda.synchronize()
    log(f"{wl.name}: timing {steps} steps")
    ms = time_region(path.step, steps, warm=0)
    log(f"{wl.name}: {ms:.4f} ms/step")

    # phases, each timed live on the launch stream with the step's launches
    logits = torch.empty(path.qc, path.ld, dtype=torch.float32, device="cuda:0")
    ids = torch.empty(T, wl.k_sel, dtype=torch.int32, device="cuda:0")
    reps = max(3, min(steps, 10))
    ms_compress = path.time_compress_cold()
    ms_logits, ms_select_expand, n_launches = path.indexer_phases(reps)
    ms_select = path.phase_select(logits, ids, reps)
    ms_expand = time_region(lambda: path.phase_expand(ids), reps)
    ms_fp8 = None
    P = sum(L // wl.kpool for L in inp.doc_lengths)
    if wl.fp8:
        rows = T * wl.H
        bufs = (torch.empty(rows, 128, dtype=torch.uint8, device="cuda:0"),
                torch.empty(rows, dtype=torch.float32, device="cuda:0"),
                torch.empty(max(P, 1), 128, dtype=torch.uint8, device="cuda:0"),
                torch.empty(max(P, 1), dtype=torch.float32, device="cuda:0"), P)
        ms_fp8 = time_region(lambda: path.phase_fp8_quant(bufs), reps)
    del logits, ids
    fused = None
    if wl.k_sel <= path.kp.kpool_fused_max_ksel(path.p):
        path.fused_step()
        ms_fused_step = time_region(path.fused_step, min(steps, 50), warm=1)
        ms_fused_idx = time_region(path.fused_indexer, reps)
        fused = (ms_fused_step, ms_fused_idx)
        log(f"{wl.name}: fused step {ms_fused_step:.4f} ms")

    flops = 2.0 * wl.H * wl.D * need_nc
    peak = PEAK_FP8_TFLOPS if wl.fp8 else PEAK_BF16_TFLOPS
    achieved = flops / (ms_logits * 1e-3) / 1e12
    by_compress = 4 * T * wl.D + 4 * wl.kpool * wl.D + 2 * P * wl.D
    by_select = 4 * need_nc + 4 * T * wl.k_sel
    by_select_expand = 4 * need_nc + 4 * T * wl.width
    by_expand = 4 * T * (wl.k_sel + wl.width)
    by_fp8 = (T * wl.H + P) * (256 + 128 + 4)

    def hbm(b, m):
        return {"bytes": b, "GB/s": round(b / (m * 1e-3) / 1e9, 1),
                "frac": round(b / (m * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    fig = {
        "config": {"workload": wl.name, "T": T, "H": wl.H, "D": wl.D, "kpool": wl.kpool,
                   "index_topk": wl.index_topk, "always_select_tail": wl.tail,
                   "query_chunk": path.qc, "docs": len(inp.doc_lengths), "fp8": wl.fp8},
        "ms_per_step": round(ms, 4),
        "queries_per_s": round(T / (ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": logits_traffic(wl.name),
                     "kernel": "logits_kernel", "launches_per_step": n_launches,
                     "algorithmic_flops_per_step": flops},
        "phases_ms": {"compress": round(ms_compress, 4), "logits": round(ms_logits, 4),
                      "select_expand": round(ms_select_expand, 4),
                      "select": round(ms_select, 4), "expand": round(ms_expand, 4)},
        "phases_hbm": {"compress": hbm(by_compress, ms_compress),
                       "select_expand": hbm(by_select_expand, ms_select_expand),
                       "select": hbm(by_select, ms_select),
                       "expand": hbm(by_expand, ms_expand)},
    }
    if ms_fp8 is not None:
        fig["phases_ms"]["fp8_quant"] = round(ms_fp8, 4)
        fig["phases_hbm"]["fp8_quant"] = hbm(by_fp8, ms_fp8)
    if fused is not None:
        # the fused entry point, timed the same way; its kernel does the
        # same FLOPs as the scoring kernel (the quantiser's time, on the FP8
        # path, is taken off with the phase measured above)
        ms_fk = fused[1] - (ms_fp8 or 0.0)
        fig["fused"] = {
            "entry": "kpool_indexer_topk_fused", "ms_per_step": round(fused[0], 4),
            "queries_per_s": round(T / (fused[0] * 1e-3), 1),
            "vs_two_kernel_step": round(ms / fused[0], 4),
            "indexer_ms": round(fused[1], 4),
            "kernel_roofline": {"bound": "mfma", "achieved": round(flops / (ms_fk * 1e-3) / 1e12, 2),
                                "peak": round(peak, 1), "unit": "TFLOP/s",
                                "frac": round(flops / (ms_fk * 1e-3) / 1e12 / peak, 4)},
            "note": "scores never leave the chip; token rows written directly"}
    del path
    torch.cuda.empty_cache()
    return inp, ms, fig


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the default times 2000 steps of the 64K workload, about 8 s of GPU work
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_T65536_H32_D128")
    ap.add_argument("--cpu-rows", type=int, default=12288)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the serving-step measurement (kpool_decode_topk)")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads (FP8 and the short ones) on the line")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the bench, run 3 device copies of this many MiB (a kernel of "
                         "known traffic that calibrates the HBM byte counters of a profiler)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the indexer here runs "
              "on a single device and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    wl = wlm.workload(int(args.workload)) if args.workload.isdigit() else wlm.workload(args.workload)
    inp, ms, fig = measure_workload(wl, args.steps, args.warmup)
    T = inp.T

    out = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if wl.fp8 else "bf16",
        "data": "synthetic",
        "config": fig["config"],
        "roofline": fig["roofline"],
        "phases_ms": fig["phases_ms"],
        "phases_hbm": fig["phases_hbm"],
    }
    if "fused" in fig:
        out["fused"] = fig["fused"]
    if not args.no_decode and wl.name == "long_T65536_H32_D128":
        reps = max(3, min(args.steps, 10))
        log("decode step, 64 sequences of 64K tokens")
        out["decode"] = decode_bench(reps)
        out["decode_fp8"] = decode_bench(reps, fp8=True)
    if not args.no_others and wl.name == "long_T65536_H32_D128":
        log("indexer projections")
        out["projections"] = projections_bench(max(3, min(args.steps, 10)))
        log("sparse MLA forward over the selected rows")
        out["sparse_mla"] = sparse_mla_bench(max(3, min(args.steps, 5)))
        # the FP8 input path and the short workloads, each timed the same way
        for key, other in (("fp8", "fp8_T32768_H32_D128"), ("tiny", "tiny_T256_H4_D64"),
                           ("single_4k", "single_T4096_H32_D128"),
                           ("packed8", "packed8_H32_D128")):
            _, _, f2 = measure_workload(wlm.workload(other), min(args.steps, 200), args.warmup)
            out[key] = f2
    if rank == 0 and not args.no_cpu_baseline:
        log(f"cpu baseline on {args.cpu_rows} rows")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_rows)
    else:
        out["cpu_baseline"] = None
    if rank == 0:
        print(json.dumps(out), flush=True)
    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 3 x {args.copy_mib} MiB read + {args.copy_mib} MiB written")


if __name__ == "__main__":
    main()
