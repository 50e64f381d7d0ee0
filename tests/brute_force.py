"""FP64 brute force of the KPool indexer for tiny inputs (a pin for the oracle).

It is written from a different angle than the oracle: pools are enumerated as
explicit token sets, a pool is causal for query t when its largest token is at
or before t, the tail is every visible token of the query's document that no
causal pool covers, selection is a full sort of (score desc, pool id asc), and
all arithmetic is Python floats (FP64) with math.exp.
"""
from __future__ import annotations

import math


def pools_of(doc_lengths, kpool):
    """List of (doc, global pool id, token list) in packed order."""
    out = []
    start = 0
    gid = 0
    for b, L in enumerate(doc_lengths):
        for p in range(L // kpool):
            out.append((b, gid, [start + p * kpool + s for s in range(kpool)]))
            gid += 1
        start += L
    return out


def doc_ranges(doc_lengths):
    rng = []
    start = 0
    for L in doc_lengths:
        rng.append((start, start + L))
        start += L
    return rng


def brute_pooled(k, gate, ape, doc_lengths, kpool):
    """Pooled keys in FP64 (no BF16 rounding)."""
    D = len(k[0])
    res = []
    for _, _, toks in pools_of(doc_lengths, kpool):
        row = []
        for d in range(D):
            logits = [float(gate[u][d]) + float(ape[s][d]) for s, u in enumerate(toks)]
            top = max(logits)
            ex = [math.exp(v - top) for v in logits]
            z = math.fsum(ex)
            row.append(math.fsum(ex[s] / z * float(k[u][d]) for s, u in enumerate(toks)))
        res.append(row)
    return res


def brute_rows(q, w, keys, doc_lengths, kpool, index_topk, tail_on, scale):
    """(token rows, pool-id rows, per-query {pool id: score}) in FP64, for every
    query of the packed batch. keys: list of pooled rows indexed by global id."""
    pools = pools_of(doc_lengths, kpool)
    ranges = doc_ranges(doc_lengths)
    H = len(q[0])
    k_sel = index_topk // kpool
    width = index_topk + kpool
    tok_rows, pool_rows, score_maps = [], [], []
    for b, (lo, hi) in enumerate(ranges):
        for t in range(lo, hi):
            causal = [(gid, toks) for (pb, gid, toks) in pools if pb == b and max(toks) <= t]
            scores = {}
            for gid, _ in causal:
                tot = 0.0
                for h in range(H):
                    dot = math.fsum(float(a) * float(c) for a, c in zip(q[t][h], keys[gid]))
                    tot += float(w[t][h]) * max(0.0, scale * dot)
                scores[gid] = tot
            ranked = sorted(scores, key=lambda g: (-scores[g], g))
            chosen = sorted(ranked[:k_sel])
            covered = set()
            for gid, toks in causal:
                covered.update(toks)
            toks = []
            for gid in chosen:
                toks.extend(dict(causal)[gid])
            if tail_on:
                toks.extend(u for u in range(lo, t + 1) if u not in covered)
            toks = sorted(toks)
            tok_rows.append(toks + [-1] * (width - len(toks)))
            pool_rows.append(chosen + [-1] * (k_sel - len(chosen)))
            score_maps.append(scores)
    return tok_rows, pool_rows, score_maps
