"""Seeded synthetic inputs for the KPool indexer (shared by the oracle tests, the
GPU tests and the benchmark).

This module only draws random numbers and casts them to the storage dtypes the
indexer consumes; it holds none of the method's arithmetic. Both the CPU oracle
and the HIP library are fed from here, and neither is imported by this file.

Workloads follow the shapes of the GLM-5.3-Flash indexer described on the
Megatron-LM PR #7054 page ("GLM-5.3-Flash at a glance": index_kpool = 4,
index_kpool_always_select_tail = true, index_topk = 2048), with synthetic
values: q, k and the gate logits ~ N(0, 1) stored as BF16, w ~ N(0, 1)/sqrt(H)
in FP32, the per-slot position bias ~ N(0, 0.1) (standard deviation 0.1) in
FP32. The long-context workloads scale the keys of 5 % of the tokens by 4 to
give heavy-tailed scores.

Draw order for one workload, from one CPU torch.Generator seeded with `seed`:
  1. document lengths (packed workloads only): randint(lo, hi + 1, (B,))
  2. q = randn(T, H, D)
  3. k = randn(T, D)
  4. w = randn(T, H) / sqrt(H)
  5. gate = randn(T, D)
  6. ape = 0.1 * randn(kpool, D)
  7. heavy-tailed workloads only: rows randperm(T)[:round(frac * T)] of k *= 4
  8. q, k and gate are cast to BF16 (round to nearest even)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int = 0                      # total tokens (single-document workloads)
    H: int = 32                     # indexer heads
    D: int = 128                    # indexer head dim
    kpool: int = 4
    index_topk: int = 2048
    tail: bool = True               # always_select_tail
    fp8: bool = False               # FP8 input path
    query_chunk: int = 0            # 0 = library default
    doc_lengths: Optional[Sequence[int]] = None   # explicit document lengths
    num_docs: int = 0               # > 0: draw this many lengths uniformly
    doc_len_range: tuple = (512, 4096)
    heavy_frac: float = 0.0         # fraction of key rows scaled by 4
    seed: int = 0

    @property
    def k_sel(self) -> int:
        return self.index_topk // self.kpool

    @property
    def width(self) -> int:
        return self.index_topk + self.kpool


# The five workloads: tiny single sequence, 4K single sequence, packed batch
# of 8 documents, 64K long context, 32K FP8 input path.
WORKLOADS = [
    Workload("tiny_T256_H4_D64", T=256, H=4, D=64, kpool=4, index_topk=64),
    Workload("single_T4096_H32_D128", T=4096),
    Workload("packed8_H32_D128", num_docs=8, doc_len_range=(512, 4096)),
    Workload("long_T65536_H32_D128", T=65536, query_chunk=4096, heavy_frac=0.05),
    Workload("fp8_T32768_H32_D128", T=32768, fp8=True, query_chunk=4096,
             heavy_frac=0.05),
]


def workload(index_or_name) -> Workload:
    if isinstance(index_or_name, int):
        return WORKLOADS[index_or_name]
    for w in WORKLOADS:
        if w.name == index_or_name:
            return w
    raise KeyError(index_or_name)


@dataclass
class Inputs:
    """CPU tensors of one workload. BF16 tensors are torch.bfloat16."""
    wl: Workload
    q: torch.Tensor          # bf16 [T, H, D]
    k: torch.Tensor          # bf16 [T, D]
    w: torch.Tensor          # f32  [T, H]
    gate: torch.Tensor       # bf16 [T, D]
    ape: torch.Tensor        # f32  [kpool, D]
    cu_seqlens: torch.Tensor  # int32 [B + 1]
    doc_lengths: list = field(default_factory=list)

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_seqlen(self) -> int:
        return max(self.doc_lengths) if self.doc_lengths else 0


def make_inputs(wl: Workload, seed: Optional[int] = None) -> Inputs:
    g = torch.Generator().manual_seed(wl.seed if seed is None else seed)
    if wl.doc_lengths is not None:
        lengths = [int(x) for x in wl.doc_lengths]
    elif wl.num_docs > 0:
        lo, hi = wl.doc_len_range
        lengths = torch.randint(lo, hi + 1, (wl.num_docs,), generator=g).tolist()
    else:
        lengths = [wl.T]
    T = sum(lengths)
    H, D, kp = wl.H, wl.D, wl.kpool
    q = torch.randn(T, H, D, generator=g)
    k = torch.randn(T, D, generator=g)
    w = torch.randn(T, H, generator=g) / math.sqrt(H)
    gate = torch.randn(T, D, generator=g)
    ape = 0.1 * torch.randn(kp, D, generator=g)
    if wl.heavy_frac > 0 and T > 0:
        heavy = torch.randperm(T, generator=g)[: int(round(wl.heavy_frac * T))]
        k[heavy] *= 4.0
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    if lengths:
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return Inputs(wl=wl, q=q.to(torch.bfloat16), k=k.to(torch.bfloat16),
                  w=w.to(torch.float32).contiguous(), gate=gate.to(torch.bfloat16),
                  ape=ape.to(torch.float32).contiguous(), cu_seqlens=cu,
                  doc_lengths=lengths)


@dataclass
class DecodeInputs:
    """CPU tensors of one serving (decode) step: B sequences, one query each,
    their complete pools in a shared cache of pooled rows."""
    q: torch.Tensor           # bf16 [B, H, D]
    w: torch.Tensor           # f32  [B, H]
    pooled: torch.Tensor      # bf16 [rows, D]: the cache
    pool_start: torch.Tensor  # int32 [B]: first cache row of each sequence
    seq_lens: torch.Tensor    # int32 [B]: tokens of each sequence so far
    token_base: torch.Tensor  # int32 [B]: id of each sequence's token 0
    kpool: int

    @property
    def B(self) -> int:
        return int(self.q.shape[0])


def make_decode_inputs(seq_lens, H: int, D: int, kpool: int, seed: int = 0, gap: int = 3,
                       heavy_frac: float = 0.05) -> DecodeInputs:
    """Seeded decode inputs. q ~ N(0, 1), w ~ N(0, 1) / sqrt(H); the cache
    holds `gap` unrelated rows before each sequence's floor(L / kpool) rows,
    all ~ N(0, 1), with heavy_frac of them scaled by 4 (heavy-tailed scores,
    as in the long prefill workloads). Token ids are laid out as in a packed
    batch (token_base = running sum of the lengths)."""
    g = torch.Generator().manual_seed(seed)
    lens = [int(x) for x in seq_lens]
    B = len(lens)
    starts, cursor = [], 0
    for L in lens:
        cursor += gap
        starts.append(cursor)
        cursor += L // kpool
    rows = cursor + gap
    q = torch.randn(B, H, D, generator=g)
    w = torch.randn(B, H, generator=g) / math.sqrt(H)
    pooled = torch.randn(rows, D, generator=g)
    if heavy_frac > 0 and rows > 0:
        heavy = torch.randperm(rows, generator=g)[: int(round(heavy_frac * rows))]
        pooled[heavy] *= 4.0
    base = [0]
    for L in lens[:-1]:
        base.append(base[-1] + L)
    return DecodeInputs(q=q.to(torch.bfloat16), w=w.to(torch.float32).contiguous(),
                        pooled=pooled.to(torch.bfloat16),
                        pool_start=torch.tensor(starts, dtype=torch.int32),
                        seq_lens=torch.tensor(lens, dtype=torch.int32),
                        token_base=torch.tensor(base, dtype=torch.int32), kpool=kpool)


def custom(name="custom", **kw) -> Workload:
    """A workload with explicit fields (tests use this for small cases)."""
    return replace(Workload(name), **kw)


def strided_rows(T: int, n: int) -> list:
    """n query rows strided uniformly over [0, T), the last row always included."""
    if T <= 0:
        return []
    if n >= T:
        return list(range(T))
    rows = sorted(set(int(round(x)) for x in torch.linspace(0, T - 1, n).tolist()))
    if rows[-1] != T - 1:
        rows.append(T - 1)
    return rows


@dataclass
class ProjInputs:
    """CPU tensors of the indexer projections for T tokens."""
    x: torch.Tensor           # bf16 [T, hidden]
    qr: torch.Tensor          # bf16 [T, q_lora]
    wq_b: torch.Tensor        # bf16 [H*D, q_lora]
    wk: torch.Tensor          # bf16 [D, hidden]
    k_norm_weight: torch.Tensor  # f32 [D]
    k_norm_bias: torch.Tensor    # f32 [D]
    wg: torch.Tensor          # bf16 [D, hidden]
    ww: torch.Tensor          # f32 [H, hidden]
    H: int
    D: int


def make_proj_inputs(T: int, hidden: int, q_lora: int, H: int, D: int = 128,
                     seed: int = 0) -> ProjInputs:
    """Seeded projection inputs: activations ~ N(0, 1), weight rows ~
    N(0, 1 / fan_in) (so the outputs are O(1)), k_norm weight 1 + 0.1 N(0, 1),
    bias 0.1 N(0, 1). Draw order: x, qr, wq_b, wk, wg, k_norm weight, bias,
    ww; BF16 tensors cast with round to nearest even."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, hidden, generator=g)
    qr = torch.randn(T, q_lora, generator=g)
    wq_b = torch.randn(H * D, q_lora, generator=g) / math.sqrt(q_lora)
    wk = torch.randn(D, hidden, generator=g) / math.sqrt(hidden)
    wg = torch.randn(D, hidden, generator=g) / math.sqrt(hidden)
    lw = 1.0 + 0.1 * torch.randn(D, generator=g)
    lb = 0.1 * torch.randn(D, generator=g)
    ww = torch.randn(H, hidden, generator=g) / math.sqrt(hidden)
    bf = lambda t: t.to(torch.bfloat16).contiguous()
    return ProjInputs(x=bf(x), qr=bf(qr), wq_b=bf(wq_b), wk=bf(wk),
                      k_norm_weight=lw.float().contiguous(), k_norm_bias=lb.float().contiguous(),
                      wg=bf(wg), ww=ww.float().contiguous(), H=H, D=D)


@dataclass
class MlaInputs:
    """CPU tensors of one sparse-attention call over listed token rows."""
    q: torch.Tensor           # bf16 [T, H, d]
    kv: torch.Tensor          # bf16 [N, d] (one latent row per token)
    indices: torch.Tensor     # int32 [T, width]; -1 and ids >= N are unused entries


def make_mla_inputs(T: int, H: int, N: int, width: int, d: int = 512, seed: int = 0,
                    causal: bool = True, unused_frac: float = 0.1, out_of_range_frac: float = 0.0,
                    pad_rows_frac: float = 0.25, q_scale: float = 1.0) -> MlaInputs:
    """Seeded inputs: q ~ q_scale * N(0, 1), kv ~ N(0, 1), both cast to BF16
    (round to nearest even). Row t lists `width` ids drawn uniformly with
    replacement from [0, min(N, t + 1)) (causal) or [0, N), so repeats occur;
    then a fraction `unused_frac` of the entries become -1, a fraction
    `out_of_range_frac` become ids in [N, 2N), and a fraction `pad_rows_frac`
    of the rows keep only a random-length prefix (the rest -1, the way an
    indexer pads its rows). Draw order: q, kv, ids, unused mask, out-of-range
    mask and ids, padded-row mask, prefix lengths."""
    g = torch.Generator().manual_seed(seed)
    q = q_scale * torch.randn(T, H, d, generator=g)
    kv = torch.randn(N, d, generator=g)
    hi = torch.clamp(torch.arange(T) + 1, max=N) if causal else torch.full((T,), N)
    ids = (torch.rand(T, width, generator=g) * hi[:, None]).floor().to(torch.int64)
    unused = torch.rand(T, width, generator=g) < unused_frac
    oor = torch.rand(T, width, generator=g) < out_of_range_frac
    oor_ids = N + (torch.rand(T, width, generator=g) * N).floor().to(torch.int64)
    ids = torch.where(oor, oor_ids, ids)
    ids[unused] = -1
    padded = torch.rand(T, generator=g) < pad_rows_frac
    keep = (torch.rand(T, generator=g) * (width + 1)).floor().to(torch.int64)
    col = torch.arange(width)[None, :]
    ids[padded[:, None] & (col >= keep[:, None])] = -1
    return MlaInputs(q=q.to(torch.bfloat16).contiguous(), kv=kv.to(torch.bfloat16).contiguous(),
                     indices=ids.to(torch.int32).contiguous())


def make_mla_inputs_device(T: int, H: int, N: int, width: int, device, d: int = 512,
                           seed: int = 0) -> MlaInputs:
    """Large sparse-attention inputs drawn directly on `device` with a seeded
    device generator (torch's Philox): q, kv ~ N(0, 1) cast to BF16; row t
    lists `width` ids drawn uniformly with replacement from [0, min(N, t+1)),
    the last `width // 8` entries of every fourth row set to -1. Draw order:
    q, kv, ids."""
    g = torch.Generator(device=device).manual_seed(seed)
    q = torch.randn(T, H, d, generator=g, device=device).to(torch.bfloat16)
    kv = torch.randn(N, d, generator=g, device=device).to(torch.bfloat16)
    hi = torch.clamp(torch.arange(T, device=device) + 1, max=N)
    ids = (torch.rand(T, width, generator=g, device=device) * hi[:, None]).floor().to(torch.int32)
    ids[::4, width - width // 8:] = -1
    return MlaInputs(q=q.contiguous(), kv=kv.contiguous(), indices=ids.contiguous())
