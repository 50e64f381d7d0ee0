"""The C ABI on the CPU: the library loads, exports every entry point that
include/kpool.h declares, sizes its workspace, and rejects bad arguments
before touching the GPU (every call here fails validation, so no HIP call is
made)."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_attention_indexer_kpool_amd as kp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    with open(os.path.join(ROOT, "include", "kpool.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^[a-z_0-9 \*]+?\b(kpool_[a-z_0-9]+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "kpool_indexer_topk" in names and "kpool_compress" in names
    lib = kp.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(kp.EXPORTS) == names
    assert kp.kpool_abi_version() == 1


def P(**kw):
    base = dict(num_docs=1, total_tokens=65536, max_seqlen=65536, num_heads=32, head_dim=128,
                kpool=4, index_topk=2048, always_select_tail=1, use_fp8=0, query_chunk=4096)
    base.update(kw)
    return kp.Params(**base)


def test_workspace_and_ld():
    p = P()
    ld = kp.kpool_logits_ld(p)
    assert ld == 16384
    ws = kp.kpool_workspace_bytes(p)
    assert ws >= 4096 * 16384 * 4
    p8 = P(use_fp8=1, total_tokens=32768, max_seqlen=32768)
    ws8 = kp.kpool_workspace_bytes(p8)
    assert ws8 >= 4096 * 8192 * 4 + 32768 * 32 * (128 + 4) + 8192 * 132
    # the fused entry point: no tile; FP8 codes and scales only
    assert kp.kpool_fused_max_ksel(p) == 1184
    assert kp.kpool_fused_max_ksel(p8) == 1344
    assert kp.kpool_fused_max_ksel(P(num_heads=4, head_dim=128)) == 0
    assert kp.kpool_fused_max_ksel(P(num_heads=12)) == 0
    assert kp.kpool_fused_workspace_bytes(p) == 0
    assert kp.kpool_fused_workspace_bytes(p8) == 32768 * 32 * (128 + 4) + 8192 * 132
    assert kp.kpool_fused_workspace_bytes(P(index_topk=4 * 1185)) == 0
    assert kp.kpool_logits_ld(P(max_seqlen=4097, total_tokens=5000)) == 1024
    assert kp.kpool_logits_ld(P(max_seqlen=4100, total_tokens=5000)) == 1088
    assert kp.kpool_workspace_bytes(P(total_tokens=0, max_seqlen=0)) == 0
    # rows per logits tile: query_chunk when set, else what fits 256 MiB
    assert kp.kpool_query_chunk_rows(P()) == 4096
    assert kp.kpool_query_chunk_rows(P(query_chunk=0)) == 4096          # 16384 pools
    assert kp.kpool_query_chunk_rows(P(query_chunk=0, total_tokens=32768, max_seqlen=32768)) == 8192
    assert kp.kpool_query_chunk_rows(P(query_chunk=0, total_tokens=19679, max_seqlen=3789)) == 19679
    assert kp.kpool_query_chunk_rows(P(query_chunk=333)) == 333
    assert kp.kpool_query_chunk_rows(P(query_chunk=10 ** 6)) == 65536   # capped at T
    assert kp.kpool_query_chunk_rows(P(total_tokens=0, max_seqlen=0)) == 0
    assert kp.kpool_workspace_bytes(P(num_heads=4, query_chunk=0, total_tokens=19679,
                                      max_seqlen=3789)) >= 19679 * 960 * 4
    # unsupported or invalid parameters size to 0
    assert kp.kpool_workspace_bytes(P(num_heads=12)) == 0
    assert kp.kpool_workspace_bytes(P(max_seqlen=70000)) == 0


def _check_plan(p):
    """Every query row in exactly one range of one launch; each range's row
    stride a multiple of 64 holding its rows' causal pools; the two ranges of
    a launch fit the tile together; the first range has the longer rows."""
    launches = kp.kpool_indexer_launches(p)
    T, qc, ld = p.total_tokens, kp.kpool_query_chunk_rows(p), kp.kpool_logits_ld(p)
    seen = np.zeros(T, np.int32)
    for a0, a1, lda, b0, b1, ldb in launches:
        assert 0 <= a0 < a1 <= T and a0 % qc == 0 and (a1 - a0 == qc or a1 == T)
        assert lda % 64 == 0 and lda >= min(p.max_seqlen // p.kpool, a1 // p.kpool)
        seen[a0:a1] += 1
        used = (a1 - a0) * lda
        if b1 > b0:
            assert 0 <= b0 < b1 <= T and b0 % qc == 0 and b0 < a0
            assert ldb % 64 == 0 and ldb >= min(p.max_seqlen // p.kpool, b1 // p.kpool)
            assert ldb <= lda
            seen[b0:b1] += 1
            used += (b1 - b0) * ldb
        else:
            assert b0 == b1 == 0 and ldb == 0
        assert used <= qc * ld
    assert np.all(seen == 1)
    return launches


def test_indexer_launch_plan():
    # 64K, 4096-row chunks: the last chunk alone, then seven pairs (chunk
    # 14 - i with chunk i), then chunk 7 alone
    L = _check_plan(P())
    assert len(L) == 9
    assert L[0] == (61440, 65536, 16384, 0, 0, 0)
    assert L[1] == (57344, 61440, 15360, 0, 4096, 1024)
    assert L[7] == (32768, 36864, 9216, 24576, 28672, 7168)
    assert L[8] == (28672, 32768, 8192, 0, 0, 0)
    assert len(_check_plan(P(use_fp8=1, total_tokens=32768, max_seqlen=32768))) == 5
    # one chunk: one launch; a ragged last chunk; short documents; kpool 3
    _check_plan(P(query_chunk=0))
    assert len(_check_plan(P(total_tokens=4096, max_seqlen=4096, query_chunk=0))) == 1
    _check_plan(P(total_tokens=20011, max_seqlen=20011, query_chunk=1500))
    _check_plan(P(num_docs=8, total_tokens=19679, max_seqlen=3789, query_chunk=1000))
    _check_plan(P(total_tokens=9001, max_seqlen=9001, kpool=3, index_topk=96, query_chunk=333))
    _check_plan(P(total_tokens=5, max_seqlen=5, kpool=8, index_topk=64, query_chunk=2))
    assert kp.kpool_indexer_launches(P(total_tokens=0, max_seqlen=0)) == []
    assert kp.kpool_indexer_launches(P(num_heads=12)) == []


def raw(name, *args):
    assert _no_gpu_visible()
    L = kp.lib()
    st = getattr(L, name)(*args)
    assert st not in (kp.KPOOL_OK, kp.KPOOL_E_LAUNCH), f"{name} passed validation: {kp.kpool_last_error()}"
    return st


def pref(p):
    return ctypes.byref(p.c())


FAKE = 1 << 20          # a 16-byte aligned non-null value never dereferenced: validation fails first


def _no_gpu_visible():
    import torch
    return torch.cuda.device_count() == 0


# Raw calls with fake pointers must never reach a launch; they only run where
# no GPU is visible, so a wrong expectation can never touch a device.
raw_calls = pytest.mark.skipif(not _no_gpu_visible(), reason="fake-pointer calls run only without a GPU")


@raw_calls
@pytest.mark.parametrize("p,status,msg", [
    (P(num_heads=12), kp.KPOOL_E_UNSUPPORTED, "num_heads"),
    (P(head_dim=96), kp.KPOOL_E_UNSUPPORTED, "head_dim"),
    (P(kpool=0), kp.KPOOL_E_UNSUPPORTED, "kpool"),
    (P(index_topk=2), kp.KPOOL_E_INVALID, "index_topk"),
    (P(use_fp8=1, head_dim=64), kp.KPOOL_E_UNSUPPORTED, "FP8"),
    (P(max_seqlen=262148, total_tokens=262148), kp.KPOOL_E_UNSUPPORTED, "pools"),
    (P(max_seqlen=10, total_tokens=5), kp.KPOOL_E_INVALID, "max_seqlen"),
    (P(num_docs=0), kp.KPOOL_E_INVALID, "num_docs"),
    (P(query_chunk=-1), kp.KPOOL_E_INVALID, "query_chunk"),
    (P(always_select_tail=2), kp.KPOOL_E_INVALID, "always_select_tail"),
])
def test_indexer_rejects_bad_params(p, status, msg):
    st = raw("kpool_indexer_topk", pref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, FAKE, None, None)
    assert st == status
    assert msg in kp.kpool_last_error()


@raw_calls
def test_pointer_checks():
    p = P()
    ws = kp.kpool_workspace_bytes(p)
    # null q
    assert raw("kpool_indexer_topk", pref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, ws, FAKE, None, None) == kp.KPOOL_E_INVALID
    assert "q is null" in kp.kpool_last_error()
    # misaligned output
    assert raw("kpool_indexer_topk", pref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, FAKE + 4, None, None) == kp.KPOOL_E_INVALID
    assert "out_token_idx" in kp.kpool_last_error()
    # workspace too small / misaligned / null
    assert raw("kpool_indexer_topk", pref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, FAKE, None, None) == kp.KPOOL_E_WORKSPACE
    assert raw("kpool_indexer_topk", pref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, ws, FAKE, None, None) == kp.KPOOL_E_INVALID
    assert raw("kpool_indexer_topk", pref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, ws, FAKE, None, None) == kp.KPOOL_E_INVALID
    assert "workspace is null" in kp.kpool_last_error()
    # the fused entry point: a K_sel beyond its list is refused first
    pbig = P(index_topk=4 * 1185)
    assert raw("kpool_indexer_topk_fused", pref(pbig), FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, None, None) == kp.KPOOL_E_UNSUPPORTED
    assert "fused" in kp.kpool_last_error()
    p8 = P(use_fp8=1, total_tokens=32768, max_seqlen=32768)
    ws8 = kp.kpool_fused_workspace_bytes(p8)
    assert raw("kpool_indexer_topk_fused", pref(p8), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws8 - 1, FAKE, None, None) == kp.KPOOL_E_WORKSPACE
    assert raw("kpool_indexer_topk_fused", pref(p), None, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, None, None) == kp.KPOOL_E_INVALID
    # compress: null keys
    assert raw("kpool_compress", pref(p), None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == kp.KPOOL_E_INVALID
    # logits: rows out of range
    assert raw("kpool_logits", pref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 5, 3, FAKE, ws, FAKE, 1, None) == kp.KPOOL_E_INVALID
    assert raw("kpool_logits", pref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 65537, FAKE, ws, FAKE, 1, None) == kp.KPOOL_E_INVALID
    assert raw("kpool_logits", pref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 16, FAKE, ws, FAKE, 8, None) == kp.KPOOL_E_INVALID
    # select / expand: null outputs
    assert raw("kpool_select", pref(p), FAKE, 0, 10, FAKE, FAKE, None, None) == kp.KPOOL_E_INVALID
    assert raw("kpool_expand", pref(p), FAKE, FAKE, FAKE, None, None) == kp.KPOOL_E_INVALID
    # fp8: negative rows, null codes
    assert raw("kpool_fp8_quantize", FAKE, -1, FAKE, FAKE, None) == kp.KPOOL_E_INVALID
    assert raw("kpool_fp8_quantize", FAKE, 4, None, FAKE, None) == kp.KPOOL_E_INVALID
    # null params
    assert raw("kpool_indexer_topk", None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, FAKE, None, None) == kp.KPOOL_E_INVALID


@raw_calls
def test_staged_indexer_checks():
    p = P()
    ws = kp.kpool_workspace_bytes(p)
    for i in (-1, 9, 1 << 30):
        assert raw("kpool_indexer_scoring", pref(p), i, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 0, None) == kp.KPOOL_E_INVALID
        assert "launch" in kp.kpool_last_error()
        assert raw("kpool_indexer_selection", pref(p), i, FAKE, FAKE, FAKE, ws, FAKE, None, None) == kp.KPOOL_E_INVALID
        assert "launch" in kp.kpool_last_error()
    # flags other than KPOOL_LOGITS_INPUTS_QUANTIZED
    for f in (kp.KPOOL_LOGITS_FILL_MASKED, kp.KPOOL_LOGITS_SKIP_ALL_SELECTED, 8):
        assert raw("kpool_indexer_scoring", pref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, f, None) == kp.KPOOL_E_INVALID
        assert "flags" in kp.kpool_last_error()
    # workspace too small, null or misaligned pointers
    assert raw("kpool_indexer_scoring", pref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws - 1, 0, None) == kp.KPOOL_E_WORKSPACE
    assert raw("kpool_indexer_scoring", pref(p), 0, None, FAKE, FAKE, FAKE, FAKE, FAKE, ws, 0, None) == kp.KPOOL_E_INVALID
    assert raw("kpool_indexer_selection", pref(p), 0, FAKE, FAKE, FAKE, ws - 1, FAKE, None, None) == kp.KPOOL_E_WORKSPACE
    assert raw("kpool_indexer_selection", pref(p), 0, FAKE, FAKE, FAKE, ws, FAKE + 4, None, None) == kp.KPOOL_E_INVALID
    assert "out_token_idx" in kp.kpool_last_error()
    assert raw("kpool_indexer_selection", pref(p), 0, FAKE, FAKE, FAKE + 16, ws, FAKE, None, None) == kp.KPOOL_E_INVALID
    # T = 0: no launches, so every index is out of range
    p0 = P(total_tokens=0, max_seqlen=0)
    assert raw("kpool_indexer_scoring", pref(p0), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, None) == kp.KPOOL_E_INVALID


@raw_calls
def test_alignment_rule_of_the_header():
    """The header's alignment rule: ape needs 16 bytes (it is read as 16-byte
    vectors), the int32 / FP32 arrays 4 bytes; a 4-byte-aligned array passes
    its own check and validation fails later, on the next argument."""
    p = P()
    # kpool_compress(p, k, gate, ape, cu_seqlens, cu_pools, pooled, stream)
    assert raw("kpool_compress", pref(p), FAKE, FAKE, FAKE + 4, FAKE, FAKE, FAKE, None) == kp.KPOOL_E_INVALID
    assert "ape is not 16-byte aligned" in kp.kpool_last_error()
    assert raw("kpool_compress", pref(p), FAKE, FAKE, FAKE + 8, FAKE, FAKE, FAKE, None) == kp.KPOOL_E_INVALID
    assert "ape" in kp.kpool_last_error()
    # cu_seqlens / cu_pools at 4-byte offsets pass; the misaligned pooled fails next
    assert raw("kpool_compress", pref(p), FAKE, FAKE, FAKE, FAKE + 4, FAKE + 4, FAKE + 4, None) == kp.KPOOL_E_INVALID
    assert "pooled is not 16-byte aligned" in kp.kpool_last_error()
    assert raw("kpool_compress", pref(p), FAKE, FAKE, FAKE, FAKE + 2, FAKE, FAKE, None) == kp.KPOOL_E_INVALID
    assert "cu_seqlens is not 4-byte aligned" in kp.kpool_last_error()
    # compress_pools: ape 16, dst_rows 4
    assert raw("kpool_compress_pools", pref(p), FAKE, FAKE, FAKE + 4, 4, FAKE, 10, FAKE, None, None) == kp.KPOOL_E_INVALID
    assert "ape is not 16-byte aligned" in kp.kpool_last_error()
    assert raw("kpool_compress_pools", pref(p), FAKE, FAKE, FAKE, 4, FAKE + 4, 10, FAKE + 4, None, None) == kp.KPOOL_E_INVALID
    assert "pooled is not 16-byte aligned" in kp.kpool_last_error()
    # the indexer: w at a 4-byte offset passes; a misaligned q fails
    ws = kp.kpool_workspace_bytes(p)
    assert raw("kpool_indexer_topk", pref(p), FAKE + 4, FAKE, FAKE, FAKE, FAKE, FAKE, ws, FAKE, None, None) == kp.KPOOL_E_INVALID
    assert "q is not 16-byte aligned" in kp.kpool_last_error()
    assert raw("kpool_indexer_topk", pref(p), FAKE, FAKE + 4, FAKE, FAKE + 4, FAKE + 4, FAKE, ws, FAKE + 8, None, None) == kp.KPOOL_E_INVALID
    assert "out_token_idx is not 16-byte aligned" in kp.kpool_last_error()


def test_decode_workspace():
    """Decode scores: one row of kpool_logits_ld floats per sequence; total
    tokens and the query chunk play no part; FP8 is refused."""
    p = P(num_docs=64, total_tokens=0, max_seqlen=65536)
    assert kp.kpool_decode_workspace_bytes(p) == 64 * 16384 * 4
    assert kp.kpool_decode_workspace_bytes(P(num_docs=3, max_seqlen=4100)) == 3 * 1088 * 4
    p8 = P(num_docs=64, total_tokens=0, max_seqlen=65536, use_fp8=1)
    assert kp.kpool_decode_workspace_bytes(p8) == 64 * 16384 * 4
    assert kp.kpool_decode_workspace_bytes(P(use_fp8=1, head_dim=64)) == 0
    assert kp.kpool_decode_workspace_bytes(P(num_docs=0)) == 0
    assert kp.kpool_decode_workspace_bytes(P(max_seqlen=262148)) == 0


@raw_calls
def test_decode_argument_checks():
    p = P(num_docs=8, max_seqlen=65536)
    ws = kp.kpool_decode_workspace_bytes(p)
    args = (FAKE, FAKE, FAKE, 100, None, FAKE, FAKE, None, FAKE, ws, FAKE, None, None)
    assert raw("kpool_decode_topk", pref(P(use_fp8=1, head_dim=64)), *args) == kp.KPOOL_E_UNSUPPORTED
    assert "FP8" in kp.kpool_last_error()
    p8 = P(num_docs=8, max_seqlen=65536, use_fp8=1)
    ws8 = kp.kpool_decode_workspace_bytes(p8)
    noscale = (FAKE, FAKE, FAKE, 100, None, FAKE, FAKE, None, FAKE, ws8, FAKE, None, None)
    assert raw("kpool_decode_topk", pref(p8), *noscale) == kp.KPOOL_E_INVALID
    assert "pooled_scale" in kp.kpool_last_error()
    assert raw("kpool_decode_topk", pref(P(num_heads=12)), *args) == kp.KPOOL_E_UNSUPPORTED
    small = (FAKE, FAKE, FAKE, 100, None, FAKE, FAKE, None, FAKE, ws - 1, FAKE, None, None)
    assert raw("kpool_decode_topk", pref(p), *small) == kp.KPOOL_E_WORKSPACE
    nolen = (FAKE, FAKE, FAKE, 100, None, FAKE, None, None, FAKE, ws, FAKE, None, None)
    assert raw("kpool_decode_topk", pref(p), *nolen) == kp.KPOOL_E_INVALID
    assert "seq_lens" in kp.kpool_last_error()
    badbase = (FAKE, FAKE, FAKE, 100, None, FAKE, FAKE, FAKE + 2, FAKE, ws, FAKE, None, None)
    assert raw("kpool_decode_topk", pref(p), *badbase) == kp.KPOOL_E_INVALID
    negrows = (FAKE, FAKE, FAKE, -1, None, FAKE, FAKE, None, FAKE, ws, FAKE, None, None)
    assert raw("kpool_decode_topk", pref(p), *negrows) == kp.KPOOL_E_INVALID
    assert raw("kpool_compress_pools", pref(p), FAKE, FAKE, FAKE, -1, FAKE, 10, FAKE, None, None) == kp.KPOOL_E_INVALID
    assert raw("kpool_compress_pools", pref(p), FAKE, FAKE, FAKE, 4, None, 10, FAKE, None, None) == kp.KPOOL_E_INVALID
    assert raw("kpool_compress_pools", pref(P(kpool=65)), FAKE, FAKE, FAKE, 4, FAKE, 10, FAKE, None, None) == kp.KPOOL_E_UNSUPPORTED
    assert raw("kpool_compress_pools", pref(P(use_fp8=1)), FAKE, FAKE, FAKE, 4, FAKE, 10, FAKE, None, None) == kp.KPOOL_E_INVALID
    assert raw("kpool_compress_pools", pref(P(use_fp8=1, head_dim=64)), FAKE, FAKE, FAKE, 4, FAKE, 10, FAKE, FAKE, None) == kp.KPOOL_E_UNSUPPORTED


def test_status_strings():
    assert kp.kpool_status_string(0) == "ok"
    assert kp.kpool_status_string(3) == "workspace too small"
    assert kp.kpool_status_string(99) == "unknown status"


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        kp.kpool_fp8_quantize(torch.zeros(4, 128, dtype=torch.bfloat16), 4,
                              torch.zeros(4, 128, dtype=torch.uint8), torch.zeros(4))


def test_header_constants_match_binding():
    """The #define constants of include/kpool.h equal the binding's."""
    import re
    hdr = open(os.path.join(os.path.dirname(__file__), "..", "include", "kpool.h")).read()
    defs = dict(re.findall(r"#define\s+(KPOOL_[A-Z_]+)\s+(\d+)", hdr))
    assert defs, "no constants found"
    for name, val in defs.items():
        if hasattr(kp, name):
            assert getattr(kp, name) == int(val), name
    for name in ("KPOOL_LOGITS_FILL_MASKED", "KPOOL_LOGITS_SKIP_ALL_SELECTED",
                 "KPOOL_LOGITS_INPUTS_QUANTIZED", "KPOOL_CU_FIRST_NOT_ZERO",
                 "KPOOL_CU_DECREASING", "KPOOL_CU_TOO_LONG", "KPOOL_CU_LAST_NOT_TOTAL"):
        assert getattr(kp, name) == int(defs[name]), name


def _mla(T=4, H=64, N=16, W=8, scale=0.0625, dqk=512, dv=512):
    return kp.MlaParams(num_tokens=T, num_heads=H, kv_rows=N, width=W, sm_scale=scale,
                        dim_qk=dqk, dim_v=dv)


@pytest.mark.parametrize("mp,status,msg", [
    (_mla(H=32), kp.KPOOL_E_UNSUPPORTED, "multiple of 64"),
    (_mla(H=0), kp.KPOOL_E_UNSUPPORTED, "multiple of 64"),
    (_mla(dqk=576), kp.KPOOL_E_UNSUPPORTED, "512"),
    (_mla(W=4097), kp.KPOOL_E_UNSUPPORTED, "4096"),
    (_mla(T=-1), kp.KPOOL_E_INVALID, ">= 0"),
    (_mla(N=-3), kp.KPOOL_E_INVALID, ">= 0"),
    (_mla(scale=float("inf")), kp.KPOOL_E_INVALID, "finite"),
    (_mla(scale=0.0), kp.KPOOL_E_INVALID, "> 0"),
    (_mla(scale=-0.5), kp.KPOOL_E_INVALID, "> 0"),
])
def test_sparse_mla_rejects_bad_params(mp, status, msg):
    """Shape and scale checks of kpool_sparse_mla_fwd come before any device
    work (the pointers here are fake host addresses never dereferenced)."""
    fake = 4096
    st = kp.lib().kpool_sparse_mla_fwd(ctypes.byref(mp.c()), fake, fake, fake, fake, fake, None)
    assert st == status
    assert msg in kp.kpool_last_error()


def test_sparse_mla_pointer_checks():
    """Null or misaligned pointers are refused; T = 0 needs none; kv and
    indices may be null when kv_rows or width is 0."""
    L = kp.lib()
    mp = _mla()
    ok = 4096
    for args, name in [((None, ok, ok, ok, ok), "q"), ((ok + 8, ok, ok, ok, ok), "q"),
                       ((ok, None, ok, ok, ok), "kv"), ((ok, ok, ok + 2, ok, ok), "indices"),
                       ((ok, ok, ok, ok + 4, ok), "out"), ((ok, ok, ok, ok, ok + 1), "lse")]:
        st = L.kpool_sparse_mla_fwd(ctypes.byref(mp.c()), *args, None)
        assert st == kp.KPOOL_E_INVALID and name in kp.kpool_last_error(), (args, name)
    assert L.kpool_sparse_mla_fwd(ctypes.byref(_mla(T=0).c()), None, None, None, None, None,
                                  None) == kp.KPOOL_OK


def test_check_cu_seqlens_argument_checks():
    """kpool_check_cu_seqlens refuses negative sizes and null or misaligned
    pointers before any launch (fake host addresses, never dereferenced)."""
    L = kp.lib()
    ok = 4096
    for args, msg in [((ok, -1, 8, 8, ok), ">= 0"), ((ok, 1, -8, 8, ok), ">= 0"),
                      ((ok, 1, 8, -1, ok), ">= 0"), ((None, 1, 8, 8, ok), "cu_seqlens"),
                      ((ok + 2, 1, 8, 8, ok), "cu_seqlens"), ((ok, 1, 8, 8, None), "flags_out"),
                      ((ok, 1, 8, 8, ok + 1), "flags_out")]:
        assert L.kpool_check_cu_seqlens(*args, None) == kp.KPOOL_E_INVALID, args
        assert msg in kp.kpool_last_error()
