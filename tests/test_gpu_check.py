"""The device-side check of the document offsets (kpool_check_cu_seqlens,
through the C ABI) on valid and broken cu_seqlens arrays: the violation bits
it reports equal the ones a host scan of the same array finds (Megatron-LM
PR #7054, section 3: pools restart at every document, so the offsets decide
every pool)."""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_kpool_amd as kp
import workloads as wlm
from gpu_common import DEV, log

pytestmark = pytest.mark.gpu


def host_bits(cu, T, max_seqlen):
    bits = 0
    if cu[0] != 0:
        bits |= kp.KPOOL_CU_FIRST_NOT_ZERO
    if cu[-1] != T:
        bits |= kp.KPOOL_CU_LAST_NOT_TOTAL
    d = np.diff(cu.astype(np.int64))
    if np.any(d < 0):
        bits |= kp.KPOOL_CU_DECREASING
    if np.any(d > max_seqlen):
        bits |= kp.KPOOL_CU_TOO_LONG
    return bits


def device_bits(cu, T, max_seqlen):
    cud = torch.from_numpy(np.ascontiguousarray(cu, dtype=np.int32)).to(DEV)
    flags = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    kp.kpool_check_cu_seqlens(cud, len(cu) - 1, T, max_seqlen, flags)
    torch.cuda.synchronize()
    return int(flags.item())


def test_valid_offsets_of_every_workload():
    for i in range(5):
        inp = wlm.make_inputs(wlm.workload(i), seed=0)
        cu = inp.cu_seqlens.numpy()
        assert device_bits(cu, inp.T, inp.max_seqlen) == 0, inp.wl.name


@pytest.mark.parametrize("case", ["first", "decreasing", "too_long", "last", "all", "many_docs"])
def test_broken_offsets_are_reported(case):
    r = np.random.default_rng(3)
    lens = r.integers(0, 50, size=3000)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T, ms = int(cu[-1]), int(lens.max())
    if case == "first":
        cu = cu + 1
    elif case == "decreasing":
        cu[1777] = cu[1776] - 1
    elif case == "too_long":
        ms = ms - 1
    elif case == "last":
        T = T + 1
    elif case == "all":
        cu = cu.copy()
        cu[0] = 5
        cu[2999] = cu[2998] - 3
        ms = 1
        T = T - 1
    elif case == "many_docs":
        cu[-2] = cu[-1] + 1          # the last two documents: decreasing, and the one before too long
    log(f"cu_seqlens check: {case}")
    assert device_bits(cu, T, ms) == host_bits(cu, T, ms) != 0
