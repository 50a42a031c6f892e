"""shared_kv_decode_noalloc (static scratch, no allocation) against shared_kv_decode.

Two calls in a row through the C ABI, the second smaller (fewer sessions, shorter
contexts, fewer decoders) so it runs on a scratch array whose contents the first
call left behind.  Each must return shared_kv_decode's bits on the same inputs
(same kernels, same work split), and match the float64 oracle within the
attention tolerance.
"""
import math

import numpy as np
import pytest

import oracle
from cross_model_shared_amd import binding
from tests import gpu_util as gu

TOL = 2e-2


def _both(case):
    import torch

    B, N, Hq, D = case["q"].shape
    msl = max(max(case["lens"]), 1)
    scale = 1.0 / math.sqrt(D)
    q, bt, lens = gu.dev_bf16(case["q"]), gu.dev_i32(case["bt"]), gu.dev_i32(case["lens"])
    ws = gu.nan_workspace(binding.decode_workspace_bytes(B, N, Hq, case["Hkv"], D, msl))
    ref = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device="cuda")
    got = torch.empty_like(ref)
    binding.decode(case["pool"], 0, q, ref, bt, lens, msl, scale, ws, dev_status=case["status"])
    binding.decode_noalloc(case["pool"], 0, q, got, bt, lens, msl, scale, dev_status=case["status"])
    gu.sync()
    return ref, got


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    big = gu.make_decode_case([5000, 17, 3001, 0, 1, 2048, 777, 4096], 8, 4, 4, 128, seed=901,
                              poison=gu.POISON_NAN)
    small = gu.make_decode_case([300, 16, 65], 2, 4, 4, 128, seed=902, poison=gu.POISON_NAN)
    for case in (big, small):
        ref, got = _both(case)
        assert np.array_equal(gu.host_bits(got), gu.host_bits(ref)), "noalloc differs from shared_kv_decode"
        want = oracle.decode_from_logical(case["q"], case["K"], case["V"], 1.0 / math.sqrt(case["D"]))
        assert float(np.max(np.abs(gu.host_f64(got) - want))) <= TOL
        assert int(case["status"].item()) == 0
