"""Decode at the batch limits, against the oracle.

Every workgroup of the decode kernels builds the per-session page prefix sum
with 256 threads, each over a run of ceil(B / 256) sessions; the cascade's plan
kernel walks the batch with 1024 threads.  These cases take both past one
session per thread: 300 sessions (runs of 2, the last one partial), 600 with
private suffixes (runs of 3), and the largest batch the library accepts (4096:
runs of 16), with short ragged lengths, empty sessions among them; the cascade
with 1500 sessions in groups of one to four.
"""
import math

import numpy as np
import pytest

import oracle
from cross_model_shared_amd import binding
from tests import gpu_util as gu
from tests.test_gpu_cascade import make_case as make_cascade_case, run_cascade
from tests.test_gpu_private import oracle_from_logical

pytestmark = pytest.mark.gpu
TOL = 2e-2
MAX_BATCH = 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


@pytest.mark.parametrize("B,hi,N,Hkv,G,D", [
    (300, 400, 3, 2, 2, 128),
    (MAX_BATCH, 48, 2, 1, 2, 64),
])
def test_decode_large_batches_match_oracle(B, hi, N, Hkv, G, D):
    rng = np.random.default_rng(B + hi)
    lens = [int(x) for x in rng.integers(0, hi + 1, size=B)]
    lens[0], lens[-1], lens[B // 2] = 0, hi, 1
    print(f"[limits] decode B={B} max len {hi} N={N} Hkv={Hkv} G={G} D={D}", flush=True)
    case = gu.make_decode_case(lens, N, Hkv, G, D, seed=B, poison=gu.POISON_NAN, spare_frac=0.01)
    out = gu.run_decode(case)
    want = oracle.decode_from_logical(case["q"], case["K"], case["V"], 1.0 / math.sqrt(D))
    err = float(np.max(np.abs(gu.host_f64(out) - want)))
    print(f"[limits] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(case["status"].item()) == 0


def test_decode_above_the_batch_limit_is_rejected():
    assert binding.decode_workspace_bytes(MAX_BATCH + 1, 1, 1, 1, 64, 16) == 0
    assert binding.decode_workspace_bytes(MAX_BATCH, 1, 1, 1, 64, 16) > 0


def test_private_decode_large_batch_matches_oracle():
    B, N = 600, 2
    rng = np.random.default_rng(17)
    lens = [int(x) for x in rng.integers(0, 60, size=B)]
    priv = [int(x) for x in rng.integers(0, 40, size=B * N)]
    print(f"[limits] private B={B} N={N}", flush=True)
    case = gu.make_private_case(lens, priv, N, 1, 2, 64, seed=18)
    out = gu.run_decode_private(case)
    want = oracle_from_logical(case)
    err = float(np.max(np.abs(gu.host_f64(out) - want)))
    print(f"[limits] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(case["status"].item()) == 0


def test_cascade_large_batch_matches_oracle():
    rng = np.random.default_rng(19)
    groups, total = [], 0
    while total < 1500:
        pre = 16 * int(rng.integers(0, 4))
        n = min(int(rng.integers(1, 5)), 1500 - total)
        groups.append((pre, [pre + int(rng.integers(0, 40)) for _ in range(n)]))
        total += n
    print(f"[limits] cascade {total} sessions in {len(groups)} groups", flush=True)
    c = make_cascade_case(groups, 2, 1, 2, 64, seed=20)
    out = gu.host_f64(run_cascade(c))
    want = oracle.decode_from_logical(c["q"], c["K"], c["V"], 1.0 / math.sqrt(64))
    err = float(np.max(np.abs(out - want)))
    print(f"[limits] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(c["status"].item()) == 0
