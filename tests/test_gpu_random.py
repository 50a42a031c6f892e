"""Seeded random sweep of shapes and lengths for every attention entry point
(decode, the fused decode step, extend, private and cascade decode)
against the float64 oracle (2e-2 max-abs).  Lengths mix the page-boundary cases
(0, 1, 15, 16, 17, whole pages) with arbitrary ones; head dims 64 and 128; GQA
groups 1-6; decoders 1-12."""
import math

import numpy as np
import pytest

import oracle
from cross_model_shared_amd import binding
from cross_model_shared_amd import workload as wlmod
from tests import gpu_util as gu
from tests.test_gpu_cascade import make_case as make_cascade_case, run_cascade
from tests.test_gpu_decode_append import expected_pool, make_step_case, run_fused
from tests.test_gpu_parity import make_extend_case, run_extend

pytestmark = pytest.mark.gpu
TOL = 2e-2
SPECIAL = [0, 1, 15, 16, 17, 32, 48, 255, 256, 257]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def draw_len(rng, hi):
    return int(rng.choice(SPECIAL)) if rng.random() < 0.4 else int(rng.integers(0, hi))


@pytest.mark.parametrize("seed", range(12))
def test_random_decode(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.integers(1, 7))
    N = int(rng.integers(1, max(2, 96 // G) if G > 1 else 13))
    N = min(N, 12)
    B = int(rng.integers(1, 10))
    lens = [draw_len(rng, 700) for _ in range(B)]
    if max(lens) == 0:
        lens[0] = 1
    print(f"[random] decode seed={seed} D={D} Hkv={Hkv} G={G} N={N} lens={lens}", flush=True)
    c = gu.make_decode_case(lens, N, Hkv, G, D, seed=2000 + seed, poison=gu.POISON_NAN)
    out = gu.host_f64(gu.run_decode(c))
    want = oracle.decode_from_logical(c["q"], c["K"], c["V"], 1.0 / math.sqrt(D))
    err = float(np.max(np.abs(out - want)))
    print(f"[random] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(c["status"].item()) == 0


@pytest.mark.parametrize("seed", range(8))
def test_random_decode_append(seed):
    rng = np.random.default_rng(5000 + seed)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.integers(1, 7))
    N = min(int(rng.integers(1, 13)), max(1, 96 // G))
    B = int(rng.integers(1, 10))
    lens = [draw_len(rng, 700) for _ in range(B)]
    if max(lens) == 0:
        lens[0] = 1
    print(f"[random] decode_append seed={seed} D={D} Hkv={Hkv} G={G} N={N} lens={lens}", flush=True)
    c = make_step_case(lens, N, Hkv, G, D, seed=6000 + seed)
    out = gu.host_f64(run_fused(c))
    assert np.array_equal(gu.pool_bits(c["pool"]), expected_pool(c))
    want = oracle.decode_from_logical(c["q"], c["K"], c["V"], 1.0 / math.sqrt(D))
    err = float(np.max(np.abs(out - want)))
    print(f"[random] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(c["status"].item()) == 0


@pytest.mark.parametrize("seed", range(8))
def test_random_extend(seed):
    rng = np.random.default_rng(3000 + seed)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.integers(1, 7))
    B = int(rng.integers(1, 6))
    prefix = [draw_len(rng, 500) for _ in range(B)]
    new = [max(1, draw_len(rng, 200)) if rng.random() < 0.85 else 0 for _ in range(B)]
    if max(new) == 0:
        new[0] = 1
    print(f"[random] extend seed={seed} D={D} Hkv={Hkv} G={G} prefix={prefix} new={new}", flush=True)
    c = make_extend_case(prefix, new, Hkv, G, D, seed=4000 + seed)
    out = gu.host_f64(run_extend(c))
    err = 0.0
    for b in range(B):
        if new[b] == 0:
            continue
        want = oracle.extend_from_logical(c["q"][c["cu"][b]:c["cu"][b + 1]], c["fk"][b], c["fv"][b], prefix[b],
                                          list(range(new[b])), 1.0 / math.sqrt(D))
        err = max(err, float(np.max(np.abs(out[c["cu"][b]:c["cu"][b + 1]] - want))))
    print(f"[random] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(c["status"].item()) == 0


@pytest.mark.parametrize("seed", range(6))
def test_random_private_decode(seed):
    rng = np.random.default_rng(5000 + seed)
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.integers(1, 5))
    N = int(rng.integers(1, max(2, 64 // G)))
    N = min(N, 8)
    B = int(rng.integers(1, 5))
    lens = [draw_len(rng, 400) for _ in range(B)]
    priv = [draw_len(rng, 100) for _ in range(B * N)]
    if max(lens) + max(priv) == 0:
        lens[0] = 1
    print(f"[random] private seed={seed} D={D} Hkv={Hkv} G={G} N={N} lens={lens} priv={priv}", flush=True)
    c = gu.make_private_case(lens, priv, N, Hkv, G, D, seed=6000 + seed)
    out = gu.host_f64(gu.run_decode_private(c))
    K = [np.concatenate([c["K"][b], c["Kp"][b * N + n]]) for b in range(B) for n in range(N)]
    V = [np.concatenate([c["V"][b], c["Vp"][b * N + n]]) for b in range(B) for n in range(N)]
    qq = c["q"].reshape(B * N, 1, Hkv * G, D)
    want = oracle.decode_from_logical(qq, K, V, 1.0 / math.sqrt(D)).reshape(B, N, Hkv * G, D)
    err = float(np.max(np.abs(out - want)))
    print(f"[random] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(c["status"].item()) == 0


@pytest.mark.parametrize("seed", range(6))
def test_random_cascade(seed):
    rng = np.random.default_rng(7000 + seed)
    D = int(rng.choice([64, 128]))
    G = int(rng.integers(1, 6))
    N = int(rng.integers(1, max(2, 64 // G)))
    N = min(N, 10)
    groups = []
    for _ in range(int(rng.integers(1, 5))):
        pre = 16 * int(rng.integers(0, 20))
        groups.append((pre, [pre + draw_len(rng, 150) for _ in range(int(rng.integers(1, 6)))]))
    print(f"[random] cascade seed={seed} D={D} G={G} N={N} groups={groups}", flush=True)
    c = make_cascade_case(groups, N, 2, G, D, seed=8000 + seed)
    out = gu.host_f64(run_cascade(c))
    want = oracle.decode_from_logical(c["q"], c["K"], c["V"], 1.0 / math.sqrt(D))
    err = float(np.max(np.abs(out - want)))
    print(f"[random] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(c["status"].item()) == 0
