"""GPU parity of shared_kv_decode_private (shared prefix + decoder-private
suffixes, PrefillShare section 3.3 / Eq. 9) against the CPU oracle.

Bars: outputs within 2e-2 max-abs of the float64 oracle (compared in fp32); with
no suffixes the call reproduces shared_kv_decode bit for bit; bad device values
are reported without faults.  Unused and spare pages hold NaN.
"""
import math

import numpy as np
import pytest

import oracle
from cross_model_shared_amd import binding
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def oracle_from_logical(case):
    """Per (session, decoder): attention over prefix ++ suffix, from the logical arrays."""
    B, N = len(case["lens"]), case["N"]
    out = np.zeros(case["q"].shape, np.float64)
    for b in range(B):
        for n in range(N):
            K = np.concatenate([case["K"][b], case["Kp"][b * N + n]])
            V = np.concatenate([case["V"][b], case["Vp"][b * N + n]])
            out[b, n:n + 1] = oracle.decode_from_logical(case["q"][b:b + 1, n:n + 1], [K], [V],
                                                         1.0 / math.sqrt(case["D"]))[0]
    return out


@pytest.mark.parametrize("lens,N,G,D,pmax", [
    ([37, 0, 130], 2, 4, 64, 70),       # an empty prefix, empty suffixes
    ([300, 17, 1000, 64], 8, 4, 128, 100),
    ([555, 2], 1, 5, 128, 300),
    ([129, 900], 16, 4, 64, 40),         # 64 rows per KV head
    ([2000, 48, 700], 3, 1, 128, 1200),
])
def test_private_decode_matches_oracle(lens, N, G, D, pmax):
    rng = np.random.default_rng(len(lens) * 100 + N + D)
    priv = [int(x) for x in rng.integers(0, pmax, size=len(lens) * N, endpoint=True)]
    priv[0] = 0
    print(f"[private] lens={lens} N={N} G={G} D={D} priv={priv}", flush=True)
    case = gu.make_private_case(lens, priv, N, 2, G, D, seed=len(lens) + N + D)
    out = gu.run_decode_private(case)
    want = oracle_from_logical(case)
    err = float(np.max(np.abs(gu.host_f64(out) - want)))
    print(f"[private] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(case["status"].item()) == 0


@pytest.mark.parametrize("lens,N,G,D,pmax", [
    ([300, 17, 900], 16, 8, 128, 60),    # 128 rows per KV head: two 64-row groups
    ([555, 0, 130], 20, 4, 64, 40),      # 80 rows: a full and a partial row group
    ([1000, 48], 5, 16, 128, 200),       # 80 rows, decoder 4 split over both row groups
])
def test_private_decode_above_64_rows_matches_oracle(lens, N, G, D, pmax):
    """More than 64 query rows per KV head run in 64-row groups; each group walks
    the session's private pages and attends those of its own decoders."""
    rng = np.random.default_rng(len(lens) * 1000 + N * G + D)
    priv = [int(x) for x in rng.integers(0, pmax, size=len(lens) * N, endpoint=True)]
    priv[1] = 0
    print(f"[private>64] lens={lens} N={N} G={G} D={D}", flush=True)
    case = gu.make_private_case(lens, priv, N, 1, G, D, seed=N * G + D)
    out = gu.run_decode_private(case)
    want = oracle_from_logical(case)
    err = float(np.max(np.abs(gu.host_f64(out) - want)))
    print(f"[private>64] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(case["status"].item()) == 0
    # without suffixes it is the plain decode, bit for bit
    nopriv = [0] * len(priv)
    a = gu.host_bits(gu.run_decode_private(case, priv=nopriv, max_priv_len=0))
    b = gu.host_bits(gu.run_decode(dict(pool=case["pool"], Hkv=1, layer=0, status=case["status"]),
                                   q_bits=case["q"], lens=lens, bt=case["bt"]))
    assert np.array_equal(a, b)


def test_private_decode_pool_path_matches_oracle_pool_path():
    """The oracle's own pool walk (both block tables) on the pool the GPU built."""
    lens, priv, N = [45, 210], [3, 0, 17, 64], 2
    case = gu.make_private_case(lens, priv, N, 2, 4, 64, seed=11)
    out = gu.run_decode_private(case)
    shape = oracle.PoolShape(1, case["num_pages"], 2, 64)
    img = gu.pool_bits(case["pool"])
    want = oracle.decode_private(img, shape, 0, case["q"], case["bt"], lens, case["pbt"], priv, 0.125)
    assert float(np.max(np.abs(gu.host_f64(out) - want))) <= TOL


def test_no_suffixes_is_shared_decode_bit_exact():
    lens = [777, 1500, 64, 0]
    N = 4
    case = gu.make_private_case(lens, [0] * (len(lens) * N), N, 2, 4, 128, seed=12)
    priv_out = gu.host_bits(gu.run_decode_private(case))
    shared = gu.host_bits(gu.run_decode(dict(pool=case["pool"], Hkv=2, layer=0, status=case["status"]),
                                        q_bits=case["q"], lens=lens, bt=case["bt"]))
    assert np.array_equal(priv_out, shared)


def test_suffix_equals_decode_over_the_joined_sequence():
    """With page-aligned prefixes, decoder n's prefix pages followed by its suffix
    pages are one block-table row of a plain decode over L + U tokens."""
    lens, N, G, D = [512, 1024], 4, 4, 128
    rng = np.random.default_rng(13)
    priv = [int(x) for x in rng.integers(1, 400, size=len(lens) * N)]
    case = gu.make_private_case(lens, priv, N, 2, G, D, seed=13)
    out = gu.host_f64(gu.run_decode_private(case))
    for n in range(N):
        rows = [np.concatenate([case["bt"][b, :lens[b] // 16],
                                case["pbt"][b * N + n, :(priv[b * N + n] + 15) // 16]]) for b in range(2)]
        width = max(len(r) for r in rows)
        bt_n = np.full((2, width), -1, np.int32)
        for b, r in enumerate(rows):
            bt_n[b, :len(r)] = r
        joined = [lens[b] + priv[b * N + n] for b in range(2)]
        alone = gu.run_decode(dict(pool=case["pool"], Hkv=2, layer=0, status=case["status"]),
                              q_bits=case["q"][:, n:n + 1].copy(), lens=joined, bt=bt_n)
        assert float(np.max(np.abs(gu.host_f64(alone)[:, 0] - out[:, n]))) <= TOL


def test_private_rejects_bad_device_values_without_faulting():
    lens, priv, N = [100, 40], [20, 33, 0, 16], 2
    case = gu.make_private_case(lens, priv, N, 2, 4, 64, seed=14)
    pbt = case["pbt"].copy()
    pbt[1, 1] = case["num_pages"] + 7        # out-of-range private page id
    out = gu.run_decode_private(case, pbt=pbt)
    assert int(case["status"].item()) & binding.DEV_BAD_PAGE
    assert np.all(np.isfinite(gu.host_f64(out)[0, 0]))   # decoder 0 of session 0 does not read that page
    case["status"].zero_()
    bad = list(priv)
    bad[3] = 10_000                          # above max_priv_len
    gu.run_decode_private(case, priv=bad, max_priv_len=40)
    assert int(case["status"].item()) & binding.DEV_BAD_LEN
