"""GPU parity of shared_kv_decode_append (the step's token appended and attended in one call).

The call must leave the pool exactly as kv_pool_append of one row per session
would (position seq_lens[b] - 1), and return what shared_kv_decode over
seq_lens[b] tokens returns after that append: bit for bit against the two-call
path, within 2e-2 of the float64 oracle.  The slot that receives each token
holds NaN before the call, so a page read that missed the new token would
poison the output.
"""
import math

import numpy as np
import pytest

import oracle
from cross_model_shared_amd import binding
from cross_model_shared_amd import workload as wlmod
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def make_step_case(lens, N, Hkv, G, D, seed, layers=1, layer=0):
    """Pool holding each session's first L-1 tokens (NaN elsewhere), the step's
    token of each session, and queries.  lens: tokens attended, counting the new one."""
    rng = np.random.default_rng(seed)
    bt, num_pages = wlmod.build_block_table(lens, seed, spare_frac=0.05)
    K = [wlmod.draw_bf16(rng, (L, Hkv, D), 1.0) for L in lens]
    V = [wlmod.draw_bf16(rng, (L, Hkv, D), 1.0) for L in lens]
    # the step's token: row L-1 of each session (random bits for empty sessions,
    # which must not be written)
    k_tok = np.stack([K[b][-1] if L else wlmod.draw_bf16(rng, (Hkv, D), 1.0) for b, L in enumerate(lens)])
    v_tok = np.stack([V[b][-1] if L else wlmod.draw_bf16(rng, (Hkv, D), 1.0) for b, L in enumerate(lens)])
    q = wlmod.draw_bf16(rng, (len(lens), N, Hkv * G, D), 1.0)
    before = [max(L - 1, 0) for L in lens]
    kk, cu = wlmod.concat_rows([K[b][:before[b]] for b in range(len(lens))])
    vv, _ = wlmod.concat_rows([V[b][:before[b]] for b in range(len(lens))])
    nan = np.int16(np.uint16(gu.POISON_NAN).view(np.int16))
    pool = binding.Pool(layers, num_pages, Hkv, D, fill=nan)
    st = gu.status_tensor()
    if kk.shape[0]:
        binding.append(pool, layer, gu.dev_bf16(kk), gu.dev_bf16(vv), gu.dev_i32(cu), gu.dev_i32(bt),
                       gu.dev_i32(np.zeros(len(lens))), max_new=max(max(before), 1),
                       max_seq_len=max(max(lens), 1), dev_status=st)
    gu.sync()
    return dict(lens=list(lens), N=N, Hkv=Hkv, G=G, D=D, bt=bt, num_pages=num_pages, K=K, V=V, q=q,
                k_tok=k_tok, v_tok=v_tok, pool=pool, status=st, layers=layers, layer=layer, before=before)


def run_fused(case, pool=None, status=None):
    import torch

    pool = case["pool"] if pool is None else pool
    status = case["status"] if status is None else status
    B, N, Hq, D = case["q"].shape
    msl = max(max(case["lens"]), 1)
    ws = gu.nan_workspace(binding.decode_workspace_bytes(B, N, Hq, case["Hkv"], D, msl))
    out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device="cuda")
    binding.decode_append(pool, case["layer"], gu.dev_bf16(case["k_tok"]), gu.dev_bf16(case["v_tok"]),
                          gu.dev_bf16(case["q"]), out, gu.dev_i32(case["bt"]), gu.dev_i32(case["lens"]), msl,
                          1.0 / math.sqrt(D), ws, dev_status=status)
    gu.sync()
    return out


def expected_pool(case, sessions=None):
    """Pool image after the step: the first L-1 tokens, then every listed session's new token."""
    B = len(case["lens"])
    sessions = [b for b in range(B) if case["lens"][b] > 0] if sessions is None else sessions
    shape = oracle.PoolShape(case["layers"], case["num_pages"], case["Hkv"], case["D"])
    base = np.full(shape.elems, gu.POISON_NAN, np.uint16)
    kk, cu = wlmod.concat_rows([case["K"][b][:case["before"][b]] for b in range(B)])
    vv, _ = wlmod.concat_rows([case["V"][b][:case["before"][b]] for b in range(B)])
    img = oracle.append(base, shape, case["layer"], kk, vv, cu, case["bt"], np.zeros(B, np.int32))
    rows = [1 if b in sessions else 0 for b in range(B)]
    cu1 = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    sel = [b for b in range(B) if rows[b]]
    return oracle.append(img, shape, case["layer"], case["k_tok"][sel], case["v_tok"][sel], cu1, case["bt"],
                         case["before"])


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N,G", [(8, 4), (2, 5), (16, 6)])
def test_decode_append_matches_oracle_and_two_call_path(D, N, G):
    """New tokens at slot 0 of a new page, mid-page and at slot 15; an empty
    session; (16, 6) has 96 rows per KV head, two row groups reading one page."""
    import torch

    lens = [1, 16, 17, 200, 0, 256, 1000, 33]
    case = make_step_case(lens, N, 2, G, D, seed=31 * N + G + D)
    out = run_fused(case)
    assert int(case["status"].item()) == 0
    got_pool = gu.pool_bits(case["pool"])
    assert np.array_equal(got_pool, expected_pool(case))
    want = oracle.decode_from_logical(case["q"], case["K"], case["V"], 1.0 / math.sqrt(D))
    assert float(np.max(np.abs(gu.host_f64(out) - want))) <= TOL
    # the two-call path on a fresh copy of the starting pool: identical bits
    ref = make_step_case(lens, N, 2, G, D, seed=31 * N + G + D)
    B = len(lens)
    rows = [1 if L else 0 for L in lens]
    cu1 = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    sel = [b for b in range(B) if rows[b]]
    binding.append(ref["pool"], 0, gu.dev_bf16(ref["k_tok"][sel]), gu.dev_bf16(ref["v_tok"][sel]),
                   gu.dev_i32(cu1), gu.dev_i32(ref["bt"]), gu.dev_i32(ref["before"]), max_new=1,
                   max_seq_len=max(lens), dev_status=ref["status"])
    out2 = gu.run_decode(ref)
    assert np.array_equal(gu.pool_bits(ref["pool"]), got_pool)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_decode_append_single_token_returns_v_exactly():
    lens = [1, 1, 0]
    case = make_step_case(lens, 3, 2, 4, 128, seed=8)
    out = gu.host_bits(run_fused(case))
    G = 4
    for b, L in enumerate(lens):
        for h in range(8):
            want = case["v_tok"][b, h // G] if L else np.zeros(128, np.uint16)
            assert np.array_equal(out[b, :, h], np.broadcast_to(want, out[b, :, h].shape)), (b, h)
    assert np.array_equal(gu.pool_bits(case["pool"]), expected_pool(case))


def test_decode_append_consecutive_steps():
    """Three decode steps in a row, each appending its token and attending it, on layer 1 of 2."""
    D, N, G, Hkv = 128, 4, 4, 2
    final = [40, 16, 300, 3]
    case = make_step_case(final, N, Hkv, G, D, seed=12, layers=2, layer=1)
    # rewind: the pool holds the first L-3 tokens; write them back step by step
    B = len(final)
    nan = np.int16(np.uint16(gu.POISON_NAN).view(np.int16))
    pool = binding.Pool(2, case["num_pages"], Hkv, D, fill=nan)
    start = [L - 3 for L in final]
    kk, cu = wlmod.concat_rows([case["K"][b][:start[b]] for b in range(B)])
    vv, _ = wlmod.concat_rows([case["V"][b][:start[b]] for b in range(B)])
    st = gu.status_tensor()
    binding.append(pool, 1, gu.dev_bf16(kk), gu.dev_bf16(vv), gu.dev_i32(cu), gu.dev_i32(case["bt"]),
                   gu.dev_i32(np.zeros(B)), max_new=max(start), max_seq_len=max(final), dev_status=st)
    for step in range(3):
        lens = [s + step + 1 for s in start]
        sub = dict(case, lens=lens, k_tok=np.stack([case["K"][b][lens[b] - 1] for b in range(B)]),
                   v_tok=np.stack([case["V"][b][lens[b] - 1] for b in range(B)]))
        out = run_fused(sub, pool=pool, status=st)
        want = oracle.decode_from_logical(case["q"], [case["K"][b][:lens[b]] for b in range(B)],
                                          [case["V"][b][:lens[b]] for b in range(B)], 1.0 / math.sqrt(D))
        assert float(np.max(np.abs(gu.host_f64(out) - want))) <= TOL, step
    assert int(st.item()) == 0
    assert np.array_equal(gu.pool_bits(pool), expected_pool(case))


def test_decode_append_bad_page_flags_and_skips_that_session():
    D = 128
    lens = [40, 70, 5]
    case = make_step_case(lens, 2, 2, 4, D, seed=21)
    bt = case["bt"].copy()
    bt[1, (lens[1] - 1) // 16] = case["num_pages"] + 7   # the new token's page id is out of range
    case_bad = dict(case, bt=bt)
    out = run_fused(case_bad)
    assert int(case["status"].item()) & 1
    # the other sessions' tokens are written, session 1's is not
    assert np.array_equal(gu.pool_bits(case["pool"]), expected_pool(case, sessions=[0, 2]))
    want = oracle.decode_from_logical(case["q"], case["K"], case["V"], 1.0 / math.sqrt(D))
    got = gu.host_f64(out)
    for b in (0, 2):
        assert float(np.max(np.abs(got[b] - want[b]))) <= TOL
