"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: the pool image after kv_pool_append is bit-exact; attention outputs are
within 2e-2 max-abs of the float64 oracle, compared in fp32.  Invariants the
pages fix (ICaRus Key designs 2-3; PrefillShare sections 3.3-4) are checked on
the GPU results directly.
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


def oracle_pool(case):
    shape = oracle.PoolShape(case["layers"], case["num_pages"], case["Hkv"], case["D"])
    base = np.full(shape.elems, case["poison"], np.uint16)
    img = oracle.append(base, shape, case["layer"], case["kk"], case["vv"], case["cu"], case["bt"],
                        np.zeros(len(case["lens"]), np.int32))
    return shape, img


def max_err(gpu_out, want):
    return float(np.max(np.abs(gu.host_f64(gpu_out) - want))) if want.size else 0.0


# ---------------------------------------------------------------------------
# kv_pool_append
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("D", [64, 128])
def test_append_whole_pool_bit_exact(D):
    lens = [200, 256, 1, 47]
    case = gu.make_decode_case(lens, 1, 2, 1, D, seed=D)
    gu.sync()
    shape, img = oracle_pool(case)
    got = gu.pool_bits(case["pool"])
    assert got.shape == img.shape
    assert np.array_equal(got, img)
    assert int(case["status"].item()) == 0


def test_append_in_pieces_equals_one_shot_and_keeps_other_bytes():
    import torch

    rng = np.random.default_rng(3)
    lens, Hkv, D = [70, 33, 16], 2, 128
    bt, num_pages = wlmod.build_block_table(lens, 3)
    base = wlmod.draw_bf16(rng, (2 * num_pages * Hkv * 32 * D,), 1.0)  # 2 layers of random bytes
    K = [wlmod.draw_bf16(rng, (L, Hkv, D), 1.0) for L in lens]
    V = [wlmod.draw_bf16(rng, (L, Hkv, D), 1.0) for L in lens]
    pool = binding.Pool(2, num_pages, Hkv, D)
    pool.data.copy_(torch.from_numpy(base.view(np.int16)).cuda())
    cuts = [3, 17, 16]     # first call writes these many rows per session, unaligned starts after
    first, cu1 = wlmod.concat_rows([K[b][:cuts[b]] for b in range(3)])
    firstv, _ = wlmod.concat_rows([V[b][:cuts[b]] for b in range(3)])
    rest, cu2 = wlmod.concat_rows([K[b][cuts[b]:] for b in range(3)])
    restv, _ = wlmod.concat_rows([V[b][cuts[b]:] for b in range(3)])
    st = gu.status_tensor()
    binding.append(pool, 1, gu.dev_bf16(first), gu.dev_bf16(firstv), gu.dev_i32(cu1), gu.dev_i32(bt),
                   gu.dev_i32([0, 0, 0]), max_new=17, max_seq_len=70, dev_status=st)
    binding.append(pool, 1, gu.dev_bf16(rest), gu.dev_bf16(restv), gu.dev_i32(cu2), gu.dev_i32(bt),
                   gu.dev_i32(cuts), max_new=67, max_seq_len=70, dev_status=st)
    gu.sync()
    shape = oracle.PoolShape(2, num_pages, Hkv, D)
    kk, cu = wlmod.concat_rows(K)
    vv, _ = wlmod.concat_rows(V)
    want = oracle.append(base, shape, 1, kk, vv, cu, bt, np.zeros(3, np.int32))
    assert np.array_equal(gu.pool_bits(pool), want)
    assert int(st.item()) == 0


# ---------------------------------------------------------------------------
# shared_kv_decode
# ---------------------------------------------------------------------------
def test_tiny_workload_decode_matches_oracle():
    wl = wlmod.make_workload("tiny")
    case = gu.make_decode_case(wl.lens, wl.num_decoders, wl.num_kv_heads, wl.group, wl.head_dim,
                               seed=wl.seed, std=wl.std)
    out = gu.run_decode(case, scale=wl.scale)
    shape, img = oracle_pool(case)
    assert np.array_equal(gu.pool_bits(case["pool"]), img)
    want = oracle.decode(img, shape, 0, case["q"], case["bt"], wl.lens, wl.scale)
    assert max_err(out, want) <= TOL
    assert int(case["status"].item()) == 0


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N,G", [(1, 1), (2, 4), (8, 4), (2, 5), (5, 8), (16, 6)])
def test_decode_row_layouts_and_splits(D, N, G):
    """Row counts R = N*G of 1..96 (one or several row groups), ragged lengths with
    partial last pages, several splits per session."""
    lens = [1000, 3001, 17, 16, 5000]
    case = gu.make_decode_case(lens, N, 2, G, D, seed=N * 100 + G + D, poison=gu.POISON_NAN)
    out = gu.run_decode(case)
    want = oracle.decode_from_logical(case["q"], case["K"], case["V"], 1.0 / math.sqrt(D))
    assert max_err(out, want) <= TOL
    assert int(case["status"].item()) == 0


@pytest.mark.parametrize("B,Hkv,N,G,D", [
    (40, 4, 16, 6, 128),   # 320 units of 64-row groups (two per KV head)
    (48, 2, 8, 4, 64),     # 96 units
    (3, 2, 16, 6, 64),     # 12 units of 64 rows at D = 64: dozens of shares per unit
])
def test_decode_split_unit_merges(B, Hkv, N, G, D):
    """Units split over several waves' shares, merged by the last wave to finish each:
    many short units, and few long ones that span dozens of shares."""
    rng = np.random.default_rng(B * 7 + D)
    lens = [int(x) for x in rng.integers(1, 400, size=B)]
    lens[0], lens[-1] = 16, 399
    if B < 8:
        lens = [6000, 4100, 33][:B]
    case = gu.make_decode_case(lens, N, Hkv, G, D, seed=B + N + D, poison=gu.POISON_NAN)
    out = gu.run_decode(case)
    want = oracle.decode_from_logical(case["q"], case["K"], case["V"], 1.0 / math.sqrt(D))
    assert max_err(out, want) <= TOL
    assert int(case["status"].item()) == 0


@pytest.mark.parametrize("lens,Hkv,N,G,D", [
    ([100000], 1, 1, 1, 64),         # one unit over all 1024 shares: a 4-level merge tree
    ([70000, 3], 2, 2, 2, 128),      # two long units (3 levels), a short one inside one share
    ([5000], 1, 3, 1, 64),           # 313 tiles: most shares empty, empty children between full ones
    ([40, 17, 1], 1, 1, 4, 128),     # a handful of tiles spread over 1024 shares
])
def test_decode_merge_tree_depths(lens, Hkv, N, G, D):
    """Units split over many shares are merged by a tree of nodes of up to 8 children;
    trees of 1 to 4 levels, with children that hold no tiles, against the oracle."""
    case = gu.make_decode_case(lens, N, Hkv, G, D, seed=sum(lens) % 1000 + D, poison=gu.POISON_NAN)
    out = gu.run_decode(case)
    want = oracle.decode_from_logical(case["q"], case["K"], case["V"], 1.0 / math.sqrt(D))
    assert max_err(out, want) <= TOL
    assert int(case["status"].item()) == 0


def test_decode_workspace_counters_back_to_zero_across_shapes():
    """One workspace serves calls of different shapes in a row: every call finds its arrival
    counters at zero and leaves them so (the first 64 KiB read back as zero), and each
    result matches the oracle, with the rest of the workspace NaN-poisoned throughout."""
    import torch

    cases = [gu.make_decode_case([6000, 4100, 33], 16, 2, 6, 64, seed=71, poison=gu.POISON_NAN),
             gu.make_decode_case([1000, 17, 3001, 16, 2500], 2, 2, 4, 64, seed=72, poison=gu.POISON_NAN)]
    ws = gu.nan_workspace(max(binding.decode_workspace_bytes(len(c["lens"]), c["N"], c["Hkv"] * c["G"], c["Hkv"],
                                                             c["D"], max(c["lens"])) for c in cases))
    for c in cases + cases:
        B, N, Hq, D = c["q"].shape
        out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device="cuda")
        binding.decode(c["pool"], 0, gu.dev_bf16(c["q"]), out, gu.dev_i32(c["bt"]), gu.dev_i32(c["lens"]),
                       max(c["lens"]), 1.0 / math.sqrt(D), ws, dev_status=c["status"])
        gu.sync()
        want = oracle.decode_from_logical(c["q"], c["K"], c["V"], 1.0 / math.sqrt(D))
        assert max_err(out, want) <= TOL
        assert not ws[:65536].cpu().numpy().any(), "arrival counters left non-zero"
        assert int(c["status"].item()) == 0


def test_decode_single_token_returns_v_exactly_and_empty_is_zero():
    lens = [1, 0, 1]
    case = gu.make_decode_case(lens, 3, 2, 4, 128, seed=5, poison=gu.POISON_NAN)
    out = gu.host_bits(gu.run_decode(case))
    for b, L in enumerate(lens):
        for n in range(3):
            for h in range(8):
                if L == 1:
                    assert np.array_equal(out[b, n, h], case["V"][b][0, h // 4])
                else:
                    assert not out[b, n, h].any()


def test_decode_uniform_scores_give_mean_of_v():
    lens = [333, 2048]
    case = gu.make_decode_case(lens, 2, 2, 4, 128, seed=6)
    q0 = np.zeros_like(case["q"])
    out = gu.host_f64(gu.run_decode(case, q_bits=q0))
    for b, L in enumerate(lens):
        mean = oracle.bf16_to_f64(case["V"][b]).mean(axis=0)     # [Hkv, D]
        for h in range(8):
            assert np.max(np.abs(out[b, :, h] - mean[h // 4])) <= TOL


def test_decode_page_permutation_and_decoder_independence_bit_exact():
    import torch

    lens = [777, 1500, 64]
    N, Hkv, G, D = 4, 2, 4, 128
    case = gu.make_decode_case(lens, N, Hkv, G, D, seed=8)
    base = gu.host_bits(gu.run_decode(case))
    # each decoder alone over the same cache: identical bits
    for n in range(N):
        alone = gu.host_bits(gu.run_decode(case, q_bits=case["q"][:, n:n + 1].copy()))
        assert np.array_equal(alone[:, 0], base[:, n])
    # move every physical page to a new id and relabel the block table
    perm = np.random.default_rng(1).permutation(case["num_pages"])
    tile = Hkv * 32 * D
    old = case["pool"].data.view(-1, tile).clone()
    case["pool"].data.view(-1, tile)[torch.from_numpy(perm).cuda()] = old
    bt2 = np.where(case["bt"] >= 0, perm[np.maximum(case["bt"], 0)], -1).astype(np.int32)
    moved = gu.host_bits(gu.run_decode(case, bt=bt2))
    assert np.array_equal(moved, base)


def test_decode_rejects_bad_device_values_without_faulting():
    lens = [100, 40]
    case = gu.make_decode_case(lens, 2, 2, 4, 64, seed=9)
    bt = case["bt"].copy()
    bt[0, 2] = case["num_pages"] + 5          # out-of-range page id
    gu.run_decode(case, bt=bt)
    assert int(case["status"].item()) & binding.DEV_BAD_PAGE
    case["status"].zero_()
    gu.run_decode(case, lens=[100, 90], max_seq_len=64)   # a length above the host bound
    assert int(case["status"].item()) & binding.DEV_BAD_LEN


# ---------------------------------------------------------------------------
# partial_prefill_extend
# ---------------------------------------------------------------------------
def make_extend_case(prefix, new, Hkv, G, D, seed, poison=gu.POISON_NAN):
    rng = np.random.default_rng(seed)
    full = [p + c for p, c in zip(prefix, new)]
    fk = [wlmod.draw_bf16(rng, (L, Hkv, D), 1.0) for L in full]
    fv = [wlmod.draw_bf16(rng, (L, Hkv, D), 1.0) for L in full]
    bt, num_pages = wlmod.build_block_table(full, seed)
    pool = binding.Pool(1, num_pages, Hkv, D, fill=np.int16(np.uint16(poison).view(np.int16)))
    st = gu.status_tensor()
    kp, cup = wlmod.concat_rows([k[:p] for k, p in zip(fk, prefix)])
    vp, _ = wlmod.concat_rows([v[:p] for v, p in zip(fv, prefix)])
    if kp.shape[0]:
        binding.append(pool, 0, gu.dev_bf16(kp), gu.dev_bf16(vp), gu.dev_i32(cup), gu.dev_i32(bt),
                       gu.dev_i32(np.zeros(len(prefix))), max_new=max(max(prefix), 1),
                       max_seq_len=max(full), dev_status=st)
    kn, cu = wlmod.concat_rows([k[p:] for k, p in zip(fk, prefix)])
    vn, _ = wlmod.concat_rows([v[p:] for v, p in zip(fv, prefix)])
    q = wlmod.draw_bf16(rng, (int(cu[-1]), Hkv * G, D), 1.0)
    return dict(prefix=prefix, new=new, Hkv=Hkv, G=G, D=D, fk=fk, fv=fv, bt=bt, num_pages=num_pages,
                pool=pool, status=st, kn=kn, vn=vn, cu=cu, q=q, poison=poison)


def run_extend(c, q=None, kn=None, vn=None, cu=None, prefix=None):
    import torch

    q = c["q"] if q is None else q
    kn = c["kn"] if kn is None else kn
    vn = c["vn"] if vn is None else vn
    cu = c["cu"] if cu is None else cu
    prefix = c["prefix"] if prefix is None else prefix
    new = np.diff(cu)
    out = torch.empty((q.shape[0], q.shape[1], c["D"]), dtype=torch.bfloat16, device="cuda")
    binding.extend(c["pool"], 0, gu.dev_bf16(q), gu.dev_bf16(kn), gu.dev_bf16(vn), out, gu.dev_i32(cu),
                   gu.dev_i32(c["bt"]), gu.dev_i32(prefix), max_new=int(max(new.max(), 1)),
                   max_seq_len=int(max(np.array(prefix) + new)), scale=1.0 / math.sqrt(c["D"]),
                   dev_status=c["status"])
    gu.sync()
    return out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 5])
def test_extend_matches_oracle_ragged(D, G):
    prefix, new = [40, 0, 16, 300, 129], [9, 33, 1, 160, 200]
    c = make_extend_case(prefix, new, 2, G, D, seed=D + G)
    out = gu.host_f64(run_extend(c))
    for b in range(len(prefix)):
        rows = list(range(new[b]))
        want = oracle.extend_from_logical(c["q"][c["cu"][b]:c["cu"][b + 1]], c["fk"][b], c["fv"][b],
                                          prefix[b], rows, 1.0 / math.sqrt(D))
        assert np.max(np.abs(out[c["cu"][b]:c["cu"][b + 1]] - want)) <= TOL, b
    assert int(c["status"].item()) == 0
    # the appended chunk is bit-exact in the pool image
    shape = oracle.PoolShape(1, c["num_pages"], 2, D)
    kk, cu_all = wlmod.concat_rows(c["fk"])
    vv, _ = wlmod.concat_rows(c["fv"])
    img = oracle.append(np.full(shape.elems, c["poison"], np.uint16), shape, 0, kk, vv, cu_all, c["bt"],
                        np.zeros(len(prefix), np.int32))
    assert np.array_equal(gu.pool_bits(c["pool"]), img)


@pytest.mark.parametrize("D", [64, 128])
def test_extend_bad_prefix_page_is_reported_without_faulting(D):
    """An out-of-range page id in a cached prefix: flagged, no fault, the other sessions exact."""
    prefix, new = [100, 60, 70], [20, 30, 1]
    c = make_extend_case(prefix, new, 2, 4, D, seed=31 + D)
    bt = c["bt"].copy()
    bt[0, 1] = c["num_pages"] + 9      # prefix tokens 16..31 of session 0
    out = gu.host_f64(run_extend(dict(c, bt=bt)))
    assert int(c["status"].item()) & binding.DEV_BAD_PAGE
    for b in (1, 2):
        rows = slice(c["cu"][b], c["cu"][b + 1])
        want = oracle.extend_from_logical(c["q"][rows], c["fk"][b], c["fv"][b], prefix[b], list(range(new[b])),
                                          1.0 / math.sqrt(D))
        assert float(np.max(np.abs(out[rows] - want))) <= TOL


def test_extend_after_prefix_equals_full_prefill_and_chunked():
    prefix, new, G, D = [200], [150], 4, 128
    c = make_extend_case(prefix, new, 2, G, D, seed=31)
    ext = gu.host_f64(run_extend(c))
    # full prefill of the same sequence into a fresh pool (P = 0, C = 350)
    full = make_extend_case([0], [350], 2, G, D, seed=31)
    qfull = np.concatenate([wlmod.draw_bf16(np.random.default_rng(7), (200, 2 * G, D), 1.0), c["q"]])
    kfull = np.concatenate([c["fk"][0][:200], c["kn"]])
    vfull = np.concatenate([c["fv"][0][:200], c["vn"]])
    pre = gu.host_f64(run_extend(full, q=qfull, kn=kfull, vn=vfull, cu=np.array([0, 350])))
    assert np.max(np.abs(pre[200:] - ext)) <= TOL
    # two chunks (70 + 80) after the same prefix
    c2 = make_extend_case(prefix, new, 2, G, D, seed=31)
    a = gu.host_f64(run_extend(c2, q=c["q"][:70], kn=c["kn"][:70], vn=c["vn"][:70], cu=np.array([0, 70])))
    b = gu.host_f64(run_extend(c2, q=c["q"][70:], kn=c["kn"][70:], vn=c["vn"][70:], cu=np.array([0, 80]),
                               prefix=[270]))
    assert np.max(np.abs(np.concatenate([a, b]) - ext)) <= TOL
    assert np.array_equal(gu.pool_bits(c2["pool"]), gu.pool_bits(c["pool"]))


def test_decode_equals_single_row_extend():
    import torch

    prefix, G, D = [611], 4, 128
    c = make_extend_case(prefix, [1], 2, G, D, seed=12)
    ext = gu.host_f64(run_extend(c))
    case = dict(pool=c["pool"], Hkv=2, layer=0, status=c["status"])
    dec = gu.host_f64(gu.run_decode(case, q_bits=c["q"][None], lens=[612], bt=c["bt"]))
    assert np.max(np.abs(dec[0, 0] - ext[0])) <= TOL


# ---------------------------------------------------------------------------
# Score ranges far beyond fp32 exp range: exercises the rescaling paths
# ---------------------------------------------------------------------------
def _growing_keys(L, Hkv, D, top):
    """K rows whose entries grow linearly from 0 to `top` along the sequence."""
    ramp = (np.arange(L, dtype=np.float32) * (top / max(L - 1, 1)))[:, None, None]
    return wlmod.f32_to_bf16_bits(np.broadcast_to(ramp, (L, Hkv, D)).copy())


@pytest.mark.parametrize("D", [64, 128])
def test_extend_huge_score_range_takes_rescaling_path(D):
    """q = 1 and K entries ramping from 0 to 8: the last key scores 8*sqrt(D) (90 at
    D=128, 130 in log2 units) above the first, far past the 2^60 headroom of the
    fixed-reference pass, so the workgroups must recompute with rescaling."""
    import torch

    prefix, new, Hkv, G = [300, 0], [40, 70], 2, 4
    rng = np.random.default_rng(77)
    full = [p + c for p, c in zip(prefix, new)]
    fk = [_growing_keys(L, Hkv, D, 8.0) for L in full]
    fv = [wlmod.draw_bf16(rng, (L, Hkv, D), 1.0) for L in full]
    bt, num_pages = wlmod.build_block_table(full, 5)
    pool = binding.Pool(1, num_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    st = gu.status_tensor()
    kk, cu_all = wlmod.concat_rows(fk)
    vv, _ = wlmod.concat_rows(fv)
    # whole sequences through extend (prefix 0), so both prefix and chunk use the pool
    q = wlmod.f32_to_bf16_bits(np.ones((int(cu_all[-1]), Hkv * G, D), np.float32))
    out = torch.empty((q.shape[0], Hkv * G, D), dtype=torch.bfloat16, device="cuda")
    binding.extend(pool, 0, gu.dev_bf16(q), gu.dev_bf16(kk), gu.dev_bf16(vv), out, gu.dev_i32(cu_all),
                   gu.dev_i32(bt), gu.dev_i32([0, 0]), max_new=max(full), max_seq_len=max(full),
                   scale=1.0 / math.sqrt(D), dev_status=st)
    gu.sync()
    got = gu.host_f64(out)
    for b in range(2):
        rows = list(range(full[b]))
        want = oracle.extend_from_logical(q[cu_all[b]:cu_all[b + 1]], fk[b], fv[b], 0, rows, 1.0 / math.sqrt(D))
        assert np.all(np.isfinite(got[cu_all[b]:cu_all[b + 1]]))
        assert np.max(np.abs(got[cu_all[b]:cu_all[b + 1]] - want)) <= TOL
    assert int(st.item()) == 0


@pytest.mark.parametrize("N,G", [(1, 4), (8, 4)])
def test_decode_huge_score_range(N, G):
    Hkv, D = 2, 128
    lens = [3000, 517, 4100]
    rng = np.random.default_rng(3)
    K = [_growing_keys(L, Hkv, D, 6.0) for L in lens]
    V = [wlmod.draw_bf16(rng, (L, Hkv, D), 1.0) for L in lens]
    bt, num_pages = wlmod.build_block_table(lens, 3)
    pool = binding.Pool(1, num_pages, Hkv, D)
    st = gu.status_tensor()
    kk, cu = wlmod.concat_rows(K)
    vv, _ = wlmod.concat_rows(V)
    binding.append(pool, 0, gu.dev_bf16(kk), gu.dev_bf16(vv), gu.dev_i32(cu), gu.dev_i32(bt),
                   gu.dev_i32([0, 0, 0]), max_new=max(lens), max_seq_len=max(lens), dev_status=st)
    q = wlmod.f32_to_bf16_bits(np.ones((3, N, Hkv * G, D), np.float32))
    case = dict(pool=pool, Hkv=Hkv, layer=0, status=st, lens=lens, bt=bt)
    out = gu.host_f64(gu.run_decode(case, q_bits=q))
    want = oracle.decode_from_logical(q, K, V, 1.0 / math.sqrt(D))
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out - want)) <= TOL
