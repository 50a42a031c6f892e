"""GPU parity of shared_kv_decode_cascade: sessions that a prefix cache gave the
same prefix pages (Prefill-as-a-Service, component 3) decode with each shared
prefix read once per unit of sessions.  The result is shared_kv_decode's: the
float64 oracle's page walk over the same (aliasing) block tables, within 2e-2."""
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


def make_case(groups, N, Hkv, G, D, seed):
    """GPU pool holding grouped sessions: each group's prefix written once, then each
    session's own tokens; logical K/V per session kept for the oracle."""
    rng = np.random.default_rng(seed)
    bt, lens, gid, pref, num_pages = wlmod.build_prefix_groups(groups, seed)
    pool = binding.Pool(1, num_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    st = gu.status_tensor()
    K, V, b = [], [], 0
    msl = max(max(lens), 1)
    for pre, ls in groups:
        pk, pv = wlmod.draw_bf16(rng, (pre, Hkv, D), 1.0), wlmod.draw_bf16(rng, (pre, Hkv, D), 1.0)
        for i, L in enumerate(ls):
            ok, ov = wlmod.draw_bf16(rng, (L - pre, Hkv, D), 1.0), wlmod.draw_bf16(rng, (L - pre, Hkv, D), 1.0)
            K.append(np.concatenate([pk, ok]))
            V.append(np.concatenate([pv, ov]))
            row = gu.dev_i32(bt[b:b + 1])
            if i == 0 and pre:
                binding.append(pool, 0, gu.dev_bf16(pk), gu.dev_bf16(pv), gu.dev_i32([0, pre]), row,
                               gu.dev_i32([0]), max_new=msl, max_seq_len=msl, dev_status=st)
            if L > pre:
                binding.append(pool, 0, gu.dev_bf16(ok), gu.dev_bf16(ov), gu.dev_i32([0, L - pre]), row,
                               gu.dev_i32([pre]), max_new=msl, max_seq_len=msl, dev_status=st)
            b += 1
    q = wlmod.draw_bf16(rng, (len(lens), N, Hkv * G, D), 1.0)
    return dict(pool=pool, bt=bt, lens=lens, gid=gid, pref=pref, K=K, V=V, q=q, status=st, Hkv=Hkv, D=D,
                num_pages=num_pages, layer=0)


def run_cascade(c, gid=None, pref=None, bt=None):
    import torch

    B, N, Hq, D = c["q"].shape
    msl = max(max(c["lens"]), 1)
    ws = gu.nan_workspace(binding.decode_workspace_bytes(B, N, Hq, c["Hkv"], D, msl))
    out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device="cuda")
    binding.decode_cascade(c["pool"], 0, gu.dev_bf16(c["q"]), out, gu.dev_i32(c["bt"] if bt is None else bt),
                           gu.dev_i32(c["lens"]), gu.dev_i32(c["gid"] if gid is None else gid),
                           gu.dev_i32(c["pref"] if pref is None else pref), msl, 1.0 / math.sqrt(D), ws,
                           dev_status=c["status"])
    gu.sync()
    return out


@pytest.mark.parametrize("groups,N,G,D", [
    ([(64, [100, 64, 300]), (0, [17]), (32, [33, 48])], 8, 4, 128),       # 2 sessions per unit
    ([(512, [512 + 7 * i for i in range(7)])], 2, 4, 64),                    # 8 per unit: one unit
    ([(160, [200, 161, 999, 160, 400])], 4, 4, 128),                           # 4 per unit, a second unit
    ([(48, [60, 70])], 16, 3, 128),                                           # 48 rows: 1 per unit
    ([(0, [0, 30]), (16, [16]), (32, [32, 90, 33, 35])], 1, 5, 64),
])
def test_cascade_matches_oracle(groups, N, G, D):
    print(f"[cascade] groups={groups} N={N} G={G} D={D}", flush=True)
    c = make_case(groups, N, 2, G, D, seed=len(groups) * 7 + N + D)
    out = gu.host_f64(run_cascade(c))
    want = oracle.decode_from_logical(c["q"], c["K"], c["V"], 1.0 / math.sqrt(D))
    err = float(np.max(np.abs(out - want)))
    print(f"[cascade] max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(c["status"].item()) == 0


def test_cascade_matches_shared_decode_and_oracle_pool_walk():
    groups = [(256, [300, 700, 256, 1000]), (0, [40]), (128, [129, 500])]
    c = make_case(groups, 8, 2, 4, 128, seed=71)
    casc = gu.host_f64(run_cascade(c))
    plain = gu.host_f64(gu.run_decode(c, q_bits=c["q"], lens=c["lens"], bt=c["bt"]))
    assert float(np.max(np.abs(casc - plain))) <= TOL
    shape = oracle.PoolShape(1, c["num_pages"], 2, 128)
    want = oracle.decode(gu.pool_bits(c["pool"]), shape, 0, c["q"], c["bt"], c["lens"], 1.0 / math.sqrt(128))
    assert float(np.max(np.abs(casc - want))) <= TOL


def test_no_groups_is_shared_decode():
    groups = [(0, [100]), (0, [33]), (0, [0]), (0, [400])]
    c = make_case(groups, 4, 2, 4, 128, seed=72)
    gid = np.full(4, -1, np.int32)
    casc = gu.host_f64(run_cascade(c, gid=gid))
    want = oracle.decode_from_logical(c["q"], c["K"], c["V"], 1.0 / math.sqrt(128))
    assert float(np.max(np.abs(casc - want))) <= TOL


def test_cascade_above_64_rows_per_session_is_shared_decode():
    """With more than 64 query rows per session a unit would hold one session:
    the call runs the plain decode over the same tables, bit for bit, and the
    group arguments are not read."""
    groups = [(64, [100, 80, 90]), (0, [33])]
    c = make_case(groups, 12, 1, 8, 128, seed=74)      # 96 rows per session
    casc = gu.host_bits(run_cascade(c))
    plain = gu.host_bits(gu.run_decode(c, q_bits=c["q"], lens=c["lens"], bt=c["bt"]))
    assert np.array_equal(casc, plain)
    want = oracle.decode_from_logical(c["q"], c["K"], c["V"], 1.0 / math.sqrt(128))
    assert float(np.max(np.abs(gu.host_f64(run_cascade(c)) - want))) <= TOL
    pref = c["pref"].copy()
    pref[1] = 2                                        # inconsistent, and not read
    run_cascade(c, pref=pref)
    assert int(c["status"].item()) == 0


def test_cascade_reports_inconsistent_groups_without_faulting():
    groups = [(64, [100, 80, 90])]
    c = make_case(groups, 8, 2, 4, 128, seed=73)
    pref = c["pref"].copy()
    pref[1] = 2                                  # claims a shorter prefix than its unit's first session
    run_cascade(c, pref=pref)
    assert int(c["status"].item()) & binding.DEV_BAD_LEN
    c["status"].zero_()
    bt = c["bt"].copy()
    bt[1, 0] = bt[0, 3] if bt[0, 3] >= 0 else 0  # a prefix entry that is not the first session's page
    out = gu.host_f64(run_cascade(c, bt=bt))
    assert int(c["status"].item()) & binding.DEV_BAD_PAGE
    assert np.all(np.isfinite(out))


def test_cascade_over_allocator_tables():
    """Sessions admitted through the prefix cache: the later sessions reuse the
    published full blocks of a system prompt (their KV is not written again, only
    the tokens past the reused pages are appended), the grouping comes from
    kvs_prefix_groups, and the cascade decode equals the oracle over each
    session's logical K/V."""
    import torch

    N, Hkv, G, D = 4, 2, 4, 128
    rng = np.random.default_rng(81)
    pc = binding.PrefixCache(64)
    sys_a = [int(x) for x in rng.integers(0, 1000, 16 * 5 + 7)]
    sys_b = [int(x) for x in rng.integers(0, 1000, 16 * 3)]
    prompts = [sys_a + [1] * 30, sys_a + [2] * 3, sys_a + [3] * 50, sys_a, sys_b + [4] * 9, sys_b]
    pool = binding.Pool(1, 64, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    st = gu.status_tensor()
    rows, K, V = [], [], []
    first_kv = {}
    for t in prompts:
        pages, matched = pc.admit(t)
        L, P = len(t), 16 * matched
        key = tuple(t[:P])
        if matched:
            pk, pv = first_kv[key]
        else:
            pk = pv = np.zeros((0, Hkv, D), np.uint16)
        ok = wlmod.draw_bf16(rng, (L - P, Hkv, D), 1.0)
        ov = wlmod.draw_bf16(rng, (L - P, Hkv, D), 1.0)
        kk, vv = np.concatenate([pk, ok]), np.concatenate([pv, ov])
        for m in range(1, L // 16 + 1):          # what a later session could reuse of this one
            first_kv.setdefault(tuple(t[:16 * m]), (kk[:16 * m], vv[:16 * m]))
        if L > P:
            binding.append(pool, 0, gu.dev_bf16(ok), gu.dev_bf16(ov), gu.dev_i32([0, L - P]),
                           gu.dev_i32(np.asarray(pages, np.int32)[None]), gu.dev_i32([P]), max_new=L,
                           max_seq_len=L, dev_status=st)
        pc.publish(t, pages)
        rows.append(pages)
        K.append(kk)
        V.append(vv)
    lens = [len(t) for t in prompts]
    bt = np.full((len(rows), max(len(r) for r in rows)), -1, np.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    gid, pref = binding.prefix_groups(bt, lens)
    assert list(gid) == [0, 0, 0, 0, 4, 4] and list(pref) == [5, 5, 5, 5, 3, 3]
    q = wlmod.draw_bf16(rng, (len(rows), N, Hkv * G, D), 1.0)
    c = dict(pool=pool, bt=bt, lens=lens, gid=gid, pref=pref, q=q, status=st, Hkv=Hkv, D=D)
    out = gu.host_f64(run_cascade(c))
    want = oracle.decode_from_logical(q, K, V, 1.0 / math.sqrt(D))
    err = float(np.max(np.abs(out - want)))
    print(f"[cascade] allocator tables: max-abs err {err:.3e}", flush=True)
    assert err <= TOL
    assert int(st.item()) == 0


def test_cascade_tables_reused_only_for_the_same_inputs():
    """One workspace serves a sequence of cascade calls: repeated calls with the same
    inputs find their tables already built (the plan kernel returns at once), and any
    change to a length, a group id or a prefix claim rebuilds them.  Every call must
    equal the same call on a fresh workspace, bit for bit."""
    import torch

    groups = [(64, [100, 64, 300]), (0, [17]), (32, [33, 48])]
    c = make_case(groups, 8, 2, 4, 128, seed=91)
    B, N, Hq, D = c["q"].shape
    msl = max(max(c["lens"]), 1)
    nbytes = binding.decode_workspace_bytes(B, N, Hq, c["Hkv"], D, msl)
    shared = gu.nan_workspace(nbytes)

    def call(ws, lens, gid, pref):
        out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device="cuda")
        binding.decode_cascade(c["pool"], 0, gu.dev_bf16(c["q"]), out, gu.dev_i32(c["bt"]), gu.dev_i32(lens),
                               gu.dev_i32(gid), gu.dev_i32(pref), msl, 1.0 / math.sqrt(D), ws,
                               dev_status=c["status"])
        gu.sync()
        return out

    lens, gid, pref = list(c["lens"]), list(c["gid"]), list(c["pref"])
    shorter = list(lens)
    shorter[1] -= 1                      # one session one token shorter (its last token dropped)
    split = list(gid)
    split[2] = -1                        # the group's third member no longer shares
    claim = list(pref)
    claim[0] = claim[1] = 2              # the first group claims 2 of its 4 prefix pages
    seq = [(lens, gid, pref), (lens, gid, pref), (shorter, gid, pref), (lens, gid, pref),
           (lens, split, pref), (lens, gid, claim), (lens, gid, pref)]
    for i, (l_, g_, p_) in enumerate(seq):
        print(f"[cascade reuse] call {i}", flush=True)
        got = call(shared, l_, g_, p_)
        want = call(gu.nan_workspace(nbytes), l_, g_, p_)
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), i
    assert int(c["status"].item()) == 0
