"""Parity at the workloads' full sizes, in the launch configuration the bench times.

The GPU path appends device-drawn K/V (torch's seeded generator, the input
generator for large sizes) into a poisoned pool with kv_pool_append, then runs
shared_kv_decode / partial_prefill_extend.  The oracle checks a seeded sample of
sessions (decode: every decoder and head of each sampled session) or rows
(extend: 8 sessions, the ends, middle and two seeded rows of every 128-row
block) from the same logical K/V copied to the host, and compares the sampled
sessions' page tiles bit for bit against its own append of those K/V.  Besides
the absolute tolerance, each sampled session must satisfy the output-scaled
bound gu.FULLSIZE_REL, which one dropped or doubled page of an 8K-token context
breaks (tests/test_fullsize_bound.py shows this on the CPU).
"""
import math

import numpy as np
import pytest

import oracle
from cross_model_shared_amd import binding
from cross_model_shared_amd import workload as W
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def host_rows(t):
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def sample_sessions(lens, k, seed):
    order = np.argsort(lens)
    picks = {int(order[0]), int(order[-1])}
    rng = np.random.default_rng(seed)
    for b in rng.permutation(len(lens)):
        if len(picks) >= k:
            break
        picks.add(int(b))
    return sorted(picks)


def check_tiles(pool, bt, layer, b, kb, vb, Hkv, D):
    """The session's pages in the GPU pool equal the oracle's append of its K/V."""
    L = kb.shape[0]
    npg = (L + 15) // 16
    shape = oracle.PoolShape(1, npg, Hkv, D)
    img = oracle.append(np.full(shape.elems, gu.POISON_NAN, np.uint16), shape, 0, kb, vb, [0, L],
                        np.arange(npg, dtype=np.int32)[None], [0])
    tile = Hkv * 32 * D
    flat = pool.data.view(-1)
    per_layer = pool.num_pages * tile
    for p in range(npg):
        pid = int(bt[b, p])
        got = flat[layer * per_layer + pid * tile:layer * per_layer + (pid + 1) * tile]
        got = got.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, img[p * tile:(p + 1) * tile]), (b, p)


@pytest.mark.parametrize("name,layers,layer", [("llama8b_n4", 1, 0), ("qwen3_8b_n8", 2, 1),
                                               ("qwen3_14b_long", 1, 0)])
def test_decode_full_size_sampled(name, layers, layer):
    import torch

    wl = W.make_workload(name)
    B, N, Hq, Hkv, D = wl.batch, wl.num_decoders, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lens = wl.lens
    print(f"[fullsize] {name}: B={B} N={N} sum(L)={sum(lens)} max(L)={max(lens)}", flush=True)
    bt, num_pages = W.build_block_table(lens, wl.seed)
    pool = binding.Pool(layers, num_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    total = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    k = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 10, layer)).view(total, Hkv, D)
    v = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 11, layer)).view(total, Hkv, D)
    st = gu.status_tensor()
    maxL = max(lens)
    bt_d = torch.from_numpy(bt).cuda()
    binding.append(pool, layer, k, v, gu.dev_i32(cu), bt_d, gu.dev_i32(np.zeros(B)), max_new=maxL,
                   max_seq_len=maxL, dev_status=st)
    q = W.device_normal_bf16(B * N * Hq * D, wl.std, W.mix_seed(wl.seed, 12, layer)).view(B, N, Hq, D)
    out = torch.empty_like(q)
    ws = gu.nan_workspace(binding.decode_workspace_bytes(B, N, Hq, Hkv, D, maxL))
    binding.decode(pool, layer, q, out, bt_d, gu.dev_i32(lens), maxL, wl.scale, ws, dev_status=st)
    gu.sync()
    assert int(st.item()) == 0
    got = gu.host_f64(out)
    assert np.all(np.isfinite(got))
    picks = sample_sessions(lens, 8, wl.seed)
    qh = host_rows(q)
    Ks = [None] * B
    Vs = [None] * B
    for b in picks:
        Ks[b] = host_rows(k[cu[b]:cu[b + 1]])
        Vs[b] = host_rows(v[cu[b]:cu[b + 1]])
    want = oracle.decode_from_logical(qh, Ks, Vs, wl.scale)
    err = max(float(np.max(np.abs(got[b] - want[b]))) for b in picks)
    rel = max(gu.session_rel_err(got[b], want[b]) for b in picks)
    print(f"[fullsize] {name}: sessions {picks} max-abs err {err:.3e}, session-relative {rel:.4f}", flush=True)
    assert err <= TOL
    assert rel <= gu.FULLSIZE_REL
    for b in sorted(picks, key=lambda b: lens[b])[:2]:   # the two shortest sampled sessions
        check_tiles(pool, bt, layer, b, Ks[b], Vs[b], Hkv, D)


def test_decode_append_full_size_sampled():
    """The bench's decode step call (shared_kv_decode_append) on the full 8-decoder workload: the pool
    holds every session's first L-1 tokens (NaN in the last slot), the call writes token L-1 and
    attends all L."""
    import torch

    wl = W.make_workload("qwen3_8b_n8")
    B, N, Hq, Hkv, D = wl.batch, wl.num_decoders, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lens, layer = wl.lens, 1
    print(f"[fullsize] decode_append {wl.name}: B={B} N={N} sum(L)={sum(lens)}", flush=True)
    bt, num_pages = W.build_block_table(lens, wl.seed)
    pool = binding.Pool(2, num_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    total = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    k = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 10, layer)).view(total, Hkv, D)
    v = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 11, layer)).view(total, Hkv, D)
    last = torch.from_numpy(cu[1:] - 1).long().cuda()
    keep = torch.ones(total, dtype=torch.bool, device="cuda")
    keep[last] = False
    st = gu.status_tensor()
    maxL = max(lens)
    bt_d = torch.from_numpy(bt).cuda()
    cu_before = np.concatenate([[0], np.cumsum([L - 1 for L in lens])]).astype(np.int32)
    binding.append(pool, layer, k[keep].contiguous(), v[keep].contiguous(), gu.dev_i32(cu_before), bt_d,
                   gu.dev_i32(np.zeros(B)), max_new=maxL, max_seq_len=maxL, dev_status=st)
    q = W.device_normal_bf16(B * N * Hq * D, wl.std, W.mix_seed(wl.seed, 12, layer)).view(B, N, Hq, D)
    out = torch.empty_like(q)
    ws = gu.nan_workspace(binding.decode_workspace_bytes(B, N, Hq, Hkv, D, maxL))
    binding.decode_append(pool, layer, k[last].contiguous(), v[last].contiguous(), q, out, bt_d, gu.dev_i32(lens),
                          maxL, wl.scale, ws, dev_status=st)
    gu.sync()
    assert int(st.item()) == 0
    got = gu.host_f64(out)
    assert np.all(np.isfinite(got))
    picks = sample_sessions(lens, 8, wl.seed + 1)
    qh = host_rows(q)
    Ks, Vs = [None] * B, [None] * B
    for b in picks:
        Ks[b] = host_rows(k[cu[b]:cu[b + 1]])
        Vs[b] = host_rows(v[cu[b]:cu[b + 1]])
    want = oracle.decode_from_logical(qh, Ks, Vs, wl.scale)
    err = max(float(np.max(np.abs(got[b] - want[b]))) for b in picks)
    rel = max(gu.session_rel_err(got[b], want[b]) for b in picks)
    print(f"[fullsize] decode_append: sessions {picks} max-abs err {err:.3e}, session-relative {rel:.4f}",
          flush=True)
    assert err <= TOL
    assert rel <= gu.FULLSIZE_REL
    for b in sorted(picks, key=lambda b: lens[b])[:2]:   # every page, the new token's included
        check_tiles(pool, bt, layer, b, Ks[b], Vs[b], Hkv, D)


def test_extend_full_size_sampled():
    import torch

    wl = W.make_workload("extend_8k_512")
    B, Hq, Hkv, D = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    full = wl.total_lens()
    print(f"[fullsize] extend_8k_512: B={B} prefix={wl.prefix[0]} new={wl.new[0]}", flush=True)
    bt, num_pages = W.build_block_table(full, wl.seed)
    pool = binding.Pool(1, num_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    bt_d = torch.from_numpy(bt).cuda()
    st = gu.status_tensor()
    P, T = sum(wl.prefix), sum(wl.new)
    kp = W.device_normal_bf16(P * Hkv * D, wl.std, W.mix_seed(wl.seed, 20)).view(P, Hkv, D)
    vp = W.device_normal_bf16(P * Hkv * D, wl.std, W.mix_seed(wl.seed, 21)).view(P, Hkv, D)
    cup = np.concatenate([[0], np.cumsum(wl.prefix)]).astype(np.int32)
    binding.append(pool, 0, kp, vp, gu.dev_i32(cup), bt_d, gu.dev_i32(np.zeros(B)), max_new=max(wl.prefix),
                   max_seq_len=max(full), dev_status=st)
    q = W.device_normal_bf16(T * Hq * D, wl.std, W.mix_seed(wl.seed, 22)).view(T, Hq, D)
    kn = W.device_normal_bf16(T * Hkv * D, wl.std, W.mix_seed(wl.seed, 23)).view(T, Hkv, D)
    vn = W.device_normal_bf16(T * Hkv * D, wl.std, W.mix_seed(wl.seed, 24)).view(T, Hkv, D)
    cu = np.concatenate([[0], np.cumsum(wl.new)]).astype(np.int32)
    out = torch.empty_like(q)
    binding.extend(pool, 0, q, kn, vn, out, gu.dev_i32(cu), bt_d, gu.dev_i32(wl.prefix), max(wl.new), max(full),
                   wl.scale, dev_status=st)
    gu.sync()
    assert int(st.item()) == 0
    got = gu.host_f64(out)
    assert np.all(np.isfinite(got))
    picks = sample_sessions(full, 8, wl.seed)
    rng = np.random.default_rng(wl.seed)
    for b in picks:
        C = wl.new[b]
        # both ends and the middle of every 128-row block (a workgroup's rows at G = 4), plus two
        # seeded rows per block
        rows = set(range(4))
        for r0 in range(0, C, 128):
            r1 = min(r0 + 128, C)
            rows |= {r0, r0 + 1, (r0 + r1) // 2, r1 - 2, r1 - 1}
            rows |= {int(x) for x in rng.integers(r0, r1, size=2)}
        rows = sorted(rows)
        kf = np.concatenate([host_rows(kp[cup[b]:cup[b + 1]]), host_rows(kn[cu[b]:cu[b + 1]])])
        vf = np.concatenate([host_rows(vp[cup[b]:cup[b + 1]]), host_rows(vn[cu[b]:cu[b + 1]])])
        want = oracle.extend_from_logical(host_rows(q[cu[b]:cu[b + 1]]), kf, vf, wl.prefix[b], rows, wl.scale)
        gs = got[cu[b] + np.array(rows)]
        err = float(np.max(np.abs(gs - want)))
        rel = gu.session_rel_err(gs, want)
        print(f"[fullsize] extend session {b}: {len(rows)} rows, max-abs err {err:.3e}, session-relative {rel:.4f}",
              flush=True)
        assert err <= TOL
        assert rel <= gu.FULLSIZE_REL
    check_tiles(pool, bt, 0, picks[-1], kf, vf, Hkv, D)  # prefix + appended chunk of the last pick


def test_layer_group_full_size_sampled():
    """partial_prefill_layers at the bench's size and launch (layers [12, 16) of a 32-layer pool,
    8 prompts of 4096 tokens, no cached prefix; paired causal row blocks): in every layer one of two
    sampled prompts, its first, last and two tokens (the block's last and a seeded one) of every
    workgroup's 128-row block, all heads, against the oracle; plus that prompt's appended tiles.""" 
    import torch

    wl = W.make_workload("llama8b_layer_group")
    B, Hq, Hkv, D = wl.batch, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    lb, nl = wl.layer_group
    full = wl.total_lens()
    print(f"[fullsize] layer group: B={B} new={wl.new[0]} layers [{lb}, {lb + nl}) of {wl.num_layers}", flush=True)
    bt, num_pages = W.build_block_table(full, wl.seed)
    pool = binding.Pool(wl.num_layers, num_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    btd = torch.from_numpy(bt).cuda()
    st = gu.status_tensor()
    T = sum(wl.new)
    q = W.device_normal_bf16(nl * T * Hq * D, wl.std, W.mix_seed(wl.seed, 70)).view(nl, T, Hq, D)
    kn = W.device_normal_bf16(nl * T * Hkv * D, wl.std, W.mix_seed(wl.seed, 71)).view(nl, T, Hkv, D)
    vn = W.device_normal_bf16(nl * T * Hkv * D, wl.std, W.mix_seed(wl.seed, 72)).view(nl, T, Hkv, D)
    out = torch.empty_like(q)
    cu = np.concatenate([[0], np.cumsum(wl.new)]).astype(np.int32)
    binding.extend_layers(pool, lb, q, kn, vn, out, gu.dev_i32(cu), btd, gu.dev_i32(wl.prefix), max(wl.new),
                          max(full), wl.scale, dev_status=st)
    gu.sync()
    assert int(st.item()) == 0
    picks = sample_sessions(full, 2, wl.seed + 3)
    rng = np.random.default_rng(wl.seed + 3)
    for li in range(nl):
        got = gu.host_f64(out[li])
        assert np.all(np.isfinite(got))
        for b in picks[li % 2:li % 2 + 1]:   # one prompt per layer, both prompts over the group
            C = wl.new[b]
            rows = {0, 1, C - 1}
            for r0 in range(0, C, 32):   # a workgroup's 128 rows are 32 tokens at G = 4
                r1 = min(r0 + 32, C)
                rows |= {r1 - 1, int(rng.integers(r0, r1))}
            rows = sorted(rows)
            kf = host_rows(kn[li, cu[b]:cu[b + 1]])
            vf = host_rows(vn[li, cu[b]:cu[b + 1]])
            want = oracle.extend_from_logical(host_rows(q[li, cu[b]:cu[b + 1]]), kf, vf, 0, rows, wl.scale)
            gs = got[cu[b] + np.array(rows)]
            err = float(np.max(np.abs(gs - want)))
            rel = gu.session_rel_err(gs, want)
            print(f"[fullsize] layer {lb + li} prompt {b}: {len(rows)} tokens, max-abs err {err:.3e}, "
                  f"session-relative {rel:.4f}", flush=True)
            assert err <= TOL
            assert rel <= gu.FULLSIZE_REL
        b = picks[li % 2]
        check_tiles(pool, bt, lb + li, b, host_rows(kn[li, cu[b]:cu[b + 1]]), host_rows(vn[li, cu[b]:cu[b + 1]]),
                    Hkv, D)
    del pool, q, kn, vn, out
    torch.cuda.empty_cache()


def test_private_decode_full_size_sampled():
    """qwen3_8b_n8_private at full size (64 sessions, 8 decoders, private suffixes up to
    2048 tokens), in the bench's launch configuration; 8 sampled sessions, every
    decoder and head, against the oracle over prefix ++ suffix."""
    import torch

    wl = W.make_workload("qwen3_8b_n8_private")
    B, N, Hq, Hkv, D = wl.batch, wl.num_decoders, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    print(f"[fullsize] private: B={B} N={N} sum(L)={sum(wl.lens)} sum(U)={sum(wl.priv)}", flush=True)
    bt, pbt, num_pages = W.build_private_tables(wl.lens, wl.priv, wl.seed)
    pool = binding.Pool(1, num_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    st = gu.status_tensor()
    logical = []
    for i, (table, lens) in enumerate(((bt, wl.lens), (pbt, wl.priv))):
        total = sum(lens)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        k = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 30 + 2 * i)).view(total, Hkv, D)
        v = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 31 + 2 * i)).view(total, Hkv, D)
        binding.append(pool, 0, k, v, gu.dev_i32(cu), torch.from_numpy(table).cuda(),
                       gu.dev_i32(np.zeros(len(lens))), max_new=max(lens), max_seq_len=max(lens), dev_status=st)
        logical.append((k, v, cu))
    q = W.device_normal_bf16(B * N * Hq * D, wl.std, W.mix_seed(wl.seed, 34)).view(B, N, Hq, D)
    out = torch.empty_like(q)
    maxL, maxU = max(wl.lens), max(wl.priv)
    ws = gu.nan_workspace(binding.decode_workspace_bytes(B, N, Hq, Hkv, D, maxL))
    binding.decode_private(pool, 0, q, out, torch.from_numpy(bt).cuda(), gu.dev_i32(wl.lens),
                           torch.from_numpy(pbt).cuda(), gu.dev_i32(wl.priv), maxL, maxU, wl.scale, ws,
                           dev_status=st)
    gu.sync()
    assert int(st.item()) == 0
    got = gu.host_f64(out)
    assert np.all(np.isfinite(got))
    picks = sample_sessions(wl.lens, 8, wl.seed)
    qh = host_rows(q)
    (ks, vs, cus), (kp, vp, cup) = logical
    err = rel = 0.0
    for b in picks:
        for n in range(N):
            r = b * N + n
            K = np.concatenate([host_rows(ks[cus[b]:cus[b + 1]]), host_rows(kp[cup[r]:cup[r + 1]])])
            V = np.concatenate([host_rows(vs[cus[b]:cus[b + 1]]), host_rows(vp[cup[r]:cup[r + 1]])])
            want = oracle.decode_from_logical(qh[b:b + 1, n:n + 1], [K], [V], wl.scale)[0]
            err = max(err, float(np.max(np.abs(got[b, n:n + 1] - want))))
            rel = max(rel, gu.session_rel_err(got[b, n:n + 1], want))
    print(f"[fullsize] private: sessions {picks} max-abs err {err:.3e}, session-relative {rel:.4f}", flush=True)
    assert err <= TOL
    assert rel <= gu.FULLSIZE_REL


def test_cascade_decode_full_size_sampled():
    """qwen3_8b_n8_cascade at full size (64 sessions in 32 pairs sharing 4K-8K-token
    prefix pages, own 0-8K tokens), in the bench's launch configuration; 8 sampled
    sessions, every decoder and head, against the oracle over prefix ++ own tokens."""
    import torch

    wl = W.make_workload("qwen3_8b_n8_cascade")
    B, N, Hq, Hkv, D = wl.batch, wl.num_decoders, wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    bt, lens, gid, pref, num_pages = W.build_prefix_groups(wl.groups, wl.seed)
    print(f"[fullsize] cascade: B={B} N={N} sum(L)={sum(lens)} pages={num_pages}", flush=True)
    pool = binding.Pool(1, num_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    st = gu.status_tensor()
    d_bt = torch.from_numpy(bt).cuda()
    firsts = [b for b in range(B) if b == 0 or gid[b] != gid[b - 1]]
    pre_tok = [wl.groups[gid[b]][0] for b in firsts]
    own = [L - int(p) * 16 for L, p in zip(lens, pref)]
    logical = []
    for i, (rows, ls, before) in enumerate(((firsts, pre_tok, [0] * len(firsts)),
                                            (list(range(B)), own, [int(p) * 16 for p in pref]))):
        total = sum(ls)
        cu = np.concatenate([[0], np.cumsum(ls)]).astype(np.int32)
        k = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 60 + 2 * i)).view(total, Hkv, D)
        v = W.device_normal_bf16(total * Hkv * D, wl.std, W.mix_seed(wl.seed, 61 + 2 * i)).view(total, Hkv, D)
        binding.append(pool, 0, k, v, gu.dev_i32(cu), d_bt[rows].contiguous(), gu.dev_i32(before),
                       max_new=max(max(ls), 1), max_seq_len=max(lens), dev_status=st)
        logical.append((k, v, cu))
    q = W.device_normal_bf16(B * N * Hq * D, wl.std, W.mix_seed(wl.seed, 64)).view(B, N, Hq, D)
    out = torch.empty_like(q)
    maxL = max(lens)
    ws = gu.nan_workspace(binding.decode_workspace_bytes(B, N, Hq, Hkv, D, maxL))
    binding.decode_cascade(pool, 0, q, out, d_bt, gu.dev_i32(lens), torch.from_numpy(gid).cuda(),
                           torch.from_numpy(pref).cuda(), maxL, wl.scale, ws, dev_status=st)
    gu.sync()
    assert int(st.item()) == 0
    got = gu.host_f64(out)
    assert np.all(np.isfinite(got))
    picks = sample_sessions(lens, 8, wl.seed)
    qh = host_rows(q)
    (kp, vp, cup), (ko, vo, cuo) = logical
    err = rel = 0.0
    for b in picks:
        f = firsts.index(max(x for x in firsts if x <= b))
        K = np.concatenate([host_rows(kp[cup[f]:cup[f + 1]]), host_rows(ko[cuo[b]:cuo[b + 1]])])
        V = np.concatenate([host_rows(vp[cup[f]:cup[f + 1]]), host_rows(vo[cuo[b]:cuo[b + 1]])])
        want = oracle.decode_from_logical(qh[b:b + 1], [K], [V], wl.scale)
        err = max(err, float(np.max(np.abs(got[b:b + 1] - want))))
        rel = max(rel, gu.session_rel_err(got[b:b + 1], want))
    print(f"[fullsize] cascade: sessions {picks} max-abs err {err:.3e}, session-relative {rel:.4f}", flush=True)
    assert err <= TOL
    assert rel <= gu.FULLSIZE_REL
