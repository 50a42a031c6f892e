"""GPU parity of the handoff calls (kv_pages_pack / kv_pages_unpack, PrefillShare
section 3.3) and of kv_pool_fetch (the inverse of kv_pool_append), through the C
ABI.  All three move bits, so every check is bit-exact against the oracle."""
import numpy as np
import pytest

import oracle
from cross_model_shared_amd import binding
from cross_model_shared_amd import workload as wlmod
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load()


def filled_pool(lens, Hkv, D, layers, seed):
    """GPU pool whose layers hold seeded sessions (appended with kv_pool_append);
    returns the pool, the block table and the logical rows per layer."""
    rng = np.random.default_rng(seed)
    bt, num_pages = wlmod.build_block_table(lens, seed, spare_frac=0.1)
    pool = binding.Pool(layers, num_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    st = gu.status_tensor()
    rows = []
    for layer in range(layers):
        K = [wlmod.draw_bf16(rng, (L, Hkv, D), 1.0) for L in lens]
        V = [wlmod.draw_bf16(rng, (L, Hkv, D), 1.0) for L in lens]
        kk, cu = wlmod.concat_rows(K)
        vv, _ = wlmod.concat_rows(V)
        binding.append(pool, layer, gu.dev_bf16(kk), gu.dev_bf16(vv), gu.dev_i32(cu), gu.dev_i32(bt),
                       gu.dev_i32(np.zeros(len(lens))), max_new=max(lens), max_seq_len=max(lens), dev_status=st)
        rows.append((kk, vv, cu))
    gu.sync()
    assert int(st.item()) == 0
    return pool, bt, num_pages, rows


@pytest.mark.parametrize("D", [64, 128])
def test_pack_matches_oracle(D):
    import torch

    lens, Hkv, layers = [70, 33, 160], 2, 3
    pool, bt, num_pages, _ = filled_pool(lens, Hkv, D, layers, seed=61 + D)
    ids = np.random.default_rng(1).choice(num_pages, size=9, replace=True).astype(np.int32)
    for lb, nl in [(0, 3), (1, 2), (2, 1)]:
        buf = torch.empty(binding.pages_buffer_bytes(pool, nl, len(ids)), dtype=torch.uint8, device="cuda")
        binding.pack(pool, lb, nl, gu.dev_i32(ids), buf)
        gu.sync()
        shape = oracle.PoolShape(layers, num_pages, Hkv, D)
        want = oracle.pack(gu.pool_bits(pool), shape, lb, nl, ids)
        got = buf.cpu().numpy().view(np.uint16).reshape(want.shape)
        assert np.array_equal(got, want), (lb, nl)


@pytest.mark.parametrize("D", [64, 128])
def test_unpack_matches_oracle(D):
    import torch

    Hkv, layers, num_pages = 2, 3, 12
    pool = binding.Pool(layers, num_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_BIG).view(np.int16)))
    before = gu.pool_bits(pool).copy()
    ids = np.array([5, 0, 11, 7], np.int32)
    shape = oracle.PoolShape(layers, num_pages, Hkv, D)
    bits = wlmod.draw_bf16(np.random.default_rng(2), (2, len(ids), Hkv, oracle.tile_elems(D)), 1.0)
    binding.unpack(pool, 1, 2, gu.dev_i32(ids), torch.from_numpy(bits.view(np.int16).ravel()).cuda())
    gu.sync()
    want = oracle.unpack(before, shape, 1, 2, ids, bits)
    assert np.array_equal(gu.pool_bits(pool), want)


def test_handoff_to_another_pool_decodes_identically():
    """Pack two sessions' pages for every layer, unpack them into a second pool of
    another size under new page ids: decode over the new pool returns the same bits."""
    import torch

    lens, N, Hkv, G, D, layers = [500, 129], 4, 2, 4, 128, 2
    pool, bt, num_pages, _ = filled_pool(lens, Hkv, D, layers, seed=63)
    npg = [(L + 15) // 16 for L in lens]
    ids = np.concatenate([bt[b, :npg[b]] for b in range(2)]).astype(np.int32)
    buf = torch.empty(binding.pages_buffer_bytes(pool, layers, len(ids)), dtype=torch.uint8, device="cuda")
    binding.pack(pool, 0, layers, gu.dev_i32(ids), buf)
    dst_pages = num_pages + 37
    dst_ids = np.random.default_rng(3).permutation(dst_pages)[:len(ids)].astype(np.int32)
    dst = binding.Pool(layers, dst_pages, Hkv, D, fill=np.int16(np.uint16(gu.POISON_NAN).view(np.int16)))
    binding.unpack(dst, 0, layers, gu.dev_i32(dst_ids), buf)
    bt2 = np.full_like(bt, -1)
    bt2[0, :npg[0]] = dst_ids[:npg[0]]
    bt2[1, :npg[1]] = dst_ids[npg[0]:]
    q = wlmod.draw_bf16(np.random.default_rng(4), (2, N, Hkv * G, D), 1.0)
    st = gu.status_tensor()
    for layer in range(layers):
        a = gu.host_bits(gu.run_decode(dict(pool=pool, Hkv=Hkv, layer=layer, status=st), q_bits=q, lens=lens, bt=bt))
        b = gu.host_bits(gu.run_decode(dict(pool=dst, Hkv=Hkv, layer=layer, status=st), q_bits=q, lens=lens, bt=bt2))
        assert np.array_equal(a, b)
    assert int(st.item()) == 0


@pytest.mark.parametrize("D", [64, 128])
def test_fetch_returns_appended_rows(D):
    import torch

    lens, Hkv, layers = [37, 0, 16, 200, 1], 3, 2
    pool, bt, num_pages, rows = filled_pool(lens, Hkv, D, layers, seed=64 + D)
    for layer in range(layers):
        kk, vv, cu = rows[layer]
        k = torch.empty((int(cu[-1]), Hkv, D), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        st = gu.status_tensor()
        binding.fetch(pool, layer, gu.dev_i32(bt), gu.dev_i32(lens), gu.dev_i32(cu), max(lens), k, v, dev_status=st)
        gu.sync()
        assert int(st.item()) == 0
        assert np.array_equal(gu.host_bits(k), kk) and np.array_equal(gu.host_bits(v), vv)
        shape = oracle.PoolShape(layers, num_pages, Hkv, D)
        ok, ov = oracle.fetch(gu.pool_bits(pool), shape, layer, bt, lens)
        assert np.array_equal(ok, kk) and np.array_equal(ov, vv)


def test_bad_ids_and_rows_are_reported_without_faults():
    import torch

    lens, Hkv, D = [40, 20], 2, 64
    pool, bt, num_pages, rows = filled_pool(lens, Hkv, D, 1, seed=65)
    ids = np.array([0, num_pages + 3, -1, 1], np.int32)
    buf = torch.zeros(binding.pages_buffer_bytes(pool, 1, 4), dtype=torch.uint8, device="cuda")
    st = gu.status_tensor()
    binding.pack(pool, 0, 1, gu.dev_i32(ids), buf, dev_status=st)
    gu.sync()
    assert int(st.item()) & binding.DEV_BAD_PAGE
    st.zero_()
    binding.unpack(pool, 0, 1, gu.dev_i32(ids), buf, dev_status=st)
    gu.sync()
    assert int(st.item()) & binding.DEV_BAD_PAGE
    kk, vv, cu = rows[0]
    k = torch.empty((int(cu[-1]), Hkv, D), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    st.zero_()
    bad_cu = cu.copy()
    bad_cu[1] += 1                                  # session 0 claims 41 rows for 40 tokens
    binding.fetch(pool, 0, gu.dev_i32(bt), gu.dev_i32(lens), gu.dev_i32(bad_cu), max(lens), k, v, dev_status=st)
    gu.sync()
    assert int(st.item()) & binding.DEV_BAD_LEN
