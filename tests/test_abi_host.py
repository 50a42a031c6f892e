"""The C ABI on the host: symbols, sizes, and argument checks (no GPU needed).

Every call below fails a host-side check, so nothing is ever enqueued; the
pointers are placeholders that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from cross_model_shared_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x1000)


@pytest.fixture(scope="module")
def L():
    return binding.load()


def header_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_][a-z_0-9]*)\s*\(", text, re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol(L):
    names = header_functions()
    assert {"kv_pool_append", "shared_kv_decode", "shared_kv_decode_append", "shared_kv_decode_private",
            "shared_kv_decode_cascade",
            "partial_prefill_extend", "partial_prefill_layers",
            "kv_pages_pack", "kv_pages_unpack", "kv_pages_buffer_bytes", "kv_pool_fetch", "kvs_pool_bytes",
            "shared_kv_decode_workspace_bytes", "shared_kv_decode_workspace_init", "kvs_last_error", "kvs_version",
            "kvs_prefix_cache_create", "kvs_prefix_cache_admit", "kvs_prefix_cache_publish",
            "kvs_prefix_cache_release", "kvs_prefix_groups"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert b"gfx950" in L.kvs_version()


def test_pool_bytes(L):
    assert L.kvs_pool_bytes(36, 1000, 8, 128, 16) == 36 * 1000 * 8 * 2 * 16 * 128 * 2
    assert L.kvs_pool_bytes(1, 0, 8, 128, 16) == 0
    assert L.kvs_pool_bytes(-1, 10, 8, 128, 16) == 0


def test_workspace_bytes_depend_on_bounds_not_device(L):
    a = L.shared_kv_decode_workspace_bytes(64, 8, 32, 8, 128, 16384)
    b = L.shared_kv_decode_workspace_bytes(64, 8, 32, 8, 128, 16384)
    assert a == b > 0
    # partials: (m, l) and a D-vector per row and split; at least one split per unit
    assert a >= 64 * 8 * 32 * (128 + 2) * 4
    assert L.shared_kv_decode_workspace_bytes(2, 2, 8, 3, 64, 100) == 0   # 8 % 3 != 0
    assert L.shared_kv_decode_workspace_bytes(0, 2, 8, 2, 64, 100) == 0


def test_workspace_init_host_checks(L):
    # rejected before anything is enqueued: no GPU call is made
    assert L.shared_kv_decode_workspace_init(None, 1 << 20, None) == binding.KVS_EINVAL
    assert binding.last_error()
    assert L.shared_kv_decode_workspace_init(FAKE, 8191, None) == binding.KVS_EWORKSPACE
    assert "8191" in binding.last_error()


def test_workspace_counters_lead_every_layout(L):
    # the arrival counters sit in the first 8 KiB whatever the bounds, so one workspace
    # serves calls of any shape: every size holds at least that region
    for args in [(1, 1, 1, 1, 64, 16), (64, 8, 32, 8, 128, 16384), (4096, 16, 64, 8, 128, 131072)]:
        assert L.shared_kv_decode_workspace_bytes(*args) > 8192


def pool(data=FAKE, layers=1, pages=8, heads=2, dim=64, page=16):
    return binding.KvsPool(data.value if data is not None else None, layers, pages, heads, dim, page)


def call_decode(L, p, layer=0, q=FAKE, out=FAKE, bt=FAKE, stride=4, lens=FAKE, batch=2, N=2, Hq=8,
                msl=64, scale=0.125, ws=FAKE, wsb=1 << 30):
    return L.shared_kv_decode(ctypes.byref(p), layer, q, out, bt, stride, lens, batch, N, Hq, msl, scale, ws,
                              wsb, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=pool(data=None)), binding.KVS_EINVAL),
    (dict(p=pool(page=32)), binding.KVS_EUNSUPPORTED),
    (dict(p=pool(dim=96)), binding.KVS_EUNSUPPORTED),
    (dict(p=pool(), layer=1), binding.KVS_ERANGE),
    (dict(p=pool(), layer=-1), binding.KVS_ERANGE),
    (dict(p=pool(), q=None), binding.KVS_EINVAL),
    (dict(p=pool(), out=None), binding.KVS_EINVAL),
    (dict(p=pool(), bt=None), binding.KVS_EINVAL),
    (dict(p=pool(), lens=None), binding.KVS_EINVAL),
    (dict(p=pool(), batch=0), binding.KVS_EINVAL),
    (dict(p=pool(), N=0), binding.KVS_EINVAL),
    (dict(p=pool(), Hq=7), binding.KVS_EUNSUPPORTED),
    (dict(p=pool(), msl=65), binding.KVS_ERANGE),          # > bt_stride * 16
    (dict(p=pool(), scale=0.0), binding.KVS_EINVAL),
    (dict(p=pool(), scale=-0.125), binding.KVS_EINVAL),
    (dict(p=pool(), scale=float("nan")), binding.KVS_EINVAL),
    (dict(p=pool(), scale=float("inf")), binding.KVS_EINVAL),
    (dict(p=pool(), scale=float("-inf")), binding.KVS_EINVAL),
    (dict(p=pool(), ws=None), binding.KVS_EWORKSPACE),
    (dict(p=pool(), wsb=16), binding.KVS_EWORKSPACE),
])
def test_decode_host_checks(L, kw, status):
    p = kw.pop("p")
    assert call_decode(L, p, **kw) == status
    assert binding.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), binding.KVS_EINVAL),
    (dict(v=None), binding.KVS_EINVAL),
    (dict(q=None), binding.KVS_EINVAL),
    (dict(p=pool(dim=96)), binding.KVS_EUNSUPPORTED),
    (dict(layer=1), binding.KVS_ERANGE),
    (dict(Hq=7), binding.KVS_EUNSUPPORTED),
    (dict(msl=65), binding.KVS_ERANGE),
    (dict(wsb=16), binding.KVS_EWORKSPACE),
])
def test_decode_append_host_checks(L, kw, status):
    a = dict(p=pool(), layer=0, k=FAKE, v=FAKE, q=FAKE, Hq=8, msl=64, wsb=1 << 30)
    a.update(kw)
    assert L.shared_kv_decode_append(ctypes.byref(a["p"]), a["layer"], a["k"], a["v"], a["q"], FAKE, FAKE, 4, FAKE,
                                     2, 2, a["Hq"], a["msl"], 0.125, FAKE, a["wsb"], None, None) == status
    assert binding.last_error()


def call_decode_private(L, p, q=FAKE, bt=FAKE, pbt=FAKE, pstride=2, plens=FAKE, N=2, Hq=8, msl=64, mpl=32,
                        ws=FAKE, wsb=1 << 30):
    return L.shared_kv_decode_private(ctypes.byref(p), 0, q, FAKE, bt, 4, FAKE, pbt, pstride, plens, 2, N, Hq,
                                      msl, mpl, 0.125, ws, wsb, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=pool(), pbt=None), binding.KVS_EINVAL),
    (dict(p=pool(), plens=None), binding.KVS_EINVAL),
    (dict(p=pool(), q=None), binding.KVS_EINVAL),
    (dict(p=pool(), pstride=0), binding.KVS_EINVAL),
    (dict(p=pool(), mpl=-1), binding.KVS_EINVAL),
    (dict(p=pool(), mpl=33), binding.KVS_ERANGE),            # > priv_bt_stride * 16
    (dict(p=pool(), N=17, wsb=16), binding.KVS_EWORKSPACE),  # 68 rows per KV head: accepted (row groups)
    (dict(p=pool(), msl=65), binding.KVS_ERANGE),
    (dict(p=pool(), wsb=16), binding.KVS_EWORKSPACE),
])
def test_decode_private_host_checks(L, kw, status):
    p = kw.pop("p")
    assert call_decode_private(L, p, **kw) == status
    assert binding.last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(gid=None), binding.KVS_EINVAL),
    (dict(pref=None), binding.KVS_EINVAL),
    (dict(N=17, wsb=16), binding.KVS_EWORKSPACE),     # 68 rows per session: accepted (plain decode)
    (dict(msl=65), binding.KVS_ERANGE),
    (dict(wsb=16), binding.KVS_EWORKSPACE),
])
def test_decode_cascade_host_checks(L, kw, status):
    a = dict(gid=FAKE, pref=FAKE, N=2, msl=64, wsb=1 << 30)
    a.update(kw)
    assert L.shared_kv_decode_cascade(ctypes.byref(pool()), 0, FAKE, FAKE, FAKE, 4, FAKE, a["gid"], a["pref"], 2,
                                      a["N"], 8, a["msl"], 0.125, FAKE, a["wsb"], None, None) == status
    assert binding.last_error()


def call_append(L, p, layer=0, k=FAKE, v=FAKE, cu=FAKE, bt=FAKE, stride=4, lens=FAKE, batch=2, total=10,
                max_new=8, msl=64):
    return L.kv_pool_append(ctypes.byref(p), layer, k, v, cu, bt, stride, lens, batch, total, max_new, msl,
                            None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=pool(page=8)), binding.KVS_EUNSUPPORTED),
    (dict(p=pool(heads=0)), binding.KVS_EINVAL),
    (dict(p=pool(), k=None), binding.KVS_EINVAL),
    (dict(p=pool(), cu=None), binding.KVS_EINVAL),
    (dict(p=pool(), max_new=0), binding.KVS_EINVAL),
    (dict(p=pool(), total=-1), binding.KVS_EINVAL),
    (dict(p=pool(), max_new=65), binding.KVS_ERANGE),
    (dict(p=pool(), msl=100), binding.KVS_ERANGE),
    (dict(p=pool(), stride=0), binding.KVS_EINVAL),
    (dict(p=pool(layers=2), layer=2), binding.KVS_ERANGE),
])
def test_append_host_checks(L, kw, status):
    p = kw.pop("p")
    assert call_append(L, p, **kw) == status


def call_append_check(L, p, cu=FAKE, bt=FAKE, stride=4, lens=FAKE, batch=2, total=10, max_new=8, msl=64,
                      scratch=FAKE, sbytes=1 << 20, status=FAKE):
    return L.kv_pool_append_check(ctypes.byref(p), cu, bt, stride, lens, batch, total, max_new, msl, scratch,
                                  sbytes, status, None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=pool(page=8)), binding.KVS_EUNSUPPORTED),
    (dict(p=pool(), cu=None), binding.KVS_EINVAL),
    (dict(p=pool(), status=None), binding.KVS_EINVAL),       # the check reports through dev_status only
    (dict(p=pool(), max_new=0), binding.KVS_EINVAL),
    (dict(p=pool(), max_new=65), binding.KVS_ERANGE),
    (dict(p=pool(), msl=100), binding.KVS_ERANGE),
    (dict(p=pool(), scratch=None), binding.KVS_EWORKSPACE),
    (dict(p=pool(pages=8), sbytes=31), binding.KVS_EWORKSPACE),  # 4 bytes per page
])
def test_append_check_host_checks(L, kw, status):
    p = kw.pop("p")
    assert call_append_check(L, p, **kw) == status
    assert binding.last_error()


def test_append_check_bytes(L):
    assert L.kv_pool_append_check_bytes(8) == 32
    assert L.kv_pool_append_check_bytes(0) == 0


def call_extend(L, p, q=FAKE, k=FAKE, v=FAKE, out=FAKE, cu=FAKE, bt=FAKE, stride=4, lens=FAKE, batch=2,
                Hq=8, total=10, max_new=8, msl=64, scale=0.125):
    return L.partial_prefill_extend(ctypes.byref(p), 0, q, k, v, out, cu, bt, stride, lens, batch, Hq, total,
                                    max_new, msl, scale, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=pool(dim=256)), binding.KVS_EUNSUPPORTED),
    (dict(p=pool(), q=None), binding.KVS_EINVAL),
    (dict(p=pool(), out=None), binding.KVS_EINVAL),
    (dict(p=pool(), Hq=5), binding.KVS_EUNSUPPORTED),
    (dict(p=pool(), max_new=0), binding.KVS_EINVAL),
    (dict(p=pool(), msl=1000), binding.KVS_ERANGE),
    (dict(p=pool(), scale=float("nan")), binding.KVS_EINVAL),
    (dict(p=pool(), scale=float("inf")), binding.KVS_EINVAL),
    (dict(p=pool(), scale=-1.0), binding.KVS_EINVAL),
    (dict(p=pool(), batch=-3), binding.KVS_EINVAL),
])
def test_extend_host_checks(L, kw, status):
    p = kw.pop("p")
    assert call_extend(L, p, **kw) == status


def call_layers(L, p, lb=0, nl=2, q=FAKE, k=FAKE, v=FAKE, out=FAKE, cu=FAKE, bt=FAKE, stride=4, lens=FAKE,
                batch=2, Hq=8, total=10, max_new=8, msl=64, scale=0.125):
    return L.partial_prefill_layers(ctypes.byref(p), lb, nl, q, k, v, out, cu, bt, stride, lens, batch, Hq, total,
                                    max_new, msl, scale, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=pool(layers=3), lb=2, nl=2), binding.KVS_ERANGE),
    (dict(p=pool(layers=3), lb=0, nl=0), binding.KVS_ERANGE),
    (dict(p=pool(layers=3), lb=-1, nl=1), binding.KVS_ERANGE),
    (dict(p=pool(layers=3), lb=3, nl=1), binding.KVS_ERANGE),
    (dict(p=pool(layers=3), k=None), binding.KVS_EINVAL),
    (dict(p=pool(layers=3), Hq=5), binding.KVS_EUNSUPPORTED),
    (dict(p=pool(layers=3), msl=1000), binding.KVS_ERANGE),
    (dict(p=pool(layers=3, dim=96)), binding.KVS_EUNSUPPORTED),
])
def test_extend_layers_host_checks(L, kw, status):
    kw = dict(kw)
    p = kw.pop("p")
    assert call_layers(L, p, **kw) == status


@pytest.mark.parametrize("unpack", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(p=pool(data=None)), binding.KVS_EINVAL),
    (dict(p=pool(layers=2), lb=2), binding.KVS_ERANGE),
    (dict(p=pool(layers=2), lb=1, nl=2), binding.KVS_ERANGE),
    (dict(p=pool(), nl=0), binding.KVS_ERANGE),
    (dict(p=pool(), n=-1), binding.KVS_EINVAL),
    (dict(p=pool(), ids=None), binding.KVS_EINVAL),
    (dict(p=pool(), buf=None), binding.KVS_EINVAL),
    (dict(p=pool(dim=96)), binding.KVS_EUNSUPPORTED),
])
def test_pack_host_checks(L, unpack, kw, status):
    kw = dict(kw)
    p = kw.pop("p", pool())
    args = dict(lb=0, nl=1, ids=FAKE, n=4, buf=FAKE)
    args.update(kw)
    fn = L.kv_pages_unpack if unpack else L.kv_pages_pack
    assert fn(ctypes.byref(p), args["lb"], args["nl"], args["ids"], args["n"], args["buf"], None, None) == status
    assert binding.last_error()


def test_pages_buffer_bytes(L):
    p = pool(layers=4, heads=8, dim=128)
    assert L.kv_pages_buffer_bytes(ctypes.byref(p), 3, 10) == 3 * 10 * 8 * 32 * 128 * 2
    assert L.kv_pages_buffer_bytes(ctypes.byref(p), 0, 10) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), binding.KVS_EINVAL),
    (dict(cu=None), binding.KVS_EINVAL),
    (dict(k=None), binding.KVS_EINVAL),
    (dict(batch=0), binding.KVS_EINVAL),
    (dict(msl=65), binding.KVS_ERANGE),
    (dict(total=-1), binding.KVS_EINVAL),
    (dict(layer=3), binding.KVS_ERANGE),
])
def test_fetch_host_checks(L, kw, status):
    a = dict(layer=0, bt=FAKE, cu=FAKE, k=FAKE, batch=2, msl=64, total=10)
    a.update(kw)
    assert L.kv_pool_fetch(ctypes.byref(pool()), a["layer"], a["bt"], 4, FAKE, a["cu"], a["batch"], a["total"],
                           a["msl"], a["k"], FAKE, None, None) == status


def test_binding_refuses_cpu_tensors():
    import torch

    with pytest.raises(ValueError, match="GPU tensor"):
        binding._ptr(torch.zeros(4), "x")
