"""ctypes binding of libkvshare.so: argument marshalling only.

Every function here checks that tensors live on the GPU with the dtype and
shape the C ABI expects, then passes raw device pointers and the current HIP
stream.  All arithmetic runs in the library's HIP kernels; there is no CPU
path, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvshare.so")

KVS_OK, KVS_EINVAL, KVS_ERANGE, KVS_EWORKSPACE, KVS_EUNSUPPORTED, KVS_EHIP, KVS_ENOSPACE = 0, -1, -2, -3, -4, -5, -6
DEV_BAD_PAGE, DEV_BAD_LEN, DEV_ALIAS = 1, 2, 4
PAGE = 16


class KvsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"kvshare status {status}: {message}")
        self.status = status


class KvsPool(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("num_layers", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32)]


_i32, _sz, _vp, _f = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_pool_p = ctypes.POINTER(KvsPool)

_SIGNATURES = {
    "kvs_pool_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "kv_pool_append": (ctypes.c_int, [_pool_p, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32,
                                      _i32, _vp, _vp]),
    "kv_pool_append_check_bytes": (_sz, [_i32]),
    "kv_pool_append_check": (ctypes.c_int, [_pool_p, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _sz, _vp,
                                            _vp]),
    "shared_kv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "shared_kv_decode_workspace_init": (ctypes.c_int, [_vp, _sz, _vp]),
    "shared_kv_decode": (ctypes.c_int, [_pool_p, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                        _f, _vp, _sz, _vp, _vp]),
    "shared_kv_decode_noalloc": (ctypes.c_int, [_pool_p, _i32, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32,
                                                _f, _vp, _vp]),
    "shared_kv_decode_append": (ctypes.c_int, [_pool_p, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                               _i32, _i32, _f, _vp, _sz, _vp, _vp]),
    "shared_kv_decode_private": (ctypes.c_int, [_pool_p, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _i32,
                                                _i32, _i32, _i32, _i32, _f, _vp, _sz, _vp, _vp]),
    "shared_kv_decode_cascade": (ctypes.c_int, [_pool_p, _i32, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32,
                                                _i32, _i32, _f, _vp, _sz, _vp, _vp]),
    "partial_prefill_extend": (ctypes.c_int, [_pool_p, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                              _i32, _i32, _i32, _i32, _i32, _f, _vp, _vp]),
    "partial_prefill_layers": (ctypes.c_int, [_pool_p, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                              _i32, _i32, _i32, _i32, _i32, _f, _vp, _vp]),
    "kv_pages_buffer_bytes": (_sz, [_pool_p, _i32, _i32]),
    "kv_pages_pack": (ctypes.c_int, [_pool_p, _i32, _i32, _vp, _i32, _vp, _vp, _vp]),
    "kv_pages_unpack": (ctypes.c_int, [_pool_p, _i32, _i32, _vp, _i32, _vp, _vp, _vp]),
    "kv_pool_fetch": (ctypes.c_int, [_pool_p, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "kvs_prefix_cache_create": (_vp, [_i32]),
    "kvs_prefix_cache_destroy": (None, [_vp]),
    "kvs_prefix_cache_admit": (ctypes.c_int, [_vp, _vp, _i32, _vp, _vp]),
    "kvs_prefix_cache_publish": (ctypes.c_int, [_vp, _vp, _i32, _vp]),
    "kvs_prefix_cache_release": (ctypes.c_int, [_vp, _vp, _i32]),
    "kvs_prefix_cache_stats": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp]),
    "kvs_prefix_cache_refcount": (ctypes.c_int, [_vp, _i32]),
    "kvs_prefix_groups": (ctypes.c_int, [_vp, _i32, _vp, _i32, _vp, _vp]),
    "kvs_last_error": (ctypes.c_char_p, []),
    "kvs_version": (ctypes.c_char_p, []),
}

_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (building it in-tree first if it is not there)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        from . import build_lib

        build_lib.build()
    if not os.path.exists(path):
        raise RuntimeError(f"libkvshare.so not found at {path}; the HIP path is required")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def last_error() -> str:
    return load().kvs_last_error().decode()


def _check(status: int):
    if status != KVS_OK:
        raise KvsError(status, last_error())


# ---------------------------------------------------------------------------
# tensor helpers (torch is only the device allocator and stream provider)
# ---------------------------------------------------------------------------
def _torch():
    import torch

    return torch


def _ptr(t, name, dtype=None, numel=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


class Pool:
    """A paged KV pool in device memory (bf16 payload, page size 16)."""

    def __init__(self, num_layers, num_pages, num_kv_heads, head_dim, device="cuda", fill=None):
        torch = _torch()
        lib = load()
        nbytes = lib.kvs_pool_bytes(num_layers, num_pages, num_kv_heads, head_dim, PAGE)
        if nbytes == 0:
            raise ValueError("invalid pool shape")
        if fill is None:
            self.data = torch.empty(nbytes // 2, dtype=torch.int16, device=device)
        else:
            self.data = torch.full((nbytes // 2,), int(fill), dtype=torch.int16, device=device)
        self.num_layers, self.num_pages = int(num_layers), int(num_pages)
        self.num_kv_heads, self.head_dim = int(num_kv_heads), int(head_dim)
        self._struct = KvsPool(self.data.data_ptr(), self.num_layers, self.num_pages,
                               self.num_kv_heads, self.head_dim, PAGE)

    @property
    def struct(self):
        return ctypes.byref(self._struct)

    @property
    def nbytes(self) -> int:
        return self.data.numel() * 2


def append(pool: Pool, layer, k_new, v_new, cu_new, block_table, seq_lens, max_new, max_seq_len,
           dev_status=None, stream=None):
    torch = _torch()
    batch = seq_lens.numel()
    total = k_new.shape[0]
    row = pool.num_kv_heads * pool.head_dim
    _check(load().kv_pool_append(
        pool.struct, layer, _ptr(k_new, "k_new", torch.bfloat16, total * row),
        _ptr(v_new, "v_new", torch.bfloat16, total * row), _ptr(cu_new, "cu_new", torch.int32, batch + 1),
        _ptr(block_table, "block_table", torch.int32), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", torch.int32), batch, total, max_new, max_seq_len,
        _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True), _stream(stream)))


def append_check(pool: Pool, cu_new, block_table, seq_lens, total_new, max_new, max_seq_len, scratch,
                 dev_status, stream=None):
    """kv_pool_append_check: OR KVS_DEV_ALIAS into dev_status when the append with these
    arguments would write one physical slot for two logical slots."""
    torch = _torch()
    batch = seq_lens.numel()
    _check(load().kv_pool_append_check(
        pool.struct, _ptr(cu_new, "cu_new", torch.int32, batch + 1), _ptr(block_table, "block_table", torch.int32),
        block_table.shape[1], _ptr(seq_lens, "seq_lens", torch.int32), batch, total_new, max_new, max_seq_len,
        _ptr(scratch, "scratch"), scratch.numel() * scratch.element_size(),
        _ptr(dev_status, "dev_status", torch.int32, 1), _stream(stream)))


def append_check_bytes(num_pages) -> int:
    return load().kv_pool_append_check_bytes(num_pages)


def decode_workspace_bytes(batch, num_decoders, num_q_heads, num_kv_heads, head_dim, max_seq_len) -> int:
    return load().shared_kv_decode_workspace_bytes(batch, num_decoders, num_q_heads, num_kv_heads,
                                                   head_dim, max_seq_len)


def decode_workspace_init(workspace, stream=None):
    """Zero a decode workspace's arrival counters (needed once, before its first call,
    unless the buffer was allocated zero-filled)."""
    _check(load().shared_kv_decode_workspace_init(_ptr(workspace, "workspace"),
                                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def decode_workspace(batch, num_decoders, num_q_heads, num_kv_heads, head_dim, max_seq_len, device="cuda"):
    """A zero-filled uint8 device tensor of decode_workspace_bytes: ready for every decode call."""
    torch = _torch()
    nbytes = decode_workspace_bytes(batch, num_decoders, num_q_heads, num_kv_heads, head_dim, max_seq_len)
    if nbytes == 0:
        raise ValueError("invalid decode bounds")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def decode(pool: Pool, layer, q, out, block_table, seq_lens, max_seq_len, scale, workspace,
           dev_status=None, stream=None):
    """q, out: bf16 [B, N, H_q, D]; workspace: a uint8 device tensor of decode_workspace_bytes."""
    torch = _torch()
    B, N, Hq, D = q.shape
    if D != pool.head_dim or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q/out shape does not match the pool")
    _check(load().shared_kv_decode(
        pool.struct, layer, _ptr(q, "q", torch.bfloat16), _ptr(out, "out", torch.bfloat16),
        _ptr(block_table, "block_table", torch.int32), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", torch.int32, B), B, N, Hq, max_seq_len, float(scale),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True), _stream(stream)))


def decode_noalloc(pool: Pool, layer, q, out, block_table, seq_lens, max_seq_len, scale, dev_status=None,
                   stream=None):
    """decode() with the library's static scratch instead of a workspace (allocates nothing)."""
    torch = _torch()
    B, N, Hq, D = q.shape
    if D != pool.head_dim or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q/out shape does not match the pool")
    _check(load().shared_kv_decode_noalloc(
        pool.struct, layer, _ptr(q, "q", torch.bfloat16), _ptr(out, "out", torch.bfloat16),
        _ptr(block_table, "block_table", torch.int32), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", torch.int32, B), B, N, Hq, max_seq_len, float(scale),
        _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True), _stream(stream)))


def decode_append(pool: Pool, layer, k_new, v_new, q, out, block_table, seq_lens, max_seq_len, scale, workspace,
                  dev_status=None, stream=None):
    """Append the step's token (k_new, v_new: bf16 [B, H_kv, D], written at position seq_lens[b] - 1),
    then decode over seq_lens[b] tokens, in one call.  q, out, workspace as for decode."""
    torch = _torch()
    B, N, Hq, D = q.shape
    if D != pool.head_dim or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q/out shape does not match the pool")
    n_kv = B * pool.num_kv_heads * D
    _check(load().shared_kv_decode_append(
        pool.struct, layer, _ptr(k_new, "k_new", torch.bfloat16, n_kv), _ptr(v_new, "v_new", torch.bfloat16, n_kv),
        _ptr(q, "q", torch.bfloat16), _ptr(out, "out", torch.bfloat16),
        _ptr(block_table, "block_table", torch.int32), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", torch.int32, B), B, N, Hq, max_seq_len, float(scale),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True), _stream(stream)))


def decode_private(pool: Pool, layer, q, out, block_table, seq_lens, priv_block_table, priv_lens,
                   max_seq_len, max_priv_len, scale, workspace, dev_status=None, stream=None):
    """Shared prefix + per-decoder private suffix.  q, out: bf16 [B, N, H_q, D];
    priv_block_table: int32 [B*N, S_p]; priv_lens: int32 [B*N]; workspace as for decode."""
    torch = _torch()
    B, N, Hq, D = q.shape
    if D != pool.head_dim or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q/out shape does not match the pool")
    if priv_block_table.dim() != 2 or priv_block_table.shape[0] != B * N:
        raise ValueError("priv_block_table must be [batch*num_decoders, stride]")
    _check(load().shared_kv_decode_private(
        pool.struct, layer, _ptr(q, "q", torch.bfloat16), _ptr(out, "out", torch.bfloat16),
        _ptr(block_table, "block_table", torch.int32), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", torch.int32, B),
        _ptr(priv_block_table, "priv_block_table", torch.int32), priv_block_table.shape[1],
        _ptr(priv_lens, "priv_lens", torch.int32, B * N), B, N, Hq, max_seq_len, max_priv_len, float(scale),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True), _stream(stream)))


def decode_cascade(pool: Pool, layer, q, out, block_table, seq_lens, group_id, group_prefix_pages, max_seq_len,
                   scale, workspace, dev_status=None, stream=None):
    """shared_kv_decode where adjacent sessions with equal group_id share their first
    group_prefix_pages pages (int32 [B] each); q, out: bf16 [B, N, H_q, D]."""
    torch = _torch()
    B, N, Hq, D = q.shape
    if D != pool.head_dim or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q/out shape does not match the pool")
    _check(load().shared_kv_decode_cascade(
        pool.struct, layer, _ptr(q, "q", torch.bfloat16), _ptr(out, "out", torch.bfloat16),
        _ptr(block_table, "block_table", torch.int32), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", torch.int32, B), _ptr(group_id, "group_id", torch.int32, B),
        _ptr(group_prefix_pages, "group_prefix_pages", torch.int32, B), B, N, Hq, max_seq_len, float(scale),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True), _stream(stream)))


def extend(pool: Pool, layer, q, k_new, v_new, out, cu_new, block_table, seq_lens, max_new,
           max_seq_len, scale, dev_status=None, stream=None):
    """q, out: bf16 [T, H_q, D]; k_new, v_new: bf16 [T, H_kv, D]."""
    torch = _torch()
    T, Hq, D = q.shape
    batch = seq_lens.numel()
    row = pool.num_kv_heads * pool.head_dim
    if D != pool.head_dim or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q/out shape does not match the pool")
    _check(load().partial_prefill_extend(
        pool.struct, layer, _ptr(q, "q", torch.bfloat16), _ptr(k_new, "k_new", torch.bfloat16, T * row),
        _ptr(v_new, "v_new", torch.bfloat16, T * row), _ptr(out, "out", torch.bfloat16),
        _ptr(cu_new, "cu_new", torch.int32, batch + 1), _ptr(block_table, "block_table", torch.int32),
        block_table.shape[1], _ptr(seq_lens, "seq_lens", torch.int32), batch, Hq, T, max_new,
        max_seq_len, float(scale), _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True),
        _stream(stream)))


def extend_layers(pool: Pool, layer_begin, q, k_new, v_new, out, cu_new, block_table, seq_lens, max_new,
                  max_seq_len, scale, dev_status=None, stream=None):
    """partial_prefill_layers: q, out bf16 [L, T, H_q, D]; k_new, v_new bf16 [L, T, H_kv, D]."""
    torch = _torch()
    L, T, Hq, D = q.shape
    batch = seq_lens.numel()
    row = pool.num_kv_heads * pool.head_dim
    if D != pool.head_dim or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q/out shape does not match the pool")
    _check(load().partial_prefill_layers(
        pool.struct, layer_begin, L, _ptr(q, "q", torch.bfloat16), _ptr(k_new, "k_new", torch.bfloat16, L * T * row),
        _ptr(v_new, "v_new", torch.bfloat16, L * T * row), _ptr(out, "out", torch.bfloat16),
        _ptr(cu_new, "cu_new", torch.int32, batch + 1), _ptr(block_table, "block_table", torch.int32),
        block_table.shape[1], _ptr(seq_lens, "seq_lens", torch.int32), batch, Hq, T, max_new,
        max_seq_len, float(scale), _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True),
        _stream(stream)))


def pages_buffer_bytes(pool: Pool, num_layers, num_ids) -> int:
    return load().kv_pages_buffer_bytes(pool.struct, num_layers, num_ids)


def pack(pool: Pool, layer_begin, num_layers, page_ids, buf, dev_status=None, stream=None):
    """All KV heads' tiles of the listed pages, layers [layer_begin, +num_layers), into buf
    (a device tensor of pages_buffer_bytes bytes), as [layer][page][head][tile]."""
    torch = _torch()
    n = page_ids.numel()
    need = pages_buffer_bytes(pool, num_layers, n)
    if buf.numel() * buf.element_size() < need:
        raise ValueError(f"buf must hold {need} bytes")
    _check(load().kv_pages_pack(pool.struct, layer_begin, num_layers, _ptr(page_ids, "page_ids", torch.int32), n,
                                _ptr(buf, "buf"), _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True),
                                _stream(stream)))


def unpack(pool: Pool, layer_begin, num_layers, page_ids, buf, dev_status=None, stream=None):
    """The inverse of pack: buffer entry i goes to page page_ids[i] of `pool`."""
    torch = _torch()
    n = page_ids.numel()
    need = pages_buffer_bytes(pool, num_layers, n)
    if buf.numel() * buf.element_size() < need:
        raise ValueError(f"buf must hold {need} bytes")
    _check(load().kv_pages_unpack(pool.struct, layer_begin, num_layers, _ptr(page_ids, "page_ids", torch.int32),
                                  n, _ptr(buf, "buf"),
                                  _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True),
                                  _stream(stream)))


def fetch(pool: Pool, layer, block_table, seq_lens, cu_rows, max_seq_len, k_out, v_out, dev_status=None,
          stream=None):
    """Logical K/V rows of each session into k_out / v_out: bf16 [total_rows, H_kv, D]."""
    torch = _torch()
    batch = seq_lens.numel()
    total = k_out.shape[0]
    row = pool.num_kv_heads * pool.head_dim
    _check(load().kv_pool_fetch(
        pool.struct, layer, _ptr(block_table, "block_table", torch.int32), block_table.shape[1],
        _ptr(seq_lens, "seq_lens", torch.int32), _ptr(cu_rows, "cu_rows", torch.int32, batch + 1), batch, total,
        max_seq_len, _ptr(k_out, "k_out", torch.bfloat16, total * row), _ptr(v_out, "v_out", torch.bfloat16, total * row),
        _ptr(dev_status, "dev_status", torch.int32, 1, allow_none=True), _stream(stream)))


# ---------------------------------------------------------------------------
# Host-side prefix cache (kvs_prefix_cache.h): host int32 arrays, no GPU.
# ---------------------------------------------------------------------------
def _host_i32(x, n=None):
    import numpy as np

    a = np.ascontiguousarray(x, dtype=np.int32)
    if n is not None and a.size < n:
        raise ValueError(f"need at least {n} int32 values, got {a.size}")
    return a


def _aptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a.size else None


class PrefixCache:
    """Page allocator with a prefix cache of full 16-token blocks."""

    def __init__(self, num_pages: int):
        self._h = load().kvs_prefix_cache_create(int(num_pages))
        if not self._h:
            raise KvsError(KVS_EINVAL, last_error())
        self.num_pages = int(num_pages)

    def close(self):
        if self._h:
            load().kvs_prefix_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def admit(self, tokens):
        """Page ids (int32 array of ceil(L/16)) and the count of reused leading pages."""
        import numpy as np

        t = _host_i32(tokens)
        out = np.zeros(max((t.size + PAGE - 1) // PAGE, 1), np.int32)
        matched = ctypes.c_int32(0)
        _check(load().kvs_prefix_cache_admit(self._h, _aptr(t), int(t.size), _aptr(out), ctypes.byref(matched)))
        return out[:(t.size + PAGE - 1) // PAGE], int(matched.value)

    def publish(self, tokens, pages):
        t = _host_i32(tokens)
        p = _host_i32(pages, t.size // PAGE)
        _check(load().kvs_prefix_cache_publish(self._h, _aptr(t), int(t.size), _aptr(p)))

    def release(self, pages):
        p = _host_i32(pages)
        _check(load().kvs_prefix_cache_release(self._h, _aptr(p), int(p.size)))

    def stats(self):
        """(free, evictable, referenced, entries)"""
        v = [ctypes.c_int32(0) for _ in range(4)]
        _check(load().kvs_prefix_cache_stats(self._h, *[ctypes.byref(x) for x in v]))
        return tuple(int(x.value) for x in v)

    def refcount(self, page: int) -> int:
        r = load().kvs_prefix_cache_refcount(self._h, int(page))
        if r < 0:
            _check(r)
        return r


def prefix_groups(block_table, seq_lens):
    """(group_id, group_prefix_pages) int32 arrays for decode_cascade, from host tables."""
    import numpy as np

    bt = _host_i32(block_table)
    lens = _host_i32(seq_lens)
    B = lens.size
    if bt.ndim != 2 or bt.shape[0] != B:
        raise ValueError("block_table must be [batch, stride]")
    gid, pref = np.zeros(B, np.int32), np.zeros(B, np.int32)
    _check(load().kvs_prefix_groups(_aptr(bt), int(bt.shape[1]), _aptr(lens), int(B), _aptr(gid), _aptr(pref)))
    return gid, pref
