"""CPU oracle for shared-KV attention — TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module.  The library never does: it has no CPU fallback.

What it computes (plain, slow, float64, no blocking or fusion):

* The pages' decomposition of a decoder-only transformer (ICaRus, Method /
  overall framework): a frozen logical encoder E_base writes K_{1:i}, V_{1:i}
  once; every task decoder computes x_{i+1} = D(x_i, K_{1:i}, V_{1:i}) by
  attending over that one cache.  The attention inside D is ordinary scaled
  dot-product attention; nothing in the method approximates it, so the oracle
  is that definition written out (softmax over all cached tokens).
* Key design 3 of the same page concatenates the query heads of every party
  that reads the same KV.  That only changes how the work is scheduled, so the
  oracle attends each (decoder, head) row separately: the concatenated kernel
  must reproduce the per-row results.
* Cached-prefix extension (PrefillShare, sections 3.3 and 7: partial prefill of
  the new tokens only; section 4: prefill with an empty past) — row i of the
  chunk sees the prefix and chunk tokens up to and including itself.
* The cache store: new K/V rows are copied bit for bit into their page slots
  (PrefillShare section 3.3: the KV is managed in blocks/pages).

Readings taken where the pages are silent (each also listed in the design
notes): query head h uses KV head h // G with G = H_q / H_kv; an empty
context gives a zero output; the causal diagonal is included; page size 16.

The pool index map below is re-implemented from the layout documented in the
library header; it is the only contract shared with the GPU side.
"""
from __future__ import annotations

import numpy as np

PAGE = 16


# ---------------------------------------------------------------------------
# bf16 <-> float64 (exact: every bf16 value is a float32, every float32 a float64)
# ---------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode raw bfloat16 bit patterns (uint16) into float64, exactly."""
    bits = np.asarray(bits, dtype=np.uint16)
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


# ---------------------------------------------------------------------------
# Pool index map (the documented layout)
# ---------------------------------------------------------------------------
def tile_elems(head_dim: int) -> int:
    """Elements in one (layer, page, head) tile: 16 K rows and 16 V rows."""
    return 2 * PAGE * head_dim


def k_offset(t: int, d: int) -> int:
    """Offset of K(slot t, dim d) inside the K part of a tile."""
    group = d // 32           # which 32-wide slab of the head dim
    sub = (d % 32) // 8       # which 8-element run inside the slab
    lane = sub * 16 + t
    return (group * 64 + lane) * 8 + d % 8


def v_offset(t: int, d: int) -> int:
    """Offset of V(slot t, dim d) inside the V part of a tile."""
    slab = d // 16                  # which 16-wide slab of the head dim
    run = (t // 8) * 16 + d % 16    # 8 consecutive slots of one head-dim value
    return (slab * 32 + run) * 8 + t % 8


def tile_start(layer: int, page: int, head: int, num_pages: int, num_kv_heads: int,
               head_dim: int) -> int:
    return ((layer * num_pages + page) * num_kv_heads + head) * tile_elems(head_dim)


def pool_elems(num_layers: int, num_pages: int, num_kv_heads: int, head_dim: int) -> int:
    return num_layers * num_pages * num_kv_heads * tile_elems(head_dim)


class PoolShape:
    """Shape of a pool; the pool itself is a flat uint16 array of bf16 bits."""

    def __init__(self, num_layers, num_pages, num_kv_heads, head_dim):
        self.num_layers = int(num_layers)
        self.num_pages = int(num_pages)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)

    @property
    def elems(self) -> int:
        return pool_elems(self.num_layers, self.num_pages, self.num_kv_heads, self.head_dim)

    def slot_index(self, layer, page, head, t, d, which):
        """Flat element index of K (which=0) or V (which=1) at (page, head, t, d)."""
        base = tile_start(layer, page, head, self.num_pages, self.num_kv_heads, self.head_dim)
        if which == 0:
            return base + k_offset(t, d)
        return base + PAGE * self.head_dim + v_offset(t, d)

    def index_tables(self):
        """[16, D] tables of in-tile offsets for K and for V (V already past the K part)."""
        D = self.head_dim
        kt = np.empty((PAGE, D), dtype=np.int64)
        vt = np.empty((PAGE, D), dtype=np.int64)
        for t in range(PAGE):
            for d in range(D):
                kt[t, d] = k_offset(t, d)
                vt[t, d] = PAGE * D + v_offset(t, d)
        return kt, vt


# ---------------------------------------------------------------------------
# The cache store (append)
# ---------------------------------------------------------------------------
def append(pool: np.ndarray, shape: PoolShape, layer: int, k_new: np.ndarray, v_new: np.ndarray,
           cu_new, block_table: np.ndarray, seq_lens) -> np.ndarray:
    """Return a copy of `pool` with each new row written into its page slot.

    Row j of session b (rows cu_new[b] .. cu_new[b+1]-1 of k_new/v_new, each
    [H_kv, D] bf16 bits) goes to logical position p = seq_lens[b] + j, i.e.
    page block_table[b, p // 16], slot p % 16.  Bits are copied unchanged.
    """
    out = np.array(pool, dtype=np.uint16, copy=True)
    k_new = np.asarray(k_new, dtype=np.uint16)
    v_new = np.asarray(v_new, dtype=np.uint16)
    kt, vt = shape.index_tables()
    for b in range(len(seq_lens)):
        for j in range(int(cu_new[b + 1]) - int(cu_new[b])):
            row = int(cu_new[b]) + j
            p = int(seq_lens[b]) + j
            page = int(block_table[b, p // PAGE])
            slot = p % PAGE
            for h in range(shape.num_kv_heads):
                base = tile_start(layer, page, h, shape.num_pages, shape.num_kv_heads, shape.head_dim)
                out[base + kt[slot]] = k_new[row, h]
                out[base + vt[slot]] = v_new[row, h]
    return out


def append_aliasing(block_table: np.ndarray, seq_lens, cu_new, num_pages: int, max_new: int,
                    max_seq_len: int) -> bool:
    """True when an append would write one physical slot for two logical slots.

    Pages hold a session's positions in blocks (PrefillShare, section 3.3), and
    full, block-aligned prefix blocks may be mapped into several sessions' tables
    (Prefill-as-a-Service, component 3), so one physical slot may be *live* for
    several sessions: that is sharing, not a fault.  A write is a fault when the
    physical slot (page, slot) of a new token of the call
      - is also the slot of another new token of the call, or
      - holds a live token of a session of the batch: position q < seq_lens[c]
        of any session c (the writing session included).
    Slots whose page id lies outside [0, num_pages), and sessions whose lengths
    the append rejects, write nothing and are left out, as the append leaves them.
    """
    B = len(seq_lens)
    live = set()
    for c in range(B):
        L = int(seq_lens[c])
        if L < 0 or L > max_seq_len:
            continue
        for q in range(L):
            page = int(block_table[c, q // PAGE])
            if 0 <= page < num_pages:
                live.add((page, q % PAGE))
    written = set()
    total_new = int(cu_new[B])
    for b in range(B):
        P, c0, c1 = int(seq_lens[b]), int(cu_new[b]), int(cu_new[b + 1])
        n = c1 - c0
        if P < 0 or n < 0 or n > max_new or P + n > max_seq_len or c0 < 0 or c1 > total_new:
            continue
        for p in range(P, P + n):
            page = int(block_table[b, p // PAGE])
            if not 0 <= page < num_pages:
                continue
            key = (page, p % PAGE)
            if key in written or key in live:
                return True
            written.add(key)
    return False


# ---------------------------------------------------------------------------
# Gather a session's logical K/V from its pages
# ---------------------------------------------------------------------------
def gather(pool: np.ndarray, shape: PoolShape, layer: int, bt_row, length: int):
    """K, V as float64 [length, H_kv, D] for logical positions 0 .. length-1."""
    H, D = shape.num_kv_heads, shape.head_dim
    kt, vt = shape.index_tables()
    K = np.empty((length, H, D), dtype=np.float64)
    V = np.empty((length, H, D), dtype=np.float64)
    for p in range(length):
        page = int(bt_row[p // PAGE])
        slot = p % PAGE
        for h in range(H):
            base = tile_start(layer, page, h, shape.num_pages, H, D)
            K[p, h] = bf16_to_f64(pool[base + kt[slot]])
            V[p, h] = bf16_to_f64(pool[base + vt[slot]])
    return K, V


def fetch(pool: np.ndarray, shape: PoolShape, layer: int, block_table: np.ndarray, seq_lens):
    """The logical K, V rows of every session, as bf16 bits [sum(seq_lens), H_kv, D].

    The inverse of `append` (DroidSpeak, section 5.4: fetch reads what store
    wrote): row cu[b] + p holds logical position p of session b, p < seq_lens[b].
    """
    H, D = shape.num_kv_heads, shape.head_dim
    kt, vt = shape.index_tables()
    total = sum(int(L) for L in seq_lens)
    K = np.empty((total, H, D), dtype=np.uint16)
    V = np.empty((total, H, D), dtype=np.uint16)
    row = 0
    for b in range(len(seq_lens)):
        for p in range(int(seq_lens[b])):
            page = int(block_table[b, p // PAGE])
            slot = p % PAGE
            for h in range(H):
                base = tile_start(layer, page, h, shape.num_pages, H, D)
                K[row, h] = pool[base + kt[slot]]
                V[row, h] = pool[base + vt[slot]]
            row += 1
    return K, V


# ---------------------------------------------------------------------------
# Page handoff between pools (PrefillShare, section 3.3: the prefill worker
# hands the cache it wrote, kept in fixed-size blocks, to the decode worker)
# ---------------------------------------------------------------------------
def pack(pool: np.ndarray, shape: PoolShape, layer_begin: int, num_layers: int, page_ids) -> np.ndarray:
    """Transfer buffer [num_layers][len(page_ids)][H_kv][tile] of the listed pages' tiles."""
    H, D = shape.num_kv_heads, shape.head_dim
    te = tile_elems(D)
    buf = np.empty((num_layers, len(page_ids), H, te), dtype=np.uint16)
    for li in range(num_layers):
        for i, pid in enumerate(page_ids):
            for h in range(H):
                base = tile_start(layer_begin + li, int(pid), h, shape.num_pages, H, D)
                buf[li, i, h] = pool[base:base + te]
    return buf


def unpack(pool: np.ndarray, shape: PoolShape, layer_begin: int, num_layers: int, page_ids,
           buf: np.ndarray) -> np.ndarray:
    """Copy of `pool` with entry i of the transfer buffer written to page page_ids[i]."""
    H, D = shape.num_kv_heads, shape.head_dim
    te = tile_elems(D)
    out = np.array(pool, dtype=np.uint16, copy=True)
    buf = np.asarray(buf, dtype=np.uint16).reshape(num_layers, len(page_ids), H, te)
    for li in range(num_layers):
        for i, pid in enumerate(page_ids):
            for h in range(H):
                base = tile_start(layer_begin + li, int(pid), h, shape.num_pages, H, D)
                out[base:base + te] = buf[li, i, h]
    return out


# ---------------------------------------------------------------------------
# Attention by definition
# ---------------------------------------------------------------------------
def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for one query row q [D] over K, V [L, D].

    Returns zeros for an empty context (L == 0), the convention adopted for a
    softmax over nothing.
    """
    L = K.shape[0]
    if L == 0:
        return np.zeros(K.shape[1], dtype=np.float64)
    s = scale * (K @ q)              # [L]
    m = s.max()
    w = np.exp(s - m)                # subtracting the max leaves softmax unchanged
    return (w @ V) / w.sum()


def decode(pool: np.ndarray, shape: PoolShape, layer: int, q_bits: np.ndarray,
           block_table: np.ndarray, seq_lens, scale: float, sessions=None) -> np.ndarray:
    """Decode attention of N decoders over the shared cache.

    q_bits: bf16 bits [B, N, H_q, D].  For session b, decoder n, head h the row
    attends K/V head h // G over positions 0 .. seq_lens[b]-1.  Returns float64
    [B, N, H_q, D]; sessions not listed in `sessions` (when given) stay zero.
    """
    B, N, Hq, D = q_bits.shape
    G = Hq // shape.num_kv_heads
    q = bf16_to_f64(q_bits)
    out = np.zeros((B, N, Hq, D), dtype=np.float64)
    for b in (range(B) if sessions is None else sessions):
        L = int(seq_lens[b])
        K, V = gather(pool, shape, layer, block_table[b], L)
        for n in range(N):
            for h in range(Hq):
                g = h // G
                out[b, n, h] = attend(q[b, n, h], K[:, g], V[:, g], scale)
    return out


def decode_private(pool: np.ndarray, shape: PoolShape, layer: int, q_bits: np.ndarray,
                   block_table: np.ndarray, seq_lens, priv_table: np.ndarray, priv_lens, scale: float,
                   sessions=None) -> np.ndarray:
    """Decode attention over a shared prefix plus each decoder's private suffix.

    PrefillShare, section 3.3: every decoder starts from the base model's cache
    C_base and then extends it with its own generated tokens (the decoder-private
    Delta C_t); the memory model of Eq. 9 keeps the shared prefix once and only
    the private parts per decoder.  Decoder n of session b therefore attends the
    sequence  shared prefix (seq_lens[b] tokens through block_table[b])  followed
    by  its private suffix (priv_lens[b*N + n] tokens through priv_table[b*N + n]).
    Returns float64 [B, N, H_q, D]; sessions not in `sessions` stay zero.
    """
    B, N, Hq, D = q_bits.shape
    G = Hq // shape.num_kv_heads
    q = bf16_to_f64(q_bits)
    out = np.zeros((B, N, Hq, D), dtype=np.float64)
    for b in (range(B) if sessions is None else sessions):
        Ks, Vs = gather(pool, shape, layer, block_table[b], int(seq_lens[b]))
        for n in range(N):
            Kp, Vp = gather(pool, shape, layer, priv_table[b * N + n], int(priv_lens[b * N + n]))
            K = np.concatenate([Ks, Kp])
            V = np.concatenate([Vs, Vp])
            for h in range(Hq):
                g = h // G
                out[b, n, h] = attend(q[b, n, h], K[:, g], V[:, g], scale)
    return out


def extend(pool: np.ndarray, shape: PoolShape, layer: int, q_bits: np.ndarray, k_new: np.ndarray,
           v_new: np.ndarray, cu_new, block_table: np.ndarray, seq_lens, scale: float,
           sessions=None, rows=None):
    """Partial prefill: append the chunk, then attend each new row causally.

    q_bits: bf16 bits [T_new, H_q, D]; k_new/v_new [T_new, H_kv, D].  Row i of
    session b sits at absolute position p = seq_lens[b] + i and attends
    positions 0 .. p of the extended cache.  Returns (out float64 [T_new, H_q, D],
    extended pool).  `sessions` / `rows` (a dict b -> list of i) restrict which
    outputs are computed; the pool is always fully extended.
    """
    new_pool = append(pool, shape, layer, k_new, v_new, cu_new, block_table, seq_lens)
    T, Hq, D = q_bits.shape
    G = Hq // shape.num_kv_heads
    q = bf16_to_f64(q_bits)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for b in (range(len(seq_lens)) if sessions is None else sessions):
        P = int(seq_lens[b])
        C = int(cu_new[b + 1]) - int(cu_new[b])
        K, V = gather(new_pool, shape, layer, block_table[b], P + C)
        chosen = range(C) if rows is None or b not in rows else rows[b]
        for i in chosen:
            p = P + i
            r = int(cu_new[b]) + i
            for h in range(Hq):
                g = h // G
                out[r, h] = attend(q[r, h], K[: p + 1, g], V[: p + 1, g], scale)
    return out, new_pool


def decode_from_logical(q_bits: np.ndarray, K_bits, V_bits, scale: float) -> np.ndarray:
    """Decode attention from logical per-session K/V (no pool involved).

    q_bits [B, N, H_q, D]; K_bits[b], V_bits[b]: bf16 bits [L_b, H_kv, D].  Used
    where the full pool is too large for a host copy: the sampled sessions'
    logical K/V come straight from the input generator.
    """
    B, N, Hq, D = q_bits.shape
    q = bf16_to_f64(q_bits)
    out = np.zeros((B, N, Hq, D), dtype=np.float64)
    for b in range(B):
        if K_bits[b] is None:
            continue
        K = bf16_to_f64(K_bits[b])
        V = bf16_to_f64(V_bits[b])
        G = Hq // K.shape[1]
        for n in range(N):
            for h in range(Hq):
                out[b, n, h] = attend(q[b, n, h], K[:, h // G], V[:, h // G], scale)
    return out


def extend_from_logical(q_bits: np.ndarray, K_bits: np.ndarray, V_bits: np.ndarray, prefix: int,
                        rows, scale: float) -> np.ndarray:
    """Partial-prefill rows of ONE session from its logical K/V (no pool).

    q_bits [C, H_q, D] for the chunk; K_bits/V_bits [prefix + C, H_kv, D]; row i
    attends positions 0 .. prefix + i.  Returns float64 [len(rows), H_q, D].
    """
    q = bf16_to_f64(q_bits)
    K = bf16_to_f64(K_bits)
    V = bf16_to_f64(V_bits)
    Hq = q.shape[1]
    G = Hq // K.shape[1]
    out = np.zeros((len(rows), Hq, q.shape[2]), dtype=np.float64)
    for k, i in enumerate(rows):
        p = prefix + int(i)
        for h in range(Hq):
            out[k, h] = attend(q[int(i), h], K[: p + 1, h // G], V[: p + 1, h // G], scale)
    return out
