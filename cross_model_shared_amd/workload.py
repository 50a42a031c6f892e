"""Seeded synthetic inputs for the shared-KV attention path.

This module only draws inputs: context lengths, block tables (a host page
allocator with shuffled physical pages), and bf16 tensors.  It holds none of the
attention arithmetic and is the one piece of code that both the library's
callers and the CPU oracle's tests use.

Workloads (shapes of the pages' agentic multi-model sessions; values are i.i.d.
normal, no trained weights exist here):

* tiny            — 2 sessions (lengths 200 and 256), N=2 decoders, 2 KV heads,
                    4 query heads per KV head per decoder, D=64, N(0, 0.5^2).
* llama8b_n4      — Llama-3.1-8B-shaped layer: 32 q / 8 KV heads, D=128, N=4,
                    32 sessions, lengths log-uniform in [1K, 8K].
* qwen3_8b_n8     — Qwen3-8B-shaped 8-model agentic decode: 32 q / 8 KV heads,
                    D=128, N=8, 64 sessions, lengths uniform in [4K, 16K],
                    36 layers.
* extend_8k_512   — 16 sessions, cached 8K prefix + 512 new tokens, 32 q / 8 KV
                    heads, D=128.
* qwen3_14b_long  — Qwen3-14B-shaped: 40 q / 8 KV heads, D=128, N=2, 8 sessions,
                    lengths truncated log-normal (sigma 1, mu 9.7869, truncated
                    to [4K, 128K], mean ~27K).
* handoff_8k      — 4 sessions of 8K tokens, Qwen3-8B-shaped (8 KV heads, D=128),
                    36 layers: the cache a prefill worker hands to a decode worker.
* llama8b_layer_group — Llama-3.1-8B-shaped (32 q / 8 KV heads, D=128, 32
                    layers): 8 prompts of 4096 tokens recomputed in full (no cached
                    prefix) in the 4-layer group [12, 16), one call for the group.
* qwen3_8b_n8_cascade — Qwen3-8B-shaped N=8 decode of 64 sessions in 32 pairs;
                    each pair shares a prefix-cached prefix of 4K-8K tokens (whole
                    pages), and each session adds 0-8K tokens of its own.
* qwen3_8b_n8_private — qwen3_8b_n8's sessions and shared prefixes, plus a
                    private suffix per decoder (its own generated tokens),
                    lengths uniform in [0, 2048].

1K = 1024 tokens.  bf16 values are float32 normal draws rounded to nearest even.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE = 16


@dataclass
class Workload:
    name: str
    batch: int
    num_decoders: int          # N (decode) — 1 for extend workloads
    num_q_heads: int           # H_q per decoder
    num_kv_heads: int
    head_dim: int
    num_layers: int
    std: float
    seed: int
    kind: str                  # "decode" or "extend"
    lens: list = field(default_factory=list)      # decode: tokens attended
    prefix: list = field(default_factory=list)    # extend: cached prefix
    new: list = field(default_factory=list)       # extend: new chunk sizes
    priv: list = field(default_factory=list)      # decode: private suffix of decoder n of session b at b*N + n
    groups: list = field(default_factory=list)    # decode: (shared prefix tokens, [session lengths]) per group
    layer_group: tuple = ()                       # extend: (first layer, layer count) recomputed together

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def total_lens(self):
        if self.kind == "decode":
            return list(self.lens)
        return [p + c for p, c in zip(self.prefix, self.new)]


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def truncated_lognormal(rng, n, mu, sigma, lo, hi):
    """Rejection-truncated log-normal integer lengths in [lo, hi]."""
    out = []
    while len(out) < n:
        x = int(math.floor(math.exp(rng.normal(mu, sigma))))
        if lo <= x <= hi:
            out.append(x)
    return out


def make_workload(name: str, seed: int | None = None) -> Workload:
    if name == "tiny":
        s = 0 if seed is None else seed
        return Workload(name, 2, 2, 8, 2, 64, 1, 0.5, s, "decode", lens=[200, 256])
    if name == "llama8b_n4":
        s = 1 if seed is None else seed
        r = _rng(s, 0)
        lens = [int(math.floor(math.exp(r.uniform(math.log(1024), math.log(8192)))))
                for _ in range(32)]
        return Workload(name, 32, 4, 32, 8, 128, 1, 1.0, s, "decode", lens=lens)
    if name == "qwen3_8b_n8":
        s = 2 if seed is None else seed
        r = _rng(s, 0)
        lens = [int(x) for x in r.integers(4096, 16384, size=64, endpoint=True)]
        return Workload(name, 64, 8, 32, 8, 128, 36, 1.0, s, "decode", lens=lens)
    if name == "qwen3_8b_n8_private":
        s = 2 if seed is None else seed
        base = make_workload("qwen3_8b_n8", s)
        r = _rng(s, 5)
        priv = [int(x) for x in r.integers(0, 2048, size=base.batch * base.num_decoders, endpoint=True)]
        return Workload(name, base.batch, base.num_decoders, base.num_q_heads, base.num_kv_heads,
                        base.head_dim, 1, base.std, s, "decode", lens=base.lens, priv=priv)
    if name == "qwen3_8b_n8_cascade":
        s = 6 if seed is None else seed
        r = _rng(s, 0)
        groups = []
        for _ in range(32):
            pre = int(r.integers(256, 512, endpoint=True)) * PAGE
            groups.append((pre, [pre + int(x) for x in r.integers(0, 8192, size=2, endpoint=True)]))
        lens = [L for _, ls in groups for L in ls]
        return Workload(name, 64, 8, 32, 8, 128, 1, 1.0, s, "decode", lens=lens, groups=groups)
    if name == "llama8b_layer_group":
        s = 7 if seed is None else seed
        return Workload(name, 8, 1, 32, 8, 128, 32, 1.0, s, "extend", prefix=[0] * 8, new=[4096] * 8,
                        layer_group=(12, 4))
    if name == "handoff_8k":
        s = 5 if seed is None else seed
        return Workload(name, 4, 1, 32, 8, 128, 36, 1.0, s, "decode", lens=[8192] * 4)
    if name == "extend_8k_512":
        s = 3 if seed is None else seed
        return Workload(name, 16, 1, 32, 8, 128, 1, 1.0, s, "extend",
                        prefix=[8192] * 16, new=[512] * 16)
    if name == "qwen3_14b_long":
        s = 4 if seed is None else seed
        r = _rng(s, 0)
        lens = truncated_lognormal(r, 8, 9.7869, 1.0, 4096, 131072)
        return Workload(name, 8, 2, 40, 8, 128, 1, 1.0, s, "decode", lens=lens)
    raise KeyError(name)


WORKLOADS = ("tiny", "llama8b_n4", "qwen3_8b_n8", "extend_8k_512", "qwen3_14b_long", "qwen3_8b_n8_private",
             "handoff_8k", "qwen3_8b_n8_cascade", "llama8b_layer_group")


# ---------------------------------------------------------------------------
# Host page allocator: shuffled physical pages with spares
# ---------------------------------------------------------------------------
def build_block_table(lengths, seed: int, spare_frac: float = 0.02, min_spare: int = 3,
                      bt_stride: int | None = None):
    """Assign ceil(len/16) physical pages per session from a seeded permutation.

    Returns (block_table int32 [B, bt_stride] with -1 in unused entries,
    num_pages).  Spare pages (never referenced) stay in the pool so that a
    kernel reading a wrong page can be caught by poisoning them.
    """
    need = [(int(L) + PAGE - 1) // PAGE for L in lengths]
    total = sum(need)
    spares = max(min_spare, int(math.ceil(total * spare_frac)))
    num_pages = total + spares
    perm = _rng(seed, 1).permutation(num_pages).astype(np.int32)
    stride = max(max(need), 1) if bt_stride is None else bt_stride
    bt = np.full((len(lengths), stride), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt, num_pages


def build_private_tables(lens, priv_lens, seed: int, spare_frac: float = 0.02):
    """Pages for B shared prefixes and B*N private suffixes from one seeded pool.

    Returns (block_table int32 [B, S], private block table int32 [B*N, S_p],
    num_pages): row b*N + n of the private table lists the pages of decoder n's
    own tokens in session b.  Both tables draw from one permutation of the pool.
    """
    B = len(lens)
    allbt, num_pages = build_block_table(list(lens) + list(priv_lens), seed, spare_frac)
    s1 = max(max((int(L) + PAGE - 1) // PAGE for L in lens), 1)
    s2 = max(max((int(U) + PAGE - 1) // PAGE for U in priv_lens), 1)
    return allbt[:B, :s1].copy(), allbt[B:, :s2].copy(), num_pages


def build_prefix_groups(groups, seed: int, spare_frac: float = 0.02):
    """Block tables for sessions that share block-aligned prefixes, as a prefix
    cache hands them out: every session of a group starts with the same physical
    pages for the group's prefix, then has pages of its own.

    groups: list of (prefix_tokens, [session lengths]) with prefix_tokens a
    multiple of 16 and every length >= prefix_tokens.  Returns (block_table int32
    [B, S], lens, group_id int32 [B], prefix_pages int32 [B], num_pages); sessions
    are numbered group by group, so each group's sessions are adjacent.
    """
    need = 0
    for pre, lens in groups:
        if pre % PAGE or any(L < pre for L in lens):
            raise ValueError("prefixes must be whole pages and no longer than their sessions")
        need += pre // PAGE + sum((L + PAGE - 1) // PAGE - pre // PAGE for L in lens)
    spares = max(3, int(math.ceil(need * spare_frac)))
    num_pages = need + spares
    perm = _rng(seed, 2).permutation(num_pages).astype(np.int32)
    lens_all = [L for _, lens in groups for L in lens]
    stride = max(max((L + PAGE - 1) // PAGE for L in lens_all), 1)
    bt = np.full((len(lens_all), stride), -1, dtype=np.int32)
    gid = np.zeros(len(lens_all), np.int32)
    pref = np.zeros(len(lens_all), np.int32)
    pos, b = 0, 0
    for g, (pre, lens) in enumerate(groups):
        shared = perm[pos:pos + pre // PAGE]
        pos += pre // PAGE
        for L in lens:
            own = (L + PAGE - 1) // PAGE - pre // PAGE
            bt[b, :pre // PAGE] = shared
            bt[b, pre // PAGE:pre // PAGE + own] = perm[pos:pos + own]
            pos += own
            gid[b], pref[b] = g, pre // PAGE
            b += 1
    return bt, lens_all, gid, pref, num_pages


# ---------------------------------------------------------------------------
# bf16 draws (float32 normal -> bf16 round-to-nearest-even), as raw uint16 bits
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def draw_bf16(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(x)


def session_kv(wl: Workload, layer: int, b: int, length: int | None = None):
    """Logical K, V bits [L, H_kv, D] of session b at `layer` (numpy stream)."""
    L = wl.total_lens()[b] if length is None else length
    r = _rng(wl.seed, 2, layer, b)
    k = draw_bf16(r, (L, wl.num_kv_heads, wl.head_dim), wl.std)
    v = draw_bf16(r, (L, wl.num_kv_heads, wl.head_dim), wl.std)
    return k, v


def decode_q(wl: Workload, layer: int = 0, step: int = 0) -> np.ndarray:
    """Decode queries, bits [B, N, H_q, D]."""
    r = _rng(wl.seed, 3, layer, step)
    return draw_bf16(r, (wl.batch, wl.num_decoders, wl.num_q_heads, wl.head_dim), wl.std)


def extend_inputs(wl: Workload, layer: int = 0):
    """Chunk queries and chunk K/V bits for an extend workload.

    Returns (q [T, H_q, D], k_new [T, H_kv, D], v_new [T, H_kv, D], cu_new [B+1]).
    The chunk K/V of session b are the last `new[b]` rows of session_kv(...) of
    length prefix[b] + new[b], so the prefix + chunk form one logical sequence.
    """
    cu = np.zeros(wl.batch + 1, dtype=np.int32)
    cu[1:] = np.cumsum(wl.new)
    r = _rng(wl.seed, 4, layer)
    q = draw_bf16(r, (int(cu[-1]), wl.num_q_heads, wl.head_dim), wl.std)
    ks, vs = [], []
    for b in range(wl.batch):
        k, v = session_kv(wl, layer, b)
        ks.append(k[wl.prefix[b]:])
        vs.append(v[wl.prefix[b]:])
    return q, np.concatenate(ks), np.concatenate(vs), cu


def concat_rows(per_session):
    """Stack per-session row arrays and return (rows, cu) with cu[b] = first row of b."""
    cu = np.zeros(len(per_session) + 1, dtype=np.int32)
    cu[1:] = np.cumsum([x.shape[0] for x in per_session])
    return np.concatenate(per_session, axis=0), cu


# ---------------------------------------------------------------------------
# Device-side draws for the full-size workloads (torch Philox stream)
# ---------------------------------------------------------------------------
def device_normal_bf16(numel: int, std: float, seed: int, device="cuda"):
    """bf16 N(0, std^2) tensor of `numel` values drawn on the device.

    Used for the large workloads, whose K/V would take minutes to draw on the
    host.  Deterministic for a given seed and torch build.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(int(numel), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def mix_seed(*key) -> int:
    """A 63-bit seed derived from integers, for device draws."""
    return int(np.random.SeedSequence([int(k) for k in key]).generate_state(1, np.uint64)[0]
               & np.uint64(0x7FFFFFFFFFFFFFFF))
