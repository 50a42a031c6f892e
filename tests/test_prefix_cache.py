"""Prefix-cache page allocator and session grouping (host side, no GPU).

The plain model in oracle/prefix_cache.py is pinned first: worked scenarios
whose outcomes follow from Prefill-as-a-Service's component 3 rules (only
block-aligned, full blocks are reused; the same prefix gets the same pages), the
page-state invariants, and a few planted mistakes the pins must catch.  The
library (C ABI through the binding) must then match the model call for call on
seeded random workloads: the same page ids, reuse counts, statistics, reference
counts and failures.
"""
import random

import numpy as np
import pytest

from cross_model_shared_amd import binding
from oracle import prefix_cache as pcm

PAGE = 16


def check_invariants(m: pcm.PrefixCacheModel, live):
    """Every page is in exactly one state; counts equal the live sessions' references."""
    want = [0] * m.num_pages
    for pages in live:
        for p in pages:
            want[p] += 1
    assert want == m.ref
    for p in range(m.num_pages):
        states = [p in m.free, p in m.released_at, m.ref[p] > 0]
        assert sum(states) == 1, (p, states)
        if p in m.released_at:
            assert p in m.entry_of_page
    assert all(m.page_of_entry[k] == p for p, k in m.entry_of_page.items())
    assert len(m.page_of_entry) == len(m.entry_of_page)


# ---------------------------------------------------------------------------
# pins of the model
# ---------------------------------------------------------------------------
def test_model_reuses_only_full_leading_blocks():
    m = pcm.PrefixCacheModel(16)
    shared = list(range(1000, 1040))             # 40 tokens: 2 full blocks + 8
    a, ma = m.admit(shared + [1, 2, 3])          # 43 tokens -> 3 pages
    assert (a, ma) == ([0, 1, 2], 0)
    m.publish(shared + [1, 2, 3], a)             # blocks 0, 1 published; block 2 is partial
    assert m.stats() == (13, 0, 3, 2)
    b, mb = m.admit(shared + [9] * 8)            # 48 tokens: block 2 differs from a's partial block
    assert (b, mb) == ([0, 1, 3], 2)
    assert m.ref[:4] == [2, 2, 1, 1]
    c, mc = m.admit(shared[:31])                 # only block 0 is full in 31 tokens
    assert (c, mc) == ([0, 4], 1)
    check_invariants(m, [a, b, c])


def test_model_needs_publish_before_reuse_and_keeps_the_first_entry():
    m = pcm.PrefixCacheModel(8)
    t = list(range(32))
    a, _ = m.admit(t)
    b, mb = m.admit(t)                           # a's KV not published yet: nothing to reuse
    assert mb == 0 and set(a).isdisjoint(b)
    m.publish(t, a)
    m.publish(t, b)                              # same prefixes already have entries (on a's pages)
    assert m.page_of_entry[tuple(t[:16])] == a[0] and b[0] not in m.entry_of_page
    m.release(b)
    assert set(b) <= m.free                      # b's pages hold no entry: freed at once
    m.release(a)
    assert set(a) == set(m.released_at)          # a's pages stay cached, evictable


def test_model_eviction_order_and_no_space():
    m = pcm.PrefixCacheModel(4)
    x, y = [1] * 16, [2] * 16
    px, _ = m.admit(x)
    m.publish(x, px)
    py, _ = m.admit(y)
    m.publish(y, py)
    m.release(py)                                # y released first
    m.release(px)
    assert m.stats() == (2, 2, 0, 2)
    z, _ = m.admit([3] * 48)                     # 3 pages: both free ones, then evict y (released first)
    assert z == [2, 3, py[0]] and tuple(y) not in m.page_of_entry and tuple(x) in m.page_of_entry
    before = (list(m.ref), set(m.free), dict(m.released_at), dict(m.page_of_entry))
    assert m.admit([4] * 33) is None             # 3 pages needed, 1 evictable: fails, nothing changes
    assert before == (list(m.ref), set(m.free), dict(m.released_at), dict(m.page_of_entry))
    assert m.admit(x + [5]) is None              # x's page is revived, so it cannot also be evicted for the rest
    w, mw = m.admit(x)                           # x alone: revived, no new page
    assert (w, mw) == ([px[0]], 1) and m.ref[px[0]] == 1
    assert m.admit([6] * 16) is None             # no free or evictable page left


def test_model_reuse_stops_at_an_evicted_parent():
    m = pcm.PrefixCacheModel(3)
    t = list(range(32))
    a, _ = m.admit(t)
    m.publish(t, a)
    m.release(a)                                 # block 0 released first, then block 1
    b, _ = m.admit([7] * 16)                     # the free page
    assert b == [2]
    c, _ = m.admit([8] * 16)                     # evicts block 0 (released earliest)
    assert c == [a[0]]
    m.release(b)                                 # unpublished: straight back to the free list
    d, md = m.admit(t)                           # block 1's entry is still cached, but its parent is gone:
    assert (d, md) == ([2, a[1]], 0)             # nothing reused; block 1's page is evicted for block 1


def test_groups_match_their_definition():
    rng = random.Random(3)
    for _ in range(200):
        B = rng.randint(0, 7)
        stride = 6
        bt = [[rng.choice([0, 1, 2]) if p < 2 else rng.randint(0, 20) for p in range(stride)] for _ in range(B)]
        lens = [rng.randint(0, stride * PAGE) for _ in range(B)]
        gid, pref = pcm.groups(bt, lens)
        for b in range(B):
            if gid[b] < 0:
                assert pref[b] == 0
                continue
            f = gid[b]
            members = [m for m in range(B) if gid[m] == f]
            assert members == list(range(f, f + len(members))) and len(members) >= 2
            P = pref[b]
            assert P >= 1 and all(bt[m][:P] == bt[f][:P] for m in members)
            assert all(lens[m] >= PAGE * P for m in members)
            full = min(lens[m] // PAGE for m in members)
            assert P == full or any(bt[m][P] != bt[f][P] for m in members)   # maximal
        # a run of equal first pages is never split, and never extended past a different first page
        for b in range(1, B):
            same = lens[b] >= PAGE and lens[b - 1] >= PAGE and bt[b][0] == bt[b - 1][0]
            if gid[b] >= 0 and gid[b - 1] >= 0:
                assert (gid[b] == gid[b - 1]) == same


# Worked tables for the grouping rule (adjacent sessions holding at least one full page
# with the same first page form a group; its prefix is the leading entries equal across
# the group, cut to the full pages every member holds).  Each expected value is worked
# out by hand from that rule.
GROUP_CASES = [
    # sessions 0-2 share page 5; session 2 holds 2 full pages, and entry 1 differs: prefix 1
    ([[5, 6, 7], [5, 6, 9], [5, 8, 1], [2, 3, 4]], [48, 48, 40, 48], [0, 0, 0, -1], [1, 1, 1, 0]),
    # session 2 holds no full page: not in the run; sessions 0-1 agree on both full pages
    ([[1, 2], [1, 2], [1, 3]], [32, 32, 15], [0, 0, -1], [2, 2, 0]),
    # four sessions with one full page each, all on page 4
    ([[4], [4], [4], [4]], [16, 16, 17, 31], [0, 0, 0, 0], [1, 1, 1, 1]),
    # equal first pages that are not adjacent form no group
    ([[1], [2], [1]], [16, 16, 16], [-1, -1, -1], [0, 0, 0]),
    # two runs side by side: prefixes 2 and 1
    ([[1, 9], [1, 9], [2, 8], [2, 8], [2, 7]], [32] * 5, [0, 0, 2, 2, 2], [2, 2, 1, 1, 1]),
    # a single session never groups
    ([[3, 3]], [64], [-1], [0]),
]


@pytest.mark.parametrize("bt,lens,gid,pref", GROUP_CASES)
def test_groups_worked_tables(bt, lens, gid, pref):
    assert pcm.groups(bt, lens) == (gid, pref)


def test_groups_are_complete():
    """Every maximal run of two or more adjacent sessions that hold a full page and share
    their first page is one group with a prefix of at least one page (a model that never
    groups, or splits runs, fails here)."""
    rng = random.Random(5)
    for _ in range(200):
        B = rng.randint(0, 8)
        bt = [[rng.choice([0, 1]) if p == 0 else rng.randint(0, 3) for p in range(4)] for _ in range(B)]
        lens = [rng.choice([0, 5, 16, 20, 32, 48, 64]) for _ in range(B)]
        gid, pref = pcm.groups(bt, lens)
        b = 0
        while b < B:
            e = b + 1
            if lens[b] >= PAGE:
                while e < B and lens[e] >= PAGE and bt[e][0] == bt[b][0]:
                    e += 1
            if e - b >= 2:
                assert gid[b:e] == [b] * (e - b) and all(p >= 1 for p in pref[b:e]), (bt, lens, gid, pref)
            b = e


MODEL_SRC = open(pcm.__file__).read()
MUTANTS = {
    "reuse_skips_a_missing_block": ("            if key not in self.page_of_entry:\n                break",
                                    "            if key not in self.page_of_entry:\n                continue"),
    "highest_free_first": ("p = min(self.free)", "p = max(self.free)"),
    "evicts_latest": ("p = min(self.released_at, key", "p = max(self.released_at, key"),
    "frees_cached_page": ("            if p in self.entry_of_page:\n                self.tick",
                          "            if False:\n                self.tick"),
    "publishes_partial_block": ("full = len(tokens) // PAGE\n        for i in range(full):\n            if not",
                                "full = -(-len(tokens) // PAGE)\n        for i in range(full):\n            if not"),
}


GROUP_MUTANTS = {
    "never_groups": ("        if e - b >= 2:\n", "        if e - b >= 99:\n"),
    "groups_pairs_only": ("            while e < B and seq_lens[e] >= PAGE",
                          "            while e < b + 2 and e < B and seq_lens[e] >= PAGE"),
    "ignores_partial_members": ("full = min(seq_lens[m] // PAGE for m in range(b, e))",
                                "full = max(seq_lens[m] // PAGE for m in range(b, e))"),
}


@pytest.mark.parametrize("name", sorted(GROUP_MUTANTS))
def test_group_pins_catch_mutant(name, monkeypatch):
    old, new = GROUP_MUTANTS[name]
    assert MODEL_SRC.count(old) == 1, name
    ns = {"__name__": "prefix_cache_mutant"}
    exec(compile(MODEL_SRC.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(pcm, "groups", ns["groups"])
    failed = 0
    pins = [lambda c=c: test_groups_worked_tables(*c) for c in GROUP_CASES] + [test_groups_are_complete,
                                                                                 test_groups_match_their_definition]
    for pin in pins:
        try:
            pin()
        except (AssertionError, IndexError):
            failed += 1
    assert failed, f"mutant {name} survived every grouping pin"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_model_pins_catch_mutant(name, monkeypatch):
    old, new = MUTANTS[name]
    assert MODEL_SRC.count(old) == 1, name
    ns = {"__name__": "prefix_cache_mutant"}
    exec(compile(MODEL_SRC.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(pcm, "PrefixCacheModel", ns["PrefixCacheModel"])
    failed = 0
    for pin in (test_model_reuses_only_full_leading_blocks, test_model_needs_publish_before_reuse_and_keeps_the_first_entry,
                test_model_eviction_order_and_no_space, test_model_reuse_stops_at_an_evicted_parent):
        try:
            pin()
        except (AssertionError, KeyError, IndexError, ValueError, TypeError):
            failed += 1
    assert failed, f"mutant {name} survived every pin"


# ---------------------------------------------------------------------------
# library against the model
# ---------------------------------------------------------------------------
def random_prompt(rng, systems):
    s = rng.choice(systems)
    cut = rng.randint(0, len(s))
    return s[:cut] + [rng.randint(0, 50) for _ in range(rng.randint(0, 40))]


@pytest.mark.parametrize("seed,num_pages", [(0, 40), (1, 64), (2, 24), (3, 200)])
def test_library_matches_model(seed, num_pages):
    rng = random.Random(seed)
    systems = [[rng.randint(0, 50) for _ in range(rng.randint(16, 90))] for _ in range(4)]
    lib, m = binding.PrefixCache(num_pages), pcm.PrefixCacheModel(num_pages)
    live = []                                    # (tokens, pages, published)
    for step in range(400):
        op = rng.random()
        if op < 0.45 or not live:
            t = random_prompt(rng, systems)
            want = m.admit(t)
            if want is None:
                with pytest.raises(binding.KvsError) as e:
                    lib.admit(t)
                assert e.value.status == binding.KVS_ENOSPACE
            else:
                pages, matched = lib.admit(t)
                assert (list(pages), matched) == (want[0], want[1]), step
                live.append([t, want[0], False])
        elif op < 0.75:
            i = rng.randrange(len(live))
            t, pages, pub = live[i]
            if not pub:
                m.publish(t, pages)
                lib.publish(t, pages)
                live[i][2] = True
        else:
            t, pages, _ = live.pop(rng.randrange(len(live)))
            m.release(pages)
            lib.release(pages)
        assert lib.stats() == m.stats(), step
        check_invariants(m, [p for _, p, _ in live])
    assert [lib.refcount(p) for p in range(num_pages)] == m.ref
    lib.close()


def test_library_rejects_bad_calls_without_change():
    lib = binding.PrefixCache(4)
    pages, _ = lib.admit(list(range(20)))
    st = lib.stats()
    for bad in ([7], [-1], [pages[0], pages[0]]):
        with pytest.raises(binding.KvsError) as e:
            lib.release(bad)
        assert e.value.status == binding.KVS_ERANGE
    with pytest.raises(binding.KvsError):
        lib.publish(list(range(16)), [3])        # page 3 is not referenced
    assert lib.stats() == st
    with pytest.raises(binding.KvsError) as e:
        lib.admit(list(range(100)))              # 7 pages, 2 left
    assert e.value.status == binding.KVS_ENOSPACE and lib.stats() == st
    assert lib.refcount(0) == 1
    with pytest.raises(binding.KvsError):
        lib.refcount(4)
    with pytest.raises(binding.KvsError):
        binding.PrefixCache(0)


def test_library_groups_match_model():
    rng = random.Random(11)
    for _ in range(300):
        B = rng.randint(1, 9)
        stride = 5
        bt = np.array([[rng.choice([0, 1]) if p < 3 else rng.randint(0, 9) for p in range(stride)]
                       for _ in range(B)], np.int32)
        lens = [rng.randint(0, stride * PAGE) for _ in range(B)]
        gid, pref = binding.prefix_groups(bt, lens)
        want = pcm.groups(bt.tolist(), lens)
        assert (list(gid), list(pref)) == (want[0], want[1])
    with pytest.raises(binding.KvsError):
        binding.prefix_groups(np.zeros((1, 2), np.int32), [33])


def test_allocator_tables_feed_the_cascade_grouping():
    """Sessions admitted with a common published system prompt share its full
    pages, and the grouping finds exactly those pages."""
    lib = binding.PrefixCache(256)
    system = list(range(500, 500 + 16 * 5 + 7))  # 5 full blocks + 7 tokens
    first, _ = lib.admit(system + [1])
    lib.publish(system + [1], first)
    rows, lens = [first], [len(system) + 1]
    for s in range(3):
        t = system + [10 + s] * (s * 20)
        pages, matched = lib.admit(t)
        assert matched == 5
        rows.append(pages)
        lens.append(len(t))
    stride = max(len(r) for r in rows)
    bt = np.full((len(rows), stride), -1, np.int32)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    gid, pref = binding.prefix_groups(bt, lens)
    assert list(gid) == [0, 0, 0, 0] and list(pref) == [5] * 4
