"""Plain model of the prefix-cache page allocator — TEST INFRASTRUCTURE ONLY.

Only the tests may import this module; the library never does.

What it models ("Prefill-as-a-Service", component 3, hybrid prefix cache
pool): prefix-cache blocks are reused across requests only when they are
block-aligned and full; the single-model form of that reuse is vLLM's prefix
caching and SGLang's RadixAttention ("DroidSpeak: KV Cache Sharing for
Cross-LLM Communication and Multi-LLM Serving", section 1), where every request
whose prompt starts with cached full blocks gets the same physical pages.

Written from the rules, with the library header's deterministic policy:

* a page is free, referenced (count > 0), or cached and unreferenced
  (evictable);
* a cache entry is keyed by the WHOLE token prefix ending with its block
  (here the literal tuple of tokens, no hashing);
* admit: reuse the longest run of leading full blocks with entries, then take
  new pages lowest free id first, then evict the evictable page released
  earliest (dropping its entry); fail without change if pages run short;
* publish: every full block without an entry gets one on its page, unless the
  page already holds an entry;
* release: a page whose count drops to 0 is freed, or becomes evictable if it
  holds an entry (stamped with a fresh tick).

Group formation for the cascade decode is written out the same way
(`groups`): runs of adjacent sessions whose first page is equal, the prefix
being the leading entries equal across the run, cut to every member's full
pages.
"""
from __future__ import annotations

PAGE = 16


class PrefixCacheModel:
    def __init__(self, num_pages: int):
        if num_pages <= 0:
            raise ValueError("num_pages must be positive")
        self.num_pages = num_pages
        self.ref = [0] * num_pages
        self.entry_of_page = {}        # page -> prefix tuple
        self.page_of_entry = {}        # prefix tuple -> page
        self.released_at = {}          # evictable page -> tick
        self.free = set(range(num_pages))
        self.tick = 0

    # -- admit ---------------------------------------------------------------
    def admit(self, tokens):
        """Returns (page ids, matched count), or None when pages run short."""
        tokens = [int(t) for t in tokens]
        L = len(tokens)
        nblocks = -(-L // PAGE)
        matched = []
        for i in range(L // PAGE):
            key = tuple(tokens[:PAGE * (i + 1)])
            if key not in self.page_of_entry:
                break
            matched.append(self.page_of_entry[key])
        need = nblocks - len(matched)
        revived = sum(1 for p in matched if self.ref[p] == 0)
        if need > len(self.free) + len(self.released_at) - revived:
            return None
        for p in matched:
            if self.ref[p] == 0:
                del self.released_at[p]
            self.ref[p] += 1
        pages = list(matched)
        for _ in range(need):
            if self.free:
                p = min(self.free)
                self.free.remove(p)
            else:
                p = min(self.released_at, key=lambda q: self.released_at[q])
                del self.released_at[p]
                del self.page_of_entry[self.entry_of_page.pop(p)]
            self.ref[p] = 1
            pages.append(p)
        return pages, len(matched)

    # -- publish -------------------------------------------------------------
    def publish(self, tokens, pages):
        tokens = [int(t) for t in tokens]
        full = len(tokens) // PAGE
        for i in range(full):
            if not (0 <= pages[i] < self.num_pages) or self.ref[pages[i]] <= 0:
                raise ValueError(f"block {i}: page {pages[i]} is not a referenced page")
        for i in range(full):
            key = tuple(tokens[:PAGE * (i + 1)])
            p = int(pages[i])
            if key not in self.page_of_entry and p not in self.entry_of_page:
                self.page_of_entry[key] = p
                self.entry_of_page[p] = key

    # -- release -------------------------------------------------------------
    def release(self, pages):
        drops = {}
        for p in pages:
            p = int(p)
            if not 0 <= p < self.num_pages:
                raise ValueError(f"page {p} outside the pool")
            drops[p] = drops.get(p, 0) + 1
            if drops[p] > self.ref[p]:
                raise ValueError(f"page {p} released more often than referenced")
        for p in pages:
            p = int(p)
            self.ref[p] -= 1
            if self.ref[p] > 0:
                continue
            if p in self.entry_of_page:
                self.tick += 1
                self.released_at[p] = self.tick
            else:
                self.free.add(p)

    def stats(self):
        """(free, evictable, referenced, entries)"""
        ev = len(self.released_at)
        return len(self.free), ev, self.num_pages - len(self.free) - ev, len(self.page_of_entry)


def groups(block_table, seq_lens):
    """(group_id, group_prefix_pages) lists for the cascade decode."""
    B = len(seq_lens)
    gid, pref = [-1] * B, [0] * B
    b = 0
    while b < B:
        e = b + 1
        if seq_lens[b] >= PAGE:
            while e < B and seq_lens[e] >= PAGE and block_table[e][0] == block_table[b][0]:
                e += 1
        P = 0
        if e - b >= 2:
            full = min(seq_lens[m] // PAGE for m in range(b, e))
            while P < full and all(block_table[m][P] == block_table[b][P] for m in range(b, e)):
                P += 1
        for m in range(b, e):
            gid[m] = b if P > 0 else -1
            pref[m] = P
        b = e
    return gid, pref
