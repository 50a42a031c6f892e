/*
 * kvs_prefix_cache.h — host-side page allocator with a prefix cache of full
 * blocks, and the grouping of sessions that share prefix pages (libkvshare.so).
 *
 * "Prefill-as-a-Service" (component 3, hybrid prefix cache pool) keeps two kinds
 * of blocks: prefix-cache blocks, reused across requests, which must be
 * block-aligned and full to be reused; and transfer blocks, dropped once their
 * KV has moved on.  The single-model form of this sharing is the prefix caching
 * of vLLM and SGLang's RadixAttention (named in "DroidSpeak: KV Cache Sharing
 * for Cross-LLM Communication and Multi-LLM Serving", section 1): every request
 * whose prompt starts with cached full blocks gets the SAME physical pages for
 * them.  This allocator does that for the paged pool of kvshare.h:
 *
 *  - A page is either free, referenced by live sessions (a reference count), or
 *    cached-and-unreferenced (holds a prefix-cache entry nobody uses right now:
 *    reusable by a later session with the same prefix, evictable when free
 *    pages run out).
 *  - A cache entry names one full 16-token block by its whole token prefix:
 *    block i of a prompt is keyed by tokens[0 .. 16(i+1)).  The key is a chain
 *    of two independent 64-bit hashes over (parent key, the block's 16 tokens);
 *    the entry also keeps the block's tokens, which a lookup compares, so two
 *    prompts alias only if both 64-bit chains collide.
 *  - Deterministic policy (so results are reproducible and testable): free pages
 *    are taken lowest id first; eviction takes the cached-and-unreferenced page
 *    whose last reference was dropped earliest (ties impossible: every dropped
 *    reference gets its own tick).
 *
 * Conventions: every pointer is a HOST pointer; token ids are int32; the page
 * size is 16 tokens.  Calls on one allocator must not overlap (no internal
 * locking); distinct allocators are independent.  Return value: KVS_OK or a
 * negative status of kvshare.h (KVS_ENOSPACE: not enough pages, nothing
 * changed); kvs_last_error() describes the last failure.
 */
#ifndef KVS_PREFIX_CACHE_H
#define KVS_PREFIX_CACHE_H

#include <stdint.h>

#include "kvshare.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvs_prefix_cache kvs_prefix_cache;

/* An allocator over pool pages 0 .. num_pages-1, all free.  NULL if num_pages <= 0
 * or on allocation failure.  Owned by the caller; free with ..._destroy. */
kvs_prefix_cache* kvs_prefix_cache_create(int32_t num_pages);
void kvs_prefix_cache_destroy(kvs_prefix_cache* pc);

/*
 * Admit a session whose prompt is tokens[0 .. L) (L >= 0).
 *  - Its longest run of leading full blocks found in the cache is reused: those
 *    pages gain a reference (a cached-and-unreferenced one stops being
 *    evictable).  *matched_pages receives that count; the caller must not write
 *    those pages (their KV is already there) and prefills tokens
 *    [16 * matched_pages, L) only.
 *  - The remaining ceil(L/16) - matched pages come from the free list, lowest id
 *    first, then by evicting cached-and-unreferenced pages, earliest released
 *    first (their cache entries are dropped).  They get one reference each.
 *  - bt_row[0 .. ceil(L/16)) receives the session's page ids in logical order.
 * KVS_ENOSPACE when free + evictable pages do not cover the new pages (nothing
 * changes).  KVS_EINVAL for NULL pointers (tokens may be NULL when L == 0) or L < 0.
 */
int kvs_prefix_cache_admit(kvs_prefix_cache* pc, const int32_t* tokens, int32_t L, int32_t* bt_row,
                           int32_t* matched_pages);

/*
 * Publish a session's full blocks once their KV is written: block i
 * (i < L/16) becomes the cache entry for tokens[0 .. 16(i+1)) on page
 * bt_row[i], unless that prefix already has an entry (then nothing changes for
 * that block).  A page holds at most one entry; a block whose page already
 * holds another entry is skipped.  The last, partial block is never published.
 * KVS_EINVAL for NULL pointers or L < 0; KVS_ERANGE for a page id outside the
 * pool or not referenced.
 */
int kvs_prefix_cache_publish(kvs_prefix_cache* pc, const int32_t* tokens, int32_t L, const int32_t* bt_row);

/*
 * Drop one reference from each of bt_row[0 .. npages).  A page left with no
 * reference returns to the free list if it holds no cache entry, else it stays
 * cached and becomes evictable.  KVS_ERANGE (nothing changes) if a page id is
 * outside the pool or not referenced often enough.
 */
int kvs_prefix_cache_release(kvs_prefix_cache* pc, const int32_t* bt_row, int32_t npages);

/* Page counts: free, cached-and-unreferenced (evictable), referenced; and the
 * number of cache entries.  Any output pointer may be NULL. */
int kvs_prefix_cache_stats(const kvs_prefix_cache* pc, int32_t* free_pages, int32_t* evictable_pages,
                           int32_t* referenced_pages, int32_t* entries);

/* Reference count of page `page` (0 for a free or evictable page), or a
 * negative status for a bad handle or page id. */
int kvs_prefix_cache_refcount(const kvs_prefix_cache* pc, int32_t page);

/*
 * Group sessions that share leading pages, as shared_kv_decode_cascade takes
 * them.  block_table: HOST int32 [batch][bt_stride]; seq_lens: HOST int32 [batch].
 * Adjacent sessions whose first page is the same (and who both hold at least
 * one full page) join one group; a group's prefix is the number of leading
 * block-table entries equal across all its members, cut to the full pages every
 * member holds (min over members of seq_len / 16).  Outputs (HOST int32 [batch]):
 * group_id = index of the group's first session, or -1 for a session that
 * shares nothing (or whose group prefix is 0); group_prefix_pages = the group's
 * prefix (0 for -1).  KVS_EINVAL for NULL pointers or batch < 0; KVS_ERANGE when
 * a length exceeds bt_stride * 16.
 */
int kvs_prefix_groups(const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens, int32_t batch,
                      int32_t* group_id, int32_t* group_prefix_pages);

#ifdef __cplusplus
}
#endif

#endif /* KVS_PREFIX_CACHE_H */
