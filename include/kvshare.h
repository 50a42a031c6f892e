/*
 * kvshare.h — C ABI of the shared-KV attention library (libkvshare.so), gfx950.
 *
 * Several task-specific decoders attend over ONE paged KV cache that a frozen
 * base model wrote once.  In the notation of "ICaRus: Identical Cache Reuse for
 * Efficient Multi-Model Inference" (Method / overall framework), a logical
 * encoder E_base produces K_{1:i}, V_{1:i} and every task decoder D_task
 * computes x_{i+1} = D(x_i, K_{1:i}, V_{1:i}) over that same cache; Key design 3
 * of that page concatenates the query heads of all parties that read the same
 * KV so the KV is read once.  "PrefillShare: A Shared Prefill Module for KV Reuse
 * in Multi-LLM Disaggregated Serving" (sections 3.3 and 7) extends a cached
 * prefix by a partial prefill over the new tokens only, and keeps the KV in
 * fixed-size blocks (pages).
 *
 * Three operations:
 *   kv_pool_append         write new K/V rows into pages        (the cache "store")
 *   shared_kv_decode       N decoders x G GQA heads, one KV read (decode attention)
 *   shared_kv_decode_workspace_init  zero the arrival counters of a new decode workspace
 *   shared_kv_decode_noalloc  shared_kv_decode on a static scratch (allocates nothing)
 *   shared_kv_decode_append  the same, writing the step's own token into the
 *                          pool in the same launch (append + decode fused)
 *   shared_kv_decode_private  the same over a shared prefix + per-decoder private suffixes
 *   shared_kv_decode_cascade  the same where sessions share prefix pages, each prefix read once
 *   kv_pages_pack / kv_pages_unpack   pages <-> contiguous transfer buffer (cache handoff)
 *   kv_pool_fetch          logical K/V rows back out of the pool (inverse of kv_pool_append)
 *   partial_prefill_extend append a chunk, then causal attention of the chunk
 *                          over cached prefix + chunk           (partial prefill)
 *   partial_prefill_layers the same over a contiguous range of layers in one launch
 *                          (recompute of a layer group)
 *
 * ---------------------------------------------------------------------------
 * Conventions common to every entry point
 * ---------------------------------------------------------------------------
 *  - Element type of K, V, q and out is bfloat16 (raw 16-bit storage).  Softmax
 *    and accumulation are done in fp32; outputs are rounded to bf16
 *    round-to-nearest-even.
 *  - Every pointer argument except `pool` and the `*_out`-less scalars is a
 *    DEVICE pointer.  `pool` points to a host struct whose `data` member is a
 *    device pointer.  The caller allocates and owns every buffer; the library
 *    never allocates, frees or synchronizes, and keeps no per-call state.
 *    All work is enqueued asynchronously on `stream` (NULL = null stream).
 *  - Return value: KVS_OK (0) or a negative status.  On a negative status other
 *    than KVS_EHIP nothing was enqueued.  kvs_last_error() returns a
 *    thread-local message describing the last non-zero status.
 *  - Host-side checks: null pointers, page_size == 16, head_dim in {64, 128},
 *    num_q_heads % num_kv_heads == 0, layer in range, positive sizes,
 *    max_seq_len <= bt_stride * 16, workspace size.
 *  - Device-resident values (page ids, seq_lens, cu_new) are not visible to the
 *    host without a sync.  The kernels check them: a page id outside
 *    [0, num_pages), a length above the host-given bound, or an inconsistent
 *    cu_new never leads to an out-of-bounds access.  The offending
 *    page/session is skipped (its output is unspecified) and, when `dev_status`
 *    is non-NULL, the bits below are OR-ed into *dev_status (a device int32 the
 *    caller zeroes; read it after the stream completes).
 *
 * ---------------------------------------------------------------------------
 * Paged pool layout (bf16 elements, page size 16, head dim D in {64, 128})
 * ---------------------------------------------------------------------------
 *  The pool holds `num_layers` independent layer slices of `num_pages` physical
 *  pages; each page holds 16 consecutive token slots for all KV heads.  One
 *  (layer, page, head) TILE is 2*16*D elements, K part first, then V part:
 *
 *    tile(layer, page, head) = ((layer*num_pages + page)*num_kv_heads + head) * 32*D
 *    K(t, d) = tile + ((d/32)*64 + ((d%32)/8)*16 + t) * 8 + d%8
 *    V(t, d) = tile + 16*D + ((d/16)*32 + (t/8)*16 + d%16) * 8 + t%8
 *
 *  t is the slot in the page (0..15), d the head-dim index.  K: each 1 KiB group
 *  (fixed d/32) is the set of 64 16-byte lane operands (8 head-dim values of one
 *  slot) of one gfx950 16x16x32 bf16 matrix-core step.  V: each 512-byte group
 *  (fixed d/16) holds the 16-byte runs of 8 consecutive slots of one head-dim
 *  value, the A operand of a 16x16x32 step whose 32 reduction indices are the
 *  slots of two pages.  Both parts are read as contiguous 16-byte loads, with
 *  no transpose.  A tile is 8 KiB at D=128.
 *
 *  Logical token position p of session b lives in page block_table[b*bt_stride
 *  + p/16], slot p%16.  Block table entries past ceil(len/16) are never read
 *  (-1 is allowed there).  The block table is shared by all layers and by all
 *  decoders of a session: the cache is stored once per session whatever the
 *  number of decoders (PrefillShare, section 4, memory model Eqs. 8-9, shared
 *  term not multiplied by N).  Slots past a session's length are never read
 *  with non-zero weight, whatever they hold (NaN included).
 */
#ifndef KVSHARE_H
#define KVSHARE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KVS_OK = 0,
  KVS_EINVAL = -1,       /* null pointer, non-positive size, bad enum value   */
  KVS_ERANGE = -2,       /* a bound exceeds the block table / pool capacity   */
  KVS_EWORKSPACE = -3,   /* workspace missing or smaller than required        */
  KVS_EUNSUPPORTED = -4, /* page_size != 16, head_dim not in {64,128}, ...    */
  KVS_EHIP = -5,         /* a HIP launch failed; see kvs_last_error()         */
  KVS_ENOSPACE = -6      /* (kvs_prefix_cache.h) not enough free pages        */
};

/* Bits OR-ed into *dev_status by the kernels. */
enum {
  KVS_DEV_BAD_PAGE = 1,  /* block-table entry outside [0, num_pages)          */
  KVS_DEV_BAD_LEN = 2,   /* seq_lens / cu_new beyond the host-given bounds    */
  KVS_DEV_ALIAS = 4,     /* (kv_pool_append_check) a write would alias a slot  */
};

typedef struct kvs_pool {
  void* data;            /* device pointer to kvs_pool_bytes(...) bytes       */
  int32_t num_layers;
  int32_t num_pages;     /* physical pages per layer                          */
  int32_t num_kv_heads;
  int32_t head_dim;      /* 64 or 128                                          */
  int32_t page_size;     /* must be 16                                         */
} kvs_pool;

/* Bytes needed by a pool of the given shape (0 if a size is non-positive). */
size_t kvs_pool_bytes(int32_t num_layers, int32_t num_pages, int32_t num_kv_heads,
                      int32_t head_dim, int32_t page_size);

/*
 * kv_pool_append — write the K/V rows of new tokens into their page slots.
 *
 * The cache-store step of the base prefill: PrefillShare (section 4, base
 * prefill produces C_base; section 3.3, partial prefill appends the new tokens'
 * KV) and ICaRus (overall framework: E_base writes the KV that all decoders
 * read).  Pure data movement: the result is bit-exact.
 *
 *  k_new, v_new  bf16 [total_new][num_kv_heads][head_dim], sessions' rows
 *                concatenated; session b owns rows cu_new[b] .. cu_new[b+1]-1.
 *  cu_new        int32 [batch+1], cu_new[0] = 0, non-decreasing,
 *                cu_new[batch] = total_new.
 *  block_table   int32 [batch][bt_stride] physical page ids.
 *  seq_lens      int32 [batch]: tokens already resident BEFORE this call; new
 *                row j of session b goes to logical position seq_lens[b] + j.
 *  max_new       host bound on cu_new[b+1]-cu_new[b] (>= 1).
 *  max_seq_len   host bound on seq_lens[b] + new tokens of b (<= bt_stride*16).
 *  Only the destination slots are written; every other pool byte is unchanged.
 *  Two new rows must never map to the same physical slot (caller's duty;
 *  kv_pool_append_check verifies it in debug runs).
 */
int kv_pool_append(const kvs_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                   const int32_t* cu_new, const int32_t* block_table, int32_t bt_stride,
                   const int32_t* seq_lens, int32_t batch, int32_t total_new, int32_t max_new,
                   int32_t max_seq_len, int32_t* dev_status, hipStream_t stream);

/* Scratch bytes kv_pool_append_check needs for a pool of num_pages pages
 * (4 per page; 0 if num_pages <= 0). */
size_t kv_pool_append_check_bytes(int32_t num_pages);

/*
 * kv_pool_append_check — debug check of a kv_pool_append call's destinations,
 * made with the same arguments before the call (the K/V rows are not needed).
 *
 * Pages hold a session's positions in blocks (PrefillShare, section 3.3) and
 * full, block-aligned prefix blocks may sit in several sessions' tables
 * (Prefill-as-a-Service, component 3): a physical slot may be live for several
 * sessions, and reading it through each is sharing.  A write aliases when the
 * physical slot (page, slot) of a new token of the call
 *   - is also the slot of another new token of the call, or
 *   - holds a live token of a session of the batch (position q < seq_lens[c]
 *     of some session c, the writing session included);
 * then KVS_DEV_ALIAS is OR-ed into *dev_status.  Sessions outside the batch are
 * not known to the call.  Slots that kv_pool_append would not write (page ids
 * out of range, lengths it rejects) are left out; the append reports those.
 *
 *  scratch       device buffer of kv_pool_append_check_bytes(pool->num_pages)
 *                bytes, cleared by the call with a fill kernel on `stream`
 *                (KVS_EWORKSPACE when smaller or NULL); its contents after the
 *                call are unspecified.
 *  dev_status    required (KVS_EINVAL when NULL).
 *  Other arguments and host checks as for kv_pool_append (the pool's layers are
 *  not read).
 */
int kv_pool_append_check(const kvs_pool* pool, const int32_t* cu_new, const int32_t* block_table,
                         int32_t bt_stride, const int32_t* seq_lens, int32_t batch, int32_t total_new,
                         int32_t max_new, int32_t max_seq_len, void* scratch, size_t scratch_bytes,
                         int32_t* dev_status, hipStream_t stream);

/* Workspace bytes needed by shared_kv_decode, shared_kv_decode_append,
 * shared_kv_decode_private and shared_kv_decode_cascade for these bounds. */
size_t shared_kv_decode_workspace_bytes(int32_t batch, int32_t num_decoders, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_seq_len);

/*
 * shared_kv_decode_workspace_init — make a decode workspace ready for its first
 * call: zero its arrival counters (the first 64 KiB) with a fill kernel on
 * `stream`.  A workspace whose first 64 KiB are already zero (e.g. allocated
 * zero-filled) needs no init.
 *
 * A decode call splits work on one unit (session, KV head) between several
 * waves; the last wave to finish a unit merges the others' partial states,
 * found through a counter that every call leaves at zero again.  So a
 * workspace needs this once, not per call, as long as only decode calls write
 * it.  The rest of the workspace needs no init.
 *  workspace        device buffer, >= 64 KiB (KVS_EWORKSPACE otherwise).
 */
int shared_kv_decode_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * shared_kv_decode — one decode step of N decoders over one shared cache.
 *
 * ICaRus, Method / overall framework (x_{i+1} = D(x_i, K_{1:i}, V_{1:i}) with
 * the KV written by E_base) and Key design 3 (query heads of every party that
 * reads the same KV are concatenated along the head dimension, so the KV is
 * read once).  For session b, decoder n, query head h (KV head g = h / G,
 * G = num_q_heads / num_kv_heads):
 *     out[b,n,h,:] = sum_t softmax_t(scale * q[b,n,h,:] . K_g[t,:]) V_g[t,:],
 *     t = 0 .. seq_lens[b]-1;   out = 0 when seq_lens[b] == 0.
 * All N*G query rows of a KV head are processed together, so every page is read
 * from memory once per call, independent of N.  Decode only reads the pool.
 *
 *  q, out        bf16 [batch][num_decoders][num_q_heads][head_dim].
 *  seq_lens      int32 [batch], tokens attended (the current token's KV is
 *                appended with kv_pool_append before the call).
 *  max_seq_len   host bound on seq_lens[b]; sizes the launch.
 *  scale         softmax scale (1/sqrt(head_dim) for the usual attention).
 *  workspace     device buffer of >= shared_kv_decode_workspace_bytes(...)
 *                bytes.  Its first 64 KiB (arrival counters) must be zero when
 *                the call starts: zero the buffer once, or call
 *                shared_kv_decode_workspace_init once; every call leaves them
 *                zero.  The rest of its contents on entry are ignored (every
 *                other byte the call reads it wrote earlier in the same call), so
 *                a workspace may be reused by later decode calls on the same
 *                stream, whatever their shapes; calls that overlap in time must
 *                use different workspaces.
 *
 * Launch plan: one 4-wave workgroup per CU of the current device (its CU count
 * rounded down to a multiple of 8, at most 256), each wave streaming one
 * contiguous share of the (KV head, session, page) list; on a 256-CU part the
 * shares on even XCDs are 276/236 the size of those on odd ones.  The result
 * depends on the split only through rounding, and for one plan it is the same
 * bits on every call.  Testing hooks, read at every call: KVS_DECODE_WORKGROUPS
 * sets the workgroup count (rounded down to a multiple of 8, in 8 .. 256) and
 * KVS_DECODE_SHARE_EVEN the even-XCD weight (1 .. 511, of 512 per XCD pair).
 */
int shared_kv_decode(const kvs_pool* pool, int32_t layer, const void* q, void* out,
                     const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                     int32_t batch, int32_t num_decoders, int32_t num_q_heads,
                     int32_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                     int32_t* dev_status, hipStream_t stream);

/*
 * shared_kv_decode_noalloc — shared_kv_decode without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * Same arguments, results and device checks as shared_kv_decode, minus
 * `workspace` / `workspace_bytes`.  The workspace is a scratch array of
 * 68,289,024 bytes (the size shared_kv_decode_workspace_bytes gives for
 * batch 4096, head_dim 128, the largest call the library accepts) that the
 * library's code object holds in device memory; each GPU the library runs on
 * holds its own copy until the process ends.  The call allocates nothing (no
 * hipMalloc, no hipFree, no allocating library routine).  On its first call on
 * a device it looks up that device's scratch address and zeroes the scratch's
 * arrival counters with a fill kernel on `stream`; every call leaves them zero.
 *  - The stream must belong to the current device.
 *  - Every call on a GPU uses that GPU's one scratch array: calls that overlap in
 *    time on one GPU (other streams, other threads) race and give wrong
 *    results.  Serialize them.
 *  - A call needing more scratch than the array holds returns KVS_EWORKSPACE
 *    (no call within the documented bounds does).
 */
int shared_kv_decode_noalloc(const kvs_pool* pool, int32_t layer, const void* q, void* out,
                             const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                             int32_t batch, int32_t num_decoders, int32_t num_q_heads,
                             int32_t max_seq_len, float scale, int32_t* dev_status, hipStream_t stream);

/*
 * shared_kv_decode_append — kv_pool_append of one token per session followed by
 * shared_kv_decode, in one call.
 *
 * ICaRus, Method / overall framework: at step i the frozen base model writes
 * the token's own K_i, V_i, and every decoder then attends K_{1:i}, V_{1:i}.
 * This call does both: for every session b with 1 <= seq_lens[b] <= max_seq_len
 * it writes the token's K/V (every KV head) at position seq_lens[b] - 1 through
 * the block table, exactly as kv_pool_append with one new row would, and it
 * returns what shared_kv_decode over seq_lens[b] tokens returns after that
 * append, bit for bit.  The token is written by the wave that attends its page,
 * which also patches the token into its on-chip copy of the page, so the write
 * needs no launch of its own.
 *
 *  k_new, v_new  bf16 [batch][num_kv_heads][head_dim]: the step's token of
 *                each session.
 *  seq_lens      int32 [batch], tokens attended, counting the new one.  A
 *                session with seq_lens[b] == 0 writes nothing and gets zeros.
 *  Other arguments, the workspace and dev_status are those of shared_kv_decode.
 *  The page that receives a session's token must not be read by another
 *  session of the same call (a page shared between sessions holds full blocks
 *  only, so this is the usual case).  Not combinable with private suffixes or
 *  cascade groups.
 */
int shared_kv_decode_append(const kvs_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                            const void* q, void* out, const int32_t* block_table, int32_t bt_stride,
                            const int32_t* seq_lens, int32_t batch, int32_t num_decoders,
                            int32_t num_q_heads, int32_t max_seq_len, float scale, void* workspace,
                            size_t workspace_bytes, int32_t* dev_status, hipStream_t stream);

/*
 * shared_kv_decode_private — one decode step of N decoders over one shared
 * prefix plus each decoder's own private suffix.
 *
 * PrefillShare, section 3.3: decoding starts from the base model's cache C_base
 * and every step of a decoder adds its own KV (Delta C_t) to what that decoder
 * attends; the memory model of Eq. 9 stores the shared prefix once and only the
 * private parts per decoder.  Decoder n of session b attends its shared prefix
 * (seq_lens[b] tokens through block_table row b) followed by its private suffix
 * (priv_lens[b*N + n] tokens through priv_block_table row b*N + n):
 *     out[b,n,h,:] = sum_t softmax_t(scale * q[b,n,h,:] . K_g[t,:]) V_g[t,:]
 * over t in  prefix(b) ++ suffix(b, n);  out = 0 when both are empty.
 * Each shared page is read once for all N decoders, each private page once.
 * With every priv_lens entry 0 the result equals shared_kv_decode's.
 *
 *  priv_block_table  int32 [batch*num_decoders][priv_bt_stride], pages of the
 *                    private suffixes in the same pool (written with
 *                    kv_pool_append using this table, row b*N + n as a session).
 *  priv_lens         int32 [batch*num_decoders], private tokens per decoder.
 *  max_priv_len      host bound on priv_lens entries, <= priv_bt_stride * 16.
 *  Other arguments as for shared_kv_decode (same workspace size).  Up to 64
 *  query rows per KV head (num_decoders * num_q_heads / num_kv_heads) one wave
 *  holds them all and every private page is read once.  Above 64 the rows run
 *  in 64-row groups, as in shared_kv_decode: each group reads the shared pages
 *  and the session's private pages, and attends the private pages of the
 *  decoders whose rows it holds.
 */
int shared_kv_decode_private(const kvs_pool* pool, int32_t layer, const void* q, void* out,
                             const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                             const int32_t* priv_block_table, int32_t priv_bt_stride,
                             const int32_t* priv_lens, int32_t batch, int32_t num_decoders,
                             int32_t num_q_heads, int32_t max_seq_len, int32_t max_priv_len,
                             float scale, void* workspace, size_t workspace_bytes,
                             int32_t* dev_status, hipStream_t stream);

/*
 * shared_kv_decode_cascade — shared_kv_decode for sessions that share prefix
 * pages: the same result, with each shared prefix read once per group.
 *
 * Prefill-as-a-Service, component 3 (hybrid prefix cache pool): prefix-cache
 * blocks are reused across requests when they are block-aligned and full, so
 * every session with the same prefix gets the same physical pages (block-table
 * rows of those sessions start with equal entries).  Sessions b with equal,
 * non-negative group_id[b] that are adjacent in the batch form a group sharing
 * their first group_prefix_pages[b] pages (the same value for all members);
 * group_id[b] < 0 means no sharing.  Each group is read in units of up to
 * 64 / (num_decoders * G) sessions: the common prefix pages are streamed once
 * for all the unit's query rows, then each session's remaining pages for its own
 * rows.  Outputs equal shared_kv_decode's over the same block tables (to
 * rounding: the work is split differently).
 *
 *  group_id, group_prefix_pages  int32 [batch], device.  A member whose
 *                prefix page count differs from its unit's first session, or
 *                whose block-table entries for the prefix differ from the first
 *                session's, is reported (KVS_DEV_BAD_LEN / KVS_DEV_BAD_PAGE);
 *                the prefix pages read are always the first session's.  The
 *                prefix is also cut to whole pages every member holds.
 *  Other arguments and the workspace as for shared_kv_decode.  With more than
 *  64 query rows per session (num_decoders * num_q_heads / num_kv_heads) a unit
 *  would hold one session and share nothing: the call then runs shared_kv_decode
 *  over the same block tables (same result, bit for bit), and group_id and
 *  group_prefix_pages are not read.
 *
 * The units are planned by a first kernel into the workspace, with a 64-bit
 * fingerprint of what they depend on (batch, sessions per unit, max_seq_len,
 * and every session's seq_lens, group_id and group_prefix_pages).  A call whose
 * inputs have the stored fingerprint reuses the planned units, so the layers of
 * a decode step that share a workspace plan once; any change to those inputs
 * plans again.  The block-table checks above run when the units are planned.
 */
int shared_kv_decode_cascade(const kvs_pool* pool, int32_t layer, const void* q, void* out,
                             const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                             const int32_t* group_id, const int32_t* group_prefix_pages, int32_t batch,
                             int32_t num_decoders, int32_t num_q_heads, int32_t max_seq_len, float scale,
                             void* workspace, size_t workspace_bytes, int32_t* dev_status,
                             hipStream_t stream);

/*
 * partial_prefill_extend — cached-prefix extension over the new tokens only.
 *
 * PrefillShare, sections 3.3 and 7: on a cache hit only the new tokens are
 * prefilled against the cached prefix; section 4: prefill
 * (y_1, C_n) = F(X, empty) is the case with an empty prefix.  First appends the
 * chunk's K/V exactly as kv_pool_append does, then for new row i of session b
 * (absolute position p = seq_lens[b] + i) and query head h:
 *     out[cu_new[b]+i, h, :] = sum_{t<=p} softmax_t(scale * q . K_g[t,:]) V_g[t,:]
 * i.e. full attention to the prefix and causal (diagonal included) within the
 * chunk.
 *
 *  q, out        bf16 [total_new][num_q_heads][head_dim].
 *  k_new, v_new  bf16 [total_new][num_kv_heads][head_dim].
 *  cu_new        int32 [batch+1] as for kv_pool_append.
 *  seq_lens      int32 [batch], prefix length of each session before the call.
 *  max_new       host bound on any session's new-token count (>= 1).
 *  max_seq_len   host bound on seq_lens[b] + new tokens of b (<= bt_stride*16).
 */
int partial_prefill_extend(const kvs_pool* pool, int32_t layer, const void* q, const void* k_new,
                           const void* v_new, void* out, const int32_t* cu_new,
                           const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                           int32_t batch, int32_t num_q_heads, int32_t total_new, int32_t max_new,
                           int32_t max_seq_len, float scale, int32_t* dev_status,
                           hipStream_t stream);

/*
 * partial_prefill_layers — partial_prefill_extend for the layers
 * [layer_begin, layer_begin + num_layers) of the pool, in one launch.
 *
 * "DroidSpeak: KV Cache Sharing for Cross-LLM Communication and Multi-LLM
 * Serving", sections 5.1 and 5.4: a receiving model reuses a sender's KV for most
 * layers and recomputes one contiguous layer group (one transition point, so the
 * layer inputs cross over once); its partial_prefill interface runs the prefill
 * of that group.  The attention part of that prefill is this call: for every
 * layer l of the range, the layer's new K/V rows are appended into pool layer
 * layer_begin + l (through the same block table; recomputing a whole prompt is
 * seq_lens = 0), then the rows attend as in partial_prefill_extend.  The
 * projections that produce q, k and v from the layer inputs are the caller's.
 *
 *  q, out        bf16 [num_layers][total_new][num_q_heads][head_dim].
 *  k_new, v_new  bf16 [num_layers][total_new][num_kv_heads][head_dim].
 *  Other arguments as for partial_prefill_extend, shared by every layer.
 *  KVS_ERANGE when the range leaves the pool.  The result equals num_layers
 *  partial_prefill_extend calls, bit for bit.
 */
int partial_prefill_layers(const kvs_pool* pool, int32_t layer_begin, int32_t num_layers, const void* q,
                           const void* k_new, const void* v_new, void* out, const int32_t* cu_new,
                           const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                           int32_t batch, int32_t num_q_heads, int32_t total_new, int32_t max_new,
                           int32_t max_seq_len, float scale, int32_t* dev_status, hipStream_t stream);

/*
 * kv_pages_pack / kv_pages_unpack — move whole pages between a pool and a
 * contiguous transfer buffer: the on-GPU half of a cache handoff.
 *
 * PrefillShare, section 3.3: the prefill worker hands the KV it wrote, kept in
 * fixed-size blocks, to the decode worker.  pack copies, for every layer in
 * [layer_begin, layer_begin + num_layers) and every listed physical page, all
 * KV heads' tiles of that page into
 *     buf[layer - layer_begin][i][head][tile]      (i = index in page_ids),
 * bit for bit; unpack writes such a buffer into the listed pages of a pool
 * (which may be another pool, of any page count, with the same num_kv_heads and
 * head_dim).  A (layer, page) entry is num_kv_heads * 32 * head_dim bf16
 * elements (64 KiB at 8 KV heads, D=128); kv_pages_buffer_bytes gives the size.
 *
 *  page_ids    int32 [num_ids], device; ids outside [0, num_pages) are skipped
 *              and reported with KVS_DEV_BAD_PAGE (their buffer entries, or
 *              pages, are left as they were).  unpack with a page listed twice
 *              leaves that page holding one of its entries.
 *  buf         device buffer of kv_pages_buffer_bytes(...) bytes, owned by the
 *              caller; it must not overlap the pool.
 */
size_t kv_pages_buffer_bytes(const kvs_pool* pool, int32_t num_layers, int32_t num_ids);
int kv_pages_pack(const kvs_pool* pool, int32_t layer_begin, int32_t num_layers, const int32_t* page_ids,
                  int32_t num_ids, void* buf, int32_t* dev_status, hipStream_t stream);
int kv_pages_unpack(const kvs_pool* pool, int32_t layer_begin, int32_t num_layers, const int32_t* page_ids,
                    int32_t num_ids, const void* buf, int32_t* dev_status, hipStream_t stream);

/*
 * kv_pool_fetch — the logical K/V rows of sessions, read back out of the pool
 * into dense arrays: the inverse of kv_pool_append.
 *
 * DroidSpeak, section 5.4: fetch returns what store wrote.  For session b and
 * position p < seq_lens[b]:
 *     k_out[cu_rows[b] + p][head][:] = K of position p,   v_out likewise,
 * bit for bit, read through block_table row b.  Used to hand a cache to a
 * consumer that keeps another layout.
 *
 *  k_out, v_out  bf16 [total_rows][num_kv_heads][head_dim], device.
 *  cu_rows       int32 [batch+1], device; cu_rows[b+1] - cu_rows[b] must equal
 *                seq_lens[b] (a session that breaks this, or whose rows would
 *                pass total_rows, is skipped and reported with KVS_DEV_BAD_LEN).
 *  max_seq_len   host bound on seq_lens[b], <= bt_stride * 16.
 */
int kv_pool_fetch(const kvs_pool* pool, int32_t layer, const int32_t* block_table, int32_t bt_stride,
                  const int32_t* seq_lens, const int32_t* cu_rows, int32_t batch, int32_t total_rows,
                  int32_t max_seq_len, void* k_out, void* v_out, int32_t* dev_status, hipStream_t stream);

/* Thread-local description of the last non-zero status returned on this thread. */
const char* kvs_last_error(void);

/* Library version string. */
const char* kvs_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVSHARE_H */
