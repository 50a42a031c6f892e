// shared_kv_decode on gfx950: N decoders x G query heads per KV head, one KV read.
//
// ICaRus (Key design 3) runs the queries of every party that reads the same KV
// side by side along the head dimension so the KV is read once.  Here all
// R = N*G query rows of a KV head sit on the N side of the matrix-core steps of
// one wave, so each (page, KV head) tile streams from HBM exactly once per call
// whatever N is.
//
// Work split (stream-K over pages): the tiles of every (KV head, row group,
// session) unit are laid end to end — unit order (KV head, row group) then
// session, pages in logical order — and the resulting list is cut into one
// contiguous share per wave of a persistent grid (one 4-wave workgroup per CU;
// shares weighted per XCD, see share_weight_before).  A wave streams its share
// through a per-wave LDS ring with direct global->LDS 16-byte loads (S pages in
// flight, no registers held by loads),
// runs the page step of attn_core.h, and at every unit boundary either writes
// the final output (unit wholly inside its share) or its partial softmax state
// (m, l, acc) (unit crossing a share boundary); the last wave to finish a split
// unit merges its shares' states (finish_split), so a call is one launch.
//
// Decoder-private suffixes (PrefillShare, section 3.3: each decoder extends
// C_base with its own generated tokens; Eq. 9 keeps the prefix once and the
// suffixes per decoder): a unit's tile list is the session's shared pages
// followed by every decoder's private pages, decoder by decoder.  A private page
// is read once, by the wave that holds all of the KV head's rows, with the rows
// of the other decoders masked out, so the shared prefix still streams once for
// all N decoders and each suffix once for its own.
//
// Prefixes shared across sessions (cascade): sessions whose block tables start
// with the same pages (a prefix cache hands the same physical pages to every
// session with that prefix) are grouped into units of up to 64 / (N*G)
// sessions by decode_cascade_plan_kernel; a unit's tile list is the common
// prefix pages, read once for all its sessions' rows, followed by each
// session's own remaining pages for that session's rows.  Those units run on
// wave pairs (decode_pair_kernel): 32 rows per wave keeps two waves per SIMD,
// which a 64-row wave's registers would not allow.
#include <limits.h>

#include "attn_core.h"
#include "kvs_internal.h"

namespace kvs {

namespace {

constexpr int kWaves = 4;

// s_waitcnt with vmcnt = VM and the other counters left alone (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] in bits 15:14).
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait for every outstanding memory access of this wave.  The wait builtin is
// not a memory access for the compiler, which may move loads and stores across
// it; the compiler fences on both sides keep them on their side.
__device__ __forceinline__ void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Direct global -> LDS copy of one 1 KiB slab: 16 bytes per lane, lane l's
// bytes from `src` + 16 l to LDS byte address `lds` + 16 l (gfx950's
// global_load_lds_dwordx4; M0 holds the LDS address, and the M0 write needs one
// wait state before the load reads it).  The load is nontemporal: a call reads
// each page once, and streaming it past the caches moves the decode calls 5-10%
// closer to the HBM rate than the default policy does.  Written in assembly so that the
// compiler does not track it: the ring's own waits (wait_ring) order these
// copies against the LDS reads, and a compiler that tracked them would also
// wait for the most recent copy before a page's LDS reads whenever it could not
// tell the ring slots apart.  The copy still counts in vmcnt, so every wait the
// compiler computes for its own loads only gets stricter.  M0 is set here, right
// before its one use; no other instruction of these kernels reads M0 (checked
// in their gfx950 assembly), so clobbering it is safe.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_slab(uint32_t lds, const void* src, int lane) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(lds), "v"(lane * 16), "s"(src)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// The kernel's argument block (its only argument, at offset 0 of the kernarg
// segment) through a pointer the compiler cannot look through.  Fields read
// through it are loaded where they are used: the code at a unit's end reads
// its pointers this way, so they do not sit in scalar registers across the
// page loop (the scalar file is full there, and what does not fit is spilled
// into vector-register lanes and reloaded on every page).
__device__ __forceinline__ const DecodeArgs& args_late() {
  uint64_t p = uint64_t(__builtin_amdgcn_kernarg_segment_ptr());
  asm volatile("" : "+s"(p));
  return *(const DecodeArgs*)(const __attribute__((address_space(4))) DecodeArgs*)p;
}
template <class T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return uint32_t(size_t((__attribute__((address_space(3))) T*)p));
}

// Wait until at most `pages_after` pages' worth of ring loads are outstanding.
template <int SLABS, int S>
__device__ __forceinline__ void wait_ring(int pages_after) {
  static_assert(S <= 8 && SLABS * (S - 1) < 64, "ring depth vs vmcnt range");
  switch (pages_after) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<SLABS * 1 < 64 ? SLABS * 1 : 0>(); break;
    case 2: wait_vmcnt<SLABS * 2 < 64 ? SLABS * 2 : 0>(); break;
    case 3: wait_vmcnt<SLABS * 3 < 64 ? SLABS * 3 : 0>(); break;
    case 4: wait_vmcnt<SLABS * 4 < 64 ? SLABS * 4 : 0>(); break;
    case 5: wait_vmcnt<SLABS * 5 < 64 ? SLABS * 5 : 0>(); break;
    case 6: wait_vmcnt<SLABS * 6 < 64 ? SLABS * 6 : 0>(); break;
    default: wait_vmcnt<SLABS * 7 < 64 ? SLABS * 7 : 0>(); break;
  }
}

__device__ __forceinline__ int clamp_len(int L, int max_len) { return L < 0 ? 0 : (L > max_len ? max_len : L); }

// Tile-list modes: plain (units are sessions), private (units are sessions,
// followed by each decoder's private pages), cascade (units are groups of
// sessions sharing prefix pages, followed by each session's own pages).
enum { kPlain = 0, kPrivate = 1, kCascade = 2 };

// Position in the tile list: unit (gr = KV head * rowgroups + row group, unit b), page.
// Pages nsh.. of a unit belong to one owner at a time (private: a decoder;
// cascade: a session of the group): page pp of owner pn (pnpg pages, plen tokens).
struct Walker {
  int gr, b, page, npg;
  int nsh, pn, pp, pnpg, plen;
};

// Cascade unit tables in the workspace: first session, session count and
// common prefix pages of each unit.
__device__ __forceinline__ int unit_first(const DecodeArgs& a, int u) { return load_uniform(a.ws_units + u); }
__device__ __forceinline__ int unit_count(const DecodeArgs& a, int u) {
  return load_uniform(a.ws_units + a.batch + u);
}
__device__ __forceinline__ int unit_prefix(const DecodeArgs& a, int u) {
  return load_uniform(a.ws_units + 2 * a.batch + u);
}

__device__ __forceinline__ int seq_len(const DecodeArgs& a, int b) {
  return clamp_len(load_uniform(a.seq_lens + b), a.max_seq_len);
}
__device__ __forceinline__ int shared_pages(const DecodeArgs& a, int b) {
  return (seq_len(a, b) + kPage - 1) / kPage;
}

// Pages of unit b before its first owner page.
template <int MODE>
__device__ __forceinline__ int head_pages(const DecodeArgs& a, int b) {
  return MODE == kCascade ? unit_prefix(a, b) : shared_pages(a, b);
}

template <int MODE>
__device__ __forceinline__ int owners(const DecodeArgs& a, int b) {
  return MODE == kCascade ? unit_count(a, b) : a.num_decoders;
}

// Tokens of owner n of unit b.
template <int MODE>
__device__ __forceinline__ int owner_len(const DecodeArgs& a, int b, int n) {
  if (MODE == kCascade) return max(seq_len(a, unit_first(a, b) + n) - unit_prefix(a, b) * kPage, 0);
  return clamp_len(load_uniform(a.plens + int64_t(b) * a.num_decoders + n), a.max_priv_len);
}

// Physical page at walker position w.
template <int MODE>
__device__ __forceinline__ int page_id(const DecodeArgs& a, const Walker& w) {
  if (MODE == kCascade) {
    const int first = unit_first(a, w.b);
    if (w.page < w.nsh) return load_uniform(a.bt + int64_t(first) * a.bt_stride + w.page);
    return load_uniform(a.bt + int64_t(first + w.pn) * a.bt_stride + w.nsh + w.pp);
  }
  if (MODE == kPrivate && w.page >= w.nsh)
    return load_uniform(a.pbt + (int64_t(w.b) * a.num_decoders + w.pn) * a.pbt_stride + w.pp);
  return load_uniform(a.bt + int64_t(w.b) * a.bt_stride + w.page);
}

// First owner at or after n with pages (the caller knows one exists).
template <int MODE>
__device__ __forceinline__ void first_owner(const DecodeArgs& a, Walker& w, int n) {
  const int no = owners<MODE>(a, w.b);
  int U = owner_len<MODE>(a, w.b, n);
  while (U == 0 && n + 1 < no) U = owner_len<MODE>(a, w.b, ++n);
  w.pn = n;
  w.pp = 0;
  w.plen = U;
  w.pnpg = (U + kPage - 1) / kPage;
}

// Owner sub-position after w.page moved to the next page of the same unit, or
// to page 0 of a new unit (w.nsh already set).
template <int MODE>
__device__ __forceinline__ void enter_page(const DecodeArgs& a, Walker& w) {
  if (MODE == kPlain || w.page < w.nsh) return;
  if (w.page == w.nsh) first_owner<MODE>(a, w, 0);
  else if (++w.pp == w.pnpg) first_owner<MODE>(a, w, w.pn + 1);
}

// Page prefix sum over units: in LDS (plain and private, each workgroup builds
// it) or in the workspace (cascade, built by the plan kernel; scalar loads, so
// the LDS ring's vector-memory counter counts ring loads only).
struct LdsCum {
  const int* p;
  __device__ __forceinline__ int operator()(int i) const { return __builtin_amdgcn_readfirstlane(p[i]); }
};
struct WsCum {
  const int* p;
  __device__ __forceinline__ int operator()(int i) const { return load_uniform(p + i); }
};

// First nonempty unit at or after b (B if none).
template <class Cum>
__device__ __forceinline__ int next_nonempty(const Cum& cum, int b, int B) {
  while (b < B && cum(b + 1) == cum(b)) ++b;
  return b;
}

template <int MODE, class Cum>
__device__ __forceinline__ Walker seek(const DecodeArgs& a, const Cum& cum, int B, int Ptot, int64_t tau) {
  Walker w{};
  w.gr = int(tau / Ptot);
  const int r = int(tau % Ptot);
  int lo = 0, hi = B;  // largest b with cum[b] <= r, among b < B
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cum(mid) <= r) lo = mid;
    else hi = mid;
  }
  lo = next_nonempty(cum, lo, B);  // cum[b] <= r < cum[b+1] skips empty units
  w.b = lo;
  w.page = r - cum(lo);
  w.npg = cum(lo + 1) - cum(lo);
  if (MODE != kPlain && lo < B) {
    w.nsh = head_pages<MODE>(a, lo);
    if (w.page >= w.nsh) {  // find the owner and page of owner position page - nsh
      int q = w.page - w.nsh, n = 0;
      const int no = owners<MODE>(a, lo);
      for (;; ++n) {
        const int U = owner_len<MODE>(a, lo, n), np = (U + kPage - 1) / kPage;
        if (q < np || n + 1 == no) {
          w.pn = n;
          w.pp = q;
          w.plen = U;
          w.pnpg = np;
          break;
        }
        q -= np;
      }
    }
  }
  return w;
}

template <int MODE, class Cum>
__device__ __forceinline__ void advance(const DecodeArgs& a, Walker& w, const Cum& cum, int B) {
  if (++w.page < w.npg) {
    enter_page<MODE>(a, w);
    return;
  }
  w.page = 0;
  int b = next_nonempty(cum, w.b + 1, B);
  if (b >= B) {
    ++w.gr;
    b = next_nonempty(cum, 0, B);
  }
  w.b = b;
  w.npg = b < B ? cum(b + 1) - cum(b) : 0;
  if (MODE != kPlain && b < B) {
    w.nsh = head_pages<MODE>(a, b);
    enter_page<MODE>(a, w);
  }
}

// q / out row (index into [batch][N][H_q]) of row r of unit b and KV head g; -1
// past the unit's rows.
template <int MODE>
__device__ __forceinline__ int64_t unit_row(const DecodeArgs& a, int b, int g, int r) {
  const int G = a.num_q_heads / a.pool.num_kv_heads, NG = a.num_decoders * G;
  if (MODE == kCascade) {
    if (r >= unit_count(a, b) * NG) return -1;
    const int s = unit_first(a, b) + r / NG, n = (r % NG) / G;
    return (int64_t(s) * a.num_decoders + n) * a.num_q_heads + g * G + r % G;
  }
  if (r >= NG) return -1;
  return (int64_t(b) * a.num_decoders + r / G) * a.num_q_heads + g * G + r % G;
}

// Stream-K share boundaries.  A call cuts its tile list into n shares, WPG
// consecutive shares per workgroup (4 waves in the stream kernel, one wave pair
// in the cascade), n = 4 x the grid's workgroups (the device's CU count, at most
// 256; the host plans it), and the hardware places workgroup i on XCD i % 8.  A
// share on an even XCD weighs `even`, one on an odd XCD 512 - even, so all n
// weigh n * 256.  On MI355X (256 CUs) per-wave timestamps show the odd XCDs
// streaming KV pages slower than the even ones, by 4% to 13% depending on the
// GPU and the workload; 276 / 236 was the fastest split measured on the
// 8-decoder workload (2% faster than equal shares, calls alternating in one
// process), and other devices get equal shares.  The weights only move
// boundaries; any split is correct.
//
// The weight before share k is scaled to a whole of 2^18 by the multiplier
// mult = floor(2^26 / n) (exactly 2^16 at n = 1024), W(k) = (weight * mult) >>
// 16, so that a boundary is a multiply and a shift, no division:
// share_start(k) = (W(k) * T) >> 18, and share_start(n) = T.  W is
// non-decreasing and W(n) <= 2^18, so the shares tile 0 .. T in order.
#ifndef KVS_RING_PAGES_D128  // LDS ring depth per wave at D = 128 (8 KiB pages)
#define KVS_RING_PAGES_D128 4
#endif
constexpr int kShareWholeLog2 = 18;
struct Shares {
  int n;     // shares of the call: a multiple of 8 * WPG, at most 2^kDecodeShareLog2
  int even;  // weight of a share on an even XCD (1 .. 511)
  int mult;  // floor(2^26 / n)
};
__device__ __forceinline__ Shares call_shares(const DecodeArgs& a) {
  return Shares{4 * a.plan.blocks, a.plan.share_even, a.plan.share_mult};
}

// weight of shares 0 .. k-1, scaled to a whole of 2^18
template <int WPG>
__device__ __forceinline__ int64_t share_weight_before(int k, const Shares& sh) {
  static_assert(WPG == 1 || WPG == 4, "shares per workgroup");
  constexpr int kPer = 8 * WPG;  // shares of one round of 8 workgroups
  const int even = sh.even, odd = 512 - even;
  const int r = k % kPer, g = r / WPG;  // workgroup within the round = its XCD
  const int prev = ((g + 1) >> 1) * even + (g >> 1) * odd;  // XCDs 0 .. g-1
  const int raw = (k / kPer) * WPG * 4 * 512 + WPG * prev + (r % WPG) * ((g & 1) ? odd : even);
  return (int64_t(raw) * sh.mult) >> 16;
}
template <int WPG>
__device__ __forceinline__ int64_t share_start(int k, int64_t T, const Shares& sh) {
  return k >= sh.n ? T : (share_weight_before<WPG>(k, sh) * T) >> kShareWholeLog2;
}
// the share holding tile t < T: the largest k < n with share_start(k) <= t, i.e.
// with W(k) * T < (t + 1) * 2^18
template <int WPG>
__device__ __forceinline__ int share_of(int64_t t, int64_t T, const Shares& sh) {
  const int64_t lim = (t + 1) << kShareWholeLog2;
  int lo = 0, hi = sh.n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (share_weight_before<WPG>(mid, sh) * T < lim) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <int D, int NB, int MODE>
__device__ __forceinline__ void load_q(QFrag<D, NB>& qf, const DecodeArgs& a, int b, int g, int rg,
                                       int lane) {
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int64_t row = unit_row<MODE>(a, b, g, rg * 16 * NB + cb * 16 + (lane & 15));
    const uint16_t* qrow = a.q + (row < 0 ? 0 : row) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
      qf.q[cb][i] = row >= 0 ? *reinterpret_cast<const u32x4*>(qrow + 32 * i + 8 * (lane >> 4))
                             : u32x4{0u, 0u, 0u, 0u};
  }
}

// Output rows of column block cb of a unit from a merged state: out = acc / den,
// bf16 (den = 0: zeros).
template <int D, int NB, int MODE>
__device__ __forceinline__ void store_block(const DecodeArgs& a, const f32x4 (&acc)[D / 16], float den, int cb,
                                            int b, int g, int rg, int lane) {
  const int64_t row = unit_row<MODE>(a, b, g, rg * 16 * NB + cb * 16 + (lane & 15));
  if (row < 0) return;
  uint16_t* o = a.out + row * D;
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const f32x4 v = acc[i] * inv;
    *reinterpret_cast<u32x2*>(o + 16 * i + 4 * (lane >> 4)) = pack_bf16x4(v[0], v[1], v[2], v[3]);
  }
}

// A unit held wholly by one wave: its state is final.
template <int D, int NB, int MODE>
__device__ __forceinline__ void write_rows(const DecodeArgs& a, const RowState<D, NB>& st, int b, int g,
                                           int rg, int lane) {
  float den[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) den[cb] = wave_sum_across_quads(st.l[cb]);  // every lane takes part
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) store_block<D, NB, MODE>(a, st.acc[cb], den[cb], cb, b, g, rg, lane);
}

// Partial-state slot `slot` (16*NB rows): the accumulators in matrix-core
// fragment order (fragment (cb, i) is a contiguous 1 KiB, lane-major), then
// (m, l) per row.
//
// A partial state is written by a wave on one XCD and read, in the same
// launch, by the merging wave, which may sit on another XCD with its own L2.
// Both sides use device-scope buffer accesses (the sc1 cache-policy bit): the
// store is written through to where every XCD sees it, the load does not hit a
// stale line in its own L2.  The writer waits for its stores to complete before
// it arrives at the unit's counter; the merger loads only after the counter
// told it that every share has arrived.  No whole-L2 write-back or invalidate
// is needed (agent-scope fences cost tens of microseconds per call here).
constexpr int kDeviceScope = 16;       // sc1 in the buffer intrinsics' cache-policy argument
constexpr int kBufferWord3 = 0x00020000;  // gfx9 buffer descriptor: raw 32-bit elements

template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t acc_rsrc(const DecodeArgs& a) {
  // 2 slots per share, up to 2 row groups of 32 per slot on wave pairs: 2^11 * 64 rows * D floats
  return __builtin_amdgcn_make_buffer_rsrc(a.ws_acc, 0, int((2 << kDecodeShareLog2) * 64 * D * 4), kBufferWord3);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ml_rsrc(const DecodeArgs& a) {
  return __builtin_amdgcn_make_buffer_rsrc(a.ws_ml, 0, int((2 << kDecodeShareLog2) * 64 * 2 * 4), kBufferWord3);
}
// Byte offset of fragment (cb, i) in slot `slot`: wave-uniform, so it goes in the
// scalar offset of the buffer access (the lane's part, 16 * lane, is the vector
// offset), which keeps the per-fragment offsets out of vector registers.
template <int D, int NB>
__device__ __forceinline__ int acc_soff(int64_t slot, int cb, int i) {
  return __builtin_amdgcn_readfirstlane(int(slot * (16 * NB) * D * 4)) + (cb * (D / 16) + i) * kWave * 16;
}
template <int NB>
__device__ __forceinline__ int ml_off(int64_t slot, int r) {
  return int(slot * (16 * NB) * 2 * 4) + r * 8;
}

template <int D, int NB>
__device__ __forceinline__ void write_partial(const DecodeArgs& a, const RowState<D, NB>& st, int64_t slot,
                                              int lane) {
  const __amdgpu_buffer_rsrc_t racc = acc_rsrc<D>(a), rml = ml_rsrc(a);
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const float l = wave_sum_across_quads(st.l[cb]);
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      __builtin_amdgcn_raw_buffer_store_b128(st.acc[cb][i], racc, lane * 16, acc_soff<D, NB>(slot, cb, i),
                                             kDeviceScope);
    if (lane < 16) {  // two 4-byte stores: a vector built from st.m kept RowState in scratch
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(st.m[cb]), rml, ml_off<NB>(slot, cb * 16 + lane), 0,
                                            kDeviceScope);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l), rml, ml_off<NB>(slot, cb * 16 + lane) + 4, 0,
                                            kDeviceScope);
    }
  }
}

// Tiles of the unit [s_u, e_u) that shares p .. q hold.
template <int WPG>
__device__ __forceinline__ int range_tiles(int p, int q, int64_t s_u, int64_t e_u, int64_t T, const Shares& sh) {
  const int64_t lo = max(s_u, share_start<WPG>(p, T, sh)), hi = min(e_u, share_start<WPG>(q + 1, T, sh));
  return hi > lo ? int(hi - lo) : 0;
}

// Merge tree over the shares of a split unit: a node at level lv joins up to
// 2^kMergeFanLog2 children (shares at level 1, level-(lv-1) nodes above), so a
// unit spanning dozens of shares is merged by several waves, a level at a time,
// instead of all by one.
constexpr int kMergeFanLog2 = 3;
constexpr int kMergeLevels = 4;  // 8^4 >= 2^10 shares
// arrival counters per level: (2 * share + x) * 2 + row group < 2^12
constexpr int kCountersPerLevel = 4 << kDecodeShareLog2;
static_assert(kMergeLevels * kCountersPerLevel * 4 <= int(kDecodeCounterBytes), "counter region");

// The end of a wave's part of a unit that other shares also hold.  The wave
// has stored its partial state (m, l, acc) with write_partial.  It then climbs
// the unit's merge tree: at each node it waits for its stores, adds its
// subtree's tile count to the node's arrival counter with a vector atomic, and
// stops unless its addition completes the node's tiles; the wave that completes
// a node merges the node's children in share order,
//   m* = max m_c,  acc* = sum_c 2^(m_c - m*) acc_c,  l* = sum_c 2^(m_c - m*) l_c,
// and writes the result into the slot of the node's first share with tiles
// (or, at the root, writes out = acc* / l*).  The tree and the order are fixed,
// so the result does not depend on which waves arrive last.  Each node's last
// arriver puts the counter back to zero, so every counter is zero again when
// the call ends.  A share begins at most one unit that it does not finish, and
// continues at most one, so the node starting at share g of a unit that begins
// in share k0 uses counter (2g + (g == k0))*mul + add of its level, and share
// f's state sits in partial slot (2f + (f == k0))*mul + add (mul = 1, add = 0
// on the stream kernel; mul = 2, add = the row group on wave pairs).
template <int D, int NB, int MODE, int WPG, int KB>
__device__ __forceinline__ void finish_split(const DecodeArgs& a, int k, bool before, int mul, int add, int mine,
                                             int npg, int64_t s_u, int64_t T, int b, int g, int rg, int lane) {
  const Shares sh = call_shares(a);
  const int64_t e_u = s_u + npg;
  const int k0 = before ? share_of<WPG>(s_u, T, sh) : k;
  const int k1 = share_of<WPG>(e_u - 1, T, sh);
  auto slot_of = [&](int f) { return int64_t(2 * f + (f == k0 ? 1 : 0)) * mul + add; };
  // Every share holds at least one tile when T * (the smallest scaled share
  // weight) >= 2^18 (a share's scaled weight is at least floor(its weight x mult / 2^16)):
  // then the unit's shares k0 .. k1 all hold tiles of it, and a range of them
  // starts with a share holding tiles.  Otherwise, search.
  const bool dense = T * ((min(sh.even, 512 - sh.even) * int64_t(sh.mult)) >> 16) >= (int64_t(1) << kShareWholeLog2);
  // the first share of p .. q that holds tiles of the unit (the range has some)
  auto first_with_tiles = [&](int p) {
    return dense ? max(p, k0) : share_of<WPG>(max(s_u, share_start<WPG>(p, T, sh)), T, sh);
  };
  const __amdgpu_buffer_rsrc_t racc = acc_rsrc<D>(a), rml = ml_rsrc(a);
  int child = k, tiles = mine;
  // the wave's partial state has reached device scope before it arrives anywhere
  drain();
#pragma unroll 1
  for (int lv = 1; lv <= kMergeLevels; ++lv) {
    const int span = 1 << (kMergeFanLog2 * lv), cspan = span >> kMergeFanLog2;
    const int g0 = k0 + ((child - k0) >> (kMergeFanLog2 * lv) << (kMergeFanLog2 * lv));
    const int g1 = min(g0 + span - 1, k1);
    const int expect = range_tiles<WPG>(g0, g1, s_u, e_u, T, sh);
    if (expect == tiles) {  // the arriving subtree is the node's only child with tiles
      child = g0;
      continue;
    }
    int* ctr = a.ws_cnt + (lv - 1) * kCountersPerLevel + (2 * g0 + (g0 == k0 ? 1 : 0)) * mul + add;
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(ctr, tiles, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readlane(old, 0);
    if (old + tiles != expect) return;
    if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // every arrival is in
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const bool root = g1 == k1 && g0 == k0;
    const int64_t dst = root ? 0 : slot_of(first_with_tiles(g0));
    // the node's children, child c on lane c: the slot holding its state, or -1
    // for a child without tiles of the unit (a level-1 child is a share, which
    // holds its own state; a higher child's state sits in its first share with
    // tiles).  One vector register instead of eight scalar pairs: scalar
    // registers live here would be spilled inside the page loop.
    int cslot = -1;
    {
      const int p = g0 + lane * cspan, q = min(p + cspan - 1, g1);
      if (lane < (1 << kMergeFanLog2) && p <= g1 && (dense || range_tiles<WPG>(p, q, s_u, e_u, T, sh) > 0))
        cslot = int(slot_of(lv == 1 ? p : first_with_tiles(p)));
    }
    const uint64_t has_child = __ballot(cslot >= 0);
    // one 16-row column block at a time (fewer live registers); children in
    // batches of KB, every load of a batch issued before any merge
#pragma unroll 1
    for (int cb = 0; cb < NB; ++cb) {
      float M = -INFINITY, den = 0.f;
      f32x4 acc[D / 16];
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c0 = 0; c0 < (1 << kMergeFanLog2); c0 += KB) {
        // (a child of only empty shares can sit between children with tiles)
        if (((has_child >> c0) & ((1u << KB) - 1)) == 0) continue;
        f32x2 mlv[KB];
        f32x4 av[KB][D / 16];
        bool use[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          const int slot = __builtin_amdgcn_readlane(cslot, c0 + u);
          use[u] = slot >= 0;
          mlv[u] = f32x2{-INFINITY, 0.f};
          if (!use[u]) continue;
          const u32x2 mlb = __builtin_amdgcn_raw_buffer_load_b64(rml, ml_off<NB>(slot, cb * 16 + (lane & 15)), 0,
                                                                 kDeviceScope);
          mlv[u] = f32x2{__uint_as_float(mlb[0]), __uint_as_float(mlb[1])};
#pragma unroll
          for (int i = 0; i < D / 16; ++i)
            av[u][i] = __builtin_amdgcn_raw_buffer_load_b128(racc, lane * 16, acc_soff<D, NB>(slot, cb, i),
                                                             kDeviceScope);
        }
#pragma unroll
        for (int u = 0; u < KB; ++u) {
          if (!use[u] || mlv[u][0] == -INFINITY) continue;  // no child, or a child that saw no key of this row
          const float Mn = fmaxf(M, mlv[u][0]);
          const float c = exp2_fast(M - Mn), w = exp2_fast(mlv[u][0] - Mn);  // exp2(-inf) = 0
          den = den * c + w * mlv[u][1];
#pragma unroll
          for (int i = 0; i < D / 16; ++i) acc[i] = acc[i] * c + w * av[u][i];
          M = Mn;
        }
      }
      if (root) {
        store_block<D, NB, MODE>(a, acc, den, cb, b, g, rg, lane);
      } else {
#pragma unroll
        for (int i = 0; i < D / 16; ++i)
          __builtin_amdgcn_raw_buffer_store_b128(acc[i], racc, lane * 16, acc_soff<D, NB>(dst, cb, i), kDeviceScope);
        if (lane < 16) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(M), rml, ml_off<NB>(dst, cb * 16 + lane), 0,
                                                kDeviceScope);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(den), rml, ml_off<NB>(dst, cb * 16 + lane) + 4, 0,
                                                kDeviceScope);
        }
      }
    }
    if (root) break;
    // the merged state has reached device scope before the next arrival
    drain();
    child = g0;
    tiles = expect;
  }
  drain();
}

// Zeros for the rows of units without tiles (softmax over nothing): units
// idx = first, first + step, ... of nunits; unit idx is (gr = idx / nb_units,
// b = idx % nb_units), empty(b) tells whether it has no tiles.
template <int D, int NB, int MODE, class Empty>
__device__ __forceinline__ void zero_empty_units(const DecodeArgs& a, int nunits, int nb_units, int rowgroups,
                                                 int rg_fixed, int first, int step, const Empty& empty,
                                                 int lane) {
  constexpr int RG = 16 * NB, CH = D / 8;  // 16-byte chunks per row
#pragma unroll 1
  for (int idx = first; idx < nunits; idx += step) {
    const int b = idx % nb_units, gr = idx / nb_units;
    if (!empty(b)) continue;
    const int g = rg_fixed >= 0 ? gr : gr / rowgroups, rg = rg_fixed >= 0 ? rg_fixed : gr % rowgroups;
#pragma unroll 1
    for (int e = lane; e < RG * CH; e += kWave) {
      const int64_t row = unit_row<MODE>(a, b, g, rg * RG + e / CH);
      if (row >= 0) reinterpret_cast<u32x4*>(a.out + row * D)[e % CH] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Private pages of all decoders of session b (per-thread loads; flags bad lengths).
__device__ __forceinline__ int priv_pages(const DecodeArgs& a, int b) {
  int pages = 0;
  for (int n = 0; n < a.num_decoders; ++n) {
    const int U = a.plens[int64_t(b) * a.num_decoders + n];
    if ((U < 0 || U > a.max_priv_len) && blockIdx.x == 0) flag_error(a.dev_status, KVS_DEV_BAD_LEN_BIT);
    pages += (clamp_len(U, a.max_priv_len) + kPage - 1) / kPage;
  }
  return pages;
}

// APPEND (plain mode): the step's token of each session is written into its
// slot, position seq_lens[b] - 1, by the wave that attends that page.  That
// wave puts the new K row and V column into its LDS copy of the page after the
// page has landed (so what the page load read of that slot does not matter), and
// the wave of row group 0 also stores them to the pool for later calls.
template <int D, int NB, int S, int MODE, bool APPEND>
__global__ __launch_bounds__(256, 1) void decode_stream_kernel(DecodeArgs a) {
  static_assert(MODE != kCascade, "cascade units run on decode_pair_kernel");
  static_assert(!APPEND || MODE == kPlain, "the fused append is a plain-mode call");
  constexpr int SLABS = D / 16;  // 1 KiB slabs per (page, head) tile: K slabs then V slabs
  __shared__ u32x4 ring[kWaves][S][SLABS * 64];
  __shared__ int cum_s[kDecodeMaxBatch + 1];
  __shared__ int part_s[256];

  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: lets the compiler
  const int Hkv = a.pool.num_kv_heads, RGs = a.plan.rowgroups;  // use scalar loads
  const int B = a.batch;

  // ---- pages per session and their exclusive prefix sum (every workgroup) ----
  // Each thread counts the pages of a run of sessions into cum_s, then turns its
  // run into an exclusive prefix sum in place once the runs' totals are scanned.
  const int chunk = (B + 255) / 256;
  int local = 0;
  for (int i = 0; i < chunk; ++i) {
    const int b = tid * chunk + i;
    if (b < B) {
      const int L = a.seq_lens[b];
      if ((L < 0 || L > a.max_seq_len) && blockIdx.x == 0) flag_error(a.dev_status, KVS_DEV_BAD_LEN_BIT);
      int pages = (clamp_len(L, a.max_seq_len) + kPage - 1) / kPage;
      if (MODE == kPrivate) pages += priv_pages(a, b);
      cum_s[b] = pages;
      local += pages;
    }
  }
  part_s[tid] = local;
  __syncthreads();
  if (wave == 0) {
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = part_s[lane * 4 + i]; s += v[i]; }
    int incl = s;  // inclusive scan over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    int run = incl - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) { part_s[lane * 4 + i] = run; run += v[i]; }
  }
  __syncthreads();
  {
    int run = part_s[tid];
    for (int i = 0; i < chunk; ++i) {
      const int b = tid * chunk + i;
      if (b < B) {
        const int pages = cum_s[b];
        cum_s[b] = run;
        run += pages;
      }
    }
    if (tid == 255) cum_s[B] = run;
  }
  __syncthreads();

  const int Ptot = cum_s[B];
  const int64_t T = int64_t(Ptot) * Hkv * RGs;
  const int k = blockIdx.x * kWaves + wave;  // the grid is a.plan.blocks workgroups
  const Shares sh = call_shares(a);
  zero_empty_units<D, NB, MODE>(a, Hkv * RGs * B, B, RGs, -1, k, sh.n,
                                [&](int b) { return cum_s[b + 1] == cum_s[b]; }, lane);
  // Nothing outstanding before the ring starts.  (Without this wait the
  // compiler also waits for every outstanding load before a ring page's LDS
  // reads, on every page.)
  __builtin_amdgcn_s_waitcnt(0);
  const int64_t tau0 = share_start<kWaves>(k, T, sh), tau1 = share_start<kWaves>(k + 1, T, sh);
  if (tau0 >= tau1) return;  // no barriers follow
  const int n = int(tau1 - tau0);

  const int num_pages = a.pool.num_pages;
  uint32_t bad = 0;  // ring slots whose page id was out of range

  // private mode: the unit's row (within its KV head) of the lane's row in
  // column block 0 (column block cb adds 16 cb); decoder n holds rows nG .. nG+G-1
  int row_base = 0;
  const int G = a.num_q_heads / Hkv;
  auto set_owners = [&](int rg) { row_base = rg * 16 * NB + (lane & 15); };

  const LdsCum cum{cum_s};
  Walker iw = seek<MODE>(a, cum, B, Ptot, tau0);
  Walker cw = iw;
  if (MODE == kPrivate) set_owners(cw.gr % RGs);
  auto issue = [&](int slot) {
    const int g = iw.gr / RGs;
    int pid = page_id<MODE>(a, iw);
    const bool ok = pid >= 0 && pid < num_pages;
    bad = ok ? (bad & ~(1u << slot)) : (bad | (1u << slot));
    if (!ok) {
      flag_error(a.dev_status, KVS_DEV_BAD_PAGE_BIT);
      __builtin_amdgcn_s_waitcnt(0);
      pid = 0;  // stream a harmless in-range page, skip it at compute time
    }
    const u32x4* tile = reinterpret_cast<const u32x4*>(a.pool.data + tile_offset(a.layer, pid, g, num_pages, Hkv, D));
    const uint32_t dst = lds_addr(&ring[wave][slot][0]);
#pragma unroll
    for (int s = 0; s < SLABS; ++s) dma_slab(dst + s * 1024, tile + s * 64, lane);
    advance<MODE>(a, iw, cum, B);
  };

  // the step's token of the current unit (APPEND): 8 head dims of K on each of
  // the first D/8 lanes, D/64 head dims of V on every lane
  u32x4 knew = {0u, 0u, 0u, 0u};
  uint16_t vnew[D / 64] = {};
  auto load_new = [&](int b, int g) {
    if constexpr (APPEND) {
      if (b >= B) return;
      const int64_t row = (int64_t(b) * Hkv + g) * D;
      if (lane < D / 8) knew = reinterpret_cast<const u32x4*>(a.k_new + row)[lane];
#pragma unroll
      for (int c = 0; c < D / 64; ++c) vnew[c] = a.v_new[row + lane + 64 * c];
    }
  };
  // write the token into slot t of a page tile (LDS copy or pool)
  auto put_token = [&](auto* tile, int t) {
    uint16_t* t16 = reinterpret_cast<uint16_t*>(tile);
    if (lane < D / 8) reinterpret_cast<u32x4*>(tile)[k_run(lane / 4, lane % 4, t)] = knew;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      const int d = lane + 64 * c;
      t16[v_run(D, d / 16, t / 8, d % 16) * 8 + t % 8] = vnew[c];
    }
  };

  // The first ring pages are issued before the queries (and the step's token)
  // are loaded, so that the two latencies overlap.  Both are waited for before
  // the page loop (vector-memory loads complete in order): any non-DMA load
  // still outstanding at the loop makes the compiler wait for every outstanding
  // load before each page's LDS reads.
#pragma unroll 1
  for (int j = 0; j < S - 1 && j < n; ++j) issue(j);
  QFrag<D, NB> qf;
  RowState<D, NB> st;
  st.init();
  load_q<D, NB, MODE>(qf, a, cw.b, cw.gr / RGs, cw.gr % RGs, lane);
  load_new(cw.b, cw.gr / RGs);
  __builtin_amdgcn_s_waitcnt(0);
  int64_t unit_begin = int64_t(cw.gr) * Ptot + cum_s[cw.b];  // first tile of the current unit

#pragma unroll 1
  for (int j = 0; j < n; ++j) {
    const int slot = j % S;
    if (j + S - 1 < n) issue((j + S - 1) % S);
    wait_ring<SLABS, S>(min(S - 1, n - 1 - j));
    if (!((bad >> slot) & 1u)) {
      if constexpr (APPEND) {
        const int L = load_uniform(a.seq_lens + cw.b);
        if (cw.page == cw.npg - 1 && L >= 1 && L <= a.max_seq_len) {  // the page of position L - 1
          const int t = (L - 1) % kPage;
          put_token(ring[wave][slot], t);
          if (cw.gr % RGs == 0) {
            const int pid = load_uniform(a.bt + int64_t(cw.b) * a.bt_stride + cw.page);  // in range: slot not bad
            put_token(a.pool.data + tile_offset(a.layer, pid, cw.gr / RGs, num_pages, Hkv, D), t);
          }
        }
      }
      u32x4 kf[D / 32];
      u32x2 vf[D / 16];
      const u32x2* v2 = reinterpret_cast<const u32x2*>(ring[wave][slot]);
#pragma unroll
      for (int i = 0; i < D / 32; ++i) kf[i] = ring[wave][slot][k_run(i, lane >> 4, lane & 15)];
#pragma unroll
      for (int i = 0; i < D / 16; ++i) vf[i] = v2[2 * v_run(D, i, lane >> 5, lane & 15) + ((lane >> 4) & 1)];
      int lim[NB], nvalid;
      bool masked;
      if (MODE == kPrivate && cw.page >= cw.nsh) {
        // a private page of decoder pn: only its rows see it (with several row
        // groups every row group walks all private pages of the session, and a
        // group holding no row of decoder pn masks the whole page)
        nvalid = min(kPage, cw.plen - cw.pp * kPage);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
          lim[cb] = uint32_t(row_base + cb * 16 - cw.pn * G) < uint32_t(G) ? nvalid : 0;
        masked = true;
      } else {
        const int L = seq_len(a, cw.b);
        nvalid = min(kPage, L - cw.page * kPage);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) lim[cb] = nvalid;
        masked = nvalid < kPage;
      }
      attend_page<D, NB>(st, qf, kf, vf, a.scale_log2, masked, lim, nvalid, lane);
    }
    const int cur_gr = cw.gr, cur_b = cw.b;
    advance<MODE>(a, cw, cum, B);
    const bool last = (j == n - 1);
    if (last || cw.gr != cur_gr || cw.b != cur_b) {
      // unit (cur_gr, cur_b) ends here for this wave
      const int npg_u = cum_s[cur_b + 1] - cum_s[cur_b];
      const int64_t unit_end = unit_begin + npg_u;
      const bool before = unit_begin < tau0, after = unit_end > tau1;
      const DecodeArgs& al = args_late();
      if (!before && !after) {
        write_rows<D, NB, MODE>(al, st, cur_b, cur_gr / RGs, cur_gr % RGs, lane);
      } else {  // split: the share's first unit (continued) or its last one (begun)
        write_partial<D, NB>(al, st, k * 2 + (before ? 0 : 1), lane);
        finish_split<D, NB, MODE, kWaves, (NB >= 4 ? 1 : 4 / NB)>(
            al, k, before, 1, 0, int(min(unit_end, tau1) - max(unit_begin, tau0)), npg_u, unit_begin, T, cur_b,
            cur_gr / RGs, cur_gr % RGs, lane);
      }
      if (!last) {
        st.init();
        load_q<D, NB, MODE>(qf, al, cw.b, cw.gr / RGs, cw.gr % RGs, lane);
        load_new(cw.b, cw.gr / RGs);
        if (MODE == kPrivate) set_owners(cw.gr % RGs);
        unit_begin = int64_t(cw.gr) * Ptot + cum_s[cw.b];
      }
      // Stores (their data registers), merge loads and q loads drained before
      // the ring resumes: whatever the compiler cannot prove complete at the
      // loop head makes it wait for every outstanding load before each page's
      // LDS reads.
      drain();
    }
  }
}

// Cascade units on wave pairs.  A unit's rows (its sessions x N x G, at most
// 64) form two 32-row groups, one per wave of a 2-wave workgroup.  Both waves
// walk the same share of the per-KV-head tile list (each unit: its common
// prefix pages once, then every session's own pages) through one shared LDS
// ring: each wave streams half of every page, paced by its own vector-memory
// counter, and one s_barrier per page tells both that the whole page has
// landed and that the slot read on the previous step may be refilled.  A wave
// skips the page step on pages none of its rows see (the own pages of a
// session whose rows sit in the other wave), so a prefix page is read once for
// all the unit's rows, an own page serves its session's rows only, and every
// wave keeps the 32-row register budget that lets two waves share a SIMD.
template <int D, int S>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void decode_pair_kernel(DecodeArgs a) {
  constexpr int MODE = kCascade, NB = 2, RG = 16 * NB;
  constexpr int SLABS = D / 16, HALF = SLABS / 2;  // 1 KiB slabs per tile; each wave loads half
  __shared__ u32x4 ring[S][SLABS * 64];

  const int lane = threadIdx.x & 63;
  const int rg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // this wave's row group
  const int Hkv = a.pool.num_kv_heads, NG = a.num_decoders * (a.num_q_heads / Hkv);
  const int B = load_uniform(a.ws_units + 3 * a.batch);
  const WsCum cum{a.ws_cum};
  const int Ptot = cum(B);
  const int64_t T = int64_t(Ptot) * Hkv;
  const int k = blockIdx.x;  // the grid is one pair per share
  // each wave zeroes its own rows of units without tiles
  const Shares sh = call_shares(a);
  zero_empty_units<D, NB, MODE>(a, Hkv * B, B, 1, rg, k, sh.n,
                                [&](int u) { return cum(u + 1) == cum(u); }, lane);
  const int64_t tau0 = share_start<1>(k, T, sh), tau1 = share_start<1>(k + 1, T, sh);
  if (tau0 >= tau1) return;  // both waves alike: no barriers follow
  const int n = int(tau1 - tau0);

  const int num_pages = a.pool.num_pages;
  uint32_t bad = 0;  // ring slots whose page id was out of range (both waves agree)
  // session (within the unit) of each of the lane's rows, and the sessions this
  // wave holds rows of
  int row_owner[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) row_owner[cb] = (rg * RG + cb * 16 + (lane & 15)) / NG;
  const int own_lo = rg * RG / NG, own_hi = (rg * RG + RG - 1) / NG;

  Walker iw = seek<MODE>(a, cum, B, Ptot, tau0);
  Walker cw = iw;
  auto issue = [&](int slot) {
    int pid = page_id<MODE>(a, iw);
    const bool ok = pid >= 0 && pid < num_pages;
    bad = ok ? (bad & ~(1u << slot)) : (bad | (1u << slot));
    if (!ok) {
      if (rg == 0) flag_error(a.dev_status, KVS_DEV_BAD_PAGE_BIT);
      __builtin_amdgcn_s_waitcnt(0);
      pid = 0;  // stream a harmless in-range page, skip it at compute time
    }
    const u32x4* tile = reinterpret_cast<const u32x4*>(a.pool.data + tile_offset(a.layer, pid, iw.gr, num_pages, Hkv, D));
    const uint32_t dst = lds_addr(&ring[slot][0]);
#pragma unroll
    for (int h = 0; h < HALF; ++h) {
      const int s = rg * HALF + h;
      dma_slab(dst + s * 1024, tile + s * 64, lane);
    }
    advance<MODE>(a, iw, cum, B);
  };

  // the first ring pages before the queries, so that the two latencies overlap
  // (both are waited for before the page loop, as in the stream kernel)
#pragma unroll 1
  for (int j = 0; j < S - 1 && j < n; ++j) issue(j);
  QFrag<D, NB> qf;
  RowState<D, NB> st;
  st.init();
  load_q<D, NB, MODE>(qf, a, cw.b, cw.gr, rg, lane);
  __builtin_amdgcn_s_waitcnt(0);
  int64_t unit_begin = int64_t(cw.gr) * Ptot + cum(cw.b);  // first tile of the current unit

#pragma unroll 1
  for (int j = 0; j < n; ++j) {
    const int slot = j % S;
    // this wave's half of page j has landed (pages j+1 .. j+S-2 may be in flight)
    wait_ring<HALF, S>(min(S - 2, n - 1 - j));
    // ... and the other wave's half; both are done reading page j-1's slot
    __builtin_amdgcn_s_barrier();
    if (j + S - 1 < n) issue((j + S - 1) % S);
    const int rows = unit_count(a, cw.b) * NG;
    const bool prefix = cw.page < cw.nsh;
    const bool mine = rg * RG < rows && (prefix || (cw.pn >= own_lo && cw.pn <= own_hi));
    if (mine && !((bad >> slot) & 1u)) {
      u32x4 kf[D / 32];
      u32x2 vf[D / 16];
      const u32x2* v2 = reinterpret_cast<const u32x2*>(ring[slot]);
#pragma unroll
      for (int i = 0; i < D / 32; ++i) kf[i] = ring[slot][k_run(i, lane >> 4, lane & 15)];
#pragma unroll
      for (int i = 0; i < D / 16; ++i) vf[i] = v2[2 * v_run(D, i, lane >> 5, lane & 15) + ((lane >> 4) & 1)];
      int lim[NB], nvalid;
      bool masked;
      if (!prefix) {  // an own page of session pn: only its rows see it
        nvalid = min(kPage, cw.plen - cw.pp * kPage);
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) lim[cb] = (row_owner[cb] == cw.pn) ? nvalid : 0;
        masked = own_lo != own_hi || nvalid < kPage;
      } else {  // prefix pages are whole pages of every session of the unit
        nvalid = kPage;
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) lim[cb] = kPage;
        masked = false;
      }
      attend_page<D, NB>(st, qf, kf, vf, a.scale_log2, masked, lim, nvalid, lane);
    }
    const int cur_gr = cw.gr, cur_b = cw.b;
    advance<MODE>(a, cw, cum, B);
    const bool last = (j == n - 1);
    if (last || cw.gr != cur_gr || cw.b != cur_b) {
      // unit (cur_gr, cur_b) ends here for this pair
      const int npg_u = cum(cur_b + 1) - cum(cur_b);
      const int64_t unit_end = unit_begin + npg_u;
      const bool before = unit_begin < tau0, after = unit_end > tau1;
      const DecodeArgs& al = args_late();
      if (!before && !after) {
        write_rows<D, NB, MODE>(al, st, cur_b, cur_gr, rg, lane);
      } else {  // each wave of the pair merges its own row group
        write_partial<D, NB>(al, st, (k * 2 + (before ? 0 : 1)) * 2 + rg, lane);
        finish_split<D, NB, MODE, 1, 1>(al, k, before, 2, rg, int(min(unit_end, tau1) - max(unit_begin, tau0)),
                                        npg_u, unit_begin, T, cur_b, cur_gr, rg, lane);
      }
      if (!last) {
        st.init();
        load_q<D, NB, MODE>(qf, al, cw.b, cw.gr, rg, lane);
        unit_begin = int64_t(cw.gr) * Ptot + cum(cw.b);
      }
      drain();  // stores and q loads drained before the ring resumes (see the stream kernel)
    }
  }
}

// Inclusive scan (op = + or max) of one value per thread over a 1024-thread
// workgroup: a shuffle scan inside each wave, then the 16 wave totals.  On
// return buf[t] holds thread t's inclusive value.
template <bool MAX>
__device__ __forceinline__ int block_scan(int x, int* buf) {
  __shared__ int wave_total[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(x, off);
    if (lane >= off) x = MAX ? max(x, t) : x + t;
  }
  if (lane == 63) wave_total[w] = x;
  __syncthreads();
  int carry = MAX ? INT_MIN : 0;
  for (int i = 0; i < w; ++i) carry = MAX ? max(carry, wave_total[i]) : carry + wave_total[i];
  x = MAX ? max(x, carry) : x + carry;
  buf[tid] = x;
  __syncthreads();  // buf complete, and wave_total free for the next scan
  return x;
}

// 64-bit finalizer of the splitmix64 generator (Steele, Lea and Flood, "Fast
// splittable pseudorandom number generators", OOPSLA 2014).
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Cascade plan.  Sessions with equal, non-negative group ids that are adjacent in
// the batch share their first group_prefix[b] pages.  Runs of such sessions are
// cut into units of at most `per_unit` sessions (all rows of a unit fit one
// wave pair); each unit gets its first session, session count, common prefix pages
// and its tile count (the prefix once, then every session's pages past it).
// One workgroup of 1024 threads, 4 sessions per thread (batch <= 4096).
// Flags: members whose group_prefix differs from the unit's first session's
// (BAD_LEN), and shared-prefix block-table entries that differ from the first
// session's (BAD_PAGE); the prefix read is always the first session's.
//
// The tables depend only on the batch, the sessions per unit, the length bound
// and every session's length, group id and prefix claim, which the layers of a
// decode step share.  A 64-bit fingerprint of those inputs is stored with the
// tables; a call whose inputs hash to the stored fingerprint finds its tables
// already in the workspace and returns at once, so a step plans once for all
// its layers (the block-table checks run when the tables are rebuilt).
__global__ __launch_bounds__(1024) void decode_cascade_plan_kernel(DecodeArgs a, int per_unit) {
  constexpr int E = 4;
  __shared__ int buf[1024];
  __shared__ int gid_s[kDecodeMaxBatch];
  __shared__ int ui_s[kDecodeMaxBatch];
  __shared__ int first_s[kDecodeMaxBatch];
  __shared__ int pref_s[kDecodeMaxBatch];
  __shared__ int voff_s[kDecodeMaxBatch + 1];
  __shared__ uint64_t fp_s[16];
  const int B = a.batch, tid = threadIdx.x;
  {
    uint64_t h = 0;
    for (int i = 0; i < E; ++i) {
      const int b = tid * E + i;
      if (b < B) {
        const uint64_t lg = (uint64_t(uint32_t(a.seq_lens[b])) << 32) | uint32_t(a.group_id[b]);
        h ^= mix64(mix64(lg ^ (uint64_t(b) << 20)) ^ uint64_t(uint32_t(a.group_prefix[b])));
      }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t lo = __shfl_xor(uint32_t(h), off), hi = __shfl_xor(uint32_t(h >> 32), off);
      h ^= (uint64_t(hi) << 32) | lo;
    }
    if ((tid & 63) == 0) fp_s[tid >> 6] = h;
    __syncthreads();
    h = mix64((uint64_t(uint32_t(B)) << 40) ^ (uint64_t(uint32_t(per_unit)) << 32) ^ uint32_t(a.max_seq_len));
#pragma unroll
    for (int w = 0; w < 16; ++w) h ^= fp_s[w];
    const uint32_t* stored = reinterpret_cast<const uint32_t*>(a.ws_units + 3 * B + 1);
    if (stored[0] == uint32_t(h) && stored[1] == uint32_t(h >> 32)) return;  // whole workgroup: uniform
    __syncthreads();  // every thread has compared before thread 0 rewrites the fingerprint below
    if (tid == 0) fp_s[0] = h;
  }
  int L[E], us[E];
  for (int i = 0; i < E; ++i) {
    const int b = tid * E + i;
    if (b < B) gid_s[b] = a.group_id[b];
    L[i] = b < B ? clamp_len(a.seq_lens[b], a.max_seq_len) : 0;
  }
  __syncthreads();
  // 1. run starts (a run: adjacent sessions of one non-negative group id)
  int rs[E], loc = INT_MIN;
  for (int i = 0; i < E; ++i) {
    const int b = tid * E + i;
    const bool start = b < B && (b == 0 || gid_s[b] < 0 || gid_s[b] != gid_s[b - 1]);
    if (start) loc = b;
    rs[i] = loc;
  }
  block_scan<true>(loc, buf);
  const int carry = tid > 0 ? buf[tid - 1] : INT_MIN;
  __syncthreads();
  // 2. unit starts and unit indices
  int cnt = 0;
  for (int i = 0; i < E; ++i) {
    const int b = tid * E + i;
    const int r = max(rs[i], carry);
    us[i] = (b < B && (b - r) % per_unit == 0) ? 1 : 0;
    cnt += us[i];
  }
  const int incl = block_scan<false>(cnt, buf);
  const int nu = buf[1023];
  __syncthreads();
  {
    int run = incl - cnt;
    for (int i = 0; i < E; ++i) {
      const int b = tid * E + i;
      run += us[i];
      if (b < B) ui_s[b] = run - 1;
      if (us[i]) first_s[run - 1] = b;
    }
  }
  __syncthreads();
  // 3. per unit: session count and common prefix pages
  for (int i = 0; i < E; ++i) {
    if (!us[i]) continue;
    const int b = tid * E + i, u = ui_s[b];
    const int count = (u + 1 < nu ? first_s[u + 1] : B) - b;
    const int claim = gid_s[b] < 0 ? 0 : a.group_prefix[b];
    int P = max(0, min(claim, L[i] / kPage));
    for (int m = b + 1; m < b + count; ++m) {
      if (a.group_prefix[m] != claim) flag_error(a.dev_status, KVS_DEV_BAD_LEN_BIT);
      P = min(P, clamp_len(a.seq_lens[m], a.max_seq_len) / kPage);
    }
    pref_s[u] = P;
    a.ws_units[u] = b;
    a.ws_units[B + u] = count;
    a.ws_units[2 * B + u] = P;
  }
  __syncthreads();
  // 4. tiles per unit: the prefix once, then every session's pages past it
  int c = 0, v = 0, cl[E], vl[E];
  for (int i = 0; i < E; ++i) {
    const int b = tid * E + i;
    const int P = b < B ? pref_s[ui_s[b]] : 0;
    cl[i] = b < B ? (L[i] + kPage - 1) / kPage - (us[i] ? 0 : P) : 0;
    vl[i] = (b < B && !us[i]) ? P : 0;
    c += cl[i];
    v += vl[i];
  }
  const int incl_c = block_scan<false>(c, buf);
  const int total = buf[1023];
  __syncthreads();
  {
    int run = incl_c - c;
    for (int i = 0; i < E; ++i) {
      if (us[i]) a.ws_cum[ui_s[tid * E + i]] = run;
      run += cl[i];
    }
  }
  if (tid == 0) {
    a.ws_cum[nu] = total;
    a.ws_units[3 * B] = nu;
  }
  __syncthreads();  // every table entry written before the fingerprint that vouches for them
  if (tid == 0) {
    const uint64_t h = fp_s[0];
    a.ws_units[3 * B + 1] = int(uint32_t(h));
    a.ws_units[3 * B + 2] = int(uint32_t(h >> 32));
  }
  // 5. check the shared-prefix entries of every non-first session
  const int incl_v = block_scan<false>(v, buf);
  const int nv = buf[1023];
  {
    int run = incl_v - v;
    for (int i = 0; i < E; ++i) {
      const int b = tid * E + i;
      if (b < B) voff_s[b] = run;
      run += vl[i];
    }
    if (tid == 0) voff_s[B] = nv;
  }
  __syncthreads();
  // 8 entries per thread and pass, all loads issued before any compare
  constexpr int V = 8;
  bool mismatch = false;
  for (int base = tid; base < nv; base += 1024 * V) {
    int x[V], y[V];
#pragma unroll
    for (int u = 0; u < V; ++u) {
      const int idx = base + u * 1024;
      x[u] = y[u] = 0;
      if (idx < nv) {
        int lo = 0, hi = B;  // largest b with voff_s[b] <= idx
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (voff_s[mid] <= idx) lo = mid;
          else hi = mid;
        }
        const int p = idx - voff_s[lo];
        const int f = first_s[ui_s[lo]];
        x[u] = a.bt[int64_t(lo) * a.bt_stride + p];
        y[u] = a.bt[int64_t(f) * a.bt_stride + p];
      }
    }
#pragma unroll
    for (int u = 0; u < V; ++u) mismatch |= x[u] != y[u];
  }
  if (mismatch) flag_error(a.dev_status, KVS_DEV_BAD_PAGE_BIT);
}

template <int D, int NB, int MODE, bool APPEND = false>
hipError_t launch_decode_mode(const DecodeArgs& a, hipStream_t stream) {
  constexpr int S = D == 128 ? KVS_RING_PAGES_D128 : 8;  // 32 KiB of ring per wave
  hipLaunchKernelGGL((decode_stream_kernel<D, NB, S, MODE, APPEND>), dim3(a.plan.blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// Cascade: the plan kernel forms the units, then 4 wave pairs per CU (two waves
// per SIMD) stream and merge them.
template <int D>
hipError_t launch_decode_cascade(const DecodeArgs& a, hipStream_t stream) {
  constexpr int S = D == 128 ? 4 : 8;  // 32 KiB of ring per pair
  const int G = a.num_q_heads / a.pool.num_kv_heads;
  hipLaunchKernelGGL(decode_cascade_plan_kernel, dim3(1), dim3(1024), 0, stream, a,
                     a.plan.rows / (a.num_decoders * G));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_pair_kernel<D, S>), dim3(4 * a.plan.blocks), dim3(128), 0, stream, a);
  return hipGetLastError();
}

template <int D, int NB>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  if (a.pbt) return launch_decode_mode<D, NB, kPrivate>(a, stream);
  if (a.k_new) return launch_decode_mode<D, NB, kPlain, true>(a, stream);
  return launch_decode_mode<D, NB, kPlain>(a, stream);
}

__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < words; i += int64_t(gridDim.x) * 256) p[i] = 0u;
}

}  // namespace

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const int64_t words = int64_t(bytes / 4);
  if (words == 0) return hipSuccess;
  const int64_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(zero_kernel, dim3(unsigned(blocks < 1024 ? blocks : 1024)), dim3(256), 0, stream,
                     static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int D = a.pool.head_dim, nb = a.plan.nb;
  if (a.group_id) return D == 128 ? launch_decode_cascade<128>(a, stream) : launch_decode_cascade<64>(a, stream);
  if (D == 128) {
    if (nb == 1) return launch_decode_t<128, 1>(a, stream);
    if (nb == 2) return launch_decode_t<128, 2>(a, stream);
    return launch_decode_t<128, 4>(a, stream);
  }
  if (nb == 1) return launch_decode_t<64, 1>(a, stream);
  if (nb == 2) return launch_decode_t<64, 2>(a, stream);
  return launch_decode_t<64, 4>(a, stream);
}

}  // namespace kvs
