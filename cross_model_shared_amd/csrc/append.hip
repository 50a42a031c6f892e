// kv_pool_append on gfx950: copy new K/V rows into their page slots, bit for bit.
//
// The cache store of the base prefill (PrefillShare, section 3.3: the KV lives
// in fixed-size blocks; ICaRus, overall framework: E_base writes the KV all
// decoders read).  One workgroup per (window of up to 16 new tokens that share a
// page, KV head, session).  K rows are moved as 16-byte runs; the V part of a
// tile is stored with 8 slots of one head-dim value side by side, so the V rows
// are read as 16-byte row pieces into LDS, and a thread gathers its 8 slots of
// one head-dim value from there and writes them as one 16-byte run when all 8
// are new, slot by slot otherwise (slots not being appended are never touched).
// (Gathering the 8 slots straight from the rows with 2-byte loads made a
// 4-layer group's call 1.6% slower.)
#include <algorithm>

#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {

namespace {

template <int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a, int z0) {
  const int w = blockIdx.x;
  const int h = blockIdx.y;
  const int z = z0 + int(blockIdx.z);
  const int b = z % a.batch, l = z / a.batch;  // session, layer of the range
  const int Hkv = a.pool.num_kv_heads;
  const int P = a.seq_lens[b];
  const int c0 = a.cu_new[b], c1 = a.cu_new[b + 1];
  const int n = c1 - c0;
  if (P < 0 || n < 0 || n > a.max_new || P + n > a.max_seq_len || c0 < 0 || c1 > a.total_new) {
    if (threadIdx.x == 0 && w == 0 && h == 0) flag_error(a.dev_status, 2);
    return;
  }
  if (n == 0) return;
  const int lp = P / kPage + w;  // logical page written by this workgroup
  const int t0 = max(lp * kPage, P), t1 = min(lp * kPage + kPage, P + n);
  if (t0 >= t1) return;
  const int64_t row_stride = int64_t(Hkv) * D;
  // new row of logical position t is c0 + (t - P)
  const uint16_t* ksrc = a.k_new + l * a.kv_lstride + int64_t(h) * D;
  const uint16_t* vsrc = a.v_new + l * a.kv_lstride + int64_t(h) * D;

  // The new rows are read before the page id, which they do not depend on, so
  // the loads overlap.  K and V: one thread per (slot, 8-value run).
  static_assert(kPage * (D / 8) <= 256 && 2 * D <= 256, "one element per thread");
  const int e = threadIdx.x;
  const int kslot = e / (D / 8), krun = e % (D / 8);
  const bool kact = e < kPage * (D / 8) && lp * kPage + kslot >= t0 && lp * kPage + kslot < t1;
  u32x4 kval = {0u, 0u, 0u, 0u}, vval = {0u, 0u, 0u, 0u};
  const int64_t krow = int64_t(c0 + lp * kPage + kslot - P) * row_stride + krun * 8;
  if (kact) {
    kval = *reinterpret_cast<const u32x4*>(ksrc + krow);
    vval = *reinterpret_cast<const u32x4*>(vsrc + krow);
  }
  const int pid = a.bt[int64_t(b) * a.bt_stride + lp];
  // V: the window's rows staged in LDS as 16-byte row pieces (each thread the
  // same slot and piece as for K), then each thread gathers its run of 8 slots
  // of one head-dim value from there
  __shared__ uint16_t vs[kPage][D];
  if (kact) *reinterpret_cast<u32x4*>(&vs[kslot][krun * 8]) = vval;
  __syncthreads();
  const int vrun = e / D, vd = e % D;
  const int base = lp * kPage + 8 * vrun;
  const bool vact = e < 2 * D && base + 7 >= t0 && base < t1;
  const bool vfull = base >= t0 && base + 7 < t1;
  uint32_t vw[4] = {0u, 0u, 0u, 0u};
  if (vact) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int t = base + c;
      if (t >= t0 && t < t1) vw[c / 2] |= uint32_t(vs[8 * vrun + c][vd]) << (16 * (c % 2));
    }
  }

  if (pid < 0 || pid >= a.pool.num_pages) {
    if (threadIdx.x == 0) flag_error(a.dev_status, 1);
    return;
  }
  uint16_t* tile = a.pool.data + tile_offset(a.layer + l, pid, h, a.pool.num_pages, Hkv, D);
  if (kact) {
    const int d0 = krun * 8;
    *reinterpret_cast<u32x4*>(tile + ((d0 / 32) * 64 + ((d0 % 32) / 8) * 16 + kslot) * 8) = kval;
  }
  // the V part of the tile holds 8 slots of one head-dim value side by side:
  // written as one 16-byte run when all 8 are new, slot by slot otherwise
  if (vact) {
    uint16_t* dst = tile + kPage * D + ((vd / 16) * 32 + vrun * 16 + vd % 16) * 8;
    if (vfull) {
      *reinterpret_cast<u32x4*>(dst) = u32x4{vw[0], vw[1], vw[2], vw[3]};
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int t = base + c;
        if (t >= t0 && t < t1) dst[c] = uint16_t(vw[c / 2] >> (16 * (c % 2)));
      }
    }
  }
}

template <int D>
hipError_t launch_append_t(const AppendArgs& a, hipStream_t stream) {
  // n new tokens starting at slot o of a page touch ceil((o + n) / 16) pages,
  // at most (n + 30) / 16 of them
  const int windows = (a.max_new + 2 * kPage - 2) / kPage;
  // (layer, session) pairs on grid z, at most 65535 per launch
  const int64_t zs = int64_t(a.batch) * a.num_layers;
  for (int64_t z0 = 0; z0 < zs; z0 += 65535) {
    const unsigned nz = unsigned(zs - z0 < 65535 ? zs - z0 : 65535);
    hipLaunchKernelGGL((append_kernel<D>), dim3(windows, a.pool.num_kv_heads, nz), dim3(256), 0, stream, a, int(z0));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---- kv_pool_append_check: the append's write-aliasing rule ----------------
//
// One 32-bit word per physical page: bit s is set when a new token of the call
// goes to slot s, bit 16 + s when slot s holds a live token of a session of the
// batch (a position below its seq_lens).  A first kernel marks every live slot;
// a second marks every new token's slot with an atomic OR and reports aliasing
// when the slot's word already had either bit: a second new token, or a live
// token (sessions may share full prefix pages, so live-live is allowed).  The
// kernels are separate launches on one stream, so every live bit is in before
// the first new token looks.  Work is a grid-stride loop over (session, page).

constexpr int kAliasThreads = 256, kAliasMaxBlocks = 4096;

__device__ __forceinline__ uint32_t slot_bits(int lo, int hi) {  // slots lo .. hi-1 of a page
  return ((hi >= 32 ? 0u : (1u << hi)) - 1u) & ~((1u << lo) - 1u);
}

__global__ __launch_bounds__(kAliasThreads) void alias_live_kernel(AliasArgs a, int pages_per_session) {
  const int64_t total = int64_t(a.batch) * pages_per_session;
  for (int64_t i = int64_t(blockIdx.x) * kAliasThreads + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * kAliasThreads) {
    const int b = int(i / pages_per_session), pi = int(i % pages_per_session);
    const int L = a.seq_lens[b];
    if (L < 0 || L > a.max_seq_len || pi * kPage >= L) continue;
    const int pid = a.bt[int64_t(b) * a.bt_stride + pi];
    if (pid < 0 || pid >= a.num_pages) continue;
    atomicOr(a.words + pid, slot_bits(0, min(kPage, L - pi * kPage)) << 16);
  }
}

__global__ __launch_bounds__(kAliasThreads) void alias_new_kernel(AliasArgs a, int windows) {
  const int64_t total = int64_t(a.batch) * windows;
  for (int64_t i = int64_t(blockIdx.x) * kAliasThreads + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * kAliasThreads) {
    const int b = int(i / windows), w = int(i % windows);
    const int P = a.seq_lens[b], c0 = a.cu_new[b], c1 = a.cu_new[b + 1], n = c1 - c0;
    // lengths the append rejects write nothing (the append reports them)
    if (P < 0 || n <= 0 || n > a.max_new || P + n > a.max_seq_len || c0 < 0 || c1 > a.total_new) continue;
    const int lp = P / kPage + w;
    const int t0 = max(lp * kPage, P), t1 = min(lp * kPage + kPage, P + n);
    if (t0 >= t1) continue;
    const int pid = a.bt[int64_t(b) * a.bt_stride + lp];
    if (pid < 0 || pid >= a.num_pages) continue;
    const uint32_t mine = slot_bits(t0 - lp * kPage, t1 - lp * kPage);
    const uint32_t old = atomicOr(a.words + pid, mine);
    if ((old & mine) || ((old >> 16) & mine)) flag_error(a.dev_status, KVS_DEV_ALIAS_BIT);
  }
}

}  // namespace

hipError_t launch_append_check(const AliasArgs& a, hipStream_t stream) {
  hipError_t e = launch_zero(a.words, size_t(a.num_pages) * 4, stream);
  if (e != hipSuccess) return e;
  const int pages = (a.max_seq_len + kPage - 1) / kPage;
  const int windows = (a.max_new + 2 * kPage - 2) / kPage;
  auto blocks = [](int64_t work) {
    return unsigned(std::min<int64_t>(kAliasMaxBlocks, std::max<int64_t>(1, (work + kAliasThreads - 1) / kAliasThreads)));
  };
  hipLaunchKernelGGL(alias_live_kernel, dim3(blocks(int64_t(a.batch) * pages)), dim3(kAliasThreads), 0, stream, a,
                     pages);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(alias_new_kernel, dim3(blocks(int64_t(a.batch) * windows)), dim3(kAliasThreads), 0, stream, a,
                     windows);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.pool.head_dim == 128) return launch_append_t<128>(a, stream);
  return launch_append_t<64>(a, stream);
}

}  // namespace kvs
