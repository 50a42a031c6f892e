// Page handoff and fetch on gfx950.
//
// kv_pages_pack / kv_pages_unpack move whole pages between a pool and a
// contiguous transfer buffer (PrefillShare, section 3.3: the prefill worker
// hands the KV it wrote, kept in fixed-size blocks, to the decode worker).  The
// (layer, page) chunk of a pool is all KV heads' tiles side by side (H_kv * 8 KiB
// at D=128), so one workgroup copies one chunk with 16-byte loads and stores;
// the buffer holds chunks in [layer][listed page] order.
//
// kv_pool_fetch reads the logical K/V rows of sessions back out of the pool into
// dense [row][H_kv][D] arrays (DroidSpeak, section 5.4: fetch returns what store
// wrote; here, the inverse of kv_pool_append), for hand-off to a consumer with
// another layout.  One workgroup per (page, KV head, session): K runs are whole
// row pieces already; V runs (8 slots of one head-dim value) are transposed
// through LDS so that rows leave as 16-byte pieces.
#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {

namespace {

#ifndef KVS_PACK_PIECE_KIB
#define KVS_PACK_PIECE_KIB 16
#endif
// One workgroup copies one PIECE-KiB part of a (layer, page) chunk: every thread
// loads all its 16-byte pieces of the part before storing any.  Both sides are
// streamed with nontemporal loads and stores: nothing copied is read again soon
// (pack: 5.4 -> 5.9 TB/s read + write, unpack 5.4 -> 5.5, calls alternating).
template <bool UNPACK>
__global__ __launch_bounds__(256) void pack_kernel(HandoffArgs a, int parts) {
  constexpr int kPer = KVS_PACK_PIECE_KIB * 1024 / 16 / 256;  // 16-byte pieces per thread
  const int i = blockIdx.x / parts;  // entry of the page list
  const int part = blockIdx.x % parts;
  const int li = blockIdx.y;       // layer within the range
  const int Hkv = a.pool.num_kv_heads, D = a.pool.head_dim;
  const int pid = a.page_ids[i];
  if (pid < 0 || pid >= a.pool.num_pages) {
    if (threadIdx.x == 0 && li == 0 && part == 0) flag_error(a.dev_status, KVS_DEV_BAD_PAGE_BIT);
    return;
  }
  const int64_t chunk = int64_t(Hkv) * 32 * D;   // elements: every head's tile of one page
  uint16_t* pool_chunk = a.pool.data + tile_offset(a.layer_begin + li, pid, 0, a.pool.num_pages, Hkv, D);
  uint16_t* buf_chunk = a.buf + (int64_t(li) * a.num_ids + i) * chunk;
  const int n = int(chunk / 8);    // 16-byte pieces of the chunk
  const int p0 = part * kPer * 256, p1 = min(n, p0 + kPer * 256);
  const u32x4* src = reinterpret_cast<const u32x4*>(UNPACK ? buf_chunk : pool_chunk);
  u32x4* dst = reinterpret_cast<u32x4*>(UNPACK ? pool_chunk : buf_chunk);
  u32x4 v[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (p0 + j * 256 < p1) v[j] = __builtin_nontemporal_load(src + p0 + j * 256 + threadIdx.x);
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    if (p0 + j * 256 < p1) __builtin_nontemporal_store(v[j], dst + p0 + j * 256 + threadIdx.x);
}

template <int D>
__global__ __launch_bounds__(256) void fetch_kernel(FetchArgs a) {
  const int w = blockIdx.x;        // logical page of the session
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int Hkv = a.pool.num_kv_heads;
  const int L = a.seq_lens[b];
  const int r0 = a.cu_rows[b], r1 = a.cu_rows[b + 1];
  if (L < 0 || L > a.max_seq_len || r1 - r0 != L || r0 < 0 || r1 > a.total_rows) {
    if (threadIdx.x == 0 && w == 0 && h == 0) flag_error(a.dev_status, KVS_DEV_BAD_LEN_BIT);
    return;
  }
  const int t0 = w * kPage, nv = min(kPage, L - t0);
  if (nv <= 0) return;
  const int pid = a.bt[int64_t(b) * a.bt_stride + w];
  if (pid < 0 || pid >= a.pool.num_pages) {
    if (threadIdx.x == 0) flag_error(a.dev_status, KVS_DEV_BAD_PAGE_BIT);
    return;
  }
  const u32x4* tile = reinterpret_cast<const u32x4*>(
      a.pool.data + tile_offset(a.layer, pid, h, a.pool.num_pages, Hkv, D));
  const int64_t row_stride = int64_t(Hkv) * D;   // elements between consecutive rows
  // K: run (i, kg, t) is 8 head dims 32i+8kg.. of slot t
  for (int e = threadIdx.x; e < 2 * D; e += 256) {
    const int t = e % kPage, kg = (e / kPage) % 4, i = e / (4 * kPage);
    if (t >= nv) continue;
    *reinterpret_cast<u32x4*>(a.k_out + (r0 + t0 + t) * row_stride + int64_t(h) * D + 32 * i + 8 * kg) =
        tile[k_run(i, kg, t)];
  }
  // V: run (s, o, m) is slots 8o..8o+7 of head dim 16s+m; transpose via LDS to [slot][dim]
  __shared__ __attribute__((aligned(16))) uint16_t vt[kPage][D];
  for (int e = threadIdx.x; e < 2 * D; e += 256) {
    const int m = e % 16, o = (e / 16) % 2, s = e / 32;
    const u32x4 r = tile[v_run(D, s, o, m)];
#pragma unroll
    for (int c = 0; c < 8; ++c) vt[8 * o + c][16 * s + m] = uint16_t(r[c / 2] >> (16 * (c % 2)));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 2 * D; e += 256) {
    const int t = e / (D / 8), piece = e % (D / 8);
    if (t >= nv) continue;
    *reinterpret_cast<u32x4*>(a.v_out + (r0 + t0 + t) * row_stride + int64_t(h) * D + 8 * piece) =
        *reinterpret_cast<const u32x4*>(&vt[t][8 * piece]);
  }
}

}  // namespace

hipError_t launch_pack(const HandoffArgs& a, bool unpack, hipStream_t stream) {
  if (a.num_ids == 0) return hipSuccess;
  const int64_t chunk_bytes = int64_t(a.pool.num_kv_heads) * 32 * a.pool.head_dim * 2;
  const int parts = int((chunk_bytes + KVS_PACK_PIECE_KIB * 1024 - 1) / (KVS_PACK_PIECE_KIB * 1024));
  if (int64_t(a.num_ids) * parts > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  dim3 grid(a.num_ids * parts, a.num_layers);
  if (unpack) hipLaunchKernelGGL(pack_kernel<true>, grid, dim3(256), 0, stream, a, parts);
  else hipLaunchKernelGGL(pack_kernel<false>, grid, dim3(256), 0, stream, a, parts);
  return hipGetLastError();
}

hipError_t launch_fetch(const FetchArgs& a, hipStream_t stream) {
  dim3 grid((a.max_seq_len + kPage - 1) / kPage, a.pool.num_kv_heads, a.batch);
  if (grid.x == 0) return hipSuccess;
  if (a.pool.head_dim == 128) hipLaunchKernelGGL(fetch_kernel<128>, grid, dim3(256), 0, stream, a);
  else hipLaunchKernelGGL(fetch_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvs
