// kv_pool_append on gfx950: copy new K/V rows into their page slots, bit for bit.
//
// The cache store of the base prefill (PrefillShare, section 3.3: the KV lives
// in fixed-size blocks; ICaRus, overall framework: E_base writes the KV all
// decoders read).  One workgroup per (window of up to 16 new tokens that share a
// page, KV head, session).  K rows are moved as 16-byte runs; the V part of a
// tile is stored with 8 slots of one head-dim value side by side, so a thread
// gathers those 8 slots and writes them as one 16-byte run when all 8 are new,
// and slot by slot otherwise (slots not being appended are never touched).
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
  const int pid = a.bt[int64_t(b) * a.bt_stride + lp];
  if (pid < 0 || pid >= a.pool.num_pages) {
    if (threadIdx.x == 0) flag_error(a.dev_status, 1);
    return;
  }
  uint16_t* tile = a.pool.data + tile_offset(a.layer + l, pid, h, a.pool.num_pages, Hkv, D);
  const int64_t row_stride = int64_t(Hkv) * D;
  // new row of logical position t is c0 + (t - P)
  const uint16_t* ksrc = a.k_new + l * a.kv_lstride + int64_t(h) * D;
  const uint16_t* vsrc = a.v_new + l * a.kv_lstride + int64_t(h) * D;

  // K: one thread per (slot, 8-value run)
  for (int e = threadIdx.x; e < kPage * (D / 8); e += 256) {
    const int slot = e / (D / 8), run = e % (D / 8);
    const int t = lp * kPage + slot;
    if (t < t0 || t >= t1) continue;
    const int d0 = run * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ksrc + int64_t(c0 + t - P) * row_stride + d0);
    *reinterpret_cast<u32x4*>(tile + ((d0 / 32) * 64 + ((d0 % 32) / 8) * 16 + slot) * 8) = v;
  }
  // V: one thread per (run of 8 slots, head-dim value)
  uint16_t* vt = tile + kPage * D;
  for (int e = threadIdx.x; e < 2 * D; e += 256) {
    const int run = e / D, d = e % D;
    const int base = lp * kPage + 8 * run;
    uint16_t* dst = vt + ((d / 16) * 32 + run * 16 + d % 16) * 8;
    if (base >= t0 && base + 7 < t1) {
      uint32_t w[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t lo = vsrc[int64_t(c0 + base + 2 * c - P) * row_stride + d];
        const uint32_t hi = vsrc[int64_t(c0 + base + 2 * c + 1 - P) * row_stride + d];
        w[c] = lo | (hi << 16);
      }
      *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int t = base + c;
        if (t >= t0 && t < t1) dst[c] = vsrc[int64_t(c0 + t - P) * row_stride + d];
      }
    }
  }
}

template <int D>
hipError_t launch_append_t(const AppendArgs& a, hipStream_t stream) {
  // a window of new tokens starting mid-page can touch one page more
  const int windows = (a.max_new + kPage - 1) / kPage + 1;
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

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  if (a.pool.head_dim == 128) return launch_append_t<128>(a, stream);
  return launch_append_t<64>(a, stream);
}

}  // namespace kvs
