// partial_prefill_extend on gfx950: the new chunk's rows attend the cached
// prefix in full and the chunk causally (PrefillShare, sections 3.3 and 7:
// partial prefill of the new tokens only; section 4: prefill is compute-bound).
//
// Rows of one (session, KV head) are the chunk's (token i, query head of the
// group) pairs, token-major, so a 16-row block spans only a few positions and
// the causal diagonal touches few pages.  A workgroup holds 128 rows (4 waves x
// 32 rows) and walks the session's pages in order; every step is the shared
// matrix-core page step.  Workgroups are laid out so that all row blocks of one
// (session, KV head) land on the same XCD: hardware hands workgroup ids to the 8
// XCDs round robin, and keeping a KV head's pages in one L2 lets its 16+ row
// blocks reuse them there.
#include "attn_core.h"
#include "kvs_internal.h"

namespace kvs {

namespace {

constexpr int kXcds = 8;
constexpr int kRowsPerWave = 32;
constexpr int kRowsPerBlock = 4 * kRowsPerWave;

template <int D>
__global__ __launch_bounds__(256) void extend_kernel(ExtendArgs a, int row_blocks) {
  constexpr int NB = 2;
  const int Hkv = a.pool.num_kv_heads;
  const int units = a.batch * Hkv;
  const int xcd = blockIdx.x % kXcds;
  const int k = blockIdx.x / kXcds;
  const int unit = (k / row_blocks) * kXcds + xcd;
  const int rb = k % row_blocks;
  if (unit >= units) return;
  const int b = unit / Hkv, g = unit % Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = a.num_q_heads / Hkv;

  int P = a.seq_lens[b];
  const int c0 = a.cu_new[b], c1 = a.cu_new[b + 1];
  int C = c1 - c0;
  if (P < 0 || C < 0 || C > a.max_new || P + C > a.max_seq_len || c0 < 0 || c1 > a.total_new) {
    if (threadIdx.x == 0 && rb == 0 && g == 0) flag_error(a.dev_status, 2);
    return;
  }
  const int rows = C * G;
  const int rbase = rb * kRowsPerBlock;
  if (rbase >= rows) return;
  const int total = P + C;
  const int r0 = rbase + wave * kRowsPerWave;
  if (r0 >= rows) return;  // no barriers below: a wave may leave early

  QFrag<D, NB> qf;
  int lim_abs[NB];
  int tok[NB], head[NB];
  bool rvalid[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int r = r0 + cb * 16 + (lane & 15);
    rvalid[cb] = r < rows;
    const int i = rvalid[cb] ? r / G : C - 1;
    tok[cb] = i;
    head[cb] = g * G + (rvalid[cb] ? r % G : 0);
    lim_abs[cb] = P + i + 1;
    const uint16_t* qrow = a.q + (int64_t(c0 + i) * a.num_q_heads + head[cb]) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf.q[cb][s] = rvalid[cb] ? *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * (lane >> 4))
                               : u32x4{0u, 0u, 0u, 0u};
  }
  // wave-uniform bounds of the key limits of this wave's rows
  const int last_row = min(r0 + kRowsPerWave, rows) - 1;
  const int lim_lo = P + r0 / G + 1;
  const int lim_hi = P + last_row / G + 1;
  const int npages = (lim_hi + kPage - 1) / kPage;

  RowState<D, NB> st;
  st.init();
  const int32_t* btrow = a.bt + int64_t(b) * a.bt_stride;
  const int num_pages = a.pool.num_pages;
  u32x4 kf[D / 32], vf[D / 32], kn[D / 32], vn[D / 32];

  int pid = btrow[0];
  bool ok = pid >= 0 && pid < num_pages;
  if (!ok) flag_error(a.dev_status, 1);
  if (ok) {
    const uint16_t* tile = a.pool.data + tile_offset(a.layer, pid, g, num_pages, Hkv, D);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      kf[s] = load_k_slab(tile, s, lane);
      vf[s] = load_v_slab(tile, D, s, lane);
    }
  }
  for (int p = 0; p < npages; ++p) {
    const int pn = p + 1;
    const int pidn = pn < npages ? btrow[pn] : -1;
    const bool okn = pidn >= 0 && pidn < num_pages;
    if (pn < npages && !okn) flag_error(a.dev_status, 1);
    if (okn) {
      const uint16_t* tile = a.pool.data + tile_offset(a.layer, pidn, g, num_pages, Hkv, D);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        kn[s] = load_k_slab(tile, s, lane);
        vn[s] = load_v_slab(tile, D, s, lane);
      }
    }
    if (ok) {
      const int pstart = p * kPage;
      const int nvalid = min(kPage, total - pstart);
      int lim[NB];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) lim[cb] = lim_abs[cb] - pstart;
      attend_page<D, NB>(st, qf, kf, vf, a.scale_log2, pstart + kPage > lim_lo, lim, nvalid, lane);
    }
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      kf[s] = kn[s];
      vf[s] = vn[s];
    }
    ok = okn;
  }

#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const float l = wave_sum_across_quads(st.l[cb]);
    if (!rvalid[cb]) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* o = a.out + (int64_t(c0 + tok[cb]) * a.num_q_heads + head[cb]) * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const f32x4 v = st.acc[cb][i] * inv;
      *reinterpret_cast<u32x2*>(o + 16 * i + 4 * (lane >> 4)) = pack_bf16x4(v[0], v[1], v[2], v[3]);
    }
  }
}

template <int D>
hipError_t launch_extend_t(const ExtendArgs& a, hipStream_t stream) {
  const int G = a.num_q_heads / a.pool.num_kv_heads;
  const int row_blocks = (a.max_new * G + kRowsPerBlock - 1) / kRowsPerBlock;
  const int units = a.batch * a.pool.num_kv_heads;
  const int unit_rounds = (units + kXcds - 1) / kXcds;
  const int64_t blocks = int64_t(unit_rounds) * row_blocks * kXcds;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((extend_kernel<D>), dim3(unsigned(blocks)), dim3(256), 0, stream, a, row_blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream) {
  if (a.pool.head_dim == 128) return launch_extend_t<128>(a, stream);
  return launch_extend_t<64>(a, stream);
}

}  // namespace kvs
