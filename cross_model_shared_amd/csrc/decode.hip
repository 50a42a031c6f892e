// shared_kv_decode on gfx950: N decoders x G query heads per KV head, one KV read.
//
// ICaRus (Key design 3) runs the queries of every party that reads the same KV
// side by side along the head dimension so the KV is read once.  Here all
// R = N*G query rows of a KV head sit in the N side of the matrix-core steps of
// one wave, so each (page, head) tile is streamed from HBM exactly once per call
// whatever N is.  Work split:
//   grid (split, KV head x row group, session), 4 waves per workgroup;
//   a workgroup takes split_pages consecutive logical pages of one session,
//   wave w takes pages w, w+4, ... of them with its own online softmax;
//   the 4 waves' partial softmax states are merged through LDS, then either the
//   output is written (one split) or the partial (m, l, acc) goes to the
//   workspace and decode_combine_kernel merges the splits.
#include "attn_core.h"
#include "kvs_internal.h"

namespace kvs {

namespace {

constexpr int kWaves = 4;

template <int D, int NB>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int RG = 16 * NB;
  const DecodePlan& pl = a.plan;
  const int split = blockIdx.x;
  const int Hkv = a.pool.num_kv_heads;
  const int g = blockIdx.y % Hkv;
  const int rg = blockIdx.y / Hkv;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int G = a.num_q_heads / Hkv;

  int L = a.seq_lens[b];
  if (L < 0 || L > a.max_seq_len) {
    if (threadIdx.x == 0 && split == 0 && blockIdx.y == 0) flag_error(a.dev_status, 2);
    L = L < 0 ? 0 : a.max_seq_len;
  }
  const int npages = (L + kPage - 1) / kPage;
  const int p_begin = split * pl.split_pages;
  const int row0 = rg * RG;

  if (L == 0) {  // softmax over nothing: zero output, written by split 0
    if (split != 0) return;
    for (int e = threadIdx.x; e < RG * (D / 8); e += 256) {
      const int r = row0 + e / (D / 8);
      if (r >= pl.rows) continue;
      const int n = r / G, h = g * G + r % G;
      uint16_t* o = a.out + ((int64_t(b) * a.num_decoders + n) * a.num_q_heads + h) * D;
      reinterpret_cast<u32x4*>(o)[e % (D / 8)] = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  if (p_begin >= npages) return;
  const int p_end = min(npages, p_begin + pl.split_pages);
  const int nsplits = (npages + pl.split_pages - 1) / pl.split_pages;

  // query operands of this row group (zero rows past R)
  QFrag<D, NB> qf;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int r = row0 + cb * 16 + (lane & 15);
    const bool valid = r < pl.rows;
    const int n = valid ? r / G : 0, h = valid ? g * G + r % G : 0;
    const uint16_t* qrow = a.q + ((int64_t(b) * a.num_decoders + n) * a.num_q_heads + h) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
      qf.q[cb][i] = valid ? *reinterpret_cast<const u32x4*>(qrow + 32 * i + 8 * (lane >> 4))
                          : u32x4{0u, 0u, 0u, 0u};
  }

  RowState<D, NB> st;
  st.init();
  const int32_t* btrow = a.bt + int64_t(b) * a.bt_stride;
  const int num_pages = a.pool.num_pages;

  u32x4 kf[D / 32], vf[D / 32], kn[D / 32], vn[D / 32];
  int p = p_begin + wave;
  int pid = p < p_end ? btrow[p] : -1;
  bool ok = pid >= 0 && pid < num_pages;
  if (p < p_end && !ok) flag_error(a.dev_status, 1);
  if (ok) {
    const uint16_t* tile = a.pool.data + tile_offset(a.layer, pid, g, num_pages, Hkv, D);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      kf[i] = load_k_slab(tile, i, lane);
      vf[i] = load_v_slab(tile, D, i, lane);
    }
  }
  while (p < p_end) {
    // issue the next page's loads before computing this one
    const int pn = p + kWaves;
    const int pidn = pn < p_end ? btrow[pn] : -1;
    const bool okn = pidn >= 0 && pidn < num_pages;
    if (pn < p_end && !okn) flag_error(a.dev_status, 1);
    if (okn) {
      const uint16_t* tile = a.pool.data + tile_offset(a.layer, pidn, g, num_pages, Hkv, D);
#pragma unroll
      for (int i = 0; i < D / 32; ++i) {
        kn[i] = load_k_slab(tile, i, lane);
        vn[i] = load_v_slab(tile, D, i, lane);
      }
    }
    if (ok) {
      const int nvalid = min(kPage, L - p * kPage);
      int lim[NB];
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) lim[cb] = nvalid;
      attend_page<D, NB>(st, qf, kf, vf, a.scale_log2, nvalid < kPage, lim, nvalid, lane);
    }
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      kf[i] = kn[i];
      vf[i] = vn[i];
    }
    ok = okn;
    p = pn;
  }

  // ---- merge the 4 waves' states (fixed order, so results are reproducible) ----
  __shared__ float sm_m[kWaves][RG];
  __shared__ float sm_l[kWaves][RG];
  __shared__ f32x4 sm_acc[NB][D / 16][kWave];
  float lrow[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) lrow[cb] = wave_sum_across_quads(st.l[cb]);
  if (lane < 16) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      sm_m[wave][cb * 16 + lane] = st.m[cb];
      sm_l[wave][cb * 16 + lane] = lrow[cb];
    }
  }
  __syncthreads();
  float mtot[NB], ltot[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int r = cb * 16 + (lane & 15);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][r]);
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][r];
      lt += (mw == -INFINITY) ? 0.f : sm_l[w][r] * exp2f(mw - M);
    }
    mtot[cb] = M;
    ltot[cb] = lt;
    const float f = (st.m[cb] == -INFINITY) ? 0.f : exp2f(st.m[cb] - M);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) st.acc[cb][i] *= f;
  }
#pragma unroll
  for (int w = 0; w < kWaves - 1; ++w) {
    if (wave == w) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int i = 0; i < D / 16; ++i)
          sm_acc[cb][i][lane] = (w == 0) ? st.acc[cb][i] : sm_acc[cb][i][lane] + st.acc[cb][i];
    }
    __syncthreads();
  }
  if (wave != kWaves - 1) return;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb)
#pragma unroll
    for (int i = 0; i < D / 16; ++i) st.acc[cb][i] += sm_acc[cb][i][lane];

  if (nsplits == 1) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int r = row0 + cb * 16 + (lane & 15);
      if (r >= pl.rows) continue;
      const int n = r / G, h = g * G + r % G;
      uint16_t* o = a.out + ((int64_t(b) * a.num_decoders + n) * a.num_q_heads + h) * D;
      const float inv = ltot[cb] > 0.f ? 1.f / ltot[cb] : 0.f;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        const f32x4 v = st.acc[cb][i] * inv;
        *reinterpret_cast<u32x2*>(o + 16 * i + 4 * (lane >> 4)) = pack_bf16x4(v[0], v[1], v[2], v[3]);
      }
    }
    return;
  }
  const int64_t unit = (int64_t(b) * Hkv + g) * pl.rowgroups + rg;
  const int64_t slot = unit * pl.max_splits + split;
  float* wacc = a.ws_acc + slot * RG * D;
  float* wml = a.ws_ml + slot * RG * 2;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int r = cb * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      *reinterpret_cast<f32x4*>(wacc + r * D + 16 * i + 4 * (lane >> 4)) = st.acc[cb][i];
    if (lane < 16) {
      wml[r * 2 + 0] = mtot[cb];
      wml[r * 2 + 1] = ltot[cb];
    }
  }
}

// Merge the split partials (m_s, l_s, acc_s) of one (session, KV head, row group):
// m* = max m_s, out = sum_s 2^(m_s - m*) acc_s / sum_s 2^(m_s - m*) l_s.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
  const DecodePlan& pl = a.plan;
  const int Hkv = a.pool.num_kv_heads;
  const int g = blockIdx.x % Hkv;
  const int rg = blockIdx.x / Hkv;
  const int b = blockIdx.y;
  const int G = a.num_q_heads / Hkv;
  int L = a.seq_lens[b];
  L = L < 0 ? 0 : (L > a.max_seq_len ? a.max_seq_len : L);
  const int npages = (L + kPage - 1) / kPage;
  const int nsplits = (npages + pl.split_pages - 1) / pl.split_pages;
  if (nsplits <= 1) return;
  const int RG = pl.rg_rows;
  const int64_t unit = (int64_t(b) * Hkv + g) * pl.rowgroups + rg;
  const float* ml = a.ws_ml + unit * pl.max_splits * RG * 2;
  const float* acc = a.ws_acc + unit * pl.max_splits * RG * D;
  for (int e = threadIdx.x; e < RG * (D / 4); e += 256) {
    const int rl = e / (D / 4), d4 = e % (D / 4);
    const int r = rg * RG + rl;
    if (r >= pl.rows) continue;
    float M = -INFINITY;
    for (int s = 0; s < nsplits; ++s) M = fmaxf(M, ml[(s * RG + rl) * 2]);
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int s = 0; s < nsplits; ++s) {
      const float ms = ml[(s * RG + rl) * 2];
      const float w = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      den += w * ml[(s * RG + rl) * 2 + 1];
      num += w * reinterpret_cast<const f32x4*>(acc + (int64_t(s) * RG + rl) * D)[d4];
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const int n = r / G, h = g * G + r % G;
    uint16_t* o = a.out + ((int64_t(b) * a.num_decoders + n) * a.num_q_heads + h) * D;
    reinterpret_cast<u32x2*>(o)[d4] = pack_bf16x4(num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
  }
}

template <int D, int NB>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const DecodePlan& pl = a.plan;
  dim3 grid(pl.max_splits, a.pool.num_kv_heads * pl.rowgroups, a.batch);
  hipLaunchKernelGGL((decode_split_kernel<D, NB>), grid, dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.max_splits <= 1) return e;
  dim3 cgrid(a.pool.num_kv_heads * pl.rowgroups, a.batch);
  hipLaunchKernelGGL((decode_combine_kernel<D>), cgrid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int D = a.pool.head_dim, nb = a.plan.nb;
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
