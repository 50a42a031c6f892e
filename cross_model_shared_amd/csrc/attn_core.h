// The per-page attention step shared by decode and extend.
//
// One wave owns NB column blocks of 16 query rows.  For a 16-token page of one
// KV head it forms S^T = K Q^T on the matrix cores (tokens on the M side, query
// rows on the N side), updates the online softmax of every row, and adds
// P V into O^T.  The QK^T result layout (lane l holds tokens 4*(l/16)+j of row
// l%16) is exactly the B-operand layout of the 16x16x16 PV step, so the
// probabilities go from one matrix-core step to the next without a shuffle.
#pragma once

#include "kvs_device.h"

namespace kvs {

template <int D, int NB>
struct RowState {
  f32x4 acc[NB][D / 16];  // O^T: acc[cb][dblk][j] = O[row 16cb + lane%16][16 dblk + 4(lane/16) + j]
  float m[NB];            // running max of scaled scores (log2 domain), per row
  float l[NB];            // running sum of exp2(s - m) over this lane's slots
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      m[cb] = -INFINITY;
      l[cb] = 0.f;
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc[cb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
};

// Query operand of column block cb, head-dim slab i (B side of S^T = K Q^T):
// lane l holds row 16cb + l%16, head dims 32i + 8(l/16) .. +7.
template <int D, int NB>
struct QFrag {
  u32x4 q[NB][D / 32];
};

// Process one page.  kf/vf: the lane's K and V slab operands of the page.
// lim[cb]: exclusive key limit of this lane's row in column block cb, as a slot
// count relative to the page start (<= 0: row sees nothing here; >= 16: all).
// nvalid: slots of the page holding data (later slots are never read).
// masked: false when every row sees all 16 slots (the common case).
template <int D, int NB>
__device__ __forceinline__ void attend_page(RowState<D, NB>& st, const QFrag<D, NB>& qf,
                                            const u32x4 (&kf)[D / 32], u32x4 (&vf)[D / 32],
                                            float scale_log2, bool masked, const int (&lim)[NB],
                                            int nvalid, int lane) {
  if (nvalid < kPage) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) vf[i] = mask_v_slab(vf[i], lane, nvalid);
  }
  const int s0 = 4 * (lane >> 4);
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 32; ++i) s = mma_16x16x32(kf[i], qf.q[cb][i], s);
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = s[j] * scale_log2;
      if (masked) x[j] = (s0 + j < lim[cb]) ? x[j] : -INFINITY;
    }
    float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tmax = wave_max_across_quads(tmax);
    const float m_new = fmaxf(st.m[cb], tmax);
    // m_new is -inf only when the row has seen no key yet and none here: keep zeros
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = exp2f(st.m[cb] - m_use);
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = exp2f(x[j] - m_use);
    st.l[cb] = st.l[cb] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    st.m[cb] = m_new;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) st.acc[cb][i] *= alpha;
    const u32x2 pb = pack_bf16x4(p[0], p[1], p[2], p[3]);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      st.acc[cb][2 * i] = mma_16x16x16(u32x2{vf[i][0], vf[i][1]}, pb, st.acc[cb][2 * i]);
      st.acc[cb][2 * i + 1] = mma_16x16x16(u32x2{vf[i][2], vf[i][3]}, pb, st.acc[cb][2 * i + 1]);
    }
  }
}

}  // namespace kvs
