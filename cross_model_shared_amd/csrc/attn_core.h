// The per-page attention step of the decode kernels.
//
// One wave owns NB column blocks of 16 query rows.  For a 16-token page of one
// KV head it forms S^T = K Q^T on the matrix cores (tokens on the M side, query
// rows on the N side), updates the online softmax of every row, and adds
// P V into O^T.  The QK^T result layout (lane l holds tokens 4*(l/16)+j of row
// l%16) is exactly the B-operand layout of the 16x16x16 PV step, so the
// probabilities go from one matrix-core step to the next without a shuffle.
//
// The running maximum is only moved when a page's maximum exceeds it by more
// than 2^kLazyLog2 (in the log2 domain): probabilities then stay below 2^8 in
// fp32, and the accumulators are rescaled only on the rare pages that move it.
// Any reference point gives the same softmax, as long as acc and l share it.
#pragma once

#include "kvs_device.h"

namespace kvs {

constexpr float kLazyLog2 = 8.0f;

template <int D, int NB>
struct RowState {
  f32x4 acc[NB][D / 16];  // O^T: acc[cb][dblk][j] = O[row 16cb + lane%16][16 dblk + 4(lane/16) + j]
  float m[NB];            // reference max of scaled scores (log2 domain), per row
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

// Process one page.  kf: the lane's K operands of the page (head dims 32i +
// 8(lane/16) .. +7 of slot lane%16); vf: its V operands (slots 4(lane/16) .. +3 of
// head dim 16s + lane%16).
// lim[cb]: exclusive key limit of this lane's row in column block cb, as a slot
// count relative to the page start (<= 0: row sees nothing here; >= 16: all).
// nvalid: slots of the page holding data (later slots are never read).
// masked: false when every row sees all 16 slots (the common case).
template <int D, int NB>
__device__ __forceinline__ void attend_page(RowState<D, NB>& st, const QFrag<D, NB>& qf,
                                            const u32x4 (&kf)[D / 32], u32x2 (&vf)[D / 16],
                                            float scale_log2, bool masked, const int (&lim)[NB],
                                            int nvalid, int lane) {
  const int s0 = 4 * (lane >> 4);
  if (nvalid < kPage) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) vf[i] = mask_v_quad(vf[i], s0, nvalid);
  }
  f32x4 s[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    s[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D / 32; ++i) s[cb] = mma_16x16x32(kf[i], qf.q[cb][i], s[cb]);
  }
  float alpha[NB];
  bool any_move = false;
  u32x2 pb[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = s[cb][j] * scale_log2;
      if (masked) x[j] = (s0 + j < lim[cb]) ? x[j] : -INFINITY;
    }
    float tmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    tmax = wave_max_across_quads(tmax);
    const float m_old = st.m[cb];
    // move the reference only when the page max exceeds it by more than 2^kLazyLog2
    const bool move = tmax > m_old + kLazyLog2;   // also true for the first seen key
    const float m_new = move ? tmax : m_old;
    any_move |= move;
    alpha[cb] = move ? exp2_fast(m_old - m_new) : 1.f;  // exp2(-inf) = 0 on the first move
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = exp2_fast(x[j] - m_use);
    st.l[cb] = st.l[cb] * alpha[cb] + ((p[0] + p[1]) + (p[2] + p[3]));
    st.m[cb] = m_new;
    pb[cb] = pack_bf16x4(p[0], p[1], p[2], p[3]);
  }
  if (__builtin_amdgcn_ballot_w64(any_move)) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int i = 0; i < D / 16; ++i) st.acc[cb][i] *= alpha[cb];
  }
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) st.acc[cb][i] = mma_16x16x16(vf[i], pb[cb], st.acc[cb][i]);
  }
}

}  // namespace kvs
