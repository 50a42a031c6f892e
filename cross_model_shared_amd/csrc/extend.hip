// partial_prefill_extend on gfx950: the new chunk's rows attend the cached
// prefix in full and the chunk causally (PrefillShare, sections 3.3 and 7:
// partial prefill of the new tokens only; section 4: prefill is compute-bound).
//
// Rows of one (session, KV head) are the chunk's (token i, query head of the
// group) pairs, token-major, so a 16-row block spans few positions and the
// causal diagonal touches few pages.  At D=128 a workgroup of 4 waves holds 128
// rows (32 per wave, Q in registers) and walks the session's keys in blocks of
// 32 (two pages), staged once per workgroup in a 3-stage LDS ring by direct
// global->LDS 16-byte loads one block ahead; three workgroups share a CU, so
// each SIMD runs three waves whose softmax and matrix-core phases interleave.
// Per 32 keys and 16 rows a wave does 8 QK^T and 8 PV steps of 16x16x32 bf16
// (plus one step for the row sums).
//
// Q is pre-multiplied by scale*log2(e) and rounded to bf16 once, so scores leave
// the matrix cores in log2 units; in the steady-state blocks the accumulators
// start at -m (the row's fixed reference), and the softmax is one exp2 per score.
//
// Workgroups are laid out so that all row blocks of one (session, KV head) land
// on the same XCD: hardware hands workgroup ids to the 8 XCDs round robin, and
// keeping a KV head's pages in one L2 lets its row blocks share them there.
#include "kvs_device.h"
#include "kvs_internal.h"

#include <type_traits>

namespace kvs {

namespace {

constexpr int kXcds = 8;
constexpr float kLazy = 8.0f;                // rescaling path: max moves when it grows by > 2^8
constexpr float kSafeSum = 1.0e18f;          // ~2^60: fixed-reference sums stay below this
constexpr int kExtendPairRounds = 4;         // paired grid >= this many full rounds of resident workgroups

template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier WITHOUT the memory fence of __syncthreads(): the fence would
// wait for every outstanding vector-memory op, i.e. drain the blocks being
// prefetched into LDS.  Each wave first waits (vmcnt) for its own share of the
// block it needs; after the barrier the whole block is in LDS.  A ring stage is
// overwritten only kStages - kLook >= 2 blocks after its last reads, whose
// results every wave has already consumed.
__device__ __forceinline__ void block_barrier() { __builtin_amdgcn_s_barrier(); }

template <int PER>
__device__ __forceinline__ void wait_blocks(int blocks_after) {
  switch (blocks_after) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<PER * 1>(); break;
    case 2: wait_vmcnt<PER * 2>(); break;
    default: wait_vmcnt<PER * 3>(); break;
  }
}

template <int D, int NB>
struct ExtendState {
  f32x4 acc[NB][D / 16];
  f32x4 lsum[NB];   // row sums of the bf16 weights: sum_k 1 * P^T[k][row], every element equal
  float m[NB];
};

// Stage layout: the two page tiles of a block as stored in the pool, the second
// one 64 bytes further on, so that lanes reading the same run index of both
// pages hit different LDS banks.
constexpr int kPad = 4;  // u32x4

// S^T for one 32-key block, as two 16-key halves h.  Lane l (row l%16 on the N
// side, group g = l/16 on the M side) reads, for half h, the K run of page
// (l%16)/8 and slot 8((l/4)%2) + 4h + l%4: the M index of a half mixes the two
// pages so that the result holds, in lane group g, block keys 8g + 4h + j (j =
// 0..3), i.e. 8 consecutive keys of one page over both halves.  That is the
// B-operand order of the PV step, whose A operand is then one 16-byte run of V
// (8 consecutive slots of one head-dim value).  koff: the lane's run index for
// half 0 (half 1 reads 4 slots further on).  The accumulators start at init[cb] (0, or -m of the row so that
// the block's scores come out already shifted by the row's reference).
template <int D, int NB>
__device__ __forceinline__ void qk_block(f32x4 (&s)[2][NB], const u32x4 (&qf)[NB][D / 32],
                                         const u32x4* stage, int koff, const float (&init)[NB]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 kf[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) kf[i] = stage[koff + k_run(i, 0, 4 * h)];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      f32x4 acc = {init[cb], init[cb], init[cb], init[cb]};
#pragma unroll
      for (int i = 0; i < D / 32; ++i) acc = mma_16x16x32(kf[i], qf[cb][i], acc);
      s[h][cb] = acc;
    }
  }
}

// q * c rounded to bf16 (8 values): the query rows carry the softmax scale in
// log2 units, so scores come out of the matrix cores ready for exp2.
__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 v, float c) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; w += 2) {
    const float f0 = __uint_as_float(v[w] << 16) * c, f1 = __uint_as_float(v[w] & 0xFFFF0000u) * c;
    const float f2 = __uint_as_float(v[w + 1] << 16) * c, f3 = __uint_as_float(v[w + 1] & 0xFFFF0000u) * c;
    const u32x2 pk = pack_bf16x4(f0, f1, f2, f3);
    r[w] = pk[0];
    r[w + 1] = pk[1];
  }
  return r;
}

// A copy of the lane id that the compiler cannot hoist or keep: values derived
// from it are recomputed where they are used (on the cold, masked paths) rather
// than held in registers across the key walk.
__device__ __forceinline__ int fresh_lane() {
  int ln = threadIdx.x & 63;
  asm volatile("" : "+v"(ln));
  return ln;
}

// Scores of one 32-key block for column block cb: 8 per lane, block keys
// s0..s0+7 (s0 = 8 * lane group), masked to -inf past each row's key limit.
template <int NB, bool MASKED>
__device__ __forceinline__ void block_scores(float (&x)[8], const f32x4 (&s)[2][NB], int cb, int kbase,
                                             int lim) {
  const int s0 = MASKED ? 8 * (fresh_lane() >> 4) : 0;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float v = s[h][cb][j];
      if (MASKED) v = (kbase + s0 + 4 * h + j < lim) ? v : -INFINITY;
      x[4 * h + j] = v;
    }
}

__device__ __forceinline__ u32x4 pack_p8(const float (&p)[8]) {
  const u32x2 lo = pack_bf16x4(p[0], p[1], p[2], p[3]);
  const u32x2 hi = pack_bf16x4(p[4], p[5], p[6], p[7]);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Softmax weights of one 32-key block against a FIXED per-row reference m
// (set from the row's first block): p = 2^(s - m), s in log2 units.  Row sums are taken by the
// PV step (an all-ones A operand), from the same bf16 weights PV uses.  Moving the reference is
// never needed for correctness, only to keep p inside fp32/bf16 range; weights
// may exceed 1, and a row whose sum leaves the safe range (checked once, after
// the loop) is recomputed by the rescaling variant below.  Keeping the
// accumulators free of vector ops lets them stay in accumulation registers.
template <int D, int NB, bool MASKED>
__device__ __forceinline__ void softmax_fixed(ExtendState<D, NB>& st, const f32x4 (&s)[2][NB], u32x4 (&pb)[NB],
                                              int kbase, const int (&lim_abs)[NB]) {
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    float x[8], p[8];
    block_scores<NB, MASKED>(x, s, cb, kbase, lim_abs[cb]);
    const float m = st.m[cb];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = exp2_fast(x[j] - m);
    pb[cb] = pack_p8(p);
  }
}

// Weights of a block whose scores already had the row reference subtracted (the
// accumulators started at -m) and that no row masks: p = 2^s.
template <int NB>
__device__ __forceinline__ void softmax_shifted(const f32x4 (&s)[2][NB], u32x4 (&pb)[NB]) {
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    float p[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) p[4 * h + j] = exp2_fast(s[h][cb][j]);
    pb[cb] = pack_p8(p);
  }
}

// First block of a row: the reference is the block's row maximum.
template <int D, int NB, bool MASKED>
__device__ __forceinline__ void softmax_first(ExtendState<D, NB>& st, const f32x4 (&s)[2][NB], u32x4 (&pb)[NB],
                                              int kbase, const int (&lim_abs)[NB]) {
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    float x[8];
    block_scores<NB, MASKED>(x, s, cb, kbase, lim_abs[cb]);
    const float t = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    const float m = wave_max_across_quads(t);
    st.m[cb] = (m == -INFINITY) ? 0.f : m;
  }
  softmax_fixed<D, NB, MASKED>(st, s, pb, kbase, lim_abs);
}

// Rescaling variant (the recomputation path): the reference follows the running
// maximum, moved only when it grows by more than 2^kLazy, and the accumulators
// are rescaled then.
template <int D, int NB, bool MASKED>
__device__ __forceinline__ void softmax_rescale(ExtendState<D, NB>& st, const f32x4 (&s)[2][NB], u32x4 (&pb)[NB],
                                                int kbase, const int (&lim_abs)[NB]) {
  float alpha[NB];
  bool any_move = false;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    float x[8], p[8];
    block_scores<NB, MASKED>(x, s, cb, kbase, lim_abs[cb]);
    const float t = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    const float tmax = wave_max_across_quads(t);
    const float m_old = st.m[cb];
    const bool move = tmax > m_old + kLazy;
    const float m_new = move ? tmax : m_old;
    any_move |= move;
    alpha[cb] = move ? exp2_fast(m_old - m_new) : 1.f;
    const float neg = (m_new == -INFINITY) ? 0.f : -m_new;
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = exp2_fast(x[j] + neg);
    st.m[cb] = m_new;
    pb[cb] = pack_p8(p);
  }
  if (__builtin_amdgcn_ballot_w64(any_move)) {
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      st.lsum[cb] *= alpha[cb];
#pragma unroll
      for (int i = 0; i < D / 16; ++i) st.acc[cb][i] *= alpha[cb];
    }
  }
}

// NB: 16-row column blocks per wave; WAVES per workgroup; kStages-deep LDS ring
// of 32-key blocks with kLook blocks in flight; BLOCKS_PER_CU workgroups share a CU.
// PIPE: QK^T of block k+1 is issued before the softmax of block k (two score
// buffers); otherwise each block runs QK^T, softmax, PV in turn (fewer registers,
// so more waves per SIMD can hide each other's latency).
template <int D, int NB, int WAVES, int kStages, int kLook, int BLOCKS_PER_CU, bool PIPE>
__global__ __launch_bounds__(64 * WAVES, BLOCKS_PER_CU) void extend_kernel(ExtendArgs a, int row_blocks, int pairs) {
  static_assert(kStages >= kLook + 2, "a stage is rewritten only after every wave has left it");
  constexpr int THREADS = 64 * WAVES;
  constexpr int kRowsPerWave = 16 * NB;
  constexpr int kRowsPerBlock = WAVES * kRowsPerWave;
  constexpr int TILE = D * 4;                 // u32x4 per page tile (K then V)
  static_assert(TILE % THREADS == 0, "a page tile must split evenly over the workgroup");
  constexpr int PER_PAGE = TILE / THREADS;    // DMA instructions per thread per page
  constexpr int PER_BLOCK = 2 * PER_PAGE;
  __shared__ u32x4 ring[kStages][2 * TILE + kPad];

  const int Hkv = a.pool.num_kv_heads;
  const int units = a.num_layers * a.batch * Hkv;  // (layer, session, KV head), KV head fastest
  // Workgroup slots per unit: one per row block, heaviest (longest key walk)
  // first; or, with pairs, one per pair of row blocks rb and row_blocks-1-rb,
  // run one after the other.  In a causal chunk the key walk grows by one block
  // per row block, so every pair walks the same number of key blocks and the
  // workgroups get equal work.
  const int slots = pairs ? (row_blocks + 1) / 2 : row_blocks;
  const int xcd = blockIdx.x % kXcds;
  const int kk = blockIdx.x / kXcds;
  const int unit = (kk / slots) * kXcds + xcd;
  const int slot = kk % slots;
  if (unit >= units) return;
  const int l = unit / (a.batch * Hkv), b = (unit / Hkv) % a.batch, g = unit % Hkv;
  const int layer = a.layer + l;
  const uint16_t* const qbase = a.q + l * a.q_lstride;
  uint16_t* const obase = a.out + l * a.q_lstride;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.num_q_heads / Hkv;

  const int P = load_uniform(a.seq_lens + b);
  const int c0 = load_uniform(a.cu_new + b), c1 = load_uniform(a.cu_new + b + 1);
  const int C = c1 - c0;
  if (P < 0 || C < 0 || C > a.max_new || P + C > a.max_seq_len || c0 < 0 || c1 > a.total_new) {
    if (threadIdx.x == 0 && slot == 0) flag_error(a.dev_status, KVS_DEV_BAD_LEN_BIT);
    return;
  }
  const int rows = C * G;
  auto row_block = [&](const int rb) {
  const int rbase = rb * kRowsPerBlock;
  if (rbase >= rows) return;  // whole workgroup: uniform
  const int total = P + C;
  const int npages = (total + kPage - 1) / kPage;
  const int wg_last_tok = (min(rbase + kRowsPerBlock, rows) - 1) / G;
  const int nblk = (P + wg_last_tok + 1 + 31) / 32;   // 32-key blocks this workgroup needs

  // ---- this wave's rows ----
  const int r0 = rbase + wave * kRowsPerWave;
  u32x4 qf[NB][D / 32];
  int lim_abs[NB];
  bool rvalid[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int r = r0 + cb * 16 + (lane & 15);
    rvalid[cb] = r < rows;
    const int i = rvalid[cb] ? r / G : C - 1;
    lim_abs[cb] = P + i + 1;
    const uint16_t* qrow = qbase + (int64_t(c0 + i) * a.num_q_heads + g * G + (rvalid[cb] ? r % G : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[cb][s] = rvalid[cb] ? scale_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * (lane >> 4)),
                                            a.scale_log2)
                             : u32x4{0u, 0u, 0u, 0u};
  }
  const bool wave_has_rows = r0 < rows;
  const int wave_lo = wave_has_rows ? P + r0 / G + 1 : 0;  // smallest key limit among the wave's rows

  const int32_t* btrow = a.bt + int64_t(b) * a.bt_stride;
  const int num_pages = a.pool.num_pages;
  const int tid = threadIdx.x;
  // tile of page pid = lg_base + pid * page_stride (u32x4 units)
  const u32x4* lg_base = reinterpret_cast<const u32x4*>(a.pool.data + tile_offset(layer, 0, g, num_pages, Hkv, D));
  const uint32_t page_stride = uint32_t(Hkv) * (32 * D / 8);
  auto issue_at = [&](int k, int stage) {
    // both page ids of the block first, so their loads share one wait; with no
    // second page the first is loaded again (never used unmasked)
    int pid[2] = {load_uniform(btrow + 2 * k), load_uniform(btrow + (2 * k + 1 < npages ? 2 * k + 1 : 2 * k))};
    if ((uint32_t(pid[0]) >= uint32_t(num_pages)) | (uint32_t(pid[1]) >= uint32_t(num_pages))) {
      flag_error(a.dev_status, KVS_DEV_BAD_PAGE_BIT);
      __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
      for (int h = 0; h < 2; ++h)  // in-range stand-in; the session's output is unspecified
        if (uint32_t(pid[h]) >= uint32_t(num_pages)) pid[h] = 0;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4* tile = lg_base + uint64_t(uint32_t(pid[h])) * page_stride;
      u32x4* dst = &ring[stage][h * (TILE + kPad)];
#pragma unroll
      for (int j = 0; j < PER_PAGE; ++j)
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(tile + j * THREADS + tid),
                                         (__attribute__((address_space(3))) void*)(dst + j * THREADS + wave * 64),
                                         16, 0, 0);
    }
  };
  auto issue = [&](int k) { issue_at(k, k % kStages); };

  ExtendState<D, NB> st;
  const float zero[NB] = {};
  const int koff = ((lane >> 3) & 1) * (TILE + kPad) + k_run(0, lane >> 4, 8 * ((lane >> 2) & 1) + (lane & 3));
  // V run of page (lane/32), slots 8((lane/16)%2) .. +7, head dim 16s + lane%16
  const int voff = (lane >> 5) * (TILE + kPad) + v_run(D, 0, (lane >> 4) & 1, lane & 15);

  // PV of block k from stage stg: one V run per 16 head dims as the A operand,
  // the bf16 weights pb as the B operand (32 keys per step).  The first VPRE
  // runs come from vpre, read before the softmax.
  constexpr int kVPre = 4;  // V runs read ahead of the softmax in the fast blocks
  auto v_operand = [&](const u32x4* stg, int i) { return stg[voff + v_run(D, i, 0, 0) - v_run(D, 0, 0, 0)]; };
  auto pv_block = [&](const u32x4* stg, const u32x4 (&pb)[NB], int nv0, int nv1, bool vmask, auto vpre_tag,
                      const u32x4 (&vpre)[kVPre]) {
    constexpr int VPRE = decltype(vpre_tag)::value;
    constexpr uint32_t kOnes = 0x3F803F80u;  // two bf16 1.0
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
      st.lsum[cb] = mma_16x16x32(u32x4{kOnes, kOnes, kOnes, kOnes}, pb[cb], st.lsum[cb]);
    const int nv = (lane >> 5) ? nv1 : nv0;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      u32x4 va = i < VPRE ? vpre[i < VPRE ? i : 0] : v_operand(stg, i);
      if (vmask) va = mask_v_run(va, 8 * ((fresh_lane() >> 4) & 1), nv);
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) st.acc[cb][i] = mma_16x16x32(va, pb[cb], st.acc[cb][i]);
    }
  };
  using NoPre = std::integral_constant<int, 0>;
  const u32x4 no_vpre[kVPre] = {};

  // Blocks below fast_end are seen in full by every row of the workgroup and are
  // followed by at least kLook more blocks: their steps have no masks and no
  // data-dependent branches, so the matrix-core steps of QK^T(k+1) and PV(k)
  // can be scheduled around the softmax of block k.
  const int wg_lo = P + rbase / G + 1;                 // smallest key limit in the workgroup
  const int fast_end = max(1, min(wg_lo / 32, nblk - kLook));

  // The whole key walk.  FAST: fixed reference per row; otherwise rescaling.
  auto run = [&](auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      st.m[cb] = -INFINITY;
      st.lsum[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < D / 16; ++i) st.acc[cb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // general step (any block): QK^T of block k+1 into nxt, softmax + PV of block k from cur
    auto step = [&](int k, f32x4 (&cur)[2][NB], f32x4 (&nxt)[2][NB]) {
      if (k + kLook < nblk) issue(k + kLook);
      if (k + 1 < nblk) {
        wait_blocks<PER_BLOCK>(min(nblk - 1, k + kLook) - (k + 1));
        block_barrier();
        qk_block<D, NB>(nxt, qf, ring[(k + 1) % kStages], koff, zero);
      }
      const int kbase = k * 32;
      const bool masked = kbase + 32 > wave_lo;  // some row of the wave stops inside this block
      u32x4 pb[NB];
      if (!FAST) {
        if (masked) softmax_rescale<D, NB, true>(st, cur, pb, kbase, lim_abs);
        else softmax_rescale<D, NB, false>(st, cur, pb, kbase, lim_abs);
      } else if (k == 0) {
        if (masked) softmax_first<D, NB, true>(st, cur, pb, kbase, lim_abs);
        else softmax_first<D, NB, false>(st, cur, pb, kbase, lim_abs);
      } else {
        if (masked) softmax_fixed<D, NB, true>(st, cur, pb, kbase, lim_abs);
        else softmax_fixed<D, NB, false>(st, cur, pb, kbase, lim_abs);
      }
      const int nv0 = total - kbase, nv1 = total - kbase - 16;
      pv_block(ring[k % kStages], pb, nv0, nv1, nv1 < kPage, NoPre{}, no_vpre);
    };
    // fast step: no masks, constant waits, unconditional prefetch
    auto fast_step = [&](int k, f32x4 (&cur)[2][NB], f32x4 (&nxt)[2][NB]) {
      issue(k + kLook);
      wait_vmcnt<PER_BLOCK * (kLook - 1)>();
      block_barrier();
      qk_block<D, NB>(nxt, qf, ring[(k + 1) % kStages], koff, zero);
      u32x4 pb[NB];
      softmax_fixed<D, NB, false>(st, cur, pb, k * 32, lim_abs);
      pv_block(ring[k % kStages], pb, kPage, kPage, false, NoPre{}, no_vpre);
    };
#pragma unroll 1
    for (int k = 0; k < kLook && k < nblk; ++k) issue(k);
    if constexpr (!PIPE) {
      // one block at a time: prefetch k+kLook, wait for k, QK^T, softmax, PV
      // stg: stage of block k; nxt: stage of block k + kLook (kept as counters)
      auto seq_step = [&](int k, bool fast, int stg_i, int nxt) {
        const u32x4* stg = ring[stg_i];
        f32x4 sc[2][NB];
        if (fast) {
          issue_at(k + kLook, nxt);
          wait_vmcnt<PER_BLOCK * kLook>();
        } else {
          if (k + kLook < nblk) issue_at(k + kLook, nxt);
          wait_blocks<PER_BLOCK>(min(nblk - 1, k + kLook) - k);
        }
        block_barrier();
        // matrix-core phases run at raised wave priority, so a SIMD's other waves
        // fill the gaps with their softmax work rather than delaying these steps
        __builtin_amdgcn_s_setprio(2);
        if (fast) {
          float negm[NB];
#pragma unroll
          for (int cb = 0; cb < NB; ++cb) negm[cb] = -st.m[cb];
          qk_block<D, NB>(sc, qf, stg, koff, negm);
        } else {
          qk_block<D, NB>(sc, qf, stg, koff, zero);
        }
        __builtin_amdgcn_s_setprio(0);
        const int kbase = k * 32;
        u32x4 pb[NB];
        if (fast) {
          // the first V runs are read now, so their LDS latency passes during the softmax
          u32x4 vpre[kVPre];
#pragma unroll
          for (int i = 0; i < kVPre; ++i) vpre[i] = v_operand(stg, i);
          __builtin_amdgcn_sched_barrier(0);
          softmax_shifted<NB>(sc, pb);
          __builtin_amdgcn_s_setprio(2);
          pv_block(stg, pb, kPage, kPage, false, std::integral_constant<int, kVPre>{}, vpre);
          __builtin_amdgcn_s_setprio(0);
          return;
        }
        const bool masked = kbase + 32 > wave_lo;
        if (!FAST) {
          if (masked) softmax_rescale<D, NB, true>(st, sc, pb, kbase, lim_abs);
          else softmax_rescale<D, NB, false>(st, sc, pb, kbase, lim_abs);
        } else if (k == 0) {
          if (masked) softmax_first<D, NB, true>(st, sc, pb, kbase, lim_abs);
          else softmax_first<D, NB, false>(st, sc, pb, kbase, lim_abs);
        } else {
          if (masked) softmax_fixed<D, NB, true>(st, sc, pb, kbase, lim_abs);
          else softmax_fixed<D, NB, false>(st, sc, pb, kbase, lim_abs);
        }
        const int nv0 = total - kbase, nv1 = total - kbase - 16;
        __builtin_amdgcn_s_setprio(2);
        pv_block(stg, pb, nv0, nv1, nv1 < kPage, NoPre{}, no_vpre);
        __builtin_amdgcn_s_setprio(0);
      };
      auto bump = [](int x) { return x + 1 == kStages ? 0 : x + 1; };
      seq_step(0, false, 0, kLook % kStages);
      int k = 1, s_cur = 1 % kStages, s_nxt = (1 + kLook) % kStages;
      if (FAST) {
        // up to a block whose stage is 0, then kStages blocks per iteration with constant stages
#pragma unroll 1
        for (; k < fast_end && s_cur != 0; ++k) {
          seq_step(k, true, s_cur, s_nxt);
          s_cur = bump(s_cur);
          s_nxt = bump(s_nxt);
        }
#pragma unroll 1
        for (; k + kStages <= fast_end; k += kStages) {
#pragma unroll
          for (int j = 0; j < kStages; ++j) seq_step(k + j, true, j, (j + kLook) % kStages);
        }
#pragma unroll 1
        for (; k < fast_end; ++k) {
          seq_step(k, true, s_cur, s_nxt);
          s_cur = bump(s_cur);
          s_nxt = bump(s_nxt);
        }
      }
#pragma unroll 1
      for (; k < nblk; ++k) {
        seq_step(k, false, s_cur, s_nxt);
        s_cur = bump(s_cur);
        s_nxt = bump(s_nxt);
      }
      return;
    }
    wait_blocks<PER_BLOCK>(min(kLook, nblk) - 1);
    block_barrier();
    f32x4 sa[2][NB], sb[2][NB];
    qk_block<D, NB>(sa, qf, ring[0], koff, zero);
    step(0, sa, sb);                        // sets each row's reference (FAST) or starts rescaling
    int k = 1;
    if (FAST) {
      // blocks 1 .. fast_end-1, two per iteration so the score buffers swap roles
#pragma unroll 1
      for (; k + 1 < fast_end; k += 2) {
        fast_step(k, sb, sa);
        fast_step(k + 1, sa, sb);
      }
      if (k < fast_end) {
        fast_step(k, sb, sa);
        ++k;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int cb = 0; cb < NB; ++cb) sb[h][cb] = sa[h][cb];
      }
    }
    // remaining blocks: the causal diagonal, the sequence end
#pragma unroll 1
    for (; k < nblk; ++k) {
      step(k, sb, sa);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) sb[h][cb] = sa[h][cb];
    }
  };

  run(std::integral_constant<bool, true>{});
  // a fixed-reference sum out of range (or not finite) sends the workgroup down the rescaling path
  // the ring is idle from here on: its first word holds the workgroup's redo flag
  int& redo = *reinterpret_cast<int*>(&ring[0][0]);
  __syncthreads();
  if (threadIdx.x == 0) redo = 0;
  __syncthreads();
  bool bad = false;
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) bad |= !(st.lsum[cb][0] < kSafeSum);
  if (__builtin_amdgcn_ballot_w64(bad) && lane == 0) redo = 1;
  __syncthreads();
  const bool do_redo = redo;
  __syncthreads();  // every wave has read the flag before a rescaling pass reloads the ring over it
  if (do_redo) run(std::integral_constant<bool, false>{});

  // the output rows are recomputed here from a fresh copy of the lane id, so that
  // no row address stays live (in registers or spilled) across the key walk
  int ln = lane, Gq = G;
  asm volatile("" : "+v"(ln), "+s"(Gq));
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const float l = st.lsum[cb][0];
    const int r = r0 + cb * 16 + (ln & 15);
    if (r >= rows) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* o = obase + (int64_t(c0 + r / Gq) * a.num_q_heads + g * Gq + r % Gq) * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const f32x4 v = st.acc[cb][i] * inv;
      *reinterpret_cast<u32x2*>(o + 16 * i + 4 * (ln >> 4)) = pack_bf16x4(v[0], v[1], v[2], v[3]);
    }
  }
  };  // row_block

  row_block(row_blocks - 1 - slot);
  if (pairs && slot != row_blocks - 1 - slot) {
    // every wave has consumed its last ring reads (their results fed the output
    // rows) before the next row block loads into the ring
    block_barrier();
    row_block(slot);
  }
}

template <int D, int NB, int WAVES, int STAGES, int LOOK, int PER_CU, bool PIPE>
hipError_t launch_extend_t(const ExtendArgs& a, hipStream_t stream) {
  constexpr int kRowsPerBlock = WAVES * 16 * NB;
  const int G = a.num_q_heads / a.pool.num_kv_heads;
  const int row_blocks = (a.max_new * G + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t units = int64_t(a.num_layers) * a.batch * a.pool.num_kv_heads;
  const int64_t unit_rounds = (units + kXcds - 1) / kXcds;
  // Pair row blocks when the halved grid still holds several rounds of
  // workgroups for the chip: short walks then share a workgroup with long ones.
  const int64_t resident = int64_t(device_cu_count()) * PER_CU;
  const int pairs = row_blocks >= 2 && unit_rounds * kXcds * ((row_blocks + 1) / 2) >= kExtendPairRounds * resident;
  const int64_t blocks = unit_rounds * (pairs ? (row_blocks + 1) / 2 : row_blocks) * kXcds;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((extend_kernel<D, NB, WAVES, STAGES, LOOK, PER_CU, PIPE>), dim3(unsigned(blocks)), dim3(64 * WAVES), 0,
                     stream, a, row_blocks, pairs);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream) {
  // D=128: three 4-wave workgroups per CU (three waves per SIMD), one block at a
  // time; D=64: 4 waves x 64 rows, the next block's QK^T ahead of this block's
  // softmax (a 4 KiB page tile is one 256-thread load)
  if (a.pool.head_dim == 128) return launch_extend_t<128, 2, 4, 3, 1, 3, false>(a, stream);
  return launch_extend_t<64, 4, 4, 6, 4, 1, true>(a, stream);
}

}  // namespace kvs
