// Host-side launch arguments and launchers shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvs {

struct PoolView {
  uint16_t* data;
  int num_layers, num_pages, num_kv_heads, head_dim;
};

struct AppendArgs {
  PoolView pool;
  int layer;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* cu_new;
  const int32_t* bt;
  int bt_stride;
  const int32_t* seq_lens;
  int batch, total_new, max_new, max_seq_len;
  int32_t* dev_status;
  // a range of layers [layer, layer + num_layers): layer l's rows start
  // l * kv_lstride elements into k_new / v_new
  int num_layers = 1;
  int64_t kv_lstride = 0;
};

// Largest batch a decode call accepts (the per-session page prefix sum lives in LDS).
constexpr int kDecodeMaxBatch = 4096;

// How a decode call is cut into work: query rows per KV head are taken in row
// groups of 16*nb (one wave holds them all); the (page, KV head, row group)
// tiles of all sessions are shared out among the 4*blocks waves of a
// persistent grid (evenly, up to a fixed weight per XCD).  Each wave has two
// partial-state slots in the workspace, and every unit split between waves
// has arrival counters there (zero between calls), in the fixed
// kDecodeCounterBytes at the start of every workspace.
struct DecodePlan {
  int rows;       // N * G query rows per KV head
  int nb;         // 16-row column blocks per wave (1, 2 or 4)
  int rg_rows;    // 16 * nb
  int rowgroups;  // ceil(rows / rg_rows)
  int blocks;     // 4-wave workgroups of the persistent grid: a multiple of 8, 8 .. kDecodeBlocks
  int share_even; // stream-K weight of a share on an even XCD (odd XCDs: 512 - share_even)
  int share_mult; // floor(2^26 / (4 * blocks)): scales the share weights to a whole of 2^18
  size_t cum_offset, units_offset, ml_offset, acc_offset, bytes;
};

// Persistent decode grid: one 4-wave workgroup per CU, at most 256 (an
// MI355X), so at most 1024 = 2^10 stream-K shares (waves, or wave pairs in the
// cascade).  The workspace is sized for the maximum, whatever the device.
constexpr int kDecodeBlocks = 256;
constexpr int kDecodeShareLog2 = 10;
static_assert(kDecodeBlocks * 4 == 1 << kDecodeShareLog2, "share count");
// Arrival counters of the split units' merge trees: per tree level (4), two
// per share and row group of a wave pair (a unit a share begins, one it
// continues): 4 * 2^12 int32 = 64 KiB.
constexpr size_t kDecodeCounterBytes = size_t(4) * (size_t(4) << kDecodeShareLog2) * 4;

// Decode workspace layout: arrival counters, then the cascade unit prefix sum
// [batch+1] and unit tables [3*batch+3] (first session, count and prefix per
// unit; the unit count; a 64-bit fingerprint of the inputs the tables were
// built from), then the partial-state slots (2 per
// wave, sized for 64-row groups): (m, l) per row, then a D-vector per row.
constexpr size_t decode_align(size_t x) { return (x + 255) / 256 * 256; }
constexpr size_t kDecodeSlots = size_t(kDecodeBlocks) * 4 * 2, kDecodeSlotRows = 64;
constexpr size_t decode_cum_offset() { return kDecodeCounterBytes; }
constexpr size_t decode_units_offset(int batch) { return decode_cum_offset() + decode_align(size_t(batch + 1) * 4); }
constexpr size_t decode_ml_offset(int batch) { return decode_units_offset(batch) + decode_align(size_t(3 * batch + 3) * 4); }
constexpr size_t decode_acc_offset(int batch) {
  return decode_ml_offset(batch) + decode_align(kDecodeSlots * kDecodeSlotRows * 2 * 4);
}
constexpr size_t decode_workspace_size(int batch, int head_dim) {
  return decode_acc_offset(batch) + kDecodeSlots * kDecodeSlotRows * size_t(head_dim) * 4;
}
// The largest workspace any decode call needs (batch <= kDecodeMaxBatch, head_dim <= 128).
constexpr size_t kDecodeWorkspaceMaxBytes = decode_workspace_size(kDecodeMaxBatch, 128);

// Compute units of the current device (read once per device, then cached;
// 256, MI355X's count, if the query fails).
int device_cu_count();

// Record a printf-style message for kvs_last_error() and return `status`.
int set_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

DecodePlan plan_decode(int batch, int num_decoders, int num_q_heads, int num_kv_heads, int head_dim,
                       int max_seq_len);

struct DecodeArgs {
  PoolView pool;
  int layer;
  const uint16_t* q;
  uint16_t* out;
  const int32_t* bt;
  int bt_stride;
  const int32_t* seq_lens;
  int batch, num_decoders, num_q_heads, max_seq_len;
  float scale_log2;
  // decoder-private suffixes (all null / 0 for a shared-only call): row b*N + n
  // of pbt lists the pages of decoder n's own tokens in session b, plens[b*N + n]
  // their count
  const int32_t* pbt;
  int pbt_stride;
  const int32_t* plens;
  int max_priv_len;
  // cascade (all null for the other calls): sessions with equal non-negative
  // group_id adjacent in the batch share their first group_prefix[b] pages
  const int32_t* group_id;
  const int32_t* group_prefix;
  // fused append (null for the other calls): the step's token of session b,
  // K/V head g at k_new / v_new + (b * H_kv + g) * D, is written at position
  // seq_lens[b] - 1 before it is attended
  const uint16_t* k_new;
  const uint16_t* v_new;
  int* ws_cnt;    // arrival counters of split units' merge trees; zero on entry and on exit
  int* ws_units;  // [3*batch+3] cascade units: first session, count, prefix pages; unit count; fingerprint
  int* ws_cum;    // [batch+1] cascade unit tile prefix sum, written by the plan kernel
  float* ws_ml;   // [4*blocks*2][rg_rows][2] partial (m, l)
  float* ws_acc;  // [4*blocks*2][rg_rows][D] partial acc
  DecodePlan plan;
  int32_t* dev_status;
};

struct ExtendArgs {
  PoolView pool;
  int layer;
  const uint16_t* q;
  uint16_t* out;
  const int32_t* cu_new;
  const int32_t* bt;
  int bt_stride;
  const int32_t* seq_lens;
  int batch, num_q_heads, total_new, max_new, max_seq_len;
  float scale_log2;
  int32_t* dev_status;
  // a range of layers [layer, layer + num_layers): layer l's q and out rows
  // start l * q_lstride elements in
  int num_layers = 1;
  int64_t q_lstride = 0;
};

// Page handoff: a contiguous transfer buffer [num_layers][num_ids][H_kv][tile].
struct HandoffArgs {
  PoolView pool;
  int layer_begin, num_layers;
  const int32_t* page_ids;
  int num_ids;
  uint16_t* buf;   // pack writes it, unpack reads it
  int32_t* dev_status;
};

// Logical rows out of the pool (the inverse of append).
struct FetchArgs {
  PoolView pool;
  int layer;
  const int32_t* bt;
  int bt_stride;
  const int32_t* seq_lens;
  const int32_t* cu_rows;
  int batch, total_rows, max_seq_len;
  uint16_t* k_out;
  uint16_t* v_out;
  int32_t* dev_status;
};

// kv_pool_append_check: the append's destinations, and one scratch word per page
struct AliasArgs {
  const int32_t* cu_new;
  const int32_t* bt;
  int bt_stride;
  const int32_t* seq_lens;
  int batch, total_new, max_new, max_seq_len, num_pages;
  uint32_t* words;
  int32_t* dev_status;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_append_check(const AliasArgs& a, hipStream_t stream);
hipError_t launch_pack(const HandoffArgs& a, bool unpack, hipStream_t stream);
hipError_t launch_fetch(const FetchArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Zero `bytes` bytes (a multiple of 4) at `p` with a fill kernel (no memset node
// in a captured graph).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t launch_extend(const ExtendArgs& a, hipStream_t stream);

}  // namespace kvs
