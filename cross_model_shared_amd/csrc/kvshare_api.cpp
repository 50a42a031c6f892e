// C ABI of libkvshare: argument checks, launch planning, status reporting.
// Every check runs before anything is enqueued; the library never allocates,
// frees or synchronizes.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>

#include "../../include/kvshare.h"
#include "kvs_internal.h"

namespace {

thread_local std::string g_last_error;

int vfail(int status, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  g_last_error = buf;
  return status;
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(status, fmt, ap);
  va_end(ap);
  return status;
}

int check_pool(const kvs_pool* pool, int32_t layer) {
  if (!pool) return fail(KVS_EINVAL, "pool is NULL");
  if (!pool->data) return fail(KVS_EINVAL, "pool->data is NULL");
  if (pool->page_size != 16)
    return fail(KVS_EUNSUPPORTED, "page_size %d unsupported (must be 16)", pool->page_size);
  if (pool->head_dim != 64 && pool->head_dim != 128)
    return fail(KVS_EUNSUPPORTED, "head_dim %d unsupported (64 or 128)", pool->head_dim);
  if (pool->num_layers <= 0 || pool->num_pages <= 0 || pool->num_kv_heads <= 0)
    return fail(KVS_EINVAL, "pool sizes must be positive (layers %d, pages %d, kv heads %d)",
                pool->num_layers, pool->num_pages, pool->num_kv_heads);
  if (layer < 0 || layer >= pool->num_layers)
    return fail(KVS_ERANGE, "layer %d outside [0, %d)", layer, pool->num_layers);
  return KVS_OK;
}

int check_table(int32_t batch, int32_t bt_stride, int32_t max_seq_len) {
  if (batch <= 0) return fail(KVS_EINVAL, "batch %d must be positive", batch);
  if (bt_stride <= 0) return fail(KVS_EINVAL, "bt_stride %d must be positive", bt_stride);
  if (max_seq_len < 0) return fail(KVS_EINVAL, "max_seq_len %d is negative", max_seq_len);
  if (int64_t(max_seq_len) > int64_t(bt_stride) * 16)
    return fail(KVS_ERANGE, "max_seq_len %d exceeds block-table capacity %lld (bt_stride %d * 16)",
                max_seq_len, (long long)bt_stride * 16, bt_stride);
  return KVS_OK;
}

kvs::PoolView view(const kvs_pool* p) {
  return kvs::PoolView{static_cast<uint16_t*>(p->data), p->num_layers, p->num_pages, p->num_kv_heads,
                       p->head_dim};
}

// A softmax scale must be a positive, finite float.  Tested on the bit pattern,
// so the check holds whatever floating-point assumptions the compiler makes.
bool valid_scale(float scale) {
  uint32_t bits;
  memcpy(&bits, &scale, sizeof bits);
  return (bits >> 31) == 0 && ((bits >> 23) & 0xFFu) != 0xFFu && (bits & 0x7FFFFFFFu) != 0;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(KVS_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return KVS_OK;
}


}  // namespace

namespace kvs {

int device_cu_count() {
  constexpr int kDevices = 64, kFallback = 256;
  static std::atomic<int> cached[kDevices];  // 0: not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return kFallback;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = kFallback;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(status, fmt, ap);
  va_end(ap);
  return status;
}

DecodePlan plan_decode(int batch, int num_decoders, int num_q_heads, int num_kv_heads, int head_dim,
                       int max_seq_len) {
  (void)max_seq_len;
  DecodePlan p{};
  p.rows = num_decoders * (num_q_heads / num_kv_heads);
  p.nb = p.rows <= 16 ? 1 : (p.rows <= 32 ? 2 : 4);
  p.rg_rows = 16 * p.nb;
  p.rowgroups = (p.rows + p.rg_rows - 1) / p.rg_rows;
  // One workgroup per CU, in whole rounds of 8 so that every XCD holds the same
  // number of workgroups.  On a 256-CU part the shares on even XCDs weigh 276 and
  // those on odd XCDs 236 (the odd XCDs stream KV pages slower there); any other
  // grid gets equal weights.  KVS_DECODE_WORKGROUPS and KVS_DECODE_SHARE_EVEN,
  // read at every call, override both (clamped to their ranges): they let the
  // tests run the general share arithmetic on any device.
  const int cus = device_cu_count();
  p.blocks = std::min(kDecodeBlocks, std::max(8, cus / 8 * 8));
  if (const char* e = std::getenv("KVS_DECODE_WORKGROUPS"))
    p.blocks = std::min(kDecodeBlocks, std::max(8, std::atoi(e) / 8 * 8));
  p.share_even = (p.blocks == 256 && cus == 256) ? 276 : 256;
  if (const char* e = std::getenv("KVS_DECODE_SHARE_EVEN"))
    p.share_even = std::min(511, std::max(1, std::atoi(e)));
  p.share_mult = (1 << 26) / (4 * p.blocks);
  // arrival counters first, at a fixed size, so that every call on a workspace
  // finds them in the same place; then the cascade tables and the partial-state
  // slots, sized for 64-row groups, so one workspace serves every decode call
  // with these bounds (a cascade unit may hold up to 64 rows)
  p.cum_offset = decode_cum_offset();
  p.units_offset = decode_units_offset(batch);
  p.ml_offset = decode_ml_offset(batch);
  p.acc_offset = decode_acc_offset(batch);
  p.bytes = decode_workspace_size(batch, head_dim);
  return p;
}

}  // namespace kvs

extern "C" {

const char* kvs_last_error(void) { return g_last_error.c_str(); }

const char* kvs_version(void) { return "kvshare 0.1 gfx950"; }

size_t kvs_pool_bytes(int32_t num_layers, int32_t num_pages, int32_t num_kv_heads, int32_t head_dim,
                      int32_t page_size) {
  if (num_layers <= 0 || num_pages <= 0 || num_kv_heads <= 0 || head_dim <= 0 || page_size <= 0)
    return 0;
  return size_t(num_layers) * num_pages * num_kv_heads * 2 * size_t(page_size) * head_dim * 2;
}

int kv_pool_append(const kvs_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                   const int32_t* cu_new, const int32_t* block_table, int32_t bt_stride,
                   const int32_t* seq_lens, int32_t batch, int32_t total_new, int32_t max_new,
                   int32_t max_seq_len, int32_t* dev_status, hipStream_t stream) {
  int s = check_pool(pool, layer);
  if (s) return s;
  if (!k_new || !v_new || !cu_new || !block_table || !seq_lens)
    return fail(KVS_EINVAL, "kv_pool_append: a required pointer is NULL");
  if ((s = check_table(batch, bt_stride, max_seq_len))) return s;
  if (max_new <= 0 || total_new < 0)
    return fail(KVS_EINVAL, "kv_pool_append: max_new %d must be >= 1, total_new %d >= 0", max_new,
                total_new);
  if (max_new > max_seq_len)
    return fail(KVS_ERANGE, "kv_pool_append: max_new %d exceeds max_seq_len %d", max_new, max_seq_len);
  kvs::AppendArgs a{view(pool), layer, static_cast<const uint16_t*>(k_new),
                    static_cast<const uint16_t*>(v_new), cu_new, block_table, bt_stride, seq_lens,
                    batch, total_new, max_new, max_seq_len, dev_status};
  return launched(kvs::launch_append(a, stream), "kv_pool_append");
}

size_t kv_pool_append_check_bytes(int32_t num_pages) { return num_pages > 0 ? size_t(num_pages) * 4 : 0; }

int kv_pool_append_check(const kvs_pool* pool, const int32_t* cu_new, const int32_t* block_table,
                         int32_t bt_stride, const int32_t* seq_lens, int32_t batch, int32_t total_new,
                         int32_t max_new, int32_t max_seq_len, void* scratch, size_t scratch_bytes,
                         int32_t* dev_status, hipStream_t stream) {
  int s = check_pool(pool, 0);
  if (s) return s;
  if (!cu_new || !block_table || !seq_lens || !dev_status)
    return fail(KVS_EINVAL, "kv_pool_append_check: a required pointer is NULL");
  if ((s = check_table(batch, bt_stride, max_seq_len))) return s;
  if (max_new <= 0 || total_new < 0)
    return fail(KVS_EINVAL, "kv_pool_append_check: max_new %d must be >= 1, total_new %d >= 0", max_new,
                total_new);
  if (max_new > max_seq_len)
    return fail(KVS_ERANGE, "kv_pool_append_check: max_new %d exceeds max_seq_len %d", max_new, max_seq_len);
  const size_t need = kv_pool_append_check_bytes(pool->num_pages);
  if (!scratch || scratch_bytes < need)
    return fail(KVS_EWORKSPACE, "kv_pool_append_check: scratch %zu bytes < required %zu",
                scratch ? scratch_bytes : size_t(0), need);
  kvs::AliasArgs a{cu_new, block_table, bt_stride, seq_lens, batch, total_new, max_new, max_seq_len,
                   pool->num_pages, static_cast<uint32_t*>(scratch), dev_status};
  return launched(kvs::launch_append_check(a, stream), "kv_pool_append_check");
}

size_t shared_kv_decode_workspace_bytes(int32_t batch, int32_t num_decoders, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_seq_len) {
  if (batch <= 0 || batch > kvs::kDecodeMaxBatch || num_decoders <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || max_seq_len < 0 || num_q_heads % num_kv_heads)
    return 0;
  return kvs::plan_decode(batch, num_decoders, num_q_heads, num_kv_heads, head_dim, max_seq_len).bytes;
}

int shared_kv_decode_workspace_init(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace) return fail(KVS_EINVAL, "shared_kv_decode_workspace_init: workspace is NULL");
  if (workspace_bytes < kvs::kDecodeCounterBytes)
    return fail(KVS_EWORKSPACE, "shared_kv_decode_workspace_init: workspace %zu bytes < %zu", workspace_bytes,
                kvs::kDecodeCounterBytes);
  return launched(kvs::launch_zero(workspace, kvs::kDecodeCounterBytes, stream), "shared_kv_decode_workspace_init");
}

}  // extern "C"

namespace {

int decode_common(const char* name, const kvs_pool* pool, int32_t layer, const void* q, void* out,
                  const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                  const int32_t* pbt, int32_t pbt_stride, const int32_t* plens, const int32_t* group_id,
                  const int32_t* group_prefix, int32_t batch, int32_t num_decoders, int32_t num_q_heads,
                  int32_t max_seq_len, int32_t max_priv_len, float scale, void* workspace,
                  size_t workspace_bytes, int32_t* dev_status, hipStream_t stream, const void* k_new = nullptr,
                  const void* v_new = nullptr) {
  int s = check_pool(pool, layer);
  if (s) return s;
  if (!q || !out || !block_table || !seq_lens) return fail(KVS_EINVAL, "%s: a required pointer is NULL", name);
  if ((s = check_table(batch, bt_stride, max_seq_len))) return s;
  if (num_decoders <= 0 || num_q_heads <= 0)
    return fail(KVS_EINVAL, "%s: num_decoders %d and num_q_heads %d must be positive", name, num_decoders,
                num_q_heads);
  if (num_q_heads % pool->num_kv_heads)
    return fail(KVS_EUNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                pool->num_kv_heads);
  if (!valid_scale(scale)) return fail(KVS_EINVAL, "%s: scale must be a positive finite number", name);
  if (batch > kvs::kDecodeMaxBatch)
    return fail(KVS_EUNSUPPORTED, "%s: batch %d above %d", name, batch, kvs::kDecodeMaxBatch);
  kvs::DecodePlan plan = kvs::plan_decode(batch, num_decoders, num_q_heads, pool->num_kv_heads,
                                          pool->head_dim, max_seq_len);
  // A cascade unit holds as many whole sessions as fit 64 rows, split into two
  // 32-row groups, one per wave of a pair.  With more than 64 rows per session a
  // unit would hold one session, whose pages plain decode reads the same way
  // (once for all its rows, in 64-row groups): such calls run plain decode over
  // the same block tables, and group_id / group_prefix_pages are not read.
  if (group_id && num_decoders * (num_q_heads / pool->num_kv_heads) > 64) group_id = group_prefix = nullptr;
  if (group_id) {
    const int ng = num_decoders * (num_q_heads / pool->num_kv_heads);
    const int per_unit = 64 / ng;
    kvs::DecodePlan full = kvs::plan_decode(batch, per_unit * num_decoders, num_q_heads, pool->num_kv_heads,
                                            pool->head_dim, max_seq_len);
    full.nb = 2;
    full.rg_rows = 32;
    full.rowgroups = 2;
    full.bytes = plan.bytes;  // same workspace layout and size
    full.cum_offset = plan.cum_offset;
    full.units_offset = plan.units_offset;
    full.ml_offset = plan.ml_offset;
    full.acc_offset = plan.acc_offset;
    plan = full;
  }
  if (pbt) {
    if (pbt_stride <= 0) return fail(KVS_EINVAL, "%s: priv_bt_stride %d must be positive", name, pbt_stride);
    if (max_priv_len < 0) return fail(KVS_EINVAL, "%s: max_priv_len %d is negative", name, max_priv_len);
    if (int64_t(max_priv_len) > int64_t(pbt_stride) * 16)
      return fail(KVS_ERANGE, "%s: max_priv_len %d exceeds private block-table capacity %lld", name,
                  max_priv_len, (long long)pbt_stride * 16);
  }
  if (!workspace || workspace_bytes < plan.bytes)
    return fail(KVS_EWORKSPACE, "%s: workspace %zu bytes < required %zu", name,
                workspace ? workspace_bytes : size_t(0), plan.bytes);
  char* ws = static_cast<char*>(workspace);
  kvs::DecodeArgs a{view(pool), layer, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                    block_table, bt_stride, seq_lens, batch, num_decoders, num_q_heads, max_seq_len,
                    scale * 1.4426950408889634f, pbt, pbt_stride, plens, max_priv_len, group_id, group_prefix,
                    static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                    reinterpret_cast<int*>(ws), reinterpret_cast<int*>(ws + plan.units_offset),
                    reinterpret_cast<int*>(ws + plan.cum_offset),
                    reinterpret_cast<float*>(ws + plan.ml_offset),
                    reinterpret_cast<float*>(ws + plan.acc_offset), plan, dev_status};
  return launched(kvs::launch_decode(a, stream), name);
}

}  // namespace

extern "C" {

int shared_kv_decode(const kvs_pool* pool, int32_t layer, const void* q, void* out,
                     const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                     int32_t batch, int32_t num_decoders, int32_t num_q_heads, int32_t max_seq_len,
                     float scale, void* workspace, size_t workspace_bytes, int32_t* dev_status,
                     hipStream_t stream) {
  return decode_common("shared_kv_decode", pool, layer, q, out, block_table, bt_stride, seq_lens, nullptr, 0,
                       nullptr, nullptr, nullptr, batch, num_decoders, num_q_heads, max_seq_len, 0, scale,
                       workspace, workspace_bytes, dev_status, stream);
}

}  // extern "C"

namespace {

// Scratch of shared_kv_decode_noalloc: a decode workspace for the largest call
// the library accepts (batch <= 4096, head_dim <= 128), in device memory the
// code object itself holds, so the entry point allocates nothing.  In host code
// `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed on.
constexpr size_t kNoAllocScratchBytes = kvs::kDecodeWorkspaceMaxBytes;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's scratch address.  At its first use on a device it also
// zeroes the arrival counters (with a fill kernel on `stream`); every decode
// call leaves them zero again.
int noalloc_scratch(void** out, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVS_EHIP, "shared_kv_decode_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KVS_EUNSUPPORTED, "shared_kv_decode_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(KVS_EHIP, "shared_kv_decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    e = kvs::launch_zero(ptr, kvs::kDecodeCounterBytes, stream);
    if (e != hipSuccess)
      return fail(KVS_EHIP, "shared_kv_decode_noalloc: clearing the scratch counters: %s", hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return KVS_OK;
}

}  // namespace

extern "C" {

int shared_kv_decode_noalloc(const kvs_pool* pool, int32_t layer, const void* q, void* out,
                             const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                             int32_t batch, int32_t num_decoders, int32_t num_q_heads, int32_t max_seq_len,
                             float scale, int32_t* dev_status, hipStream_t stream) {
  const char* name = "shared_kv_decode_noalloc";
  if (!pool) return fail(KVS_EINVAL, "%s: pool is NULL", name);
  if (batch > kvs::kDecodeMaxBatch)
    return fail(KVS_EUNSUPPORTED, "%s: batch %d above %d", name, batch, kvs::kDecodeMaxBatch);
  if (batch > 0 && pool->head_dim > 0 && pool->head_dim <= 128) {
    const size_t need = kvs::decode_workspace_size(batch, pool->head_dim);
    if (need > kNoAllocScratchBytes)
      return fail(KVS_EWORKSPACE, "%s: the call needs %zu bytes of scratch, above the static %zu", name, need,
                  kNoAllocScratchBytes);
  }
  void* ws = nullptr;
  int s = noalloc_scratch(&ws, stream);
  if (s) return s;
  return decode_common(name, pool, layer, q, out, block_table, bt_stride, seq_lens, nullptr, 0, nullptr, nullptr,
                       nullptr, batch, num_decoders, num_q_heads, max_seq_len, 0, scale, ws, kNoAllocScratchBytes,
                       dev_status, stream);
}

int shared_kv_decode_append(const kvs_pool* pool, int32_t layer, const void* k_new, const void* v_new,
                            const void* q, void* out, const int32_t* block_table, int32_t bt_stride,
                            const int32_t* seq_lens, int32_t batch, int32_t num_decoders, int32_t num_q_heads,
                            int32_t max_seq_len, float scale, void* workspace, size_t workspace_bytes,
                            int32_t* dev_status, hipStream_t stream) {
  if (!k_new || !v_new) return fail(KVS_EINVAL, "shared_kv_decode_append: a required pointer is NULL");
  return decode_common("shared_kv_decode_append", pool, layer, q, out, block_table, bt_stride, seq_lens, nullptr,
                       0, nullptr, nullptr, nullptr, batch, num_decoders, num_q_heads, max_seq_len, 0, scale,
                       workspace, workspace_bytes, dev_status, stream, k_new, v_new);
}

int shared_kv_decode_private(const kvs_pool* pool, int32_t layer, const void* q, void* out,
                             const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                             const int32_t* priv_block_table, int32_t priv_bt_stride,
                             const int32_t* priv_lens, int32_t batch, int32_t num_decoders,
                             int32_t num_q_heads, int32_t max_seq_len, int32_t max_priv_len,
                             float scale, void* workspace, size_t workspace_bytes,
                             int32_t* dev_status, hipStream_t stream) {
  if (!priv_block_table || !priv_lens)
    return fail(KVS_EINVAL, "shared_kv_decode_private: a required pointer is NULL");
  return decode_common("shared_kv_decode_private", pool, layer, q, out, block_table, bt_stride, seq_lens,
                       priv_block_table, priv_bt_stride, priv_lens, nullptr, nullptr, batch, num_decoders,
                       num_q_heads, max_seq_len, max_priv_len, scale, workspace, workspace_bytes, dev_status,
                       stream);
}

int shared_kv_decode_cascade(const kvs_pool* pool, int32_t layer, const void* q, void* out,
                             const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                             const int32_t* group_id, const int32_t* group_prefix_pages, int32_t batch,
                             int32_t num_decoders, int32_t num_q_heads, int32_t max_seq_len, float scale,
                             void* workspace, size_t workspace_bytes, int32_t* dev_status,
                             hipStream_t stream) {
  if (!group_id || !group_prefix_pages)
    return fail(KVS_EINVAL, "shared_kv_decode_cascade: a required pointer is NULL");
  return decode_common("shared_kv_decode_cascade", pool, layer, q, out, block_table, bt_stride, seq_lens,
                       nullptr, 0, nullptr, group_id, group_prefix_pages, batch, num_decoders, num_q_heads,
                       max_seq_len, 0, scale, workspace, workspace_bytes, dev_status, stream);
}

}  // extern "C"

namespace {

int extend_common(const char* name, const kvs_pool* pool, int32_t layer, int32_t num_layers, const void* q,
                  const void* k_new, const void* v_new, void* out, const int32_t* cu_new, const int32_t* block_table,
                  int32_t bt_stride, const int32_t* seq_lens, int32_t batch, int32_t num_q_heads, int32_t total_new,
                  int32_t max_new, int32_t max_seq_len, float scale, int32_t* dev_status, hipStream_t stream) {
  int s = check_pool(pool, layer);
  if (s) return s;
  if (num_layers <= 0 || int64_t(layer) + num_layers > pool->num_layers)
    return fail(KVS_ERANGE, "%s: layers [%d, %d + %d) outside the pool's %d", name, layer, layer, num_layers,
                pool->num_layers);
  if (!q || !k_new || !v_new || !out || !cu_new || !block_table || !seq_lens)
    return fail(KVS_EINVAL, "%s: a required pointer is NULL", name);
  if ((s = check_table(batch, bt_stride, max_seq_len))) return s;
  if (num_q_heads <= 0 || max_new <= 0 || total_new < 0)
    return fail(KVS_EINVAL, "%s: num_q_heads %d, max_new %d must be >= 1", name, num_q_heads, max_new);
  if (max_new > max_seq_len)
    return fail(KVS_ERANGE, "%s: max_new %d exceeds max_seq_len %d", name, max_new, max_seq_len);
  if (num_q_heads % pool->num_kv_heads)
    return fail(KVS_EUNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                pool->num_kv_heads);
  if (!valid_scale(scale)) return fail(KVS_EINVAL, "%s: scale must be a positive finite number", name);
  const int64_t units = int64_t(num_layers) * batch * pool->num_kv_heads;
  if (units > (int64_t(1) << 30))
    return fail(KVS_EUNSUPPORTED, "%s: %lld (layer, session, KV head) units in one call", name, (long long)units);
  const int64_t kv_stride = int64_t(total_new) * pool->num_kv_heads * pool->head_dim;
  const int64_t q_stride = int64_t(total_new) * num_q_heads * pool->head_dim;
  kvs::AppendArgs ap{view(pool), layer, static_cast<const uint16_t*>(k_new),
                     static_cast<const uint16_t*>(v_new), cu_new, block_table, bt_stride, seq_lens,
                     batch, total_new, max_new, max_seq_len, dev_status, num_layers, kv_stride};
  char what[96];
  snprintf(what, sizeof what, "%s (append)", name);
  if ((s = launched(kvs::launch_append(ap, stream), what))) return s;
  kvs::ExtendArgs a{view(pool), layer, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
                    cu_new, block_table, bt_stride, seq_lens, batch, num_q_heads, total_new, max_new,
                    max_seq_len, scale * 1.4426950408889634f, dev_status, num_layers, q_stride};
  return launched(kvs::launch_extend(a, stream), name);
}

}  // namespace

extern "C" {

int partial_prefill_extend(const kvs_pool* pool, int32_t layer, const void* q, const void* k_new,
                           const void* v_new, void* out, const int32_t* cu_new,
                           const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                           int32_t batch, int32_t num_q_heads, int32_t total_new, int32_t max_new,
                           int32_t max_seq_len, float scale, int32_t* dev_status, hipStream_t stream) {
  return extend_common("partial_prefill_extend", pool, layer, 1, q, k_new, v_new, out, cu_new, block_table,
                       bt_stride, seq_lens, batch, num_q_heads, total_new, max_new, max_seq_len, scale, dev_status,
                       stream);
}

int partial_prefill_layers(const kvs_pool* pool, int32_t layer_begin, int32_t num_layers, const void* q,
                           const void* k_new, const void* v_new, void* out, const int32_t* cu_new,
                           const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                           int32_t batch, int32_t num_q_heads, int32_t total_new, int32_t max_new,
                           int32_t max_seq_len, float scale, int32_t* dev_status, hipStream_t stream) {
  return extend_common("partial_prefill_layers", pool, layer_begin, num_layers, q, k_new, v_new, out, cu_new,
                       block_table, bt_stride, seq_lens, batch, num_q_heads, total_new, max_new, max_seq_len, scale,
                       dev_status, stream);
}

size_t kv_pages_buffer_bytes(const kvs_pool* pool, int32_t num_layers, int32_t num_ids) {
  if (!pool || num_layers <= 0 || num_ids < 0 || pool->num_kv_heads <= 0 || pool->head_dim <= 0) return 0;
  return size_t(num_layers) * size_t(num_ids) * size_t(pool->num_kv_heads) * 32 * size_t(pool->head_dim) * 2;
}

}  // extern "C"

namespace {

int pack_common(const char* name, bool unpack, const kvs_pool* pool, int32_t layer_begin, int32_t num_layers,
                const int32_t* page_ids, int32_t num_ids, const void* buf, int32_t* dev_status,
                hipStream_t stream) {
  int s = check_pool(pool, layer_begin);
  if (s) return s;
  if (num_layers <= 0 || int64_t(layer_begin) + num_layers > pool->num_layers)
    return fail(KVS_ERANGE, "%s: layers [%d, %d + %d) outside the pool's %d", name, layer_begin, layer_begin,
                num_layers, pool->num_layers);
  if (num_ids < 0) return fail(KVS_EINVAL, "%s: num_ids %d is negative", name, num_ids);
  if (num_layers > 65535) return fail(KVS_EUNSUPPORTED, "%s: %d layers in one call (at most 65535)", name, num_layers);
  if (num_ids > 0 && (!page_ids || !buf)) return fail(KVS_EINVAL, "%s: a required pointer is NULL", name);
  kvs::HandoffArgs a{view(pool), layer_begin, num_layers, page_ids, num_ids,
                     static_cast<uint16_t*>(const_cast<void*>(buf)), dev_status};
  return launched(kvs::launch_pack(a, unpack, stream), name);
}

}  // namespace

extern "C" {

int kv_pages_pack(const kvs_pool* pool, int32_t layer_begin, int32_t num_layers, const int32_t* page_ids,
                  int32_t num_ids, void* buf, int32_t* dev_status, hipStream_t stream) {
  return pack_common("kv_pages_pack", false, pool, layer_begin, num_layers, page_ids, num_ids, buf, dev_status,
                     stream);
}

int kv_pages_unpack(const kvs_pool* pool, int32_t layer_begin, int32_t num_layers, const int32_t* page_ids,
                    int32_t num_ids, const void* buf, int32_t* dev_status, hipStream_t stream) {
  return pack_common("kv_pages_unpack", true, pool, layer_begin, num_layers, page_ids, num_ids, buf, dev_status,
                     stream);
}

int kv_pool_fetch(const kvs_pool* pool, int32_t layer, const int32_t* block_table, int32_t bt_stride,
                  const int32_t* seq_lens, const int32_t* cu_rows, int32_t batch, int32_t total_rows,
                  int32_t max_seq_len, void* k_out, void* v_out, int32_t* dev_status, hipStream_t stream) {
  int s = check_pool(pool, layer);
  if (s) return s;
  if (!block_table || !seq_lens || !cu_rows || !k_out || !v_out)
    return fail(KVS_EINVAL, "kv_pool_fetch: a required pointer is NULL");
  if ((s = check_table(batch, bt_stride, max_seq_len))) return s;
  if (total_rows < 0) return fail(KVS_EINVAL, "kv_pool_fetch: total_rows %d is negative", total_rows);
  if (batch > 65535) return fail(KVS_EUNSUPPORTED, "kv_pool_fetch: batch %d above 65535", batch);
  kvs::FetchArgs a{view(pool), layer, block_table, bt_stride, seq_lens, cu_rows, batch, total_rows, max_seq_len,
                   static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out), dev_status};
  return launched(kvs::launch_fetch(a, stream), "kv_pool_fetch");
}

}  // extern "C"
