// C ABI of libpagedkv: host-side argument validation and kernel dispatch.
// Declarations and the contract of every entry point: include/pagedkv.h.

#include "pagedkv.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <vector>

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

pkv_status fail(pkv_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

pkv_status hip_fail(hipError_t err, const char* what) {
  return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(err));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---- metadata check mode -----------------------------------------------------
// Device metadata (block tables, lengths, slots, pairs) is trusted: the
// kernels never let a bad entry move an access outside its buffer, but the
// result is then undefined.  With PAGEDKV_CHECK=1 in the environment each
// entry point first copies its metadata to the host (on its stream, then
// waits for it) and rejects what breaks the contract with PKV_ECHECK.  Debug
// only: the wait is not allowed while the stream is being captured.

bool check_mode() {
  const char* v = getenv("PAGEDKV_CHECK");
  return v && v[0] == '1' && v[1] == '\0';
}

pkv_status fetch_i32(std::vector<int32_t>& h, const int32_t* d, size_t count, hipStream_t stream,
                     const char* what) {
  h.assign(count, 0);
  if (count == 0) return PKV_OK;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone)
    return fail(PKV_EUNSUPPORTED, "%s: PAGEDKV_CHECK=1 waits for the stream, which capture forbids",
                what);
  hipError_t err = hipMemcpyAsync(h.data(), d, count * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (err == hipSuccess) err = hipStreamSynchronize(stream);
  return err == hipSuccess ? PKV_OK : hip_fail(err, what);
}

// ids[0..n) inside [0, num_blocks) and, if `unique`, pairwise distinct
pkv_status check_ids(const char* what, const char* name, const std::vector<int32_t>& ids,
                     size_t stride, size_t offset, int32_t num_blocks, bool unique) {
  std::vector<int32_t> seen;
  for (size_t i = offset; i < ids.size(); i += stride) {
    const int32_t id = ids[i];
    if (id < 0 || id >= num_blocks)
      return fail(PKV_ECHECK, "%s: %s entry %zu = %d is outside the pool [0, %d)", what, name,
                  (i - offset) / stride, id, num_blocks);
    if (unique) seen.push_back(id);
  }
  std::sort(seen.begin(), seen.end());
  for (size_t i = 1; i < seen.size(); ++i)
    if (seen[i] == seen[i - 1])
      return fail(PKV_ECHECK, "%s: %s names block %d more than once", what, name, seen[i]);
  return PKV_OK;
}

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16:
    case PKV_BF16: return 2;
    default: return 0;
  }
}

pkv_status check_pool(const pkv_pool& pool) {
  if (elem_bytes(pool.dtype) == 0) return fail(PKV_EUNSUPPORTED, "dtype %d is not f32/f16/bf16", pool.dtype);
  if (pool.num_blocks <= 0 || pool.num_kv_heads <= 0)
    return fail(PKV_EINVAL, "pool needs num_blocks > 0 and num_kv_heads > 0 (got %d, %d)",
                pool.num_blocks, pool.num_kv_heads);
  if (pool.block_size != 16 && pool.block_size != 32)
    return fail(PKV_EUNSUPPORTED, "block_size %d is not 16 or 32", pool.block_size);
  if (pool.head_dim != 64 && pool.head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "head_dim %d is not 64 or 128", pool.head_dim);
  return PKV_OK;
}

size_t pool_block_bytes(const pkv_pool& pool) {
  return (size_t)pool.num_kv_heads * pool.block_size * pool.head_dim * elem_bytes(pool.dtype);
}

constexpr int kMaxDevices = 64;

// Workgroups of the stream attention kernel on the current device: two per
// compute unit (its occupancy), a multiple of the 8 XCDs.  Cached per device.
int stream_workgroups() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int wgs = cached[dev].load(std::memory_order_relaxed);
  if (wgs == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    wgs = (2 * cus) / 8 * 8;
    if (wgs < 8) wgs = 8;
    cached[dev].store(wgs, std::memory_order_relaxed);
  }
  return wgs;
}

// PAGEDKV_DECODE_PATH=grid in the environment sends every decode call (and
// its workspace query) to the grid path: one workgroup per (kv head,
// sequence, 512-token partition) and the partition merge, whatever the batch.
// For measuring and testing that path at any shape; read on every call.
bool force_grid_path() {
  const char* v = getenv("PAGEDKV_DECODE_PATH");
  return v && strcmp(v, "grid") == 0;
}

// PAGEDKV_K_LOAD=direct: decode calls on the stream path load K straight in
// the MFMA operand order instead of whole 128-byte lines re-dealt through
// LDS.  A measurement variant of one shape (bf16, D 128, 16-token blocks),
// ignored elsewhere; same result bit for bit.  Read on every call.
bool k_direct_loads() {
  const char* v = getenv("PAGEDKV_K_LOAD");
  return v && strcmp(v, "direct") == 0;
}

// ---- clock records (measurement) -------------------------------------------
// PAGEDKV_CLOCK=1 in the environment: attention calls of the shape the clock
// builds exist for (bf16, D 128, 16-token blocks) run them, which record each
// decode wave's or prefill workgroup's start, end and XCD into this array
// (one per GPU, held until the process ends; cleared on the call's stream
// first).  pkv_clock_read copies it out.  Calls under graph capture, and
// calls of other shapes, run the normal kernels.  Read on every call.
constexpr size_t kClockBytes = (size_t)pkv::kClockRecords * pkv::kClockWords * sizeof(unsigned long long);
static __device__ __align__(256) unsigned long long clock_records[pkv::kClockRecords * pkv::kClockWords];

bool clock_mode() {
  const char* v = getenv("PAGEDKV_CLOCK");
  return v && v[0] == '1' && v[1] == '\0';
}

// Device address of this GPU's record array (looked up once per device with
// that device current), or nullptr.
unsigned long long* clock_on_current_device() {
  static std::atomic<void*> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = cached[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(clock_records)) != hipSuccess) return nullptr;
    cached[dev].store(ptr, std::memory_order_release);
  }
  return static_cast<unsigned long long*>(ptr);
}

// Workgroups of the stream path for this call on the current device, or 0
// where it cannot take the call: a batch above its LDS tables, or more
// positions (kv heads x column groups x sub-tiles) than it indexes.  Decode
// calls then take the grid path; multi-token calls are refused.
int32_t stream_wgs_for(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                       int32_t max_groups, bool multi) {
  if (num_seqs > (multi ? pkv::kMaxMultiSeqs : pkv::kMaxStreamSeqs)) return 0;
  if (!multi && force_grid_path()) return 0;
  const long long subs = ((long long)(max_context_len > 0 ? max_context_len : 0) + pkv::kSubTokens - 1) /
                         pkv::kSubTokens;
  if ((long long)num_seqs * num_kv_heads * max_groups * subs > pkv::kMaxStreamPositions) return 0;
  return stream_workgroups();
}

// Column geometry of a call: groups of 16 (new token, query head) columns.
int32_t max_groups_for(int32_t max_query_len, int32_t group) {
  return (int32_t)(((long long)max_query_len * group + pkv::kSubTokens - 1) / pkv::kSubTokens);
}
// Multi-token calls whose longest sequence has at least kPrefillMinCols
// (new token, query head) columns take the prefill path.
bool prefill_route(int32_t max_query_len, int32_t group) {
  return (long long)max_query_len * group >= pkv::kPrefillMinCols;
}
int32_t slot_cols_for(int32_t max_query_len, int32_t group) {
  const long long c = (long long)max_query_len * group;
  return (int32_t)(c < pkv::kSubTokens ? c : pkv::kSubTokens);
}

int32_t partitions_for(int32_t max_context_len) {
  const int32_t P = (max_context_len + pkv::kPartitionTokens - 1) / pkv::kPartitionTokens;
  return P > 0 ? P : 1;
}

}  // namespace

extern "C" {

int32_t pkv_partition_tokens(void) { return pkv::kPartitionTokens; }

const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported configuration";
    case PKV_EWORKSPACE: return "workspace missing or too small";
    case PKV_EHIP: return "HIP runtime error";
    case PKV_ECHECK: return "metadata check failed";
  }
  return "unknown status";
}

const char* pkv_last_error(void) { return g_err; }

pkv_status paged_kv_append(const void* key, const void* value, void* k_cache, void* v_cache,
                           pkv_pool pool, const int32_t* slot_mapping, int32_t num_tokens,
                           hipStream_t stream) {
  g_err[0] = '\0';
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_EINVAL, "null pointer argument");
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_EINVAL, "key, value and the pools must be 16-byte aligned");
  if ((long long)pool.num_blocks * pool.block_size > 0x7fffffffLL)
    return fail(PKV_EINVAL, "num_blocks * block_size exceeds the int32 slot range");
  if (check_mode()) {
    std::vector<int32_t> slots;
    st = fetch_i32(slots, slot_mapping, (size_t)num_tokens, stream, "paged_kv_append check");
    if (st != PKV_OK) return st;
    const int32_t nslots = pool.num_blocks * pool.block_size;
    std::vector<int32_t> used;
    for (int32_t i = 0; i < num_tokens; ++i) {
      if (slots[i] >= nslots)
        return fail(PKV_ECHECK, "paged_kv_append: slot_mapping[%d] = %d is outside the pool's %d slots",
                    i, slots[i], nslots);
      if (slots[i] >= 0) used.push_back(slots[i]);
    }
    std::sort(used.begin(), used.end());
    for (size_t i = 1; i < used.size(); ++i)
      if (used[i] == used[i - 1])
        return fail(PKV_ECHECK, "paged_kv_append: slot %d is written more than once", used[i]);
  }
  hipError_t err = pkv::launch_kv_append(key, value, k_cache, v_cache, slot_mapping, num_tokens,
                                         pool.num_kv_heads, pool.block_size, pool.head_dim,
                                         elem_bytes(pool.dtype), pool.num_blocks, stream);
  return err == hipSuccess ? PKV_OK : hip_fail(err, "paged_kv_append launch");
}

}  // extern "C"

namespace {

// Workspace of a decode (max_query_len 1, multi false) or multi-token call,
// or 0 with a reason for a call that is refused.
size_t attention_workspace(const pkv_pool& pool, int32_t num_seqs, int32_t num_q_heads,
                           int32_t max_query_len, int32_t max_context_len, bool multi) {
  if (check_pool(pool) != PKV_OK || num_seqs <= 0 || num_q_heads <= 0 || max_context_len < 0 ||
      max_query_len <= 0 || num_q_heads % pool.num_kv_heads != 0)
    return 0;
  const int32_t group = num_q_heads / pool.num_kv_heads;
  const int32_t groups = max_groups_for(max_query_len, group);
  if (multi && prefill_route(max_query_len, group)) {
    const int32_t parts =
        pkv::prefill_plan(num_seqs, pool.num_kv_heads, groups, max_context_len, pool.dtype).parts;
    // every query row may belong to a split context: bound by the rows the
    // batch can hold (num_seqs * max_query_len)
    const long long rows = (long long)num_seqs * max_query_len;
    if (rows > 0x7fffffffLL) return 0;
    return pkv::prefill_workspace_layout((int32_t)rows, num_q_heads, pool.head_dim, parts).bytes;
  }
  const int32_t wgs = stream_wgs_for(num_seqs, pool.num_kv_heads, max_context_len, groups, multi);
  if (multi && wgs == 0) return 0;
  return pkv::attn_workspace_layout(num_seqs, slot_cols_for(max_query_len, group), num_q_heads,
                                    pool.head_dim, max_context_len, wgs)
      .bytes;
}

// Validation and launch shared by paged_attention_decode (query_start null:
// row s is sequence s's one new token) and paged_attention_multi.
pkv_status attention_call(const char* what, void* out, const void* q, const void* k_cache,
                          const void* v_cache, const pkv_pool& pool, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          const int32_t* query_start, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_query_tokens, int32_t max_query_len, float scale,
                          int32_t max_context_len, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  const bool multi = query_start != nullptr;
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_seqs < 0) return fail(PKV_EINVAL, "num_seqs %d < 0", num_seqs);
  if (num_seqs == 0) return PKV_OK;
  if (num_q_heads <= 0 || num_q_heads % pool.num_kv_heads != 0)
    return fail(PKV_EINVAL, "num_q_heads %d is not a positive multiple of num_kv_heads %d",
                num_q_heads, pool.num_kv_heads);
  const int32_t group = num_q_heads / pool.num_kv_heads;
  if (group > 16) return fail(PKV_EUNSUPPORTED, "query heads per kv head %d > 16", group);
  if (max_context_len < 0) return fail(PKV_EINVAL, "max_context_len %d < 0", max_context_len);
  if (max_blocks_per_seq < 0 || (long long)max_blocks_per_seq * pool.block_size < max_context_len)
    return fail(PKV_EINVAL, "max_blocks_per_seq %d * block_size %d < max_context_len %d",
                max_blocks_per_seq, pool.block_size, max_context_len);
  if (!(scale == scale)) return fail(PKV_EINVAL, "scale is NaN");
  if (multi) {
    if (num_query_tokens < 0 || max_query_len < 0)
      return fail(PKV_EINVAL, "num_query_tokens %d / max_query_len %d < 0", num_query_tokens,
                  max_query_len);
    if (num_query_tokens == 0 || max_query_len == 0) return PKV_OK;
  }
  if (!out || !q || !k_cache || !v_cache || !context_lens || (max_blocks_per_seq > 0 && !block_tables))
    return fail(PKV_EINVAL, "null pointer argument");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PKV_EINVAL, "out, q and the pools must be 16-byte aligned");
  const int32_t groups = max_groups_for(max_query_len, group);
  const bool prefill = multi && prefill_route(max_query_len, group);
  if (prefill && num_seqs > 65535)
    return fail(PKV_EUNSUPPORTED, "the prefill path takes at most 65535 sequences");
  const int32_t stream_wgs =
      prefill ? 0 : stream_wgs_for(num_seqs, pool.num_kv_heads, max_context_len, groups, multi);
  if (multi && !prefill && stream_wgs == 0)
    return fail(PKV_EUNSUPPORTED,
                "multi-token attention takes at most %d sequences and 2^28 positions "
                "(kv heads x 16-column groups x 16-token sub-tiles)",
                pkv::kMaxMultiSeqs);
  const int32_t cols = slot_cols_for(max_query_len, group);
  const pkv::PrefillPlan plan =
      prefill ? pkv::prefill_plan(num_seqs, pool.num_kv_heads, groups, max_context_len, pool.dtype)
              : pkv::PrefillPlan{1, 0, 1};
  const int32_t pf_blocks = plan.blocks;
  const int32_t pf_parts = plan.parts;
  const pkv::AttnWorkspace lay =
      prefill ? pkv::prefill_workspace_layout(num_query_tokens, num_q_heads, pool.head_dim, pf_parts)
              : pkv::attn_workspace_layout(num_seqs, cols, num_q_heads, pool.head_dim,
                                           max_context_len, stream_wgs);
  if (lay.bytes > 0 && (!workspace || workspace_bytes < lay.bytes))
    return fail(PKV_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, lay.bytes);
  if (lay.bytes > 0 && !aligned16(workspace)) return fail(PKV_EINVAL, "workspace must be 16-byte aligned");

  if (check_mode()) {
    std::vector<int32_t> lens, tables, qs;
    st = fetch_i32(lens, context_lens, (size_t)num_seqs, stream, what);
    if (st == PKV_OK && max_blocks_per_seq > 0)
      st = fetch_i32(tables, block_tables, (size_t)num_seqs * max_blocks_per_seq, stream, what);
    if (st == PKV_OK && multi) st = fetch_i32(qs, query_start, (size_t)num_seqs + 1, stream, what);
    if (st != PKV_OK) return st;
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t n = lens[s];
      if (n < 0 || n > max_context_len)
        return fail(PKV_ECHECK, "context_lens[%d] = %d is outside [0, max_context_len %d]", s, n,
                    max_context_len);
      const int32_t nb = (n + pool.block_size - 1) / pool.block_size;
      for (int32_t j = 0; j < nb; ++j) {
        const int32_t id = tables[(size_t)s * max_blocks_per_seq + j];
        if (id < 0 || id >= pool.num_blocks)
          return fail(PKV_ECHECK, "block_tables[%d][%d] = %d is outside the pool [0, %d)", s, j, id,
                      pool.num_blocks);
      }
      if (multi) {
        const int32_t L = qs[s + 1] - qs[s];
        if (qs[s] < 0 || L < 0 || L > n || L > max_query_len)
          return fail(PKV_ECHECK,
                      "query_start[%d..%d] = %d..%d: %d new tokens, with a context of %d and "
                      "max_query_len %d",
                      s, s + 1, qs[s], qs[s + 1], L, n, max_query_len);
      }
    }
    if (multi && (qs[0] != 0 || qs[num_seqs] != num_query_tokens))
      return fail(PKV_ECHECK, "query_start runs from %d to %d, not from 0 to num_query_tokens %d",
                  qs[0], qs[num_seqs], num_query_tokens);
  }

  pkv::AttnParams prm;
  prm.out = out;
  prm.q = q;
  prm.k_cache = k_cache;
  prm.v_cache = v_cache;
  prm.block_tables = block_tables;
  prm.context_lens = context_lens;
  prm.max_blocks_per_seq = max_blocks_per_seq;
  prm.num_seqs = num_seqs;
  prm.num_q_heads = num_q_heads;
  prm.num_kv_heads = pool.num_kv_heads;
  prm.group = group;
  prm.num_blocks = pool.num_blocks;
  prm.max_context_len = max_context_len;
  prm.scale_log2 = scale * 1.4426950408889634f;
  char* base = static_cast<char*>(workspace);
  prm.seq_prefix = lay.bytes > 0 ? reinterpret_cast<int32_t*>(base + lay.prefix_off) : nullptr;
  prm.part_o = lay.bytes > 0 ? reinterpret_cast<float*>(base + lay.part_o_off) : nullptr;
  prm.part_ml = lay.bytes > 0 ? reinterpret_cast<float*>(base + lay.part_ml_off) : nullptr;
  prm.stream_wgs = stream_wgs;
  prm.max_partitions = partitions_for(max_context_len);
  prm.query_start = query_start;
  prm.num_query_tokens = multi ? num_query_tokens : num_seqs;
  prm.max_query_len = multi ? max_query_len : 1;
  prm.max_groups = groups;
  prm.slot_cols = cols;
  prm.prefill_blocks = pf_blocks;
  prm.prefill_parts = pf_parts;
  prm.prefill_wave_groups = plan.wave_groups;
  prm.k_direct = !multi && k_direct_loads() ? 1 : 0;
  prm.clock = nullptr;
  if (clock_mode()) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone) {
      unsigned long long* rec = clock_on_current_device();
      if (rec && hipMemsetAsync(rec, 0, kClockBytes, stream) == hipSuccess) prm.clock = rec;
    }
  }
  hipError_t err = pkv::launch_paged_attention(prm, pool.dtype, pool.head_dim, pool.block_size, stream);
  return err == hipSuccess ? PKV_OK : hip_fail(err, what);
}

}  // namespace

extern "C" {

size_t paged_attention_workspace_bytes(pkv_pool pool, int32_t num_seqs, int32_t num_q_heads,
                                       int32_t max_context_len) {
  g_err[0] = '\0';
  return attention_workspace(pool, num_seqs, num_q_heads, 1, max_context_len, false);
}

pkv_status paged_attention_decode(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, pkv_pool pool,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, float scale, int32_t max_context_len,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  return attention_call("paged_attention_decode launch", out, q, k_cache, v_cache, pool,
                        block_tables, max_blocks_per_seq, context_lens, nullptr, num_seqs,
                        num_q_heads, num_seqs, 1, scale, max_context_len, workspace,
                        workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of paged_attention_decode_noalloc: the decode workspace (sequence
// offsets and the fp32 partial states of split sequences) for callers that
// cannot allocate.  Each GPU the library runs on holds its own copy of the
// array until the process ends.  On the host, `scratch` names a host-side
// stand-in, never the device memory: only the address hipGetSymbolAddress
// returns for the current device is passed to kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this GPU's scratch array, looked up once per device with
// that device current, or nullptr (with the error set) if the lookup fails.
void* scratch_on_current_device() {
  static std::atomic<void*> cached[kMaxDevices];
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) {
    hip_fail(err, "paged_attention_decode_noalloc: hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(PKV_EUNSUPPORTED, "paged_attention_decode_noalloc: device %d beyond the %d supported",
         dev, kMaxDevices);
    return nullptr;
  }
  void* ptr = cached[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess || ptr == nullptr) {
      hip_fail(err != hipSuccess ? err : hipErrorInvalidSymbol,
               "paged_attention_decode_noalloc: hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    cached[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

extern "C" {

size_t paged_attention_noalloc_max_bytes(void) { return kScratchBytes; }

int32_t pkv_clock_records(void) { return pkv::kClockRecords; }

pkv_status pkv_clock_read(unsigned long long* host, size_t records) {
  g_err[0] = '\0';
  if (records > (size_t)pkv::kClockRecords)
    return fail(PKV_EINVAL, "pkv_clock_read: %zu records asked for, %d held", records,
                pkv::kClockRecords);
  if (records == 0) return PKV_OK;
  if (!host) return fail(PKV_EINVAL, "pkv_clock_read: null host buffer");
  unsigned long long* rec = clock_on_current_device();
  if (!rec) return fail(PKV_EHIP, "pkv_clock_read: record array not found on this device");
  hipError_t err = hipDeviceSynchronize();
  if (err == hipSuccess)
    err = hipMemcpy(host, rec, records * pkv::kClockWords * sizeof(unsigned long long),
                    hipMemcpyDeviceToHost);
  return err == hipSuccess ? PKV_OK : hip_fail(err, "pkv_clock_read");
}

pkv_status paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                          const void* v_cache, pkv_pool pool,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_q_heads, float scale,
                                          int32_t max_context_len, hipStream_t stream) {
  g_err[0] = '\0';
  if (check_mode())
    return fail(PKV_EUNSUPPORTED,
                "paged_attention_decode_noalloc: PAGEDKV_CHECK=1 copies metadata into host "
                "buffers and waits; use paged_attention_decode for checked calls");
  // the size first: an oversized call is refused before any device call
  const size_t need =
      attention_workspace(pool, num_seqs, num_q_heads, 1, max_context_len, false);
  if (need > kScratchBytes)
    return fail(PKV_EWORKSPACE,
                "paged_attention_decode_noalloc: this call needs %zu bytes of workspace, above "
                "the %zu-byte scratch array (use paged_attention_decode with a workspace)",
                need, kScratchBytes);
  if (num_seqs <= 0 || need == 0)  // nothing to hold: validation alone decides
    return attention_call("paged_attention_decode_noalloc launch", out, q, k_cache, v_cache, pool,
                          block_tables, max_blocks_per_seq, context_lens, nullptr, num_seqs,
                          num_q_heads, num_seqs, 1, scale, max_context_len, nullptr, 0, stream);
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return PKV_EHIP;
  return attention_call("paged_attention_decode_noalloc launch", out, q, k_cache, v_cache, pool,
                        block_tables, max_blocks_per_seq, context_lens, nullptr, num_seqs,
                        num_q_heads, num_seqs, 1, scale, max_context_len, ws, kScratchBytes,
                        stream);
}

size_t paged_attention_multi_workspace_bytes(pkv_pool pool, int32_t num_seqs, int32_t num_q_heads,
                                             int32_t max_query_len, int32_t max_context_len) {
  g_err[0] = '\0';
  return attention_workspace(pool, num_seqs, num_q_heads, max_query_len, max_context_len, true);
}

pkv_status paged_attention_multi(void* out, const void* q, const void* k_cache,
                                 const void* v_cache, pkv_pool pool, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 const int32_t* query_start, int32_t num_seqs, int32_t num_q_heads,
                                 int32_t num_query_tokens, int32_t max_query_len, float scale,
                                 int32_t max_context_len, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  g_err[0] = '\0';
  if (!query_start) return fail(PKV_EINVAL, "null pointer argument (query_start)");
  return attention_call("paged_attention_multi launch", out, q, k_cache, v_cache, pool,
                        block_tables, max_blocks_per_seq, context_lens, query_start, num_seqs,
                        num_q_heads, num_query_tokens, max_query_len, scale, max_context_len,
                        workspace, workspace_bytes, stream);
}

pkv_status paged_copy_blocks(void* k_cache, void* v_cache, pkv_pool pool,
                             const int32_t* block_mapping, int32_t num_pairs, hipStream_t stream) {
  g_err[0] = '\0';
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_pairs < 0) return fail(PKV_EINVAL, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_mapping) return fail(PKV_EINVAL, "null pointer argument");
  if (!aligned16(k_cache) || !aligned16(v_cache)) return fail(PKV_EINVAL, "pools must be 16-byte aligned");
  if (num_pairs > 0x3fffffff) return fail(PKV_EINVAL, "num_pairs %d too large", num_pairs);
  if (check_mode()) {
    std::vector<int32_t> pairs;
    st = fetch_i32(pairs, block_mapping, (size_t)num_pairs * 2, stream, "paged_copy_blocks check");
    if (st == PKV_OK) st = check_ids("paged_copy_blocks", "block_mapping src", pairs, 2, 0, pool.num_blocks, false);
    if (st == PKV_OK) st = check_ids("paged_copy_blocks", "block_mapping dst", pairs, 2, 1, pool.num_blocks, true);
    if (st != PKV_OK) return st;
    std::vector<int32_t> srcs;
    for (int32_t i = 0; i < num_pairs; ++i) srcs.push_back(pairs[2 * i]);
    std::sort(srcs.begin(), srcs.end());
    for (int32_t i = 0; i < num_pairs; ++i)
      if (std::binary_search(srcs.begin(), srcs.end(), pairs[2 * i + 1]))
        return fail(PKV_ECHECK, "paged_copy_blocks: block %d is both a destination and a source",
                    pairs[2 * i + 1]);
  }
  hipError_t err = pkv::launch_copy_blocks(k_cache, v_cache, block_mapping, num_pairs,
                                           pool_block_bytes(pool), pool.num_blocks, stream);
  return err == hipSuccess ? PKV_OK : hip_fail(err, "paged_copy_blocks launch");
}

namespace {

// Shared checks of the two swap directions; *per_run = blocks per staging run.
pkv_status swap_check(const char* what, const void* k_cache, const void* v_cache,
                      const pkv_pool& pool, const int32_t* block_ids, int32_t num_ids,
                      const void* host_image, const void* staging, size_t staging_bytes,
                      int32_t* per_run) {
  pkv_status st = check_pool(pool);
  if (st != PKV_OK) return st;
  if (num_ids < 0) return fail(PKV_EINVAL, "%s: num_ids %d < 0", what, num_ids);
  if (num_ids == 0) return PKV_OK;
  if (!k_cache || !v_cache || !block_ids || !host_image || !staging)
    return fail(PKV_EINVAL, "%s: null pointer argument", what);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(staging))
    return fail(PKV_EINVAL, "%s: pools and staging must be 16-byte aligned", what);
  const size_t entry = 2 * pool_block_bytes(pool);
  if (staging_bytes < entry)
    return fail(PKV_EWORKSPACE, "%s: staging holds %zu bytes, one block needs %zu", what,
                staging_bytes, entry);
  const size_t run = staging_bytes / entry;
  *per_run = run > 0x3fffffff ? 0x3fffffff : (int32_t)run;
  return PKV_OK;
}

}  // namespace

pkv_status paged_swap_out(const void* k_cache, const void* v_cache, pkv_pool pool,
                          const int32_t* block_ids, int32_t num_ids, void* host_image,
                          void* staging, size_t staging_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  int32_t per_run = 0;
  pkv_status st = swap_check("paged_swap_out", k_cache, v_cache, pool, block_ids, num_ids,
                             host_image, staging, staging_bytes, &per_run);
  if (st != PKV_OK || num_ids == 0) return st;
  if (check_mode()) {
    std::vector<int32_t> ids;
    st = fetch_i32(ids, block_ids, (size_t)num_ids, stream, "paged_swap_out check");
    if (st == PKV_OK) st = check_ids("paged_swap_out", "block_ids", ids, 1, 0, pool.num_blocks, true);
    if (st != PKV_OK) return st;
  }
  const size_t bb = pool_block_bytes(pool);
  for (int32_t start = 0; start < num_ids; start += per_run) {
    const int32_t cnt = num_ids - start < per_run ? num_ids - start : per_run;
    hipError_t err = pkv::launch_swap_gather(k_cache, v_cache, block_ids + start, cnt, staging, bb,
                                             pool.num_blocks, stream);
    if (err != hipSuccess) return hip_fail(err, "paged_swap_out gather launch");
    err = hipMemcpyAsync(static_cast<char*>(host_image) + (size_t)start * 2 * bb, staging,
                         (size_t)cnt * 2 * bb, hipMemcpyDeviceToHost, stream);
    if (err != hipSuccess) return hip_fail(err, "paged_swap_out copy to host");
  }
  return PKV_OK;
}

pkv_status paged_swap_in(const void* host_image, int32_t num_ids, void* k_cache, void* v_cache,
                         pkv_pool pool, const int32_t* block_ids, void* staging,
                         size_t staging_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  int32_t per_run = 0;
  pkv_status st = swap_check("paged_swap_in", k_cache, v_cache, pool, block_ids, num_ids,
                             host_image, staging, staging_bytes, &per_run);
  if (st != PKV_OK || num_ids == 0) return st;
  if (check_mode()) {
    std::vector<int32_t> ids;
    st = fetch_i32(ids, block_ids, (size_t)num_ids, stream, "paged_swap_in check");
    if (st == PKV_OK) st = check_ids("paged_swap_in", "block_ids", ids, 1, 0, pool.num_blocks, true);
    if (st != PKV_OK) return st;
  }
  const size_t bb = pool_block_bytes(pool);
  for (int32_t start = 0; start < num_ids; start += per_run) {
    const int32_t cnt = num_ids - start < per_run ? num_ids - start : per_run;
    hipError_t err = hipMemcpyAsync(staging,
                                    static_cast<const char*>(host_image) + (size_t)start * 2 * bb,
                                    (size_t)cnt * 2 * bb, hipMemcpyHostToDevice, stream);
    if (err != hipSuccess) return hip_fail(err, "paged_swap_in copy from host");
    err = pkv::launch_swap_scatter(k_cache, v_cache, block_ids + start, cnt, staging, bb,
                                   pool.num_blocks, stream);
    if (err != hipSuccess) return hip_fail(err, "paged_swap_in scatter launch");
  }
  return PKV_OK;
}

pkv_status pkv_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  g_err[0] = '\0';
  if (bytes == 0) return PKV_OK;
  if (!dst || !src) return fail(PKV_EINVAL, "null pointer argument");
  if (!aligned16(dst) || !aligned16(src) || (bytes & 15u))
    return fail(PKV_EINVAL, "pointers and byte count must be multiples of 16");
  hipError_t err = pkv::launch_stream_copy(dst, src, bytes, stream);
  return err == hipSuccess ? PKV_OK : hip_fail(err, "pkv_stream_copy launch");
}

pkv_status pkv_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  g_err[0] = '\0';
  if (bytes == 0) return PKV_OK;
  if (!src || !sink) return fail(PKV_EINVAL, "null pointer argument");
  if (!aligned16(src) || (bytes & 15u))
    return fail(PKV_EINVAL, "src and byte count must be multiples of 16");
  hipError_t err = pkv::launch_stream_read(src, bytes, sink, stream);
  return err == hipSuccess ? PKV_OK : hip_fail(err, "pkv_stream_read launch");
}

pkv_status pkv_stream_reread(const void* src, size_t bytes, int32_t rounds, uint32_t* sink,
                             hipStream_t stream) {
  g_err[0] = '\0';
  if (rounds < 0) return fail(PKV_EINVAL, "rounds %d < 0", rounds);
  if (bytes == 0 || rounds == 0) return PKV_OK;
  if (!src || !sink) return fail(PKV_EINVAL, "null pointer argument");
  if (!aligned16(src) || (bytes & 15u))
    return fail(PKV_EINVAL, "src and byte count must be multiples of 16");
  hipError_t err = pkv::launch_stream_reread(src, bytes, rounds, sink, stream);
  return err == hipSuccess ? PKV_OK : hip_fail(err, "pkv_stream_reread launch");
}

}  // extern "C"
