// Internal launch interface between the C ABI (pagedkv_api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/pagedkv.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace pkv {

// Tokens per MFMA sub-tile: the unit of work of the decode kernels.
constexpr int kSubTokens = 16;

// ---- stream path (default) -------------------------------------------------
// Workgroups of 4 independent waves, two per compute unit.  The work of one
// call is the ordered list of (kv head, sequence, 16-token sub-tile)
// positions; wave v of the grid takes positions [v * chunk, (v + 1) * chunk),
// so a workgroup holds 4 consecutive chunks.  A wave writes a whole sequence
// it covers straight to `out`; the pieces of a sequence cut by chunk
// boundaries are merged inside the workgroup at its end, and what crosses a
// workgroup boundary goes to one of the workgroup's two partial slots,
// merged afterwards in logical order.
constexpr int kStreamWaves = 4;           // waves per workgroup
constexpr int kMaxStreamSeqs = 4096;      // batch limit (per-sequence tables live in LDS)
constexpr int kMinChunk = 4;              // sub-tiles per wave at least
constexpr int kMaxMultiSeqs = 2048;       // batch limit with several new tokens per sequence
// Multi-token calls with at least this many columns (max_query_len * G) per
// sequence take the prefill path.
constexpr int kPrefillMinCols = 64;
// Column groups of 16 per wave on the prefill path: two (16-bit types only;
// each K/V operand a wave reads from LDS serves both, two workgroups per
// compute unit) or one (three workgroups per compute unit).  A workgroup
// (column block) takes kStreamWaves times as many.
// Up to this many sequences the prefill path dispatches them longest context
// first (each workgroup ranks the context lengths itself).
constexpr int kPrefillRankSeqs = 256;
// The prefill path splits contexts when a call has fewer than this many
// (sequence, kv head, column block) workgroups, into at most kPrefillMaxParts
// parts of at least kPrefillMinPartTokens tokens.  (512: one workgroup per
// slot of the chip at two per compute unit.)
constexpr int kPrefillMinWorkgroups = 512;
constexpr int kPrefillMaxParts = 16;
constexpr int kPrefillMinPartTokens = 512;
// Positions (H_kv x sub-tiles of the batch) the stream path indexes in 32 bits;
// the host sends calls whose bound B * ceil(max_ctx / 16) * H_kv exceeds it to
// the grid path.
constexpr int kMaxStreamPositions = 1 << 28;

// ---- grid path (batches above kMaxStreamSeqs) --------------------------------
// One workgroup per (kv head, sequence, partition of kPartitionTokens tokens).
constexpr int kPartitionTokens = 512;

struct AttnParams {
  void* out;                    // [B, H_q, D] pool dtype
  const void* q;                // [B, H_q, D]
  const void* k_cache;          // [NB, H_kv, bs, D]
  const void* v_cache;
  const int32_t* block_tables;  // [B, max_blocks_per_seq]
  const int32_t* context_lens;  // [B]
  int32_t max_blocks_per_seq;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;                // H_q / H_kv
  int32_t num_blocks;
  int32_t max_context_len;
  float scale_log2;             // scale * log2(e): logits kept in base-2 units
  // Workspace views.  Stream path: seq_prefix [B + 1] (sub-tiles of the
  // sequences before each one), part_o [2 * workgroups + waves, slot_cols, D]
  // (two partial slots per workgroup, then a parking row per wave), part_ml
  // [same rows, slot_cols, 2] (max logit in log2 units, normaliser).  Grid path:
  // part_o [B, H_q, P, D], part_ml [B, H_q, P, 2]; seq_prefix unused.
  int32_t* seq_prefix;
  float* part_o;
  float* part_ml;
  int32_t stream_wgs;           // > 0: stream path with this many workgroups
  int32_t max_partitions;       // grid path: ceil(max_context_len / kPartitionTokens)
  // Several new tokens per sequence (stream path only).  query_start [B+1]
  // device prefix of query rows, or nullptr for decode (row s = sequence s).
  // Columns of a sequence: (new token, query head) pairs in groups of 16.
  const int32_t* query_start;
  int32_t num_query_tokens;     // rows of q / out
  int32_t max_query_len;        // host-known bound of the new tokens per sequence
  int32_t max_groups;           // ceil(max_query_len * G / 16)
  int32_t slot_cols;            // columns per partial slot: min(16, max_query_len * G)
  // > 0: prefill path, this many column blocks per (sequence, kv head), each
  // taking four 16-column groups (ceil(max_groups / 4)).
  int32_t prefill_blocks;
  // Prefill path: the context of each (sequence, kv head, column block) is
  // cut into this many stage-aligned parts, one workgroup each.  With more
  // than one, part states go to part_o [rows * H_q * parts, D] and part_ml
  // [rows * H_q * parts, 2] (row = query row) and a merge writes `out`.
  int32_t prefill_parts;
  // Prefill path: column groups per wave (1 or 2; see prefill_plan).
  int32_t prefill_wave_groups;
  // Decode on the stream path, measurement variant: 1 = K loaded straight in
  // the MFMA operand order instead of whole lines re-dealt through LDS
  // (built for bf16, D 128, 16-token blocks only; ignored elsewhere).
  int32_t k_direct;
  // Measurement only: when non-null, the clock build of the kernel (bf16,
  // D 128, 16-token blocks) records kClockWords words per wave (stream
  // decode: record wave index) or per workgroup (prefill: record linear
  // block id), up to kClockRecords records; see pkv_clock_read.
  unsigned long long* clock;
};

constexpr int kClockRecords = 32768;
constexpr int kClockWords = 4;

// Workspace layout of one decode call, shared by the size query and the call.
struct AttnWorkspace {
  size_t prefix_off, part_o_off, part_ml_off, bytes;
};
// slot_cols: columns per partial slot (min(16, max_query_len * G)).
AttnWorkspace attn_workspace_layout(int32_t num_seqs, int32_t slot_cols, int32_t num_q_heads,
                                    int32_t head_dim, int32_t max_context_len, int32_t stream_wgs);
// Prefill path: parts per (sequence, kv head, column block), and the
// workspace of the part states (0 bytes with one part).
int32_t prefill_parts_for(int32_t num_seqs, int32_t num_kv_heads, int32_t prefill_blocks,
                          int32_t max_context_len);
// Launch plan of a prefill-path call (max_groups 16-column groups per
// sequence and kv head; dtype 0 f32, 1 f16, 2 bf16): column groups per wave,
// column blocks (workgroups) per (sequence, kv head) and context parts.  Two
// groups per wave where the call is cut into equal parts or has at least two
// workgroups per slot of the chip; otherwise one, whose twice as many
// smaller workgroups balance unequal contexts better.
struct PrefillPlan {
  int32_t wave_groups, blocks, parts;
};
PrefillPlan prefill_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t max_groups,
                         int32_t max_context_len, int dtype);
AttnWorkspace prefill_workspace_layout(int32_t num_query_tokens, int32_t num_q_heads,
                                       int32_t head_dim, int32_t parts);

// dtype: 0 f32, 1 f16, 2 bf16.  Returns hipErrorInvalidValue for a (dtype,
// head_dim, block_size) combination that is not instantiated.  Calls with
// prefill_blocks > 0 go to launch_prefill.
hipError_t launch_paged_attention(const AttnParams& p, int dtype, int head_dim,
                                  int block_size, hipStream_t stream);
// The prefill path (prefill.hip).
hipError_t launch_prefill(const AttnParams& p, int dtype, int head_dim, int block_size,
                          hipStream_t stream);

hipError_t launch_kv_append(const void* key, const void* value, void* k_cache,
                            void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                            int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                            int32_t elem_bytes, int32_t num_blocks, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                              int32_t num_pairs, size_t block_bytes, int32_t num_blocks,
                              hipStream_t stream);

// Swap staging: entry 2i / 2i+1 of `staging` is block ids[i]'s K / V tile
// (block_bytes each, every KV head).
hipError_t launch_swap_gather(const void* k_cache, const void* v_cache, const int32_t* ids,
                              int32_t count, void* staging, size_t block_bytes, int32_t num_blocks,
                              hipStream_t stream);
hipError_t launch_swap_scatter(void* k_cache, void* v_cache, const int32_t* ids, int32_t count,
                               const void* staging, size_t block_bytes, int32_t num_blocks,
                               hipStream_t stream);
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

// sink: kStreamReadWorkgroups uint32 words, one per workgroup.
constexpr int kStreamReadWorkgroups = 256 * 8;
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_stream_reread(const void* src, size_t bytes, int32_t rounds, uint32_t* sink,
                                hipStream_t stream);

}  // namespace pkv
