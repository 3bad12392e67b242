// Internal launch interface between the C ABI (pagedkv_api.cpp) and the HIP
// kernels.  Not installed; the public interface is include/pagedkv.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace pkv {

// Tokens per split-context partition.  A multiple of every supported block
// size, so partitions start on block boundaries.
constexpr int kPartitionTokens = 512;

struct AttnParams {
  void* out;                    // [B, H_q, D] pool dtype
  float* part_o;                // [B, H_q, P, D] fp32 unnormalised partition outputs
  float* part_ml;               // [B, H_q, P, 2] fp32 (max logit in log2 units, normaliser)
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
  int32_t max_partitions;       // ceil(max_context_len / kPartitionTokens), >= 1
  float scale_log2;             // scale * log2(e): logits kept in base-2 units
};

// Largest batch the persistent attention kernel takes (its work list lives in
// LDS); larger batches use the grid kernel.
constexpr int kMaxPersistentSeqs = 2048;

// dtype: 0 f32, 1 f16, 2 bf16.  persistent_wgs: workgroups of the persistent
// kernel (a multiple of 8), or 0 for the grid kernel.  Returns
// hipErrorInvalidValue for a (dtype, head_dim, block_size) combination that
// is not instantiated.
hipError_t launch_paged_attention(const AttnParams& p, int dtype, int head_dim,
                                  int block_size, int persistent_wgs, hipStream_t stream);

hipError_t launch_kv_append(const void* key, const void* value, void* k_cache,
                            void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                            int32_t num_kv_heads, int32_t block_size, int32_t head_dim,
                            int32_t elem_bytes, int32_t num_blocks, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                              int32_t num_pairs, size_t block_bytes, int32_t num_blocks,
                              hipStream_t stream);

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

// sink: kStreamReadWorkgroups uint32 words, one per workgroup.
constexpr int kStreamReadWorkgroups = 256 * 8;
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace pkv
