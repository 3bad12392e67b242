// Cache writes for gfx950: append of new tokens into their slots, copy-on-write
// block duplication, and a plain streaming copy used as a bandwidth and
// counter reference.  All three are raw 16-byte bit copies.
//
// Append: a sequence's newest tokens go into free slots of its blocks as they
// arrive ("Optimizing LLM Inference: From PagedAttention to AI Infra", section
// "On-Demand Allocation"; "The Memory Wall", "How it Works Under the Hood").
// The slot encodes block * block_size + offset.
// Copy: a writer to a shared block first gets a private copy while the shared
// block stays unchanged ("05 PagedAttention", "KV Cache Sharing
// (Copy-on-Write)"; first page, "Copy-on-Write").
// Swap: when the pool runs short, blocks move to CPU RAM and come back later
// ("The Memory Wall", "The Infrastructure Impact: Scale and Complexity", item
// "The Block Manager"; "05 PagedAttention", "Managing Virtual Memory (Block
// Manager)").  A gather packs the listed blocks into a contiguous device
// staging run so that one DMA copy moves the run over PCIe; a scatter unpacks
// a run copied back.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;

// One thread per 16-byte chunk of one token's [H_kv, D] row, for K and V.
// Consecutive threads cover consecutive chunks of a head, so reads of the
// input rows are fully coalesced and each (head, slot) destination row of
// D * elem_bytes bytes is written contiguously.
__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    const uint4* __restrict__ key, const uint4* __restrict__ value, char* __restrict__ k_cache,
    char* __restrict__ v_cache, const int32_t* __restrict__ slot_mapping, int32_t num_tokens,
    int32_t chunks_per_head, int32_t num_kv_heads, int32_t block_size, int64_t num_slots) {
  const int64_t per_token = (int64_t)chunks_per_head * num_kv_heads;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (gid >= per_token * num_tokens) return;
  const int64_t i = gid / per_token;
  const int64_t rem = gid - i * per_token;
  const int32_t slot = slot_mapping[i];
  if (slot < 0 || (int64_t)slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int64_t off = slot - blk * block_size;
  const int64_t h = rem / chunks_per_head;
  const int64_t c = rem - h * chunks_per_head;
  const int64_t dst = (((blk * num_kv_heads + h) * block_size + off) * chunks_per_head + c) * 16;
  reinterpret_cast<uint4*>(k_cache + dst)[0] = key[gid];
  reinterpret_cast<uint4*>(v_cache + dst)[0] = value[gid];
}

// One workgroup per (pair, K or V): copies a whole block of every KV head.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    char* __restrict__ k_cache, char* __restrict__ v_cache, const int32_t* __restrict__ block_mapping,
    int64_t block_chunks, int32_t num_blocks) {
  const int pair = blockIdx.x >> 1;
  char* pool = (blockIdx.x & 1) ? v_cache : k_cache;
  const int32_t src = block_mapping[2 * pair];
  const int32_t dst = block_mapping[2 * pair + 1];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
  const uint4* from = reinterpret_cast<const uint4*>(pool + (int64_t)src * block_chunks * 16);
  uint4* to = reinterpret_cast<uint4*>(pool + (int64_t)dst * block_chunks * 16);
  for (int64_t c = threadIdx.x; c < block_chunks; c += kThreads) to[c] = from[c];
}

// Swap gather: workgroup (i, K or V) copies block ids[i]'s tile of every KV
// head into staging entry 2i (K) or 2i+1 (V).  An id outside the pool gives a
// zero entry.  Both sides are contiguous runs of tile_chunks 16-byte chunks.
__global__ __launch_bounds__(kThreads) void swap_gather_kernel(
    const char* __restrict__ k_cache, const char* __restrict__ v_cache,
    const int32_t* __restrict__ ids, uint4* __restrict__ staging, int64_t tile_chunks,
    int32_t num_blocks) {
  const int i = blockIdx.x >> 1;
  const char* pool = (blockIdx.x & 1) ? v_cache : k_cache;
  const int32_t b = ids[i];
  uint4* to = staging + (int64_t)blockIdx.x * tile_chunks;
  if ((unsigned)b >= (unsigned)num_blocks) {
    for (int64_t c = threadIdx.x; c < tile_chunks; c += kThreads) to[c] = make_uint4(0, 0, 0, 0);
    return;
  }
  const uint4* from = reinterpret_cast<const uint4*>(pool + (int64_t)b * tile_chunks * 16);
  for (int64_t c = threadIdx.x; c < tile_chunks; c += kThreads) to[c] = from[c];
}

// Swap scatter: the reverse; an id outside the pool is skipped.
__global__ __launch_bounds__(kThreads) void swap_scatter_kernel(
    char* __restrict__ k_cache, char* __restrict__ v_cache, const int32_t* __restrict__ ids,
    const uint4* __restrict__ staging, int64_t tile_chunks, int32_t num_blocks) {
  const int i = blockIdx.x >> 1;
  char* pool = (blockIdx.x & 1) ? v_cache : k_cache;
  const int32_t b = ids[i];
  if ((unsigned)b >= (unsigned)num_blocks) return;
  const uint4* from = staging + (int64_t)blockIdx.x * tile_chunks;
  uint4* to = reinterpret_cast<uint4*>(pool + (int64_t)b * tile_chunks * 16);
  for (int64_t c = threadIdx.x; c < tile_chunks; c += kThreads) to[c] = from[c];
}

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(uint4* __restrict__ dst,
                                                               const uint4* __restrict__ src,
                                                               int64_t chunks) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < chunks; c += stride)
    dst[c] = src[c];
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// XOR-fold of the 16-byte chunks [begin, end) of src read by this workgroup
// with nontemporal loads (the attention kernels' policy), eight in flight per
// thread.
__device__ __forceinline__ void fold_range(u32x4& acc, const u32x4* __restrict__ src,
                                           int64_t begin, int64_t end) {
  int64_t c = begin + threadIdx.x;
  for (; c + 7 * kThreads < end; c += 8 * kThreads) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + c + u * kThreads);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; c < end; c += kThreads) acc ^= __builtin_nontemporal_load(src + c);
}

// One word per workgroup, so the loads cannot be dropped.
__device__ __forceinline__ void write_fold(const u32x4& acc, uint32_t* __restrict__ sink) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Read-only stream: workgroup b reads the contiguous range
// [b * per_wg, (b + 1) * per_wg) of 16-byte chunks once.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                               int64_t chunks, int64_t per_wg,
                                                               uint32_t* __restrict__ sink) {
  const int64_t begin = (int64_t)blockIdx.x * per_wg;
  u32x4 acc = {0u, 0u, 0u, 0u};
  fold_range(acc, src, begin, begin + per_wg < chunks ? begin + per_wg : chunks);
  write_fold(acc, sink);
}

// Re-read: the buffer is cut into gridDim.x ranges and in round r workgroup b
// reads range (b + 8 r) mod gridDim.x, so every round reads each range once.
// Workgroups go to the 8 XCDs round-robin (XCD b mod 8), so an XCD only ever
// reads the ranges of its own residue class: a buffer of up to 8 L2s stays in
// the XCDs' L2s, a larger one is served from the Infinity Cache (or HBM).
// Consecutive rounds of one workgroup read different ranges, so the compute
// unit's own L1 does not serve them.
__global__ __launch_bounds__(kThreads) void stream_reread_kernel(const u32x4* __restrict__ src,
                                                                 int64_t chunks, int64_t per_wg,
                                                                 int32_t rounds,
                                                                 uint32_t* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int32_t r = 0; r < rounds; ++r) {
    const int64_t rng = ((int64_t)blockIdx.x + 8LL * r) % gridDim.x;
    const int64_t begin = rng * per_wg;
    fold_range(acc, src, begin, begin + per_wg < chunks ? begin + per_wg : chunks);
  }
  write_fold(acc, sink);
}

}  // namespace

hipError_t launch_kv_append(const void* key, const void* value, void* k_cache, void* v_cache,
                            const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                            int32_t block_size, int32_t head_dim, int32_t elem_bytes,
                            int32_t num_blocks, hipStream_t stream) {
  if (num_tokens <= 0) return hipSuccess;
  const int32_t chunks_per_head = head_dim * elem_bytes / 16;
  const int64_t total = (int64_t)chunks_per_head * num_kv_heads * num_tokens;
  const int64_t nwg = (total + kThreads - 1) / kThreads;
  if (nwg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache), slot_mapping,
                     num_tokens, chunks_per_head, num_kv_heads, block_size,
                     (int64_t)num_blocks * block_size);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                              int32_t num_pairs, size_t block_bytes, int32_t num_blocks,
                              hipStream_t stream) {
  if (num_pairs <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs * 2u), dim3(kThreads), 0, stream,
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache), block_mapping,
                     (int64_t)(block_bytes / 16), num_blocks);
  return hipGetLastError();
}

hipError_t launch_swap_gather(const void* k_cache, const void* v_cache, const int32_t* ids,
                              int32_t count, void* staging, size_t block_bytes, int32_t num_blocks,
                              hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(swap_gather_kernel, dim3((unsigned)count * 2u), dim3(kThreads), 0, stream,
                     static_cast<const char*>(k_cache), static_cast<const char*>(v_cache), ids,
                     static_cast<uint4*>(staging), (int64_t)(block_bytes / 16), num_blocks);
  return hipGetLastError();
}

hipError_t launch_swap_scatter(void* k_cache, void* v_cache, const int32_t* ids, int32_t count,
                               const void* staging, size_t block_bytes, int32_t num_blocks,
                               hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(swap_scatter_kernel, dim3((unsigned)count * 2u), dim3(kThreads), 0, stream,
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache), ids,
                     static_cast<const uint4*>(staging), (int64_t)(block_bytes / 16), num_blocks);
  return hipGetLastError();
}

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const int64_t chunks = (int64_t)(bytes / 16);
  if (chunks == 0) return hipSuccess;
  int64_t nwg = (chunks + kThreads - 1) / kThreads;
  if (nwg > 256 * 64) nwg = 256 * 64;  // grid-stride beyond 64 workgroups per CU
  hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)nwg), dim3(kThreads), 0, stream,
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), chunks);
  return hipGetLastError();
}

}  // namespace pkv

namespace pkv {

hipError_t launch_stream_reread(const void* src, size_t bytes, int32_t rounds, uint32_t* sink,
                                hipStream_t stream) {
  const int64_t chunks = (int64_t)(bytes / 16);
  if (chunks == 0 || rounds <= 0) return hipSuccess;
  const int64_t per_wg = (chunks + kStreamReadWorkgroups - 1) / kStreamReadWorkgroups;
  hipLaunchKernelGGL(stream_reread_kernel, dim3(kStreamReadWorkgroups), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), chunks, per_wg, rounds, sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  const int64_t chunks = (int64_t)(bytes / 16);
  if (chunks == 0) return hipSuccess;
  const int64_t per_wg = (chunks + kStreamReadWorkgroups - 1) / kStreamReadWorkgroups;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadWorkgroups), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(src), chunks, per_wg, sink);
  return hipGetLastError();
}

}  // namespace pkv
