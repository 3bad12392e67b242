/*
 * libpagedkv — paged KV-cache decode for AMD Instinct MI355X (gfx950).
 *
 * The KV cache of one attention layer lives in a shared pool of fixed-size
 * physical blocks; each sequence owns a block table that maps its logical
 * blocks to physical ones, so its context is contiguous logically but
 * scattered physically.  Sources: "Optimizing LLM Inference: From
 * PagedAttention to AI Infra" (sections "PagedAttention: Decoupling Logical
 * Context from Contiguous GPU Memory", "On-Demand Allocation", "Copy-on-Write");
 * "The Memory Wall" (sections "How it Works Under the Hood", "Show Me The
 * Code: A Conceptual PagedAttention Kernel"); "05 PagedAttention" (sections
 * "How PagedAttention Works (vLLM)", "KV Cache Sharing (Copy-on-Write)").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pool layout, K and V alike: [num_blocks, num_kv_heads, block_size,
 *    head_dim], row-major, elements of the pool's dtype.  One (block, head)
 *    tile of block_size x head_dim elements is contiguous.
 *  - dtype is one of pkv_dtype; every tensor passed to one call shares it.
 *  - All pointers are DEVICE pointers owned by the caller.  The library
 *    allocates and frees nothing.  Pointers must be 16-byte aligned.
 *  - Calls are asynchronous on `stream` (0 = the null stream): they validate
 *    their scalar arguments on the host, enqueue kernels and return.  Inputs
 *    must stay valid and unmodified until the stream reaches the work.
 *  - Host-side validation failures return PKV_EINVAL / PKV_EUNSUPPORTED and
 *    enqueue nothing; a failed launch returns PKV_EHIP.  pkv_last_error()
 *    then holds a message (per calling thread).
 *  - Device-side metadata (block ids, context lengths, slots) is trusted for
 *    correctness but never for memory safety: a block id or slot outside the
 *    pool is never dereferenced, and a context length is clamped to
 *    [0, max_context_len].
 *  - Thread safety: the library keeps no mutable global state apart from the
 *    per-thread error message.  Calls on different streams may overlap.
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_API __attribute__((visibility("default")))

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* bad pointer, shape or scalar argument */
  PKV_EUNSUPPORTED = 2,  /* valid but not built: head_dim, block_size, dtype, group */
  PKV_EWORKSPACE = 3,    /* workspace missing or smaller than required */
  PKV_EHIP = 4,          /* a HIP runtime call or kernel launch failed */
  PKV_ECHECK = 5         /* metadata check failed (PAGEDKV_CHECK=1, see below) */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2 } pkv_dtype;

/*
 * Metadata check mode.  Device metadata (block tables, context lengths,
 * query starts, slots, copy pairs, swap ids) is trusted: a bad entry never
 * moves an access outside its buffer, but the result is then undefined.
 * With the environment variable PAGEDKV_CHECK=1 every entry point first
 * copies its metadata to the host on its stream, waits for it, and returns
 * PKV_ECHECK (nothing enqueued, pkv_last_error naming the entry) for:
 *  - attention: context_lens[s] outside [0, max_context_len]; a block id a
 *    context uses (entries j < ceil(n / block_size)) outside the pool;
 *    query_start not starting at 0, not ending at num_query_tokens, or
 *    giving a sequence a negative count of new tokens or more than
 *    min(n, max_query_len);
 *  - paged_kv_append: a slot at or past num_blocks * block_size, or one slot
 *    written twice (negative slots are skipped);
 *  - paged_copy_blocks: a block id outside the pool, a destination named
 *    twice, or a destination that is also a source;
 *  - swaps: a block id outside the pool or named twice.
 * Debug only: the wait costs a round trip per call, and under stream
 * capture (where waiting is not allowed) the calls return PKV_EUNSUPPORTED.
 */

/* Shape of the K and V pools (they share it). */
typedef struct {
  int32_t num_blocks;    /* physical blocks in the pool, > 0 */
  int32_t num_kv_heads;  /* H_kv, > 0 */
  int32_t block_size;    /* tokens per block: 16 or 32 */
  int32_t head_dim;      /* D: 64 or 128 */
  int32_t dtype;         /* pkv_dtype */
} pkv_pool;

/* Tokens per split-context partition of paged_attention_decode for batches
 * above 4096 sequences (512); smaller batches split at 16-token granularity. */
PKV_API int32_t pkv_partition_tokens(void);

/*
 * paged_kv_append — write new tokens' K and V into their cache slots
 * ("On-Demand Allocation" on the first page: a sequence's newest tokens go
 * into the next free slots of its blocks; "How it Works Under the Hood" on
 * "The Memory Wall": the model writes a logically contiguous sequence).
 *
 *   key, value    [num_tokens, num_kv_heads, head_dim]  contiguous, pool dtype
 *   k_cache, v_cache  pools (see above), written in place
 *   slot_mapping  [num_tokens] int32: slot = physical_block * block_size + offset;
 *                 a negative slot or one >= num_blocks * block_size is skipped.
 *                 Two tokens naming the same slot in one call race (undefined).
 *   num_tokens    >= 0 (0 enqueues nothing)
 * Every element is a raw bit copy.  Returns PKV_OK once enqueued.
 */
PKV_API pkv_status paged_kv_append(const void* key, const void* value,
                                   void* k_cache, void* v_cache, pkv_pool pool,
                                   const int32_t* slot_mapping, int32_t num_tokens,
                                   hipStream_t stream);

/*
 * Bytes of workspace paged_attention_decode needs for this shape on the
 * current device (the kernel's grid follows the device's compute-unit count):
 * per-sequence sub-tile offsets and fp32 partial softmax states of the
 * sequences whose context is split between waves.  Query it on the device
 * the call will run on.  Up to 4096 sequences (the stream path) the size is
 * independent of the context lengths, and non-zero even for short contexts:
 * every workgroup has two partial-state slots and every wave a parking row,
 * (2 * workgroups + waves) * min(16, G) rows of head_dim + 2 floats, plus
 * num_seqs + 1 int32 offsets.  Above 4096 sequences (the grid path) it is
 * num_seqs * num_q_heads * ceil(max_context_len / 512) * (head_dim + 2)
 * floats, and 0 when max_context_len <= 512.  Returns 0 for invalid input
 * (including num_q_heads not a multiple of pool.num_kv_heads).
 *
 * Measurement switch: with PAGEDKV_DECODE_PATH=grid in the environment,
 * every decode call and this query take the grid path (one workgroup per
 * (kv head, sequence, 512-token partition), then the partition merge)
 * whatever the batch.  Read on every call; the query and the call must see
 * the same setting.  PAGEDKV_K_LOAD=direct, likewise for measurement only:
 * stream-path decode calls of one shape (bf16, head_dim 128, block_size 16)
 * load K straight in the matrix-core operand order instead of whole
 * 128-byte lines re-dealt through LDS; the result is the same bit for bit.
 */
PKV_API size_t paged_attention_workspace_bytes(pkv_pool pool, int32_t num_seqs,
                                               int32_t num_q_heads, int32_t max_context_len);

/*
 * paged_attention_decode — one query token per sequence attends to its whole
 * cached context, gathered block by block through its block table (first
 * page, "PagedAttention: Decoupling Logical Context from Contiguous GPU
 * Memory"; "The Memory Wall", "Show Me The Code: A Conceptual PagedAttention
 * Kernel").  For sequence s and query head h, with n = context_lens[s] and
 * G = num_q_heads / num_kv_heads, query head h reads KV head h / G:
 *
 *     out[s, h, :] = softmax_t(scale * q[s, h, :] . K_s[h/G, t, :]) @ V_s[h/G, t, :]
 *
 * over logical tokens t < n; token t lives in physical block
 * block_tables[s, t / block_size] at offset t % block_size.  n = 0 gives a
 * zero row.  Softmax and accumulation are fp32; out is rounded to nearest
 * even in the pool dtype.  The context is cut into 16-token sub-tiles and
 * the call's sub-tiles into equal chunks, one per wave of the kernel; where a
 * sequence's context spans several chunks, their partial states (running
 * max, normaliser, unnormalised output) are merged exactly by a log-sum-exp
 * rescale.  The chunk boundaries depend only on the context lengths and the
 * device's compute-unit count, and every reduction runs in logical token
 * order, so the result is bit-identical under any physical placement of the
 * blocks and across repeated calls.  A block id
 * outside the pool is never dereferenced (its tokens read as zeros).
 *
 *   out           [num_seqs, num_q_heads, head_dim]  pool dtype, written
 *   q             [num_seqs, num_q_heads, head_dim]  pool dtype
 *   k_cache, v_cache  pools, read only
 *   block_tables  [num_seqs, max_blocks_per_seq] int32; entries at
 *                 j >= ceil(n / block_size) are never read
 *   context_lens  [num_seqs] int32, each <= max_context_len
 *   num_q_heads   multiple of num_kv_heads, with G = num_q_heads/num_kv_heads <= 16
 *   scale         logit scale, usually 1/sqrt(head_dim)
 *   max_context_len  host-known upper bound of context_lens (no device read);
 *                 max_blocks_per_seq * block_size must be >= it
 *   workspace     device buffer of >= paged_attention_workspace_bytes(pool,
 *                 num_seqs, num_q_heads, max_context_len) bytes, 16-byte
 *                 aligned (may be NULL when that is 0); scratch, needs no
 *                 initialisation.  Calls that can run concurrently must not
 *                 share it.
 */
PKV_API pkv_status paged_attention_decode(void* out, const void* q,
                                          const void* k_cache, const void* v_cache,
                                          pkv_pool pool,
                                          const int32_t* block_tables,
                                          int32_t max_blocks_per_seq,
                                          const int32_t* context_lens,
                                          int32_t num_seqs, int32_t num_q_heads,
                                          float scale, int32_t max_context_len,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/*
 * paged_attention_decode_noalloc — paged_attention_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same computation, kernels and
 * result, bit for bit, with the workspace taken from a scratch array the
 * library holds in device memory, one per GPU, for the life of the process
 * (paged_attention_noalloc_max_bytes() bytes, 32 MiB).  The caller passes
 * only inputs and outputs; the arguments mean what they mean for
 * paged_attention_decode.  The call allocates nothing: no hipMalloc, no
 * hipFree, no allocating library routine (its first call on a device looks
 * up that device's copy of the array once).
 *  - A call whose workspace (paged_attention_workspace_bytes of the same
 *    shape) exceeds the scratch returns PKV_EWORKSPACE and enqueues nothing.
 *    Every decode on the stream path fits (at most 25.6 MB on a 256-CU
 *    device, at G = 16 and D = 128); a grid-path call above 4096 sequences
 *    with long contexts may not.
 *  - All calls on one GPU share its scratch, and the workspace needs no
 *    initialisation: calls that overlap on one GPU (different streams or
 *    threads with no ordering between them) race and give undefined
 *    results.  Calls ordered on one stream are safe.
 *  - Under PAGEDKV_CHECK=1 it returns PKV_EUNSUPPORTED: the metadata check
 *    copies to host buffers and waits.
 */
PKV_API pkv_status paged_attention_decode_noalloc(void* out, const void* q,
                                                  const void* k_cache, const void* v_cache,
                                                  pkv_pool pool,
                                                  const int32_t* block_tables,
                                                  int32_t max_blocks_per_seq,
                                                  const int32_t* context_lens,
                                                  int32_t num_seqs, int32_t num_q_heads,
                                                  float scale, int32_t max_context_len,
                                                  hipStream_t stream);
/* Bytes of the per-GPU scratch array behind paged_attention_decode_noalloc. */
PKV_API size_t paged_attention_noalloc_max_bytes(void);

/*
 * Bytes of workspace paged_attention_multi needs for this shape on the
 * current device, or 0 for invalid input, for a call it refuses, or for a
 * prefill-path call (max_query_len * G >= 64) that keeps each context whole.
 * A prefill-path call with fewer than 512 (sequence, kv head, column block)
 * workgroups cuts contexts into parts and needs room for the parts' states:
 * num_seqs * max_query_len rows are assumed.
 */
PKV_API size_t paged_attention_multi_workspace_bytes(pkv_pool pool, int32_t num_seqs,
                                                     int32_t num_q_heads, int32_t max_query_len,
                                                     int32_t max_context_len);

/*
 * paged_attention_multi — several new tokens per sequence attend to the
 * paged context at once: a chunk of a long prompt batched with other
 * requests' decode tokens (the second page, "Chunked Prefill: Don't Let Long
 * Prompts Consume the Entire Budget"), or a large model verifying a draft
 * model's guessed tokens in one pass ("The Memory Wall", "The Next Frontier:
 * Speculative Decoding and Beyond").  Sequence s has n = context_lens[s]
 * cached tokens whose last L = query_start[s+1] - query_start[s] are its new
 * ones (their K/V already appended); new token i (0 <= i < L), query row
 * query_start[s] + i, attends to logical tokens 0 .. n - L + i:
 *
 *     out[row, h, :] = softmax_t(scale * q[row, h, :] . K_s[h/G, t, :]) @ V_s[h/G, t, :],
 *                      t <= n - L + i
 *
 * With L = 1 for every sequence this is paged_attention_decode.  The MFMA
 * columns are (new token, query head) pairs in groups of 16.  Two paths:
 *  - max_query_len * G < 64 (speculative verification, mixed small chunks):
 *    the decode kernel's stream of sub-tiles, one pass over the context per
 *    column group (L * G <= 16, e.g. 4 draft tokens at G = 4, reads every
 *    K/V byte once), partial states merged afterwards; num_seqs <= 2048,
 *    at most 2^28 positions (kv heads x column groups x 16-token sub-tiles);
 *  - max_query_len * G >= 64 (prompt chunks): one workgroup per (sequence,
 *    kv head, column block) streams the context once through LDS for the
 *    block's columns and writes its rows directly; num_seqs <= 65535; up to
 *    256 sequences are dispatched longest context first.  A block is eight
 *    16-column groups (two per wave) for 16-bit types where the call has at
 *    least 1024 such workgroups or fewer than 512, else four (one per wave);
 *    fp32 always four.  When a call has fewer than 512 workgroups, each
 *    context is cut into up to 16 parts of at least 512 tokens, one
 *    workgroup each, whose states are merged in part order afterwards
 *    (workspace needed, deterministic as above).
 * Both give the same result up to fp32 rounding order.  Precision,
 * determinism and metadata trust as for paged_attention_decode; rows of a
 * sequence are clamped to [0, num_query_tokens] and to at most
 * min(n, max_query_len), so malformed query_start values never move a read
 * or write outside its buffer.
 *
 *   out, q        [num_query_tokens, num_q_heads, head_dim]  pool dtype, rows
 *                 packed sequence by sequence (no padding)
 *   query_start   [num_seqs + 1] int32 device prefix of query rows,
 *                 query_start[0] = 0, non-decreasing, last = num_query_tokens
 *   max_query_len host-known upper bound of L over the batch
 *   other arguments as for paged_attention_decode
 *   workspace     >= paged_attention_multi_workspace_bytes(...) bytes (may be
 *                 NULL when that is 0)
 */
PKV_API pkv_status paged_attention_multi(void* out, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         pkv_pool pool,
                                         const int32_t* block_tables,
                                         int32_t max_blocks_per_seq,
                                         const int32_t* context_lens,
                                         const int32_t* query_start,
                                         int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_query_tokens, int32_t max_query_len,
                                         float scale, int32_t max_context_len,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * paged_copy_blocks — copy-on-write block duplication ("05 PagedAttention",
 * "KV Cache Sharing (Copy-on-Write)": a sequence that diverges gets its own
 * copy of a shared block while the shared block stays as it was).  For each
 * pair i, block block_mapping[2i] is copied to block block_mapping[2i+1],
 * every KV head of K and of V, as raw bits.
 *
 *   block_mapping [num_pairs, 2] int32 (src, dst) on the device.  Destinations
 *                 must be distinct and no destination may be a source in the
 *                 same call (else the result depends on scheduling).  Pairs
 *                 naming a block outside the pool are skipped.
 */
PKV_API pkv_status paged_copy_blocks(void* k_cache, void* v_cache, pkv_pool pool,
                                     const int32_t* block_mapping, int32_t num_pairs,
                                     hipStream_t stream);

/*
 * paged_swap_out / paged_swap_in — move blocks to host memory and back when
 * the pool runs short ("The Memory Wall", "The Infrastructure Impact: Scale
 * and Complexity", item "The Block Manager"; "05 PagedAttention", "Managing
 * Virtual Memory (Block Manager)": inactive blocks go to CPU RAM and return
 * when needed).
 *
 *   block_ids     [num_ids] int32 on the device.  Out: the blocks to copy, in
 *                 order (an id outside the pool gives an all-zero entry).  In:
 *                 the destination of each entry; they must be distinct (else
 *                 the result depends on scheduling); an id outside the pool
 *                 is skipped.
 *   host_image    HOST memory of num_ids entries of 2 * block_bytes bytes,
 *                 block_bytes = num_kv_heads * block_size * head_dim * element
 *                 size: entry i is block_ids[i]'s K tile then its V tile, each
 *                 [num_kv_heads, block_size, head_dim] ([num_ids, 2, H_kv, bs,
 *                 D] in all).  Pinned memory (hipHostMalloc) keeps the copies
 *                 asynchronous; pageable memory works but blocks the caller.
 *   staging       DEVICE scratch of staging_bytes >= 2 * block_bytes (else
 *                 PKV_EWORKSPACE); no initialisation needed.  Blocks move in
 *                 runs of floor(staging_bytes / (2 * block_bytes)): a gather
 *                 kernel packs a run into staging and one hipMemcpyAsync
 *                 moves it to the host (paged_swap_in: the copy, then a
 *                 scatter kernel).  Larger staging, fewer and larger copies.
 *   num_ids       >= 0 (0 enqueues nothing)
 * All work is enqueued on `stream`; host_image (out) or the pools (in) are
 * complete when the stream reaches the end of it.  Raw bit copies.
 */
PKV_API pkv_status paged_swap_out(const void* k_cache, const void* v_cache, pkv_pool pool,
                                  const int32_t* block_ids, int32_t num_ids, void* host_image,
                                  void* staging, size_t staging_bytes, hipStream_t stream);
PKV_API pkv_status paged_swap_in(const void* host_image, int32_t num_ids, void* k_cache,
                                 void* v_cache, pkv_pool pool, const int32_t* block_ids,
                                 void* staging, size_t staging_bytes, hipStream_t stream);

/*
 * pkv_stream_copy — plain device-to-device copy of `bytes` bytes (a multiple
 * of 16) with 16-byte vector loads and stores.  A bandwidth and counter
 * reference for the kernels above, not part of the attention method.
 */
PKV_API pkv_status pkv_stream_copy(void* dst, const void* src, size_t bytes,
                                   hipStream_t stream);

/*
 * pkv_stream_read — read `bytes` bytes (a multiple of 16) once with 16-byte
 * vector loads; each of 2048 workgroups writes one XOR-fold word to
 * sink[0..2047] (device, caller-owned).  The achievable-read-bandwidth
 * reference for the decode kernel, not part of the attention method.
 */
PKV_API pkv_status pkv_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                   hipStream_t stream);

/*
 * pkv_stream_reread — read `bytes` bytes (a multiple of 16) `rounds` times
 * with the same loads, each XCD re-reading only its own eighth of the buffer
 * (workgroup b of 2048, on XCD b mod 8, reads range (b + 8 r) mod 2048 of the
 * buffer in round r).  With a buffer of up to 8 L2s the re-reads are served
 * by the XCDs' L2s, with a larger one by the Infinity Cache: the cache
 * ceilings for a decode whose blocks are shared between sequences.  sink as
 * for pkv_stream_read.  Not part of the attention method.
 */
PKV_API pkv_status pkv_stream_reread(const void* src, size_t bytes, int32_t rounds,
                                     uint32_t* sink, hipStream_t stream);

/*
 * Clock records — measurement only, not part of the attention method.  With
 * PAGEDKV_CLOCK=1 in the environment (read on every call), an attention call
 * on a bf16 pool with head_dim 128 and 16-token blocks, not under graph
 * capture, runs a build of its kernels that also records, per stream-decode
 * wave (record index = wave of the grid) or per prefill workgroup that
 * streams a context (record index = linear block id), 4 words:
 *   [0] the real-time counter (100 MHz) at its start, [1] at its end,
 *   [2] bits 0-7 the XCD it ran on; decode: bits 8-39 its positions (kv head
 *       x 16-token sub-tile), bits 40-63 the pieces it finished; prefill:
 *       bits 8-31 the sequence, 32-47 the kv head, 48-63 the column block,
 *   [3] decode: its workgroup (in the order positions are dealt); prefill:
 *       bits 0-19 the stages (64 tokens) it streamed, 20-31 its part of the
 *       context, 32-63 the context length.
 * Outputs are those of the normal kernels bit for bit.  The records live in
 * a library-held array per GPU (pkv_clock_records() records), cleared on the
 * call's stream before each such call; records not written read as zeros.
 * pkv_clock_read waits for all work on the current device, then copies the
 * first `records` records into host (records * 4 uint64); PKV_EINVAL if more
 * than pkv_clock_records() are asked for.
 */
PKV_API int32_t pkv_clock_records(void);
PKV_API pkv_status pkv_clock_read(unsigned long long* host, size_t records);

/* ------------------------------------------------------------------------
 * Host block manager (host memory only; no device work).
 *
 * The pool's free list, per-block reference counts and per-sequence block
 * tables, grown on demand: a sequence takes one more block only when its last
 * block is full, and freed blocks return to the pool ("Optimizing LLM
 * Inference: From PagedAttention to AI Infra", "On-Demand Allocation"; "05
 * PagedAttention", "Managing Virtual Memory (Block Manager)").  A fork shares
 * its parent's blocks; appending to a shared, partly filled last block first
 * copies it (copy-on-write: the pair is returned for paged_copy_blocks) while
 * the shared block stays unchanged (first page, "Copy-on-Write"; "05
 * PagedAttention", "KV Cache Sharing (Copy-on-Write)").  With the prefix
 * cache on, every block that fills is remembered under a 128-bit hash chain
 * of the token ids of the whole prefix it ends, and a new sequence reuses its
 * longest run of remembered leading full blocks (the second page, "Prefix
 * Caching"; "The Memory Wall", "Sharing is Caring: Prefix Caching").
 *
 * Policy: the lowest-numbered free block that holds no remembered prefix is
 * taken first; then the remembered free block released longest ago is
 * evicted and reused; a sequence's blocks are released last block first; a
 * prompt never reuses the block of its last token; an add or append the pool
 * cannot hold returns PKV_EWORKSPACE and changes nothing.  Slots are
 * block * block_size + offset, as paged_kv_append takes them.  One manager
 * must not be used by two threads at once.  Errors: pkv_bm_last_error().
 * ------------------------------------------------------------------------ */
typedef struct pkv_block_manager pkv_block_manager;

typedef struct {
  int64_t blocks_in_use;   /* blocks with a reference */
  int64_t tokens_stored;   /* token slots holding a token, over distinct blocks */
  int64_t slots_reserved;  /* blocks_in_use * block_size */
  int64_t cached_blocks;   /* blocks remembered by the prefix cache (used or free) */
  int64_t free_blocks;     /* blocks an allocation can take */
  int64_t num_sequences;
} pkv_bm_stats;

/* NULL on invalid sizes (num_blocks * block_size must be < 2^31) or no memory. */
PKV_API pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size,
                                         int32_t prefix_cache);
PKV_API void pkv_bm_destroy(pkv_block_manager* bm);
PKV_API const char* pkv_bm_last_error(void);
PKV_API int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm);

/* New sequence with its prompt (host array of num_tokens token ids).  Writes
 * *num_reused (leading prompt tokens found in the prefix cache, a multiple of
 * block_size) and slots[num_tokens]: -1 for reused tokens (their K/V already
 * sit in shared blocks), else the slot the token's K/V go to. */
PKV_API pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id,
                                       const int32_t* tokens, int32_t num_tokens,
                                       int32_t* num_reused, int32_t* slots);

/* Append num_tokens new tokens: writes slots[num_tokens]; when the last block
 * was shared and partly filled, *num_cow = 1 and cow_pair = {src, dst} must be
 * copied (paged_copy_blocks) before the new tokens are written; else
 * *num_cow = 0. */
PKV_API pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                                 int32_t num_tokens, int32_t* slots, int32_t* cow_pair,
                                 int32_t* num_cow);

/* One decode step: token tokens[i] appended to sequence seq_ids[i] for
 * i = 0 .. num_seqs-1, in that order (each id at most once).  Writes slots
 * [num_seqs] and the step's copy-on-write pairs, in order, to
 * cow_pairs[num_seqs, 2] with their count in *num_cow.  The exact block demand
 * of the whole step is checked first: PKV_EWORKSPACE leaves every sequence as
 * it was. */
PKV_API pkv_status pkv_bm_append_step(pkv_block_manager* bm, const int64_t* seq_ids,
                                      int32_t num_seqs, const int32_t* tokens, int32_t* slots,
                                      int32_t* cow_pairs, int32_t* num_cow);

/* Swap a sequence out of the pool when it runs short ("The Memory Wall", "The
 * Infrastructure Impact: Scale and Complexity", item "The Block Manager"; "05
 * PagedAttention", "Managing Virtual Memory (Block Manager)"): writes its block
 * table to block_ids[capacity] (*num_ids entries, table order: the blocks to
 * pass to paged_swap_out before anything reuses them) and releases them.  The
 * sequence keeps its tokens; until pkv_bm_swap_in it can only be freed. */
PKV_API pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq_id, int32_t* block_ids,
                                   int32_t capacity, int32_t* num_ids);
/* Bring a swapped-out sequence back: takes ceil(tokens / block_size) blocks
 * like any allocation and writes them to block_ids (table order: the
 * destinations to pass to paged_swap_in with the host image).  PKV_EWORKSPACE,
 * nothing changed, when the pool cannot hold it. */
PKV_API pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq_id, int32_t* block_ids,
                                  int32_t capacity, int32_t* num_ids);

/* child shares all of parent's blocks (parallel sampling, beam search). */
PKV_API pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);
PKV_API pkv_status pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id);
PKV_API pkv_status pkv_bm_sequence_info(const pkv_block_manager* bm, int64_t seq_id,
                                        int32_t* num_tokens, int32_t* num_blocks);

/* block_tables [num_seqs, max_blocks_per_seq] (-1 past each sequence's
 * blocks) and context_lens [num_seqs] of the listed sequences, host arrays
 * ready for paged_attention_decode once copied to the device. */
PKV_API pkv_status pkv_bm_build_batch(const pkv_block_manager* bm, const int64_t* seq_ids,
                                      int32_t num_seqs, int32_t* block_tables,
                                      int32_t max_blocks_per_seq, int32_t* context_lens);
PKV_API pkv_status pkv_bm_get_stats(const pkv_block_manager* bm, pkv_bm_stats* out);

PKV_API const char* pkv_status_string(pkv_status status);
/* Message of the calling thread's last failed call ("" if none). */
PKV_API const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
