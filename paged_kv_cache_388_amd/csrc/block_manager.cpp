// Host block manager of the paged KV cache: the pool's free list, per-block
// reference counts, per-sequence block tables grown on demand, copy-on-write
// of a shared partly filled block, and a cache of full blocks by prefix.
//
// A sequence takes blocks as its tokens arrive, one more only when its last
// block is full, and freed blocks go back to the pool ("Optimizing LLM
// Inference: From PagedAttention to AI Infra", "On-Demand Allocation"; the
// second page, "On-Demand Allocation, Reducing Internal Waste"; "05
// PagedAttention", "Managing Virtual Memory (Block Manager)").  A fork points
// at its parent's blocks, and a writer to a shared block first gets a private
// copy while the shared one stays as it was (first page, "Copy-on-Write";
// "05 PagedAttention", "KV Cache Sharing (Copy-on-Write)").  A prompt whose
// leading blocks were computed before reuses them (the second page, "Prefix
// Caching"; "The Memory Wall", "Sharing is Caring: Prefix Caching").
//
// Policy (deterministic, so that results are reproducible):
//  - allocation takes the lowest-numbered free block that holds no cached
//    prefix; when none is left, the cached free block released longest ago is
//    evicted and reused;
//  - a sequence's blocks are released from its last block to its first;
//  - only full blocks are cached, keyed by a 128-bit hash chain over the
//    token ids of the whole prefix they end (parent key, then the block's
//    tokens);
//  - a new sequence reuses its longest run of cached leading full blocks, but
//    never the block holding its last prompt token;
//  - an add or append the pool cannot hold fails before changing anything;
//  - a sequence swapped out to host memory releases all its blocks and keeps
//    its tokens; brought back, it takes fresh blocks like any allocation
//    ("The Memory Wall", "The Infrastructure Impact: Scale and Complexity",
//    item "The Block Manager"; "05 PagedAttention", "Managing Virtual Memory
//    (Block Manager)").
// Not thread-safe: one manager is driven by one thread at a time.

#include <stdint.h>
#include <string.h>

#include <new>
#include <queue>
#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

#include "pagedkv.h"

namespace {

thread_local char g_bm_err[256] = "";

pkv_status bm_fail(pkv_status st, const char* msg) {
  strncpy(g_bm_err, msg, sizeof(g_bm_err) - 1);
  g_bm_err[sizeof(g_bm_err) - 1] = '\0';
  return st;
}

struct Key {
  uint64_t a, b;
  bool operator==(const Key& o) const { return a == o.a && b == o.b; }
};
struct KeyHash {
  size_t operator()(const Key& k) const { return (size_t)(k.a ^ (k.b * 0x9E3779B97F4A7C15ull)); }
};

// One step of the prefix hash chain: mix the parent key with a block's token
// ids.  Two independent 64-bit lanes (different odd multipliers and seeds).
inline uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xBF58476D1CE4E5B9ull;
  x ^= x >> 27;
  x *= 0x94D049BB133111EBull;
  x ^= x >> 31;
  return x;
}
Key chain_key(const Key& parent, const int32_t* tokens, int n) {
  uint64_t a = mix64(parent.a ^ 0x243F6A8885A308D3ull);
  uint64_t b = mix64(parent.b ^ 0x13198A2E03707344ull);
  for (int i = 0; i < n; ++i) {
    const uint64_t t = (uint64_t)(uint32_t)tokens[i];
    a = mix64(a + t * 0x9E3779B97F4A7C15ull);
    b = mix64(b ^ (t * 0xC2B2AE3D27D4EB4Full + 0x165667B19E3779F9ull));
  }
  return Key{a, b};
}
const Key kRootKey{0x6A09E667F3BCC908ull, 0xBB67AE8584CAA73Bull};

struct Sequence {
  std::vector<int32_t> blocks;
  std::vector<int32_t> tokens;  // every token id (needed to key its full blocks)
  Key tail_key = kRootKey;      // key of the prefix ending at its last cached-or-keyed full block
  int32_t keyed_blocks = 0;     // leading full blocks whose keys are folded into tail_key
  bool swapped = false;         // blocks moved to host memory; none held in the pool
};

}  // namespace

struct pkv_block_manager {
  int32_t num_blocks = 0, block_size = 0;
  bool prefix_cache = true;
  std::vector<int32_t> ref;
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_blocks;
  std::set<std::pair<uint64_t, int32_t>> cached_free;  // (release tick, block)
  std::vector<uint64_t> release_tick;
  std::vector<uint8_t> cached;                          // block holds a cached prefix
  std::vector<Key> block_key;
  std::unordered_map<Key, int32_t, KeyHash> block_of;
  uint64_t tick = 0;
  std::unordered_map<int64_t, Sequence> seqs;

  int32_t num_free() const { return (int32_t)(free_blocks.size() + cached_free.size()); }

  int32_t take() {
    int32_t b;
    if (!free_blocks.empty()) {
      b = free_blocks.top();
      free_blocks.pop();
    } else {
      auto it = cached_free.begin();
      b = it->second;
      cached_free.erase(it);
      block_of.erase(block_key[b]);
      cached[b] = 0;
    }
    ref[b] = 1;
    return b;
  }

  void release(int32_t b) {
    if (--ref[b] == 0) {
      ++tick;
      if (cached[b]) {
        release_tick[b] = tick;
        cached_free.insert({tick, b});
      } else {
        free_blocks.push(b);
      }
    }
  }

  void reuse(int32_t b) {
    if (ref[b] == 0) cached_free.erase({release_tick[b], b});
    ++ref[b];
  }

  // Fold the sequence's newly full blocks into its key chain and cache each
  // one whose prefix is not cached yet.
  void register_full(Sequence& s) {
    const int32_t full = (int32_t)(s.tokens.size() / (size_t)block_size);
    while (s.keyed_blocks < full) {
      const int32_t j = s.keyed_blocks;
      s.tail_key = chain_key(s.tail_key, s.tokens.data() + (size_t)j * block_size, block_size);
      ++s.keyed_blocks;
      if (!prefix_cache) continue;
      const int32_t b = s.blocks[j];
      if (cached[b] || block_of.count(s.tail_key)) continue;
      cached[b] = 1;
      block_key[b] = s.tail_key;
      block_of.emplace(s.tail_key, b);
    }
  }

  int32_t needed(const Sequence& s, int32_t k) const {
    const int64_t n = (int64_t)s.tokens.size();
    const int64_t bs = block_size;
    const int64_t fresh = (n + k + bs - 1) / bs - (n + bs - 1) / bs;
    const int64_t cow = (k > 0 && n % bs != 0 && ref[s.blocks.back()] > 1) ? 1 : 0;
    return (int32_t)(fresh + cow);
  }

  // Append tokens (capacity already checked).  Writes one slot per token and
  // reports a copy-on-write pair if the shared last block had to be copied.
  void append(Sequence& s, const int32_t* toks, int32_t k, int32_t* slots, int32_t* cow,
              int32_t* num_cow) {
    for (int32_t i = 0; i < k; ++i) {
      const int64_t n = (int64_t)s.tokens.size();
      if (n % block_size == 0) {
        s.blocks.push_back(take());
      } else {
        const int32_t last = s.blocks.back();
        if (ref[last] > 1) {
          const int32_t fresh = take();
          release(last);
          s.blocks.back() = fresh;
          if (cow) {
            cow[0] = last;
            cow[1] = fresh;
          }
          if (num_cow) *num_cow = 1;
        }
      }
      if (slots) slots[i] = (int32_t)(s.blocks.back() * (int64_t)block_size + n % block_size);
      s.tokens.push_back(toks[i]);
    }
    register_full(s);
  }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_cache) {
  if (num_blocks <= 0 || block_size <= 0 || (int64_t)num_blocks * block_size > 0x7fffffffLL) {
    bm_fail(PKV_EINVAL, "num_blocks and block_size must be positive, num_blocks * block_size < 2^31");
    return nullptr;
  }
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
  if (!bm) {
    bm_fail(PKV_EINVAL, "out of host memory");
    return nullptr;
  }
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->prefix_cache = prefix_cache != 0;
    bm->ref.assign((size_t)num_blocks, 0);
    bm->release_tick.assign((size_t)num_blocks, 0);
    bm->cached.assign((size_t)num_blocks, 0);
    bm->block_key.assign((size_t)num_blocks, kRootKey);
    for (int32_t b = 0; b < num_blocks; ++b) bm->free_blocks.push(b);
  } catch (...) {
    delete bm;
    bm_fail(PKV_EINVAL, "out of host memory");
    return nullptr;
  }
  return bm;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

const char* pkv_bm_last_error(void) { return g_bm_err; }

int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) { return bm ? bm->num_free() : -1; }

pkv_status pkv_bm_add_sequence(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                               int32_t num_tokens, int32_t* num_reused, int32_t* slots) {
  g_bm_err[0] = '\0';
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !tokens))
    return bm_fail(PKV_EINVAL, "bad argument");
  if (bm->seqs.count(seq_id)) return bm_fail(PKV_EINVAL, "sequence id already in use");
  try {
    const int32_t bs = bm->block_size;
    // leading full blocks found in the cache, never the block of the last token
    std::vector<int32_t> found;
    Key key = kRootKey;
    if (bm->prefix_cache) {
      for (int64_t j = 0; (j + 1) * bs < num_tokens; ++j) {
        const Key next = chain_key(key, tokens + j * bs, bs);
        auto it = bm->block_of.find(next);
        if (it == bm->block_of.end()) break;
        found.push_back(it->second);
        key = next;
      }
    }
    const int32_t reused = (int32_t)found.size() * bs;
    int32_t idle = 0;
    for (int32_t b : found) idle += bm->ref[b] == 0 ? 1 : 0;
    const int32_t need = (num_tokens - reused + bs - 1) / bs;
    if (bm->num_free() - idle < need) return bm_fail(PKV_EWORKSPACE, "block pool exhausted");
    for (int32_t b : found) bm->reuse(b);
    Sequence& s = bm->seqs[seq_id];
    s.blocks = found;
    s.tokens.assign(tokens, tokens + reused);
    s.tail_key = key;
    s.keyed_blocks = (int32_t)found.size();
    if (slots)
      for (int32_t i = 0; i < reused; ++i) slots[i] = -1;
    bm->append(s, tokens + reused, num_tokens - reused, slots ? slots + reused : nullptr, nullptr,
               nullptr);
    if (num_reused) *num_reused = reused;
  } catch (...) {
    return bm_fail(PKV_EINVAL, "out of host memory");
  }
  return PKV_OK;
}

pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq_id, const int32_t* tokens,
                         int32_t num_tokens, int32_t* slots, int32_t* cow_pair, int32_t* num_cow) {
  g_bm_err[0] = '\0';
  if (!bm || num_tokens < 0 || (num_tokens > 0 && !tokens)) return bm_fail(PKV_EINVAL, "bad argument");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return bm_fail(PKV_EINVAL, "unknown sequence id");
  if (it->second.swapped) return bm_fail(PKV_EINVAL, "sequence is swapped out");
  if (num_cow) *num_cow = 0;
  if (bm->num_free() < bm->needed(it->second, num_tokens))
    return bm_fail(PKV_EWORKSPACE, "block pool exhausted");
  try {
    bm->append(it->second, tokens, num_tokens, slots, cow_pair, num_cow);
  } catch (...) {
    return bm_fail(PKV_EINVAL, "out of host memory");
  }
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  g_bm_err[0] = '\0';
  if (!bm) return bm_fail(PKV_EINVAL, "bad argument");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return bm_fail(PKV_EINVAL, "unknown sequence id");
  if (bm->seqs.count(child)) return bm_fail(PKV_EINVAL, "sequence id already in use");
  if (it->second.swapped) return bm_fail(PKV_EINVAL, "sequence is swapped out");
  try {
    Sequence copy = it->second;
    for (int32_t b : copy.blocks) bm->reuse(b);
    bm->seqs.emplace(child, std::move(copy));
  } catch (...) {
    return bm_fail(PKV_EINVAL, "out of host memory");
  }
  return PKV_OK;
}

pkv_status pkv_bm_free_sequence(pkv_block_manager* bm, int64_t seq_id) {
  g_bm_err[0] = '\0';
  if (!bm) return bm_fail(PKV_EINVAL, "bad argument");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return bm_fail(PKV_EINVAL, "unknown sequence id");
  const std::vector<int32_t>& blocks = it->second.blocks;
  for (size_t j = blocks.size(); j-- > 0;) bm->release(blocks[j]);
  bm->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_bm_append_step(pkv_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                              const int32_t* tokens, int32_t* slots, int32_t* cow_pairs,
                              int32_t* num_cow) {
  g_bm_err[0] = '\0';
  if (!bm || num_seqs < 0 || (num_seqs > 0 && (!seq_ids || !tokens || !slots || !cow_pairs)) ||
      !num_cow)
    return bm_fail(PKV_EINVAL, "bad argument");
  *num_cow = 0;
  try {
    std::vector<Sequence*> seqs((size_t)num_seqs);
    std::unordered_map<int32_t, int32_t> shared_left;  // last block -> references left to copy away
    int64_t need = 0;
    for (int32_t i = 0; i < num_seqs; ++i) {
      auto it = bm->seqs.find(seq_ids[i]);
      if (it == bm->seqs.end()) return bm_fail(PKV_EINVAL, "unknown sequence id");
      if (it->second.swapped) return bm_fail(PKV_EINVAL, "sequence is swapped out");
      seqs[(size_t)i] = &it->second;
    }
    {
      std::unordered_map<const Sequence*, int32_t> seen;
      for (int32_t i = 0; i < num_seqs; ++i)
        if (seen[seqs[(size_t)i]]++) return bm_fail(PKV_EINVAL, "sequence listed twice");
    }
    // Exact block demand of the whole step, in order: a full last block needs
    // a new one; a shared partly filled one needs a copy, unless every other
    // holder of it has already copied it away earlier in this step.
    for (int32_t i = 0; i < num_seqs; ++i) {
      const Sequence& q = *seqs[(size_t)i];
      if (q.tokens.size() % (size_t)bm->block_size == 0) {
        ++need;
        continue;
      }
      const int32_t last = q.blocks.back();
      auto f = shared_left.find(last);
      const int32_t refs = f == shared_left.end() ? bm->ref[last] : f->second;
      if (refs > 1) {
        ++need;
        shared_left[last] = refs - 1;
      }
    }
    if (need > bm->num_free()) return bm_fail(PKV_EWORKSPACE, "block pool exhausted");
    for (int32_t i = 0; i < num_seqs; ++i) {
      int32_t one = 0;
      bm->append(*seqs[(size_t)i], tokens + i, 1, slots + i, cow_pairs + 2 * (size_t)*num_cow, &one);
      *num_cow += one;
    }
  } catch (...) {
    return bm_fail(PKV_EINVAL, "out of host memory");
  }
  return PKV_OK;
}

pkv_status pkv_bm_swap_out(pkv_block_manager* bm, int64_t seq_id, int32_t* block_ids,
                           int32_t capacity, int32_t* num_ids) {
  g_bm_err[0] = '\0';
  if (!bm || !num_ids || capacity < 0 || (capacity > 0 && !block_ids))
    return bm_fail(PKV_EINVAL, "bad argument");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return bm_fail(PKV_EINVAL, "unknown sequence id");
  Sequence& s = it->second;
  if (s.swapped) return bm_fail(PKV_EINVAL, "sequence is swapped out");
  if ((int64_t)s.blocks.size() > capacity) return bm_fail(PKV_EINVAL, "block_ids too short");
  *num_ids = (int32_t)s.blocks.size();
  for (size_t j = 0; j < s.blocks.size(); ++j) block_ids[j] = s.blocks[j];
  for (size_t j = s.blocks.size(); j-- > 0;) bm->release(s.blocks[j]);
  s.blocks.clear();
  s.swapped = true;
  return PKV_OK;
}

pkv_status pkv_bm_swap_in(pkv_block_manager* bm, int64_t seq_id, int32_t* block_ids,
                          int32_t capacity, int32_t* num_ids) {
  g_bm_err[0] = '\0';
  if (!bm || !num_ids || capacity < 0 || (capacity > 0 && !block_ids))
    return bm_fail(PKV_EINVAL, "bad argument");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return bm_fail(PKV_EINVAL, "unknown sequence id");
  Sequence& s = it->second;
  if (!s.swapped) return bm_fail(PKV_EINVAL, "sequence is not swapped out");
  const int64_t bs = bm->block_size;
  const int32_t need = (int32_t)(((int64_t)s.tokens.size() + bs - 1) / bs);
  if (need > capacity) return bm_fail(PKV_EINVAL, "block_ids too short");
  if (need > bm->num_free()) return bm_fail(PKV_EWORKSPACE, "block pool exhausted");
  try {
    s.blocks.reserve((size_t)need);
    for (int32_t j = 0; j < need; ++j) s.blocks.push_back(bm->take());
    s.swapped = false;
    s.tail_key = kRootKey;
    s.keyed_blocks = 0;
    bm->register_full(s);
  } catch (...) {
    return bm_fail(PKV_EINVAL, "out of host memory");
  }
  *num_ids = need;
  for (int32_t j = 0; j < need; ++j) block_ids[j] = s.blocks[(size_t)j];
  return PKV_OK;
}

pkv_status pkv_bm_sequence_info(const pkv_block_manager* bm, int64_t seq_id, int32_t* num_tokens,
                                int32_t* num_blocks) {
  if (!bm) return bm_fail(PKV_EINVAL, "bad argument");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return bm_fail(PKV_EINVAL, "unknown sequence id");
  if (num_tokens) *num_tokens = (int32_t)it->second.tokens.size();
  if (num_blocks) *num_blocks = (int32_t)it->second.blocks.size();
  return PKV_OK;
}

pkv_status pkv_bm_build_batch(const pkv_block_manager* bm, const int64_t* seq_ids, int32_t num_seqs,
                              int32_t* block_tables, int32_t max_blocks_per_seq,
                              int32_t* context_lens) {
  g_bm_err[0] = '\0';
  if (!bm || num_seqs < 0 || (num_seqs > 0 && (!seq_ids || !block_tables || !context_lens)) ||
      max_blocks_per_seq < 0)
    return bm_fail(PKV_EINVAL, "bad argument");
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end()) return bm_fail(PKV_EINVAL, "unknown sequence id");
    if (it->second.swapped) return bm_fail(PKV_EINVAL, "sequence is swapped out");
    if ((int64_t)it->second.blocks.size() > max_blocks_per_seq)
      return bm_fail(PKV_EINVAL, "a sequence has more blocks than max_blocks_per_seq");
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Sequence& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (size_t)i * max_blocks_per_seq;
    const size_t nb = s.blocks.size();
    for (size_t j = 0; j < (size_t)max_blocks_per_seq; ++j) row[j] = j < nb ? s.blocks[j] : -1;
    context_lens[i] = (int32_t)s.tokens.size();
  }
  return PKV_OK;
}

pkv_status pkv_bm_get_stats(const pkv_block_manager* bm, pkv_bm_stats* out) {
  if (!bm || !out) return bm_fail(PKV_EINVAL, "bad argument");
  std::vector<int32_t> filled((size_t)bm->num_blocks, 0);
  for (const auto& kv : bm->seqs) {
    const Sequence& s = kv.second;
    const int64_t n = (int64_t)s.tokens.size();
    for (size_t j = 0; j < s.blocks.size(); ++j) {
      int64_t k = n - (int64_t)j * bm->block_size;
      k = k > bm->block_size ? bm->block_size : k;
      int32_t& f = filled[(size_t)s.blocks[j]];
      if (k > f) f = (int32_t)k;
    }
  }
  int64_t used = 0, stored = 0;
  for (int32_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->ref[b] > 0) {
      ++used;
      stored += filled[(size_t)b];
    }
  }
  out->blocks_in_use = used;
  out->tokens_stored = stored;
  out->slots_reserved = used * bm->block_size;
  out->cached_blocks = (int64_t)bm->block_of.size();
  out->free_blocks = bm->num_free();
  out->num_sequences = (int64_t)bm->seqs.size();
  return PKV_OK;
}

}  // extern "C"
