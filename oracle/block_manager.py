"""Plain reference model of the host block manager and its prefix cache.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only ``tests/`` (and ``bench.py``'s
``cpu_baseline`` leg) use it.  It shares no code with the C++ manager in
``paged_kv_cache_388_amd/csrc`` and imports nothing from it.  Every structure
is a Python list or dict scanned linearly, so each rule below can be checked
by eye.

What the pages describe, and the readings taken where they are silent
--------------------------------------------------------------------
* A pool of fixed-size physical blocks; a sequence takes blocks on demand as
  its tokens arrive, one more only when its last block is full; freed blocks
  return to the pool ("Optimizing LLM Inference: From PagedAttention to AI
  Infra", "On-Demand Allocation"; the second page, "On-Demand Allocation,
  Reducing Internal Waste" and "Fixed Block Size"; "05 PagedAttention",
  "Managing Virtual Memory (Block Manager)").
* Sharing: a forked sequence points at its parent's blocks; a writer to a
  shared block first gets a private copy and the shared block stays as it was
  (first page, "Copy-on-Write"; "05 PagedAttention", "KV Cache Sharing
  (Copy-on-Write)").
* Prefix caching: the KV of a prefix seen before is reused instead of being
  recomputed; requests with the same long prompt point their tables at the
  same physical blocks (second page, "Prefix Caching"; "The Memory Wall",
  "Sharing is Caring: Prefix Caching").

Readings (the pages fix none of these):
* allocation takes the lowest-numbered free block;
* only full blocks are cached, keyed by the exact token ids of the whole
  prefix up to and including the block (a lookup compares token ids, so
  there are no false hits); a block is offered to the cache once, when it
  becomes full, and is not cached if its prefix already is;
* a cached block whose last user leaves stays cached but reusable; when no
  never-cached block is free, the cached free block released longest ago is
  evicted (least recently used) and reused;
* a sequence's blocks are released from its last block to its first, so the
  end of a prefix is evicted before its beginning;
* a sequence added with a prompt reuses the longest run of leading full
  blocks found in the cache, but never the block holding its last prompt
  token (that token must be computed to produce the next one); its slot is
  -1 for every reused token;
* appending to a sequence whose last block is partly filled and shared first
  copies that block (one copy-on-write pair), then writes into the copy;
* an add or append the pool cannot hold fails before changing anything;
* a decode step appends one token to each listed sequence, in list order, and
  fails before changing anything unless the pool holds the whole step;
* swapping a sequence out (its blocks go to CPU RAM: "The Memory Wall", "The
  Infrastructure Impact: Scale and Complexity", item "The Block Manager"; "05
  PagedAttention", "Managing Virtual Memory (Block Manager)") returns its
  block table, the blocks to copy out in order, and releases them last block
  first; the sequence keeps its tokens.  Swapping it back in takes
  ceil(n / block_size) blocks the way any allocation does and offers its full
  blocks to the cache again.  A swapped-out sequence can only be swapped in
  or freed.
"""

import copy


class BlockManagerModel:
    def __init__(self, num_blocks, block_size, prefix_cache=True):
        self.nb = int(num_blocks)
        self.bs = int(block_size)
        self.prefix_cache = bool(prefix_cache)
        self.ref = [0] * self.nb
        self.free = list(range(self.nb))          # free blocks never cached (or evicted)
        self.cached_free = []                     # [(release_tick, block)] cached, unused
        self.tick = 0
        self.key_of = {}                          # block -> full-prefix token tuple
        self.block_of = {}                        # full-prefix token tuple -> block
        self.seqs = {}      # seq_id -> {"blocks": [...], "tokens": [...], "keyed": full blocks offered}

    # ---- allocation -------------------------------------------------------
    def _take(self):
        if self.free:
            b = min(self.free)
            self.free.remove(b)
        elif self.cached_free:
            t, b = min(self.cached_free)
            self.cached_free.remove((t, b))
            key = self.key_of.pop(b)
            del self.block_of[key]
        else:
            raise MemoryError("no free block")
        self.ref[b] = 1
        return b

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.tick += 1
            if b in self.key_of:
                self.cached_free.append((self.tick, b))
            else:
                self.free.append(b)

    def _reuse(self, b):
        if self.ref[b] == 0:
            for item in self.cached_free:
                if item[1] == b:
                    self.cached_free.remove(item)
                    break
        self.ref[b] += 1

    def num_free(self):
        return len(self.free) + len(self.cached_free)

    # ---- prefix cache ----------------------------------------------------
    def _register_full_blocks(self, seq):
        """Cache each block that has just become full, unless the block or its
        prefix is cached already."""
        toks = seq["tokens"]
        while seq["keyed"] < len(toks) // self.bs:
            j = seq["keyed"]
            seq["keyed"] += 1
            if not self.prefix_cache:
                continue
            b = seq["blocks"][j]
            key = tuple(toks[:(j + 1) * self.bs])
            if b in self.key_of or key in self.block_of:
                continue
            self.key_of[b] = key
            self.block_of[key] = b

    # ---- sequences -------------------------------------------------------
    def _lookup(self, tokens):
        """Leading full blocks of `tokens` found in the cache, never the block
        holding the last token."""
        found = []
        if self.prefix_cache:
            j = 0
            while (j + 1) * self.bs < len(tokens):
                b = self.block_of.get(tuple(tokens[:(j + 1) * self.bs]))
                if b is None:
                    break
                found.append(b)
                j += 1
        return found

    def _needed(self, seq, k):
        """Blocks an append of k tokens takes: new blocks, plus one
        copy-on-write copy when the last block is partly filled and shared."""
        n = len(seq["tokens"])
        new = -(-(n + k) // self.bs) - (-(-n // self.bs))
        cow = 1 if (k > 0 and n % self.bs != 0 and self.ref[seq["blocks"][-1]] > 1) else 0
        return new + cow

    def add_sequence(self, seq_id, tokens):
        """New sequence with its prompt.  Returns (number of reused leading
        tokens, slot per prompt token: -1 where reused).  Raises MemoryError,
        changing nothing, when the pool cannot hold it."""
        if seq_id in self.seqs:
            raise KeyError("sequence exists")
        tokens = [int(t) for t in tokens]
        found = self._lookup(tokens)
        reused = len(found) * self.bs
        idle = sum(1 for b in found if self.ref[b] == 0)   # reused blocks now counted as free
        need = -(-(len(tokens) - reused) // self.bs)
        if self.num_free() - idle < need:
            raise MemoryError("no free block")
        for b in found:
            self._reuse(b)
        seq = {"blocks": list(found), "tokens": tokens[:reused], "keyed": len(found)}
        self.seqs[seq_id] = seq
        return reused, [-1] * reused + self._append(seq, tokens[reused:])[0]

    def _append(self, seq, new_tokens):
        slots = []
        cow = None
        for t in new_tokens:
            n = len(seq["tokens"])
            if n % self.bs == 0:
                seq["blocks"].append(self._take())
            else:
                last = seq["blocks"][-1]
                if self.ref[last] > 1:                  # shared and partly filled: copy on write
                    fresh = self._take()
                    self._release(last)
                    seq["blocks"][-1] = fresh
                    cow = (last, fresh)
            slots.append(seq["blocks"][-1] * self.bs + n % self.bs)
            seq["tokens"].append(int(t))
        self._register_full_blocks(seq)
        return slots, cow

    def _live(self, seq_id):
        seq = self.seqs[seq_id]
        if seq.get("swapped"):
            raise KeyError("sequence is swapped out")
        return seq

    def append(self, seq_id, tokens):
        """Append new tokens.  Returns (slots, copy-on-write pair or None).
        Raises MemoryError, changing nothing, when the pool cannot hold them."""
        seq = self._live(seq_id)
        tokens = list(tokens)
        if self.num_free() < self._needed(seq, len(tokens)):
            raise MemoryError("no free block")
        return self._append(seq, tokens)

    def fork(self, parent, child):
        if child in self.seqs:
            raise KeyError("sequence exists")
        p = self._live(parent)
        for b in p["blocks"]:
            self._reuse(b)
        self.seqs[child] = {"blocks": list(p["blocks"]), "tokens": list(p["tokens"]),
                            "keyed": p["keyed"]}

    def free_sequence(self, seq_id):
        seq = self.seqs.pop(seq_id)
        for b in reversed(seq["blocks"]):
            self._release(b)

    def append_step(self, seq_ids, tokens):
        """One decode step: token tokens[i] appended to sequence seq_ids[i], in
        order.  Returns (slots, copy-on-write pairs in order).  If the pool
        cannot hold the whole step, raises MemoryError with nothing changed
        (the step is tried on a copy of the state first)."""
        if len(set(seq_ids)) != len(seq_ids):
            raise KeyError("sequence listed twice")
        for sid in seq_ids:
            self._live(sid)
        trial = copy.deepcopy(self)
        for sid, t in zip(seq_ids, tokens):
            trial.append(sid, [t])            # raises MemoryError on exhaustion
        slots, cows = [], []
        for sid, t in zip(seq_ids, tokens):
            sl, cow = self.append(sid, [t])
            slots += sl
            if cow is not None:
                cows.append(cow)
        return slots, cows

    def swap_out(self, seq_id):
        """Release a sequence's blocks (last first); returns them in table
        order, the blocks whose contents go to host memory."""
        seq = self._live(seq_id)
        blocks = list(seq["blocks"])
        for b in reversed(blocks):
            self._release(b)
        seq["blocks"] = []
        seq["swapped"] = True
        return blocks

    def swap_in(self, seq_id):
        """Give a swapped-out sequence fresh blocks; returns them in table
        order, the blocks its host copy goes back into.  Raises MemoryError,
        changing nothing, when the pool cannot hold it."""
        seq = self.seqs[seq_id]
        if not seq.get("swapped"):
            raise KeyError("sequence is not swapped out")
        need = -(-len(seq["tokens"]) // self.bs)
        if self.num_free() < need:
            raise MemoryError("no free block")
        seq["blocks"] = [self._take() for _ in range(need)]
        seq["swapped"] = False
        seq["keyed"] = 0
        self._register_full_blocks(seq)
        return list(seq["blocks"])

    def block_table(self, seq_id):
        return list(self._live(seq_id)["blocks"])

    def num_tokens(self, seq_id):
        return len(self.seqs[seq_id]["tokens"])

    # ---- accounting --------------------------------------------------------
    def stats(self):
        """Blocks in use, tokens stored (over distinct blocks), reserved slots
        and the fraction of reserved slots that hold no token."""
        used = [b for b in range(self.nb) if self.ref[b] > 0]
        filled = {}
        for seq in self.seqs.values():
            for j, b in enumerate(seq["blocks"]):
                k = min(self.bs, len(seq["tokens"]) - j * self.bs)
                filled[b] = max(filled.get(b, 0), k)
        stored = sum(filled.values())
        reserved = len(used) * self.bs
        return {"blocks_in_use": len(used), "tokens_stored": stored, "slots_reserved": reserved,
                "waste": (reserved - stored) / reserved if reserved else 0.0,
                "cached_blocks": len(self.key_of)}


def contiguous_reservation_utilisation(max_len, lengths):
    """Share of reserved token positions that hold a token when every request
    reserves max_len positions up front (the scheme paging replaces)."""
    return sum(lengths) / (max_len * len(lengths))


def paged_utilisation(block_size, lengths):
    """Share of reserved positions that hold a token when each request takes
    ceil(n / block_size) blocks."""
    reserved = sum(-(-n // block_size) * block_size for n in lengths)
    return sum(lengths) / reserved
