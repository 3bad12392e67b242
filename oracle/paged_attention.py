"""fp64 NumPy oracle for paged KV-cache decode.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg use it.

What is computed, and where the pages state it
----------------------------------------------
* The KV cache of one attention layer is cut into fixed-size blocks (16 tokens
  by default) held in one shared physical pool; a per-sequence block table maps
  logical block j to a physical block id.  Sources: "Optimizing LLM Inference:
  From PagedAttention to AI Infra" (cuicaihao.github.io), sections "PagedAttention:
  Decoupling Logical Context from Contiguous GPU Memory" and "On-Demand
  Allocation"; "The Memory Wall" (architects-blueprint.vercel.app), section
  "How it Works Under the Hood"; "05 PagedAttention" (ai-system-design-guide),
  section "How PagedAttention Works (vLLM)".
* Paging changes where the bytes live, not the mathematics: the first page says
  vLLM kept the Transformer's mathematical definition, and the conceptual kernel
  on "The Memory Wall" ("Show Me The Code") leaves the arithmetic to standard
  attention.  The oracle therefore materialises each sequence's K/V in logical
  order from the block table and evaluates plain scaled-dot-product attention,
  ``softmax(scale * q K^T) V``, in fp64.
* Tokens are written into their slot as they arrive (first page, "On-Demand
  Allocation"; "The Memory Wall", "How it Works Under the Hood"): ``kv_append``.
* Copy-on-write gives a writer its own copy of a shared block while the shared
  block stays unchanged ("05 PagedAttention", section "KV Cache Sharing
  (Copy-on-Write)"; first page, section "Copy-on-Write"): ``copy_blocks``.
* Blocks can be moved to CPU RAM and back when the pool runs short ("The
  Memory Wall", "The Infrastructure Impact: Scale and Complexity"; "05
  PagedAttention", "Managing Virtual Memory (Block Manager)"): ``swap_out`` and
  ``swap_in``.

Readings where the pages are silent:
* pool layout ``[num_blocks, H_kv, block_size, D]`` for K and V alike;
* query head h reads KV head ``h // G`` with ``G = H_q // H_kv``;
* the single query attends to all ``context_lens[s]`` cached tokens, the token
  appended in the same step included;
* ``slot = physical_block * block_size + offset``; a negative slot is skipped;
* a sequence with zero context yields a zero output row;
* a swapped-out batch of blocks is one contiguous host image, entry i holding
  the i-th listed block's K tile then its V tile;
* storage types are fp32, fp16 and bf16; fp16/bf16 arrays are passed as their
  raw 16-bit patterns (``uint16``) and decoded exactly to fp64.
"""

import numpy as np

DTYPES = ("f32", "f16", "bf16")


# ---------------------------------------------------------------------------
# storage decoding (exact)
# ---------------------------------------------------------------------------

def storage_to_f64(raw, dtype):
    """Decode stored values to float64 exactly.

    fp32 arrays are float32; fp16 and bf16 arrays are their raw uint16 bit
    patterns.  bf16 is the top half of an IEEE binary32, so its value is the
    pattern shifted into the high 16 bits of a 32-bit word.
    """
    raw = np.asarray(raw)
    if dtype == "f32":
        return raw.astype(np.float32, copy=False).astype(np.float64)
    if dtype == "f16":
        return raw.astype(np.uint16, copy=False).view(np.float16).astype(np.float64)
    if dtype == "bf16":
        wide = raw.astype(np.uint16, copy=False).astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _bits(a):
    """View an array as unsigned integers of the same width (bit copies)."""
    a = np.asarray(a)
    return a.view({2: np.uint16, 4: np.uint32}[a.dtype.itemsize])


# ---------------------------------------------------------------------------
# block counting (first page, "On-Demand Allocation"; "The Memory Wall",
# "Why this is a 'Holy Grail' moment")
# ---------------------------------------------------------------------------

def blocks_for_tokens(num_tokens, block_size):
    """Blocks a sequence of ``num_tokens`` tokens occupies: ceil(n / bs)."""
    num_tokens = int(num_tokens)
    block_size = int(block_size)
    return (num_tokens + block_size - 1) // block_size


def last_block_fill(num_tokens, block_size):
    """(tokens stored in the last block, free slots left in it)."""
    nb = blocks_for_tokens(num_tokens, block_size)
    if nb == 0:
        return 0, 0
    used = num_tokens - (nb - 1) * block_size
    return used, block_size - used


def mean_tail_waste(block_size):
    """Mean free slots in the last block when the length's residue modulo the
    block size is uniformly distributed: the average of bs - used over
    used = 1..bs."""
    return float(np.mean([block_size - used for used in range(1, block_size + 1)]))


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_bytes):
    """KV-cache bytes per token: one K and one V vector per KV head per layer.
    First page, "Understanding KV Cache Before Diving into PagedAttention"
    (the formula's legend: 2, L, H_kv, D, T, B_dtype)."""
    return 2 * num_layers * num_kv_heads * head_dim * dtype_bytes


# ---------------------------------------------------------------------------
# gathering one sequence's context through its block table
# ---------------------------------------------------------------------------

def gather_context(cache, block_table_row, num_tokens, dtype):
    """Materialise one sequence's K (or V) in logical token order.

    ``cache`` is the pool ``[NB, H_kv, bs, D]``; logical block j lives in
    physical block ``block_table_row[j]``.  Returns fp64 ``[H_kv, n, D]``.
    Only the first ceil(n / bs) table entries are read.
    """
    bs = cache.shape[2]
    nb = blocks_for_tokens(num_tokens, bs)
    if nb == 0:
        return np.zeros((cache.shape[1], 0, cache.shape[3]))
    ids = [int(block_table_row[j]) for j in range(nb)]
    tiles = [cache[i] for i in ids]                      # each [H_kv, bs, D]
    joined = np.concatenate(tiles, axis=1)               # [H_kv, nb*bs, D]
    return storage_to_f64(joined[:, :num_tokens, :], dtype)


# ---------------------------------------------------------------------------
# decode attention
# ---------------------------------------------------------------------------

def _softmax_weighted_sum(scores, values):
    """Plain softmax over the token axis followed by the weighted sum."""
    m = scores.max()
    p = np.exp(scores - m)
    return (p @ values) / p.sum()


def decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale,
                     dtype, seq_ids=None):
    """Paged decode attention, one query token per sequence, in fp64.

    q            [B, H_q, D]          storage dtype
    k_cache      [NB, H_kv, bs, D]    storage dtype
    v_cache      [NB, H_kv, bs, D]    storage dtype
    block_tables [B, max_blocks]      int
    context_lens [B]                  int
    Returns fp64 ``[len(seq_ids), H_q, D]`` (all sequences by default).
    """
    B, H_q, D = q.shape
    H_kv = k_cache.shape[1]
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    if seq_ids is None:
        seq_ids = range(B)
    seq_ids = list(seq_ids)
    out = np.zeros((len(seq_ids), H_q, D))
    for row, s in enumerate(seq_ids):
        n = int(context_lens[s])
        if n == 0:
            continue
        K = gather_context(k_cache, block_tables[s], n, dtype)
        V = gather_context(v_cache, block_tables[s], n, dtype)
        qs = storage_to_f64(q[s], dtype)
        for h in range(H_q):
            kv = h // G
            scores = scale * (K[kv] @ qs[h])
            out[row, h] = _softmax_weighted_sum(scores, V[kv])
    return out


# ---------------------------------------------------------------------------
# several new tokens per sequence: speculative-decode verification and
# chunked-prefill chunks
# ---------------------------------------------------------------------------

def multi_query_attention(q, k_cache, v_cache, block_tables, context_lens, query_lens,
                          scale, dtype):
    """Paged attention of several new tokens per sequence, in fp64.

    A chunk of a long prompt is processed together with other requests' decode
    tokens (the second page, "Chunked Prefill"), and a large model checks a
    draft model's guessed tokens in one pass (*The Memory Wall*, "The Next
    Frontier: Speculative Decoding and Beyond").  Both put L_s new tokens of
    sequence s through attention at once.  Reading taken: the L_s new tokens
    are the last L_s of the sequence's n_s cached tokens (their K/V were
    appended first), and new token i, at logical position n_s - L_s + i,
    attends to logical tokens 0 .. n_s - L_s + i (itself and everything
    before it).  L_s = 1 is decode.

    q            [T, H_q, D]   the new tokens, packed sequence by sequence
                               (T = sum of query_lens, no padding)
    k_cache      [NB, H_kv, bs, D]
    v_cache      [NB, H_kv, bs, D]
    block_tables [B, max_blocks]
    context_lens [B]           n_s, counting the new tokens
    query_lens   [B]           L_s, 0 <= L_s <= n_s
    Returns fp64 ``[T, H_q, D]``.
    """
    T, H_q, D = q.shape
    H_kv = k_cache.shape[1]
    if H_q % H_kv != 0:
        raise ValueError("H_q must be a multiple of H_kv")
    G = H_q // H_kv
    query_lens = [int(x) for x in query_lens]
    if sum(query_lens) != T:
        raise ValueError("query_lens must sum to the number of query rows")
    out = np.zeros((T, H_q, D))
    row = 0
    for s, L in enumerate(query_lens):
        n = int(context_lens[s])
        if L > n:
            raise ValueError("a sequence has more new tokens than cached tokens")
        if L == 0:
            continue
        K = gather_context(k_cache, block_tables[s], n, dtype)
        V = gather_context(v_cache, block_tables[s], n, dtype)
        for i in range(L):
            visible = n - L + i + 1
            qs = storage_to_f64(q[row + i], dtype)
            for h in range(H_q):
                kv = h // G
                scores = scale * (K[kv, :visible] @ qs[h])
                out[row + i, h] = _softmax_weighted_sum(scores, V[kv, :visible])
        row += L
    return out


# ---------------------------------------------------------------------------
# split-context decode: per-partition softmax state and its exact merge
# ---------------------------------------------------------------------------

def partition_states(q, k_cache, v_cache, block_table_row, num_tokens, scale,
                     dtype, head, num_kv_heads_per_q, partition_tokens):
    """Softmax state of each context partition for one (sequence, query head).

    Partition p covers logical tokens [p*P, min((p+1)*P, n)).  For each it
    returns m_p = max score, l_p = sum exp(score - m_p) and the unnormalised
    o_p = sum exp(score - m_p) v.  ``q`` is this sequence's [H_q, D] row.
    """
    K = gather_context(k_cache, block_table_row, num_tokens, dtype)
    V = gather_context(v_cache, block_table_row, num_tokens, dtype)
    kv = head // num_kv_heads_per_q
    qh = storage_to_f64(q[head], dtype)
    scores = scale * (K[kv] @ qh)
    ms, ls, os_ = [], [], []
    for start in range(0, num_tokens, partition_tokens):
        sc = scores[start:start + partition_tokens]
        vv = V[kv][start:start + partition_tokens]
        m = sc.max()
        p = np.exp(sc - m)
        ms.append(m)
        ls.append(p.sum())
        os_.append(p @ vv)
    return np.array(ms), np.array(ls), np.array(os_)


def merge_partitions(ms, ls, os_):
    """Merge partition states: rescale each by exp(m_p - max m) and divide the
    summed outputs by the summed normalisers."""
    M = ms.max()
    w = np.exp(ms - M)
    return (w[:, None] * os_).sum(axis=0) / (w * ls).sum()


def split_decode_attention(q, k_cache, v_cache, block_tables, context_lens,
                           scale, dtype, partition_tokens, seq_ids=None):
    """Decode attention evaluated partition by partition and merged."""
    B, H_q, D = q.shape
    G = H_q // k_cache.shape[1]
    if seq_ids is None:
        seq_ids = range(B)
    seq_ids = list(seq_ids)
    out = np.zeros((len(seq_ids), H_q, D))
    for row, s in enumerate(seq_ids):
        n = int(context_lens[s])
        if n == 0:
            continue
        for h in range(H_q):
            ms, ls, os_ = partition_states(q[s], k_cache, v_cache,
                                           block_tables[s], n, scale, dtype,
                                           h, G, partition_tokens)
            out[row, h] = merge_partitions(ms, ls, os_)
    return out


# ---------------------------------------------------------------------------
# append and copy-on-write copies (bit copies)
# ---------------------------------------------------------------------------

def kv_append(k_cache, v_cache, key, value, slot_mapping):
    """Write token i's K/V ([T, H_kv, D]) into slot ``slot_mapping[i]``.

    slot = block * bs + offset; a negative slot is skipped.  Returns new pools;
    the inputs are not modified.  Values are copied as raw bits.
    """
    kc = _bits(k_cache).copy()
    vc = _bits(v_cache).copy()
    kk = _bits(key)
    vv = _bits(value)
    bs = kc.shape[2]
    for i in range(len(slot_mapping)):
        slot = int(slot_mapping[i])
        if slot < 0:
            continue
        kc[slot // bs, :, slot % bs, :] = kk[i]
        vc[slot // bs, :, slot % bs, :] = vv[i]
    return kc.view(np.asarray(k_cache).dtype), vc.view(np.asarray(v_cache).dtype)


def copy_blocks(k_cache, v_cache, block_mapping):
    """Copy whole blocks (every KV head of K and of V) for each (src, dst)
    pair.  Destinations must be distinct and must not be a source in the same
    call, so the result does not depend on the order of the pairs."""
    pairs = [(int(a), int(b)) for a, b in np.asarray(block_mapping).reshape(-1, 2)]
    dsts = [d for _, d in pairs]
    srcs = {s for s, _ in pairs}
    if len(set(dsts)) != len(dsts):
        raise ValueError("copy_blocks: duplicate destination block")
    if srcs & set(dsts):
        raise ValueError("copy_blocks: a destination is also a source")
    kc = _bits(k_cache).copy()
    vc = _bits(v_cache).copy()
    k0 = _bits(k_cache)
    v0 = _bits(v_cache)
    for src, dst in pairs:
        kc[dst] = k0[src]
        vc[dst] = v0[src]
    return kc.view(np.asarray(k_cache).dtype), vc.view(np.asarray(v_cache).dtype)


# ---------------------------------------------------------------------------
# swap to host memory and back (bit copies)
# ---------------------------------------------------------------------------
#
# When the pool runs short the block manager may move a sequence's blocks out
# to CPU RAM and bring them back later ("The Memory Wall", "The Infrastructure
# Impact: Scale and Complexity", item "The Block Manager"; "05 PagedAttention",
# "Managing Virtual Memory (Block Manager)", its eviction entry).  The pages
# fix no host layout.  Reading taken: a swap moves an ordered list of block ids
# into one contiguous host image, entry i holding block ids[i]'s K tile and
# then its V tile ([n, 2, H_kv, bs, D]); bringing it back writes entry i into
# block ids[i] of the pools, which need not be the block it came from.

def swap_out(k_cache, v_cache, block_ids):
    """Host image [n, 2, H_kv, bs, D] of the listed blocks, raw bits.  An id
    outside the pool gives an all-zero entry."""
    kc = _bits(k_cache)
    vc = _bits(v_cache)
    nb = kc.shape[0]
    image = np.zeros((len(block_ids), 2) + kc.shape[1:], dtype=kc.dtype)
    for i, b in enumerate(block_ids):
        b = int(b)
        if 0 <= b < nb:
            image[i, 0] = kc[b]
            image[i, 1] = vc[b]
    return image.view(np.asarray(k_cache).dtype)


def swap_in(k_cache, v_cache, image, block_ids):
    """Write entry i of a host image into block block_ids[i] of both pools.
    Destinations must be distinct; an id outside the pool is skipped.  Returns
    new pools; the inputs are not modified."""
    ids = [int(b) for b in block_ids]
    inside = [b for b in ids if 0 <= b < np.asarray(k_cache).shape[0]]
    if len(set(inside)) != len(inside):
        raise ValueError("swap_in: duplicate destination block")
    kc = _bits(k_cache).copy()
    vc = _bits(v_cache).copy()
    img = _bits(image)
    for i, b in enumerate(ids):
        if 0 <= b < kc.shape[0]:
            kc[b] = img[i, 0]
            vc[b] = img[i, 1]
    return kc.view(np.asarray(k_cache).dtype), vc.view(np.asarray(v_cache).dtype)
