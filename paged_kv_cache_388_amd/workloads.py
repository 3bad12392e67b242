"""Seeded synthetic decode workloads.

This module only draws inputs.  It holds none of the attention arithmetic and
is shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()`` so that
the HIP path and the CPU oracle see identical bytes.

Every array is host NumPy: fp32 data as ``float32``, fp16/bf16 data as their
raw ``uint16`` bit patterns (values are drawn in fp32 and rounded to nearest
even).  Pools use the layout ``[num_blocks, H_kv, block_size, D]``; block
tables are int32 ``[B, max_blocks]`` with -1 in entries a sequence does not
use; a step's appended tokens are addressed by ``slot = block * bs + offset``.

Draw order for a seed: context lengths, the pool permutation, q, the K pool,
the V pool, then the appended K/V.  Named workloads use seed 388000 + k.

The five named workloads (structure as stated with each builder):
  1 ``tiny_f32``      4 sequences, contexts {5, 16, 33, 70}, 2/2 heads, D 64
  2 ``llama2_7b_f16`` 64 sequences, 32/32 heads, D 128, contexts U{128..2048}
  3 ``llama3_8b_gqa`` 128 sequences, 32/8 heads, D 128, log-uniform [256, 8192]
  4 ``shared_prefix`` 100 sequences sharing a 5000-token prefix, CoW copies,
                      unique suffixes of 16..512 tokens, 32/8 heads, D 128
  5 ``long_ctx``      32 sequences, 64/8 heads, D 128, log-uniform
                      [1024, 32768], block size 16 or 32
Several new tokens per sequence:
    ``spec_verify``   the Llama-3-8B GQA shape with 4 draft tokens per sequence
    ``prefill_chunk`` 8 prompts each processing a 256-token chunk
"""

import math
from dataclasses import dataclass, field

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}

NAMED = ("tiny_f32", "llama2_7b_f16", "llama3_8b_gqa", "shared_prefix", "long_ctx")
MULTI = ("spec_verify", "prefill_chunk", "long_prompt_chunk")


@dataclass
class Workload:
    name: str
    dtype: str
    seed: int
    q: np.ndarray               # [B, H_q, D]
    k_cache: np.ndarray         # [NB, H_kv, bs, D]  state before the step
    v_cache: np.ndarray
    block_tables: np.ndarray    # [B, max_blocks] int32
    context_lens: np.ndarray    # [B] int32, after the step's appends
    scale: float
    # the step's cache writes, applied in this order before attention
    block_mapping: np.ndarray = field(default=None)   # [N, 2] int32 (src, dst)
    slot_mapping: np.ndarray = field(default=None)    # [T] int32
    new_key: np.ndarray = field(default=None)         # [T, H_kv, D]
    new_value: np.ndarray = field(default=None)
    # several new tokens per sequence: q holds [T, H_q, D] packed rows and
    # query_start [B + 1] their prefix (None for decode: row s = sequence s)
    query_start: np.ndarray = field(default=None)

    @property
    def multi(self):
        return self.query_start is not None

    @property
    def max_query_len(self):
        if not self.multi:
            return 1
        return int(np.diff(self.query_start).max()) if len(self.query_start) > 1 else 0

    @property
    def num_seqs(self):
        return self.context_lens.shape[0]

    @property
    def num_q_heads(self):
        return self.q.shape[1]

    @property
    def head_dim(self):
        return self.q.shape[2]

    @property
    def num_blocks(self):
        return self.k_cache.shape[0]

    @property
    def num_kv_heads(self):
        return self.k_cache.shape[1]

    @property
    def block_size(self):
        return self.k_cache.shape[2]

    @property
    def max_blocks_per_seq(self):
        return self.block_tables.shape[1]

    @property
    def max_context_len(self):
        return int(self.context_lens.max()) if self.num_seqs else 0

    def kv_bytes(self):
        """Bytes of K and V one decode step reads: every cached token once."""
        return (2 * int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads
                * self.head_dim * ELEM_BYTES[self.dtype])

    def describe(self):
        return dict(workload=self.name, dtype=self.dtype, seed=self.seed,
                    num_seqs=self.num_seqs, num_q_heads=self.num_q_heads,
                    num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
                    block_size=self.block_size, num_blocks=self.num_blocks,
                    mean_context=float(self.context_lens.mean()),
                    max_context=self.max_context_len,
                    appended_tokens=int(len(self.slot_mapping)),
                    copied_blocks=int(len(self.block_mapping)))


# ---------------------------------------------------------------------------
# value drawing
# ---------------------------------------------------------------------------

def _normal(rng, shape, dtype):
    """N(0, 1) drawn in fp32 and rounded to the storage type (RNE)."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    import torch
    t = torch.from_numpy(x).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def uniform_lengths(rng, n, lo, hi):
    return rng.integers(lo, hi + 1, size=n).astype(np.int32)


def log_uniform_lengths(rng, n, lo, hi):
    u = rng.uniform(math.log(lo), math.log(hi + 1), size=n)
    return np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int32)


def _poison(pool, dtype):
    if dtype == "f32":
        pool[...] = np.float32(np.nan)
    else:
        pool[...] = NAN_BITS[dtype]


# ---------------------------------------------------------------------------
# generic builder
# ---------------------------------------------------------------------------

def build(name, seed, rng, ctx, H_q, H_kv, D, bs, dtype, scale=None,
          num_blocks=None, free_frac=0.10, max_blocks=None, append_last=True,
          poison=False, query_lens=None):
    """Private blocks per sequence, drawn through one shuffled pool.

    ``ctx`` are the context lengths after the step.  With ``append_last`` the
    step appends each sequence's final token (position ctx-1) before attention.
    With ``query_lens`` (several new tokens per sequence) the step appends the
    last query_lens[s] tokens of every sequence and q holds one packed row per
    new token.  ``poison`` fills every slot the step does not define (free
    blocks, tail slots, the slots about to be appended) with NaN.
    """
    ctx = np.asarray(ctx, dtype=np.int32)
    B = len(ctx)
    nbs = [(int(n) + bs - 1) // bs for n in ctx]
    need = sum(nbs)
    NB = num_blocks if num_blocks is not None else int(math.ceil(need * (1 + free_frac)))
    NB = max(NB, need, 1)
    perm = rng.permutation(NB).astype(np.int32)
    if max_blocks is None:
        max_blocks = max(1, max(nbs) if nbs else 1)
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    nxt = 0
    for s in range(B):
        bt[s, :nbs[s]] = perm[nxt:nxt + nbs[s]]
        nxt += nbs[s]
    qstart = None
    if query_lens is not None:
        query_lens = np.asarray(query_lens, dtype=np.int32)
        if np.any(query_lens > ctx) or np.any(query_lens < 0):
            raise ValueError("need 0 <= query_lens <= ctx")
        qstart = np.concatenate([[0], np.cumsum(query_lens)]).astype(np.int32)
    q = _normal(rng, (B if qstart is None else int(qstart[-1]), H_q, D), dtype)
    k_cache = _normal(rng, (NB, H_kv, bs, D), dtype)
    v_cache = _normal(rng, (NB, H_kv, bs, D), dtype)
    if qstart is not None:
        slots = np.array([bt[s, t // bs] * bs + t % bs
                          for s in range(B) for t in range(int(ctx[s]) - int(query_lens[s]),
                                                           int(ctx[s]))], dtype=np.int32)
        new_key = _normal(rng, (len(slots), H_kv, D), dtype)
        new_value = _normal(rng, (len(slots), H_kv, D), dtype)
    elif append_last:
        live = [s for s in range(B) if ctx[s] > 0]
        slots = np.array([bt[s, (ctx[s] - 1) // bs] * bs + (ctx[s] - 1) % bs for s in live],
                         dtype=np.int32)
        new_key = _normal(rng, (len(live), H_kv, D), dtype)
        new_value = _normal(rng, (len(live), H_kv, D), dtype)
    else:
        slots = np.zeros((0,), dtype=np.int32)
        new_key = np.zeros((0, H_kv, D), dtype=STORAGE[dtype])
        new_value = np.zeros((0, H_kv, D), dtype=STORAGE[dtype])
    if poison:
        used = np.zeros((NB, bs), dtype=bool)
        for s in range(B):
            for t in range(int(ctx[s])):
                used[bt[s, t // bs], t % bs] = True
        for slot in slots:
            used[slot // bs, slot % bs] = False
        for b in range(NB):
            for o in range(bs):
                if not used[b, o]:
                    _poison(k_cache[b, :, o, :], dtype)
                    _poison(v_cache[b, :, o, :], dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Workload(name=name, dtype=dtype, seed=seed, q=q, k_cache=k_cache,
                    v_cache=v_cache, block_tables=bt, context_lens=ctx, scale=float(scale),
                    block_mapping=np.zeros((0, 2), dtype=np.int32), slot_mapping=slots,
                    new_key=new_key, new_value=new_value, query_start=qstart)


# ---------------------------------------------------------------------------
# named workloads
# ---------------------------------------------------------------------------

def tiny_f32(seed=388001, poison=False):
    """4 sequences with contexts {5, 16, 33, 70}, H_q = H_kv = 2, D = 64, 16-token
    blocks, a 32-block pool whose ids come from a seeded permutation, fp32,
    scale 1/8."""
    rng = np.random.default_rng(seed)
    return build("tiny_f32", seed, rng, [5, 16, 33, 70], 2, 2, 64, 16, "f32",
                 scale=1 / 8, num_blocks=32, poison=poison)


def llama2_7b_f16(seed=388002, poison=False, num_seqs=64):
    """Llama-2-7B-shaped layer: 32/32 heads of 128, fp16, contexts U{128..2048},
    pool = needed blocks + 10% free."""
    rng = np.random.default_rng(seed)
    ctx = uniform_lengths(rng, num_seqs, 128, 2048)
    return build("llama2_7b_f16", seed, rng, ctx, 32, 32, 128, 16, "f16",
                 max_blocks=128, poison=poison)


def llama3_8b_gqa(seed=388003, poison=False, num_seqs=128):
    """Llama-3-8B-shaped GQA layer: 32 query / 8 KV heads of 128, bf16,
    contexts log-uniform in [256, 8192], pool = needed blocks + 10% free."""
    rng = np.random.default_rng(seed)
    ctx = log_uniform_lengths(rng, num_seqs, 256, 8192)
    return build("llama3_8b_gqa", seed, rng, ctx, 32, 8, 128, 16, "bf16",
                 max_blocks=512, poison=poison)


def long_ctx(block_size=16, seed=388005, poison=False, num_seqs=32):
    """Long-context GQA layer: 64 query / 8 KV heads of 128, bf16, contexts
    log-uniform in [1024, 32768] (same lengths at either block size); the
    step appends each sequence's newest token before attention."""
    rng = np.random.default_rng(seed)
    ctx = log_uniform_lengths(rng, num_seqs, 1024, 32768)
    return build(f"long_ctx_bs{block_size}", seed, rng, ctx, 64, 8, 128, block_size, "bf16",
                 max_blocks=32768 // block_size, poison=poison)


def shared_prefix(seed=388004, poison=False, num_seqs=100, prefix_tokens=5000,
                  suffix_lo=16, suffix_hi=512, H_q=32, H_kv=8, D=128, bs=16):
    """Shared-prefix decode.  Every sequence's table starts with the same
    physical blocks of a common ``prefix_tokens`` prompt.  The partial last
    prefix block is copied (copy-on-write) into a private block per sequence;
    the sequence's suffix tokens fill that copy's free slots and then fresh
    blocks.  The step: copy the blocks, append every suffix token, attend.
    """
    rng = np.random.default_rng(seed)
    S = uniform_lengths(rng, num_seqs, suffix_lo, suffix_hi)
    ctx = (prefix_tokens + S).astype(np.int32)
    n_full, tail = divmod(prefix_tokens, bs)
    n_prefix = n_full + (1 if tail else 0)
    own = []                          # private blocks per sequence (CoW copy first)
    for s in range(num_seqs):
        rest = int(S[s]) - ((bs - tail) if tail else 0)
        own.append((1 if tail else 0) + max(0, (rest + bs - 1) // bs))
    need = n_prefix + sum(own)
    NB = int(math.ceil(need * 1.10))
    perm = rng.permutation(NB).astype(np.int32)
    prefix_ids = perm[:n_prefix]
    max_blocks = (prefix_tokens + suffix_hi + bs - 1) // bs
    bt = np.full((num_seqs, max_blocks), -1, dtype=np.int32)
    pairs = []
    nxt = n_prefix
    for s in range(num_seqs):
        ids = perm[nxt:nxt + own[s]]
        nxt += own[s]
        bt[s, :n_full] = prefix_ids[:n_full]
        bt[s, n_full:n_full + own[s]] = ids
        if tail:
            pairs.append((int(prefix_ids[n_full]), int(ids[0])))
    dtype = "bf16"
    q = _normal(rng, (num_seqs, H_q, D), dtype)
    k_cache = _normal(rng, (NB, H_kv, bs, D), dtype)
    v_cache = _normal(rng, (NB, H_kv, bs, D), dtype)
    slots = []
    for s in range(num_seqs):
        for t in range(prefix_tokens, int(ctx[s])):
            slots.append(int(bt[s, t // bs]) * bs + t % bs)
    slots = np.array(slots, dtype=np.int32)
    new_key = _normal(rng, (len(slots), H_kv, D), dtype)
    new_value = _normal(rng, (len(slots), H_kv, D), dtype)
    if poison:
        defined = np.zeros((NB, bs), dtype=bool)
        for j in range(n_prefix):
            for o in range(bs if (j < n_full or not tail) else tail):
                defined[prefix_ids[j], o] = True
        for b in range(NB):
            for o in range(bs):
                if not defined[b, o]:
                    _poison(k_cache[b, :, o, :], dtype)
                    _poison(v_cache[b, :, o, :], dtype)
    return Workload(name="shared_prefix", dtype=dtype, seed=seed, q=q, k_cache=k_cache,
                    v_cache=v_cache, block_tables=bt, context_lens=ctx,
                    scale=1.0 / math.sqrt(D),
                    block_mapping=np.array(pairs, dtype=np.int32).reshape(-1, 2),
                    slot_mapping=slots, new_key=new_key, new_value=new_value)


def spec_verify(seed=388006, poison=False, num_seqs=128, draft=4):
    """Speculative-decode verification on the Llama-3-8B-shaped GQA layer: the
    same shape and context distribution as ``llama3_8b_gqa`` (32 query / 8 KV
    heads of 128, bf16, contexts log-uniform in [256, 8192]), with ``draft``
    guessed tokens per sequence appended and attended at once (4 tokens x 4
    query heads per KV head = 16 MFMA columns)."""
    rng = np.random.default_rng(seed)
    ctx = log_uniform_lengths(rng, num_seqs, 256, 8192)
    return build("spec_verify", seed, rng, ctx, 32, 8, 128, 16, "bf16", max_blocks=512,
                 poison=poison, query_lens=np.full(num_seqs, draft, dtype=np.int32))


def prefill_chunk(seed=388007, poison=False, num_seqs=8, chunk=256):
    """Chunked prefill on the Llama-3-8B-shaped GQA layer: ``num_seqs``
    prompts, each processing a chunk of ``chunk`` new tokens on top of an
    earlier context (total contexts uniform in [chunk, 4096]), bf16."""
    rng = np.random.default_rng(seed)
    ctx = uniform_lengths(rng, num_seqs, chunk, 4096)
    return build("prefill_chunk", seed, rng, ctx, 32, 8, 128, 16, "bf16", max_blocks=256,
                 poison=poison, query_lens=np.full(num_seqs, chunk, dtype=np.int32))


def long_prompt_chunk(seed=388010, poison=False, context=32768, chunk=256):
    """Chunked prefill of one long prompt on the Llama-3-8B-shaped GQA layer:
    the chunk of ``chunk`` new tokens that ends a ``context``-token prompt
    (each new token attends to everything before it), bf16.  A single
    sequence gives the prefill path only 16 x 8 (column block, kv head)
    workgroups, so its context is cut into parts."""
    rng = np.random.default_rng(seed)
    return build("long_prompt_chunk", seed, rng, [context], 32, 8, 128, 16, "bf16",
                 poison=poison, query_lens=[chunk])


def named(name, **kw):
    """Build a named workload: one of NAMED, or ``long_ctx_bs16``/``long_ctx_bs32``."""
    if name == "tiny_f32":
        return tiny_f32(**kw)
    if name == "llama2_7b_f16":
        return llama2_7b_f16(**kw)
    if name == "llama3_8b_gqa":
        return llama3_8b_gqa(**kw)
    if name == "shared_prefix":
        return shared_prefix(**kw)
    if name in ("long_ctx", "long_ctx_bs16"):
        return long_ctx(block_size=16, **kw)
    if name == "long_ctx_bs32":
        return long_ctx(block_size=32, **kw)
    if name == "spec_verify":
        return spec_verify(**kw)
    if name == "prefill_chunk":
        return prefill_chunk(**kw)
    if name == "long_prompt_chunk":
        return long_prompt_chunk(**kw)
    raise KeyError(name)
