"""Pins for the CPU oracle: each check ties it to something other than itself.

* values the pages print (``tests/golden/*.txt``, each with its citation);
* closed forms of softmax attention;
* brute force on tiny inputs against unpaged attention written independently
  here, and against torch's scaled-dot-product attention in fp64;
* the invariants the pages state: physical placement does not matter, shared
  blocks equal private copies, copy-on-write leaves the shared block unchanged;
* the exact identity behind split-context decoding.

A final group plants plausible mistakes in copies of the oracle and checks
that these pins reject every one of them.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import paged_attention as pa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------
# helpers that build paged inputs from contiguous ones (test-side scatter)
# ---------------------------------------------------------------------------

def _round(x, dtype):
    """fp32 values -> (stored array, exact fp64 value of what was stored)."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy(), x.astype(np.float64)
    if dtype == "f16":
        h = x.astype(np.float16)
        return h.view(np.uint16).copy(), h.astype(np.float64)
    t = torch.from_numpy(x.copy()).to(torch.bfloat16)
    return (t.view(torch.int16).numpy().view(np.uint16).copy(),
            t.to(torch.float64).numpy())


def _paged_from_contiguous(kc, vc, ctx, bs, rng, extra_blocks=3, dtype="f32"):
    """Scatter contiguous K/V [B, H_kv, n_max, D] (already stored values) into
    a shuffled pool [NB, H_kv, bs, D].  Unused slots and blocks are filled with
    NaN so that reading them would show."""
    B, H_kv, n_max, D = kc.shape
    nbs = [-(-int(n) // bs) for n in ctx]
    NB = sum(nbs) + extra_blocks
    perm = rng.permutation(NB)
    max_blocks = max(1, max(nbs))
    bt = np.full((B, max_blocks), -1, dtype=np.int32)
    nan = {"f32": np.float32(np.nan), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}[dtype]
    kpool = np.full((NB, H_kv, bs, D), nan, dtype=kc.dtype)
    vpool = np.full((NB, H_kv, bs, D), nan, dtype=vc.dtype)
    nxt = 0
    for s in range(B):
        for j in range(nbs[s]):
            phys = int(perm[nxt])
            nxt += 1
            bt[s, j] = phys
            for t in range(j * bs, min((j + 1) * bs, int(ctx[s]))):
                kpool[phys, :, t - j * bs, :] = kc[s, :, t, :]
                vpool[phys, :, t - j * bs, :] = vc[s, :, t, :]
    return kpool, vpool, bt


def _make_case(rng, B, H_q, H_kv, D, ctx, bs, dtype):
    n_max = max(1, max(ctx))
    q_st, q64 = _round(rng.standard_normal((B, H_q, D)), dtype)
    k_st, k64 = _round(rng.standard_normal((B, H_kv, n_max, D)), dtype)
    v_st, v64 = _round(rng.standard_normal((B, H_kv, n_max, D)), dtype)
    kpool, vpool, bt = _paged_from_contiguous(k_st, v_st, ctx, bs, rng, dtype=dtype)
    return dict(q=q_st, kpool=kpool, vpool=vpool, bt=bt,
                ctx=np.array(ctx, dtype=np.int32), q64=q64, k64=k64, v64=v64)


def _loop_attention(q64, k64, v64, ctx, scale, G):
    """Unpaged attention over contiguous arrays with Python loops and math.exp;
    written independently of the oracle."""
    B, H_q, D = q64.shape
    out = np.zeros((B, H_q, D))
    for s in range(B):
        n = int(ctx[s])
        if n == 0:
            continue
        for h in range(H_q):
            kvh = h // G
            sc = [scale * sum(q64[s, h, d] * k64[s, kvh, t, d] for d in range(D))
                  for t in range(n)]
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            den = sum(e)
            for d in range(D):
                out[s, h, d] = sum(e[t] * v64[s, kvh, t, d] for t in range(n)) / den
    return out


def _sdpa_attention(q64, k64, v64, ctx, scale, G):
    """torch's scaled_dot_product_attention in fp64 on CPU, KV heads repeated."""
    B, H_q, D = q64.shape
    out = np.zeros((B, H_q, D))
    for s in range(B):
        n = int(ctx[s])
        if n == 0:
            continue
        q = torch.from_numpy(q64[s]).reshape(1, H_q, 1, D)
        k = torch.from_numpy(k64[s, :, :n]).repeat_interleave(G, dim=0).reshape(1, H_q, n, D)
        v = torch.from_numpy(v64[s, :, :n]).repeat_interleave(G, dim=0).reshape(1, H_q, n, D)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
        out[s] = o.reshape(H_q, D).numpy()
    return out


# ---------------------------------------------------------------------------
# storage decoding
# ---------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x3FC0, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001,
                     0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.5, math.inf, -math.inf, 0.0, -0.0, 2.0 ** -133, 3.140625]
    got = oracle.storage_to_f64(pats, "bf16")
    assert list(got) == want
    assert math.copysign(1.0, got[6]) == -1.0


def test_storage_decode_matches_torch_on_all_16bit_patterns():
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dtype, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        ref = torch.from_numpy(pats.view(np.int16).copy()).view(tdt).to(torch.float64).numpy()
        got = oracle.storage_to_f64(pats, dtype)
        fin = np.isfinite(ref)
        assert np.array_equal(got[fin], ref[fin])
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


# ---------------------------------------------------------------------------
# values printed on the pages
# ---------------------------------------------------------------------------

def test_block_counting_golden():
    rows = _rows("block_counting.txt")
    assert len(rows) == 3
    for tokens, bs, blocks, last, free in (map(int, r) for r in rows):
        assert oracle.blocks_for_tokens(tokens, bs) == blocks
        assert oracle.last_block_fill(tokens, bs) == (last, free)


def test_tail_waste_golden():
    (bs, exact, page), = _rows("tail_waste.txt")
    assert oracle.mean_tail_waste(int(bs)) == float(exact)
    assert round(oracle.mean_tail_waste(int(bs))) == int(page)


def test_kv_bytes_golden():
    for model, L, H, D, b, per_tok, T, total in _rows("kv_bytes.txt"):
        got = oracle.kv_bytes_per_token(int(L), int(H), int(D), int(b))
        assert got == int(per_tok), model
        assert got * int(T) == int(total), model
    # The page figures: about 800 KiB / 1.6 GiB for OPT-13B, 1-2 GB for Llama-2-7B.
    assert oracle.kv_bytes_per_token(40, 40, 128, 2) / 1024 == 800
    assert abs(oracle.kv_bytes_per_token(40, 40, 128, 2) * 2048 / 2 ** 30 - 1.6) < 0.05
    assert 1e9 <= oracle.kv_bytes_per_token(32, 32, 128, 2) * 2048 <= 2e9


def test_shared_prefix_golden():
    (users, prefix, unshared, shared), = (list(map(int, r)) for r in _rows("shared_prefix.txt"))
    assert users * prefix == unshared and prefix == shared
    # in blocks: every user's table names the same physical prefix blocks
    nb = oracle.blocks_for_tokens(prefix, 16)
    assert nb == 313


def test_block_table_examples_gather_order():
    """Gathering follows the printed logical->physical maps: tag every
    physical block with its own id and read the tags back in logical order."""
    NB, H, bs, D = 16, 1, 4, 2
    pool = np.zeros((NB, H, bs, D), dtype=np.float32)
    for b in range(NB):
        pool[b] = b
    for row in _rows("block_table_examples.txt"):
        pairs = [tuple(map(int, x.split(":"))) for x in row[1:]]
        table = np.array([p for _, p in sorted(pairs)], dtype=np.int32)
        n = len(table) * bs - 1                       # last block partial
        ctx = oracle.gather_context(pool, table, n, "f32")
        assert ctx.shape == (H, n, D)
        want = np.repeat(table.astype(np.float64), bs)[:n]
        assert np.array_equal(ctx[0, :, 0], want)


# ---------------------------------------------------------------------------
# brute force against unpaged attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("H_q,H_kv", [(2, 2), (4, 2), (4, 1)])
def test_brute_force_vs_unpaged(dtype, H_q, H_kv):
    rng = np.random.default_rng(11)
    ctx = [1, 4, 5, 9, 0]
    bs, D = 4, 8
    c = _make_case(rng, len(ctx), H_q, H_kv, D, ctx, bs, dtype)
    scale = 1 / math.sqrt(D)
    got = oracle.decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], scale, dtype)
    G = H_q // H_kv
    loop = _loop_attention(c["q64"], c["k64"], c["v64"], c["ctx"], scale, G)
    sdpa = _sdpa_attention(c["q64"], c["k64"], c["v64"], c["ctx"], scale, G)
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got - loop)) <= 1e-12
    assert np.max(np.abs(got - sdpa)) <= 1e-12


def test_brute_force_larger_sdpa():
    rng = np.random.default_rng(12)
    ctx = [1, 15, 16, 17, 31, 32, 33, 70]
    c = _make_case(rng, len(ctx), 8, 2, 64, ctx, 16, "bf16")
    scale = 0.125
    got = oracle.decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], scale, "bf16")
    ref = _sdpa_attention(c["q64"], c["k64"], c["v64"], c["ctx"], scale, 4)
    assert np.max(np.abs(got - ref)) <= 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    c = _make_case(rng, 3, 4, 2, 8, [1, 1, 1], 4, "f32")
    got = oracle.decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], 0.7, "f32")
    for s in range(3):
        for h in range(4):
            assert np.array_equal(got[s, h], c["v64"][s, h // 2, 0])


def test_zero_scale_and_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    ctx = [3, 7, 16, 21]
    c = _make_case(rng, 4, 2, 2, 8, ctx, 8, "f32")
    got = oracle.decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], 0.0, "f32")
    for s, n in enumerate(ctx):
        for h in range(2):
            assert np.allclose(got[s, h], c["v64"][s, h, :n].mean(axis=0), rtol=0, atol=1e-14)
    # identical K rows: every score equal whatever the scale
    kc = np.repeat(c["k64"][:, :, :1, :], c["k64"].shape[2], axis=2).astype(np.float32)
    kpool, vpool, bt = _paged_from_contiguous(kc, c["v64"].astype(np.float32), ctx, 8,
                                              np.random.default_rng(3))
    got = oracle.decode_attention(c["q"], kpool, vpool, bt, c["ctx"], 1.3, "f32")
    for s, n in enumerate(ctx):
        assert np.allclose(got[s, 0], c["v64"][s, 0, :n].mean(axis=0), rtol=0, atol=1e-14)


def test_constant_values_are_returned():
    rng = np.random.default_rng(4)
    ctx = [2, 9, 33]
    c = _make_case(rng, 3, 2, 1, 16, ctx, 16, "f32")
    vconst = np.full_like(c["v64"], 0.375).astype(np.float32)
    kpool, vpool, bt = _paged_from_contiguous(c["k64"].astype(np.float32), vconst, ctx, 16,
                                              np.random.default_rng(5))
    got = oracle.decode_attention(c["q"], kpool, vpool, bt, c["ctx"], 0.25, "f32")
    assert np.allclose(got, 0.375, rtol=0, atol=1e-15)


def test_two_tokens_sigmoid_form():
    rng = np.random.default_rng(6)
    c = _make_case(rng, 2, 2, 2, 8, [2, 2], 4, "f32")
    scale = 0.9
    got = oracle.decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], scale, "f32")
    for s in range(2):
        for h in range(2):
            s0 = scale * c["q64"][s, h] @ c["k64"][s, h, 0]
            s1 = scale * c["q64"][s, h] @ c["k64"][s, h, 1]
            w0 = 1.0 / (1.0 + math.exp(s1 - s0))
            w1 = 1.0 / (1.0 + math.exp(s0 - s1))
            want = w0 * c["v64"][s, h, 0] + w1 * c["v64"][s, h, 1]
            assert np.max(np.abs(got[s, h] - want)) <= 1e-14


def test_empty_context_gives_zeros():
    rng = np.random.default_rng(7)
    c = _make_case(rng, 3, 2, 2, 8, [0, 5, 0], 4, "bf16")
    got = oracle.decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], 0.3, "bf16")
    assert np.array_equal(got[0], np.zeros((2, 8)))
    assert np.array_equal(got[2], np.zeros((2, 8)))
    assert np.all(np.isfinite(got[1])) and np.any(got[1] != 0)


# ---------------------------------------------------------------------------
# invariants the pages state
# ---------------------------------------------------------------------------

def test_physical_permutation_invariance_bitwise():
    """Logical order, not physical placement, defines the result."""
    rng = np.random.default_rng(8)
    ctx = [5, 16, 33, 70]
    c = _make_case(rng, 4, 4, 2, 16, ctx, 16, "bf16")
    base = oracle.decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], 0.25, "bf16")
    NB = c["kpool"].shape[0]
    pi = rng.permutation(NB)
    kp = np.empty_like(c["kpool"])
    vp = np.empty_like(c["vpool"])
    kp[pi] = c["kpool"]
    vp[pi] = c["vpool"]
    bt = np.where(c["bt"] >= 0, pi[np.maximum(c["bt"], 0)], -1).astype(np.int32)
    moved = oracle.decode_attention(c["q"], kp, vp, bt, c["ctx"], 0.25, "bf16")
    assert np.array_equal(base, moved)


def test_shared_prefix_equals_private_copies_bitwise():
    rng = np.random.default_rng(9)
    B, H_q, H_kv, D, bs = 5, 4, 2, 8, 4
    prefix_blocks = 3
    NB = prefix_blocks + B * 2 + 2
    kpool = rng.standard_normal((NB, H_kv, bs, D)).astype(np.float32)
    vpool = rng.standard_normal((NB, H_kv, bs, D)).astype(np.float32)
    q = rng.standard_normal((B, H_q, D)).astype(np.float32)
    ctx = np.array([prefix_blocks * bs + 1 + s for s in range(B)], dtype=np.int32)
    bt = np.full((B, prefix_blocks + 2), -1, dtype=np.int32)
    for s in range(B):
        bt[s, :prefix_blocks] = [0, 1, 2]
        bt[s, prefix_blocks] = prefix_blocks + 2 * s
        bt[s, prefix_blocks + 1] = prefix_blocks + 2 * s + 1
    shared = oracle.decode_attention(q, kpool, vpool, bt, ctx, 0.35, "f32")
    # duplicate the prefix blocks per sequence
    kd = np.concatenate([kpool] + [kpool[:prefix_blocks]] * B)
    vd = np.concatenate([vpool] + [vpool[:prefix_blocks]] * B)
    bt2 = bt.copy()
    for s in range(B):
        bt2[s, :prefix_blocks] = NB + s * prefix_blocks + np.arange(prefix_blocks)
    private = oracle.decode_attention(q, kd, vd, bt2, ctx, 0.35, "f32")
    assert np.array_equal(shared, private)


def test_poisoned_free_blocks_and_tail_slots_do_not_matter():
    rng = np.random.default_rng(10)
    ctx = [5, 17, 32]
    c = _make_case(rng, 3, 2, 2, 8, ctx, 16, "f16")   # pool already NaN-filled
    got = oracle.decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], 0.3, "f16")
    assert np.all(np.isfinite(got))
    # replace the NaNs by ordinary numbers: same result
    kp = c["kpool"].copy()
    vp = c["vpool"].copy()
    kp[kp == 0x7E00] = 0x3C00
    vp[vp == 0x7E00] = 0x4000
    again = oracle.decode_attention(c["q"], kp, vp, c["bt"], c["ctx"], 0.3, "f16")
    assert np.array_equal(got, again)


def test_split_partitions_merge_to_the_unsplit_result():
    rng = np.random.default_rng(13)
    ctx = [1, 16, 17, 100, 513]
    c = _make_case(rng, len(ctx), 4, 2, 16, ctx, 16, "bf16")
    whole = oracle.decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], 0.25, "bf16")
    for P in (1, 16, 37, 512, 4096):
        split = oracle.split_decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"],
                                              0.25, "bf16", P)
        assert np.max(np.abs(split - whole)) <= 1e-12, P


def test_merge_of_two_hand_partitions():
    # partition A: scores {0, ln 3} -> m = ln 3, l = 1/3 + 1, o = v0/3 + v1
    # partition B: score {ln 2}     -> m = ln 2, l = 1,      o = v2
    v = np.array([[3.0], [6.0], [9.0]])
    ms = np.array([math.log(3), math.log(2)])
    ls = np.array([1 / 3 + 1, 1.0])
    os_ = np.array([v[0] / 3 + v[1], v[2]])
    # weights 1 : 3 : 2 over v0, v1, v2
    want = (1 * 3.0 + 3 * 6.0 + 2 * 9.0) / 6
    assert abs(oracle.merge_partitions(ms, ls, os_)[0] - want) <= 1e-14


# ---------------------------------------------------------------------------
# append and copy-on-write
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_writes_each_slot_once_and_nothing_else(dtype):
    rng = np.random.default_rng(14)
    NB, H, bs, D, T = 6, 3, 4, 5, 7
    store = np.float32 if dtype == "f32" else np.uint16
    kpool = rng.integers(0, 30000, (NB, H, bs, D)).astype(store)
    vpool = rng.integers(0, 30000, (NB, H, bs, D)).astype(store)
    key = rng.integers(30000, 60000, (T, H, D)).astype(store)
    val = rng.integers(30000, 60000, (T, H, D)).astype(store)
    slots = rng.choice(NB * bs, size=T, replace=False).astype(np.int32)
    slots[2] = -1
    k2, v2 = oracle.kv_append(kpool, vpool, key, val, slots)
    owner = {int(s): i for i, s in enumerate(slots) if s >= 0}
    for b in range(NB):
        for h in range(H):
            for o in range(bs):
                i = owner.get(b * bs + o)
                if i is None:
                    assert np.array_equal(k2[b, h, o], kpool[b, h, o])
                    assert np.array_equal(v2[b, h, o], vpool[b, h, o])
                else:
                    assert np.array_equal(k2[b, h, o], key[i, h])
                    assert np.array_equal(v2[b, h, o], val[i, h])
    # inputs untouched
    assert not np.array_equal(k2, kpool)


def test_append_copies_nan_payload_bits():
    kpool = np.zeros((2, 1, 2, 1), dtype=np.float32)
    key = np.array([[[0]]], dtype=np.uint32)
    key[...] = 0x7FC01234
    key = key.view(np.float32)
    k2, _ = oracle.kv_append(kpool, kpool, key, key, np.array([3], dtype=np.int32))
    assert k2.view(np.uint32)[1, 0, 1, 0] == 0x7FC01234


def test_copy_blocks_copy_on_write():
    rng = np.random.default_rng(15)
    NB, H, bs, D = 8, 2, 4, 3
    kpool = rng.integers(0, 60000, (NB, H, bs, D)).astype(np.uint16)
    vpool = rng.integers(0, 60000, (NB, H, bs, D)).astype(np.uint16)
    pairs = np.array([[1, 5], [1, 6], [2, 7]], dtype=np.int32)
    k2, v2 = oracle.copy_blocks(kpool, vpool, pairs)
    for src, dst in pairs:
        assert np.array_equal(k2[dst], kpool[src])
        assert np.array_equal(v2[dst], vpool[src])
    for b in (0, 1, 2, 3, 4):
        assert np.array_equal(k2[b], kpool[b])          # shared blocks unchanged
        assert np.array_equal(v2[b], vpool[b])
    with pytest.raises(ValueError):
        oracle.copy_blocks(kpool, vpool, np.array([[1, 5], [2, 5]]))
    with pytest.raises(ValueError):
        oracle.copy_blocks(kpool, vpool, np.array([[1, 5], [5, 6]]))


def test_cow_then_append_leaves_the_shared_block_and_other_readers_unchanged():
    rng = np.random.default_rng(16)
    H_q, H_kv, D, bs = 2, 1, 8, 4
    NB = 6
    kpool = rng.standard_normal((NB, H_kv, bs, D)).astype(np.float32)
    vpool = rng.standard_normal((NB, H_kv, bs, D)).astype(np.float32)
    q = rng.standard_normal((2, H_q, D)).astype(np.float32)
    # both sequences share blocks 0 and 1 (the last holds 2 of 4 tokens)
    bt = np.array([[0, 1], [0, 1]], dtype=np.int32)
    ctx = np.array([6, 6], dtype=np.int32)
    before = oracle.decode_attention(q, kpool, vpool, bt, ctx, 0.5, "f32")
    # sequence 1 writes a token: it gets its own copy of block 1 first
    k2, v2 = oracle.copy_blocks(kpool, vpool, np.array([[1, 4]]))
    new = rng.standard_normal((1, H_kv, D)).astype(np.float32)
    k3, v3 = oracle.kv_append(k2, v2, new, new, np.array([4 * bs + 2], dtype=np.int32))
    bt2 = np.array([[0, 1], [0, 4]], dtype=np.int32)
    ctx2 = np.array([6, 7], dtype=np.int32)
    after = oracle.decode_attention(q, k3, v3, bt2, ctx2, 0.5, "f32")
    assert np.array_equal(k3[1], kpool[1]) and np.array_equal(v3[1], vpool[1])
    assert np.array_equal(after[0], before[0])
    assert not np.array_equal(after[1], before[1])


# ---------------------------------------------------------------------------
# planted mistakes: copies of the oracle with one plausible bug each must be
# rejected by the pins above (run on the CPU only)
# ---------------------------------------------------------------------------

def _mutant_decode(kind):
    def run(q, k_cache, v_cache, block_tables, context_lens, scale, dtype):
        B, H_q, D = q.shape
        H_kv = k_cache.shape[1]
        G = H_q // H_kv
        out = np.zeros((B, H_q, D))
        for s in range(B):
            n = int(context_lens[s])
            if n == 0:
                continue
            n_read = n - 1 if kind == "drop_last" and n > 1 else n
            row = block_tables[s]
            if kind == "reverse_blocks":
                nb = pa.blocks_for_tokens(n, k_cache.shape[2])
                row = row[:nb][::-1]
            K = pa.gather_context(k_cache, row, n_read, dtype)
            V = pa.gather_context(v_cache, row, n_read, dtype)
            qs = pa.storage_to_f64(q[s], dtype)
            for h in range(H_q):
                kv = h % H_kv if kind == "head_modulo" else h // G
                sc = (K[kv] @ qs[h]) * (1.0 if kind == "no_scale" else scale)
                p = np.exp(sc - sc.max())
                if kind == "transposed_v":
                    out[s, h] = (p @ V[(kv + 1) % H_kv]) / p.sum()
                else:
                    out[s, h] = (p @ V[kv]) / p.sum()
        return out
    return run


@pytest.mark.parametrize("kind", ["drop_last", "reverse_blocks", "head_modulo",
                                  "no_scale", "transposed_v"])
def test_pins_reject_planted_mistakes(kind):
    rng = np.random.default_rng(17)
    ctx = [1, 4, 5, 9]
    c = _make_case(rng, len(ctx), 4, 2, 8, ctx, 4, "f32")
    scale = 1 / math.sqrt(8)
    ref = _sdpa_attention(c["q64"], c["k64"], c["v64"], c["ctx"], scale, 2)
    bad = _mutant_decode(kind)(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], scale, "f32")
    ok = _mutant_decode("none")(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], scale, "f32")
    assert np.max(np.abs(ok - ref)) <= 1e-12
    assert not (np.max(np.abs(bad - ref)) <= 1e-12)


# ---------------------------------------------------------------------------
# swap to host memory and back
# ---------------------------------------------------------------------------

def _coordinate_pools(NB, H, bs, D):
    """Pools whose every element encodes its own (K or V, block, head, token,
    dim), so an image element tells where it was read from."""
    kv, b, h, t, d = np.meshgrid(np.arange(2), np.arange(NB), np.arange(H), np.arange(bs),
                                 np.arange(D), indexing="ij")
    code = ((((kv * 100 + b) * 10 + h) * 100 + t) * 100 + d).astype(np.uint32)
    return code[0], code[1]


def test_swap_out_image_entries_name_their_source():
    NB, H, bs, D = 7, 3, 4, 5
    kpool, vpool = _coordinate_pools(NB, H, bs, D)
    ids = [5, 0, 5, 3]
    img = oracle.swap_out(kpool, vpool, ids)
    assert img.shape == (4, 2, H, bs, D)
    for i, b in enumerate(ids):
        for kv in range(2):
            for h in range(H):
                for t in range(bs):
                    for d in range(D):
                        want = (((kv * 100 + b) * 10 + h) * 100 + t) * 100 + d
                        assert img[i, kv, h, t, d] == want
    # ids outside the pool give zero entries
    img = oracle.swap_out(kpool, vpool, [NB, -1, 2])
    assert not img[0].any() and not img[1].any()
    assert img[2, 1, 2, 3, 4] == (((100 + 2) * 10 + 2) * 100 + 3) * 100 + 4


def test_swap_round_trip_and_moved_blocks_keep_attention():
    """A sequence swapped out and brought back into other blocks, with its
    table rewritten, attends exactly as before; blocks not named are left
    alone."""
    rng = np.random.default_rng(17)
    H_q, H_kv, D, bs, NB = 4, 2, 8, 4, 12
    kpool = rng.standard_normal((NB, H_kv, bs, D)).astype(np.float32)
    vpool = rng.standard_normal((NB, H_kv, bs, D)).astype(np.float32)
    q = rng.standard_normal((1, H_q, D)).astype(np.float32)
    table = np.array([[3, 9, 1]], dtype=np.int32)
    ctx = np.array([10], dtype=np.int32)
    before = oracle.decode_attention(q, kpool, vpool, table, ctx, 0.3, "f32")
    img = oracle.swap_out(kpool, vpool, table[0])
    # the pool is reused meanwhile: scribble over the old blocks
    wiped_k, wiped_v = kpool.copy(), vpool.copy()
    wiped_k[[3, 9, 1]] = np.nan
    wiped_v[[3, 9, 1]] = np.nan
    new_ids = [0, 11, 6]
    k2, v2 = oracle.swap_in(wiped_k, wiped_v, img, new_ids)
    after = oracle.decode_attention(q, k2, v2, np.array([new_ids], dtype=np.int32), ctx, 0.3, "f32")
    assert np.array_equal(before, after)
    for b in range(NB):
        if b not in new_ids:
            assert np.array_equal(k2[b], wiped_k[b], equal_nan=True)
    # swap_in of the image at the original ids is the identity on those blocks
    k3, v3 = oracle.swap_in(wiped_k, wiped_v, img, table[0])
    assert np.array_equal(k3[table[0]], kpool[table[0]]) and np.array_equal(v3[table[0]], vpool[table[0]])
    with pytest.raises(ValueError):
        oracle.swap_in(kpool, vpool, img, [2, 2, 4])
    k4, _ = oracle.swap_in(kpool, vpool, img, [NB, -1, 4])       # outside the pool: skipped
    assert np.array_equal(k4[4], kpool[1]) and np.array_equal(np.delete(k4, 4, 0), np.delete(kpool, 4, 0))
