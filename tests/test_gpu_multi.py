"""Multi-token paged attention (several new tokens per sequence) on the GPU
against the CPU oracle, through the C ABI (needs an MI355X).

Ragged numbers of new tokens per sequence, every dtype / head_dim /
block_size, query-head groups of 1 to 16, column groups beyond one MFMA tile
(L * G > 16), whole-context chunks (L = n), empty sequences, NaN-poisoned
pools; bit-identical results under a physical permutation of the pool.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_388_amd import _lib
from paged_kv_cache_388_amd import workloads as wl

from gpu_common import (DeviceWorkload, abs_pool, check_attention, check_step,
                        takes_fp16_pv, to_host)

pytestmark = pytest.mark.gpu

CTX = [1, 5, 16, 17, 40, 300, 513, 700]
QLENS = [1, 5, 3, 17, 0, 7, 16, 2]


def _run(w, what):
    print(f"[gpu] {what}: B={w.num_seqs} T={w.q.shape[0]} Hq={w.num_q_heads} "
          f"Hkv={w.num_kv_heads} D={w.head_dim} bs={w.block_size} {w.dtype} "
          f"maxq={w.max_query_len} maxctx={w.max_context_len}", flush=True)
    dw = DeviceWorkload(w)
    out = dw.step()
    torch.cuda.synchronize()
    return check_step(to_host(out, w.dtype), w, what)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_multi_grid(dtype, D, bs, G):
    rng = np.random.default_rng(41)
    w = wl.build(f"multi_{dtype}_{D}_{bs}_{G}", 41, rng, CTX, 2 * G, 2, D, bs, dtype,
                 poison=True, query_lens=QLENS)
    _run(w, f"multi {dtype} D{D} bs{bs} G{G}")


@pytest.mark.parametrize("G", [3, 16])
def test_multi_other_groups(G):
    rng = np.random.default_rng(42)
    w = wl.build(f"multi_G{G}", 42, rng, [9, 130, 600], G, 1, 128, 16, "bf16", poison=True,
                 query_lens=[9, 4, 11])
    _run(w, f"multi G{G}")


@pytest.mark.parametrize("mult", [-1.0, 0.0, 3.0])
@pytest.mark.parametrize("path,dtype", [("decode", "bf16"), ("stream", "bf16"), ("prefill", "bf16"),
                                        ("prefill", "f16")])
def test_scale_negative_zero_and_large(path, dtype, mult):
    """The logit scale is a caller argument of any sign: a negative scale
    attends by the negated scores, a zero scale weighs every visible token
    equally, a large one peaks the softmax.  Decode, the multi-token stream
    path (L * G <= 16) and the prefill path (L * G >= 64) against the oracle."""
    rng = np.random.default_rng(60)
    ctx = [1, 17, 300, 700]
    qlens = {"decode": None, "stream": [1, 3, 4, 2], "prefill": [1, 17, 32, 20]}[path]
    w = wl.build(f"scale_{path}_{mult}", 60, rng, ctx, 8, 2, 128, 16, dtype,
                 scale=mult / np.sqrt(128), poison=True, query_lens=qlens)
    if path == "prefill":
        assert w.max_query_len * 4 >= 64
    _run(w, f"{path} {dtype} scale {mult}/sqrt(D)")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("plan", ["one_group_per_wave", "two_groups_per_wave"])
def test_prefill_path_wave_group_plans(dtype, D, plan):
    """The prefill path runs one or two 16-column groups per wave by the
    call's workgroup count: 64 sequences x 8 kv heads with 32 new tokens at
    G = 4 (8 groups, one 8-group block each) give 512 two-group workgroups,
    which takes one group per wave; 128 sequences give 1024, which takes two.
    Ragged new-token counts and contexts, NaN-poisoned pools."""
    B = 64 if plan == "one_group_per_wave" else 128
    rng = np.random.default_rng(61)
    ctx = rng.integers(32, 200, size=B).tolist()
    qlens = [32] + rng.integers(1, 33, size=B - 1).tolist()
    w = wl.build(f"pf_plan_{plan}_{dtype}", 61, rng, ctx, 32, 8, D, 16, dtype, poison=True,
                 query_lens=qlens)
    assert w.max_query_len * 4 >= 64
    _run(w, f"prefill path, {plan}, {dtype} D{D}")


@pytest.mark.parametrize("G", [3, 5])
@pytest.mark.parametrize("batch", ["64_sequences", "3_sequences_split"])
def test_prefill_path_groups_straddling_tokens(G, batch):
    """Query-head groups that do not divide 16: a 16-column group straddles
    new tokens and a column block ends inside one.  64 sequences x 8 kv heads
    with 32 new tokens give 512 two-group workgroups at G = 3 (one group per
    wave, 4-group blocks) and 1024 at G = 5 (two groups per wave, 8-group
    blocks); 3 sequences x 2 kv heads with up to 100 new tokens give 18 or 24
    (two groups per wave, contexts cut into two parts and merged)."""
    rng = np.random.default_rng(62)
    if batch == "64_sequences":
        B, Hkv = 64, 8
        ctx = rng.integers(40, 300, size=B).tolist()
        qlens = [32] + rng.integers(1, 33, size=B - 1).tolist()
    else:
        B, Hkv = 3, 2
        ctx, qlens = [700, 90, 1500], [64, 30, 100]
    w = wl.build(f"pf_G{G}_{batch}", 62, rng, ctx, G * Hkv, Hkv, 128, 16, "bf16", poison=True,
                 query_lens=qlens)
    assert w.max_query_len * G >= 64
    _run(w, f"prefill path G={G}, {batch}")


def test_whole_context_chunks():
    rng = np.random.default_rng(43)
    ctx = [1, 16, 33, 64]
    w = wl.build("whole", 43, rng, ctx, 8, 2, 128, 16, "bf16", poison=True, query_lens=ctx)
    _run(w, "L = n")


def test_one_token_each_matches_decode_bitwise():
    rng = np.random.default_rng(44)
    ctx = [3, 200, 900, 2100]
    w = wl.build("one", 44, rng, ctx, 16, 4, 128, 16, "bf16", query_lens=[1, 1, 1, 1])
    multi = to_host(DeviceWorkload(w).step(), "bf16")
    w.query_start = None
    dec = to_host(DeviceWorkload(w).step(), "bf16")
    assert np.array_equal(multi, dec)


def test_physical_permutation_invariance_bitwise():
    rng = np.random.default_rng(45)
    w = wl.build("perm", 45, rng, [20, 600, 1500], 32, 8, 128, 16, "bf16", query_lens=[4, 4, 4])
    base = to_host(DeviceWorkload(w).step(), "bf16")
    dw = DeviceWorkload(w)
    dw.write_step()
    kc, vc = to_host(dw.k_cache, "bf16"), to_host(dw.v_cache, "bf16")
    pi = np.random.default_rng(46).permutation(kc.shape[0])
    kp, vp = np.empty_like(kc), np.empty_like(vc)
    kp[pi], vp[pi] = kc, vc
    bt = np.where(w.block_tables >= 0, pi[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    w2 = wl.Workload(name="perm2", dtype="bf16", seed=0, q=w.q, k_cache=kp, v_cache=vp,
                     block_tables=bt, context_lens=w.context_lens, scale=w.scale,
                     block_mapping=np.zeros((0, 2), np.int32), slot_mapping=np.zeros((0,), np.int32),
                     new_key=w.new_key[:0], new_value=w.new_value[:0], query_start=w.query_start)
    moved = to_host(DeviceWorkload(w2).step(), "bf16")
    assert np.array_equal(base, moved)


def test_too_many_sequences_refused():
    rng = np.random.default_rng(47)
    w = wl.build("big", 47, rng, np.full(2049, 2), 4, 1, 64, 16, "f16",
                 query_lens=np.full(2049, 1))
    dw = DeviceWorkload(w)
    with pytest.raises(_lib.PagedKVError):
        dw.attend()


@pytest.mark.parametrize("name", ["spec_verify", "prefill_chunk", "long_prompt_chunk"])
def test_full_size_multi_workloads(name):
    """Every row of the full-size multi-token workloads (the long prompt's
    context cut into parts and merged) against the oracle, on NaN-poisoned
    pools."""
    w = wl.named(name, poison=True)
    err = _run(w, name)
    print(f"[gpu] {name}: max |gpu - oracle| = {err:.3e}", flush=True)


# ---------------------------------------------------------------------------
# the prefill path (max_query_len * G >= 64): one workgroup per (sequence,
# kv head, 64 columns), longest context first up to 256 sequences
# ---------------------------------------------------------------------------

def test_prefill_path_ranked_ties_and_mixed_lengths():
    """Equal contexts (rank ties), sequences with 0, 1 and many new tokens,
    a chunk longer than one 64-column block, an empty context."""
    rng = np.random.default_rng(48)
    ctx = [700, 700, 65, 1300, 0, 700, 31]
    ql = [40, 1, 17, 64, 0, 0, 31]
    w = wl.build("pf_mixed", 48, rng, ctx, 8, 2, 128, 16, "bf16", poison=True, query_lens=ql)
    assert w.max_query_len * 4 >= 64
    # 7 sequences x 2 kv heads x 4 column blocks = 56 workgroups: contexts are
    # cut in two (1300 // 512 caps the parts), part states for 7 x 64 rows x 8 heads
    rows, parts, D = 7 * 64, 2, 128
    want = -(-(rows * 8 * parts * D * 4) // 256) * 256 + rows * 8 * parts * 2 * 4
    assert _lib.paged_attention_multi_workspace_bytes(
        DeviceWorkload(w).k_cache, w.num_seqs, w.num_q_heads, w.max_query_len,
        w.max_context_len) == want
    _run(w, "prefill path, ranked")


@pytest.mark.parametrize("dtype,D,bs", [("f16", 64, 32), ("f32", 128, 16)])
def test_prefill_path_more_than_ranked_sequences(dtype, D, bs):
    """300 sequences: past the ranking limit, dispatched in index order."""
    rng = np.random.default_rng(49)
    ctx = rng.integers(1, 90, size=300)
    ctx[7] = max(int(ctx[7]), 20)
    ql = np.minimum(rng.integers(0, 22, size=300), ctx)
    ql[7] = 20
    w = wl.build(f"pf_many_{dtype}", 49, rng, ctx, 4, 1, D, bs, dtype, poison=True, query_lens=ql)
    assert w.max_query_len * 4 >= 64
    _run(w, f"prefill path, 300 sequences {dtype}")


def test_prefill_path_permutation_invariance_bitwise():
    rng = np.random.default_rng(50)
    w = wl.build("pfperm", 50, rng, [20, 600, 1500], 32, 8, 128, 16, "bf16",
                  query_lens=[20, 32, 32])
    assert w.max_query_len * 4 >= 64
    base = to_host(DeviceWorkload(w).step(), "bf16")
    dw = DeviceWorkload(w)
    dw.write_step()
    kc, vc = to_host(dw.k_cache, "bf16"), to_host(dw.v_cache, "bf16")
    pi = np.random.default_rng(51).permutation(kc.shape[0])
    kp, vp = np.empty_like(kc), np.empty_like(vc)
    kp[pi], vp[pi] = kc, vc
    bt = np.where(w.block_tables >= 0, pi[np.maximum(w.block_tables, 0)], -1).astype(np.int32)
    w2 = wl.Workload(name="pfperm2", dtype="bf16", seed=0, q=w.q, k_cache=kp, v_cache=vp,
                     block_tables=bt, context_lens=w.context_lens, scale=w.scale,
                     block_mapping=np.zeros((0, 2), np.int32), slot_mapping=np.zeros((0,), np.int32),
                     new_key=w.new_key[:0], new_value=w.new_value[:0], query_start=w.query_start)
    moved = to_host(DeviceWorkload(w2).step(), "bf16")
    assert np.array_equal(base, moved)


@pytest.mark.parametrize("ctx,ql,hq,hkv,dtype", [
    ([5000], [64], 8, 2, "bf16"),                 # one long prompt: 8 workgroups, cut into 9 parts
    ([3000, 700], [100, 40], 8, 1, "f16"),        # G = 8, parts per sequence differ
    ([2500, 1], [256, 1], 4, 4, "bf16"),          # G = 1, a 256-token chunk
])
def test_prefill_path_split_context(ctx, ql, hq, hkv, dtype):
    """Too few workgroups to fill the chip: each context is cut into parts,
    one workgroup each, and a merge combines their states."""
    rng = np.random.default_rng(52)
    w = wl.build(f"pf_split_{len(ctx)}_{dtype}", 52, rng, ctx, hq, hkv, 128, 16, dtype,
                 poison=True, query_lens=ql)
    G = hq // hkv
    assert w.max_query_len * G >= 64
    dw = DeviceWorkload(w)
    assert _lib.paged_attention_multi_workspace_bytes(
        dw.k_cache, w.num_seqs, w.num_q_heads, w.max_query_len, w.max_context_len) > 0
    _run(w, f"prefill path, split contexts {ctx}")


def test_long_prompt_chunk_sampled_rows():
    """The full-size one-long-prompt chunk (256 new tokens ending a
    32768-token context; its context is cut into parts).  Sampled rows are
    checked against decode attention over the tokens each row may see, the
    form the multi-token oracle reduces to row by row."""
    import oracle
    from gpu_common import oracle_pools_after_step
    w = wl.named("long_prompt_chunk")
    print(f"[gpu] long_prompt_chunk: n={w.max_context_len} L={w.max_query_len}", flush=True)
    dw = DeviceWorkload(w)
    out = to_host(dw.step(), w.dtype)
    torch.cuda.synchronize()
    kc, vc = oracle_pools_after_step(w)
    n, L = int(w.context_lens[0]), int(w.max_query_len)
    rows = np.array([0, 1, 63, 64, 127, 200, 254, 255])
    args = (np.repeat(w.block_tables[:1], len(rows), 0), (n - L + rows + 1).astype(np.int32),
            w.scale, w.dtype)
    ref = oracle.decode_attention(w.q[rows], kc, vc, *args)
    assert takes_fp16_pv(w)
    slack = 2.0 ** -11 * np.abs(oracle.decode_attention(w.q[rows], kc, abs_pool(vc, w.dtype), *args))
    check_attention(out[rows], ref, w.dtype, "long_prompt_chunk sampled rows", slack=slack)


def test_prefill_path_v_beyond_fp16_range():
    """The prefill path's fp16 PV form cannot hold bf16 values of magnitude
    2^16 and above (they become +-inf).  The workgroups whose context holds
    one stream it again in the exact form (bf16 V, P split in two parts);
    the others keep the fp16 form.  Every output must stay finite and within
    the bound: on the fast form alone those rows would be inf or NaN."""
    rng = np.random.default_rng(53)
    w = wl.build("pf_bigv", 53, rng, [700, 300, 1200], 8, 2, 128, 16, "bf16", poison=True,
                 query_lens=[40, 17, 64])
    assert w.max_query_len * 4 >= 64
    v = w.v_cache.copy()
    # kv head 0 of sequence 0 (token 53) and kv head 1 of sequence 2 (token
    # 900), both well before the appended tokens: 70144, -131072, 65536
    b0 = int(w.block_tables[0, 53 // 16])
    v[b0, 0, 53 % 16, :8] = np.array([0x4789, 0xC800, 0x4780, 0x4789] * 2, dtype=np.uint16)
    b2 = int(w.block_tables[2, 900 // 16])
    v[b2, 1, 900 % 16, 100:104] = np.array([0xC789, 0x4800, 0x4780, 0xC780], dtype=np.uint16)
    w.v_cache = v
    err = _run(w, "prefill path, V beyond the fp16 range")
    print(f"[gpu] V beyond fp16 range: max |gpu - oracle| = {err:.3e}", flush=True)
