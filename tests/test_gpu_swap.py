"""Swap to host memory and back through the C ABI against the oracle's
swap_out / swap_in (needs an MI355X).  Raw bit copies: every comparison is
bit-exact, over whole images and whole pools."""

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_388_amd import _lib
from paged_kv_cache_388_amd import workloads as wl

from gpu_common import to_dev, to_host

pytestmark = pytest.mark.gpu


def _pool(rng, dtype, shape):
    if dtype == "f32":
        return rng.standard_normal(shape).astype(np.float32)
    return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)    # any bit pattern, NaNs too


def _host_bits(t, dtype):
    return t.numpy() if dtype == "f32" else t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype,H,bs,D,staging_entries", [
    ("bf16", 8, 16, 128, 7),      # Llama-3-8B-shaped tiles, runs of 7 with a ragged tail
    ("f16", 4, 32, 64, 1),        # one block per run
    ("f32", 2, 16, 64, None),     # library default staging
])
def test_swap_out_in_bit_exact(dtype, H, bs, D, staging_entries):
    rng = np.random.default_rng(31)
    NB = 300
    print(f"[gpu] swap {dtype} H={H} bs={bs} D={D} staging={staging_entries}", flush=True)
    k = _pool(rng, dtype, (NB, H, bs, D))
    v = _pool(rng, dtype, (NB, H, bs, D))
    kc, vc = to_dev(k, dtype), to_dev(v, dtype)
    ids = rng.integers(0, NB, size=61).astype(np.int32)
    ids[[3, 40]] = [NB, -5]                     # outside the pool: zero entries
    ids[10] = ids[11]                           # a duplicate source is fine
    entry = 2 * H * bs * D * kc.element_size()
    staging = (None if staging_entries is None else
               torch.empty(staging_entries * entry + 48, dtype=torch.uint8, device="cuda"))
    img = _lib.paged_swap_out(kc, vc, to_dev(ids, dtype), staging=staging)
    torch.cuda.synchronize()
    want = oracle.swap_out(k, v, ids)
    assert np.array_equal(_host_bits(img, dtype).view(np.uint8), want.view(np.uint8))

    # back into other, distinct blocks of a second pool (some outside it)
    dst = rng.permutation(NB)[:61].astype(np.int32)
    dst[[5, 6]] = [NB + 3, -1]
    k2 = _pool(rng, dtype, (NB, H, bs, D))
    v2 = _pool(rng, dtype, (NB, H, bs, D))
    kc2, vc2 = to_dev(k2, dtype), to_dev(v2, dtype)
    _lib.paged_swap_in(img, kc2, vc2, to_dev(dst, dtype), staging=staging)
    torch.cuda.synchronize()
    wk, wv = oracle.swap_in(k2, v2, want, dst)
    assert np.array_equal(to_host(kc2, dtype).view(np.uint8), wk.view(np.uint8))
    assert np.array_equal(to_host(vc2, dtype).view(np.uint8), wv.view(np.uint8))


def test_swap_empty_and_into_given_image():
    rng = np.random.default_rng(32)
    k = _pool(rng, "bf16", (8, 2, 16, 64))
    kc = to_dev(k, "bf16")
    vc = kc.clone()
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    img = _lib.paged_swap_out(kc, vc, empty)
    assert img.shape == (0, 2, 2, 16, 64)
    _lib.paged_swap_in(img, kc, vc, empty)
    # a caller-owned pinned image is filled in place
    host = torch.zeros((3, 2, 2, 16, 64), dtype=torch.bfloat16, pin_memory=True)
    ids = np.array([7, 0, 7], dtype=np.int32)
    got = _lib.paged_swap_out(kc, vc, to_dev(ids, "bf16"), host_image=host)
    torch.cuda.synchronize()
    assert got is host
    assert np.array_equal(_host_bits(host, "bf16"), oracle.swap_out(k, k, ids))
    torch.cuda.synchronize()
    assert np.array_equal(to_host(kc, "bf16"), k)


def test_swap_full_size_pool():
    """The Llama-3-8B-shaped decode pool: swap out the blocks of its eight
    longest sequences, scribble over them, bring them back into the same blocks
    and get the pool back bit for bit."""
    w = wl.named("llama3_8b_gqa")
    print(f"[gpu] swap full pool: {w.num_blocks} blocks", flush=True)
    kc = to_dev(w.k_cache, w.dtype)
    vc = to_dev(w.v_cache, w.dtype)
    longest = np.argsort(w.context_lens)[-8:]
    ids = np.concatenate([w.block_tables[s, :-(-int(w.context_lens[s]) // w.block_size)]
                          for s in longest]).astype(np.int32)
    ids_dev = to_dev(ids, w.dtype)
    img = _lib.paged_swap_out(kc, vc, ids_dev)
    torch.cuda.synchronize()
    assert np.array_equal(_host_bits(img, w.dtype), oracle.swap_out(w.k_cache, w.v_cache, ids))
    kc[ids_dev.long()] = 0
    vc[ids_dev.long()] = 0
    _lib.paged_swap_in(img, kc, vc, ids_dev)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(kc, w.dtype), w.k_cache)
    assert np.array_equal(to_host(vc, w.dtype), w.v_cache)
