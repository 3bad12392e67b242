"""paged_attention_decode_noalloc through the C ABI (needs an MI355X).

The entry point for callers that cannot allocate takes its workspace from a
scratch array the library keeps on each GPU.  It runs the same kernels on the
same grid as paged_attention_decode, so its output must equal that entry
point's bit for bit, and both must meet the oracle's bar.  Calls in a row
share the array and find the previous call's partial states in it: the
second call is smaller than the first, and the first uses the largest
stream-path workspace (16 query heads per kv head, head dim 128).
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_388_amd import _lib
from paged_kv_cache_388_amd import workloads as wl

from gpu_common import DeviceWorkload, check_attention, oracle_step, to_host

pytestmark = pytest.mark.gpu


def _both(w, what):
    print(f"[gpu] noalloc {what}: B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"D={w.head_dim} bs={w.block_size} {w.dtype} maxctx={w.max_context_len}", flush=True)
    dw = DeviceWorkload(w)
    dw.write_step()
    ref_out = to_host(dw.attend(), w.dtype).copy()
    out = torch.full_like(dw.q, float("nan"))
    _lib.paged_attention_decode_noalloc(out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables,
                                        dw.context_lens, w.scale, w.max_context_len)
    torch.cuda.synchronize()
    got = to_host(out, w.dtype)
    assert np.array_equal(got.view(np.uint8), ref_out.view(np.uint8)), what
    check_attention(got, oracle_step(w), w.dtype, what)


def test_noalloc_matches_decode_on_two_calls_in_a_row():
    need = _lib.paged_attention_workspace_bytes(
        torch.empty((1, 4, 16, 128), dtype=torch.bfloat16, device="cuda"), 40, 64, 6000)
    assert 0 < need <= _lib.paged_attention_noalloc_max_bytes()
    rng = np.random.default_rng(71)
    ctx = rng.integers(1, 6000, size=40)
    big = wl.build("noalloc_big", 71, rng, ctx, 64, 4, 128, 16, "bf16", poison=True)
    _both(big, "first call, G=16 D=128")
    rng = np.random.default_rng(72)
    small = wl.build("noalloc_small", 72, rng, [1, 17, 300, 0, 900], 8, 2, 64, 32, "f16",
                     poison=True)
    _both(small, "second call, smaller")


def test_noalloc_full_size_decode_then_tiny():
    _both(wl.named("llama3_8b_gqa"), "llama3_8b_gqa")
    _both(wl.tiny_f32(poison=True), "tiny_f32")
