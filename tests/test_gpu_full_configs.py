"""The five named decode workloads at their full sizes, through the C ABI, in
the launch configuration bench.py times, against the CPU oracle (needs an
MI355X).

Every output row of every sequence is compared (the oracle finishes each
workload in seconds), and the pools after the step's cache writes are
compared bit for bit with the oracle's.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_388_amd import workloads as wl

from gpu_common import (DeviceWorkload, check_attention, oracle_pools_after_step, oracle_step,
                        to_host)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_f32", "llama2_7b_f16", "llama3_8b_gqa", "shared_prefix",
                                  "long_ctx_bs16", "long_ctx_bs32"])
def test_full_size_workload(name):
    w = wl.named(name)
    print(f"[gpu] {name}: B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"bs={w.block_size} NB={w.num_blocks} maxctx={w.max_context_len}", flush=True)
    dw = DeviceWorkload(w)
    out = dw.step()
    torch.cuda.synchronize()
    got = to_host(out, w.dtype)
    kc, vc = oracle_pools_after_step(w)
    assert np.array_equal(to_host(dw.k_cache, w.dtype).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(to_host(dw.v_cache, w.dtype).view(np.uint8), vc.view(np.uint8))
    ref = oracle_step(w, pools=(kc, vc))
    err = check_attention(got, ref, w.dtype, name)
    print(f"[gpu] {name}: max |gpu - oracle| = {err:.3e}", flush=True)
