"""The five named decode workloads at their full sizes, through the C ABI, in
the launch configuration bench.py times, against the CPU oracle (needs an
MI355X).

Every output row of every sequence is compared (the oracle finishes each
workload in seconds), and the pools after the step's cache writes are
compared bit for bit with the oracle's.  Every slot the step does not define
(free blocks, the tail slots of each sequence's last block, the slots about
to be appended) holds NaN, as in the edge tests: the same draws as the timed
workloads, whose outputs must not see those slots.  Here the stated bar holds literally:
max |gpu - oracle| <= 2e-3 for 16-bit storage and 2e-5 for fp32, with no
allowance for the output's own rounding (these outputs stay below 1 in
magnitude, where half a bf16 ulp is under 2e-3).  Each case prints one
``[gpu-result]`` JSON line with its error figures.

The long-context workloads also run on the 512-token partition path (one
workgroup per (kv head, sequence, partition), then the partition merge),
forced with PAGEDKV_DECODE_PATH=grid: the split-context reading of the
long-context workload, at its full size.
"""

import json

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_388_amd import workloads as wl

from gpu_common import (DeviceWorkload, check_attention, oracle_pools_after_step, oracle_step,
                        to_host)

pytestmark = pytest.mark.gpu

LITERAL_BAR = {"f32": 2e-5, "f16": 2e-3, "bf16": 2e-3}


@pytest.mark.parametrize("name,path", [("tiny_f32", "default"), ("llama2_7b_f16", "default"),
                                       ("llama3_8b_gqa", "default"), ("shared_prefix", "default"),
                                       ("long_ctx_bs16", "default"), ("long_ctx_bs32", "default"),
                                       ("llama3_8b_gqa", "grid"), ("long_ctx_bs16", "grid"),
                                       ("long_ctx_bs32", "grid")])
def test_full_size_workload(name, path, monkeypatch):
    if path == "grid":
        monkeypatch.setenv("PAGEDKV_DECODE_PATH", "grid")
    w = wl.named(name, poison=True)
    print(f"[gpu] {name} ({path} path): B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"bs={w.block_size} NB={w.num_blocks} maxctx={w.max_context_len}", flush=True)
    dw = DeviceWorkload(w)
    out = dw.step()
    torch.cuda.synchronize()
    got = to_host(out, w.dtype)
    kc, vc = oracle_pools_after_step(w)
    assert np.array_equal(to_host(dw.k_cache, w.dtype).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(to_host(dw.v_cache, w.dtype).view(np.uint8), vc.view(np.uint8))
    ref = oracle_step(w, pools=(kc, vc))
    check_attention(got, ref, w.dtype, name)
    err = np.abs(oracle.storage_to_f64(got, w.dtype) - ref)
    bar = LITERAL_BAR[w.dtype]
    print("[gpu-result] " + json.dumps({
        "workload": name, "path": path, "dtype": w.dtype, "outputs": int(err.size),
        "max_abs_err": float(err.max()), "mean_abs_err": float(err.mean()),
        "max_abs_ref": float(np.abs(ref).max()), "bar": bar,
        "above_bar": int((err > bar).sum())}), flush=True)
    assert err.max() <= bar, f"{name}: max error {err.max():.3e} above {bar}"
