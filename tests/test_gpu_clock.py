"""The clock builds (PAGEDKV_CLOCK=1: per-wave / per-workgroup start and end
records, a measurement variant of bf16 / D 128 / 16-token blocks) give the
normal kernels' outputs bit for bit, and their records account for the
call's work (needs an MI355X)."""

import numpy as np
import pytest
import torch

from paged_kv_cache_388_amd import _lib
from paged_kv_cache_388_amd import workloads as wl

from gpu_common import DeviceWorkload, to_host

pytestmark = pytest.mark.gpu


def _both(w, monkeypatch):
    dw = DeviceWorkload(w)
    dw.write_step()
    base = to_host(dw.attend(), w.dtype).copy()
    monkeypatch.setenv("PAGEDKV_CLOCK", "1")
    clocked = to_host(dw.attend(), w.dtype).copy()
    rec = _lib.pkv_clock_read()
    monkeypatch.delenv("PAGEDKV_CLOCK")
    assert np.array_equal(base.view(np.uint16), clocked.view(np.uint16))
    return rec[rec[:, 1] != 0]


def test_decode_clock_build(monkeypatch):
    rng = np.random.default_rng(61)
    ctx = [1, 15, 17, 300, 2000, 4100, 0, 700, 33, 5000]
    w = wl.build("clock_decode", 61, rng, ctx, 32, 8, 128, 16, "bf16", poison=True)
    print(f"[gpu] clock build, decode: B={w.num_seqs}", flush=True)
    rec = _both(w, monkeypatch)
    # every wave of the grid records, and the waves' positions cover the call
    # (kv heads x 16-token sub-tiles of every context) exactly
    assert rec.shape[0] % 8 == 0 and rec.shape[0] >= 8
    assert np.all(rec[:, 1] >= rec[:, 0])
    xcd = rec[:, 2] & np.uint64(0xff)
    assert np.all(xcd < 8)
    positions = ((rec[:, 2] >> np.uint64(8)) & np.uint64(0xffffffff)).astype(np.int64)
    assert positions.sum() == 8 * sum((c + 15) // 16 for c in ctx)


def test_prefill_clock_build(monkeypatch):
    rng = np.random.default_rng(62)
    ctx, ql = [300, 2100, 65, 900], [64, 64, 40, 0]
    w = wl.build("clock_prefill", 62, rng, ctx, 32, 8, 128, 16, "bf16", poison=True,
                 query_lens=ql)
    print(f"[gpu] clock build, prefill: B={w.num_seqs}", flush=True)
    rec = _both(w, monkeypatch)
    assert np.all(rec[:, 1] >= rec[:, 0])
    seq = ((rec[:, 2] >> np.uint64(8)) & np.uint64(0xffffff)).astype(np.int64)
    ctx_rec = (rec[:, 3] >> np.uint64(32)).astype(np.int64)
    # only sequences with new tokens stream their context, each with its own length
    assert set(seq.tolist()) == {0, 1, 2}
    for s in (0, 1, 2):
        assert np.all(ctx_rec[seq == s] == ctx[s])


def test_clock_ignored_for_other_shapes(monkeypatch):
    """PAGEDKV_CLOCK=1 on a shape without a clock build (fp16) runs the
    normal kernels: same output, no records."""
    rng = np.random.default_rng(63)
    w = wl.build("clock_f16", 63, rng, [5, 300, 1000], 8, 2, 128, 16, "f16")
    print(f"[gpu] clock switch on an fp16 pool: B={w.num_seqs}", flush=True)
    rec = _both(w, monkeypatch)
    assert rec.shape[0] == 0
