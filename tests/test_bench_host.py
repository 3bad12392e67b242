"""Host-side arithmetic of bench.py: the algorithmic bytes and flops its
roofline line is priced on, the counter-traffic lookup, and the one-GPU
refusal.  No GPU is touched."""

import os
import subprocess
import sys

import numpy as np

import bench
from paged_kv_cache_388_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_by_hand():
    # 4 sequences, contexts 5, 16, 33, 70 (124 tokens), 2 query / 2 KV heads
    # of 64, fp32, 16-token blocks
    w = wl.tiny_f32()
    kv = 2 * 124 * 2 * 64 * 4                 # K and V of every context token
    q_out = 2 * 4 * 2 * 64 * 4                # one q row in, one out row back
    ids = 4 * (1 + 1 + 3 + 5)                 # ceil(ctx / 16) block ids
    lens = 4 * 4
    assert w.kv_bytes() == kv == 126976
    assert bench.algorithmic_bytes(w) == kv + q_out + ids + lens == 131128
    assert bench.unique_kv_bytes(w) == kv     # no block is shared


def test_attention_flops_by_hand():
    w = wl.tiny_f32()
    # one new token per sequence sees its whole context: 4 * D per
    # (query head, token) for QK and PV multiply-adds
    assert bench.attention_flops(w) == 4 * 64 * 2 * 124
    # four new tokens per sequence, causal among themselves: rows see
    # ctx-3, ctx-2, ctx-1, ctx tokens
    m = wl.build("m", 1, np.random.default_rng(1), [10, 20], 4, 2, 64, 16,
                 "bf16", query_lens=[4, 4])
    seen = sum(4 * n - 6 for n in (10, 20))
    assert bench.attention_flops(m) == 4 * 64 * 4 * seen


def test_shared_blocks_count_once():
    w = wl.shared_prefix(num_seqs=4, prefix_tokens=100)
    assert bench.unique_kv_bytes(w) < w.kv_bytes()
    one_seq = 2 * int(w.context_lens.max()) * w.num_kv_heads * w.head_dim * 2
    assert bench.unique_kv_bytes(w) > one_seq


def test_counter_traffic_follows_the_source(monkeypatch, tmp_path):
    """A counter summary counts only for the kernel source it was taken on."""
    import hashlib
    src = tmp_path / "attention.hip"
    src.write_text("// kernel source\n")
    common = tmp_path / "attn_common.h"
    common.write_text("// shared device code\n")
    sha = hashlib.sha256(src.read_bytes() + common.read_bytes()).hexdigest()
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "attn_grid_kernel_long_ctx_bs16_hbm_counters.md").write_text(
        f"# summary\n\ntraffic_bytes_per_call: 1234567\nsource_sha256: `{sha}`\n")
    monkeypatch.setattr(bench, "DECODE_SOURCES", [str(src), str(common)])
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    assert bench.counter_traffic("long_ctx_bs16", "attn_grid_kernel") == 1234567
    assert bench.counter_traffic("long_ctx_bs16") is None             # another kernel's file
    assert bench.counter_traffic("no_such_workload", "attn_grid_kernel") is None
    common.write_text("// changed\n")
    assert bench.counter_traffic("long_ctx_bs16", "attn_grid_kernel") is None


def test_committed_counter_summaries_name_their_source():
    """Every committed HBM counter summary carries the per-call traffic and
    the SHA-256 of the source it was taken on."""
    import glob
    files = glob.glob(os.path.join(ROOT, "profiles", "*_hbm_counters.md"))
    assert files
    for path in files:
        text = open(path).read()
        assert "traffic_bytes_per_call:" in text and "source_sha256:" in text, path


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_shared_block_bytes_by_hand():
    """A 100-token prefix at 16-token blocks: 6 full blocks shared by every
    sequence (the 7th, partly filled, is copied per sequence), each read by
    all 4 sequences; nothing is shared in a private-table workload."""
    w = wl.shared_prefix(num_seqs=4, prefix_tokens=100)
    sb, reads = bench.shared_block_bytes(w)
    assert reads == 4
    assert sb == 2 * 6 * 16 * w.num_kv_heads * w.head_dim * 2
    assert bench.shared_block_bytes(wl.tiny_f32()) == (0, 0.0)


def test_clock_summary_by_hand():
    """bench.py --clock: per-XCD end times, the within-XCD spread and the
    per-sequence prefill figures from hand-made records (100 MHz counter)."""
    def rec(start, end, w2, w3):
        return [start, end, w2, w3]
    # decode: two waves per XCD, ending at 100 + 10 x and 104 + 10 x us
    rows = []
    for x in range(8):
        for k, extra in enumerate((0, 4)):
            pieces = 1 + k
            rows.append(rec(1000, 1000 + (100 + 10 * x + extra) * 100, x | (50 << 8) | (pieces << 40), 0))
    rows.append(rec(0, 0, 0, 0))  # an unwritten record is skipped
    s = bench.clock_summary(np.array(rows, dtype=np.uint64), multi=False)
    assert s["units"] == 16
    assert s["end_max_us"] == 174.0
    assert s["xcd_end_p50_us"] == [102.0 + 10 * x for x in range(8)]
    assert s["xcd_end_max_us"] == [104.0 + 10 * x for x in range(8)]
    assert s["within_xcd_p10_us"] == -2.0 and s["within_xcd_p90_us"] == 2.0
    assert s["pieces_mean"] == 1.5 and s["corr_end_pieces_within_xcd"] == 1.0
    # prefill: sequence 3 (context 640, 10 stages) on two workgroups, sequence 5 on one
    rows = [rec(0, 2000, 0 | (3 << 8), 10 | (640 << 32)),
            rec(100, 2100, 1 | (3 << 8), 10 | (640 << 32)),
            rec(500, 1500, 2 | (5 << 8), 4 | (1 << 20) | (256 << 32))]
    s = bench.clock_summary(np.array(rows, dtype=np.uint64), multi=True)
    assert s["units"] == 3 and s["end_max_us"] == 21.0
    assert s["sequences"] == [
        {"seq": 3, "context": 640, "workgroups": 2, "start_p50_us": 0.5, "end_max_us": 21.0,
         "us_per_stage_p50": 2.0},
        {"seq": 5, "context": 256, "workgroups": 1, "start_p50_us": 5.0, "end_max_us": 15.0,
         "us_per_stage_p50": 2.5}]
    assert s["running_at_tenths"][0] == 1 and s["running_at_tenths"][-1] == 0
