"""Decode-step benchmark of the paged KV-cache hot path on one MI355X.

A step is one decode iteration of one attention layer over the whole batch:
the step's cache writes (copy-on-write block copies, then the append of the
new tokens' K/V into their slots) followed by paged decode attention.  The
default workload is the Llama-3-8B-shaped GQA layer: 128 sequences, 32 query
/ 8 KV heads of 128, bf16, 16-token blocks, contexts log-uniform in
[256, 8192], shuffled physical pool.  Inputs are seeded and synthetic and are
resident in HBM before timing starts.  Before the warmup steps the attention
call runs untimed for --settle-ms (200 ms): the GPU idles during the host-side
setup and its clocks take tens of milliseconds of load to come back up, which
a handful of warmup steps of a 0.1 ms call does not cover.

Prints ONE JSON line.  ``value`` is the KV bytes a step reads (each cached
token's K and V once) divided by the measured step time, in GB/s.
``roofline`` prices the decode call (the stream kernel and its piece merge,
launched by one paged_attention_decode call) against MI355X's 8 TB/s HBM
peak, with its duration measured by HIP events on the launching stream;
``traffic`` is the HBM bytes the rocprofv3 counters measured for that call
(profiles/, calibrated against a plain copy), reported only while the kernel
source is the one the counters were taken on.  A multi-token workload that
takes the prefill path (prompt chunks) is priced instead on its attention
flops against the dense MFMA peak of its dtype.  ``cpu_baseline`` times the CPU
oracle on the same step's inputs.
"""

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Worker processes of the CPU baseline re-import this file; they need only
# NumPy and the oracle, not the library (or torch).
_CPU_WORKER = os.environ.get("PKV_BENCH_CPU_WORKER") == "1"
if not _CPU_WORKER:
    from paged_kv_cache_388_amd import workloads as wl  # noqa: E402

PEAK_HBM_GBS = 8000.0
# the CPU baseline runs at most this many oracle processes, whatever the host
CPU_PROCESS_CAP = 16
# dense MFMA peaks of MI355X, TFLOP/s, by the dtype the products run in
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}
PREFILL_MIN_COLS = 64      # max_query_len * G at which a multi call takes the prefill path
# the sources the decode kernels compile from; counter summaries record the
# SHA-256 of their contents in this order
DECODE_SOURCES = [os.path.join(ROOT, "paged_kv_cache_388_amd", "csrc", f)
                  for f in ("attention.hip", "attn_common.h")]
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "paged decode attention: achieved KV HBM GB/s (% of peak) and seqs/s"


def algorithmic_bytes(w):
    """Bytes one attention call must move: every context token's K and V once,
    q in and out back (one row per new token), the block ids, the context
    lengths (and the query-row prefix of a multi-token call)."""
    b = wl.ELEM_BYTES[w.dtype]
    ids = sum((int(n) + w.block_size - 1) // w.block_size for n in w.context_lens)
    rows = w.q.shape[0]
    extra = 4 * (w.num_seqs + 1) if w.multi else 0
    return (w.kv_bytes() + 2 * rows * w.num_q_heads * w.head_dim * b + 4 * ids
            + 4 * w.num_seqs + extra)


def unique_kv_bytes(w):
    """Bytes of K and V held by the distinct physical blocks the batch reads
    (each block counted up to the most tokens any sequence reads from it):
    the traffic floor when blocks are shared.  Equal to kv_bytes() without
    sharing."""
    b = wl.ELEM_BYTES[w.dtype]
    fill = {}
    for s in range(w.num_seqs):
        n = int(w.context_lens[s])
        for j in range((n + w.block_size - 1) // w.block_size):
            blk = int(w.block_tables[s, j])
            fill[blk] = max(fill.get(blk, 0), min(w.block_size, n - j * w.block_size))
    return 2 * sum(fill.values()) * w.num_kv_heads * w.head_dim * b


def shared_block_bytes(w):
    """Bytes of K and V held by the physical blocks that more than one
    sequence reads, and the mean number of sequences reading each of them."""
    b = wl.ELEM_BYTES[w.dtype]
    refs, fill = {}, {}
    for s in range(w.num_seqs):
        n = int(w.context_lens[s])
        for j in range((n + w.block_size - 1) // w.block_size):
            blk = int(w.block_tables[s, j])
            refs[blk] = refs.get(blk, 0) + 1
            fill[blk] = max(fill.get(blk, 0), min(w.block_size, n - j * w.block_size))
    shared = [blk for blk, k in refs.items() if k > 1]
    if not shared:
        return 0, 0.0
    nbytes = 2 * sum(fill[blk] for blk in shared) * w.num_kv_heads * w.head_dim * b
    return nbytes, sum(refs[blk] for blk in shared) / len(shared)


def attention_flops(w):
    """QK and PV multiply-adds of one call: 4 * D flops per (new token, query
    head, visible context token)."""
    G = w.num_q_heads // w.num_kv_heads
    qlens = np.diff(w.query_start) if w.multi else (w.context_lens > 0).astype(np.int64)
    visible = 0
    for n, L in zip(w.context_lens.astype(np.int64), qlens):
        visible += int(L) * int(n) - int(L) * (int(L) - 1) // 2
    return 4 * w.head_dim * G * w.num_kv_heads * visible


def decode_source_sha():
    """SHA-256 of the decode kernels' sources, concatenated in order."""
    import hashlib
    h = hashlib.sha256()
    for path in DECODE_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(workload, kernel="attn_stream_kernel"):
    """HBM bytes per attention call from the committed counter summary of this
    kernel and workload, or None if there is none or the kernel source has
    changed since the counters were taken (the summary records the source's
    SHA-256)."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.strip().startswith(("traffic_bytes_per_call", "source_sha256")):
                k, v = line.strip().split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("source_sha256") != decode_source_sha() or "traffic_bytes_per_call" not in fields:
        return None
    return int(fields["traffic_bytes_per_call"])


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_pass(A, seq_list, seconds):
    """The oracle over the sequences of seq_list, round after round, until
    ``seconds`` have passed: (query rows, sequence-attentions, KV bytes).  A
    holds the step's host arrays (pools after the cache writes) and shape
    facts.  A multi-token sequence's new rows go in slices of up to 16: a
    slice of rows [a, e) is the last e - a tokens of a context of n - L + e
    tokens, which is what each of its rows sees."""
    import oracle
    rows = seqs = kv = 0
    per_token = 2 * A["num_kv_heads"] * A["head_dim"] * A["elem_bytes"]
    t1 = time.perf_counter()
    while True:
        for s in seq_list:
            if A["multi"]:
                r0, r1 = int(A["query_start"][s]), int(A["query_start"][s + 1])
                n, L = int(A["context_lens"][s]), r1 - r0
                for a in range(0, L, 16):
                    e = min(a + 16, L)
                    oracle.multi_query_attention(
                        A["q"][r0 + a:r0 + e], A["k_cache"], A["v_cache"], A["block_tables"][s:s + 1],
                        np.array([n - L + e], dtype=np.int32), [e - a], A["scale"], A["dtype"])
                    kv += (n - L + e) * per_token
                    rows += e - a
                    if time.perf_counter() - t1 > seconds:
                        break
            else:
                oracle.decode_attention(A["q"], A["k_cache"], A["v_cache"], A["block_tables"],
                                        A["context_lens"], A["scale"], A["dtype"], seq_ids=[s])
                kv += int(A["context_lens"][s]) * per_token
                rows += 1
            seqs += 1
            if time.perf_counter() - t1 > seconds:
                return rows, seqs, kv
        if not seq_list:
            return rows, seqs, kv


_WORKER_ARRAYS = {}


def _oracle_worker_init(arrays, facts):
    """A spawned baseline worker: one BLAS thread, the step's arrays mapped
    from shared memory."""
    from multiprocessing import shared_memory
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)
    for name, (shm_name, shape, dtype) in arrays.items():
        shm = shared_memory.SharedMemory(name=shm_name)
        _WORKER_ARRAYS["_shm_" + name] = shm
        _WORKER_ARRAYS[name] = np.ndarray(shape, dtype=np.dtype(dtype), buffer=shm.buf)
    _WORKER_ARRAYS.update(facts)


def _oracle_worker_run(task):
    idx, workers, seconds = task
    A = _WORKER_ARRAYS
    return _oracle_pass(A, list(range(idx, A["num_seqs"], workers)), seconds)


def cpu_baseline(w, min_seconds, workers):
    """The fp64 oracle on this step's inputs: the step's cache writes into the
    host pools (one thread), then attention over the batch's sequences split
    round-robin over ``workers`` spawned processes of one BLAS thread each
    (the pools shared through shared memory), each repeating its sequences
    for about ``min_seconds``.  Also a one-process pass of a third of that
    time, for the scaling.  Rates in KV GB/s (and query rows/s) of the
    attention work finished."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor
    from concurrent.futures.process import BrokenProcessPool
    from multiprocessing import shared_memory
    from threadpoolctl import threadpool_limits

    import oracle
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        kc, vc = w.k_cache, w.v_cache
        if len(w.block_mapping):
            kc, vc = oracle.copy_blocks(kc, vc, w.block_mapping)
        if len(w.slot_mapping):
            kc, vc = oracle.kv_append(kc, vc, w.new_key, w.new_value, w.slot_mapping)
        t_writes = time.perf_counter() - t0
        arrays = {"k_cache": kc, "v_cache": vc, "q": w.q, "block_tables": w.block_tables,
                  "context_lens": w.context_lens}
        if w.multi:
            arrays["query_start"] = w.query_start
        facts = {"num_seqs": w.num_seqs, "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                 "elem_bytes": wl.ELEM_BYTES[w.dtype], "multi": bool(w.multi), "scale": w.scale,
                 "dtype": w.dtype}
        one_s = min_seconds / 3
        t1 = time.perf_counter()
        r1, s1, kv1 = _oracle_pass({**arrays, **facts}, list(range(w.num_seqs)), one_s)
        one_rate = kv1 / (time.perf_counter() - t1)

    used, note = 1, ""
    rate, rows, seqs, dt = one_rate, r1, s1, one_s
    shms = []
    try:
        if workers > 1:
            spec = {}
            for name, arr in arrays.items():
                arr = np.ascontiguousarray(arr)
                shm = shared_memory.SharedMemory(create=True, size=max(1, arr.nbytes))
                shms.append(shm)
                np.ndarray(arr.shape, dtype=arr.dtype, buffer=shm.buf)[...] = arr
                spec[name] = (shm.name, arr.shape, arr.dtype.str)
            saved = {k: os.environ.get(k) for k in ("PKV_BENCH_CPU_WORKER", "OMP_NUM_THREADS",
                                                     "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
            os.environ.update({"PKV_BENCH_CPU_WORKER": "1", "OMP_NUM_THREADS": "1",
                               "OPENBLAS_NUM_THREADS": "1", "MKL_NUM_THREADS": "1"})
            try:
                # a worker that fails to start breaks the pool (an error here),
                # it is not started again
                with ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn"),
                                         initializer=_oracle_worker_init,
                                         initargs=(spec, facts)) as pool:
                    list(pool.map(_oracle_worker_run, [(i, workers, 0.0) for i in range(workers)]))
                    t2 = time.perf_counter()
                    res = list(pool.map(_oracle_worker_run,
                                        [(i, workers, min_seconds) for i in range(workers)]))
                    dt = time.perf_counter() - t2
            finally:
                for k, v in saved.items():
                    if v is None:
                        os.environ.pop(k, None)
                    else:
                        os.environ[k] = v
            rows = sum(r[0] for r in res)
            seqs = sum(r[1] for r in res)
            rate = sum(r[2] for r in res) / dt
            used = workers
    except (OSError, BrokenProcessPool) as e:  # no shared memory or processes here
        note = f"; {workers} worker processes unavailable ({type(e).__name__}), one process"
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    return {"value": round(rate / 1e9, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
            "usable_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "process_cap": CPU_PROCESS_CAP,
            "sample": (f"{rows} query rows of {seqs} sequence-attentions of this step "
                       f"({seqs / w.num_seqs:.2f} passes over the {w.num_seqs}-sequence batch, "
                       f"the last one possibly in part) after its cache writes "
                       f"({t_writes:.1f} s), fp64 NumPy, {used} process(es) of one BLAS thread, "
                       f"{dt:.1f} s{note}"),
            "rows_per_s": round(rows / dt, 2),
            "one_process_GBps": round(one_rate / 1e9, 4)}


def block_manager_trace(seed=388008, num_seqs=256, system_tokens=1000, steps=256):
    """Serving-style bookkeeping trace: num_seqs prompts sharing a
    system_tokens-token system prompt plus their own 16..256 tokens, then
    `steps` decode steps appending one token to every sequence; every 32 steps
    a quarter of the sequences is freed and replaced by new ones, and every 16
    steps some sequences fork (parallel sampling)."""
    rng = np.random.default_rng(seed)
    system = [int(t) for t in rng.integers(0, 32000, size=system_tokens)]
    ops = []
    next_id = 0
    live = []
    for _ in range(num_seqs):
        ops.append(("add", next_id, system + [int(t) for t in rng.integers(0, 32000, size=int(rng.integers(16, 257)))]))
        live.append(next_id)
        next_id += 1
    for step in range(steps):
        if step and step % 32 == 0:
            for sid in list(rng.choice(live, size=len(live) // 4, replace=False)):
                ops.append(("free", int(sid), None))
                live.remove(int(sid))
                ops.append(("add", next_id, system + [int(t) for t in rng.integers(0, 32000, size=int(rng.integers(16, 257)))]))
                live.append(next_id)
                next_id += 1
        if step and step % 16 == 0:
            for sid in list(rng.choice(live, size=4, replace=False)):
                ops.append(("fork", int(sid), next_id))
                live.append(next_id)
                next_id += 1
        ops.append(("step", [int(t) for t in rng.integers(0, 32000, size=len(live))], list(live)))
    return ops


def run_block_manager_trace(mgr, ops, max_blocks, seconds=None):
    """Replay the trace on a manager (the library's or the model) until its end
    or, with `seconds`, until that much time has passed.  Returns a dict of
    counts and of the time spent in decode steps (one token for every live
    sequence plus the step's block tables) and in the other operations."""
    r = {"steps": 0, "ops": 0, "adds": 0, "reused": 0, "cows": 0, "step_s": 0.0, "add_s": 0.0,
         "other_s": 0.0}
    t_start = time.perf_counter()
    for op in ops:
        t0 = time.perf_counter()
        if op[0] == "add":
            r["reused"] += mgr.add_sequence(op[1], op[2])[0]
            r["adds"] += 1
        elif op[0] == "free":
            mgr.free_sequence(op[1])
        elif op[0] == "fork":
            mgr.fork(op[1], op[2])
        else:
            r["cows"] += len(mgr.append_step(op[2], op[1])[1])
            if hasattr(mgr, "build_batch"):
                mgr.build_batch(op[2], max_blocks)
            else:
                for sid in op[2]:
                    mgr.block_table(sid)
            r["steps"] += 1
        dt = time.perf_counter() - t0
        r[{"step": "step_s", "add": "add_s"}.get(op[0], "other_s")] += dt
        r["ops"] += 1
        if seconds is not None and time.perf_counter() - t_start > seconds:
            break
    return r


def block_manager_bench(cpu_seconds):
    """Host bookkeeping of the decode loop: the library's block manager on a
    serving-style trace.  The value is the mean time of one decode step's
    bookkeeping (one token appended to every live sequence with its
    copy-on-write pairs, then the step's block tables and lengths)."""
    from paged_kv_cache_388_amd import _lib
    ops = block_manager_trace()
    nb, bs, max_blocks = 40000, 16, 128
    mgr = _lib.BlockManager(nb, bs)
    r = run_block_manager_trace(mgr, ops, max_blocks)
    st = mgr.stats()
    live = [op for op in ops if op[0] == "step"][-1][2]
    line = {"metric": "block manager: host microseconds per decode step",
            "value": round(r["step_s"] / r["steps"] * 1e6, 2), "unit": "us/step",
            "higher_is_better": False, "steps": r["steps"], "data": "synthetic",
            "config": {"workload": "block_manager_trace", "num_blocks": nb, "block_size": bs,
                       "live_sequences_at_end": len(live), "system_prompt_tokens": 1000,
                       "step": "pkv_bm_append_step + pkv_bm_build_batch through the Python binding"},
            "add_sequence_us_mean": round(r["add_s"] / max(r["adds"], 1) * 1e6, 2),
            "sequences_added": r["adds"], "reused_prompt_tokens": r["reused"],
            "copy_on_write_pairs": r["cows"],
            "blocks_in_use": st["blocks_in_use"], "tokens_stored": st["tokens_stored"],
            "waste": round(st["waste"], 5), "cached_blocks": st["cached_blocks"]}
    if cpu_seconds > 0:
        import oracle.block_manager as obm
        m = run_block_manager_trace(obm.BlockManagerModel(nb, bs), ops, max_blocks,
                                    seconds=cpu_seconds)
        line["cpu_baseline"] = {
            "value": round(m["step_s"] / max(m["steps"], 1) * 1e6, 1), "unit": "us/step",
            "cores": 1, "kind": "oracle",
            "sample": f"the Python model on the first {m['ops']} operations ({m['steps']} decode "
                      f"steps) of the same trace, {m['step_s'] + m['add_s'] + m['other_s']:.1f} s"}
    print(json.dumps(line))


def swap_bench(steps, warmup, cpu_seconds):
    """Swap of a preempted batch between the pool and pinned host memory: a
    Llama-3-8B-shaped layer pool (bf16, 8 KV heads, 16-token blocks, D=128) of
    8192 blocks, 2048 scattered blocks (eight 4096-token contexts, 128 MiB of
    K+V) out to host and back into other blocks, with the library's default
    64 MiB staging.  Rates are bytes of K+V moved per second, PCIe included,
    beside a plain contiguous device<->pinned copy of the same size."""
    import torch
    from paged_kv_cache_388_amd import _lib
    _lib.load()
    NB, H, BS, D, n = 8192, 8, 16, 128, 2048
    g = torch.Generator(device="cuda")
    g.manual_seed(388009)
    kc = torch.empty((NB, H, BS, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    kc.view(torch.int16).random_(-32768, 32767, generator=g)
    vc.view(torch.int16).random_(-32768, 32767, generator=g)
    rng = np.random.default_rng(388009)
    perm = rng.permutation(NB).astype(np.int32)
    out_ids = torch.from_numpy(perm[:n].copy()).cuda()
    in_ids = torch.from_numpy(perm[n:2 * n].copy()).cuda()
    moved = n * 2 * H * BS * D * 2
    image = torch.empty((n, 2, H, BS, D), dtype=torch.bfloat16, pin_memory=True)
    staging = torch.empty(_lib.SWAP_STAGING_BYTES, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for i in range(steps):
            a[i].record(stream)
            fn()
            b[i].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([x.elapsed_time(y) for x, y in zip(a, b)]))

    ms_out = timed(lambda: _lib.paged_swap_out(kc, vc, out_ids, host_image=image, staging=staging))
    ms_in = timed(lambda: _lib.paged_swap_in(image, kc, vc, in_ids, staging=staging))
    # the round trip moved out_ids' blocks into in_ids' blocks (bit patterns:
    # the random pools hold NaNs)
    for c in (kc.view(torch.int16), vc.view(torch.int16)):
        assert torch.equal(c[in_ids.long()], c[out_ids.long()])
    dev_flat = torch.empty(moved, dtype=torch.uint8, device="cuda")
    host_flat = torch.empty(moved, dtype=torch.uint8, pin_memory=True)
    ms_d2h = timed(lambda: host_flat.copy_(dev_flat, non_blocking=True))
    ms_h2d = timed(lambda: dev_flat.copy_(host_flat, non_blocking=True))
    gbs = lambda ms: round(moved / (ms * 1e-3) / 1e9, 2)
    line = {"metric": "swap out / in of a preempted batch (K+V bytes moved per second)",
            "value": gbs(ms_out), "unit": "GB/s", "higher_is_better": True, "steps": steps,
            "warmup": warmup, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "swap_llama3_8b_layer", "pool_blocks": NB, "num_kv_heads": H,
                       "block_size": BS, "head_dim": D, "blocks_moved": n,
                       "staging_bytes": _lib.SWAP_STAGING_BYTES},
            "swap_out_ms": round(ms_out, 3), "swap_out_GBps": gbs(ms_out),
            "swap_in_ms": round(ms_in, 3), "swap_in_GBps": gbs(ms_in),
            "plain_d2h_GBps": gbs(ms_d2h), "plain_h2d_GBps": gbs(ms_h2d),
            "swap_out_vs_plain_copy": round(ms_d2h / ms_out, 3),
            "swap_in_vs_plain_copy": round(ms_h2d / ms_in, 3)}
    if cpu_seconds > 0:
        import oracle
        kh = kc.view(torch.int16).cpu().numpy().view(np.uint16)
        vh = vc.view(torch.int16).cpu().numpy().view(np.uint16)
        ids = perm[:n]
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.swap_out(kh, vh, ids)
            reps += 1
            if time.perf_counter() - t0 > cpu_seconds:
                break
        dt = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": round(reps * moved / dt / 1e9, 2), "unit": "GB/s",
                                "cores": 1, "kind": "oracle",
                                "sample": f"oracle swap_out of the same {n} blocks from host "
                                          f"arrays, {reps} repetitions in {dt:.1f} s"}
    print(json.dumps(line))


def copy_probe(mib, steps, warmup):
    """Time the library's plain 16-byte-vector copy: its duration gives the
    achievable read+write rate, and its FETCH_SIZE / WRITE_SIZE counters per
    dispatch calibrate the attention kernel's counters (known bytes moved)."""
    import torch
    from paged_kv_cache_388_amd import _lib
    _lib.load()
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        _lib.pkv_stream_copy(dst, src)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        a[i].record(stream)
        _lib.pkv_stream_copy(dst, src)
        b[i].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([x.elapsed_time(y) for x, y in zip(a, b)]))
    assert torch.equal(dst, src)
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n,
                      "ms_per_copy": round(ms, 4),
                      "read_plus_write_GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}))


def read_probe(mib, steps, warmup):
    """Time the library's plain streaming read: the achievable read rate that
    the decode kernel's bandwidth is compared with."""
    import torch
    from paged_kv_cache_388_amd import _lib
    _lib.load()
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    sink = torch.zeros(_lib.STREAM_READ_WORKGROUPS, dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        _lib.pkv_stream_read(src, sink)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        a[i].record(stream)
        _lib.pkv_stream_read(src, sink)
        b[i].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([x.elapsed_time(y) for x, y in zip(a, b)]))
    print(json.dumps({"read_probe_bytes": n, "ms_per_read": round(ms, 4),
                      "read_GBps": round(n / (ms * 1e-3) / 1e9, 1)}))


def reread_rate(nbytes, rounds, steps, warmup):
    """Mean duration (ms) of the library's re-read probe over a buffer of
    nbytes read `rounds` times per call, each XCD re-reading only its own
    eighth, and the rate in GB/s.  Up to 8 L2s (32 MiB) the re-reads come
    from the XCDs' L2s, above that from the Infinity Cache: the cache-side
    read ceilings that a decode over blocks shared between sequences runs
    against."""
    import torch
    from paged_kv_cache_388_amd import _lib
    _lib.load()
    n = max(16, int(nbytes) // 16 * 16)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    sink = torch.zeros(_lib.STREAM_READ_WORKGROUPS, dtype=torch.int32, device="cuda")
    for _ in range(warmup):
        _lib.pkv_stream_reread(src, rounds, sink)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    a = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    b = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        a[i].record(stream)
        _lib.pkv_stream_reread(src, rounds, sink)
        b[i].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([x.elapsed_time(y) for x, y in zip(a, b)]))
    return n, ms, n * rounds / (ms * 1e-3) / 1e9


def clock_summary(rec, multi):
    """Summary of one call's clock records (pkv_clock_read: uint64 [n, 4]):
    decode waves or prefill workgroups, times in microseconds from the
    earliest start (the counter runs at 100 MHz)."""
    rec = np.asarray(rec, dtype=np.uint64)
    rec = rec[rec[:, 1] != 0]
    t0 = rec[:, 0].astype(np.int64)
    t1 = rec[:, 1].astype(np.int64)
    base = t0.min()
    start = (t0 - base) / 100.0
    end = (t1 - base) / 100.0
    xcd = (rec[:, 2] & np.uint64(0xff)).astype(np.int64)
    r1 = lambda x: round(float(x), 1)
    out = {"units": int(rec.shape[0]), "start_max_us": r1(start.max()),
           "end_p50_us": r1(np.median(end)), "end_max_us": r1(end.max()),
           "xcd_end_p50_us": [r1(np.median(end[xcd == x])) if (xcd == x).any() else None
                              for x in range(8)],
           "xcd_end_max_us": [r1(end[xcd == x].max()) if (xcd == x).any() else None
                              for x in range(8)]}
    if not multi:
        pieces = (rec[:, 2] >> np.uint64(40)).astype(np.int64)
        resid = np.zeros_like(end)
        for x in range(8):
            m = xcd == x
            if m.any():
                resid[m] = end[m] - np.median(end[m])
        out.update({"within_xcd_p10_us": r1(np.percentile(resid, 10)),
                    "within_xcd_p90_us": r1(np.percentile(resid, 90)),
                    "pieces_mean": round(float(pieces.mean()), 2),
                    "corr_end_pieces_within_xcd":
                        round(float(np.corrcoef(resid, pieces)[0, 1]), 3) if pieces.std() > 0 else None})
    else:
        seq = ((rec[:, 2] >> np.uint64(8)) & np.uint64(0xffffff)).astype(np.int64)
        stages = (rec[:, 3] & np.uint64(0xfffff)).astype(np.int64)
        ctx = (rec[:, 3] >> np.uint64(32)).astype(np.int64)
        per_seq = []
        for sv in np.unique(seq):
            m = seq == sv
            per_seq.append({"seq": int(sv), "context": int(ctx[m][0]), "workgroups": int(m.sum()),
                            "start_p50_us": r1(np.median(start[m])), "end_max_us": r1(end[m].max()),
                            "us_per_stage_p50": round(float(np.median((end[m] - start[m]) /
                                                                      np.maximum(stages[m], 1))), 3)})
        ts = np.linspace(0.0, float(end.max()), 11)
        out.update({"sequences": per_seq,
                    "running_at_tenths": [int(((start <= t) & (end > t)).sum()) for t in ts]})
    return out


def reread_probe(mib, rounds, steps, warmup):
    """Print the re-read probe's rate for a buffer of `mib` MiB."""
    n, ms, gbs = reread_rate(mib * (1 << 20), rounds, steps, warmup)
    print(json.dumps({"reread_probe_bytes": n, "rounds": rounds, "ms_per_call": round(ms, 4),
                      "read_GBps": round(gbs, 1)}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed attention calls for this long before the warmup steps: "
                         "after the host-side setup the GPU has idled, and its clocks take "
                         "tens of milliseconds of load to ramp up")
    ap.add_argument("--workload", default="llama3_8b_gqa",
                    help="one of: " + ", ".join(wl.NAMED[:4]) + ", long_ctx_bs16, long_ctx_bs32, "
                         + ", ".join(wl.MULTI))
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="duration of the CPU oracle baseline (0 disables it)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes of the CPU oracle baseline (default: the usable cores, "
                         f"at most {CPU_PROCESS_CAP})")
    ap.add_argument("--read-probe-mib", type=int, default=0,
                    help="instead of the decode step, time pkv_stream_read of this many MiB "
                         "(the achievable read-bandwidth reference)")
    ap.add_argument("--reread-probe-mib", type=float, default=0,
                    help="instead of the decode step, time pkv_stream_reread of this many MiB "
                         "(the L2 / Infinity Cache read ceiling; see --reread-rounds)")
    ap.add_argument("--reread-rounds", type=int, default=64,
                    help="times the re-read probe reads its buffer per call")
    ap.add_argument("--cold", action="store_true",
                    help="write a 1 GiB scrub buffer before every timed step, so that no "
                         "K/V byte is served from L2 or the Infinity Cache")
    ap.add_argument("--decode-path", choices=("stream", "grid"), default="stream",
                    help="grid: every decode call takes the 512-token partition path (one "
                         "workgroup per (kv head, sequence, partition) and the partition "
                         "merge; PAGEDKV_DECODE_PATH=grid) instead of the stream path")
    ap.add_argument("--k-load", choices=("lines", "direct"), default="lines",
                    help="direct: stream-path decode of bf16 / D 128 / 16-token blocks loads K "
                         "straight in the matrix-core operand order instead of whole lines "
                         "re-dealt through LDS (PAGEDKV_K_LOAD=direct; a measurement variant)")
    ap.add_argument("--graph", action="store_true",
                    help="replay the step as one captured HIP graph (the attention call's "
                         "events are then taken in a loop of their own)")
    ap.add_argument("--swap", action="store_true",
                    help="instead of the decode step, time swap out / in of a preempted batch")
    ap.add_argument("--block-manager", action="store_true",
                    help="instead of the decode step, time the host block manager on a "
                         "serving-style trace")
    ap.add_argument("--clock", action="store_true",
                    help="after the warmup, run --steps attention calls of the clock build "
                         "(PAGEDKV_CLOCK=1; bf16, D 128, 16-token blocks) and print each "
                         "call's per-wave (decode) or per-workgroup (prefill) start/end "
                         "summary instead of the bench line")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="instead of the decode step, time pkv_stream_copy of this many MiB "
                         "(the reference copy for bandwidth and HBM counter calibration)")
    args = ap.parse_args()
    if args.graph and args.cold:
        ap.error("--graph and --cold exclude each other (the scrub is not part of the step)")

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    if args.block_manager:
        block_manager_bench(args.cpu_seconds)
        return
    if args.swap:
        swap_bench(args.steps, args.warmup, args.cpu_seconds)
        return
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib, args.steps, args.warmup)
        return
    if args.read_probe_mib > 0:
        read_probe(args.read_probe_mib, args.steps, args.warmup)
        return
    if args.reread_probe_mib > 0:
        reread_probe(args.reread_probe_mib, args.reread_rounds, args.steps, args.warmup)
        return

    if args.decode_path == "grid":
        os.environ["PAGEDKV_DECODE_PATH"] = "grid"   # read by the library on every call
    if args.k_load == "direct":
        os.environ["PAGEDKV_K_LOAD"] = "direct"
    t_gen = time.perf_counter()
    w = wl.named(args.workload)
    print(f"[bench] workload {w.name} generated in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    cpu = None
    if args.cpu_seconds > 0:
        workers = args.cpu_workers or min(CPU_PROCESS_CAP, len(os.sched_getaffinity(0)))
        cpu = cpu_baseline(w, args.cpu_seconds, workers)
        print(f"[bench] cpu oracle: {cpu['sample']}", file=sys.stderr, flush=True)

    import torch
    from paged_kv_cache_388_amd import _lib
    _lib.load()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.int32 or w.dtype == "f32":
            return torch.from_numpy(a).to(dev)
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        return torch.from_numpy(a.view(np.int16)).to(dev).view(tdt)

    q = up(w.q)
    k_cache, v_cache = up(w.k_cache), up(w.v_cache)
    block_tables, context_lens = up(w.block_tables), up(w.context_lens)
    block_mapping = up(w.block_mapping.astype(np.int32))
    slot_mapping = up(w.slot_mapping.astype(np.int32))
    new_key, new_value = up(w.new_key), up(w.new_value)
    out = torch.empty_like(q)
    if w.multi:
        query_start = up(w.query_start.astype(np.int32))
        ws_bytes = _lib.paged_attention_multi_workspace_bytes(k_cache, w.num_seqs, w.num_q_heads,
                                                              w.max_query_len, w.max_context_len)
    else:
        ws_bytes = _lib.paged_attention_workspace_bytes(k_cache, w.num_seqs, w.num_q_heads,
                                                        w.max_context_len)
    workspace = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    max_ctx = w.max_context_len
    torch.cuda.synchronize()

    def write_step():
        if block_mapping.shape[0]:
            _lib.paged_copy_blocks(k_cache, v_cache, block_mapping)
        if slot_mapping.shape[0]:
            _lib.paged_kv_append(new_key, new_value, k_cache, v_cache, slot_mapping)

    def attend():
        if w.multi:
            _lib.paged_attention_multi(out, q, k_cache, v_cache, block_tables, context_lens,
                                       query_start, w.scale, max_ctx, w.max_query_len, workspace)
        else:
            _lib.paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens,
                                        w.scale, max_ctx, workspace)

    # clock settle (see --settle-ms), in batches of calls between waits
    t_settle = time.perf_counter() + args.settle_ms * 1e-3
    while time.perf_counter() < t_settle:
        for _ in range(20):
            attend()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        write_step()
        attend()
    torch.cuda.synchronize()

    if args.clock:
        if w.dtype != "bf16" or w.head_dim != 128 or w.block_size != 16:
            print("--clock: the clock build exists for bf16, head_dim 128, 16-token blocks only",
                  file=sys.stderr)
            sys.exit(2)
        calls = []
        for i in range(args.steps):
            os.environ["PAGEDKV_CLOCK"] = "1"
            attend()
            del os.environ["PAGEDKV_CLOCK"]
            calls.append(clock_summary(_lib.pkv_clock_read(), w.multi))
            print(f"[bench] clock call {i}: last end {calls[-1]['end_max_us']} us",
                  file=sys.stderr, flush=True)
        print(json.dumps({"clock": w.name, "calls": calls}))
        return

    stream = torch.cuda.current_stream()
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if args.cold else None
    wstarts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    wends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    if args.graph:
        # the step (cache writes + attention) captured once as a HIP graph and
        # replayed: one launch per step instead of one per kernel
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            write_step()
            attend()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        # the attention call alone, for its events (roofline)
        for i in range(args.steps):
            starts[i].record(stream)
            attend()
            ends[i].record(stream)
        torch.cuda.synchronize()
    else:
        t0 = time.perf_counter()
        for i in range(args.steps):
            if scrub is not None:
                scrub.fill_(i & 0xff)
                wstarts[i].record(stream)
            write_step()
            starts[i].record(stream)
            attend()
            ends[i].record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    if scrub is None:
        # the cache writes alone, outside the timed region (an extra event per
        # step inside it would lengthen the step it measures); they rewrite
        # the same values into the same slots
        for i in range(args.steps):
            wstarts[i].record(stream)
            write_step()
            wends[i].record(stream)
        torch.cuda.synchronize()
    else:
        wends = starts
    write_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(wstarts, wends)]))

    # the achievable-read reference on the same device: 4 GiB read once
    probe_src = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    probe_sink = torch.zeros(_lib.STREAM_READ_WORKGROUPS, dtype=torch.int32, device=dev)
    for _ in range(2):
        _lib.pkv_stream_read(probe_src, probe_sink)
    pa = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    pb = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    for i in range(5):
        pa[i].record(stream)
        _lib.pkv_stream_read(probe_src, probe_sink)
        pb[i].record(stream)
    torch.cuda.synchronize()
    probe_gbs = (4 << 30) / (float(np.mean([a.elapsed_time(b) for a, b in zip(pa, pb)])) * 1e-3) / 1e9
    del probe_src

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    attn_avg_ms = float(np.mean(attn_ms))
    if args.cold:
        # the scrub is not part of the step: take the step from its events
        ms_per_step = write_ms + attn_avg_ms
    kv = w.kv_bytes()
    value = kv / (ms_per_step * 1e-3) / 1e9
    alg = algorithmic_bytes(w)
    uniq = unique_kv_bytes(w)
    shared = uniq < kv
    if shared:
        # blocks shared between sequences are read once from HBM at best:
        # the roofline is taken on the distinct bytes
        alg = alg - kv + uniq
    achieved = alg / (attn_avg_ms * 1e-3) / 1e9
    flops = attention_flops(w)
    l2 = None
    if shared and not w.multi:
        # blocks read by many sequences are served by the L2 of the XCD that
        # streams their kv head: the ceiling is the L2 re-read rate over a
        # buffer of the shared blocks' size, read as many times as they are
        sb, reads = shared_block_bytes(w)
        rounds = max(1, int(round(reads)))
        _, l2_ms, l2_gbs = reread_rate(sb, rounds, 10, 2)
        logical = algorithmic_bytes(w)
        l2 = {"shared_block_bytes": sb, "reads_per_shared_block": round(reads, 2),
              "probe_rounds": rounds, "probe_GBps": round(l2_gbs, 1),
              "logical_bytes_per_launch": logical,
              "logical_GBps": round(logical / (attn_avg_ms * 1e-3) / 1e9, 1)}
    G = w.num_q_heads // w.num_kv_heads
    if w.multi and w.max_query_len * G >= PREFILL_MIN_COLS:
        # the prefill path reads each context once per 64 columns and does
        # 4*D flops per (column, visible token): far above the MFMA/HBM ridge
        # (2.5 PFLOP/s / 8 TB/s = 312 flop/B), so it is priced on the matrix cores
        tflops = flops / (attn_avg_ms * 1e-3) / 1e12
        peak = PEAK_MFMA_TFLOPS[w.dtype]
        roofline = {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": None,
                    "kernel": (f"attn_prefill_kernel<{w.dtype},{w.head_dim},{w.block_size}> "
                               "(+ attn_prefill_merge_kernel when contexts are cut into "
                               "parts; one paged_attention_multi call)"),
                    "algorithmic_flops_per_launch": flops,
                    "algorithmic_bytes_per_launch": alg,
                    "hbm_GBps_of_algorithmic_bytes": round(achieved, 1)}
    elif l2 is not None:
        # shared blocks: not HBM-bound; every logical byte passes through L2
        roofline = {"bound": "l2", "achieved": l2["logical_GBps"], "peak": l2["probe_GBps"],
                    "unit": "GB/s", "frac": round(l2["logical_GBps"] / l2["probe_GBps"], 4),
                    "traffic": None,
                    "peak_source": ("measured in this run: pkv_stream_reread over the shared "
                                    "blocks' bytes, as many rounds as each is read (no "
                                    "published L2 figure)"),
                    "kernel": (f"attn_stream_kernel<{w.dtype},{w.head_dim},{w.block_size}> + "
                               "attn_stream_merge_kernel (one paged_attention_decode call)"),
                    "algorithmic_bytes_per_launch": l2["logical_bytes_per_launch"],
                    "kv_bytes_unique": uniq,
                    "unique_bytes_GBps": round(achieved, 1),
                    "unique_frac_of_hbm_peak": round(achieved / PEAK_HBM_GBS, 4),
                    **{k: l2[k] for k in ("shared_block_bytes", "reads_per_shared_block",
                                          "probe_rounds")}}
    else:
        grid = args.decode_path == "grid" and not w.multi
        kname = "attn_grid_kernel" if grid else "attn_stream_kernel"
        merge = "attn_reduce_kernel" if grid else "attn_stream_merge_kernel"
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": counter_traffic(w.name, kname),
                    "kernel": (f"{kname}<{w.dtype},{w.head_dim},{w.block_size}> + {merge} (one "
                               f"{'paged_attention_multi' if w.multi else 'paged_attention_decode'}"
                               " call)"),
                    "algorithmic_bytes_per_launch": alg,
                    **({"kv_bytes_logical": kv, "kv_bytes_unique": uniq,
                        "note": ("K/V shared between sequences: achieved counts each distinct "
                                 "byte once; the distinct footprint fits in the Infinity "
                                 "Cache, so a warm run is not HBM-bound (see --cold)")}
                       if shared else {})}
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "num_blocks": w.num_blocks,
                   "mean_context": round(float(w.context_lens.mean()), 1),
                   "max_context": max_ctx, "kv_bytes_per_step": kv, "seed": w.seed,
                   "step": ("copy_blocks + paged_kv_append + "
                            + ("paged_attention_multi" if w.multi else "paged_attention_decode")),
                   "new_tokens": int(w.q.shape[0]),
                   "parallelism": "single GPU", "cold": bool(args.cold),
                   "graph": bool(args.graph),
                   **({"decode_path": args.decode_path, "k_load": args.k_load}
                      if not w.multi else {})},
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "seqs_per_s": round(w.num_seqs / (ms_per_step * 1e-3), 1),
        "new_tokens_per_s": round(w.q.shape[0] / (ms_per_step * 1e-3), 1),
        "attention_tflops": round(flops / (attn_avg_ms * 1e-3) / 1e12, 2),
        "cache_writes_ms": round(write_ms, 4),
        "read_probe_GBps": round(probe_gbs, 1),
        "frac_of_read_probe": round(achieved / probe_gbs, 4),
        "attention_ms": {"mean": round(attn_avg_ms, 4),
                         "p10": round(float(np.percentile(attn_ms, 10)), 4),
                         "p50": round(float(np.percentile(attn_ms, 50)), 4),
                         "p90": round(float(np.percentile(attn_ms, 90)), 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
