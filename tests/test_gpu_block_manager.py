"""The host block manager driving the device path (needs an MI355X).

A small serving loop: prompts that share a system prompt (prefix-cache
reuse), forks whose next token triggers copy-on-write, frees, new sequences
that land in released and evicted blocks, and a sequence swapped out to host
memory while others reuse its blocks, then swapped back into other blocks.  Every step the manager's
slots, copy-on-write pairs and block tables feed paged_copy_blocks,
paged_kv_append and paged_attention_decode; the outputs are compared with
attention over each sequence's logical K/V kept on the host, which involves
no pool or table at all.  A token's K/V are a function of the whole prefix
ending at it, as in a real model, so reused prefix blocks hold exactly what a
recomputation would write.
"""

import hashlib

import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_388_amd import BlockManager
from paged_kv_cache_388_amd import _lib

from gpu_common import check_attention, to_dev, to_host

pytestmark = pytest.mark.gpu

H_KV, G, D, BS = 2, 4, 64, 16
H_Q = H_KV * G
DT = "bf16"


def _kv_of_prefix(tokens):
    """K and V of the last token of `tokens`, seeded by the whole prefix."""
    h = hashlib.sha256(np.asarray(tokens, dtype=np.int64).tobytes()).digest()
    rng = np.random.default_rng(int.from_bytes(h[:8], "little"))
    kv = rng.standard_normal((2, H_KV, D)).astype(np.float32)
    t = torch.from_numpy(kv).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _oracle_decode(q_rows, logical):
    """fp64 attention of q_rows[i] over logical[i] = (K [n, H_kv, D], V ...)."""
    outs = []
    for q, (k, v) in zip(q_rows, logical):
        n = k.shape[0]
        nb = -(-n // BS)
        kp = np.zeros((nb, H_KV, BS, D), dtype=np.uint16)
        vp = np.zeros((nb, H_KV, BS, D), dtype=np.uint16)
        for t in range(n):
            kp[t // BS, :, t % BS] = k[t]
            vp[t // BS, :, t % BS] = v[t]
        outs.append(oracle.decode_attention(q[None], kp, vp, np.arange(nb)[None], np.array([n]),
                                            1 / np.sqrt(D), DT)[0])
    return np.stack(outs)


def test_block_manager_drives_decode():
    rng = np.random.default_rng(71)
    NB = 160
    bm = BlockManager(NB, BS)
    dev = torch.device("cuda", 0)
    kc = torch.zeros((NB, H_KV, BS, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    tokens = {}      # seq id -> token ids
    logical = {}     # seq id -> [K list, V list]
    cow_pairs = []

    def write(sid, new_toks, slots, cow):
        if cow is not None:
            cow_pairs.append(cow)
            _lib.paged_copy_blocks(kc, vc, to_dev(np.array([cow], dtype=np.int32), DT))
        base = len(tokens[sid])
        keys, vals = [], []
        for i, t in enumerate(new_toks):
            tokens[sid].append(int(t))
            kv = _kv_of_prefix(tokens[sid])
            logical[sid][0].append(kv[0])
            logical[sid][1].append(kv[1])
            keys.append(kv[0])
            vals.append(kv[1])
        assert len(tokens[sid]) == base + len(new_toks)
        _lib.paged_kv_append(to_dev(np.stack(keys), DT), to_dev(np.stack(vals), DT), kc, vc,
                             to_dev(np.asarray(slots, dtype=np.int32), DT))

    def add(sid, prompt):
        reused, slots = bm.add_sequence(sid, prompt)
        tokens[sid], logical[sid] = [], [[], []]
        # reused tokens' K/V are already in shared blocks: only the logical copy is made
        for t in prompt[:reused]:
            tokens[sid].append(int(t))
            kv = _kv_of_prefix(tokens[sid])
            logical[sid][0].append(kv[0])
            logical[sid][1].append(kv[1])
        write(sid, prompt[reused:], slots[reused:], None)
        return reused

    def fork(parent, child):
        bm.fork(parent, child)
        tokens[child] = list(tokens[parent])
        logical[child] = [list(logical[parent][0]), list(logical[parent][1])]

    swapped = {}     # seq id -> host image

    def decode_all(step):
        live = sorted(set(tokens) - set(swapped))
        toks = [int(t) for t in rng.integers(0, 1000, size=len(live))]
        slots, cows = bm.append_step(live, toks)
        for c in cows:                  # every copy lands before any of the step's writes
            cow_pairs.append(tuple(int(x) for x in c))
        if len(cows):
            _lib.paged_copy_blocks(kc, vc, to_dev(np.ascontiguousarray(cows), DT))
        for sid, tok, slot in zip(live, toks, slots):
            write(sid, [tok], [slot], None)
        bt, lens = bm.build_batch(live, 64)
        q = rng.standard_normal((len(live), H_Q, D)).astype(np.float32)
        q_st = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        out = torch.empty((len(live), H_Q, D), dtype=torch.bfloat16, device=dev)
        _lib.paged_attention_decode(out, to_dev(q_st, DT), kc, vc, to_dev(bt, DT),
                                    to_dev(lens, DT), 1 / np.sqrt(D), int(lens.max()))
        torch.cuda.synchronize()
        ref = _oracle_decode(q_st, [(np.stack(logical[s][0]), np.stack(logical[s][1]))
                                    for s in live])
        check_attention(to_host(out, DT), ref, DT, f"step {step}")

    system = list(rng.integers(0, 1000, size=100))
    reuses = [add(u, system + list(rng.integers(0, 1000, size=int(rng.integers(5, 40)))))
              for u in range(5)]
    assert reuses[0] == 0 and all(r == 96 for r in reuses[1:])   # 6 full blocks of the prompt
    for step in range(24):
        if step == 3:
            fork(1, 10)
            fork(2, 11)
        if step == 8:
            bm.free_sequence(0)
            del tokens[0], logical[0]
        if step == 12:
            add(20, system + [7, 7, 7])
        if step == 14:
            ids = bm.swap_out(3)
            swapped[3] = _lib.paged_swap_out(kc, vc, to_dev(ids, DT))
            torch.cuda.synchronize()
        if step == 15:                  # takes blocks sequence 3 gave up
            add(21, list(rng.integers(0, 1000, size=60)))
        if step == 19:
            ids = bm.swap_in(3)
            _lib.paged_swap_in(swapped.pop(3), kc, vc, to_dev(ids, DT))
        decode_all(step)
    assert len(cow_pairs) >= 2          # each fork's first write copied the shared block
    st = bm.stats()
    assert st["num_sequences"] == len(tokens)
    assert st["tokens_stored"] <= st["slots_reserved"]
