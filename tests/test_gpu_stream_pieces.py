"""Chunk and workgroup boundaries of the stream path (needs an MI355X).

The stream kernel cuts the ordered positions (kv head, sequence, 16-token
sub-tile) into one equal chunk per wave, at least 4 positions each; a
workgroup's 4 waves hold consecutive chunks.  Pieces of a group span that
cross a wave boundary inside a workgroup are merged there in LDS and written
directly; what crosses a workgroup boundary goes to the workgroup's slot 0
or 1 and the merge kernel finishes it.  With few positions (at most 4 per
wave on a 256-CU device) every chunk is 4 positions and a workgroup 16, so
context lengths in multiples of 64 and 256 tokens put span ends exactly on
wave and workgroup boundaries: spans inside one wave, spans over 2..4 waves
of one workgroup, spans that start exactly at a workgroup start, spans
covering whole workgroups, and spans straddling workgroup boundaries at
every phase, with empty contexts and empty trailing waves between them.
Decode and 4 new tokens per sequence (one 16-column group) are both
checked against the oracle.
"""

import numpy as np
import pytest
import torch

from paged_kv_cache_388_amd import workloads as wl

from gpu_common import DeviceWorkload, check_attention, oracle_step, to_host

pytestmark = pytest.mark.gpu

# positions per kv head: 4 4 8 16 0 16 32 64 1 3 16 24 128 2 16 17 256 2 0 48
CTX = [64, 64, 128, 256, 0, 256, 512, 1024, 16, 48, 256, 384, 2048, 17, 255, 257, 4096, 32, 0,
       768]


def _run(w, what):
    print(f"[gpu] {what}: B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"D={w.head_dim} {w.dtype} maxctx={w.max_context_len}", flush=True)
    out = DeviceWorkload(w).step()
    torch.cuda.synchronize()
    return check_attention(to_host(out, w.dtype), oracle_step(w), w.dtype, what)


@pytest.mark.parametrize("H_kv", [1, 2])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_decode_spans_on_chunk_boundaries(H_kv, dtype):
    rng = np.random.default_rng(61)
    w = wl.build(f"pieces_{H_kv}_{dtype}", 61, rng, CTX, 4 * H_kv, H_kv, 128, 16, dtype,
                 poison=True)
    _run(w, f"decode, aligned spans, H_kv={H_kv}")


@pytest.mark.parametrize("H_kv", [1, 2])
def test_verify_spans_on_chunk_boundaries(H_kv):
    rng = np.random.default_rng(62)
    ql = [min(4, c) for c in CTX]
    w = wl.build(f"pieces_multi_{H_kv}", 62, rng, CTX, 4 * H_kv, H_kv, 128, 16, "bf16",
                 poison=True, query_lens=ql)
    assert w.max_query_len * 4 == 16  # one 16-column group per sequence: the per-group merge
    _run(w, f"4 new tokens, aligned spans, H_kv={H_kv}")


def test_spans_shifted_by_one_position():
    """The same lengths behind one extra 16-token sequence: every span end
    moves one position off the boundaries it sat on."""
    rng = np.random.default_rng(63)
    w = wl.build("pieces_shift", 63, rng, [16] + CTX, 8, 2, 64, 16, "bf16", poison=True)
    _run(w, "decode, spans shifted by one position")
