"""Pins for the oracle's multi-token paged attention (several new tokens per
sequence: speculative-decode verification, chunked-prefill chunks).

* one new token per sequence reduces to decode attention, which is pinned on
  its own;
* against torch's causal scaled-dot-product attention in fp64 (a library
  routine) over each whole unpaged sequence: the last L rows of full causal
  self-attention are exactly the L new tokens' outputs;
* row i equals decode attention over the first n - L + i + 1 tokens;
* physical placement does not matter (bit for bit);
* planted mistakes in the causal offset or the row order are rejected.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from test_oracle_pins import _make_case, _paged_from_contiguous, _round


def _case(rng, ctx, qlens, H_q, H_kv, D, bs, dtype):
    """Paged pool of every sequence's K/V plus packed queries for the last
    qlens[s] positions; also returns full-sequence fp64 queries (random for
    the earlier positions) for the causal SDPA pin."""
    B = len(ctx)
    c = _make_case(rng, B, H_q, H_kv, D, ctx, bs, dtype)
    n_max = max(1, max(ctx))
    qfull_st, qfull64 = _round(rng.standard_normal((B, n_max, H_q, D)), dtype)
    rows = []
    rows64 = []
    for s in range(B):
        n, L = ctx[s], qlens[s]
        for i in range(L):
            rows.append(qfull_st[s, n - L + i])
            rows64.append(qfull64[s, n - L + i])
    shape = (0, H_q, D)
    q = np.stack(rows) if rows else np.zeros(shape, dtype=qfull_st.dtype)
    q64 = np.stack(rows64) if rows64 else np.zeros(shape)
    return c, q, q64, qfull64


def _causal_sdpa_last_rows(c, qfull64, ctx, qlens, scale, G):
    out = []
    for s, (n, L) in enumerate(zip(ctx, qlens)):
        if L == 0:
            continue
        H_q = qfull64.shape[2]
        D = qfull64.shape[3]
        q = torch.from_numpy(qfull64[s, :n].transpose(1, 0, 2).copy()).reshape(1, H_q, n, D)
        k = torch.from_numpy(c["k64"][s, :, :n]).repeat_interleave(G, dim=0).reshape(1, H_q, n, D)
        v = torch.from_numpy(c["v64"][s, :, :n]).repeat_interleave(G, dim=0).reshape(1, H_q, n, D)
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
        o = o.reshape(H_q, n, D).numpy().transpose(1, 0, 2)
        out.append(o[n - L:])
    return np.concatenate(out) if out else np.zeros((0,) + qfull64.shape[2:])


def test_one_new_token_is_decode():
    rng = np.random.default_rng(31)
    ctx = [1, 4, 17, 33]
    c = _make_case(rng, len(ctx), 4, 2, 8, ctx, 4, "bf16")
    got = oracle.multi_query_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"],
                                       [1] * len(ctx), 0.3, "bf16")
    want = oracle.decode_attention(c["q"], c["kpool"], c["vpool"], c["bt"], c["ctx"], 0.3, "bf16")
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H_q,H_kv", [(2, 2), (4, 1), (8, 2)])
def test_causal_sdpa_last_rows(dtype, H_q, H_kv):
    rng = np.random.default_rng(32)
    ctx = [1, 5, 9, 16, 23, 40]
    qlens = [1, 5, 3, 0, 7, 16]       # includes a whole-context chunk (L = n)
    D, bs = 8, 4
    c, q, _, qfull64 = _case(rng, ctx, qlens, H_q, H_kv, D, bs, dtype)
    scale = 1 / math.sqrt(D)
    got = oracle.multi_query_attention(q, c["kpool"], c["vpool"], c["bt"], c["ctx"], qlens, scale,
                                       dtype)
    ref = _causal_sdpa_last_rows(c, qfull64, ctx, qlens, scale, H_q // H_kv)
    assert got.shape == ref.shape == (sum(qlens), H_q, D)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_rows_equal_decode_over_truncated_contexts():
    rng = np.random.default_rng(33)
    ctx = [6, 20, 35]
    qlens = [4, 1, 6]
    c, q, _, _ = _case(rng, ctx, qlens, 4, 2, 16, 8, "bf16")
    got = oracle.multi_query_attention(q, c["kpool"], c["vpool"], c["bt"], c["ctx"], qlens, 0.25,
                                       "bf16")
    row = 0
    for s, (n, L) in enumerate(zip(ctx, qlens)):
        for i in range(L):
            one = oracle.decode_attention(q[row:row + 1], c["kpool"], c["vpool"], c["bt"][s:s + 1],
                                          np.array([n - L + i + 1]), 0.25, "bf16")
            assert np.array_equal(got[row], one[0])
            row += 1


def test_physical_permutation_invariance_bitwise():
    rng = np.random.default_rng(34)
    ctx = [7, 18, 40]
    qlens = [3, 5, 8]
    c, q, _, _ = _case(rng, ctx, qlens, 8, 2, 16, 4, "bf16")
    base = oracle.multi_query_attention(q, c["kpool"], c["vpool"], c["bt"], c["ctx"], qlens, 0.2,
                                        "bf16")
    NB = c["kpool"].shape[0]
    pi = rng.permutation(NB)
    kp = np.empty_like(c["kpool"])
    vp = np.empty_like(c["vpool"])
    kp[pi] = c["kpool"]
    vp[pi] = c["vpool"]
    bt = np.where(c["bt"] >= 0, pi[np.maximum(c["bt"], 0)], -1).astype(np.int32)
    moved = oracle.multi_query_attention(q, kp, vp, bt, c["ctx"], qlens, 0.2, "bf16")
    assert np.array_equal(base, moved)


def test_rejects_more_new_tokens_than_cached():
    rng = np.random.default_rng(35)
    c = _make_case(rng, 1, 2, 2, 8, [3], 4, "f32")
    with pytest.raises(ValueError):
        oracle.multi_query_attention(np.zeros((4, 2, 8), np.float32), c["kpool"], c["vpool"],
                                     c["bt"], c["ctx"], [4], 0.1, "f32")


# ---------------------------------------------------------------------------
# planted mistakes (copies of the oracle with one plausible bug each)
# ---------------------------------------------------------------------------

def _mutant(kind):
    from oracle import paged_attention as pa

    def run(q, kpool, vpool, bt, ctx, qlens, scale, dtype):
        H_q = q.shape[1]
        G = H_q // kpool.shape[1]
        out = np.zeros(q.shape)
        row = 0
        for s, L in enumerate(qlens):
            n = int(ctx[s])
            if L == 0:
                continue
            K = pa.gather_context(kpool, bt[s], n, dtype)
            V = pa.gather_context(vpool, bt[s], n, dtype)
            for i in range(L):
                visible = n - L + i + (0 if kind == "exclusive" else 1)
                if kind == "from_start":
                    visible = i + 1
                src = row + (L - 1 - i if kind == "reversed_rows" else i)
                qs = pa.storage_to_f64(q[src], dtype)
                for h in range(H_q):
                    sc = scale * (K[h // G, :visible] @ qs[h])
                    p = np.exp(sc - sc.max())
                    out[row + i, h] = (p @ V[h // G, :visible]) / p.sum()
            row += L
        return out
    return run


@pytest.mark.parametrize("kind", ["exclusive", "from_start", "reversed_rows"])
def test_pins_reject_planted_mistakes(kind):
    rng = np.random.default_rng(36)
    ctx = [5, 9, 12]
    qlens = [3, 2, 4]
    c, q, _, qfull64 = _case(rng, ctx, qlens, 4, 2, 8, 4, "f32")
    scale = 1 / math.sqrt(8)
    ref = _causal_sdpa_last_rows(c, qfull64, ctx, qlens, scale, 2)
    ok = _mutant("none")(q, c["kpool"], c["vpool"], c["bt"], c["ctx"], qlens, scale, "f32")
    bad = _mutant(kind)(q, c["kpool"], c["vpool"], c["bt"], c["ctx"], qlens, scale, "f32")
    assert np.max(np.abs(ok - ref)) <= 1e-12
    assert not (np.max(np.abs(bad - ref)) <= 1e-12)
