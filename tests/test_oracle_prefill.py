"""Pins of the chunked-prefill oracle (multi-query paged attention) against
things other than itself: a Python-float brute force with the causal rule
written out, torch's scaled_dot_product_attention with an explicit mask, the
decode oracle (n_q = 1), invariance under how a prompt is cut into chunks
and under block placement, closed forms, the flop count, and the page's
prefix-hit example.  A last test plants mistakes and checks that a pin fails.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import chunked_prefill as cp
from oracle import paged_attention as pa_oracle
from tests.test_oracle import BS, build_pool


def make_case(rng, lens, nqs, Hq, Hkv, D, extra_blocks=3):
    """Contiguous K/V per sequence scattered into a shuffled pool by the test's
    own layout code; q rows for the last nqs[s] positions of each sequence."""
    nbs = [-(-n // BS) for n in lens]
    NB = sum(nbs) + extra_blocks
    perm = rng.permutation(NB)
    MB = max(max(nbs), 1)
    tab = np.full((len(lens), MB), -1, dtype=np.int32)
    tables, kl, vl, at = [], [], [], 0
    for s, n in enumerate(lens):
        row = perm[at:at + nbs[s]]
        at += nbs[s]
        tab[s, :len(row)] = row
        tables.append(row)
        kl.append(rng.standard_normal((n, Hkv, D), dtype=np.float32).astype(np.float16))
        vl.append(rng.standard_normal((n, Hkv, D), dtype=np.float32).astype(np.float16))
    kc, vc = build_pool(kl, vl, tables, NB, Hkv, D)
    starts = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
    q = rng.standard_normal((int(starts[-1]), Hq, D), dtype=np.float32).astype(np.float16)
    return q, kl, vl, tab, np.asarray(lens, dtype=np.int32), starts, kc, vc


def brute_force_causal(q, starts, lens, kl, vl, scale, Hkv):
    """Python floats: row i of sequence s's chunk is at position
    len - nq + i and sees keys 0..that position."""
    T, Hq, D = q.shape
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    sc = float(np.float32(scale))
    for s in range(len(lens)):
        n = int(lens[s])
        nq = int(starts[s + 1] - starts[s])
        for i in range(nq):
            pos = n - nq + i
            row = int(starts[s]) + i
            for h in range(Hq):
                kh = h // G
                logits = []
                for j in range(pos + 1):
                    acc = 0.0
                    for d in range(D):
                        acc += float(q[row, h, d]) * float(kl[s][j, kh, d])
                    logits.append(acc * sc)
                mx = max(logits)
                w = [math.exp(z - mx) for z in logits]
                tot = sum(w)
                for d in range(D):
                    out[row, h, d] = sum(w[j] * float(vl[s][j, kh, d]) for j in range(pos + 1)) / tot
    return out


def sdpa_masked(q, starts, lens, kl, vl, scale, Hkv):
    """torch scaled_dot_product_attention in float64 with a boolean mask
    allowing key j for the query at position len - nq + i when j <= it."""
    T, Hq, D = q.shape
    G = Hq // Hkv
    out = np.zeros((T, Hq, D))
    for s in range(len(lens)):
        n = int(lens[s])
        t0, t1 = int(starts[s]), int(starts[s + 1])
        nq = t1 - t0
        if nq == 0:
            continue
        qt = torch.from_numpy(q[t0:t1].astype(np.float64)).permute(1, 0, 2).unsqueeze(0)
        kt = torch.from_numpy(kl[s].astype(np.float64)).permute(1, 0, 2)
        vt = torch.from_numpy(vl[s].astype(np.float64)).permute(1, 0, 2)
        kt = kt.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        vt = vt.repeat_interleave(G, dim=0).unsqueeze(0).contiguous()
        pos = torch.arange(n - nq, n).reshape(nq, 1)
        mask = torch.arange(n).reshape(1, n) <= pos
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=float(np.float32(scale)))
        out[t0:t1] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("Hq,Hkv,D,lens,nqs", [
    (4, 4, 16, [1, 16, 17, 50], [1, 5, 17, 20]),
    (8, 2, 16, [33, 48, 5], [33, 3, 0]),
    (4, 1, 8, [20, 40], [7, 40]),
])
def test_prefill_matches_brute_force(Hq, Hkv, D, lens, nqs):
    rng = np.random.default_rng(sum(lens) + Hq)
    q, kl, vl, tab, la, starts, kc, vc = make_case(rng, lens, nqs, Hq, Hkv, D)
    got = oracle.prefill(q, kc, vc, tab, la, starts, np.float32(0.3), Hkv)
    ref = brute_force_causal(q, starts, la, kl, vl, np.float32(0.3), Hkv)
    assert np.abs(got - ref).max() < 1e-12


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 32), (6, 6, 64), (16, 4, 128)])
def test_prefill_matches_masked_sdpa(Hq, Hkv, D):
    rng = np.random.default_rng(Hq * D)
    lens, nqs = [100, 37, 64, 130], [64, 37, 1, 70]
    q, kl, vl, tab, la, starts, kc, vc = make_case(rng, lens, nqs, Hq, Hkv, D)
    scale = np.float32(1.0 / math.sqrt(D))
    got = oracle.prefill(q, kc, vc, tab, la, starts, scale, Hkv)
    ref = sdpa_masked(q, starts, la, kl, vl, scale, Hkv)
    assert np.abs(got - ref).max() < 1e-12


def test_chunks_of_one_are_decode():
    """n_q = 1 everywhere is a decode step: bit-identical to the decode
    oracle, which has pins of its own."""
    rng = np.random.default_rng(5)
    lens = [1, 15, 16, 17, 90]
    q, kl, vl, tab, la, starts, kc, vc = make_case(rng, lens, [1] * 5, 8, 2, 32)
    got = oracle.prefill(q, kc, vc, tab, la, starts, np.float32(0.2), 2)
    ref = oracle.decode(q, kc, vc, tab, la, np.float32(0.2), 2)
    assert np.array_equal(got, ref)


def test_cutting_a_prompt_into_chunks_changes_nothing():
    """Chunked prefill: the rows of a prompt computed as one chunk equal the
    rows computed chunk by chunk, each chunk with the context it has grown to
    (ttlab section 3, chunked prefill).  Bit-identical: every row meets the
    same keys in the same order."""
    rng = np.random.default_rng(9)
    n = 150
    q, kl, vl, tab, la, starts, kc, vc = make_case(rng, [n], [n], 8, 2, 32)
    whole = oracle.prefill(q, kc, vc, tab, la, starts, np.float32(0.25), 2)
    cuts = [0, 40, 41, 100, 150]
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = oracle.prefill(q[a:b], kc, vc, tab, np.array([b], np.int32),
                              np.array([0, b - a], np.int32), np.float32(0.25), 2)
        assert np.array_equal(part, whole[a:b])


def test_prefix_hit_continuation_page_example():
    """aquanode "Prefix caching": a 2,100-token prompt with 2,000 tokens in
    125 cached full blocks leaves a 100-token chunk.  That chunk, attending
    to the cached blocks, equals the last 100 rows of the whole prompt's
    prefill (small heads to keep the oracle quick)."""
    rng = np.random.default_rng(12)
    prompt, cached = 2100, 125 * BS
    assert cached == 2000
    nq = prompt - cached
    q, kl, vl, tab, la, starts, kc, vc = make_case(rng, [prompt], [nq], 2, 1, 8)
    got = oracle.prefill(q, kc, vc, tab, la, starts, np.float32(0.35), 1)
    q_all = np.concatenate([rng.standard_normal((cached, 2, 8), dtype=np.float32)
                            .astype(np.float16), q])
    whole = oracle.prefill(q_all, kc, vc, tab, la, np.array([0, prompt], np.int32),
                           np.float32(0.35), 1)
    assert np.array_equal(got, whole[cached:])


def test_first_position_returns_its_value_row():
    """A chunk that starts the sequence: its first row sees only position 0,
    so the output is V[0] (softmax over one logit is 1)."""
    rng = np.random.default_rng(3)
    q, kl, vl, tab, la, starts, kc, vc = make_case(rng, [40, 9], [40, 9], 8, 4, 16)
    got = oracle.prefill(q, kc, vc, tab, la, starts, np.float32(0.5), 4)
    for s, t0 in enumerate(starts[:-1]):
        for h in range(8):
            assert np.array_equal(got[t0, h], vl[s][0, h // 2].astype(np.float64))


def test_permuted_placement_bit_identical():
    rng = np.random.default_rng(21)
    lens, nqs = [70, 33], [30, 33]
    q, kl, vl, tab, la, starts, kc, vc = make_case(rng, lens, nqs, 8, 2, 16)
    base = oracle.prefill(q, kc, vc, tab, la, starts, np.float32(0.3), 2)
    NB = kc.shape[0]
    perm = rng.permutation(NB)          # old block b moves to perm[b]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    tab2 = np.where(tab >= 0, perm[np.maximum(tab, 0)], -1).astype(np.int32)
    moved = oracle.prefill(q, kc2, vc2, tab2, la, starts, np.float32(0.3), 2)
    assert np.array_equal(base, moved)


def test_flop_count_closed_form():
    lens, starts = [10, 7, 300], [0, 4, 4, 104]
    brute = 0
    for s in range(3):
        n, nq = lens[s], starts[s + 1] - starts[s]
        for i in range(nq):
            brute += (n - nq + i + 1) * 2 * 64 * 2 * 8     # q.K and p.V, 8 heads, D 64
    assert oracle.prefill_flops(lens, starts, 8, 64) == brute


# ---------------------------------------------------------------------------
# planted mistakes: each must make one of the pins above fail
# ---------------------------------------------------------------------------

def _brute_error():
    rng = np.random.default_rng(77)
    lens, nqs = [30, 21], [12, 21]
    q, kl, vl, tab, la, starts, kc, vc = make_case(rng, lens, nqs, 8, 2, 8)
    try:
        got = oracle.prefill(q, kc, vc, tab, la, starts, np.float32(0.4), 2)
    except Exception:
        return np.inf
    ref = brute_force_causal(q, starts, la, kl, vl, np.float32(0.4), 2)
    err = np.abs(got - ref)
    return np.inf if not np.isfinite(err).all() else float(err.max())


def test_pins_catch_planted_mistakes(monkeypatch):
    assert _brute_error() < 1e-12
    mutants = [
        # the chunk counted from position 0 instead of ending the context
        ("query_position", lambda n, nq, i: i),
        # one position too far (sees the next token)
        ("query_position", lambda n, nq, i: min(n - nq + i + 1, n - 1)),
        # not causal: every row sees the whole context
        ("query_position", lambda n, nq, i: n - 1),
    ]
    for name, fn in mutants:
        orig = getattr(cp, name)
        monkeypatch.setattr(cp, name, fn)
        assert _brute_error() > 1e-6, name
        monkeypatch.setattr(cp, name, orig)

    orig_att = pa_oracle.attention_one_query

    def no_scale(qv, kc, vc, scale):
        return orig_att(qv, kc, vc, 1.0)
    monkeypatch.setattr(pa_oracle, "attention_one_query", no_scale)
    assert _brute_error() > 1e-6
    monkeypatch.setattr(pa_oracle, "attention_one_query", orig_att)
