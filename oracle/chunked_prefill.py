"""Plain CPU oracle for multi-query paged attention: a chunk of new query
tokens per sequence attending to its paged context (chunked prefill and the
continuation after a prefix-cache hit).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it, and it shares no code with the HIP library.

Sources (web pages; sections named by their headings):

* "KV Cache in Serving Engines: PagedAttention, Continuous Batching, and
  Prefix Caching" (ttlab), section 3 "New Problem: Long Prefills Pause
  Decoding": a long prompt's prefill is cut into chunks that run over several
  steps, interleaved with decoding.  Section 4 "Prefix Caching": blocks found
  in the cache are reused and their prefill is skipped.
* "PagedAttention and Continuous Batching Explained (2026)" (aquanode.io),
  section "Prefix caching": on a hit only the tokens after the cached full
  blocks are prefilled (2,100-token prompt, 2,000 cached: about 100 left).
* The same pages, "FAQ" and section 2 "Blocks and Block Tables": the
  attention is the ordinary one, computed as over a contiguous array.

Reading (the pages do not spell out the mask): a chunk holds the LAST n_q of
the sequence's context_lens[s] positions, its K/V already in the cache, and
the query at position p attends to positions 0..p, as every token does in
the model's own (causal) attention.  A decode step is the case n_q = 1.
"""
from __future__ import annotations

import numpy as np

from . import paged_attention as _pa
from .paged_attention import BLOCK_SIZE


def query_position(n, nq, i):
    """Position of row i of a chunk of nq queries that ends a context of n
    tokens: the chunk is the last nq positions, n - nq .. n - 1."""
    return n - nq + i


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, num_kv_heads,
            block_size=BLOCK_SIZE):
    """Causal attention of each sequence's query chunk, float64 [T, Hq, D].

    q: fp16 [T, Hq, D], the chunks of all sequences packed: rows
    query_start[s] .. query_start[s+1]-1 belong to sequence s.  With
    n = context_lens[s] and n_q its chunk length, row i of the chunk sits at
    position p = n - n_q + i and, for query head h and KV head kh = h // G,
        out[row, h] = softmax(scale * K_s[kh][:p+1] q[row, h]) V_s[kh][:p+1].
    """
    q = np.asarray(q)
    T, Hq, D = q.shape
    assert Hq % num_kv_heads == 0
    G = Hq // num_kv_heads
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens).reshape(-1)
    starts = np.asarray(query_start).reshape(-1)
    S = lens.shape[0]
    assert starts.shape[0] == S + 1 and starts[0] == 0 and starts[-1] == T
    scale64 = np.float64(np.float32(scale))
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in range(S):
        n, t0, t1 = int(lens[s]), int(starts[s]), int(starts[s + 1])
        nq = t1 - t0
        assert 0 <= nq <= n, "a chunk is at most the sequence's context"
        if nq == 0:
            continue
        assert n <= tables.shape[1] * block_size, "context longer than its block table"
        kc, vc = _pa.gather_sequence(k_cache, v_cache, tables[s], n, num_kv_heads, D, block_size)
        for i in range(nq):
            p = query_position(n, nq, i)
            for h in range(Hq):
                kh = h // G
                out[t0 + i, h] = _pa.attention_one_query(q[t0 + i, h].astype(np.float64),
                                                         kc[kh, :p + 1], vc[kh, :p + 1], scale64)
    return out


def prefill_flops(context_lens, query_start, num_q_heads, head_dim):
    """Multiply-adds x 2 of the two products: the query at position p meets
    p + 1 keys, 2 * D flops each for q.K and again for p.V."""
    lens = np.asarray(context_lens, dtype=np.int64).reshape(-1)
    starts = np.asarray(query_start, dtype=np.int64).reshape(-1)
    total = 0
    for s in range(lens.shape[0]):
        n, nq = int(lens[s]), int(starts[s + 1] - starts[s])
        # sum over p = n-nq .. n-1 of (p + 1)
        total += (n * (n + 1) - (n - nq) * (n - nq + 1)) // 2
    return 4 * total * num_q_heads * head_dim
