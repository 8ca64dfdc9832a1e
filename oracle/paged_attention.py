"""Plain CPU oracle for paged decode attention, the KV-cache append and the
block copy-on-write copy.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP library (no kernels, headers, helpers or constants); the one module both
sides consume is the seeded input generator, which holds none of the method's
arithmetic.

Everything here is deliberately slow and literal: NumPy, float64 for every
floating-point step, one sequence and one head at a time, no blocking, fusion
or reordering beyond the definitions it follows.

Sources (web pages; sections named by their headings):

* "PagedAttention and Continuous Batching Explained (2026)" (aquanode.io),
  sections "PagedAttention: a block table for the KV cache" and "FAQ": each
  request's KV cache is cut into fixed blocks of 16 tokens; a per-request
  block table maps logical block j to a physical block that may sit anywhere;
  the attention result is the ordinary attention, unchanged by where the
  blocks live.  Section "Why the KV cache is the problem": the cache holds one
  key and one value vector per layer per token; bytes per token equals
  2 x layers x KV heads x head dim x bytes per value.  Section "TL;DR": the
  cache grows by one entry per token per request.
* "KV Cache in Serving Engines: PagedAttention, Continuous Batching, and
  Prefix Caching" (ttlab), section 2 "Blocks and Block Tables": a new block is
  taken only when the current one is full, so only the last block of a request
  is partly empty; the kernel reads K and V through the table and the
  computation is the same as over a contiguous array.  Section 2 "Sharing
  Blocks": blocks are shared with reference counts and copied block-wise
  (copy-on-write) when one holder must append.
* "Continuous batching and paged attention" (abhi-g.dev), section "Paged
  attention": keys and values are gathered through the block table instead of
  from one contiguous buffer.

What the pages leave open is fixed by these readings (each is listed, with
its reason, in the design notes of the repository):

* Cache layout (the pages only say "blocks").  Separate K and V pools, fp16:
    K: [num_blocks][num_kv_heads][head_dim/8][16][8]
       element (block b, head h, slot offset o, dim d) at
       k[b, h, d // 8, o, d % 8]
    V: [num_blocks][num_kv_heads][2][head_dim][8]
       element (b, h, o, d) at v[b, h, o // 8, d, o % 8]
  A slot index is ``physical_block * 16 + offset``; negative means "skip".
* Grouped-query heads: query head ``h`` reads KV head ``h // G`` with
  ``G = num_q_heads // num_kv_heads``.
* ``context_lens[s]`` counts every token of sequence ``s`` including the one
  appended in the same step; a length of 0 gives an all-zero output row.
* The softmax scale is a caller-supplied float32; it is promoted exactly to
  float64 here.
* Output: float64, not rounded (the GPU rounds to fp16; tolerances absorb it).
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16     # tokens per block ("PagedAttention: a block table ..." / ttlab section 2)
CHUNK = 8           # fp16 elements per 16-byte chunk in the K layout / per half-block in V


# ---------------------------------------------------------------------------
# Layout: views of the pools as logical [num_blocks, num_kv_heads, BS, D]
# (BS = block size: 16 by default, 8 and 32 as the variants the pages name as
# the one tunable of the kernel: "FAQ", "What block size should I use?")
# ---------------------------------------------------------------------------

def _k5(k_cache: np.ndarray, num_kv_heads: int, head_dim: int, block_size=BLOCK_SIZE):
    """The K pool as its 5-d ABI shape [NB, Hkv, D/8, BS, 8] (a view)."""
    nb = k_cache.size // (num_kv_heads * head_dim * block_size)
    return k_cache.reshape(nb, num_kv_heads, head_dim // CHUNK, block_size, CHUNK)


def _v5(v_cache: np.ndarray, num_kv_heads: int, head_dim: int, block_size=BLOCK_SIZE):
    """The V pool as its 5-d ABI shape [NB, Hkv, BS/8, D, 8] (a view)."""
    nb = v_cache.size // (num_kv_heads * head_dim * block_size)
    return v_cache.reshape(nb, num_kv_heads, block_size // CHUNK, head_dim, CHUNK)


def logical_k_blocks(k_cache, phys, num_kv_heads, head_dim, block_size=BLOCK_SIZE):
    """K of the listed physical blocks as [len(phys), Hkv, BS, D] (a copy).

    Element (b, h, o, d) is read from k[b, h, d // 8, o, d % 8].
    """
    k5 = _k5(k_cache, num_kv_heads, head_dim, block_size)[np.asarray(phys, dtype=np.int64)]
    # [n, Hkv, D/8, BS, 8] -> [n, Hkv, BS, D/8, 8] -> [n, Hkv, BS, D]
    return k5.transpose(0, 1, 3, 2, 4).reshape(len(phys), num_kv_heads, block_size, head_dim)


def logical_v_blocks(v_cache, phys, num_kv_heads, head_dim, block_size=BLOCK_SIZE):
    """V of the listed physical blocks as [len(phys), Hkv, BS, D] (a copy).

    Element (b, h, o, d) is read from v[b, h, o // 8, d, o % 8].
    """
    v5 = _v5(v_cache, num_kv_heads, head_dim, block_size)[np.asarray(phys, dtype=np.int64)]
    # [n, Hkv, BS/8, D, 8] -> [n, Hkv, BS/8, 8, D] -> [n, Hkv, BS, D]
    return v5.transpose(0, 1, 2, 4, 3).reshape(len(phys), num_kv_heads, block_size, head_dim)


# ---------------------------------------------------------------------------
# O1: append the new tokens' K/V into their slots
# ---------------------------------------------------------------------------

def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, block_size=BLOCK_SIZE):
    """Write token t's K and V rows into slot ``slot_mapping[t]``.

    The cache grows by one entry per token ("TL;DR"); the entry lands in
    physical block ``slot // BS`` at offset ``slot % BS`` (block table
    semantics, "PagedAttention: a block table for the KV cache").  Negative
    slots are padding and are skipped.  The write is a bit copy.

    k, v: fp16 [T, Hkv, D].  Returns new (k_cache, v_cache); inputs untouched.
    """
    k = np.asarray(k)
    v = np.asarray(v)
    T, Hkv, D = k.shape
    slots = np.asarray(slot_mapping, dtype=np.int64).reshape(-1)
    assert slots.shape[0] == T and v.shape == k.shape
    live = slots[slots >= 0]
    assert np.unique(live).size == live.size, "two tokens share one slot"
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    k5 = _k5(kc, Hkv, D, block_size)
    v5 = _v5(vc, Hkv, D, block_size)
    nb = k5.shape[0]
    for t in range(T):
        s = int(slots[t])
        if s < 0:
            continue
        b, o = divmod(s, block_size)
        assert 0 <= b < nb, "slot outside the pool"
        # K: k[b, h, d // 8, o, d % 8] = k_new[t, h, d]
        k5[b, :, :, o, :] = k[t].reshape(Hkv, D // CHUNK, CHUNK)
        # V: v[b, h, o // 8, d, o % 8] = v_new[t, h, d]
        v5[b, :, o // CHUNK, :, o % CHUNK] = v[t]
    return kc, vc


# ---------------------------------------------------------------------------
# O2: copy-on-write block copy
# ---------------------------------------------------------------------------

def copy_blocks(k_cache, v_cache, block_mapping, num_kv_heads, head_dim, block_size=BLOCK_SIZE):
    """For each (src, dst) pair copy the whole block, K and V, all KV heads.

    Copy-on-write at block granularity when a shared block must take an append
    (ttlab section 2 "Sharing Blocks"; aquanode "PagedAttention: a block table
    for the KV cache", sharing bullet).  A pair with src == dst is a no-op.
    dsts must be distinct and must not also be a src of another pair.
    Returns new (k_cache, v_cache).
    """
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    k5 = _k5(kc, num_kv_heads, head_dim, block_size)
    v5 = _v5(vc, num_kv_heads, head_dim, block_size)
    nb = k5.shape[0]
    if pairs.shape[0] == 0:
        return kc, vc
    src, dst = pairs[:, 0], pairs[:, 1]
    assert ((src >= 0) & (src < nb) & (dst >= 0) & (dst < nb)).all(), "block id outside the pool"
    moving = src != dst
    assert np.unique(dst[moving]).size == int(moving.sum()), "two pairs write one block"
    assert not np.isin(dst[moving], src).any(), "a destination is also a source"
    snap_k = k5[src[moving]].copy()
    snap_v = v5[src[moving]].copy()
    k5[dst[moving]] = snap_k
    v5[dst[moving]] = snap_v
    return kc, vc


# ---------------------------------------------------------------------------
# O3: decode attention through the block table
# ---------------------------------------------------------------------------

def gather_sequence(k_cache, v_cache, table_row, n, num_kv_heads, head_dim, block_size=BLOCK_SIZE):
    """Rebuild one sequence's contiguous K and V, each [Hkv, n, D] float64.

    Logical block j lives in physical block ``table_row[j]``; only the first
    ceil(n / 16) entries are read and only the first n positions kept, so the
    unused tail of the last block never enters (ttlab section 2 "Blocks and
    Block Tables": only the last block is partly filled).
    """
    nb = -(-n // block_size)
    phys = np.asarray(table_row[:nb], dtype=np.int64)
    kb = logical_k_blocks(k_cache, phys, num_kv_heads, head_dim, block_size)   # [nb, Hkv, BS, D]
    vb = logical_v_blocks(v_cache, phys, num_kv_heads, head_dim, block_size)
    kc = kb.transpose(1, 0, 2, 3).reshape(num_kv_heads, nb * block_size, head_dim)[:, :n]
    vc = vb.transpose(1, 0, 2, 3).reshape(num_kv_heads, nb * block_size, head_dim)[:, :n]
    return kc.astype(np.float64), vc.astype(np.float64)


def attention_one_query(qv, kc, vc, scale):
    """softmax(scale * K q) V for one query vector, float64.

    qv: [D]; kc, vc: [n, D].  The maximum is subtracted before exp, which does
    not change the exact value.
    """
    z = (kc @ qv) * scale
    p = np.exp(z - z.max())
    return (p @ vc) / p.sum()


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads,
           block_size=BLOCK_SIZE):
    """One decode step of attention for every sequence, float64 [S, Hq, D].

    Same attention as over contiguous K/V ("FAQ": it is not a different
    attention algorithm; ttlab section 2: the computation stays the same):
    for sequence s and query head h with KV head kh = h // G,
        out[s, h] = softmax(scale * K_s[kh] q[s, h]) V_s[kh]
    over the first context_lens[s] positions, K_s and V_s read through
    block_tables[s].
    """
    q = np.asarray(q)
    S, Hq, D = q.shape
    assert Hq % num_kv_heads == 0
    G = Hq // num_kv_heads
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens).reshape(-1)
    scale64 = np.float64(np.float32(scale))
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in range(S):
        n = int(lens[s])
        if n <= 0:
            continue
        assert n <= tables.shape[1] * block_size, "context longer than its block table"
        kc, vc = gather_sequence(k_cache, v_cache, tables[s], n, num_kv_heads, D, block_size)
        for h in range(Hq):
            kh = h // G
            out[s, h] = attention_one_query(q[s, h].astype(np.float64), kc[kh], vc[kh], scale64)
    return out


def decode_step(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                slot_mapping, block_mapping, scale, num_kv_heads, block_size=BLOCK_SIZE):
    """One whole decode step in order: copy-on-write, append, attention.

    The order follows the pages: a shared block is copied before the holder
    appends to it (ttlab section 2 "Sharing Blocks"), and attention then reads
    the cache that includes the new token.  Returns (out, k_cache, v_cache).
    """
    D = q.shape[2]
    kc, vc = copy_blocks(k_cache, v_cache, block_mapping, num_kv_heads, D, block_size)
    kc, vc = reshape_and_cache(k_new, v_new, kc, vc, slot_mapping, block_size)
    out = decode(q, kc, vc, block_tables, context_lens, scale, num_kv_heads, block_size)
    return out, kc, vc


def swap_blocks(src_k, src_v, dst_k, dst_v, block_mapping, num_kv_heads, head_dim,
                block_size=BLOCK_SIZE):
    """Copy whole blocks, K and V, between two pools of the same layout:
    block src of the source pool to block dst of the destination pool.  The
    pool that a request was preempted to (host memory) and the device pool
    ("Continuous batching and paged attention", section "Why they depend on
    each other": preemption by recomputation or by swap to host memory).
    Pairs with an id outside its pool are skipped.  Returns new (dst_k, dst_v)."""
    pairs = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    dk = np.array(dst_k, copy=True)
    dv = np.array(dst_v, copy=True)
    sk5 = _k5(np.asarray(src_k), num_kv_heads, head_dim, block_size)
    sv5 = _v5(np.asarray(src_v), num_kv_heads, head_dim, block_size)
    dk5 = _k5(dk, num_kv_heads, head_dim, block_size)
    dv5 = _v5(dv, num_kv_heads, head_dim, block_size)
    for src, dst in pairs:
        if 0 <= src < sk5.shape[0] and 0 <= dst < dk5.shape[0]:
            dk5[dst] = sk5[src]
            dv5[dst] = sv5[src]
    return dk, dv


# ---------------------------------------------------------------------------
# Closed form printed on the pages
# ---------------------------------------------------------------------------

def kv_bytes_per_token(layers, kv_heads, head_dim, bytes_per_value):
    """2 (K and V) x layers x KV heads x head dim x bytes per value.

    "Why the KV cache is the problem" (aquanode).
    """
    return 2 * layers * kv_heads * head_dim * bytes_per_value
