"""Seeded synthetic decode-step inputs and the block manager that lays them out.

This module builds inputs only.  It holds none of the attention, append or
copy arithmetic: the HIP library computes those on the GPU and the CPU
oracle recomputes them independently; both receive the arrays made here.

What it models (web pages, sections named by their headings):

* "PagedAttention and Continuous Batching Explained (2026)" (aquanode.io),
  "PagedAttention: a block table for the KV cache": a sequence's cache is a
  list of 16-token blocks taken one at a time from a free pool as it grows;
  a per-request table maps logical block j to its physical block; freeing a
  request returns whole blocks that others take at once.
* "KV Cache in Serving Engines ..." (ttlab), section 2 "Blocks and Block
  Tables" / "Sharing Blocks": a block is taken only when the previous one is
  full; shared blocks carry reference counts and are copied (copy-on-write)
  when a holder must append into one.
* "Continuous batching, paged attention, prefix caching" (backplane.click),
  "Static versus continuous batching": a finished request's blocks go back to
  the pool and a newcomer takes them, still holding the old owner's bytes.

Input recipe (every draw comes from ``numpy.random.default_rng(seed)`` in the
order listed):
  1. context lengths, integer-uniform and inclusive: ``rng.integers(lo, hi+1)``
     (fixed lists where a workload names them);
  2. physical placement: ``rng.permutation(num_blocks)`` is the free list,
     blocks are taken from its front in logical order;
  3. K pool then V pool, every element ``standard_normal(float32)`` rounded to
     fp16, drawn in memory order in chunks of 2**22 elements;
  4. q [S, Hq, D], then the appended tokens' k and v [S, Hkv, D], same law.
Then, without further draws: blocks no table references and fresh
copy-on-write destinations are filled with NaN; slots at or past each
sequence's append position in its last block hold canaries (NaN, +65504,
-65504, cycling with the offset) or, in "stale" mode, keep their random bytes
as if left by a previous owner.
"""
from __future__ import annotations

import math
from collections import deque
from dataclasses import dataclass, field

import numpy as np

BLOCK_SIZE = 16
CHUNK = 8
FP16_NAN = np.uint16(0x7E00)
FP16_MAX = np.uint16(0x7BFF)     # +65504
FP16_MIN = np.uint16(0xFBFF)     # -65504
_CANARIES = (FP16_NAN, FP16_MAX, FP16_MIN)
_DRAW_CHUNK = 1 << 22


class PoolExhausted(RuntimeError):
    """The free list is empty: a serving engine would preempt here."""


# ---------------------------------------------------------------------------
# Block manager (harness): free list, tables, reference counts, copy-on-write
# ---------------------------------------------------------------------------

class BlockManager:
    """Per-sequence block tables over a pool of ``num_blocks`` physical blocks.

    ``free_order`` is the order in which free blocks are handed out (a seeded
    permutation scatters a sequence's blocks across the pool).  Freed blocks
    go to the back of the free list.
    """

    def __init__(self, num_blocks: int, free_order=None, block_size: int = BLOCK_SIZE):
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        order = range(num_blocks) if free_order is None else [int(b) for b in free_order]
        self.free = deque(order)
        self.refcount = np.zeros(num_blocks, dtype=np.int64)
        self.tables: dict = {}
        self.lens: dict = {}

    # -- queries -----------------------------------------------------------
    def blocks_for(self, n_tokens: int) -> int:
        """Blocks a sequence of n tokens occupies (the last may be partial)."""
        return -(-int(n_tokens) // self.block_size)

    def num_free(self) -> int:
        return len(self.free)

    def slot(self, seq, pos: int) -> int:
        """Slot index of logical position ``pos``: physical block * BS + offset."""
        j, off = divmod(int(pos), self.block_size)
        return self.tables[seq][j] * self.block_size + off

    # -- mutation ----------------------------------------------------------
    def _take(self) -> int:
        if not self.free:
            raise PoolExhausted("no free block left")
        b = self.free.popleft()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def allocate(self, seq, n_tokens: int) -> list:
        """Start sequence ``seq`` with ``n_tokens`` tokens (its prompt)."""
        assert seq not in self.tables
        need = self.blocks_for(n_tokens)
        if need > len(self.free):
            raise PoolExhausted(f"need {need} blocks, {len(self.free)} free")
        self.tables[seq] = [self._take() for _ in range(need)]
        self.lens[seq] = int(n_tokens)
        return list(self.tables[seq])

    def fork(self, parent, child) -> None:
        """``child`` shares every block of ``parent`` (reference counts grow)."""
        assert child not in self.tables
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.refcount[b] += 1

    def append_token(self, seq):
        """Reserve the slot of the next token of ``seq``.

        Returns ``(slot, cow)`` where ``cow`` is ``(src, dst)`` when the last
        block was shared and had to be copied first, else ``None``.  A fresh
        block is taken when the last one is full.
        """
        pos = self.lens[seq]
        table = self.tables[seq]
        cow = None
        if pos % self.block_size == 0:
            table.append(self._take())
        else:
            last = table[-1]
            if self.refcount[last] > 1:
                dst = self._take()
                self.refcount[last] -= 1
                table[-1] = dst
                cow = (last, dst)
        self.lens[seq] = pos + 1
        return self.slot(seq, pos), cow

    def free_seq(self, seq) -> None:
        """Drop ``seq``; blocks whose count reaches zero return to the pool."""
        for b in self.tables.pop(seq):
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.lens[seq]

    def table_array(self, seqs, max_blocks: int) -> np.ndarray:
        """int32 [len(seqs), max_blocks]; unused entries are -1."""
        out = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            row = self.tables[s]
            assert len(row) <= max_blocks
            out[i, :len(row)] = row
        return out


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: np.float32
    q: np.ndarray               # fp16 [S, Hq, D]
    k_cache: np.ndarray         # fp16 [NB, Hkv, D/8, BS, 8]
    v_cache: np.ndarray         # fp16 [NB, Hkv, BS/8, D, 8]
    block_tables: np.ndarray    # int32 [S, MB], -1 past the last block
    context_lens: np.ndarray    # int32 [S], includes the appended token
    k_new: np.ndarray           # fp16 [S, Hkv, D]
    v_new: np.ndarray           # fp16 [S, Hkv, D]
    slot_mapping: np.ndarray    # int64 [S]
    block_mapping: np.ndarray   # int64 [P, 2] (src, dst)
    meta: dict = field(default_factory=dict)
    block_size: int = BLOCK_SIZE

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def kv_bytes_per_token_layer(self) -> int:
        """K and V bytes one token occupies in one layer at fp16."""
        return 2 * self.num_kv_heads * self.head_dim * 2

    def decode_bytes(self) -> int:
        """Logical bytes of the decode step: every sequence's valid K/V
        positions (a block shared by several sequences counts once per
        holder), q and out, the table entries it reads, the lengths.

        Unused tail slots of last blocks and split-context partials are not
        counted.  ``unique_decode_bytes`` counts shared blocks once.
        """
        lens = self.context_lens.astype(np.int64)
        kv = int(lens.sum()) * self.kv_bytes_per_token_layer()
        return kv + self._decode_side_bytes()

    def _decode_side_bytes(self) -> int:
        """q and out, table entries, lengths."""
        lens = self.context_lens.astype(np.int64)
        qo = 2 * self.num_seqs * self.num_q_heads * self.head_dim * 2
        table = int((-(-lens // self.block_size)).sum()) * 4
        return qo + table + 4 * self.num_seqs

    def unique_kv_bytes(self) -> int:
        """Valid K/V bytes with each physical block counted once, at the
        largest number of its positions any holder reads."""
        fill = {}
        for s in range(self.num_seqs):
            n = int(self.context_lens[s])
            for pos in range(0, n, self.block_size):
                b = int(self.block_tables[s, pos // self.block_size])
                fill[b] = max(fill.get(b, 0), min(self.block_size, n - pos))
        return sum(fill.values()) * self.kv_bytes_per_token_layer()

    def unique_decode_bytes(self) -> int:
        """Bytes the decode step must move when shared blocks are read once:
        unique K/V plus q and out, table entries, lengths.  Equal to
        ``decode_bytes`` for batches that share no block."""
        return self.unique_kv_bytes() + self._decode_side_bytes()

    def shares_blocks(self) -> bool:
        """Some physical block appears in more than one table row."""
        used = [self.block_tables[s, :-(-int(n) // self.block_size)]
                for s, n in enumerate(self.context_lens) if n > 0]
        if not used:
            return False
        used = np.concatenate(used)
        return np.unique(used).size < used.size

    def append_bytes(self) -> int:
        """Bytes the append moves: read k, v rows and write them into the pool."""
        live = int((self.slot_mapping >= 0).sum())
        return 2 * live * self.kv_bytes_per_token_layer()

    def copy_bytes(self) -> int:
        """Bytes the copy-on-write moves: read and write whole blocks, K and V."""
        moving = int((self.block_mapping[:, 0] != self.block_mapping[:, 1]).sum()) \
            if self.block_mapping.size else 0
        return 2 * moving * self.block_size * self.kv_bytes_per_token_layer()


def _fill_normal_fp16(rng, out: np.ndarray) -> None:
    flat = out.reshape(-1)
    for start in range(0, flat.size, _DRAW_CHUNK):
        n = min(_DRAW_CHUNK, flat.size - start)
        flat[start:start + n] = rng.standard_normal(n, dtype=np.float32).astype(np.float16)


def _set_slot_bits(k_u16, v_u16, block: int, offset: int, bits) -> None:
    """Every element of one slot (all heads, all dims) of K and V to ``bits``."""
    k_u16[block, :, :, offset, :] = bits
    v_u16[block, :, offset // CHUNK, :, offset % CHUNK] = bits


def make_workload(name, seed, num_q_heads, num_kv_heads, head_dim, context_lens=None,
                  len_range=None, num_seqs=None, max_context_bound=None, pool_factor=1.25,
                  num_blocks=None, prefix_groups=0, prefix_len=0, suffix_range=None,
                  tail="canary", scale=None, placement="shuffled",
                  block_size=BLOCK_SIZE) -> Workload:
    """Build one decode step: pools, tables, lengths, q, new k/v, slots, CoW pairs.

    ``context_lens`` (or ``len_range`` + ``num_seqs``) give each sequence's
    length after this step's append.  With ``prefix_groups`` > 0 the batch is
    that many groups of sequences sharing ``prefix_len`` prompt tokens
    (a multiple of 16) followed by private suffixes drawn from
    ``suffix_range``; the block holding each sequence's append position is
    shared with a forked sibling, so the append first copies it
    (copy-on-write).  ``tail`` is "canary" or "stale".  ``placement`` is
    "shuffled" (free list = a seeded permutation of the pool) or "sequential"
    (free list in pool order: each sequence's blocks end up contiguous).
    """
    assert num_q_heads % num_kv_heads == 0 and head_dim % CHUNK == 0
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    BS = int(block_size)
    assert BS % CHUNK == 0

    # 1. lengths
    if prefix_groups:
        assert prefix_len % BS == 0 and num_seqs % prefix_groups == 0
        lo, hi = suffix_range
        suffix = rng.integers(lo, hi + 1, size=num_seqs)
        lens = (prefix_len + suffix).astype(np.int64)
        bound = prefix_len + hi
    elif context_lens is not None:
        lens = np.asarray(context_lens, dtype=np.int64)
        bound = int(lens.max()) if lens.size else 0
    else:
        lo, hi = len_range
        lens = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int64)
        bound = hi
    S = lens.size
    if max_context_bound is not None:
        bound = max(bound, max_context_bound)
    MB = max(1, -(-bound // BS))

    # pool size
    if num_blocks is None:
        if prefix_groups:
            shared = prefix_groups * (prefix_len // BS)
            private = int(sum(-(-int(n) // BS) - prefix_len // BS for n in lens))
            needed = shared + private + S            # + one copy-on-write spare each
        else:
            needed = int(sum(-(-int(n) // BS) for n in lens))
        num_blocks = max(1, math.ceil(pool_factor * needed))
    NB = int(num_blocks)

    # 2. placement (the permutation is drawn in both modes, to keep the stream)
    perm = rng.permutation(NB)
    bm = BlockManager(NB, free_order=perm if placement == "shuffled" else None, block_size=BS)
    slots = np.full(S, -1, dtype=np.int64)
    cows = []
    shadows = []
    if prefix_groups:
        per = S // prefix_groups
        for g in range(prefix_groups):
            bm.allocate(("prompt", g), prefix_len)
            for i in range(per):
                s = g * per + i
                bm.fork(("prompt", g), s)
                for _ in range(int(lens[s]) - 1 - prefix_len):
                    bm.append_token(s)
            bm.free_seq(("prompt", g))
        for s in range(S):
            # a forked sibling keeps the pre-append blocks
            bm.fork(s, ("sibling", s))
            shadows.append(("sibling", s))
    else:
        for s in range(S):
            if lens[s] > 0:
                bm.allocate(s, int(lens[s]) - 1)
            else:
                bm.tables[s] = []
                bm.lens[s] = 0
    pre_tables = {s: list(bm.tables[s]) for s in range(S)}
    for s in range(S):
        if lens[s] > 0:
            slot, cow = bm.append_token(s)
            slots[s] = slot
            if cow is not None:
                cows.append(cow)
    tables = bm.table_array(range(S), MB)

    # 3. pools
    k_cache = np.empty((NB, Hkv, D // CHUNK, BS, CHUNK), dtype=np.float16)
    v_cache = np.empty((NB, Hkv, BS // CHUNK, D, CHUNK), dtype=np.float16)
    _fill_normal_fp16(rng, k_cache)
    _fill_normal_fp16(rng, v_cache)
    # 4. queries and the appended tokens
    q = np.empty((S, Hq, D), dtype=np.float16)
    _fill_normal_fp16(rng, q)
    k_new = np.empty((S, Hkv, D), dtype=np.float16)
    v_new = np.empty((S, Hkv, D), dtype=np.float16)
    _fill_normal_fp16(rng, k_new)
    _fill_normal_fp16(rng, v_new)

    # canaries (no draws)
    ku = k_cache.view(np.uint16)
    vu = v_cache.view(np.uint16)
    referenced = np.zeros(NB, dtype=bool)
    for s in range(S):
        referenced[pre_tables[s]] = True
        referenced[bm.tables[s]] = True
    for sh in shadows:
        referenced[bm.tables[sh]] = True
    ku[~referenced] = FP16_NAN
    vu[~referenced] = FP16_NAN
    for _, dst in cows:
        ku[dst] = FP16_NAN
        vu[dst] = FP16_NAN
    for s in range(S):
        n = int(lens[s])
        if n == 0:
            continue
        pos = n - 1                       # the append position
        j, off = divmod(pos, BS)
        # the block that holds the append position before any copy
        blk = pre_tables[s][j] if j < len(pre_tables[s]) else bm.tables[s][j]
        for o in range(off, BS):
            if tail == "stale" and o > off:
                continue
            _set_slot_bits(ku, vu, blk, o, _CANARIES[o % 3] if o > off else FP16_NAN)

    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Workload(
        name=name, seed=seed, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        num_blocks=NB, max_blocks_per_seq=MB, scale=np.float32(scale), q=q,
        k_cache=k_cache, v_cache=v_cache, block_tables=tables,
        context_lens=lens.astype(np.int32), k_new=k_new, v_new=v_new,
        slot_mapping=slots, block_mapping=np.asarray(cows, dtype=np.int64).reshape(-1, 2),
        meta={"tail": tail, "prefix_groups": prefix_groups, "prefix_len": prefix_len,
              "pool_factor": pool_factor, "placement": placement},
        block_size=BS,
    )


# Named workloads: the shapes of the decode batches this library is measured on.
WORKLOADS = {
    # 4 sequences of lengths 1, 16, 17, 50 (single token, a full block, one past
    # a block, a mid-block slot), 4 q heads = 4 KV heads, head_dim 64, 64-block pool.
    "tiny_d64": dict(seed=1, num_q_heads=4, num_kv_heads=4, head_dim=64,
                     context_lens=[1, 16, 17, 50], num_blocks=64, scale=1.0 / 8.0),
    # Llama-3.1-8B-shaped layer: batch 64, 32 q / 8 KV heads, head_dim 128,
    # lengths uniform in [128, 2048], pool 1.25x the blocks needed.
    "llama8b_b64": dict(seed=2, num_q_heads=32, num_kv_heads=8, head_dim=128,
                        len_range=(128, 2048), num_seqs=64),
    # Llama-3.1-70B-shaped layer: 64 q / 8 KV heads (a group of 8), otherwise
    # llama8b_b64 (same seed: the same lengths, the same K/V bytes).
    "llama70b_b64": dict(seed=2, num_q_heads=64, num_kv_heads=8, head_dim=128,
                         len_range=(128, 2048), num_seqs=64),
    # Llama-3.1-405B-shaped layer: 128 q / 8 KV heads (a group of 16), the
    # lengths and K/V bytes of llama8b_b64.
    "llama405b_b64": dict(seed=2, num_q_heads=128, num_kv_heads=8, head_dim=128,
                          len_range=(128, 2048), num_seqs=64),
    # 96 q / 8 KV heads (a group of 12: Mistral-Large-2-shaped), the lengths
    # and K/V bytes of llama8b_b64.
    "g12_b64": dict(seed=2, num_q_heads=96, num_kv_heads=8, head_dim=128,
                    len_range=(128, 2048), num_seqs=64),
    # a multi-query layer (32 query heads on one KV head), 512 sequences of
    # the Llama lengths: about the units and K/V bytes of llama8b_b64, with
    # two passes of 16 query heads over each unit
    "mqa_b512": dict(seed=2, num_q_heads=32, num_kv_heads=1, head_dim=128,
                     len_range=(128, 2048), num_seqs=512),
    # OPT-13B-shaped multi-head layer: batch 128, 40 heads, head_dim 128,
    # lengths uniform in [1, 2048].
    "opt13b_b128": dict(seed=3, num_q_heads=40, num_kv_heads=40, head_dim=128,
                        len_range=(1, 2048), num_seqs=128),
    # Long context: batch 16, 32 q / 8 KV heads, lengths uniform in [8192, 32768].
    "longctx_b16": dict(seed=4, num_q_heads=32, num_kv_heads=8, head_dim=128,
                        len_range=(8192, 32768), num_seqs=16),
    # Shared prefix: 32 groups of 8 sequences share a 1024-token prompt
    # (64 blocks, reference-counted), private suffixes uniform in [16, 512];
    # each append first copies its shared last block.
    "prefix_b256": dict(seed=5, num_q_heads=32, num_kv_heads=8, head_dim=128,
                        num_seqs=256, prefix_groups=32, prefix_len=1024,
                        suffix_range=(16, 512)),
}


def make_named(name: str, **overrides) -> Workload:
    kw = dict(WORKLOADS[name])
    kw.update(overrides)
    return make_workload(name, **kw)


# ---------------------------------------------------------------------------
# Multi-query (chunked prefill) inputs
# ---------------------------------------------------------------------------

@dataclass
class PrefillWorkload:
    """One step of chunked prefill: each sequence's context already holds its
    first ``context_lens - chunk_lens`` positions; this step appends the
    chunk's K/V at the next positions and its queries attend causally."""
    name: str
    seed: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: np.float32
    q: np.ndarray               # fp16 [T, Hq, D], chunks packed in sequence order
    k_cache: np.ndarray         # fp16 [NB, Hkv, D/8, BS, 8]
    v_cache: np.ndarray         # fp16 [NB, Hkv, BS/8, D, 8]
    block_tables: np.ndarray    # int32 [S, MB]
    context_lens: np.ndarray    # int32 [S], including the chunk
    query_start: np.ndarray     # int32 [S + 1]
    k_new: np.ndarray           # fp16 [T, Hkv, D], the chunk's keys
    v_new: np.ndarray           # fp16 [T, Hkv, D]
    slot_mapping: np.ndarray    # int64 [T]
    meta: dict = field(default_factory=dict)
    block_size: int = BLOCK_SIZE

    @property
    def num_tokens(self) -> int:
        return int(self.query_start[-1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(np.diff(self.query_start).max()) if self.num_seqs else 0

    def kv_bytes_per_token_layer(self) -> int:
        return 2 * self.num_kv_heads * self.head_dim * 2

    def flops(self) -> int:
        """Algorithmic flops of the step's attention: the query at position p
        meets the p + 1 keys at or before it, with 2 D flops per key for q.K
        and 2 D for the weighted sum of V, per query head."""
        lens = self.context_lens.astype(np.int64)
        nq = np.diff(self.query_start.astype(np.int64))
        keys = (lens * (lens + 1) - (lens - nq) * (lens - nq + 1)) // 2
        return int(4 * int(keys.sum()) * self.num_q_heads * self.head_dim)

def make_prefill_workload(name, seed, num_q_heads, num_kv_heads, head_dim, context_lens=None,
                          chunk_lens=None, num_seqs=None, cached_range=None, chunk=None,
                          pool_factor=1.25, scale=None, block_size=BLOCK_SIZE) -> PrefillWorkload:
    """Chunks of ``chunk_lens`` query tokens ending contexts of ``context_lens``
    (or: ``num_seqs`` sequences with ``rng.integers`` cached lengths in
    ``cached_range`` plus a fixed ``chunk``).  Draws, in order: cached lengths
    (if drawn), the pool permutation, K pool, V pool, q, the chunk's k and v.
    Blocks no table references and the chunk's own slots (until the append)
    are NaN; slots past the context in its last block hold canaries."""
    rng = np.random.default_rng(seed)
    Hq, Hkv, D = num_q_heads, num_kv_heads, head_dim
    BS = int(block_size)
    if context_lens is None:
        lo, hi = cached_range
        cached = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int64)
        nqs = np.full(num_seqs, chunk, dtype=np.int64)
        lens = cached + nqs
    else:
        lens = np.asarray(context_lens, dtype=np.int64)
        nqs = np.asarray(chunk_lens, dtype=np.int64)
    assert (nqs >= 0).all() and (nqs <= lens).all()
    S = lens.size
    MB = max(1, -(-int(lens.max()) // BS))
    needed = int(sum(-(-int(n) // BS) for n in lens))
    NB = max(1, math.ceil(pool_factor * needed))
    perm = rng.permutation(NB)
    bm = BlockManager(NB, free_order=perm, block_size=BS)
    slots = []
    for s in range(S):
        bm.allocate(s, int(lens[s] - nqs[s]))
        for _ in range(int(nqs[s])):
            slot, cow = bm.append_token(s)
            assert cow is None
            slots.append(slot)
    tables = bm.table_array(range(S), MB)
    T = int(nqs.sum())
    k_cache = np.empty((NB, Hkv, D // CHUNK, BS, CHUNK), dtype=np.float16)
    v_cache = np.empty((NB, Hkv, BS // CHUNK, D, CHUNK), dtype=np.float16)
    _fill_normal_fp16(rng, k_cache)
    _fill_normal_fp16(rng, v_cache)
    q = np.empty((T, Hq, D), dtype=np.float16)
    _fill_normal_fp16(rng, q)
    k_new = np.empty((T, Hkv, D), dtype=np.float16)
    v_new = np.empty((T, Hkv, D), dtype=np.float16)
    _fill_normal_fp16(rng, k_new)
    _fill_normal_fp16(rng, v_new)
    ku, vu = k_cache.view(np.uint16), v_cache.view(np.uint16)
    referenced = np.zeros(NB, dtype=bool)
    for s in range(S):
        referenced[bm.tables[s]] = True
    ku[~referenced] = FP16_NAN
    vu[~referenced] = FP16_NAN
    for slot in slots:
        _set_slot_bits(ku, vu, slot // BS, slot % BS, FP16_NAN)
    for s in range(S):
        n = int(lens[s])
        if n % BS:
            blk = bm.tables[s][n // BS]
            for o in range(n % BS, BS):
                _set_slot_bits(ku, vu, blk, o, _CANARIES[o % 3])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return PrefillWorkload(
        name=name, seed=seed, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        num_blocks=NB, max_blocks_per_seq=MB, scale=np.float32(scale), q=q,
        k_cache=k_cache, v_cache=v_cache, block_tables=tables,
        context_lens=lens.astype(np.int32),
        query_start=np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32),
        k_new=k_new, v_new=v_new, slot_mapping=np.asarray(slots, dtype=np.int64),
        meta={"pool_factor": pool_factor}, block_size=BS)


PREFILL_WORKLOADS = {
    # tiny: chunks that start a sequence, a single token, one crossing a block
    # boundary, one shorter than its context
    "prefill_tiny": dict(seed=11, num_q_heads=4, num_kv_heads=4, head_dim=64,
                         context_lens=[5, 16, 40, 100], chunk_lens=[5, 1, 17, 64], scale=1.0 / 8.0),
    # chunked prefill on the Llama-3.1-8B layer shape: 16 sequences each adding
    # a 512-token chunk (one of the chunk sizes the ttlab page measures) to a
    # cached context uniform in [0, 3584] tokens
    "chunked_prefill_llama": dict(seed=12, num_q_heads=32, num_kv_heads=8, head_dim=128,
                                  num_seqs=16, cached_range=(0, 3584), chunk=512),
    # prefix-cache hit continuation (aquanode "Prefix caching" example): a
    # 2,100-token prompt with 2,000 tokens cached leaves a 100-token chunk;
    # 32 such sequences on the Llama-3.1-8B layer shape
    "prefix_hit_llama": dict(seed=13, num_q_heads=32, num_kv_heads=8, head_dim=128,
                             context_lens=[2100] * 32, chunk_lens=[100] * 32),
}


def make_named_prefill(name: str, **overrides) -> PrefillWorkload:
    kw = dict(PREFILL_WORKLOADS[name])
    kw.update(overrides)
    return make_prefill_workload(name, **kw)
