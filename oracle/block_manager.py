"""Plain Python model of a paged KV-cache block manager with prefix caching.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use
it; it shares no code with the library's C++ block manager.

Sources (web pages; sections named by their headings):

* "PagedAttention and Continuous Batching Explained (2026)" (aquanode.io),
  "PagedAttention: a block table for the KV cache": fixed blocks of 16
  tokens, a per-request block table, blocks taken one at a time as a
  sequence grows, shared blocks copied (copy-on-write) when they diverge,
  freed blocks taken by anyone at once.  "Prefix caching": each full block
  is hashed from its parent block's hash, its own tokens and extra keys
  (LoRA id, multimodal inputs, a cache salt); a new request looks its
  blocks up by hash and reuses the ones that exist; unreferenced blocks are
  evicted least-recently-used; only full blocks are cached; sha256 is the
  default hash.
* "KV Cache in Serving Engines" (ttlab), section 2 "Blocks and Block Tables"
  and "Sharing Blocks" (reference counts; copy when a holder appends);
  section 4 "Prefix Caching": key = Hash(previous block's key, this block's
  token ids, additional info); only full blocks are cached; a finished
  request's blocks are not deleted but queued with their contents, the
  oldest evicted first, and the blocks of a finished request enter the
  queue from its back so that its tail, less likely to be reused, is
  evicted first.
* "Continuous batching, paged attention, prefix caching" (backplane.click),
  "Prefix caching": sharing ends at the first differing token; blocks are
  reference counted and evicted least-recently-used.

Readings where the pages leave a step open:

* The key of the first block chains from 32 zero bytes.  The hashed bytes
  are the parent key, then the block's token ids as little-endian int32,
  then the request's extra bytes.  The non-cryptographic choice is 64-bit
  FNV-1a over the same bytes, written little-endian into the first 8 bytes
  of a 32-byte key (the rest zero).
* The free queue starts in the pool's order (or a given order).  Taking a
  block pops the queue's front and drops the block's cached key, if any.
  A cache hit on a queued block takes it out of the queue.
* Admitting a prompt: its leading full blocks are looked up in order and
  reused while they hit; the first miss ends the shared part.  The other
  blocks are taken fresh; the fresh full ones are registered under their
  keys (their K/V is computed by this prompt's prefill) unless the key is
  already held by another block.  A prompt that cannot get its blocks takes
  none (everything is rolled back).
* A block that fills up through appended tokens is registered the same way.
* Freeing a request drops one reference per block, visiting its blocks from
  the last to the first; each block that reaches zero goes to the back of
  the queue.
"""
from __future__ import annotations

import hashlib
from collections import OrderedDict

HASH_SHA256 = 0
HASH_FNV1A64 = 1
ZERO_KEY = bytes(32)

_FNV_OFFSET = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3


class PoolExhausted(RuntimeError):
    pass


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a (Fowler, Noll, Vo): for each byte, xor then multiply."""
    h = _FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * _FNV_PRIME) & 0xFFFFFFFFFFFFFFFF
    return h


def block_key(parent: bytes, tokens, extra: bytes = b"", kind: int = HASH_SHA256) -> bytes:
    """Key of a full block: Hash(parent key, this block's token ids, extras)."""
    data = bytes(parent) + b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens) \
        + bytes(extra)
    if kind == HASH_SHA256:
        return hashlib.sha256(data).digest()
    if kind == HASH_FNV1A64:
        return fnv1a64(data).to_bytes(8, "little") + bytes(24)
    raise ValueError("unknown hash kind")


class Request:
    def __init__(self, extra: bytes):
        self.blocks: list = []
        self.tokens: list = []
        self.extra = bytes(extra)
        self.last_key = ZERO_KEY     # key of the last full block (chain parent)


class BlockManagerModel:
    """Free queue (LRU), reference counts, prefix-key cache, block tables."""

    def __init__(self, num_blocks: int, block_size: int = 16, hash_kind: int = HASH_SHA256,
                 free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.hash_kind = hash_kind
        order = range(self.num_blocks) if free_order is None else [int(b) for b in free_order]
        self.free = OrderedDict((b, None) for b in order)   # front = next to take
        assert len(self.free) == self.num_blocks
        self.refcount = [0] * self.num_blocks
        self.key_of = {}          # block -> key it holds (cached)
        self.block_of = {}        # key -> block
        self.requests = {}

    # -- pool ---------------------------------------------------------------
    def num_free(self) -> int:
        return len(self.free)

    def num_cached(self) -> int:
        return len(self.block_of)

    def _take(self) -> int:
        if not self.free:
            raise PoolExhausted("no free block")
        b, _ = self.free.popitem(last=False)
        if b in self.key_of:                      # evict its cached contents
            del self.block_of[self.key_of.pop(b)]
        self.refcount[b] = 1
        return b

    def _ref(self, b: int) -> None:
        if self.refcount[b] == 0:
            del self.free[b]                      # a hit on a queued block
        self.refcount[b] += 1

    def _unref(self, b: int) -> None:
        self.refcount[b] -= 1
        assert self.refcount[b] >= 0
        if self.refcount[b] == 0:
            self.free[b] = None                   # to the back of the queue

    def _register(self, b: int, key: bytes) -> None:
        if key not in self.block_of and b not in self.key_of:
            self.block_of[key] = b
            self.key_of[b] = key

    # -- requests ---------------------------------------------------------------
    def add_request(self, rid, tokens, extra: bytes = b"") -> int:
        """Admit a prompt; returns the number of its tokens found in the cache."""
        assert rid not in self.requests
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        r = Request(extra)
        n_full = len(tokens) // bs
        hits, parent, keys = 0, ZERO_KEY, []
        for j in range(n_full):
            k = block_key(parent, tokens[j * bs:(j + 1) * bs], r.extra, self.hash_kind)
            keys.append(k)
            parent = k
        # the leading run of hits
        while hits < n_full and keys[hits] in self.block_of:
            hits += 1
        need = -(-len(tokens) // bs) - hits
        # a hit may take a queued block out of the queue: count what stays free
        queued_hits = sum(1 for j in range(hits) if self.refcount[self.block_of[keys[j]]] == 0)
        if need > len(self.free) - queued_hits:
            raise PoolExhausted(f"need {need} blocks")
        for j in range(hits):
            b = self.block_of[keys[j]]
            self._ref(b)
            r.blocks.append(b)
        for j in range(hits, hits + need):
            b = self._take()
            r.blocks.append(b)
            if j < n_full:
                self._register(b, keys[j])
        r.tokens = tokens
        r.last_key = keys[n_full - 1] if n_full else ZERO_KEY
        self.requests[rid] = r
        return hits * bs

    def fork(self, parent, child) -> None:
        """The child shares every block of the parent (parallel sampling)."""
        assert child not in self.requests
        p = self.requests[parent]
        c = Request(p.extra)
        c.blocks = list(p.blocks)
        c.tokens = list(p.tokens)
        c.last_key = p.last_key
        for b in c.blocks:
            self._ref(b)
        self.requests[child] = c

    def append_token(self, rid, token):
        """Slot of the new token, and the (src, dst) copy made first, or None."""
        r = self.requests[rid]
        bs = self.block_size
        pos = len(r.tokens)
        cow = None
        if pos % bs == 0:
            r.blocks.append(self._take())
        else:
            last = r.blocks[-1]
            if self.refcount[last] > 1:           # shared: copy before writing
                nb = self._take()
                self._unref(last)
                r.blocks[-1] = nb
                cow = (last, nb)
        r.tokens.append(int(token))
        slot = r.blocks[-1] * bs + pos % bs
        if (pos + 1) % bs == 0:                   # the block is now full: cache it
            k = block_key(r.last_key, r.tokens[pos + 1 - bs:pos + 1], r.extra, self.hash_kind)
            r.last_key = k
            self._register(r.blocks[-1], k)
        return slot, cow

    def free_request(self, rid) -> None:
        r = self.requests.pop(rid)
        for b in reversed(r.blocks):              # tail first
            self._unref(b)

    def block_table(self, rid) -> list:
        return list(self.requests[rid].blocks)

    def num_tokens(self, rid) -> int:
        return len(self.requests[rid].tokens)

    def lookup(self, key: bytes):
        return self.block_of.get(bytes(key), -1)

    def decode_step(self, rids, tokens):
        """Append one token to each request in order; returns (slots, copies)."""
        slots, copies = [], []
        for rid, t in zip(rids, tokens):
            s, cow = self.append_token(rid, t)
            slots.append(s)
            if cow is not None:
                copies.append(cow)
        return slots, copies
