"""Continuous-batching decode simulator over the library's block manager and,
optionally, its GPU kernels.

What it follows (web pages, sections named by their headings):

* "Continuous batching and paged attention" (abhi-g.dev), "Continuous
  batching": batch membership changes every iteration; finished sequences
  leave and waiting ones are admitted into the freed slots; a new sequence's
  prefill runs alongside other sequences' decode steps, and chunked prefill
  splits a prompt across iterations.  "Paged attention": admission asks
  whether there are enough free blocks for the prompt plus a margin for
  generation.  "Why they depend on each other": when blocks run out, a
  request is preempted, by recomputation or by swap to host memory.
  "Operational implications": max_num_batched_tokens bounds the work per
  iteration; block utilisation is the capacity metric.
* "Continuous batching, paged attention, prefix caching" (backplane.click),
  "Static versus continuous batching": the four-step figure in which a
  finished request's blocks are taken by a newcomer.
* "KV Cache in Serving Engines" (ttlab), section 3 (chunked prefill, decodes
  scheduled first) and section 5 "When KV Space Falls Short" (preempted
  requests recompute their prefill).

Scheduling, per iteration (readings where the pages leave a step open):
  1. swapped-out requests come back first (oldest first) when their blocks fit;
  2. waiting requests are admitted in arrival order while the running count is
     below max_running and the free blocks cover the prompt's uncached blocks
     plus ``margin_blocks``; admission goes through the block manager, so full
     prompt blocks already cached are reused;
  3. every running request past its prefill decodes one token (decodes first);
     one that needs a block when none is free preempts the most recently
     admitted running request (itself, if it is the latest) -- by
     recomputation (its blocks are freed; its prompt plus generated tokens go
     back to the front of the queue) or by swap (its blocks are copied to a
     host pool, then freed on the device);
  4. the rest of the token budget goes to prefill chunks, in admission order;
  5. requests that have generated their output leave and free their blocks.

Tokens are synthetic: the token after position p, and the K, V and q of
position p, are functions of the prefix tokens[0..p] alone (a rolling FNV-1a
hash seeds them).  So blocks reused through the prefix cache hold exactly the
K/V the request would have computed, and a check can rebuild any request's
logical K/V from its tokens.
"""
from __future__ import annotations

import argparse
import json
import math
from collections import deque
from dataclasses import dataclass, field

import numpy as np

from . import block_manager as cbm

_FNV_OFFSET = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3
_MASK = 0xFFFFFFFFFFFFFFFF


def roll(h: int, token: int) -> int:
    """FNV-1a over one more token (4 little-endian bytes)."""
    for b in int(token & 0xFFFFFFFF).to_bytes(4, "little"):
        h = ((h ^ b) * _FNV_PRIME) & _MASK
    return h


def prefix_hashes(tokens) -> list:
    h, out = _FNV_OFFSET, []
    for t in tokens:
        h = roll(h, t)
        out.append(h)
    return out


def next_token(h: int, vocab: int) -> int:
    return int((h >> 17) % vocab)


def token_tensors(h: int, num_q_heads: int, num_kv_heads: int, head_dim: int):
    """q [Hq, D], k [Hkv, D], v [Hkv, D] fp16 of the position whose prefix
    hash is h."""
    rng = np.random.default_rng(h)
    x = rng.standard_normal(num_q_heads * head_dim + 2 * num_kv_heads * head_dim,
                            dtype=np.float32).astype(np.float16)
    q = x[:num_q_heads * head_dim].reshape(num_q_heads, head_dim)
    k = x[num_q_heads * head_dim:][:num_kv_heads * head_dim].reshape(num_kv_heads, head_dim)
    v = x[num_q_heads * head_dim + num_kv_heads * head_dim:].reshape(num_kv_heads, head_dim)
    return q, k, v


@dataclass
class Request:
    rid: int
    arrival: int
    prompt: list
    output_len: int
    tokens: list = field(default_factory=list)   # prompt + generated so far
    hashes: list = field(default_factory=list)   # prefix hash of each position
    generated: int = 0
    computed: int = 0          # tokens whose K/V are in the cache
    admitted_at: int = -1
    first_token_step: int = -1
    finished_step: int = -1
    preemptions: int = 0
    host_blocks: list = field(default_factory=list)   # while swapped out


@dataclass
class Config:
    num_blocks: int = 256
    block_size: int = 16
    max_running: int = 32
    max_batched_tokens: int = 512
    margin_blocks: int = 1
    preemption: str = "recompute"          # or "swap"
    host_blocks: int = 1024
    hash_kind: int = cbm.HASH_SHA256
    vocab: int = 32000
    num_q_heads: int = 8
    num_kv_heads: int = 2
    head_dim: int = 64


class Simulator:
    """Iteration-level scheduler over a C++ block manager.  With ``gpu=True``
    every iteration also runs the library's kernels on real pools: copies,
    appends, prefill chunks, decode, swaps."""

    def __init__(self, cfg: Config, gpu: bool = False, check_every: int = 0, check_row=None):
        """``check_every`` > 0 checks the decoded rows every that many steps
        with ``check_row(request, position, row, scale) -> max abs error``
        (a caller-supplied reference: a request's K, V and q at every position
        follow from its token hashes through ``token_tensors``)."""
        if check_every and check_row is None:
            raise ValueError("checking rows needs a check_row callback")
        self.cfg = cfg
        self.bm = cbm.BlockManager(cfg.num_blocks, cfg.block_size, cfg.hash_kind)
        self.waiting: deque = deque()
        self.swapped: deque = deque()
        self.running: list = []
        self.finished: list = []
        self.host_free = deque(range(cfg.host_blocks))
        self.step_no = 0
        self.stats = {"preempt_recompute": 0, "preempt_swap": 0, "swap_out_blocks": 0,
                      "swap_in_blocks": 0, "prefix_hit_tokens": 0, "prefill_tokens": 0,
                      "decode_tokens": 0, "copies": 0}
        self.trace = []
        self.gpu = gpu
        self.check_every = check_every
        self.check_row = check_row
        self.checked_rows = 0
        self.max_abs_err = 0.0
        if gpu:
            self._init_gpu()

    # -- request intake -----------------------------------------------------------
    def submit(self, req: Request) -> None:
        req.tokens = list(req.prompt)
        req.hashes = prefix_hashes(req.tokens)
        self.waiting.append(req)

    # -- helpers ------------------------------------------------------------------
    def _blocks_for(self, n: int) -> int:
        return -(-n // self.cfg.block_size)

    def _admit(self, req: Request) -> bool:
        need = self._blocks_for(len(req.tokens)) + self.cfg.margin_blocks
        if self.bm.num_free() < need:   # counts blocks hits would reuse too: conservative
            return False
        cached = self.bm.add_request(req.rid, req.tokens)
        self.stats["prefix_hit_tokens"] += cached
        req.computed = min(cached, len(req.tokens) - 1) if req.tokens else 0
        if req.admitted_at < 0:
            req.admitted_at = self.step_no
        self.running.append(req)
        return True

    def _preempt(self, victim: Request) -> None:
        self.running.remove(victim)
        victim.preemptions += 1
        if self.cfg.preemption == "swap" and len(self.host_free) >= len(self.bm.block_table(victim.rid)):
            table = self.bm.block_table(victim.rid)
            victim.host_blocks = [self.host_free.popleft() for _ in table]
            if self.gpu:
                self._swap(list(zip(table, victim.host_blocks)), out=True)
            self.stats["swap_out_blocks"] += len(table)
            self.stats["preempt_swap"] += 1
            self.bm.free_request(victim.rid)
            self.swapped.append(victim)
        else:
            self.bm.free_request(victim.rid)
            victim.computed = 0
            self.stats["preempt_recompute"] += 1
            self.waiting.appendleft(victim)

    def _swap_in(self, req: Request) -> bool:
        need = self._blocks_for(len(req.tokens)) + self.cfg.margin_blocks
        if self.bm.num_free() < need:
            return False
        cached = self.bm.add_request(req.rid, req.tokens)
        table = self.bm.block_table(req.rid)
        first = cached // self.cfg.block_size       # blocks the prefix cache still held
        pairs = list(zip(req.host_blocks[first:], table[first:]))
        if self.gpu and pairs:
            self._swap(pairs, out=False)
        self.stats["swap_in_blocks"] += len(pairs)
        self.host_free.extend(req.host_blocks)
        req.host_blocks = []
        self.running.append(req)
        return True

    # -- one iteration ------------------------------------------------------------
    def step(self) -> dict:
        cfg = self.cfg
        # 1. swapped-out requests first, then waiting ones, in order
        while self.swapped and len(self.running) < cfg.max_running and self._swap_in(self.swapped[0]):
            self.swapped.popleft()
        while self.waiting and len(self.running) < cfg.max_running and not self.swapped:
            if not self._admit(self.waiting[0]):
                break
            self.waiting.popleft()

        budget = cfg.max_batched_tokens
        decode_reqs, decode_slots, decode_pos, copies = [], [], [], []
        # 2. decodes first: one token each for requests past their prefill
        for req in list(self.running):
            if req not in self.running or req.computed < len(req.tokens) or budget <= 0:
                continue
            while True:
                try:
                    tok = self._next_token(req)
                    slot, cow = self.bm.append_token(req.rid, tok)
                    break
                except cbm.PoolExhausted:
                    victim = max(self.running, key=lambda r: (r.admitted_at, r.rid))
                    self._preempt(victim)
                    if victim is req:
                        break
            if req not in self.running:
                continue
            req.tokens.append(tok)
            req.hashes.append(roll(req.hashes[-1] if req.hashes else _FNV_OFFSET, tok))
            req.computed += 1
            req.generated += 1
            if req.first_token_step < 0:
                req.first_token_step = self.step_no
            if cow is not None:
                copies.append(cow)
            decode_reqs.append(req)
            decode_slots.append(slot)
            decode_pos.append(len(req.tokens) - 1)
            budget -= 1
        # 3. prefill chunks with what is left of the budget
        chunks = []
        for req in self.running:
            if budget <= 0:
                break
            left = len(req.tokens) - req.computed
            if left <= 0 or req in decode_reqs:
                continue
            n = min(left, budget)
            chunks.append((req, req.computed, n))
            req.computed += n
            budget -= n
        self.stats["decode_tokens"] += len(decode_reqs)
        self.stats["prefill_tokens"] += sum(n for _, _, n in chunks)
        self.stats["copies"] += len(copies)
        if self.gpu:
            self._run_gpu(decode_reqs, decode_slots, decode_pos, copies, chunks)
        ran = [r.rid for r in self.running]
        # 4. finished requests leave
        for req in list(self.running):
            if req.computed >= len(req.tokens) and req.generated >= req.output_len:
                self.running.remove(req)
                self.bm.free_request(req.rid)
                req.finished_step = self.step_no
                self.finished.append(req)
        rec = self._record(ran, decode_reqs, chunks)
        self.step_no += 1
        return rec

    def _next_token(self, req: Request) -> int:
        return next_token(req.hashes[-1] if req.hashes else _FNV_OFFSET, self.cfg.vocab)

    def _record(self, ran, decode_reqs, chunks) -> dict:
        """The iteration's batch (the requests that ran in it) and the pool
        after it: blocks in use, and the fraction of the slots of the running
        requests' blocks that hold tokens (block utilisation)."""
        used_blocks = self.cfg.num_blocks - self.bm.num_free()
        held_tokens = sum(self.bm.num_tokens(r.rid) for r in self.running)
        held_blocks = sum(len(self.bm.block_table(r.rid)) for r in self.running)
        rec = {"step": self.step_no, "running": ran,
               "decoded": len(decode_reqs), "prefilled": sum(n for _, _, n in chunks),
               "free_blocks": self.bm.num_free(), "used_blocks": used_blocks,
               # requests holding every token of their prompt and output at once
               "full": sum(1 for r in self.running
                           if self.bm.num_tokens(r.rid) >= len(r.prompt) + r.output_len),
               "utilisation": held_tokens / (held_blocks * self.cfg.block_size) if held_blocks else 1.0}
        self.trace.append(rec)
        return rec

    def run(self, arrivals, max_steps: int = 100000) -> dict:
        """arrivals: list of (arrival_step, Request), in order."""
        pending = deque(sorted(arrivals, key=lambda x: (x[0], x[1].rid)))
        while (pending or self.waiting or self.running or self.swapped) and self.step_no < max_steps:
            while pending and pending[0][0] <= self.step_no:
                self.submit(pending.popleft()[1])
            self.step()
        return self.summary()

    def summary(self) -> dict:
        util = [r["utilisation"] for r in self.trace if r["running"]]
        s = dict(self.stats)
        s.update({"steps": self.step_no, "finished": len(self.finished),
                  "peak_running": max((len(r["running"]) for r in self.trace), default=0),
                  "mean_block_utilisation": float(np.mean(util)) if util else 1.0,
                  "min_block_utilisation": float(np.min(util)) if util else 1.0})
        if self.gpu:
            s["checked_rows"] = self.checked_rows
            s["max_abs_err"] = self.max_abs_err
        return s

    # -- GPU execution ----------------------------------------------------------------
    def _init_gpu(self) -> None:
        import torch
        from . import binding as pk
        self.torch, self.pk = torch, pk
        c = self.cfg
        BS, Hkv, D = c.block_size, c.num_kv_heads, c.head_dim
        self.kc = torch.zeros((c.num_blocks, Hkv, D // 8, BS, 8), dtype=torch.float16, device="cuda")
        self.vc = torch.zeros((c.num_blocks, Hkv, BS // 8, D, 8), dtype=torch.float16, device="cuda")
        self.hk = torch.zeros((c.host_blocks, Hkv, D // 8, BS, 8), dtype=torch.float16).pin_memory()
        self.hv = torch.zeros((c.host_blocks, Hkv, BS // 8, D, 8), dtype=torch.float16).pin_memory()
        self.scale = 1.0 / math.sqrt(D)

    def _swap(self, pairs, out: bool) -> None:
        torch, pk = self.torch, self.pk
        m = torch.tensor(pairs, dtype=torch.int64, device="cuda").reshape(-1, 2)
        if out:
            pk.pa_swap_blocks(self.kc, self.vc, self.hk, self.hv, m)
        else:
            pk.pa_swap_blocks(self.hk, self.hv, self.kc, self.vc, m)

    def _slot(self, req: Request, pos: int) -> int:
        table = self.bm.block_table(req.rid)
        return table[pos // self.cfg.block_size] * self.cfg.block_size + pos % self.cfg.block_size

    def _run_gpu(self, decode_reqs, decode_slots, decode_pos, copies, chunks) -> None:
        torch, pk, c = self.torch, self.pk, self.cfg
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        if copies:
            pk.pa_copy_blocks(self.kc, self.vc, dev(np.asarray(copies, dtype=np.int64)))
        # append: every token whose K/V this iteration computes
        rows = []                         # (req, pos, slot)
        for req, start, n in chunks:
            for p in range(start, start + n):
                rows.append((req, p, self._slot(req, p)))
        for req, slot, p in zip(decode_reqs, decode_slots, decode_pos):
            rows.append((req, p, slot))
        if rows:
            ks, vs = [], []
            for req, p, _ in rows:
                _, k, v = token_tensors(req.hashes[p], c.num_q_heads, c.num_kv_heads, c.head_dim)
                ks.append(k)
                vs.append(v)
            pk.pa_reshape_and_cache(dev(np.stack(ks)), dev(np.stack(vs)), self.kc, self.vc,
                                    dev(np.asarray([s for _, _, s in rows], dtype=np.int64)))
        MB = max((len(self.bm.block_table(r.rid)) for r in self.running), default=1)
        checks = []
        # prefill chunks: rows at positions start .. start+n-1 of contexts start+n
        if chunks:
            qs, lens, tabs, starts = [], [], [], [0]
            for req, start, n in chunks:
                for p in range(start, start + n):
                    qs.append(token_tensors(req.hashes[p], c.num_q_heads, c.num_kv_heads,
                                            c.head_dim)[0])
                lens.append(start + n)
                t = self.bm.block_table(req.rid)
                tabs.append(t + [-1] * (MB - len(t)))
                starts.append(starts[-1] + n)
            q = dev(np.stack(qs))
            out = torch.empty_like(q)
            pk.pa_prefill(out, q, self.kc, self.vc, dev(np.asarray(tabs, np.int32)),
                          dev(np.asarray(lens, np.int32)), dev(np.asarray(starts, np.int32)),
                          self.scale, c.num_kv_heads, max_context_len=MB * c.block_size,
                          max_query_len=max(n for _, _, n in chunks))
            last = [(req, start + n - 1, starts[i + 1] - 1) for i, (req, start, n) in enumerate(chunks)]
            checks.append((out, last))
        if decode_reqs:
            qs, lens, tabs = [], [], []
            for req, p in zip(decode_reqs, decode_pos):
                qs.append(token_tensors(req.hashes[p], c.num_q_heads, c.num_kv_heads,
                                        c.head_dim)[0])
                lens.append(p + 1)
                t = self.bm.block_table(req.rid)
                tabs.append(t + [-1] * (MB - len(t)))
            q = dev(np.stack(qs))
            out = torch.empty_like(q)
            pk.pa_decode(out, q, self.kc, self.vc, dev(np.asarray(tabs, np.int32)),
                         dev(np.asarray(lens, np.int32)), self.scale, c.num_kv_heads,
                         max_context_len=MB * c.block_size)
            checks.append((out, [(req, p, i) for i, (req, p) in enumerate(zip(decode_reqs, decode_pos))]))
        if self.check_every and self.step_no % self.check_every == 0:
            torch.cuda.synchronize()
            for out, items in checks:
                o = out.cpu().numpy()
                for req, p, row in items:
                    err = self.check_row(req, p, o[row], self.scale)
                    self.max_abs_err = max(self.max_abs_err, float(err))
                    self.checked_rows += 1


def synthetic_arrivals(num_requests: int, seed: int, rate: float, prompt_range, output_range,
                       shared_prefix: int = 0, vocab: int = 32000, first_id: int = 0):
    """Seeded arrivals: gaps ~ exponential(1/rate) steps, prompts and outputs
    integer-uniform; optionally every prompt starts with one shared prefix."""
    rng = np.random.default_rng(seed)
    prefix = rng.integers(0, vocab, size=shared_prefix).tolist()
    t, out = 0.0, []
    for i in range(num_requests):
        t += rng.exponential(1.0 / rate) if rate > 0 else 0.0
        n_in = int(rng.integers(prompt_range[0], prompt_range[1] + 1))
        n_out = int(rng.integers(output_range[0], output_range[1] + 1))
        prompt = prefix + rng.integers(0, vocab, size=n_in).tolist()
        out.append((int(t), Request(rid=first_id + i, arrival=int(t), prompt=prompt,
                                    output_len=n_out)))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--num-blocks", type=int, default=1378)
    ap.add_argument("--block-size", type=int, default=16)
    ap.add_argument("--requests", type=int, default=200)
    ap.add_argument("--rate", type=float, default=2.0, help="arrivals per iteration")
    ap.add_argument("--prompt", type=int, nargs=2, default=(256, 768))
    ap.add_argument("--output", type=int, nargs=2, default=(64, 256))
    ap.add_argument("--shared-prefix", type=int, default=0)
    ap.add_argument("--max-running", type=int, default=64)
    ap.add_argument("--max-batched-tokens", type=int, default=2048)
    ap.add_argument("--preemption", choices=["recompute", "swap"], default="recompute")
    ap.add_argument("--seed", type=int, default=1)
    a = ap.parse_args(argv)
    cfg = Config(num_blocks=a.num_blocks, block_size=a.block_size, max_running=a.max_running,
                 max_batched_tokens=a.max_batched_tokens, preemption=a.preemption,
                 host_blocks=4 * a.num_blocks)
    sim = Simulator(cfg)
    arr = synthetic_arrivals(a.requests, a.seed, a.rate, a.prompt, a.output, a.shared_prefix)
    print(json.dumps(sim.run(arr)))


if __name__ == "__main__":
    main()
