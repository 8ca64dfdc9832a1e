"""Parity of the HIP multi-query paged attention (chunked prefill) with the CPU
oracle, through the C-ABI, on the GPU.

Every case appends the chunk's K/V with pa_reshape_and_cache (T tokens,
several per sequence) and then runs pa_prefill; the oracle does the same two
steps on the CPU.  Small cases are checked row by row in full; the full-size
batches on sampled rows, each computed by the oracle as a chunk of one that
ends at the row's position (the oracle's own chunking invariance, pinned in
test_oracle_prefill.py).
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_59_amd import binding as pk
from paged_kv_cache_59_amd import workloads as wl
from tests.gpu_util import compare, dev, log

pytestmark = pytest.mark.gpu


def to_device_prefill(w):
    return {
        "q": dev(w.q), "k_cache": dev(w.k_cache), "v_cache": dev(w.v_cache),
        "block_tables": dev(w.block_tables), "context_lens": dev(w.context_lens),
        "query_start": dev(w.query_start), "k_new": dev(w.k_new), "v_new": dev(w.v_new),
        "slot_mapping": dev(w.slot_mapping),
        "out": torch.full(w.q.shape, float("nan"), dtype=torch.float16, device="cuda"),
    }


def gpu_prefill_step(w, d, max_query_len=None):
    pk.pa_reshape_and_cache(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"])
    pk.pa_prefill(d["out"], d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                  d["context_lens"], d["query_start"], float(w.scale), w.num_kv_heads,
                  max_context_len=w.max_context_len,
                  max_query_len=w.max_query_len if max_query_len is None else max_query_len)
    torch.cuda.synchronize()
    return d["out"].cpu().numpy()


def oracle_pools_prefill(w):
    return oracle.reshape_and_cache(w.k_new, w.v_new, w.k_cache, w.v_cache, w.slot_mapping,
                                    block_size=w.block_size)


def oracle_rows(w, kc, vc, rows):
    """Oracle output of the given packed rows, each as a chunk of one ending at
    its own position."""
    seq_of = np.searchsorted(w.query_start, rows, side="right") - 1
    out = np.zeros((len(rows), w.num_q_heads, w.head_dim))
    for k, (t, s) in enumerate(zip(rows, seq_of)):
        n, t0, t1 = int(w.context_lens[s]), int(w.query_start[s]), int(w.query_start[s + 1])
        p = n - (t1 - t0) + (t - t0)
        out[k] = oracle.prefill(w.q[t:t + 1], kc, vc, w.block_tables[s:s + 1],
                                np.array([p + 1], np.int32), np.array([0, 1], np.int32),
                                w.scale, w.num_kv_heads, block_size=w.block_size)[0]
    return out


def run_full_parity(w, label):
    log(f"prefill case {label}: S={w.num_seqs} T={w.num_tokens} Hq={w.num_q_heads} "
        f"Hkv={w.num_kv_heads} D={w.head_dim} maxctx={w.max_context_len}")
    d = to_device_prefill(w)
    out = gpu_prefill_step(w, d)
    kc, vc = oracle_pools_prefill(w)
    assert np.array_equal(d["k_cache"].cpu().numpy().view(np.uint16), kc.view(np.uint16))
    assert np.array_equal(d["v_cache"].cpu().numpy().view(np.uint16), vc.view(np.uint16))
    ref = oracle.prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.query_start, w.scale,
                         w.num_kv_heads, block_size=w.block_size)
    compare(out, ref, label)
    return out


def test_prefill_tiny():
    run_full_parity(wl.make_named_prefill("prefill_tiny"), "prefill_tiny")


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 64), (8, 2, 64), (32, 8, 128), (12, 4, 128),
                                      (16, 1, 64), (6, 6, 128)])
def test_prefill_shapes_chunks_and_tails(Hq, Hkv, D):
    """Chunks of 1 (a decode step), whole prompts, chunks crossing 32-row
    tiles and 32-key steps, empty chunks, contexts ending mid-block."""
    lens = [1, 9, 40, 64, 65, 100, 300, 517, 33, 700]
    nqs = [1, 9, 7, 33, 1, 100, 64, 0, 33, 129]
    w = wl.make_prefill_workload("shapes", 500 + Hq + D, Hq, Hkv, D, context_lens=lens,
                                 chunk_lens=nqs)
    run_full_parity(w, f"shapes Hq{Hq} Hkv{Hkv} D{D}")


def test_prefill_chunk_of_one_matches_decode_kernel():
    """n_q = 1 for every sequence is a decode step: pa_prefill and pa_decode
    agree within rounding (different kernels, different summation order)."""
    lens = [1, 17, 200, 1000, 64]
    w = wl.make_prefill_workload("one", 601, 32, 8, 128, context_lens=lens, chunk_lens=[1] * 5)
    d = to_device_prefill(w)
    out = gpu_prefill_step(w, d)
    dec = torch.empty_like(d["q"])
    pk.pa_decode(dec, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                 float(w.scale), 8, max_context_len=w.max_context_len)
    torch.cuda.synchronize()
    assert np.abs(out.astype(np.float64) - dec.cpu().numpy().astype(np.float64)).max() < 4e-3


def test_prefill_chunked_equals_whole_prompt():
    """A prompt prefilled in one chunk and the same prompt in three chunks
    (each chunk appended, then attended) give the same rows within rounding."""
    n = 300
    w = wl.make_prefill_workload("whole", 602, 8, 2, 128, context_lens=[n], chunk_lens=[n])
    d = to_device_prefill(w)
    whole = gpu_prefill_step(w, d)
    cuts = [0, 100, 101, 300]
    for a, b in zip(cuts[:-1], cuts[1:]):
        out = torch.full((b - a, 8, 128), float("nan"), dtype=torch.float16, device="cuda")
        pk.pa_prefill(out, d["q"][a:b].contiguous(), d["k_cache"], d["v_cache"], d["block_tables"],
                      dev(np.array([b], np.int32)), dev(np.array([0, b - a], np.int32)),
                      float(w.scale), 2, max_context_len=n, max_query_len=b - a)
        torch.cuda.synchronize()
        diff = np.abs(out.cpu().numpy().astype(np.float64) - whole[a:b].astype(np.float64))
        assert diff.max() < 2e-3, (a, b)


def test_prefill_peaky_softmax():
    w = wl.make_prefill_workload("peaky", 603, 16, 4, 128, context_lens=[90, 400],
                                 chunk_lens=[90, 70], scale=8.0 / np.sqrt(128))
    run_full_parity(w, "peaky")


def test_prefill_chunks_past_num_tokens_are_skipped():
    """num_tokens below query_start's last entry: the chunks that would reach
    past it are skipped (their rows keep their NaN), the rest are computed."""
    w = wl.make_named_prefill("prefill_tiny")
    d = to_device_prefill(w)
    pk.pa_reshape_and_cache(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"])
    cut = int(w.query_start[2])  # sequences 0, 1 fit; 2, 3 reach past the cut
    L = pk.lib()
    code = L.pa_prefill(d["out"].data_ptr(), d["q"].data_ptr(), d["k_cache"].data_ptr(),
                        d["v_cache"].data_ptr(), d["block_tables"].data_ptr(),
                        d["context_lens"].data_ptr(), d["query_start"].data_ptr(), cut,
                        float(w.scale), 4, 4, 4, 64, 16, int(w.block_tables.shape[1]),
                        int(w.num_blocks), w.max_context_len, w.max_query_len, None)
    assert code == 0
    torch.cuda.synchronize()
    out = d["out"].cpu().numpy()
    kc, vc = oracle_pools_prefill(w)
    ref = oracle.prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.query_start, w.scale, 4)
    compare(out[:cut], ref[:cut], "rows before the cut")
    assert np.isnan(out[cut:].astype(np.float32)).all()


def test_prefill_rows_past_max_query_len_untouched_and_errors():
    w = wl.make_named_prefill("prefill_tiny")
    d = to_device_prefill(w)
    # a bound below a chunk: that chunk's rows stay unwritten (NaN), the others are right
    out = gpu_prefill_step(w, d, max_query_len=20)
    kc, vc = oracle_pools_prefill(w)
    ref = oracle.prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.query_start, w.scale,
                         w.num_kv_heads)
    big = int(np.argmax(np.diff(w.query_start)))
    rows = np.arange(w.query_start[big], w.query_start[big + 1])
    assert np.isnan(out[rows].astype(np.float32)).all()
    keep = np.setdiff1d(np.arange(w.num_tokens), rows)
    compare(out[keep], ref[keep], "bounded")
    L = pk.lib()
    args = [d["out"].data_ptr(), d["q"].data_ptr(), d["k_cache"].data_ptr(), d["v_cache"].data_ptr(),
            d["block_tables"].data_ptr(), d["context_lens"].data_ptr(), d["query_start"].data_ptr(),
            w.num_tokens, float(w.scale), 4, 4, 4, 64, 16, int(w.block_tables.shape[1]),
            int(w.num_blocks), w.max_context_len, w.max_query_len, None]
    assert L.pa_prefill(*args) == 0
    bad = list(args)
    bad[13] = 24                                        # block size not 8, 16 or 32
    assert L.pa_prefill(*bad) == -2
    bad = list(args)
    bad[17] = w.max_context_len + 1                     # chunk bound above the context bound
    assert L.pa_prefill(*bad) == -1
    bad = list(args)
    bad[6] = None                                       # query_start missing
    assert L.pa_prefill(*bad) == -1
    bad = list(args)
    bad[17] = 0                                         # nothing to do
    assert L.pa_prefill(*bad) == 0
    bad = list(args)
    bad[7] = -1                                         # negative row count
    assert L.pa_prefill(*bad) == -1
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["chunked_prefill_llama", "prefix_hit_llama"])
def test_prefill_full_size_sampled(name):
    """The benchmarked batches at full size: appended pools bit-exact, sampled
    rows (first, last and middle rows of several sequences) against the oracle,
    every output finite."""
    w = wl.make_named_prefill(name)
    log(f"prefill full {name}: S={w.num_seqs} T={w.num_tokens} maxctx={w.max_context_len}")
    d = to_device_prefill(w)
    out = gpu_prefill_step(w, d)
    assert np.isfinite(out.astype(np.float32)).all()
    kc, vc = oracle_pools_prefill(w)
    assert np.array_equal(d["k_cache"].cpu().numpy().view(np.uint16), kc.view(np.uint16))
    rng = np.random.default_rng(7)
    seqs = rng.choice(w.num_seqs, size=4, replace=False)
    rows = []
    for s in seqs:
        t0, t1 = int(w.query_start[s]), int(w.query_start[s + 1])
        rows += [t0, t0 + 1, (t0 + t1) // 2, t1 - 1]
    rows = np.unique(rows)
    compare(out[rows], oracle_rows(w, kc, vc, rows), f"{name} sampled")


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_prefill_negative_and_zero_scale(scale):
    """A negative scale enters as a sign flip of q (exact); a zero scale gives
    every visible key the same weight: the mean of the visible V rows."""
    w = wl.make_prefill_workload("scale", 604, 8, 2, 128, context_lens=[70, 300],
                                 chunk_lens=[70, 45], scale=scale)
    out = run_full_parity(w, f"scale {scale}")
    if scale == 0.0:
        kc, vc = oracle_pools_prefill(w)
        k, v = oracle.gather_sequence(kc, vc, w.block_tables[0], 70, 2, 128)
        for i in (0, 1, 69):
            mean = v[:, :i + 1].mean(axis=1)              # [Hkv, D]
            assert np.abs(out[i].astype(np.float64) - np.repeat(mean, 4, axis=0)).max() < 2e-3


@pytest.mark.parametrize("BS", [8, 32])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (8, 8, 64), (16, 2, 64)])
def test_prefill_block_sizes(BS, Hq, Hkv, D):
    """Block sizes 8 and 32: a 32-key step spans 4 blocks, or one; contexts
    and chunks ending inside and at block edges."""
    lens = [1, 8, 9, 31, 32, 33, 100, 257, 64]
    nqs = [1, 8, 3, 31, 1, 17, 64, 100, 0]
    w = wl.make_prefill_workload("pbs", 800 + BS + Hq + D, Hq, Hkv, D, context_lens=lens,
                                 chunk_lens=nqs, block_size=BS)
    run_full_parity(w, f"prefill BS{BS} Hq{Hq} Hkv{Hkv} D{D}")
