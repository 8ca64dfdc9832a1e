"""Parity of the fused append + decode (pa_decode_append) with the oracle's
append followed by its decode, on the GPU, through the C-ABI.

The fused launch takes each sequence's last position from the new rows
instead of the pools and stores the rows into their slots: the pools must
then equal the oracle's after its append, bit for bit, and the output the
oracle's attention over them.  Cases cover runs whose last 64-token unit
holds only the new token (lengths 64k + 1, alone in a piece when every unit
is its own share), cut runs, padding slots, empty rows, every block size,
and the full-size batches in the benchmark's launch configuration.
"""
import numpy as np
import pytest
import torch

import oracle
from paged_kv_cache_59_amd import binding as pk
from paged_kv_cache_59_amd import workloads as wl
from tests.gpu_util import (assert_pools_equal, compare, decode_control_bytes, gpu_step, log,
                            named, oracle_decode, oracle_pools, to_device)

pytestmark = pytest.mark.gpu

# lengths around unit (64) and block boundaries; 1, 65, 129, 1025: the new
# token alone in the run's last unit
FUSED_LENS = [1, 2, 15, 16, 17, 63, 64, 65, 66, 127, 128, 129, 257, 511, 513, 1025, 1000]


def fused_step(w, d, num_workers=0, workspace=None, shared_blocks=False):
    """copy-on-write (if any), then one pa_decode_append; out as numpy fp16."""
    if w.block_mapping.shape[0]:
        pk.pa_copy_blocks(d["k_cache"], d["v_cache"], d["block_mapping"])
    pk.pa_decode_append(d["out"], d["q"], d["k_new"], d["v_new"], d["slot_mapping"],
                        d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                        float(w.scale), w.num_kv_heads, max_context_len=w.max_context_len,
                        num_workers=num_workers, workspace=workspace, shared_blocks=shared_blocks)
    torch.cuda.synchronize()
    return d["out"].cpu().numpy()


def run_fused(w, num_workers=0, label="", shared_blocks=False):
    log(f"fused case {label}: S={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
        f"D={w.head_dim} BS={w.block_size} maxctx={w.max_context_len} workers={num_workers}")
    d = to_device(w)
    out = fused_step(w, d, num_workers, shared_blocks=shared_blocks)
    kc, vc = oracle_pools(w)
    assert_pools_equal(d, kc, vc, label)
    compare(out, oracle_decode(w, kc, vc), label)
    return out


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 4, 64), (32, 8, 128), (8, 8, 128), (12, 4, 128),
                                      (2, 1, 64)])
@pytest.mark.parametrize("workers", [0, 1, 7, 64, 5000])
def test_fused_shapes_and_work_splits(Hq, Hkv, D, workers):
    """workers = 5000: every unit its own share, so a run of length 64k + 1
    ends in a piece holding the new token only; workers = 1: one worker
    stores every row after its last unit."""
    w = wl.make_workload("fused", 300 + Hq + D, Hq, Hkv, D, context_lens=FUSED_LENS)
    run_fused(w, workers, f"fused Hq{Hq} Hkv{Hkv} D{D} workers{workers}")


@pytest.mark.parametrize("BS", [8, 32])
@pytest.mark.parametrize("workers", [0, 5000])
def test_fused_block_sizes(BS, workers):
    w = wl.make_workload("fused-bs", 320 + BS, 32, 8, 128, context_lens=FUSED_LENS, block_size=BS)
    run_fused(w, workers, f"fused BS{BS} workers{workers}")


@pytest.mark.parametrize("n_len,workers", [(4097, 64), (4161, 65), (32769, 512)])
def test_fused_long_run_many_pieces(n_len, workers):
    """One run cut into a piece per worker; its last unit holds the new token
    only, and the piece holding it folds the token in before the merge."""
    w = wl.make_workload("fused-long", 330 + workers, 4, 1, 128, context_lens=[n_len, 5])
    run_fused(w, workers, f"fused run of {n_len} over {workers} workers")


def test_fused_batch_above_one_launch():
    """More sequences than one launch takes: each launch's new rows, slots and
    outputs start at its first sequence.  Pools bit for bit, outputs on both
    launches' sequences."""
    w = wl.make_workload("fused-wide", 347, 2, 1, 64, len_range=(1, 40), num_seqs=4100)
    d = to_device(w)
    out = fused_step(w, d, 0)
    kc, vc = oracle_pools(w)
    assert_pools_equal(d, kc, vc, "fused 4100")
    seqs = np.r_[0:40, 4050:4100]
    compare(out[seqs], oracle_decode(w, kc, vc, seqs), "fused 4100 sequences")


def test_fused_zero_length_rows():
    w = wl.make_workload("fused-zero", 340, 8, 2, 64, context_lens=[0, 1, 0, 65, 0])
    out = run_fused(w, 0, "fused zero rows")
    assert not out[[0, 2, 4]].any()


@pytest.mark.parametrize("shared_blocks", [False, True])
@pytest.mark.parametrize("BS,D", [(16, 128), (16, 64), (8, 128), (8, 64), (32, 128), (32, 64)])
def test_fused_prefix_sharing_with_copies(shared_blocks, BS, D):
    """Copy-on-write before the fused launch: the new token lands in the copy.
    With the shared-blocks flag the prefix pass and the decode's shared
    variant run, at every block size and head dimension."""
    w = wl.make_workload("fused-prefix", 341 + BS + D, 32, 8, D, num_seqs=16, prefix_groups=4,
                         prefix_len=256, suffix_range=(1, 200), block_size=BS)
    assert w.block_mapping.shape[0] > 0 and w.shares_blocks()
    run_fused(w, 0, f"fused prefix BS{BS} D{D} shared={shared_blocks}",
              shared_blocks=shared_blocks)


# Shared-prefix batches (shared-blocks flag): groups of sequences with a
# common prefix are attended to it once by the prefix pass; the decode
# covers the rest and folds both.  (groups, seqs, prefix tokens, suffix
# range): groups across the 8-sequence windows the pass groups in, several
# groups in one window, a prefix that is not a multiple of 64 (the pass
# takes 64 of 96), one-token suffixes, groups of one (nothing shared), a
# prefix in two chunks of 1024 keys and one in four chunks of 1280.
PREFIX_CASES = [(2, 20, 256, (1, 150)), (4, 12, 96, (1, 80)), (3, 24, 1024, (1, 3)),
                (8, 8, 128, (1, 40)), (2, 6, 2048, (100, 700)), (2, 6, 5120, (1, 64))]


@pytest.mark.parametrize("groups,seqs,plen,suffix", PREFIX_CASES)
@pytest.mark.parametrize("workers", [0, 1, 5000])
def test_fused_shared_prefix_groups(groups, seqs, plen, suffix, workers):
    w = wl.make_workload("prefix-groups", 350 + groups + seqs + plen, 16, 4, 128, num_seqs=seqs,
                         prefix_groups=groups, prefix_len=plen, suffix_range=suffix)
    run_fused(w, workers, f"prefix groups {groups}x{seqs // groups} P{plen} workers{workers}",
              shared_blocks=True)


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 8, 64), (8, 4, 128), (32, 8, 64)])
@pytest.mark.parametrize("scale", [None, -0.3])
def test_fused_shared_prefix_shapes(Hq, Hkv, D, scale):
    """MHA, G = 2 and G = 4, both head dims; a negative scale (the prefix
    pass flips q's sign)."""
    w = wl.make_workload("prefix-shapes", 360 + Hq + Hkv + D, Hq, Hkv, D, num_seqs=18,
                         prefix_groups=3, prefix_len=512, suffix_range=(1, 300), scale=scale)
    run_fused(w, 0, f"prefix shapes Hq{Hq} Hkv{Hkv} D{D} scale{scale}", shared_blocks=True)


def test_fused_padding_slot_attends_but_does_not_store():
    """slot < 0: the row enters the attention but the pools keep their bits."""
    w = wl.make_workload("fused-pad", 342, 8, 2, 128, context_lens=[70, 3, 200, 64])
    d = to_device(w)
    pad = w.slot_mapping.copy()
    pad[[1, 3]] = -1
    d["slot_mapping"] = torch.from_numpy(pad).cuda()
    out = fused_step(w, d, 0)
    # pools: the oracle's append with the padded slots
    kc, vc = oracle.copy_blocks(w.k_cache, w.v_cache, w.block_mapping, w.num_kv_heads,
                                w.head_dim, block_size=w.block_size)
    kc, vc = oracle.reshape_and_cache(w.k_new, w.v_new, kc, vc, pad, block_size=w.block_size)
    assert_pools_equal(d, kc, vc, "fused pad")
    # attention: every new row at its position, as with the true slots
    kt, vt = oracle_pools(w)
    compare(out, oracle_decode(w, kt, vt), "fused pad")


def test_fused_matches_separate_calls_bit_for_bit():
    """Append then decode (two launches) against the fused launch, same
    workers: the pools are identical, and the outputs agree to the
    tolerance (the new token's weight enters in fp32 in the fused path)."""
    w = wl.make_workload("fused-vs", 343, 32, 8, 128, len_range=(1, 900), num_seqs=24)
    d1, d2 = to_device(w), to_device(w)
    a = gpu_step(w, d1, 64)
    b = fused_step(w, d2, 64)
    # bit patterns (the unaddressed tail slots hold NaN canaries)
    for pool in ("k_cache", "v_cache"):
        assert torch.equal(d1[pool].view(torch.int16), d2[pool].view(torch.int16)), pool
    kc, vc = oracle_pools(w)
    ref = oracle_decode(w, kc, vc)
    compare(a, ref, "separate")
    compare(b, ref, "fused")


def test_fused_and_plain_share_a_workspace():
    """Alternating fused and plain calls of different shapes on one workspace:
    every call leaves the arrival counters at zero."""
    big = wl.make_workload("fused-ws1", 344, 32, 8, 128, len_range=(100, 3000), num_seqs=40)
    small = wl.make_workload("fused-ws2", 345, 8, 2, 64, context_lens=FUSED_LENS)
    n = max(pk.pa_decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                        w.max_context_len, 64)
            for w in (big, small))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for w, fused in ((big, True), (small, False), (small, True), (big, False)):
        d = to_device(w)
        out = fused_step(w, d, 64, ws) if fused else gpu_step_ws(w, d, ws)
        kc, vc = oracle_pools(w)
        compare(out, oracle_decode(w, kc, vc), f"{w.name} fused={fused}")
        control = decode_control_bytes(w.num_seqs, w.num_kv_heads)
        assert not ws[len(ws) - control:].any()


def gpu_step_ws(w, d, ws):
    pk.pa_reshape_and_cache(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"])
    pk.pa_decode(d["out"], d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                 d["context_lens"], float(w.scale), w.num_kv_heads,
                 max_context_len=w.max_context_len, num_workers=64, workspace=ws)
    torch.cuda.synchronize()
    return d["out"].cpu().numpy()


def test_fused_errors():
    w = wl.make_workload("fused-err", 346, 8, 2, 64, context_lens=[5, 9])
    d = to_device(w)
    L = pk.lib()
    # null new rows
    code = L.pa_decode_append(d["out"].data_ptr(), d["q"].data_ptr(), None, d["v_new"].data_ptr(),
                              d["slot_mapping"].data_ptr(), d["k_cache"].data_ptr(),
                              d["v_cache"].data_ptr(), d["block_tables"].data_ptr(),
                              d["context_lens"].data_ptr(), 0.125, 2, 2, 8, 64, 16,
                              int(w.block_tables.shape[1]), int(w.num_blocks), w.max_context_len,
                              0, 0, None, 0, None)
    assert code == pk.PA_ERR_INVALID_ARG
    # a misaligned K row buffer
    kn = torch.empty(d["k_new"].numel() + 1, dtype=torch.float16, device="cuda")
    ws = pk.new_workspace(2, 8, 2, 64, w.max_context_len)
    code = L.pa_decode_append(d["out"].data_ptr(), d["q"].data_ptr(), kn.data_ptr() + 2,
                              d["v_new"].data_ptr(), d["slot_mapping"].data_ptr(),
                              d["k_cache"].data_ptr(), d["v_cache"].data_ptr(),
                              d["block_tables"].data_ptr(), d["context_lens"].data_ptr(), 0.125, 2,
                              2, 8, 64, 16, int(w.block_tables.shape[1]), int(w.num_blocks),
                              w.max_context_len, 0, 0, ws.data_ptr(), ws.numel(), None)
    assert code == pk.PA_ERR_INVALID_ARG
    # an unknown flag bit
    code = L.pa_decode_append(d["out"].data_ptr(), d["q"].data_ptr(), d["k_new"].data_ptr(),
                              d["v_new"].data_ptr(), d["slot_mapping"].data_ptr(),
                              d["k_cache"].data_ptr(), d["v_cache"].data_ptr(),
                              d["block_tables"].data_ptr(), d["context_lens"].data_ptr(), 0.125, 2,
                              2, 8, 64, 16, int(w.block_tables.shape[1]), int(w.num_blocks),
                              w.max_context_len, 0, 2, ws.data_ptr(), ws.numel(), None)
    assert code == pk.PA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["llama8b_b64", "prefix_b256", "opt13b_b128", "longctx_b16",
                                  "llama70b_b64", "g12_b64", "llama405b_b64", "mqa_b512"])
def test_fused_full_size(name):
    """The benchmark's batches in its launch configuration (automatic worker
    count, the shared-blocks flag where blocks are shared): pools bit for bit,
    outputs on every sequence."""
    w = named(name)
    d = to_device(w)
    out = fused_step(w, d, 0, shared_blocks=w.shares_blocks())  # as the benchmark runs it
    kc, vc = oracle_pools(w)
    assert_pools_equal(d, kc, vc, name)
    log(f"{name}: oracle decode on all {w.num_seqs} sequences")
    compare(out, oracle_decode(w, kc, vc), name)
