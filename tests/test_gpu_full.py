"""Full-size decode batches on the GPU, in the launch configuration the
benchmark times (automatic worker count), against the oracle.

Pools are compared bit for bit after the copy-on-write and the append; the
attention output is compared on every sequence, or on a sample of sequences
(always including the longest and the shortest) where the oracle would take
too long.
"""
import numpy as np
import pytest

from paged_kv_cache_59_amd import workloads as wl
from tests.gpu_util import (assert_pools_equal, compare, gpu_step, log, oracle_decode,
                            oracle_pools, to_device)

pytestmark = pytest.mark.gpu

SAMPLE = {"llama8b_b64": None, "prefix_b256": None, "longctx_b16": 6, "opt13b_b128": 24}


@pytest.mark.parametrize("name", ["llama8b_b64", "prefix_b256", "longctx_b16", "opt13b_b128"])
def test_full_size_step(name):
    log(f"generating {name}")
    w = wl.make_named(name)
    log(f"{name}: S={w.num_seqs} NB={w.num_blocks} maxctx={w.max_context_len} "
        f"copies={w.block_mapping.shape[0]}")
    d = to_device(w)
    out = gpu_step(w, d, 0)
    log(f"{name}: gpu step done; oracle pools")
    kc, vc = oracle_pools(w)
    assert_pools_equal(d, kc, vc, name)
    n = SAMPLE[name]
    if n is None:
        seqs = np.arange(w.num_seqs)
    else:
        rng = np.random.default_rng(99)
        order = np.argsort(w.context_lens)
        seqs = np.unique(np.concatenate([order[:1], order[-1:],
                                         rng.choice(w.num_seqs, n - 2, replace=False)]))
    log(f"{name}: oracle decode on {len(seqs)} sequences")
    ref = oracle_decode(w, kc, vc, seqs)
    compare(out[seqs], ref, name)
