"""Full-size decode batches on the GPU, in the launch configuration the
benchmark times (automatic worker count), against the oracle.

Pools are compared bit for bit after the copy-on-write and the append; the
attention output is compared on every sequence.
"""
import pytest

from tests.gpu_util import (assert_pools_equal, compare, gpu_step, log, named, oracle_decode,
                            oracle_pools, to_device)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["llama8b_b64", "prefix_b256", "longctx_b16", "opt13b_b128"])
def test_full_size_step(name):
    log(f"generating {name}")
    w = named(name)
    log(f"{name}: S={w.num_seqs} NB={w.num_blocks} maxctx={w.max_context_len} "
        f"copies={w.block_mapping.shape[0]}")
    d = to_device(w)
    out = gpu_step(w, d, 0)
    log(f"{name}: gpu step done; oracle pools")
    kc, vc = oracle_pools(w)
    assert_pools_equal(d, kc, vc, name)
    log(f"{name}: oracle decode on all {w.num_seqs} sequences")
    compare(out, oracle_decode(w, kc, vc), name)
