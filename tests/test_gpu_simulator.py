"""The continuous-batching simulator driving the GPU kernels: every
iteration's copies, appends, prefill chunks, decodes and swaps run on the
device through the C-ABI, and outputs are checked against the oracle's
attention over each request's logical K/V, rebuilt from its tokens alone.
This covers the block manager, prefix reuse, copy-on-write-free recompute
and swap preemption together with the kernels."""
import numpy as np
import pytest

import oracle
from paged_kv_cache_59_amd import simulator as sim
from tests.gpu_util import ABS_TOL, log

pytestmark = pytest.mark.gpu


def oracle_row_error(cfg):
    """Max abs error of a decoded row against the oracle's attention of the
    request's position p, rebuilt from its tokens alone (fp64)."""
    G = cfg.num_q_heads // cfg.num_kv_heads

    def check(req, p, got, scale):
        qkv = [sim.token_tensors(h, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim)
               for h in req.hashes[:p + 1]]
        K = np.stack([x[1] for x in qkv]).astype(np.float64)  # [p + 1, Hkv, D]
        V = np.stack([x[2] for x in qkv]).astype(np.float64)
        q = qkv[-1][0].astype(np.float64)
        sc = np.float64(np.float32(scale))
        return max(float(np.abs(got[h].astype(np.float64)
                                - oracle.attention_one_query(q[h], K[:, h // G], V[:, h // G], sc)).max())
                   for h in range(cfg.num_q_heads))
    return check


@pytest.mark.parametrize("BS,policy", [(16, "recompute"), (16, "swap"), (8, "swap"),
                                       (32, "recompute")])
def test_simulation_on_gpu_matches_oracle(BS, policy):
    # a 320-token pool: requests get preempted and come back
    cfg = sim.Config(num_blocks=320 // BS, block_size=BS, max_running=8, max_batched_tokens=48,
                     margin_blocks=0, preemption=policy, host_blocks=400,
                     num_q_heads=8, num_kv_heads=2, head_dim=64)
    s = sim.Simulator(cfg, gpu=True, check_every=1, check_row=oracle_row_error(cfg))
    out = s.run(sim.synthetic_arrivals(14, 21, 2.0, (20, 90), (20, 60), shared_prefix=40))
    log(f"simulation BS={BS} {policy}: {out}")
    assert out["finished"] == 14
    assert out["preempt_recompute"] + out["preempt_swap"] > 0
    assert out["prefix_hit_tokens"] > 0
    assert out["checked_rows"] > 100
    assert out["max_abs_err"] <= ABS_TOL
