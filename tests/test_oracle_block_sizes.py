"""Pins of the oracle at block sizes 8 and 32 (next to the default 16) and of
the swap copy.  The test lays out the same logical K/V itself, from the ABI's
element formulas, at each block size: decode and prefill must not depend on
the block size (equal up to the last bits of fp64, where BLAS may sum in a
different order for differently aligned buffers), and must match brute
force."""
import numpy as np
import pytest

import oracle
from tests.test_oracle import brute_force


def k_flat(b, h, o, d, Hkv, D, BS):
    return ((((b * Hkv + h) * (D // 8) + d // 8) * BS + o) * 8) + d % 8


def v_flat(b, h, o, d, Hkv, D, BS):
    return ((((b * Hkv + h) * (BS // 8) + o // 8) * D + d) * 8) + o % 8


def scatter(k_log, v_log, lens, Hkv, D, BS, rng, fill=np.nan):
    """Pools and tables holding each sequence's contiguous K/V [n, Hkv, D] at
    block size BS, blocks placed by a seeded permutation."""
    nbs = [-(-n // BS) for n in lens]
    NB = sum(nbs) + 3
    perm = rng.permutation(NB)
    kf = np.full(NB * Hkv * BS * D, fill, dtype=np.float16)
    vf = np.full(NB * Hkv * BS * D, fill, dtype=np.float16)
    tab = np.full((len(lens), max(max(nbs), 1)), -1, dtype=np.int32)
    dd = np.arange(D)
    at = 0
    for s, n in enumerate(lens):
        row = perm[at:at + nbs[s]]
        at += nbs[s]
        tab[s, :len(row)] = row
        for pos in range(n):
            b, o = int(row[pos // BS]), pos % BS
            for h in range(Hkv):
                kf[k_flat(b, h, o, dd, Hkv, D, BS)] = k_log[s][pos, h]
                vf[v_flat(b, h, o, dd, Hkv, D, BS)] = v_log[s][pos, h]
    return kf.reshape(NB, Hkv, D // 8, BS, 8), vf.reshape(NB, Hkv, BS // 8, D, 8), tab


def test_decode_independent_of_block_size_and_matches_brute_force():
    rng = np.random.default_rng(5)
    Hq, Hkv, D = 8, 2, 16
    lens = [1, 7, 8, 9, 31, 32, 33, 70]
    kl = [rng.standard_normal((n, Hkv, D), dtype=np.float32).astype(np.float16) for n in lens]
    vl = [rng.standard_normal((n, Hkv, D), dtype=np.float32).astype(np.float16) for n in lens]
    q = rng.standard_normal((len(lens), Hq, D), dtype=np.float32).astype(np.float16)
    la = np.asarray(lens, np.int32)
    outs = []
    for BS in (8, 16, 32):
        kc, vc, tab = scatter(kl, vl, lens, Hkv, D, BS, np.random.default_rng(BS))
        outs.append(oracle.decode(q, kc, vc, tab, la, np.float32(0.3), Hkv, block_size=BS))
    assert np.abs(outs[0] - outs[1]).max() < 1e-13 and np.abs(outs[1] - outs[2]).max() < 1e-13
    assert np.abs(outs[0] - brute_force(q, kl, vl, np.float32(0.3), Hkv)).max() < 1e-12


def test_prefill_independent_of_block_size():
    rng = np.random.default_rng(6)
    Hq, Hkv, D = 4, 1, 16
    lens, nqs = [20, 41, 64], [20, 9, 33]
    kl = [rng.standard_normal((n, Hkv, D), dtype=np.float32).astype(np.float16) for n in lens]
    vl = [rng.standard_normal((n, Hkv, D), dtype=np.float32).astype(np.float16) for n in lens]
    starts = np.concatenate([[0], np.cumsum(nqs)]).astype(np.int32)
    q = rng.standard_normal((int(starts[-1]), Hq, D), dtype=np.float32).astype(np.float16)
    outs = []
    for BS in (8, 16, 32):
        kc, vc, tab = scatter(kl, vl, lens, Hkv, D, BS, np.random.default_rng(BS + 1))
        outs.append(oracle.prefill(q, kc, vc, tab, np.asarray(lens, np.int32), starts,
                                   np.float32(0.25), Hkv, block_size=BS))
    assert np.abs(outs[0] - outs[1]).max() < 1e-13 and np.abs(outs[1] - outs[2]).max() < 1e-13


@pytest.mark.parametrize("BS", [8, 32])
def test_append_writes_exactly_its_slots(BS):
    """Hand-computed flat indices: the append touches exactly the slot's
    elements, at block size BS."""
    rng = np.random.default_rng(BS)
    Hkv, D, NB = 2, 16, 5
    kc = rng.standard_normal((NB, Hkv, D // 8, BS, 8), dtype=np.float32).astype(np.float16)
    vc = rng.standard_normal((NB, Hkv, BS // 8, D, 8), dtype=np.float32).astype(np.float16)
    kn = rng.standard_normal((3, Hkv, D), dtype=np.float32).astype(np.float16)
    vn = rng.standard_normal((3, Hkv, D), dtype=np.float32).astype(np.float16)
    slots = np.array([BS * 3 + BS - 1, -1, BS * 1 + 5], dtype=np.int64)
    k2, v2 = oracle.reshape_and_cache(kn, vn, kc, vc, slots, block_size=BS)
    ek, ev = kc.reshape(-1).copy(), vc.reshape(-1).copy()
    dd = np.arange(D)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        b, o = divmod(int(s), BS)
        for h in range(Hkv):
            ek[k_flat(b, h, o, dd, Hkv, D, BS)] = kn[t, h]
            ev[v_flat(b, h, o, dd, Hkv, D, BS)] = vn[t, h]
    assert np.array_equal(k2.reshape(-1).view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(v2.reshape(-1).view(np.uint16), ev.view(np.uint16))


@pytest.mark.parametrize("BS", [8, 16, 32])
def test_swap_copies_whole_blocks_between_pools(BS):
    rng = np.random.default_rng(40 + BS)
    Hkv, D = 2, 16
    sk = rng.standard_normal((6, Hkv, D // 8, BS, 8), dtype=np.float32).astype(np.float16)
    sv = rng.standard_normal((6, Hkv, BS // 8, D, 8), dtype=np.float32).astype(np.float16)
    dk = rng.standard_normal((4, Hkv, D // 8, BS, 8), dtype=np.float32).astype(np.float16)
    dv = rng.standard_normal((4, Hkv, BS // 8, D, 8), dtype=np.float32).astype(np.float16)
    pairs = np.array([[5, 0], [2, 3], [7, 1], [1, 9]], dtype=np.int64)   # last two out of range
    k2, v2 = oracle.swap_blocks(sk, sv, dk, dv, pairs, Hkv, D, block_size=BS)
    ek, ev = dk.copy(), dv.copy()
    ek[0], ev[0] = sk[5], sv[5]          # whole (block, all heads) tiles
    ek[3], ev[3] = sk[2], sv[2]
    assert np.array_equal(k2.view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(v2.view(np.uint16), ev.view(np.uint16))
