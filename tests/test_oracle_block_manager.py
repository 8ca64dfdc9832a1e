"""Pins of the block-manager model (oracle/block_manager.py) against the pages:
their printed numbers and figures, the prefix-key rules they state, published
hash test vectors, and invariants that any correct state must satisfy."""
import json
import os

import numpy as np
import pytest

from oracle import block_manager as obm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden():
    with open(os.path.join(GOLDEN, "page_numbers.json")) as f:
        return json.load(f)


def check_invariants(m: obm.BlockManagerModel):
    """Reference counts equal the number of table entries naming each block;
    the free queue is exactly the unreferenced blocks; the key maps agree."""
    counts = [0] * m.num_blocks
    for r in m.requests.values():
        for b in r.blocks:
            counts[b] += 1
    assert counts == m.refcount
    assert set(m.free) == {b for b in range(m.num_blocks) if m.refcount[b] == 0}
    assert len(m.free) == len(set(m.free))
    for k, b in m.block_of.items():
        assert m.key_of[b] == k
    assert len(m.key_of) == len(m.block_of)


# ---------------------------------------------------------------------------
# hashes: published test vectors
# ---------------------------------------------------------------------------

# FIPS 180-2, appendix B.2: the 448-bit two-block message and its SHA-256 digest
_FIPS_B2_MSG = b"abcdbcdecdefdefgefghfghighijhijkijkljklmklmnlmnomnopnopq"
_FIPS_B2_DIGEST = "248d6a61d20638b8e5c026930c3e6039a33ce45964ff2167f6ecedd419db06c1"


def _as_tokens(data: bytes):
    """The int32 token ids whose little-endian bytes are ``data``."""
    return [int.from_bytes(data[i:i + 4], "little", signed=True) for i in range(0, len(data), 4)]


def test_sha256_block_key_byte_layout_against_published_digest():
    """The oracle's sha256 block key hashes exactly parent key || token ids
    as little-endian int32 || extra bytes: the 56-byte FIPS message cut into
    (parent, tokens, extra) three ways must give the published digest."""
    m = _FIPS_B2_MSG
    assert obm.block_key(b"", _as_tokens(m)).hex() == _FIPS_B2_DIGEST
    assert obm.block_key(m[:32], _as_tokens(m[32:])).hex() == _FIPS_B2_DIGEST
    assert obm.block_key(m[:8], _as_tokens(m[8:48]), m[48:]).hex() == _FIPS_B2_DIGEST


def test_fnv1a64_reference_vectors():
    """FNV-1a 64-bit of '', 'a' and 'foobar' (the FNV reference test values)."""
    assert obm.fnv1a64(b"") == 0xCBF29CE484222325
    assert obm.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert obm.fnv1a64(b"foobar") == 0x85944171F73967E8


# ---------------------------------------------------------------------------
# prefix keys (ttlab section 4; aquanode "Prefix caching")
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", [obm.HASH_SHA256, obm.HASH_FNV1A64])
def test_same_tokens_after_different_prefix_have_different_keys(kind):
    toks = list(range(16))
    k0a = obm.block_key(obm.ZERO_KEY, list(range(100, 116)), b"", kind)
    k0b = obm.block_key(obm.ZERO_KEY, list(range(200, 216)), b"", kind)
    assert obm.block_key(k0a, toks, b"", kind) != obm.block_key(k0b, toks, b"", kind)
    assert obm.block_key(k0a, toks, b"", kind) == obm.block_key(k0a, toks, b"", kind)


def test_extra_keys_isolate_tenants():
    """A different cache salt (extra key) gives no hit on the same tokens."""
    m = obm.BlockManagerModel(64)
    toks = list(range(100))
    assert m.add_request("a", toks, b"salt-1") == 0
    assert m.add_request("b", toks, b"salt-2") == 0
    assert m.add_request("c", toks, b"salt-1") == 96          # 6 full blocks
    check_invariants(m)


def test_only_full_blocks_are_cached():
    m = obm.BlockManagerModel(16)
    m.add_request("a", list(range(20)))                       # one full block + 4 tokens
    assert m.num_cached() == 1
    assert m.add_request("b", list(range(20))) == 16          # the 4-token tail is recomputed
    check_invariants(m)


def test_page_prefix_example():
    """aquanode "Prefix caching": a 2,100-token prompt holds 131 full blocks
    (2,096 tokens); another with the same first 2,000 tokens finds 125 of
    them and has about 100 tokens left to prefill."""
    g = golden()["prefix_example"]
    m = obm.BlockManagerModel(400)
    rng = np.random.default_rng(1)
    shared = rng.integers(0, 32000, size=g["shared_prefix_tokens"]).tolist()
    a = shared + rng.integers(0, 32000, size=g["prompt_tokens"] - len(shared)).tolist()
    b = shared + rng.integers(32000, 64000, size=g["prompt_tokens"] - len(shared)).tolist()
    assert m.add_request("a", a) == 0
    assert m.num_cached() == g["full_blocks"] == g["full_block_tokens"] // 16
    hit = m.add_request("b", b)
    assert hit == g["shared_blocks"] * 16 == g["shared_prefix_tokens"]
    assert g["prompt_tokens"] - hit == g["remaining_prefill_approx"]
    assert m.block_table("a")[:125] == m.block_table("b")[:125]
    assert m.block_table("a")[125] != m.block_table("b")[125]
    check_invariants(m)


def test_worked_example_slots():
    """aquanode "Worked example": 1,000 tokens occupy 1,008 slots."""
    g = golden()["worked_example"]
    m = obm.BlockManagerModel(100)
    m.add_request("r", list(range(g["tokens"])))
    assert len(m.block_table("r")) * 16 == g["slots"]


# ---------------------------------------------------------------------------
# sharing, copy-on-write, freeing and eviction
# ---------------------------------------------------------------------------

def test_shared_prefix_figure():
    """backplane "Prefix caching" figure: A, B, C over one stored P0-P2,
    11 physical blocks, two free; C's suffix blocks return when C ends."""
    m = obm.BlockManagerModel(11)
    prompt = list(range(48))                                 # P0 P1 P2
    m.add_request("A", prompt + list(range(1000, 1032)))     # + A3 A4
    m.add_request("B", prompt + list(range(2000, 2016)))     # + B3
    m.add_request("C", prompt + list(range(3000, 3048)))     # + C3 C4 C5
    t = {r: m.block_table(r) for r in "ABC"}
    assert [len(t[r]) for r in "ABC"] == [5, 4, 6]
    assert t["A"][:3] == t["B"][:3] == t["C"][:3]
    assert m.num_free() == 2
    m.free_request("C")
    assert m.num_free() == 5 and set(t["C"][3:]) <= set(m.free)
    assert all(m.refcount[b] == 2 for b in t["A"][:3])
    check_invariants(m)


def test_finished_request_blocks_taken_by_newcomer():
    """backplane "Static versus continuous batching": B finishes, D takes the
    blocks B released."""
    m = obm.BlockManagerModel(4)
    m.add_request("A", list(range(20)))
    m.add_request("B", list(range(100, 130)))
    b_blocks = m.block_table("B")
    with pytest.raises(obm.PoolExhausted):
        m.add_request("C", list(range(200, 240)))
    assert m.num_free() == 0                                 # the failed admission took nothing
    m.free_request("B")
    m.add_request("D", list(range(300, 325)))
    assert sorted(m.block_table("D")) == sorted(b_blocks)
    check_invariants(m)


def test_tail_blocks_evicted_before_prefix_blocks():
    """ttlab section 4: a finished request's blocks enter the free queue from
    its back, so its tail is evicted before its prefix."""
    m = obm.BlockManagerModel(6)
    toks = list(range(64))                                   # 4 full blocks
    m.add_request("a", toks)
    blocks = m.block_table("a")
    m.free_request("a")
    assert list(m.free)[-4:] == blocks[::-1]                 # tail first
    m.add_request("x", list(range(500, 548)))                # 3 fresh: 2 never used + a's tail
    assert m.num_cached() == 3 + 3                           # a's last block evicted
    assert m.lookup(obm.block_key(obm.ZERO_KEY, toks[:16])) == blocks[0]
    m.free_request("x")
    assert m.add_request("a2", toks) == 48                   # prefix of a still cached
    check_invariants(m)


def test_copy_on_write_after_fork():
    """ttlab "Sharing Blocks": a shared block is copied when a holder appends
    into it; once private, further appends write in place."""
    m = obm.BlockManagerModel(8)
    m.add_request("p", list(range(20)))                      # blocks [x, y], y holds 4 tokens
    m.fork("p", "c")
    x, y = m.block_table("p")
    slot, cow = m.append_token("c", 7)
    assert cow is not None and cow[0] == y and cow[1] != y
    assert slot == cow[1] * 16 + 4
    assert m.block_table("c") == [x, cow[1]] and m.refcount[y] == 1
    slot, cow = m.append_token("p", 9)
    assert cow is None and slot == y * 16 + 4
    check_invariants(m)


def test_block_filled_by_appends_is_cached_with_chained_key():
    m = obm.BlockManagerModel(8)
    toks = list(range(30))
    m.add_request("r", toks[:20])
    for t in toks[20:32 - 2]:
        m.append_token("r", t)
    assert m.num_cached() == 1
    m.append_token("r", 30)
    m.append_token("r", 31)                                  # block 1 now full
    assert m.num_cached() == 2
    k0 = obm.block_key(obm.ZERO_KEY, list(range(16)))
    assert m.lookup(obm.block_key(k0, list(range(16, 30)) + [30, 31])) == m.block_table("r")[1]


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(3)
    m = obm.BlockManagerModel(96, hash_kind=obm.HASH_FNV1A64)
    live, nid = [], 0
    prefixes = [rng.integers(0, 50, size=int(rng.integers(0, 80))).tolist() for _ in range(4)]
    for _ in range(600):
        op = rng.integers(0, 4)
        try:
            if op == 0 or not live:
                toks = prefixes[rng.integers(0, 4)] + rng.integers(0, 50, size=int(rng.integers(1, 40))).tolist()
                m.add_request(nid, toks, b"" if rng.random() < 0.8 else b"s")
                live.append(nid)
                nid += 1
            elif op == 1:
                m.append_token(live[rng.integers(0, len(live))], int(rng.integers(0, 50)))
            elif op == 2:
                m.fork(live[rng.integers(0, len(live))], nid)
                live.append(nid)
                nid += 1
            else:
                m.free_request(live.pop(rng.integers(0, len(live))))
        except obm.PoolExhausted:
            m.free_request(live.pop(0))
        check_invariants(m)
