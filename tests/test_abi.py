"""The C-ABI library on the CPU: it loads, exports what include/*.h declare,
and rejects bad arguments on the host before any HIP call.  Calls here never
reach a kernel launch (no GPU in this container)."""
import ctypes
import os
import re
import subprocess

import pytest

from paged_kv_cache_59_amd import binding
from paged_kv_cache_59_amd import block_manager

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("pa.h", "pa_block_manager.h")]


def declared_functions(headers=HEADERS):
    names = set()
    for h in headers:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_every_header_is_checked():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(
        os.path.basename(h) for h in HEADERS)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding._LIB_PATH):
        pytest.fail("libpagedkv.so is not built (python -m paged_kv_cache_59_amd.build)")
    return binding.lib()


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("pa_reshape_and_cache", "pa_decode", "pa_copy_blocks"):
        assert n in names
    assert set(declared_functions(HEADERS[:1])) == set(binding.EXPORTED)
    assert set(declared_functions(HEADERS[1:])) == set(block_manager.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", binding._LIB_PATH],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name
        assert hasattr(L, name)


def test_version_and_messages(L):
    assert L.pa_version() >= 100
    for code in (0, -1, -2, -3, -4, 7):
        assert L.pa_strerror(code)


NULL = None


def dec(L, **kw):
    args = dict(out=1, q=1, k=1, v=1, tab=1, lens=1, scale=0.125, hkv=8, S=4, hq=32, D=128,
                bs=16, mb=8, nb=100, maxctx=100, workers=64, ws=NULL, wsb=0)
    args.update(kw)
    a = args
    return L.pa_decode(a["out"], a["q"], a["k"], a["v"], a["tab"], a["lens"], a["scale"],
                       a["hkv"], a["S"], a["hq"], a["D"], a["bs"], a["mb"], a["nb"], a["maxctx"],
                       a["workers"], a["ws"], a["wsb"], NULL)


def test_decode_argument_errors(L):
    E = binding
    assert dec(L, hq=30) == E.PA_ERR_INVALID_ARG            # Hq % Hkv != 0
    assert dec(L, D=96) == E.PA_ERR_UNSUPPORTED
    assert dec(L, bs=24) == E.PA_ERR_UNSUPPORTED             # block size not 8, 16 or 32
    # G = 8 and G = 7 (sub-groups): past the argument checks, to the missing workspace
    assert dec(L, hq=64) == E.PA_ERR_WORKSPACE
    assert dec(L, hq=56) == E.PA_ERR_WORKSPACE
    assert dec(L, maxctx=129) == E.PA_ERR_INVALID_ARG        # > 8 blocks * 16
    assert dec(L, S=-1) == E.PA_ERR_INVALID_ARG
    assert dec(L, workers=-3) == E.PA_ERR_INVALID_ARG
    assert dec(L, scale=float("nan")) == E.PA_ERR_INVALID_ARG
    assert dec(L, out=NULL) == E.PA_ERR_INVALID_ARG
    assert dec(L, S=0, out=NULL) == E.PA_OK                  # empty batch: no-op
    # a decode always needs its workspace
    assert dec(L) == E.PA_ERR_WORKSPACE
    need = L.pa_decode_workspace_size(4, 32, 8, 128, 100, 64)
    assert dec(L, ws=256, wsb=need - 1) == E.PA_ERR_WORKSPACE
    assert dec(L, ws=257, wsb=need) == E.PA_ERR_WORKSPACE    # misaligned


def test_workspace_sizes(L):
    # partial slots: one per run (64 x 8) and one per worker, each of 4 rows x
    # (2 + 128) floats, (max, sum) pairs and vectors 256-byte aligned; then
    # the shared-prefix area: prefix lengths (64 ints), and for 4 chunks x 64
    # sequences x 8 KV heads x 4 query heads a log-sum-exp (fp32) and a row of
    # 128 fp16; then one arrival counter per run and 256 bytes ending in the
    # status word
    need = L.pa_decode_workspace_size(64, 32, 8, 128, 2048, 2048)
    slots = 64 * 8 + 2048
    a256 = lambda x: -(-x // 256) * 256
    pre_rows = 4 * 64 * 8 * 4
    assert need == (slots * 8 * 4 + slots * 4 * 128 * 4 + a256(64 * 4) + a256(pre_rows * 4)
                    + a256(pre_rows * 128 * 2) + 64 * 8 * 4 + 256)
    # batches above one launch (4096 sequences) reuse the counters
    assert (L.pa_decode_workspace_size(10000, 32, 8, 128, 100, 64)
            == L.pa_decode_workspace_size(4096, 32, 8, 128, 100, 64))
    assert L.pa_decode_workspace_size(64, 32, 8, 64, 2048, 2048) < need
    assert L.pa_decode_workspace_size(64, 32, 8, 128, 2048, 4096) > need
    # fewer query heads per KV head take the same slots (4 rows each)
    assert L.pa_decode_workspace_size(64, 8, 8, 128, 2048, 2048) == need
    assert L.pa_decode_workspace_size(-1, 32, 8, 128, 100, 16) == 0
    assert L.pa_decode_workspace_size(4, 32, 8, 128, -1, 16) == 0
    assert L.pa_decode_workspace_size(4, 32, 8, 128, 100, -2) == 0
    assert L.pa_decode_workspace_size(4, 30, 8, 128, 100, 16) == 0   # Hq % Hkv != 0
    # a KV head of G = 8 or 7 query heads: 2 sub-groups of up to 4 rows, one
    # copy of the batch each (128 virtual sequences x 8 KV heads), attended
    # in one pass: two share slots per worker
    for hq in (64, 56):
        v = 128 * 8 + 2 * 2048
        pre = 4 * 128 * 8 * 4
        assert L.pa_decode_workspace_size(64, hq, 8, 128, 2048, 2048) == (
            v * 8 * 4 + v * 4 * 128 * 4 + a256(128 * 4) + a256(pre * 4) + a256(pre * 128 * 2)
            + 128 * 8 * 4 + 256)
    # G = 16, 12: 4 or 3 sub-groups (virtual sequences 64 each), attended in
    # one pass: a share slot per worker for each
    for hq, sub in ((128, 4), (96, 3)):
        v = sub * 64 * 8 + sub * 2048
        pre = 4 * sub * 64 * 8 * 4
        assert L.pa_decode_workspace_size(64, hq, 8, 128, 2048, 2048) == (
            v * 8 * 4 + v * 4 * 128 * 4 + a256(sub * 64 * 4) + a256(pre * 4)
            + a256(pre * 128 * 2) + sub * 64 * 8 * 4 + 256)
    # G = 20: 5 sub-groups, rounded up to 8 (two copies of the batch, 4
    # sub-groups per pass): four share slots per worker
    v = 8 * 64 * 8 + 4 * 2048
    pre = 4 * 8 * 64 * 8 * 4
    assert L.pa_decode_workspace_size(64, 160, 8, 128, 2048, 2048) == (
        v * 8 * 4 + v * 4 * 128 * 4 + a256(8 * 64 * 4) + a256(pre * 4) + a256(pre * 128 * 2)
        + 8 * 64 * 8 * 4 + 256)


def test_cache_op_argument_errors(L):
    E = binding
    r = L.pa_reshape_and_cache
    assert r(1, 1, 1, 1, 1, 4, 8, 96, 16, 10, NULL) == E.PA_ERR_UNSUPPORTED
    assert r(1, 1, 1, 1, 1, 4, 8, 128, 24, 10, NULL) == E.PA_ERR_UNSUPPORTED   # block size
    assert r(1, 1, 1, 1, 1, -1, 8, 128, 16, 10, NULL) == E.PA_ERR_INVALID_ARG
    assert r(NULL, 1, 1, 1, 1, 4, 8, 128, 16, 10, NULL) == E.PA_ERR_INVALID_ARG
    assert r(NULL, NULL, NULL, NULL, NULL, 0, 8, 128, 16, 10, NULL) == E.PA_OK
    c = L.pa_copy_blocks
    assert c(1, 1, 1, 2, 8, 64, 16, 0, NULL) == E.PA_ERR_INVALID_ARG
    assert c(1, 1, 1, 2, 8, 80, 16, 10, NULL) == E.PA_ERR_UNSUPPORTED
    assert c(1, NULL, 1, 2, 8, 64, 16, 10, NULL) == E.PA_ERR_INVALID_ARG
    assert c(NULL, NULL, NULL, 0, 8, 64, 16, 10, NULL) == E.PA_OK
    assert c(1, 1, 1, 2, 8, 64, 4, 10, NULL) == E.PA_ERR_UNSUPPORTED
    w = L.pa_swap_blocks
    assert w(1, 2, 3, 4, 5, 2, 8, 64, 12, 10, 10, NULL) == E.PA_ERR_UNSUPPORTED   # block size
    assert w(1, 2, 3, 4, 5, 2, 8, 64, 16, 0, 10, NULL) == E.PA_ERR_INVALID_ARG
    assert w(1, 2, 1, 4, 5, 2, 8, 64, 16, 10, 10, NULL) == E.PA_ERR_INVALID_ARG   # one pool
    assert w(1, 2, 3, 4, NULL, 2, 8, 64, 16, 10, 10, NULL) == E.PA_ERR_INVALID_ARG
    assert w(NULL, NULL, NULL, NULL, NULL, 0, 8, 64, 32, 10, 10, NULL) == E.PA_OK


def test_binding_refuses_cpu_tensors():
    import torch
    t = torch.zeros(4, dtype=torch.float16)
    with pytest.raises(ValueError):
        binding.pa_copy_blocks(t, t, torch.zeros(1, 2, dtype=torch.int64))


def test_noalloc_rejects_a_batch_above_its_array_on_the_host(L):
    """With the worker count given, the size check needs no device: a batch
    whose partial results exceed the library's 32 MiB array is refused
    before any HIP call (the pointers are never dereferenced)."""
    fake = ctypes.c_void_p(0x1000)
    code = L.pa_decode_append_noalloc(fake, fake, fake, fake, fake, fake, fake, fake, fake,
                                      0.125, 64, 256, 64, 128, 16, 4, 1000, 40, 512, 0, None)
    assert code == binding.PA_ERR_SCRATCH_LIMIT
    assert b"static" in L.pa_strerror(code)
