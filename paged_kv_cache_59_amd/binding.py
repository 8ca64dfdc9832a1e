"""Thin ctypes binding of ``libpagedkv.so`` (argument marshalling only).

Each function has the name of the C entry point it calls (declared in
``include/pa.h``), takes torch tensors that already live on the GPU, checks
dtypes, shapes and contiguity, and passes raw device pointers, sizes and the
current HIP stream.  All computation happens in the library's kernels; there
is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")
_lib = None
# PA_LIBRARY_VARIANT=<variant> loads a measurement build instead (the test
# suite run against it: see use_variant_library)
if os.environ.get("PA_LIBRARY_VARIANT"):
    _LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                             f"libpagedkv_{os.environ['PA_LIBRARY_VARIANT']}.so")

PA_OK = 0
PA_ERR_INVALID_ARG = -1
PA_ERR_UNSUPPORTED = -2
PA_ERR_WORKSPACE = -3
PA_ERR_HIP = -4
PA_ERR_SCRATCH_LIMIT = -5
BLOCK_SIZE = 16

EXPORTED = ("pa_reshape_and_cache", "pa_copy_blocks", "pa_swap_blocks", "pa_decode",
            "pa_decode_timed", "pa_decode_append", "pa_decode_append_timed",
            "pa_decode_append_noalloc", "pa_read_probe",
            "pa_prefill", "pa_decode_workspace_size",
            "pa_decode_num_workers", "pa_strerror", "pa_version")


def use_variant_library(variant: str) -> None:
    """Load a measurement build, libpagedkv_<variant>.so (the same entry
    points; "trace": the decode kernel also writes per-worker timestamps at
    the start of its workspace; "valu": it forms q.K and P.V on the vector
    ALUs), instead of libpagedkv.so.  Call before the first call into the
    library."""
    global _LIB_PATH
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"libpagedkv_{variant}.so")
    if _lib is not None and _LIB_PATH != path:
        raise RuntimeError("the library is already loaded")
    _LIB_PATH = path


def use_trace_library() -> None:
    use_variant_library("trace")


TRACE_SLOTS = 32  # per-worker 64-bit words the measurement build writes


class PagedKVError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {pa_strerror(code)} ({code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """The loaded library, with argument and return types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with `python -m paged_kv_cache_59_amd.build` "
            "(there is no fallback path)")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.pa_reshape_and_cache.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i64, vp]
    L.pa_reshape_and_cache.restype = ctypes.c_int
    L.pa_copy_blocks.argtypes = [vp, vp, vp, i64, i32, i32, i32, i64, vp]
    L.pa_copy_blocks.restype = ctypes.c_int
    L.pa_swap_blocks.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i32, i64, i64, vp]
    L.pa_swap_blocks.restype = ctypes.c_int
    L.pa_decode_num_workers.argtypes = []
    L.pa_decode_num_workers.restype = i32
    L.pa_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    L.pa_decode_workspace_size.restype = sz
    L.pa_decode.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, i32, i32, i32,
                            i32, i64, i32, i32, vp, sz, vp]
    L.pa_decode.restype = ctypes.c_int
    L.pa_decode_timed.argtypes = L.pa_decode.argtypes + [vp, vp]
    L.pa_decode_timed.restype = ctypes.c_int
    L.pa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, i32,
                                   i32, i32, i32, i32, i64, i32, i32, ctypes.c_uint32, vp, sz, vp]
    L.pa_decode_append.restype = ctypes.c_int
    L.pa_decode_append_timed.argtypes = L.pa_decode_append.argtypes + [vp, vp]
    L.pa_decode_append_timed.restype = ctypes.c_int
    # pa_decode_append without the workspace pointer and size
    L.pa_decode_append_noalloc.argtypes = L.pa_decode_append.argtypes[:20] + [vp]
    L.pa_decode_append_noalloc.restype = ctypes.c_int
    L.pa_read_probe.argtypes = [vp, i64, vp, i64, i32, vp, vp, vp, vp]
    L.pa_read_probe.restype = ctypes.c_int
    L.pa_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, ctypes.c_float, i32, i32, i32, i32,
                             i32, i32, i64, i32, i32, vp]
    L.pa_prefill.restype = ctypes.c_int
    L.pa_strerror.argtypes = [ctypes.c_int]
    L.pa_strerror.restype = ctypes.c_char_p
    L.pa_version.argtypes = []
    L.pa_version.restype = ctypes.c_int
    _lib = L
    return L


def pa_strerror(code: int) -> str:
    return lib().pa_strerror(int(code)).decode()


def pa_version() -> int:
    return int(lib().pa_version())


def _check(code: int, what: str) -> None:
    if code != PA_OK:
        raise PagedKVError(code, what)


def _dev(t: torch.Tensor, name: str, dtype) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(t: torch.Tensor, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _cache_geometry(k_cache: torch.Tensor, v_cache: torch.Tensor):
    """(num_blocks, num_kv_heads, head_dim, block_size) of a K/V pool pair."""
    if k_cache.dim() != 5 or k_cache.shape[4] != 8:
        raise ValueError("k_cache must be [num_blocks, num_kv_heads, head_dim/8, block_size, 8]")
    nb, hkv, d8, bs = k_cache.shape[:4]
    d = d8 * 8
    if bs % 8 or tuple(v_cache.shape) != (nb, hkv, bs // 8, d, 8):
        raise ValueError("v_cache must be [num_blocks, num_kv_heads, block_size/8, head_dim, 8]")
    return int(nb), int(hkv), int(d), int(bs)


def pa_reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, stream=None) -> None:
    """Write k[t], v[t] ([T, Hkv, D] fp16) into slot slot_mapping[t] (int64)."""
    for t, n in ((k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n, torch.float16)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    T = int(slot_mapping.numel())
    if tuple(k.shape) != (T, hkv, d) or tuple(v.shape) != (T, hkv, d):
        raise ValueError("k and v must be [num_tokens, num_kv_heads, head_dim]")
    code = lib().pa_reshape_and_cache(k.data_ptr(), v.data_ptr(), k_cache.data_ptr(),
                                      v_cache.data_ptr(), slot_mapping.data_ptr(), T, hkv, d,
                                      bs, nb, _stream(k_cache, stream))
    _check(code, "pa_reshape_and_cache")


def pa_copy_blocks(k_cache, v_cache, block_mapping, stream=None) -> None:
    """Copy whole blocks (K and V, all heads) for each (src, dst) row of block_mapping."""
    _dev(k_cache, "k_cache", torch.float16)
    _dev(v_cache, "v_cache", torch.float16)
    _dev(block_mapping, "block_mapping", torch.int64)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [num_pairs, 2]")
    code = lib().pa_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), block_mapping.data_ptr(),
                                int(block_mapping.shape[0]), hkv, d, bs, nb,
                                _stream(k_cache, stream))
    _check(code, "pa_copy_blocks")


def pa_decode_num_workers() -> int:
    """Workers pa_decode uses by default on the current device (2 per CU)."""
    n = int(lib().pa_decode_num_workers())
    _check(min(n, 0), "pa_decode_num_workers")
    return n


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                             num_workers=0) -> int:
    return int(lib().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              max_context_len, num_workers))


def new_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, num_workers=0,
                  device="cuda"):
    """A zero-filled decode workspace (the counters must start at zero)."""
    n = pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                 num_workers)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def decode_status(workspace) -> int:
    """The workspace's status word (its last int32, read after the caller's
    synchronisation): 0, or 1 once a bounded wait between a decode worker's
    waves gave up (that call's results are undefined; zero the workspace
    before reusing it)."""
    n = workspace.numel() // 4 * 4
    return int(workspace[n - 4:n].view(torch.int32).item())


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_kv_heads,
              max_context_len=None, num_workers=0, workspace=None, stream=None,
              kernel_events=None):
    """Paged decode attention; writes out [S, Hq, D] fp16 and returns it.

    ``max_context_len`` is the host-known bound of ``context_lens``; when None
    the table width bound ``max_blocks_per_seq * 16`` is used.  ``workspace``
    is a zero-filled uint8 GPU tensor of pa_decode_workspace_size(...) bytes
    (reusable across calls that do not overlap); when None a fresh one is made.
    ``kernel_events`` = (start, stop) timing-enabled torch.cuda.Events, each
    recorded at least once before (torch creates the HIP event at its first
    record), calls pa_decode_timed: start.elapsed_time(stop) is then the
    kernel's own execution time.
    """
    _dev(out, "out", torch.float16)
    _dev(q, "q", torch.float16)
    _dev(k_cache, "k_cache", torch.float16)
    _dev(v_cache, "v_cache", torch.float16)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    if hkv != int(num_kv_heads):
        raise ValueError("num_kv_heads does not match k_cache")
    S, hq, dq = q.shape
    if dq != d or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [num_seqs, num_q_heads, head_dim]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq], context_lens [num_seqs]")
    mb = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = mb * bs
    if workspace is None:
        workspace = new_workspace(S, hq, hkv, d, int(max_context_len), num_workers, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    if not math.isfinite(float(scale)):
        raise ValueError("scale must be finite")
    args = (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), float(scale), hkv, S, hq, d,
            bs, mb, nb, int(max_context_len), int(num_workers), workspace.data_ptr(),
            workspace.numel(), _stream(q, stream))
    if kernel_events is None:
        _check(lib().pa_decode(*args), "pa_decode")
    else:
        start, stop = kernel_events
        if not start.cuda_event or not stop.cuda_event:
            raise ValueError("kernel_events must have been recorded once (torch creates them lazily)")
        _check(lib().pa_decode_timed(*args, start.cuda_event, stop.cuda_event), "pa_decode_timed")
    return out


PA_DECODE_SHARED_BLOCKS = 1


def pa_decode_append(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                     context_lens, scale, num_kv_heads, max_context_len=None, num_workers=0,
                     workspace=None, stream=None, kernel_events=None, shared_blocks=False):
    """Append each sequence's new token and decode, in one launch: the same
    results as pa_reshape_and_cache(k_new, v_new, k_cache, v_cache,
    slot_mapping) followed by pa_decode(...), when token s is sequence s's
    token at position context_lens[s] - 1 and slot_mapping[s] is that
    position's slot (negative: attended, not stored).  k_new and v_new are
    [num_seqs, Hkv, D] fp16; the other arguments as pa_decode.
    ``shared_blocks``: sequences of the batch share blocks (prefix caching,
    forks); a prefix pass then attends each group of sequences that start
    with the same blocks to their common prefix once, and the decode covers
    the rest (same results up to rounding)."""
    _dev(out, "out", torch.float16)
    _dev(q, "q", torch.float16)
    _dev(k_new, "k_new", torch.float16)
    _dev(v_new, "v_new", torch.float16)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(k_cache, "k_cache", torch.float16)
    _dev(v_cache, "v_cache", torch.float16)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    if hkv != int(num_kv_heads):
        raise ValueError("num_kv_heads does not match k_cache")
    S, hq, dq = q.shape
    if dq != d or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [num_seqs, num_q_heads, head_dim]")
    if tuple(k_new.shape) != (S, hkv, d) or tuple(v_new.shape) != (S, hkv, d):
        raise ValueError("k_new and v_new must be [num_seqs, num_kv_heads, head_dim]")
    if slot_mapping.numel() != S:
        raise ValueError("slot_mapping must be [num_seqs]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq], context_lens [num_seqs]")
    mb = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = mb * bs
    if workspace is None:
        workspace = new_workspace(S, hq, hkv, d, int(max_context_len), num_workers, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    if not math.isfinite(float(scale)):
        raise ValueError("scale must be finite")
    args = (out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
            slot_mapping.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), float(scale), hkv, S, hq, d, bs, mb,
            nb, int(max_context_len), int(num_workers),
            PA_DECODE_SHARED_BLOCKS if shared_blocks else 0, workspace.data_ptr(),
            workspace.numel(), _stream(q, stream))
    if kernel_events is None:
        _check(lib().pa_decode_append(*args), "pa_decode_append")
    else:
        start, stop = kernel_events
        if not start.cuda_event or not stop.cuda_event:
            raise ValueError("kernel_events must have been recorded once (torch creates them lazily)")
        _check(lib().pa_decode_append_timed(*args, start.cuda_event, stop.cuda_event),
               "pa_decode_append_timed")
    return out


def pa_decode_append_noalloc(out, q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables,
                             context_lens, scale, num_kv_heads, max_context_len=None,
                             num_workers=0, stream=None, shared_blocks=False):
    """pa_decode_append without a workspace: the library's own device array
    (32 MiB per GPU) holds the partial results.  Calls that overlap in time
    on one GPU race.  Arguments as pa_decode_append."""
    for t, n in ((out, "out"), (q, "q"), (k_new, "k_new"), (v_new, "v_new"),
                 (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n, torch.float16)
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    if hkv != int(num_kv_heads):
        raise ValueError("num_kv_heads does not match k_cache")
    S, hq, dq = q.shape
    if dq != d or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [num_seqs, num_q_heads, head_dim]")
    if tuple(k_new.shape) != (S, hkv, d) or tuple(v_new.shape) != (S, hkv, d):
        raise ValueError("k_new and v_new must be [num_seqs, num_kv_heads, head_dim]")
    if slot_mapping.numel() != S:
        raise ValueError("slot_mapping must be [num_seqs]")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq], context_lens [num_seqs]")
    mb = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = mb * bs
    if not math.isfinite(float(scale)):
        raise ValueError("scale must be finite")
    code = lib().pa_decode_append_noalloc(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), slot_mapping.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
        float(scale), hkv, S, hq, d, bs, mb, nb, int(max_context_len), int(num_workers),
        PA_DECODE_SHARED_BLOCKS if shared_blocks else 0, _stream(q, stream))
    _check(code, "pa_decode_append_noalloc")
    return out


def pa_read_probe(buf, sink, tile_order=None, tile_bytes=4096, stream=None, kernel_events=None):
    """Read-bandwidth probe: read the uint8 GPU buffer ``buf`` once
    (sequentially, or the tiles of ``tile_bytes`` that the int32 GPU tensor
    ``tile_order`` lists, in that order); the int32 GPU tensor ``sink`` (one
    element, zeroed by the caller) receives the XOR of every 32-bit word
    read.  ``kernel_events`` as in pa_decode."""
    _dev(buf, "buf", torch.uint8)
    _dev(sink, "sink", torch.int32)
    order, n = None, 0
    if tile_order is not None:
        _dev(tile_order, "tile_order", torch.int32)
        order, n = tile_order.data_ptr(), int(tile_order.numel())
    ev = (None, None)
    if kernel_events is not None:
        start, stop = kernel_events
        if not start.cuda_event or not stop.cuda_event:
            raise ValueError("kernel_events must have been recorded once (torch creates them lazily)")
        ev = (start.cuda_event, stop.cuda_event)
    _check(lib().pa_read_probe(buf.data_ptr(), int(buf.numel()), order, n, int(tile_bytes),
                               sink.data_ptr(), _stream(buf, stream), *ev), "pa_read_probe")


def pa_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
               num_kv_heads, max_context_len=None, max_query_len=None, stream=None):
    """Multi-query paged attention (chunked prefill); writes out [T, Hq, D] fp16.

    ``query_start`` is an int32 GPU tensor of num_seqs + 1 row offsets into q;
    each sequence's chunk is the last positions of its context, already
    appended to the cache.  ``max_context_len`` / ``max_query_len`` are
    host-known bounds (defaults: the table width and min(T, that)).
    """
    _dev(out, "out", torch.float16)
    _dev(q, "q", torch.float16)
    _dev(k_cache, "k_cache", torch.float16)
    _dev(v_cache, "v_cache", torch.float16)
    _dev(block_tables, "block_tables", torch.int32)
    _dev(context_lens, "context_lens", torch.int32)
    _dev(query_start, "query_start", torch.int32)
    nb, hkv, d, bs = _cache_geometry(k_cache, v_cache)
    if hkv != int(num_kv_heads):
        raise ValueError("num_kv_heads does not match k_cache")
    T, hq, dq = q.shape
    if dq != d or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [num_tokens, num_q_heads, head_dim]")
    S = int(context_lens.numel())
    if block_tables.dim() != 2 or block_tables.shape[0] != S or query_start.numel() != S + 1:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq], "
                         "query_start [num_seqs + 1]")
    mb = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = mb * bs
    if max_query_len is None:
        max_query_len = min(int(T), int(max_context_len))
    if not math.isfinite(float(scale)):
        raise ValueError("scale must be finite")
    code = lib().pa_prefill(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                            block_tables.data_ptr(), context_lens.data_ptr(),
                            query_start.data_ptr(), int(T), float(scale), hkv, S, hq, d,
                            bs, mb,
                            nb, int(max_context_len), int(max_query_len), _stream(q, stream))
    _check(code, "pa_prefill")
    return out


def _dev_or_pinned(t: torch.Tensor, name: str, dtype) -> None:
    if not isinstance(t, torch.Tensor) or not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a GPU tensor or a pinned host tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def pa_swap_blocks(src_k, src_v, dst_k, dst_v, block_mapping, stream=None) -> None:
    """Copy blocks src -> dst between two pools (one of them may be pinned
    host memory: preemption by swap); block_mapping int64 [P, 2] (src, dst)
    on the GPU or pinned."""
    for t, n in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v")):
        _dev_or_pinned(t, n, torch.float16)
    _dev_or_pinned(block_mapping, "block_mapping", torch.int64)
    snb, hkv, d, bs = _cache_geometry(src_k, src_v)
    dnb, dhkv, dd, dbs = _cache_geometry(dst_k, dst_v)
    if (hkv, d, bs) != (dhkv, dd, dbs):
        raise ValueError("source and destination pools differ in heads, head_dim or block size")
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [num_pairs, 2]")
    dev_t = next((t for t in (src_k, dst_k) if t.is_cuda), None)
    if dev_t is None:
        raise ValueError("one of the pools must be on the GPU")
    code = lib().pa_swap_blocks(src_k.data_ptr(), src_v.data_ptr(), dst_k.data_ptr(),
                                dst_v.data_ptr(), block_mapping.data_ptr(),
                                int(block_mapping.shape[0]), hkv, d, bs, snb, dnb,
                                _stream(dev_t, stream))
    _check(code, "pa_swap_blocks")
