"""Paged KV-cache decode path for AMD Instinct MI355X (gfx950).

The compute lives in ``libpagedkv.so`` (hand-written HIP kernels behind a C
ABI, ``include/pa.h``); ``binding`` is its thin ctypes wrapper and
``workloads`` builds seeded synthetic decode-step inputs.
"""
from .binding import (  # noqa: F401
    PagedKVError,
    pa_copy_blocks,
    pa_decode,
    pa_decode_num_workers,
    pa_decode_workspace_size,
    pa_reshape_and_cache,
    pa_strerror,
    pa_version,
    new_workspace,
)

__all__ = [
    "PagedKVError", "pa_copy_blocks", "pa_decode", "pa_decode_num_workers",
    "pa_decode_workspace_size", "pa_reshape_and_cache", "pa_strerror", "pa_version",
    "new_workspace",
]
