"""Binding of libpkv_probe.so (include/pkv_probe.h): read-bandwidth and
matrix-core probes, a measurement aid beside the library.  Argument
marshalling only."""
from __future__ import annotations

import ctypes
import os

from . import _stream_ptr

PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv_probe.so")
SIGNATURES = {
    "pkv_probe_stream_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_void_p]),
    "pkv_probe_slab_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int32,
                                           ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]),
    "pkv_probe_mfma_f16": (ctypes.c_int, [ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                          ctypes.c_void_p]),
}
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(PATH):
            raise RuntimeError(f"{PATH} is missing; build it with `python -m paged_kv_cache_pkv_amd.build`")
        L = ctypes.CDLL(PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _ok(rc):
    if rc != 0:
        raise RuntimeError(f"probe call failed ({rc})")


def stream_read(src, sink, nontemporal=True, stream=None):
    """Read the whole device tensor `src` once (its bytes a multiple of 16)."""
    _ok(lib().pkv_probe_stream_read(ctypes.c_void_p(src.data_ptr()), src.numel() * src.element_size(),
                                    ctypes.c_void_p(sink.data_ptr()), int(bool(nontemporal)), _stream_ptr(stream)))


def slab_read(base, slab_index, slab_bytes, sink, nontemporal=True, stream=None):
    """Read slabs slab_index[i] (a device int32 tensor) of slab_bytes each from the device tensor `base`."""
    _ok(lib().pkv_probe_slab_read(ctypes.c_void_p(base.data_ptr()), base.numel() * base.element_size(),
                                  ctypes.c_void_p(slab_index.data_ptr()), int(slab_index.numel()), int(slab_bytes),
                                  ctypes.c_void_p(sink.data_ptr()), int(bool(nontemporal)), _stream_ptr(stream)))


def mfma_f16(iters, sink, stream=None):
    """Queue the matrix-core probe; returns the launch's floating-point operations."""
    flops = ctypes.c_double(0.0)
    _ok(lib().pkv_probe_mfma_f16(int(iters), ctypes.c_void_p(sink.data_ptr()), ctypes.byref(flops),
                                 _stream_ptr(stream)))
    return flops.value
