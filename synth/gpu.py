"""ctypes wrapper of libsynth.so: GPU fills of the seeded synthetic inputs
(definition in synth/__init__.py), and the benchmark's HBM calibration
probes (plain read, write and copy)."""
from __future__ import annotations

import ctypes
import os

from . import _build, scale_for

_lib = None


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise ImportError(f"libsynth.so not built at {_build.LIB}")
        import torch  # noqa: F401  -- bind to torch's HIP runtime (see zero_sharded_mixed_02_amd.load)
        L = ctypes.CDLL(_build.LIB)
        L.synth_probe.restype = ctypes.c_int
        L.synth_probe.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_void_p]
        L.synth_probe_sink_words.restype = ctypes.c_int64
        L.synth_probe_sink_words.argtypes = [ctypes.c_int64]
        L.synth_fill.restype = ctypes.c_int
        L.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                 ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_void_p]
        _lib = L
    return _lib


def fill(addr: int, dt: int, n: int, key: int, pos_base: int, sigma: float, stream: int,
         mix: bool = False, sel_key: int = 0) -> None:
    """Fill n elements at device address addr with the values at flat
    positions pos_base .. pos_base + n - 1."""
    if n <= 0:
        return
    err = load().synth_fill(ctypes.c_void_p(addr), dt, n, key, sel_key, 1 if mix else 0, pos_base,
                            ctypes.c_float(float(scale_for(sigma))), ctypes.c_void_p(stream))
    if err != 0:
        raise RuntimeError(f"synth_fill failed with HIP error {err}")


PROBE_READ, PROBE_WRITE, PROBE_COPY = 0, 1, 2


def probe_sink_words(nbytes: int) -> int:
    """Words of sink memory the read probe of nbytes writes (one per workgroup)."""
    return int(load().synth_probe_sink_words(nbytes))


def probe(kind: int, dst: int, src: int, nbytes: int, sink: int, stream: int) -> None:
    """One calibration launch: read nbytes at src, write nbytes at dst, or
    copy nbytes from src to dst (16-byte aligned, nbytes a multiple of 16)."""
    err = load().synth_probe(kind, ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, ctypes.c_void_p(sink),
                             ctypes.c_void_p(stream))
    if err != 0:
        raise RuntimeError(f"synth_probe({kind}) failed with HIP error {err}")
