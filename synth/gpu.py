"""ctypes wrapper of libsynth.so: GPU fills of the seeded synthetic inputs
(definition in synth/__init__.py), the benchmark's HBM calibration probes
(plain read, write and copy), and streams restricted to a set of compute
units."""
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
        L.synth_probe_copy_capped.restype = ctypes.c_int
        L.synth_probe_copy_capped.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_void_p]
        L.synth_cu_count.restype = ctypes.c_int
        L.synth_cu_count.argtypes = [ctypes.POINTER(ctypes.c_int)]
        L.synth_stream_create_cu_masked.restype = ctypes.c_int
        L.synth_stream_create_cu_masked.argtypes = [ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32),
                                                    ctypes.POINTER(ctypes.c_void_p)]
        L.synth_elastic_compute.restype = ctypes.c_int
        L.synth_elastic_compute.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.synth_stream_destroy.restype = ctypes.c_int
        L.synth_stream_destroy.argtypes = [ctypes.c_void_p]
        L.synth_fill.restype = ctypes.c_int
        L.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64,
                                 ctypes.c_uint64, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_int, ctypes.c_void_p]
        _lib = L
    return _lib


def fill(addr: int, dt: int, n: int, key: int, pos_base: int, sigma: float, stream: int,
         mix: bool = False, sel_key: int = 0, nt: bool = False) -> None:
    """Fill n elements at device address addr with the values at flat
    positions pos_base .. pos_base + n - 1 (nt: with non-temporal stores)."""
    if n <= 0:
        return
    err = load().synth_fill(ctypes.c_void_p(addr), dt, n, key, sel_key, 1 if mix else 0, pos_base,
                            ctypes.c_float(float(scale_for(sigma))), 1 if nt else 0, ctypes.c_void_p(stream))
    if err != 0:
        raise RuntimeError(f"synth_fill failed with HIP error {err}")


PROBE_READ, PROBE_WRITE, PROBE_COPY, PROBE_READ_CACHED = 0, 1, 2, 3


def probe_sink_words(nbytes: int) -> int:
    """Words of sink memory the read probe of nbytes writes (one per workgroup)."""
    return int(load().synth_probe_sink_words(nbytes))


def probe(kind: int, dst: int, src: int, nbytes: int, sink: int, stream: int) -> None:
    """One calibration launch: read nbytes at src (non-temporal loads, or
    cached loads with PROBE_READ_CACHED), write nbytes at dst, or copy nbytes
    from src to dst (16-byte aligned, nbytes a multiple of 16)."""
    err = load().synth_probe(kind, ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, ctypes.c_void_p(sink),
                             ctypes.c_void_p(stream))
    if err != 0:
        raise RuntimeError(f"synth_probe({kind}) failed with HIP error {err}")


def probe_copy_capped(dst: int, src: int, nbytes: int, max_blocks: int, stream: int) -> None:
    """The copy probe on a grid of at most max_blocks workgroups, each walking
    the buffer in strides of the grid (a rate-limited background copy)."""
    err = load().synth_probe_copy_capped(ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, max_blocks,
                                         ctypes.c_void_p(stream))
    if err != 0:
        raise RuntimeError(f"synth_probe_copy_capped failed with HIP error {err}")


def cu_count() -> int:
    n = ctypes.c_int(0)
    err = load().synth_cu_count(ctypes.byref(n))
    if err != 0:
        raise RuntimeError(f"synth_cu_count failed with HIP error {err}")
    return n.value


def cu_mask_words(cus, n_cus: int):
    """32-bit mask words with bit i set for every CU index i in cus."""
    words = [0] * ((n_cus + 31) // 32)
    for i in cus:
        if not 0 <= i < n_cus:
            raise ValueError(f"CU {i} outside [0, {n_cus})")
        words[i // 32] |= 1 << (i % 32)
    return words


def balanced_cus(k: int, n_cus: int, n_xcd: int = 8):
    """k CU indices that give every one of the n_xcd dies the same share,
    whether the runtime numbers CUs die by die (index // (n_cus / n_xcd)) or
    round-robin across dies (index % n_xcd): die x takes the indices
    x * per + ((x + j) % n_xcd) + n_xcd * (j // n_xcd) for j < k / n_xcd.
    A kernel's workgroups are split across the dies ahead of time, so a set
    that left a die without CUs would leave that die's workgroups unrun."""
    per = n_cus // n_xcd
    if n_cus % n_xcd or per % n_xcd or k % n_xcd or not 0 < k < n_cus:
        raise ValueError(f"cannot split {k} of {n_cus} CUs evenly over {n_xcd} dies")
    m = k // n_xcd
    return sorted(x * per + (x + j) % n_xcd + n_xcd * (j // n_xcd) for x in range(n_xcd) for j in range(m))


class MaskedStream:
    """A HIP stream whose kernels run only on the given CUs, wrapped as a
    torch external stream (``.torch``).  Default priority."""

    def __init__(self, torch, cus, device=None):
        n = cu_count()
        words = cu_mask_words(cus, n)
        if not any(words):
            raise ValueError("empty CU mask")
        arr = (ctypes.c_uint32 * len(words))(*words)
        h = ctypes.c_void_p()
        err = load().synth_stream_create_cu_masked(len(words), arr, ctypes.byref(h))
        if err != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed with HIP error {err}")
        self.handle = h.value
        self.cus = sorted(set(cus))
        self.torch = torch.cuda.ExternalStream(self.handle, device=device)

    def close(self):
        if self.handle:
            self.torch.synchronize()
            load().synth_stream_destroy(ctypes.c_void_p(self.handle))
            self.handle = None


def elastic_compute(w_addr: int, n: int, iters: int, blocks: int, out_addr: int, stream: int,
                    lds_bytes: int = 4) -> None:
    """The elastic compute stand-in of the Stage-3 prefetch study (see
    streams.hip): `blocks` workgroups, each thread `iters` dependent FMAs on a
    16-bit weight of the n at w_addr, each workgroup holding lds_bytes of LDS;
    one float per workgroup to out_addr."""
    err = load().synth_elastic_compute(ctypes.c_void_p(w_addr), n, iters, blocks, lds_bytes,
                                       ctypes.c_void_p(out_addr), ctypes.c_void_p(stream))
    if err != 0:
        raise RuntimeError(f"synth_elastic_compute failed with HIP error {err}")
