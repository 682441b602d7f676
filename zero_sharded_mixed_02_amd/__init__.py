"""Python binding of libzero.so: one data-parallel rank's share of a ZeRO
mixed-precision training step on an MI355X (gfx950).

Thin ctypes marshalling over the C ABI in ``include/zero.h``: every function
here has the C entry point's name and arguments, converts tensors to device
addresses and streams to ``hipStream_t`` handles, and raises ``ZeroError`` on a
non-OK status.  All computation happens in the HIP kernels of libzero.so; if
the library has not been built, loading fails loudly (there is no fallback).

Tensors may be passed as ``torch.Tensor`` (their ``data_ptr()`` is used) or as
plain integer device addresses.  ``stream=None`` means torch's current stream
on the current device.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libzero.so")

ZERO_F32, ZERO_F16, ZERO_BF16 = 0, 1, 2
ZERO_OK, ZERO_EINVAL, ZERO_EUNSUPPORTED, ZERO_ENOMEM, ZERO_EHIP = 0, -1, -2, -3, -4
ZERO_MAX_RANKS = 128

STATUS_NAMES = {0: "ZERO_OK", -1: "ZERO_EINVAL", -2: "ZERO_EUNSUPPORTED", -3: "ZERO_ENOMEM",
                -4: "ZERO_EHIP"}

# Names of every entry point include/zero.h declares.
ENTRY_POINTS = ("zero_version", "zero_last_error", "zero_plan", "zero_plan_destroy",
                "zero_plan_info", "zero_plan_bucket", "zero_plan_tensor", "zero_flatten",
                "zero_shard_reduce", "zero_adam_step", "zero_gather_pack", "zero_reshard",
                "zero_set_write_window")


class ZeroError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class _AdamHyper(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("grad_scale", ctypes.c_double)]


class _GradSrc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("n", ctypes.c_int32),
                ("ptrs", ctypes.POINTER(ctypes.c_void_p)), ("is_full", ctypes.POINTER(ctypes.c_uint8))]


_lib = None


def _share_torch_hip_runtime():
    """PyTorch brings its own copy of the HIP runtime (same soname as
    /opt/rocm's).  Device memory and streams come from torch, so libzero.so
    must bind to that same runtime: loading torch first makes the dynamic
    loader resolve libzero's libamdhip64.so.7 to torch's already-loaded copy
    instead of opening a second runtime in the process."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def load():
    """Load libzero.so.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libzero.so not built at {LIB_PATH}; run __graft_entry__.build()")
    _share_torch_hip_runtime()
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    p_i64, p_i32 = ctypes.POINTER(i64), ctypes.POINTER(i32)
    L.zero_version.restype = i32
    L.zero_version.argtypes = []
    L.zero_last_error.restype = ctypes.c_char_p
    L.zero_last_error.argtypes = []
    L.zero_plan.restype = i32
    L.zero_plan.argtypes = [i64, i32, p_i64, i32, i64, i32, ctypes.POINTER(vp)]
    L.zero_plan_destroy.restype = None
    L.zero_plan_destroy.argtypes = [vp]
    L.zero_plan_info.restype = i32
    L.zero_plan_info.argtypes = [vp, p_i64, p_i64, p_i32, p_i32]
    L.zero_plan_bucket.restype = i32
    L.zero_plan_bucket.argtypes = [vp, i32, p_i64, p_i64, p_i64, p_i64, p_i64]
    L.zero_plan_tensor.restype = i32
    L.zero_plan_tensor.argtypes = [vp, i32, p_i32, p_i64]
    L.zero_flatten.restype = i32
    L.zero_flatten.argtypes = [vp, ctypes.POINTER(vp), i32, vp, vp]
    L.zero_shard_reduce.restype = i32
    L.zero_shard_reduce.argtypes = [vp, i32, ctypes.POINTER(_GradSrc), ctypes.c_double, vp, vp]
    L.zero_adam_step.restype = i32
    L.zero_adam_step.argtypes = [vp, i32, ctypes.POINTER(_AdamHyper), i64, ctypes.POINTER(_GradSrc),
                                 vp, vp, vp, vp, vp, i32, i32, vp]
    L.zero_gather_pack.restype = i32
    L.zero_gather_pack.argtypes = [vp, ctypes.POINTER(vp), i32, vp, vp]
    L.zero_reshard.restype = i32
    L.zero_reshard.argtypes = [vp, vp, i32, ctypes.POINTER(vp), i32, vp, vp]
    L.zero_set_write_window.restype = i32
    L.zero_set_write_window.argtypes = [i64, i64]
    _lib = L
    return L


def _check(status: int):
    if status != ZERO_OK:
        raise ZeroError(status, load().zero_last_error().decode(errors="replace"))


def _addr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def _ptr_array(xs) -> ctypes.Array:
    return (ctypes.c_void_p * max(1, len(xs)))(*[_addr(x) for x in xs])


def zero_version() -> int:
    return int(load().zero_version())


WINDOW_AUTO = -1


def zero_set_write_window(period_ticks: int, open_ticks: int = 0) -> None:
    """Store scheduling of the fused step and the reduction (results are
    identical): -1 automatic (default), 0 none, else a period of period_ticks
    real-time-counter ticks (10 ns) whose first open_ticks admit stores."""
    _check(load().zero_set_write_window(period_ticks, open_ticks))


def zero_last_error() -> str:
    return load().zero_last_error().decode(errors="replace")


class Plan:
    """Owner of a zero_plan_t handle, with its queries."""

    def __init__(self, handle: int, n_tensors: int):
        self._h = ctypes.c_void_p(handle)
        self.n_tensors = n_tensors
        L = load()
        psi_pad, shard_total = ctypes.c_int64(), ctypes.c_int64()
        nb, nd = ctypes.c_int32(), ctypes.c_int32()
        _check(L.zero_plan_info(self._h, ctypes.byref(psi_pad), ctypes.byref(shard_total),
                                ctypes.byref(nb), ctypes.byref(nd)))
        self.psi_pad, self.shard_total = psi_pad.value, shard_total.value
        self.n_buckets, self.n_d = nb.value, nd.value

    @property
    def handle(self):
        return self._h

    def bucket(self, b: int):
        """(flat_off, numel, padded, shard_numel, shard_off) of bucket b."""
        vals = [ctypes.c_int64() for _ in range(5)]
        _check(load().zero_plan_bucket(self._h, b, *[ctypes.byref(v) for v in vals]))
        return tuple(v.value for v in vals)

    def tensor(self, t: int):
        """(bucket, flat_off) of tensor t."""
        b, off = ctypes.c_int32(), ctypes.c_int64()
        _check(load().zero_plan_tensor(self._h, t, ctypes.byref(b), ctypes.byref(off)))
        return b.value, off.value

    def buckets(self):
        return [self.bucket(b) for b in range(self.n_buckets)]

    def close(self):
        if self._h is not None and self._h.value:
            load().zero_plan_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def zero_plan(psi: int, n_d: int, tensor_numel: Sequence[int], bucket_cap: int = 0,
              shard_align: int = 64) -> Plan:
    n = len(tensor_numel)
    arr = (ctypes.c_int64 * max(1, n))(*tensor_numel)
    h = ctypes.c_void_p()
    _check(load().zero_plan(psi, n_d, arr, n, bucket_cap, shard_align, ctypes.byref(h)))
    return Plan(h.value, n)


class GradSrc:
    """The N_d gradient contributions (zero_grad_src)."""

    def __init__(self, dtype: int, ptrs: Sequence, is_full: Optional[Sequence[int]] = None):
        self.dtype = dtype
        self._ptrs = _ptr_array(ptrs)
        self.n = len(ptrs)
        self._full = None if is_full is None else (ctypes.c_uint8 * max(1, len(is_full)))(*is_full)
        self.c = _GradSrc(dtype, self.n, ctypes.cast(self._ptrs, ctypes.POINTER(ctypes.c_void_p)),
                          None if self._full is None else ctypes.cast(self._full, ctypes.POINTER(ctypes.c_uint8)))


def zero_flatten(plan: Plan, tensors: Sequence, dt: int, flat, stream=None) -> None:
    _check(load().zero_flatten(plan.handle, _ptr_array(tensors), dt, _addr(flat), _stream(stream)))


def zero_shard_reduce(plan: Plan, rank: int, src: GradSrc, grad_scale: float, out, stream=None) -> None:
    _check(load().zero_shard_reduce(plan.handle, rank, ctypes.byref(src.c), grad_scale, _addr(out),
                                    _stream(stream)))


def zero_adam_step(plan: Plan, rank: int, lr: float, beta1: float, beta2: float, eps: float,
                   grad_scale: float, t: int, slices: Optional[GradSrc], reduced, master, m, v,
                   param_dst, param_dt: int, dst_is_full: bool, stream=None) -> None:
    hp = _AdamHyper(lr, beta1, beta2, eps, grad_scale)
    _check(load().zero_adam_step(plan.handle, rank, ctypes.byref(hp), t,
                                 None if slices is None else ctypes.byref(slices.c), _addr(reduced),
                                 _addr(master), _addr(m), _addr(v), _addr(param_dst), param_dt,
                                 1 if dst_is_full else 0, _stream(stream)))


def zero_gather_pack(plan: Plan, shards: Sequence, dt: int, full, stream=None) -> None:
    _check(load().zero_gather_pack(plan.handle, _ptr_array(shards), dt, _addr(full), _stream(stream)))


def zero_reshard(src_plan: Plan, dst_plan: Plan, dst_rank: int, src_shards: Sequence, dt: int, dst_shard,
                 stream=None) -> None:
    _check(load().zero_reshard(src_plan.handle, dst_plan.handle, dst_rank, _ptr_array(src_shards), dt,
                               _addr(dst_shard), _stream(stream)))
