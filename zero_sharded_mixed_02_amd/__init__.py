"""Python binding of libzero.so: one data-parallel rank's share of a ZeRO
mixed-precision training step on an MI355X (gfx950).

Thin ctypes marshalling over the C ABI in ``include/zero.h``: every function
here has the C entry point's name and arguments, converts tensors to device
addresses and streams to ``hipStream_t`` handles, and raises ``ZeroError`` on a
non-OK status.  All computation happens in the HIP kernels of libzero.so; if
the library has not been built, loading fails loudly (there is no fallback).

Tensors may be passed as ``torch.Tensor`` or as plain integer device
addresses.  A tensor is checked against the plan before the C call -- a
contiguous GPU tensor of the right element size holding at least the elements
the plan needs (exactly tensor t's size for flatten inputs) -- and pointer
lists must have one entry per rank or tensor; a failed check raises
``ValueError`` and nothing is launched.  A plain integer address is passed
through unchecked: the caller vouches for it.  ``stream=None`` means torch's
current stream on the current device.
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
                "zero_plan_info", "zero_plan_bucket", "zero_plan_tensor", "zero_flatten_workspace_bytes",
                "zero_flatten", "zero_shard_reduce", "zero_adam_step", "zero_gather_pack", "zero_reshard",
                "zero_set_write_window", "zero_set_stream_write_window", "zero_set_warm_read")


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
    L.zero_flatten_workspace_bytes.restype = ctypes.c_size_t
    L.zero_flatten_workspace_bytes.argtypes = [vp]
    L.zero_flatten.restype = i32
    L.zero_flatten.argtypes = [vp, ctypes.POINTER(vp), i32, vp, vp, ctypes.c_size_t, vp]
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
    L.zero_set_stream_write_window.restype = i32
    L.zero_set_stream_write_window.argtypes = [vp, i64, i64]
    L.zero_set_warm_read.restype = i32
    L.zero_set_warm_read.argtypes = [i32]
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


ESIZE = {ZERO_F32: 4, ZERO_F16: 2, ZERO_BF16: 2}


def _esize(dt: int) -> int:
    if dt not in ESIZE:
        raise ValueError(f"unknown dtype {dt}")
    return ESIZE[dt]


def _tensor_props(x, name: str, esize: int):
    """(element count, on a GPU) of tensor x after checking what does not
    depend on the plan: a contiguous tensor whose elements are esize bytes."""
    if not hasattr(x, "data_ptr") or not hasattr(x, "element_size"):
        raise TypeError(f"{name}: expected a torch tensor or an integer device address, got {type(x).__name__}")
    if x.element_size() != esize:
        raise ValueError(f"{name}: elements of {x.element_size()} bytes ({x.dtype}), expected {esize}")
    if not x.is_contiguous():
        raise ValueError(f"{name} is not contiguous")
    return int(x.numel()), bool(x.is_cuda)


def _arg(x, name: str, esize: int, need: int, exact: bool = False) -> int:
    """Device address of x.  A tensor must be a contiguous GPU tensor holding
    at least `need` elements of esize bytes (exactly `need` with exact=True);
    None and integer addresses are passed through (the C side rejects a NULL
    it cannot accept)."""
    if x is None or isinstance(x, int):
        return _addr(x)
    n, on_gpu = _tensor_props(x, name, esize)
    if n < need or (exact and n != need):
        raise ValueError(f"{name} holds {n} elements, the plan needs {'exactly ' if exact else ''}{need}")
    if not on_gpu:
        raise ValueError(f"{name} is not on a GPU ({x.device})")
    return int(x.data_ptr())


def _arg_list(xs, name: str, count: int, esize: int, need: int, exact: bool = False) -> ctypes.Array:
    if xs is None:
        raise ValueError(f"{name} is None")
    xs = list(xs)
    if len(xs) != count:
        raise ValueError(f"{name} has {len(xs)} entries, the plan needs {count}")
    per = isinstance(need, (list, tuple))
    addrs = []
    for i, x in enumerate(xs):
        want = need[i] if per else need
        # Fast path for the common case (a contiguous GPU tensor of the right
        # element size and length); anything else goes through _arg, which
        # raises with the argument's name.
        try:
            if x.element_size() == esize and x.is_contiguous() and x.is_cuda:
                n = x.numel()
                if n == want or (n > want and not exact):
                    addrs.append(x.data_ptr())
                    continue
        except AttributeError:
            pass
        addrs.append(_arg(x, f"{name}[{i}]", esize, want, exact))
    return (ctypes.c_void_p * max(1, count))(*addrs)


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def zero_version() -> int:
    return int(load().zero_version())


WINDOW_AUTO = -1


def zero_set_write_window(period_ticks: int, open_ticks: int = 0) -> None:
    """Process-wide default store scheduling of the fused step and the
    reduction (results are identical): -1 automatic (default), 0 none, else a
    period of period_ticks real-time-counter ticks whose first open_ticks
    admit stores."""
    _check(load().zero_set_write_window(period_ticks, open_ticks))


WINDOW_INHERIT = -2


def zero_set_stream_write_window(stream, period_ticks: int, open_ticks: int = 0) -> None:
    """The same setting for launches on one stream only; -2 removes the
    stream's own setting so it follows the process-wide default again."""
    _check(load().zero_set_stream_write_window(_stream(stream), period_ticks, open_ticks))


def zero_set_warm_read(enable: bool) -> None:
    """Read up to 256 MiB of the fused step's own state just before each
    large fused step (process-wide; off by default)."""
    _check(load().zero_set_warm_read(1 if enable else 0))


def zero_last_error() -> str:
    return load().zero_last_error().decode(errors="replace")


class Plan:
    """Owner of a zero_plan_t handle, with its queries."""

    def __init__(self, handle: int, tensor_numel: Sequence[int]):
        self._h = ctypes.c_void_p(handle)
        self.tensor_numel = [int(n) for n in tensor_numel]
        self.n_tensors = len(self.tensor_numel)
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
    return Plan(h.value, tensor_numel)


class GradSrc:
    """The N_d gradient contributions (zero_grad_src).  Tensors are checked
    here (16-bit elements, contiguous, on a GPU) and kept referenced; their
    sizes are compared with the plan at every call."""

    def __init__(self, dtype: int, ptrs: Sequence, is_full: Optional[Sequence[int]] = None):
        if dtype not in (ZERO_F16, ZERO_BF16):
            raise ValueError(f"gradient dtype {dtype} is not 16-bit")
        ptrs = list(ptrs)
        self.dtype = dtype
        self.n = len(ptrs)
        if is_full is not None and len(is_full) != self.n:
            raise ValueError(f"is_full has {len(is_full)} entries for {self.n} gradient buffers")
        self.is_full = [0] * self.n if is_full is None else [1 if f else 0 for f in is_full]
        self._keep = ptrs
        # Smallest tensor among the compact and among the full contributions
        # (plain addresses are not counted: the caller vouches for them).
        self.min_compact = self.min_full = None
        self.not_on_gpu = None   # name of the first tensor that is not on a GPU
        for q, x in enumerate(ptrs):
            if x is None or isinstance(x, int):
                continue
            n, on_gpu = _tensor_props(x, f"gradient of rank {q}", 2)
            if not on_gpu and self.not_on_gpu is None:
                self.not_on_gpu = f"gradient of rank {q} ({x.device})"
            if self.is_full[q]:
                self.min_full = n if self.min_full is None else min(self.min_full, n)
            else:
                self.min_compact = n if self.min_compact is None else min(self.min_compact, n)
        self._ptrs = (ctypes.c_void_p * max(1, self.n))(*[_addr(x) for x in ptrs])
        self._full = None if is_full is None else (ctypes.c_uint8 * max(1, self.n))(*self.is_full)
        self.c = _GradSrc(dtype, self.n, ctypes.cast(self._ptrs, ctypes.POINTER(ctypes.c_void_p)),
                          None if self._full is None else ctypes.cast(self._full, ctypes.POINTER(ctypes.c_uint8)))

    def check(self, plan: "Plan") -> None:
        if self.n != plan.n_d:
            raise ValueError(f"gradient source has {self.n} ranks, the plan has n_d={plan.n_d}")
        if self.min_compact is not None and self.min_compact < plan.shard_total:
            raise ValueError(f"a compact gradient slice holds {self.min_compact} elements, "
                             f"the plan needs {plan.shard_total}")
        if self.min_full is not None and self.min_full < plan.psi_pad:
            raise ValueError(f"a full gradient buffer holds {self.min_full} elements, the plan needs {plan.psi_pad}")
        if self.not_on_gpu is not None:
            raise ValueError(f"{self.not_on_gpu} is not on a GPU")


def zero_flatten_workspace_bytes(plan: Plan) -> int:
    return int(load().zero_flatten_workspace_bytes(plan.handle))


def zero_flatten(plan: Plan, tensors: Sequence, dt: int, flat, stream=None, workspace=None,
                 ws_bytes: int = 0) -> None:
    es = _esize(dt)
    arr = _arg_list(tensors, "tensors", plan.n_tensors, es, plan.tensor_numel, exact=True)
    out = _arg(flat, "flat", es, plan.psi_pad)
    ws = _addr(workspace)
    _check(load().zero_flatten(plan.handle, arr, dt, out, ws, ws_bytes, _stream(stream)))


def zero_shard_reduce(plan: Plan, rank: int, src: GradSrc, grad_scale: float, out, stream=None) -> None:
    src.check(plan)
    o = _arg(out, "out", 4, plan.shard_total)
    _check(load().zero_shard_reduce(plan.handle, rank, ctypes.byref(src.c), grad_scale, o, _stream(stream)))


def zero_adam_step(plan: Plan, rank: int, lr: float, beta1: float, beta2: float, eps: float,
                   grad_scale: float, t: int, slices: Optional[GradSrc], reduced, master, m, v,
                   param_dst, param_dt: int, dst_is_full: bool, stream=None) -> None:
    S = plan.shard_total
    if slices is not None:
        slices.check(plan)
        red = 0
    else:
        red = _arg(reduced, "reduced", 4, S)
    w_, m_, v_ = _arg(master, "master", 4, S), _arg(m, "m", 4, S), _arg(v, "v", 4, S)
    if param_dt not in (ZERO_F16, ZERO_BF16):
        raise ValueError(f"parameter dtype {param_dt} is not 16-bit")
    dst = _arg(param_dst, "param_dst", 2, plan.psi_pad if dst_is_full else S)
    hp = _AdamHyper(lr, beta1, beta2, eps, grad_scale)
    _check(load().zero_adam_step(plan.handle, rank, ctypes.byref(hp), t,
                                 None if slices is None else ctypes.byref(slices.c), red,
                                 w_, m_, v_, dst, param_dt, 1 if dst_is_full else 0, _stream(stream)))


def zero_gather_pack(plan: Plan, shards: Sequence, dt: int, full, stream=None) -> None:
    es = _esize(dt)
    arr = _arg_list(shards, "shards", plan.n_d, es, plan.shard_total)
    out = _arg(full, "full", es, plan.psi_pad)
    _check(load().zero_gather_pack(plan.handle, arr, dt, out, _stream(stream)))


def zero_reshard(src_plan: Plan, dst_plan: Plan, dst_rank: int, src_shards: Sequence, dt: int, dst_shard,
                 stream=None) -> None:
    es = _esize(dt)
    arr = _arg_list(src_shards, "src_shards", src_plan.n_d, es, src_plan.shard_total)
    out = _arg(dst_shard, "dst_shard", es, dst_plan.shard_total)
    _check(load().zero_reshard(src_plan.handle, dst_plan.handle, dst_rank, arr, dt, out, _stream(stream)))
