"""Seeded synthetic inputs, shared by the oracle side and the GPU side.

This module holds no arithmetic of the ZeRO step.  It only defines which
numbers sit at which position of which buffer, so that the CPU oracle and the
GPU library can be fed identical bytes without either producing the other's
inputs.  The same definition is implemented three times: with numpy here
(the readable reference, ``*_np``), in ``synth_cpu.c`` (the fast host path the
oracle side uses) and in ``synth_fill.hip`` (bulk fills on the GPU).  Tests
check them against each other bit for bit.

Definition
----------
* Counter-based hash: SplitMix64 (Steele, Lea & Flood, "Fast splittable
  pseudorandom number generators", OOPSLA 2014).  ``mix64`` is its output
  function; the i-th output of a generator whose state starts at ``k`` is
  ``mix64(k + (i + 1) * GAMMA)``.
* Key of a stream: ``k = seed``; then for each field f of
  (stream id, rank, step): ``k = mix64((k ^ f) + GAMMA)``.
* Value at flat position ``pos``: ``u = mix64(key + (pos + 1) * GAMMA)``.
* Approximately normal draw (Irwin-Hall with four terms): the four 16-bit
  fields of ``u`` are summed and centred, ``s = a + b + c + d - 131070``, an
  integer in [-131070, 131070] with standard deviation
  ``SD = sqrt((65536**2 - 1) / 3)``.  The fp32 value is
  ``float32(s) * float32(sigma / SD)`` -- one correctly rounded fp32 multiply,
  so both implementations agree exactly.  It is a bounded (|x| <= 3.46 sigma)
  stand-in for N(0, sigma), chosen because it needs no transcendental
  function whose last bit could differ between the host and the GPU.
* 16-bit values are the round-to-nearest-even conversion of that fp32 value
  (numpy's float16 conversion and torch's bfloat16 conversion here; the GPU's
  conversion instructions there).
* The zero/outlier mix: a second draw ``w`` from the MIXSEL stream at the same
  position; with ``x = w >> 32``: ``x < ZERO_CUT`` gives 0, else
  ``x < ZERO_CUT + OUTLIER_CUT`` gives +-100 (sign from bit 0 of ``w``), else
  the normal draw.  ZERO_CUT = floor(0.01 * 2^32), OUTLIER_CUT =
  floor(0.001 * 2^32).
"""
from __future__ import annotations

import math

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
M64 = (1 << 64) - 1

STREAM_GRAD = 1
STREAM_MASTER = 2
STREAM_MIXSEL = 3

SD_IRWIN_HALL4 = math.sqrt((65536.0 ** 2 - 1.0) / 3.0)
ZERO_CUT = int(0.01 * 2 ** 32)       # 42949672
OUTLIER_CUT = int(0.001 * 2 ** 32)   # 4294967
OUTLIER_VALUE = 100.0

F32, F16, BF16 = 0, 1, 2


def mix64_int(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * MIX1) & M64
    z = ((z ^ (z >> 27)) * MIX2) & M64
    return z ^ (z >> 31)


def key_of(seed: int, stream: int, rank: int, step: int) -> int:
    k = seed & M64
    for f in (stream, rank, step):
        k = mix64_int(((k ^ (f & M64)) + GAMMA) & M64)
    return k


def scale_for(sigma: float) -> np.float32:
    """The fp32 multiplier of the Irwin-Hall integer (rounded once from fp64)."""
    return np.float32(sigma / SD_IRWIN_HALL4)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    with np.errstate(over="ignore"):
        z ^= z >> np.uint64(30)
        z *= np.uint64(MIX1)
        z ^= z >> np.uint64(27)
        z *= np.uint64(MIX2)
        z ^= z >> np.uint64(31)
    return z


def draw_u64(key: int, positions: np.ndarray) -> np.ndarray:
    pos = np.asarray(positions, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(key) + (pos + np.uint64(1)) * np.uint64(GAMMA)
    return _mix64_np(state)


def irwin_hall_int(u: np.ndarray) -> np.ndarray:
    m = np.uint64(0xFFFF)
    s = (u & m) + ((u >> np.uint64(16)) & m) + ((u >> np.uint64(32)) & m) + (u >> np.uint64(48))
    return s.astype(np.int64) - 131070


def normal_f32_np(key: int, positions: np.ndarray, sigma: float) -> np.ndarray:
    s = irwin_hall_int(draw_u64(key, positions)).astype(np.float32)
    return (s * scale_for(sigma)).astype(np.float32)


def mix_f32_np(key: int, sel_key: int, positions: np.ndarray, sigma: float) -> np.ndarray:
    x = normal_f32_np(key, positions, sigma)
    w = draw_u64(sel_key, positions)
    hi = w >> np.uint64(32)
    zero = hi < np.uint64(ZERO_CUT)
    outl = (~zero) & (hi < np.uint64(ZERO_CUT + OUTLIER_CUT))
    sign = np.where((w & np.uint64(1)) == 1, np.float32(-OUTLIER_VALUE), np.float32(OUTLIER_VALUE))
    x = np.where(zero, np.float32(0.0), x)
    x = np.where(outl, sign, x).astype(np.float32)
    return x


_cpu_lib = None


def _cpu():
    """The C implementation of the same definition (synth_cpu.c), for speed."""
    global _cpu_lib
    if _cpu_lib is None:
        import ctypes
        import os
        from . import _build
        if not os.path.exists(_build.CPU_LIB):
            _build.build_cpu()
        L = ctypes.CDLL(_build.CPU_LIB)
        L.synth_values_f32.restype = None
        L.synth_values_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint64,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_float]
        _cpu_lib = L
    return _cpu_lib


def values_f32_c(key: int, sel_key: int, mix: bool, positions: np.ndarray, sigma: float) -> np.ndarray:
    import ctypes
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    out = np.empty(pos.size, dtype=np.float32)
    _cpu().synth_values_f32(ctypes.c_void_p(out.ctypes.data), pos.size, key & M64, sel_key & M64,
                            1 if mix else 0, ctypes.c_void_p(pos.ctypes.data), 0,
                            ctypes.c_float(float(scale_for(sigma))))
    return out


def normal_f32(key: int, positions: np.ndarray, sigma: float) -> np.ndarray:
    return values_f32_c(key, 0, False, positions, sigma)


def mix_f32(key: int, sel_key: int, positions: np.ndarray, sigma: float) -> np.ndarray:
    return values_f32_c(key, sel_key, True, positions, sigma)


def to_dtype_bits(x: np.ndarray, dt: int) -> np.ndarray:
    """fp32 -> storage bits of dtype dt (uint16 for 16-bit types, float32 for F32)."""
    x = np.asarray(x, dtype=np.float32)
    if dt == F32:
        return x.copy()
    if dt == F16:
        return x.astype(np.float16).view(np.uint16)
    if dt == BF16:
        import torch
        return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dt)


def grad_values(seed: int, rank: int, step: int, positions: np.ndarray, sigma: float,
                dt: int, mix: bool = False, pad_mask: np.ndarray | None = None) -> np.ndarray:
    """Gradient of simulated rank ``rank`` at step ``step`` at the given flat
    positions, as storage bits; positions flagged in pad_mask are zero."""
    k = key_of(seed, STREAM_GRAD, rank, step)
    if mix:
        x = mix_f32(k, key_of(seed, STREAM_MIXSEL, rank, step), positions, sigma)
    else:
        x = normal_f32(k, positions, sigma)
    if pad_mask is not None and pad_mask.any():
        x[pad_mask] = np.float32(0.0)
    return to_dtype_bits(x, dt)


def master_values(seed: int, positions: np.ndarray, sigma: float,
                  pad_mask: np.ndarray | None = None) -> np.ndarray:
    k = key_of(seed, STREAM_MASTER, 0, 0)
    x = normal_f32(k, positions, sigma)
    if pad_mask is not None and pad_mask.any():
        x[pad_mask] = np.float32(0.0)
    return x
