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
* Normal draw (Box & Muller, "A note on the generation of random normal
  deviates", Ann. Math. Statist. 29, 1958): z = sqrt(-2 ln u1) cos(2 pi u2)
  with two independent uniforms taken from ``u``:
    u1 = (u >> 40 + 1) * 2^-24, in (0, 1]  (24 bits; the draw reaches 5.77 sigma)
    k  = (u & 0xFFFFFFFF) >> 8              (24 bits: the angle 2 pi k / 2^24)
  Everything is computed in fp32 with +, -, *, / and sqrt only -- all of
  them correctly rounded on the host and on the GPU -- in the fixed order
  below, so the three implementations agree bit for bit:
    ln u1: write u1 = m 2^E exactly with m in [sqrt2/2, sqrt2) (m in [1, 2)
      from the binary exponent, halved once if m >= fp32(sqrt 2));
      s = (m - 1) / (m + 1), s2 = s * s, and ln m = 2 atanh(s) from the
      series 2 (s + s^3/3 + ... + s^13/13), evaluated as
      q = L6; q = L_j + s2 * q for j = 5..0; t = s * q; ln m = t + t;
      ln u1 = (E * LN2) + ln m.
    r = sqrt(ln u1 * -2).
    cos(2 pi k / 2^24): quadrant h = k >> 22, x = (k & (2^22 - 1)) * QSTEP in
      [0, pi/2); x2 = x * x; cos x and sin x from their Taylor series to x^14
      and x^15, each by the same Horner loop (p = c7; p = c_j + x2 * p for
      j = 6..0; sin x = x * p); the value is cos x, -sin x, -cos x, sin x for
      h = 0, 1, 2, 3.
    z = r * that cosine; the fp32 value is z * fp32(sigma).
  The coefficients are the fp32 roundings of 1/(2j)!, 1/(2j+1)! and 1/(2j+1)
  (with alternating signs for the Taylor series); LN2, SQRT2 and QSTEP =
  fp32(pi) * 2^-23 are fp32 constants.  Every approximation error is below
  2e-7 relative; only the bits matter for parity, the shape for the
  workloads.
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

# fp32 constants of the normal draw (hex floats: exact fp32 values).
_f = np.float32
COS_C = tuple(_f(float.fromhex(h)) for h in (
    "0x1.0p+0", "-0x1.0p-1", "0x1.555556p-5", "-0x1.6c16c2p-10", "0x1.a01a02p-16", "-0x1.27e4fcp-22",
    "0x1.1eed8ep-29", "-0x1.93974ap-37"))                      # fp32((-1)^j / (2j)!)
SIN_C = tuple(_f(float.fromhex(h)) for h in (
    "0x1.0p+0", "-0x1.555556p-3", "0x1.111112p-7", "-0x1.a01a02p-13", "0x1.71de3ap-19", "-0x1.ae6456p-26",
    "0x1.612462p-33", "-0x1.ae7f3ep-41"))                      # fp32((-1)^j / (2j+1)!)
LOG_C = tuple(_f(float.fromhex(h)) for h in (
    "0x1.0p+0", "0x1.555556p-2", "0x1.99999ap-3", "0x1.24924ap-3", "0x1.c71c72p-4", "0x1.745d18p-4",
    "0x1.3b13b2p-4"))                                           # fp32(1 / (2j+1))
LN2 = _f(float.fromhex("0x1.62e43p-1"))
SQRT2 = _f(float.fromhex("0x1.6a09e6p+0"))
QSTEP = _f(float.fromhex("0x1.921fb6p-22"))                     # fp32(pi) * 2^-23
U1_STEP = _f(2.0 ** -24)
Z_MAX = math.sqrt(-2.0 * math.log(2.0 ** -24))                  # largest |z|: 5.77
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
    """The fp32 multiplier of the unit normal draw: fp32(sigma)."""
    return np.float32(sigma)


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


def _horner(coef, x2: np.ndarray) -> np.ndarray:
    p = np.full(x2.shape, coef[-1], np.float32)
    for c in coef[-2::-1]:
        p = (c + x2 * p).astype(np.float32)
    return p


def unit_normal_np(u: np.ndarray) -> np.ndarray:
    """Box-Muller unit normal draw of each 64-bit hash u, in fp32 (see the
    module docstring for the exact sequence of operations)."""
    u = np.asarray(u, np.uint64)
    f32 = np.float32
    u1 = ((u >> np.uint64(40)) + np.uint64(1)).astype(f32) * U1_STEP          # exact
    mant, ex = np.frexp(u1)                                                      # u1 = mant 2^ex, mant in [0.5, 1)
    m = (mant * f32(2)).astype(f32)
    e = ex.astype(np.int32) - 1
    big = m >= SQRT2
    m = np.where(big, m * f32(0.5), m).astype(f32)
    e = np.where(big, e + 1, e)
    s = ((m - f32(1)) / (m + f32(1))).astype(f32)
    s2 = (s * s).astype(f32)
    t = (s * _horner(LOG_C, s2)).astype(f32)
    ln_u1 = (e.astype(f32) * LN2 + (t + t)).astype(f32)
    r = np.sqrt((ln_u1 * f32(-2)).astype(f32)).astype(f32)
    k = (u & np.uint64(0xFFFFFFFF)) >> np.uint64(8)
    h = (k >> np.uint64(22)).astype(np.int64)
    x = ((k & np.uint64(0x3FFFFF)).astype(f32) * QSTEP).astype(f32)
    x2 = (x * x).astype(f32)
    cos_x = _horner(COS_C, x2)
    sin_x = (x * _horner(SIN_C, x2)).astype(f32)
    c = np.select([h == 0, h == 1, h == 2], [cos_x, -sin_x, -cos_x], sin_x).astype(f32)
    return (r * c).astype(f32)


def normal_f32_np(key: int, positions: np.ndarray, sigma: float) -> np.ndarray:
    return (unit_normal_np(draw_u64(key, positions)) * scale_for(sigma)).astype(np.float32)


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
