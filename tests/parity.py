"""Comparison rules of the parity tests.

fp32 state (master, m, v): max |x - y| / |y| <= 1e-6 over y != 0, and x == y
where y == 0 (-0 equals +0).  16-bit parameters: at most 1 ulp apart.  NaN
matches NaN (payload bits may differ between the host and the GPU).  Besides
the tolerance, the helpers count elements whose bits differ: the pinned fp32
operation order makes the GPU and the oracle agree bit for bit.
"""
import numpy as np

REL_TOL_F32 = 1e-6
ULP_TOL_16 = 1


def f32_report(got: np.ndarray, want: np.ndarray) -> dict:
    got = np.asarray(got, np.float32).ravel()
    want = np.asarray(want, np.float32).ravel()
    assert got.shape == want.shape
    gn, wn = np.isnan(got), np.isnan(want)
    nan_bad = int(np.count_nonzero(gn != wn))
    ok = ~(gn | wn)
    g, w = got[ok].astype(np.float64), want[ok].astype(np.float64)
    inf_bad = int(np.count_nonzero((np.isinf(g) | np.isinf(w)) & (g != w)))
    fin = np.isfinite(g) & np.isfinite(w)
    g, w = g[fin], w[fin]
    zero = w == 0
    zero_bad = int(np.count_nonzero(g[zero] != 0))
    rel = np.abs(g[~zero] - w[~zero]) / np.abs(w[~zero])
    max_rel = float(rel.max()) if rel.size else 0.0
    bits_diff = int(np.count_nonzero(got[ok].view(np.uint32) != want[ok].view(np.uint32)))
    return {"nan_bad": nan_bad, "inf_bad": inf_bad, "zero_bad": zero_bad, "max_rel": max_rel,
            "bits_diff": bits_diff, "n": int(got.size)}


def _ordered16(h: np.ndarray) -> np.ndarray:
    h = h.astype(np.int64)
    return np.where(h & 0x8000, -(h & 0x7FFF), h & 0x7FFF)


def _is_nan16(h: np.ndarray, dt: int) -> np.ndarray:
    h = h.astype(np.int64)
    if dt == 2:   # bf16
        return ((h & 0x7F80) == 0x7F80) & ((h & 0x7F) != 0)
    return ((h & 0x7C00) == 0x7C00) & ((h & 0x3FF) != 0)


def p16_report(got: np.ndarray, want: np.ndarray, dt: int) -> dict:
    got = np.asarray(got).view(np.uint16).ravel()
    want = np.asarray(want).view(np.uint16).ravel()
    assert got.shape == want.shape
    gn, wn = _is_nan16(got, dt), _is_nan16(want, dt)
    nan_bad = int(np.count_nonzero(gn != wn))
    ok = ~(gn | wn)
    d = np.abs(_ordered16(got[ok]) - _ordered16(want[ok]))
    return {"nan_bad": nan_bad, "max_ulp": int(d.max()) if d.size else 0,
            "bits_diff": int(np.count_nonzero(got[ok] != want[ok])), "n": int(got.size)}


def assert_f32(got, want, what="", bitwise=False):
    r = f32_report(got, want)
    assert r["nan_bad"] == 0 and r["inf_bad"] == 0 and r["zero_bad"] == 0, (what, r)
    assert r["max_rel"] <= REL_TOL_F32, (what, r)
    if bitwise:
        assert r["bits_diff"] == 0, (what, r)
    return r


def assert_p16(got, want, dt, what="", bitwise=False):
    r = p16_report(got, want, dt)
    assert r["nan_bad"] == 0 and r["max_ulp"] <= ULP_TOL_16, (what, r)
    if bitwise:
        assert r["bits_diff"] == 0, (what, r)
    return r


def assert_state(got: dict, want: dict, pdt: int, what="", bitwise=True):
    """master/m/v against the oracle, and the parameters ('full' buffer or
    'params' sample)."""
    out = {}
    for k in ("master", "m", "v"):
        out[k] = assert_f32(got[k], want[k], f"{what}:{k}", bitwise)
    for k in ("full", "params", "shards"):
        if k in got and k in want and want[k] is not None:
            out[k] = assert_p16(np.asarray(got[k]), np.asarray(want[k]), pdt, f"{what}:{k}", bitwise)
    return out
