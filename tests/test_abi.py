"""The C ABI without a GPU: libzero.so loads, exports exactly what
include/zero.h declares, its host-side plan matches the oracle's bit for bit,
and bad arguments are rejected before anything is launched."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from tests.test_oracle_pins import _random_plans

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero.h")


def declared_entry_points():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ZERO_API\s+[\w\s\*]*?\b(zero_\w+)\s*\(", text)))


def test_header_and_binding_agree(zero_lib):
    assert declared_entry_points() == sorted(zero_lib.ENTRY_POINTS)


def test_library_exports_every_declared_symbol(zero_lib):
    out = subprocess.run(["nm", "-D", "--defined-only", zero_lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({line.split()[-1] for line in out.splitlines() if " T " in line})
    assert exported == declared_entry_points()
    L = zero_lib.load()
    for name in declared_entry_points():
        assert hasattr(L, name)


def test_version(zero_lib):
    assert zero_lib.zero_version() == 200


def _plan_tuple_lib(Z, p, n_tensors):
    return ([p.bucket(b) for b in range(p.n_buckets)], [p.tensor(t) for t in range(n_tensors)],
            p.psi_pad, p.shard_total)


def _plan_tuple_oracle(op):
    return ([(b.flat_off, b.numel, b.padded, b.shard_numel, b.shard_off) for b in op.buckets],
            list(zip(op.tensor_bucket, op.tensor_off)), op.psi_pad, op.shard_total)


def test_plan_matches_oracle_bruteforce(zero_lib, oracle_lib):
    for n_d, align, sizes, cap in _random_plans(21, 500):
        psi = sum(sizes)
        lp = zero_lib.zero_plan(psi, n_d, sizes, cap, align)
        op = oracle_lib.plan(psi, n_d, sizes, cap, align)
        assert _plan_tuple_lib(zero_lib, lp, len(sizes)) == _plan_tuple_oracle(op)
        assert lp.n_d == n_d


@pytest.mark.parametrize("name", ["tiny", "gpt2-small", "7.5B-stage2", "13B-stage1", "stage3-h8192x8"])
def test_plan_matches_oracle_workloads(zero_lib, oracle_lib, name):
    from synth.workloads import WORKLOADS
    c = WORKLOADS[name]
    lp = zero_lib.zero_plan(c.psi, c.n_d, list(c.sizes), c.bucket_cap, c.align)
    op = oracle_lib.plan(c.psi, c.n_d, list(c.sizes), c.bucket_cap, c.align)
    assert _plan_tuple_lib(zero_lib, lp, len(c.sizes)) == _plan_tuple_oracle(op)


def test_plan_many_buckets_and_empty(zero_lib, oracle_lib):
    sizes = [3, 0, 5, 0, 0, 7] * 50
    for cap in (1, 4, 8, 12, 0):
        lp = zero_lib.zero_plan(sum(sizes), 3, sizes, cap, 8)
        op = oracle_lib.plan(sum(sizes), 3, sizes, cap, 8)
        assert _plan_tuple_lib(zero_lib, lp, len(sizes)) == _plan_tuple_oracle(op)
    empty = zero_lib.zero_plan(0, 4, [], 0, 64)
    assert (empty.psi_pad, empty.shard_total, empty.n_buckets) == (0, 0, 0)


# ---------------------------------------------------------------------------
# Error paths (all return before any launch, so no GPU is touched)
# ---------------------------------------------------------------------------

def _status(Z, fn, *args):
    return getattr(Z.load(), fn)(*args)


def test_plan_rejects_bad_arguments(zero_lib):
    Z = zero_lib
    L = Z.load()
    h = ctypes.c_void_p()
    sizes = (ctypes.c_int64 * 2)(5, 6)
    assert L.zero_plan(11, 0, sizes, 2, 0, 1, ctypes.byref(h)) == Z.ZERO_EINVAL
    assert "n_d" in Z.zero_last_error()
    assert L.zero_plan(12, 2, sizes, 2, 0, 1, ctypes.byref(h)) == Z.ZERO_EINVAL
    assert "sum" in Z.zero_last_error()
    assert L.zero_plan(11, 2, sizes, 2, 0, 0, ctypes.byref(h)) == Z.ZERO_EINVAL
    assert L.zero_plan(11, 2, sizes, 2, -1, 1, ctypes.byref(h)) == Z.ZERO_EINVAL
    assert L.zero_plan(11, 2, None, 2, 0, 1, ctypes.byref(h)) == Z.ZERO_EINVAL
    assert L.zero_plan(11, 2, sizes, 2, 0, 1, None) == Z.ZERO_EINVAL
    neg = (ctypes.c_int64 * 2)(-1, 12)
    assert L.zero_plan(11, 2, neg, 2, 0, 1, ctypes.byref(h)) == Z.ZERO_EINVAL
    with pytest.raises(Z.ZeroError):
        Z.zero_plan(10, 3, [4, 4])


def test_plan_queries_reject_bad_index(zero_lib):
    Z = zero_lib
    p = Z.zero_plan(100, 4, [60, 40], 50, 1)
    assert p.n_buckets == 2
    with pytest.raises(Z.ZeroError):
        p.bucket(2)
    with pytest.raises(Z.ZeroError):
        p.tensor(-1)
    assert Z.load().zero_plan_info(None, None, None, None, None) == Z.ZERO_EINVAL


BASE = 1 << 40       # fake, never dereferenced: every call below fails its checks first


def _adam(Z, plan, rank=0, t=1, slices=None, reduced=0, master=BASE, m=BASE + (1 << 30),
          v=BASE + (2 << 30), dst=BASE + (3 << 30), pdt=1, full=True, hp=True):
    L = Z.load()
    h = Z._AdamHyper(1e-4, 0.9, 0.999, 1e-8, 0.25)
    return L.zero_adam_step(plan.handle if plan is not None else None, rank,
                            ctypes.byref(h) if hp else None, t,
                            None if slices is None else ctypes.byref(slices.c), reduced, master, m, v,
                            dst, pdt, 1 if full else 0, None)


def test_adam_step_rejects_bad_arguments(zero_lib):
    Z = zero_lib
    p = Z.zero_plan(1000, 4, [1000], 0, 8)
    g = [BASE + (4 << 30) + q * (1 << 20) for q in range(4)]
    src = Z.GradSrc(Z.ZERO_BF16, g)
    assert _adam(Z, None, slices=src) == Z.ZERO_EINVAL
    assert _adam(Z, p, rank=4, slices=src) == Z.ZERO_EINVAL
    assert _adam(Z, p, rank=-1, slices=src) == Z.ZERO_EINVAL
    assert _adam(Z, p, t=0, slices=src) == Z.ZERO_EINVAL and "t must be" in Z.zero_last_error()
    assert _adam(Z, p, slices=src, hp=False) == Z.ZERO_EINVAL
    assert _adam(Z, p, slices=None, reduced=0) == Z.ZERO_EINVAL
    assert _adam(Z, p, slices=Z.GradSrc(Z.ZERO_BF16, g[:3])) == Z.ZERO_EINVAL
    # The binding refuses a non-16-bit source itself; the C check is reached
    # with a hand-built struct.
    with pytest.raises(ValueError):
        Z.GradSrc(Z.ZERO_F32, g)
    raw_ptrs = (ctypes.c_void_p * 4)(*g)
    raw = Z._GradSrc(Z.ZERO_F32, 4, ctypes.cast(raw_ptrs, ctypes.POINTER(ctypes.c_void_p)), None)

    class _Raw:
        c = raw
    assert _adam(Z, p, slices=_Raw) == Z.ZERO_EUNSUPPORTED
    assert _adam(Z, p, slices=src, pdt=Z.ZERO_F32) == Z.ZERO_EUNSUPPORTED
    assert _adam(Z, p, slices=Z.GradSrc(Z.ZERO_BF16, [g[0], 0, g[2], g[3]])) == Z.ZERO_EINVAL
    assert _adam(Z, p, slices=Z.GradSrc(Z.ZERO_BF16, [g[0] + 1] + g[1:])) == Z.ZERO_EINVAL
    assert _adam(Z, p, slices=src, master=0) == Z.ZERO_EINVAL
    assert _adam(Z, p, slices=src, master=BASE + 2) == Z.ZERO_EINVAL   # not 4-byte aligned
    # Overlaps: state arrays with each other, with the destination, with a gradient.
    assert _adam(Z, p, slices=src, m=BASE + 16) == Z.ZERO_EINVAL and "overlaps" in Z.zero_last_error()
    assert _adam(Z, p, slices=src, dst=BASE + (2 << 30) + 64) == Z.ZERO_EINVAL
    assert _adam(Z, p, slices=src, master=g[1] + 8) == Z.ZERO_EINVAL
    assert _adam(Z, p, slices=None, reduced=BASE + (1 << 30) + 4) == Z.ZERO_EINVAL


def test_fused_step_rank_limit(zero_lib):
    Z = zero_lib
    n = Z.ZERO_MAX_RANKS + 1
    p = Z.zero_plan(n * 8, n, [n * 8], 0, 8)
    src = Z.GradSrc(Z.ZERO_BF16, [BASE + (8 << 30) + q * 4096 for q in range(n)])
    assert _adam(Z, p, slices=src) == Z.ZERO_EUNSUPPORTED
    assert "zero_shard_reduce" in Z.zero_last_error()


def test_reduce_flatten_gather_reject_bad_arguments(zero_lib):
    Z = zero_lib
    L = Z.load()
    p = Z.zero_plan(1000, 4, [600, 400], 512, 8)
    g = [BASE + q * (1 << 20) for q in range(4)]
    src = Z.GradSrc(Z.ZERO_F16, g)
    out = BASE + (1 << 30)
    assert L.zero_shard_reduce(p.handle, 9, ctypes.byref(src.c), 0.25, out, None) == Z.ZERO_EINVAL
    assert L.zero_shard_reduce(p.handle, 0, None, 0.25, out, None) == Z.ZERO_EINVAL
    assert L.zero_shard_reduce(p.handle, 0, ctypes.byref(src.c), 0.25, 0, None) == Z.ZERO_EINVAL
    assert L.zero_shard_reduce(p.handle, 0, ctypes.byref(src.c), 0.25, g[2] + 4, None) == Z.ZERO_EINVAL
    tens = (ctypes.c_void_p * 2)(BASE, BASE + 4096)
    assert L.zero_flatten(p.handle, tens, 7, out, None, 0, None) == Z.ZERO_EINVAL
    assert L.zero_flatten(p.handle, None, Z.ZERO_BF16, out, None, 0, None) == Z.ZERO_EINVAL
    assert L.zero_flatten(p.handle, tens, Z.ZERO_BF16, BASE + 100, None, 0, None) == Z.ZERO_EINVAL  # overlap
    assert L.zero_flatten(p.handle, tens, Z.ZERO_F32, out + 2, None, 0, None) == Z.ZERO_EINVAL      # alignment
    shards = (ctypes.c_void_p * 4)(*g)
    assert L.zero_gather_pack(p.handle, shards, Z.ZERO_F16, g[3] + 2, None) == Z.ZERO_EINVAL
    assert L.zero_gather_pack(p.handle, None, Z.ZERO_F16, out, None) == Z.ZERO_EINVAL
    assert L.zero_gather_pack(None, shards, Z.ZERO_F16, out, None) == Z.ZERO_EINVAL


def test_last_error_is_per_thread(zero_lib):
    import threading
    Z = zero_lib
    Z.load().zero_plan(1, 0, None, 0, 0, 1, None)
    msg = Z.zero_last_error()
    seen = []
    th = threading.Thread(target=lambda: seen.append(Z.zero_last_error()))
    th.start()
    th.join()
    assert msg and seen == [""]


def test_binding_without_library_fails_loudly(tmp_path, monkeypatch):
    import importlib
    import zero_sharded_mixed_02_amd as Z
    monkeypatch.setattr(Z, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(Z, "_lib", None)
    with pytest.raises(ImportError):
        Z.load()
    importlib.reload(Z)


def test_single_hip_runtime_in_process():
    """libzero.so and libsynth.so must bind to the HIP runtime torch loaded,
    whichever is opened first (two runtimes in one process see no device)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import zero_sharded_mixed_02_amd as Z; Z.load()\n"
            "from synth import gpu; gpu.load()\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n") % ROOT
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "1"


def test_reshard_rejects_bad_arguments(zero_lib):
    Z = zero_lib
    L = Z.load()
    a = Z.zero_plan(1000, 4, [600, 400], 512, 8)
    b = Z.zero_plan(1000, 3, [600, 400], 0, 1)
    c = Z.zero_plan(1000, 3, [500, 500], 0, 1)
    shards = (ctypes.c_void_p * 4)(*[BASE + q * (1 << 20) for q in range(4)])
    out = BASE + (1 << 30)
    assert L.zero_reshard(a.handle, c.handle, 0, shards, Z.ZERO_F32, out, None) == Z.ZERO_EINVAL
    assert "tensor lists" in Z.zero_last_error()
    assert L.zero_reshard(a.handle, b.handle, 3, shards, Z.ZERO_F32, out, None) == Z.ZERO_EINVAL
    assert L.zero_reshard(None, b.handle, 0, shards, Z.ZERO_F32, out, None) == Z.ZERO_EINVAL
    assert L.zero_reshard(a.handle, b.handle, 0, None, Z.ZERO_F32, out, None) == Z.ZERO_EINVAL
    assert L.zero_reshard(a.handle, b.handle, 0, shards, 9, out, None) == Z.ZERO_EINVAL
    assert L.zero_reshard(a.handle, b.handle, 0, shards, Z.ZERO_F32, BASE + 8, None) == Z.ZERO_EINVAL
    assert L.zero_reshard(a.handle, b.handle, 0, shards, Z.ZERO_F32, out + 2, None) == Z.ZERO_EINVAL


def test_write_window_setting(zero_lib):
    """zero_set_write_window range checks (no launch involved)."""
    Z = zero_lib
    for bad in ((-2, 0), (100_001, 1), (100, 0), (100, 101)):
        with pytest.raises(Z.ZeroError) as ei:
            Z.zero_set_write_window(*bad)
        assert ei.value.status == Z.ZERO_EINVAL
    for good in ((6000, 750), (1, 1), (100_000, 100_000), (0, 0), (-1, 0)):
        Z.zero_set_write_window(*good)
    for bad in ((-3, 0), (100_001, 1), (100, 0), (100, 101)):
        with pytest.raises(Z.ZeroError) as ei:
            Z.zero_set_stream_write_window(0x1234, *bad)
        assert ei.value.status == Z.ZERO_EINVAL
    for good in ((6000, 750), (0, 0), (-1, 0), (-2, 0)):
        Z.zero_set_stream_write_window(0x1234, *good)


def test_warm_read_setting(zero_lib):
    """zero_set_warm_read accepts 0 and 1 only (no launch involved)."""
    Z = zero_lib
    for bad in (2, -1):
        assert Z.load().zero_set_warm_read(bad) == Z.ZERO_EINVAL
    for good in (True, False):
        Z.zero_set_warm_read(good)


def test_flatten_needs_no_workspace(zero_lib):
    Z = zero_lib
    for sizes, cap in (([10], 0), ([5, 0, 7000, 3], 100), (list(range(1, 300)), 50)):
        p = Z.zero_plan(sum(sizes), 3, sizes, cap, 8)
        assert Z.zero_flatten_workspace_bytes(p) == 0


def test_plan_rejects_overflowing_layout(zero_lib):
    Z = zero_lib
    with pytest.raises(Z.ZeroError) as ei:
        Z.zero_plan(5, 1 << 30, [1] * 5, 1, 1 << 30)
    assert ei.value.status == Z.ZERO_EINVAL and "padded layout" in str(ei.value)


# ---------------------------------------------------------------------------
# The binding checks tensors against the plan before any C call
# ---------------------------------------------------------------------------

def _bad_args_cases(torch, S, P):
    f32, i16 = torch.float32, torch.int16
    return {
        "short": (torch.empty(S - 1, dtype=f32), "holds"),
        "wide dtype": (torch.empty(S, dtype=torch.float64), "bytes"),
        "strided": (torch.empty(2 * S, dtype=f32)[::2], "contiguous"),
        "16-bit state": (torch.empty(S, dtype=i16), "bytes"),
        "cpu": (torch.empty(S, dtype=f32), "not on a GPU"),
    }


def test_binding_checks_state_tensors(zero_lib):
    import torch
    Z = zero_lib
    p = Z.zero_plan(1000, 4, [600, 400], 512, 8)
    S, P = p.shard_total, p.psi_pad
    good16 = [1 << 30] * 4                      # plain addresses pass through unchecked
    src = Z.GradSrc(Z.ZERO_BF16, good16)
    ok32 = 1 << 34
    import zero_sharded_mixed_02_amd as ZZ
    saved = ZZ.load
    ZZ.load = lambda: (_ for _ in ()).throw(AssertionError("the C library was called"))
    try:
        for name, (x, msg) in _bad_args_cases(torch, S, P).items():
            for slot in ("master", "m", "v"):
                kw = dict(master=ok32, m=ok32, v=ok32)
                kw[slot] = x
                with pytest.raises(ValueError, match=msg):
                    Z.zero_adam_step(p, 0, 1e-4, 0.9, 0.999, 1e-8, 0.25, 1, src, None, kw["master"], kw["m"],
                                     kw["v"], ok32, Z.ZERO_F16, True, stream=0)
            with pytest.raises(ValueError, match=msg):
                Z.zero_adam_step(p, 0, 1e-4, 0.9, 0.999, 1e-8, 0.25, 1, None, x, ok32, ok32, ok32, ok32,
                                 Z.ZERO_F16, True, stream=0)
            with pytest.raises(ValueError, match=msg):
                Z.zero_shard_reduce(p, 0, src, 0.25, x, stream=0)
        # The 16-bit destination: full buffer (psi_pad) or shard (shard_total).
        with pytest.raises(ValueError, match="holds"):
            Z.zero_adam_step(p, 0, 1e-4, 0.9, 0.999, 1e-8, 0.25, 1, src, None, ok32, ok32, ok32,
                             torch.empty(P - 1, dtype=torch.int16), Z.ZERO_F16, True, stream=0)
        with pytest.raises(ValueError, match="bytes"):
            Z.zero_adam_step(p, 0, 1e-4, 0.9, 0.999, 1e-8, 0.25, 1, src, None, ok32, ok32, ok32,
                             torch.empty(S, dtype=torch.float32), Z.ZERO_F16, False, stream=0)
        with pytest.raises(ValueError, match="not on a GPU"):
            Z.zero_adam_step(p, 0, 1e-4, 0.9, 0.999, 1e-8, 0.25, 1, src, None, ok32, ok32, ok32,
                             torch.empty(S, dtype=torch.int16), Z.ZERO_F16, False, stream=0)
    finally:
        ZZ.load = saved


def test_binding_checks_gradient_sources(zero_lib):
    import torch
    Z = zero_lib
    p = Z.zero_plan(1000, 4, [600, 400], 512, 8)
    S, P = p.shard_total, p.psi_pad
    ok32 = 1 << 34
    with pytest.raises(ValueError, match="is_full"):
        Z.GradSrc(Z.ZERO_BF16, [1 << 30] * 4, [0, 1])
    with pytest.raises(ValueError, match="bytes"):
        Z.GradSrc(Z.ZERO_BF16, [torch.empty(S, dtype=torch.float32)] + [1 << 30] * 3)
    with pytest.raises(ValueError, match="contiguous"):
        Z.GradSrc(Z.ZERO_BF16, [torch.empty(2 * S, dtype=torch.int16)[::2]] + [1 << 30] * 3)
    with pytest.raises(ValueError, match="16-bit"):
        Z.GradSrc(Z.ZERO_F32, [1 << 30] * 4)
    cases = {
        "ranks": Z.GradSrc(Z.ZERO_BF16, [1 << 30] * 3),
        "holds": Z.GradSrc(Z.ZERO_BF16, [torch.empty(S - 1, dtype=torch.int16)] + [1 << 30] * 3),
        "full gradient buffer holds": Z.GradSrc(Z.ZERO_BF16, [torch.empty(S, dtype=torch.int16)] + [1 << 30] * 3,
                                                [1, 0, 0, 0]),
        "not on a GPU": Z.GradSrc(Z.ZERO_BF16, [torch.empty(S, dtype=torch.int16)] + [1 << 30] * 3),
    }
    import zero_sharded_mixed_02_amd as ZZ
    saved = ZZ.load
    ZZ.load = lambda: (_ for _ in ()).throw(AssertionError("the C library was called"))
    try:
        for msg, src in cases.items():
            with pytest.raises(ValueError, match=msg):
                Z.zero_adam_step(p, 0, 1e-4, 0.9, 0.999, 1e-8, 0.25, 1, src, None, ok32, ok32, ok32, ok32,
                                 Z.ZERO_F16, True, stream=0)
            with pytest.raises(ValueError, match=msg):
                Z.zero_shard_reduce(p, 0, src, 0.25, ok32, stream=0)
    finally:
        ZZ.load = saved


def test_binding_checks_copy_arguments(zero_lib):
    import torch
    Z = zero_lib
    p = Z.zero_plan(1000, 4, [600, 400], 512, 8)
    q = Z.zero_plan(1000, 3, [600, 400], 0, 1)
    S, P = p.shard_total, p.psi_pad
    import zero_sharded_mixed_02_amd as ZZ
    saved = ZZ.load
    ZZ.load = lambda: (_ for _ in ()).throw(AssertionError("the C library was called"))
    try:
        with pytest.raises(ValueError, match="entries"):
            Z.zero_flatten(p, [1 << 30], Z.ZERO_BF16, 1 << 34, stream=0)
        with pytest.raises(ValueError, match="exactly 400"):
            Z.zero_flatten(p, [1 << 30, torch.empty(401, dtype=torch.int16)], Z.ZERO_BF16, 1 << 34, stream=0)
        with pytest.raises(ValueError, match="holds"):
            Z.zero_flatten(p, [1 << 30, 1 << 31], Z.ZERO_BF16, torch.empty(P - 1, dtype=torch.int16), stream=0)
        with pytest.raises(ValueError, match="entries"):
            Z.zero_gather_pack(p, [1 << 30] * 3, Z.ZERO_F16, 1 << 34, stream=0)
        with pytest.raises(ValueError, match="holds"):
            Z.zero_gather_pack(p, [1 << 30] * 3 + [torch.empty(S - 1, dtype=torch.int16)], Z.ZERO_F16, 1 << 34,
                               stream=0)
        with pytest.raises(ValueError, match="bytes"):
            Z.zero_gather_pack(p, [1 << 30] * 4, Z.ZERO_F32, torch.empty(P, dtype=torch.int16), stream=0)
        with pytest.raises(ValueError, match="unknown dtype"):
            Z.zero_gather_pack(p, [1 << 30] * 4, 7, 1 << 34, stream=0)
        with pytest.raises(ValueError, match="entries"):
            Z.zero_reshard(p, q, 0, [1 << 30] * 3, Z.ZERO_F32, 1 << 34, stream=0)
        with pytest.raises(ValueError, match="holds"):
            Z.zero_reshard(p, q, 0, [1 << 30] * 4, Z.ZERO_F32, torch.empty(q.shard_total - 1), stream=0)
        with pytest.raises(ValueError, match="not on a GPU"):
            Z.zero_reshard(p, q, 0, [1 << 30] * 4, Z.ZERO_F32, torch.empty(q.shard_total), stream=0)
    finally:
        ZZ.load = saved
