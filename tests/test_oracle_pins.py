"""Pins of the CPU oracle to facts fixed outside itself: the numbers the
ZeRO pages print (tests/golden/), closed forms of the Adam recurrence, exact
arithmetic facts, brute force on tiny inputs, and exhaustive checks of the
16-bit conversions against independent references.  No GPU needed."""
import math
import os
import subprocess

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------
# Numbers printed on the pages
# ---------------------------------------------------------------------------

def test_memory_table1_closed_form(oracle_lib):
    O = oracle_lib
    g = {k: v for k, v in read_golden("table1_memory.txt")}
    psi, n_d, k = int(g["psi"]), int(g["n_d"]), int(g["k"])
    mem = O.memory_closed_form(psi, n_d, k)
    for stage in ("dp", "os", "os_g", "os_g_p"):
        assert f"{mem[stage] / 1e9:.1f}" == g[stage], stage
    # The default K is the concept page's 12 bytes of fp32 optimizer state.
    assert O.memory_closed_form(psi, n_d) == mem


@pytest.mark.parametrize("align", [1, 64])
def test_memory_table1_from_layout(oracle_lib, align):
    """The same figures counted from the buffers each stage keeps resident."""
    O = oracle_lib
    g = {k: v for k, v in read_golden("table1_memory.txt")}
    psi, n_d, k = int(g["psi"]), int(g["n_d"]), int(g["k"])
    p = O.plan(psi, n_d, [psi], 0, align)
    for stage in ("dp", "os", "os_g", "os_g_p"):
        assert f"{O.memory_from_layout(p, stage, k) / 1e9:.1f}" == g[stage], (stage, align)


def test_stage_table(oracle_lib):
    O = oracle_lib
    for stage, optim, grads, params in read_golden("stage_table.txt"):
        want = {name for name, flag in (("optim", optim), ("grads", grads), ("params", params))
                if flag == "1"}
        assert O.STAGE_SHARDED[stage] == want


@pytest.mark.parametrize("align", [1, 64])
def test_comm_volume(oracle_lib, align):
    O = oracle_lib
    g = {k: v for k, v in read_golden("comm_volume.txt")}
    psi, n_d = 7_500_000_000, 64
    p = O.plan(psi, n_d, [psi], 0, align)
    vols = {s: O.comm_volume(p, s) for s in ("dp", "os", "os_g", "os_g_p")}
    for s in vols:
        assert vols[s]["elements"] == int(g[s]) * p.psi_pad
        # The off-rank share is exactly (n_d - 1) / n_d of it.
        assert vols[s]["off_rank_elements"] * n_d == vols[s]["elements"] * (n_d - 1)
    assert vols["os_g_p"]["elements"] / vols["dp"]["elements"] == float(g["ratio_os_g_p_over_dp"])
    if align == 1:   # psi divides evenly: no padding, exactly 2 Psi and 3 Psi
        assert vols["dp"]["elements"] == 15_000_000_000
        assert vols["os_g_p"]["elements"] == 22_500_000_000


def test_ownership_abcd(oracle_lib):
    """Four equal blocks over four ranks: rank i owns the i-th block."""
    O = oracle_lib
    rows = read_golden("ownership_abcd.txt")
    blocks = "ABCD"
    block_len = 5
    p = O.plan(4 * block_len, 4, [block_len] * 4, 0, 1)
    for rank, name in rows:
        lo, hi = p.owner_range(0, int(rank))
        assert (lo // block_len, hi - lo) == (blocks.index(name), block_len)


# ---------------------------------------------------------------------------
# Plan: closed cases and brute force
# ---------------------------------------------------------------------------

def test_plan_closed_cases(oracle_lib):
    O = oracle_lib
    assert O.plan(7_500_000_000, 64, [7_500_000_000], 0, 1).shard_total == 117_187_500
    assert O.plan(13_000_000_000, 16, [13_000_000_000], 0, 1).shard_total == 812_500_000
    h = 8192
    L = 12 * h * h + 13 * h
    p5 = O.plan(L, 64, [L], 0, 64)
    assert (L, p5.shard_total, p5.psi_pad - L) == (805_412_864, 12_584_576, 0)
    p1 = O.plan(1_000_003, 4, [1_000_003], 0, 64)
    assert (p1.psi_pad, p1.shard_total) == (1_000_192, 250_048)


def test_plan_gpt2_buckets(oracle_lib):
    from synth.workloads import gpt2_small_sizes
    O = oracle_lib
    sizes = gpt2_small_sizes()
    assert len(sizes) == 193 and sum(sizes) == 123_651_840
    p = O.plan(sum(sizes), 8, sizes, 1 << 24, 64)
    assert len(p.buckets) == 7
    assert p.psi_pad == 123_652_608
    assert p.shard_total == 15_456_576


def _random_plans(seed, count):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        n_d = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 64]))
        align = int(rng.choice([1, 64]))
        nt = int(rng.integers(0, 9))
        sizes = [int(x) for x in rng.integers(0, 40, size=nt)]
        if nt and rng.random() < 0.3:
            sizes[int(rng.integers(0, nt))] = 0
        cap = int(rng.choice([0, 1, 7, 30, 100]))
        yield n_d, align, sizes, cap


def test_plan_bruteforce_invariants(oracle_lib):
    O = oracle_lib
    for n_d, align, sizes, cap in _random_plans(7, 400):
        psi = sum(sizes)
        p = O.plan(psi, n_d, sizes, cap, align)
        # Every real element belongs to exactly one rank's shard.
        owner = np.full(p.psi_pad, -1)
        for r in range(n_d):
            for b in range(len(p.buckets)):
                lo, hi = p.owner_range(b, r)
                assert np.all(owner[lo:hi] == -1)
                owner[lo:hi] = r
        assert np.all(owner >= 0)
        # Pads < n_d * align per bucket, all shards the same size.
        for bk in p.buckets:
            assert 0 <= bk.padded - bk.numel < n_d * align
            assert bk.padded % (n_d * align) == 0 and bk.shard_numel * n_d == bk.padded
        # Tensors: contiguous, in list order, never split, inside their bucket.
        for t, n in enumerate(sizes):
            bk = p.buckets[p.tensor_bucket[t]]
            assert bk.flat_off <= p.tensor_off[t] and p.tensor_off[t] + n <= bk.flat_off + bk.numel
        # Greedy cap rule: a bucket holding several tensors stays within the
        # cap, and every bucket but the last was closed only because its
        # successor's first tensor would have taken it past the cap (a bucket
        # may be filled exactly to the cap).
        for b, bk in enumerate(p.buckets):
            members = [t for t in range(len(sizes)) if p.tensor_bucket[t] == b]
            if cap and len(members) > 1:
                assert bk.numel <= cap
            if cap and b + 1 < len(p.buckets):
                first_next = min(t for t in range(len(sizes)) if p.tensor_bucket[t] == b + 1)
                assert bk.numel + sizes[first_next] > cap
        # flatten / unflatten round trip, pads zero.
        rng = np.random.default_rng(psi)
        ts = [rng.integers(1, 2 ** 16, size=n, dtype=np.uint16) for n in sizes]
        flat = O.flatten(p, ts)
        for t, x in zip(O.unflatten(p, flat), ts):
            assert np.array_equal(t, x)
        for bk in p.buckets:
            assert np.all(flat[bk.flat_off + bk.numel: bk.flat_off + bk.padded] == 0)
        # gather_pack of every rank's shard reproduces the flat buffer.
        shards = [O.shard_of(p, r, flat) for r in range(n_d)]
        assert np.array_equal(O.gather_pack(p, shards), flat)


def test_runner_positions_match_shard_of(oracle_lib):
    """The oracle driver's index -> flat position map is the plan's ownership
    rule: it equals shard_of applied to the identity, and flags exactly the
    padding."""
    from dataclasses import replace
    from oracle.runner import OracleRun
    from synth.workloads import Config
    O = oracle_lib
    for n_d, align, sizes, cap in _random_plans(31, 80):
        if not sizes:
            continue
        cfg = Config("t", tuple(sizes), n_d=n_d, gdt=O.BF16, pdt=O.F16, bucket_cap=cap, align=align)
        for rank in range(n_d):
            run = OracleRun(replace(cfg, owner=rank))
            p = run.plan
            ident = np.arange(p.psi_pad, dtype=np.int64)
            assert np.array_equal(run.pos, O.shard_of(p, rank, ident))
            assert np.array_equal(run.pad, np.array([p.is_pad(int(x)) for x in run.pos], bool))


def test_plan_rejects_bad_arguments(oracle_lib):
    O = oracle_lib
    with pytest.raises(ValueError):
        O.plan(10, 0, [10])
    with pytest.raises(ValueError):
        O.plan(11, 2, [10])
    with pytest.raises(ValueError):
        O.plan(10, 2, [10], 0, 0)


# ---------------------------------------------------------------------------
# Casts
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def cast_checker(oracle_lib, tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("native") / "cast_exhaustive")
    src = os.path.join(ROOT, "tests", "native", "cast_exhaustive.c")
    libdir = os.path.join(ROOT, "oracle")
    subprocess.run(["gcc", "-O2", "-mf16c", "-fopenmp", src, "-o", exe, "-L" + libdir, "-loracle",
                    "-Wl,-rpath," + libdir], check=True)
    return exe


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_casts_exhaustive(cast_checker, fmt):
    """All 2^32 fp32 patterns: fp16 against the F16C instruction, bf16
    against integer round-half-even of the dropped bits."""
    r = subprocess.run([cast_checker, fmt], capture_output=True, text=True, timeout=600)
    if r.returncode == 2:
        pytest.skip(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr


def test_cast_special_values(oracle_lib):
    O = oracle_lib
    f = np.float32
    cases16 = [(0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3C00), (65504.0, 0x7BFF), (65520.0, 0x7C00),
               (65519.99, 0x7BFF), (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000),
               (1.5 * 2.0 ** -25, 0x0001), (float("inf"), 0x7C00), (-float("inf"), 0xFC00)]
    for x, want in cases16:
        assert O.f32_to_16(np.array([x], f), O.F16)[0] == want, x
    casesbf = [(1.0, 0x3F80), (-2.0, 0xC000), (1.0 + 2 ** -8, 0x3F80), (1.0 + 3 * 2 ** -8, 0x3F82)]
    for x, want in casesbf:
        assert O.f32_to_16(np.array([x], f), O.BF16)[0] == want, x
    nan = O.f32_to_16(np.array([np.nan], f), O.BF16)[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F)


def test_cast_matches_numpy_float16(oracle_lib):
    """fp16 against numpy's own conversion on a large random sample."""
    O = oracle_lib
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(O.f32_to_16(x, O.F16), want)


# ---------------------------------------------------------------------------
# Reduction
# ---------------------------------------------------------------------------

def _bits(x, dt, O):
    return O.f32_to_16(np.asarray(x, np.float32), dt)


def test_reduce_identical_slices_exact(oracle_lib):
    """n_d identical 16-bit slices sum exactly (at most 11 + 6 significant
    bits), and the power-of-two mean returns the slice itself."""
    O = oracle_lib
    rng = np.random.default_rng(1)
    for dt in (O.F16, O.BF16):
        g = _bits(rng.normal(0, 1e-3, 4096), dt, O)
        for n_d in (1, 2, 4, 8, 16, 64):
            red = O.reduce([g] * n_d, dt, 1.0 / n_d)
            assert np.array_equal(red, O.value16(g, dt).astype(np.float32))


def test_reduce_fixed_rank_order(oracle_lib):
    """1 + 2^24 - 2^24 folds to 0 left to right (the 1 is absorbed), but to 1
    in any order that adds the large terms first: the fold order is 0..n-1."""
    O = oracle_lib
    dt = O.BF16
    g = [_bits([1.0], dt, O), _bits([2.0 ** 24], dt, O), _bits([-(2.0 ** 24)], dt, O)]
    assert O.reduce(g, dt, 1.0)[0] == 0.0
    assert O.reduce([g[1], g[2], g[0]], dt, 1.0)[0] == 1.0


def test_reduce_error_bound(oracle_lib):
    """|fold - exact sum| <= (n-1) * 2^-24 * sum |g_q| (recursive summation
    bound), with the exact sum from math.fsum."""
    O = oracle_lib
    rng = np.random.default_rng(2)
    for dt, n_d in ((O.BF16, 64), (O.F16, 16), (O.F16, 3)):
        slices = [_bits(rng.normal(0, 1e-3, 2000), dt, O) for _ in range(n_d)]
        red = O.reduce(slices, dt, 1.0)
        vals = np.stack([O.value16(s, dt) for s in slices])
        for j in range(0, 2000, 7):
            exact = math.fsum(vals[:, j])
            bound = (n_d - 1) * 2.0 ** -24 * math.fsum(np.abs(vals[:, j]))
            assert abs(float(red[j]) - exact) <= bound


def test_reduce_keeps_negative_zero(oracle_lib):
    O = oracle_lib
    z = np.array([0x8000], np.uint16)
    red = O.reduce([z, z], O.F16, 0.5)
    assert red[0] == 0.0 and np.signbit(red[0])


# ---------------------------------------------------------------------------
# Adam
# ---------------------------------------------------------------------------

LR, B1, B2, EPS = 1e-4, 0.9, 0.999, 1e-8


def test_adam_constants_rounded_once(oracle_lib):
    O = oracle_lib
    c = O.adam_consts(LR, B1, B2, EPS, 1 / 64, 3)
    assert c[1] == np.float32(1 - 0.9) and c[1] != np.float32(1) - np.float32(0.9)
    assert c[4] == np.float32(1 - 0.9 ** 3) and c[5] == np.float32(1 - 0.999 ** 3)
    assert c[8] == np.float32(2.0 ** -6)


def _adam_run(O, gseq, w0=0.02):
    n = gseq.shape[1]
    w = np.full(n, w0, np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    out = []
    for t, g in enumerate(gseq, start=1):
        c = O.adam_consts(LR, B1, B2, EPS, 1.0, t)
        before = w.copy()
        O.adam(np.ascontiguousarray(g, np.float32), w, m, v, c, O.F16)
        out.append((before.astype(np.float64), w.astype(np.float64), m.copy(), v.copy()))
    return out


def test_adam_first_step_closed_form(oracle_lib):
    """From m = v = 0 the bias-corrected moments are g and g^2, so the first
    step is lr * g / (|g| + eps)."""
    O = oracle_lib
    g = np.array([[1e-3, -2e-3, 5e-7, -3.0, 1e-9, 0.0]], np.float32)
    (before, after, m, v), = _adam_run(O, g)
    gd = g[0].astype(np.float64)
    want = before - LR * gd / (np.abs(gd) + EPS)
    assert np.allclose(after, want, rtol=0, atol=4 * 2.0 ** -24 * 0.02 + 1e-12)


def test_adam_impulse_response(oracle_lib):
    """A single gradient g at step 1 then zeros: at step k the corrected
    moments are b1^(k-1) (1-b1) g / (1-b1^k) and b2^(k-1) (1-b2) g^2 / (1-b2^k),
    which separates beta1 from beta2 and pins both bias corrections."""
    O = oracle_lib
    g0 = np.array([1e-3, -4e-2, 7.0], np.float32)
    gseq = np.zeros((6, g0.size), np.float32)
    gseq[0] = g0
    for k, (before, after, m, v) in enumerate(_adam_run(O, gseq), start=1):
        gd = g0.astype(np.float64)
        mh = B1 ** (k - 1) * (1 - B1) * gd / (1 - B1 ** k)
        vh = B2 ** (k - 1) * (1 - B2) * gd * gd / (1 - B2 ** k)
        step = LR * mh / (np.sqrt(vh) + EPS)
        assert np.allclose(before - after, step, rtol=1e-4, atol=1e-12), k
        assert np.allclose(m, B1 ** (k - 1) * (1 - B1) * gd, rtol=1e-5)


def test_adam_zero_gradient_element(oracle_lib):
    O = oracle_lib
    w = np.array([0.5, -0.25], np.float32)
    m = np.array([1e-3, -2e-3], np.float32)
    v = np.array([0.0, 0.0], np.float32)
    c = O.adam_consts(LR, B1, B2, EPS, 1.0, 4)
    O.adam(np.zeros(2, np.float32), w2 := w.copy(), m2 := m.copy(), v2 := v.copy(), c, O.F16)
    assert np.array_equal(m2, (np.float32(B1) * m).astype(np.float32))
    assert np.array_equal(v2, v)
    # v = 0 makes the denominator eps: the weight moves by lr * mh / eps.
    mh = m2.astype(np.float64) / np.float32(1 - B1 ** 4)
    assert np.allclose(w - w2, LR * mh / EPS, rtol=1e-5)


def test_adam_pad_elements_stay_zero(oracle_lib):
    O = oracle_lib
    z = np.zeros(16, np.float32)
    w, m, v = z.copy(), z.copy(), z.copy()
    for t in range(1, 5):
        p = O.adam(z, w, m, v, O.adam_consts(LR, B1, B2, EPS, 1.0, t), O.BF16)
        assert not np.any(w) and not np.any(m) and not np.any(v) and not np.any(p)
        assert not np.any(np.signbit(w))


def test_adam_accuracy_against_fp64(oracle_lib):
    """The fp32 recurrence tracks the fp64 one over 10 steps to a few ulps of
    the weight plus a few ulps of the summed steps."""
    O = oracle_lib
    rng = np.random.default_rng(5)
    n = 5000
    w32 = rng.normal(0, 0.02, n).astype(np.float32)
    w64 = w32.astype(np.float64)
    m32, v32 = np.zeros(n, np.float32), np.zeros(n, np.float32)
    m64, v64 = np.zeros(n), np.zeros(n)
    for t in range(1, 11):
        g = rng.normal(0, 1e-3, n).astype(np.float32)
        O.adam(g, w32, m32, v32, O.adam_consts(LR, B1, B2, EPS, 1.0, t), O.F16)
        O.adam_f64(g.astype(np.float64), w64, m64, v64, LR, B1, B2, EPS, t)
        err = np.abs(w32.astype(np.float64) - w64)
        # Each step adds at most a couple of ulps of w and a few ulps of the
        # lr-sized update.
        bound = t * (2.0 ** -22 * np.abs(w64) + 2.0 ** -18 * LR)
        assert np.all(err <= bound), t
        # Moments: cancellation makes relative error meaningless near zero, so
        # the bound is a few ulps of the largest term per step.
        assert np.all(np.abs(m32 - m64) <= t * 2.0 ** -22 * np.abs(g).max())
        assert np.all(np.abs(v32 - v64) <= t * 2.0 ** -22 * np.abs(v64).max())


def _adam_f32_sequence(c, g, w, m, v):
    """The stated update, each binary operation evaluated by numpy in IEEE
    binary32 (one rounding per operation, no fused multiply-add)."""
    f = np.float32
    b1, c1, b2, c2, bc1, bc2, lr, eps = (f(x) for x in c[:8])
    mn = f(b1 * m) + f(c1 * g)
    vn = f(b2 * v) + f(c2 * f(g * g))
    den = f(np.sqrt(f(vn / bc2))) + eps
    wn = w - f(lr * f(f(mn / bc1) / den))
    return f(wn), f(mn), f(vn)


def _fma32(a, b, c):
    """fp32 fused multiply-add: the product of two fp32 values is exact in
    fp64, so a*b + c rounded once to fp64 and then to fp32 (double rounding
    is possible only at rare ties; enough to show the inputs are sensitive)."""
    return np.float32(np.float64(a) * np.float64(b) + np.float64(c))


def test_adam_one_rounding_per_operation(oracle_lib):
    """The oracle rounds after every operation of the update and fuses none:
    on inputs where contracting any multiply-add of the rule (b1*m + c1*g,
    b2*v + c2*g^2, w - lr*r) changes the fp32 result, it equals the
    operation-by-operation binary32 evaluation bit for bit."""
    O = oracle_lib
    rng = np.random.default_rng(21)
    n = 4096
    g = rng.normal(0, 1e-3, n).astype(np.float32)
    w = rng.normal(0, 0.02, n).astype(np.float32)
    m = rng.normal(0, 1e-4, n).astype(np.float32)
    v = np.abs(rng.normal(0, 1e-7, n)).astype(np.float32)
    c = O.adam_consts(LR, B1, B2, EPS, 1.0, 7)
    ww, mm, vv = w.copy(), m.copy(), v.copy()
    O.adam(g, ww, mm, vv, c, O.F16)
    want = [_adam_f32_sequence(c, g[i], w[i], m[i], v[i]) for i in range(n)]
    got = list(zip(ww, mm, vv))
    assert all(np.float32(a).view(np.uint32) == np.float32(b).view(np.uint32)
               for gw, ww_ in zip(got, want) for a, b in zip(gw, ww_))
    # The inputs have teeth: each contraction changes some results.
    f = np.float32
    fused_m = sum(_fma32(c[0], m[i], f(c[1] * g[i])) != want[i][1] for i in range(n))
    fused_v = sum(_fma32(c[2], v[i], f(c[3] * f(g[i] * g[i]))) != want[i][2] for i in range(n))
    fused_w = 0
    for i in range(n):
        den = f(np.sqrt(f(want[i][2] / c[5]))) + c[7]
        r = f(f(want[i][1] / c[4]) / den)
        fused_w += _fma32(-c[6], r, w[i]) != want[i][0]
    assert fused_m > 0 and fused_v > 0 and fused_w > 0, (fused_m, fused_v, fused_w)


def test_decode16_exhaustive(oracle_lib):
    """Every 16-bit pattern decodes to its IEEE value: binary16 against
    numpy's float16, bfloat16 against the fp32 whose upper half it is."""
    O = oracle_lib
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.value16(h, O.F16)
    want = h.view(np.float16).astype(np.float64)
    assert np.array_equal(got, want, equal_nan=True)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    got = O.value16(h, O.BF16)
    with np.errstate(invalid="ignore"):     # signalling-NaN patterns widen quietly
        want = (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(got, want, equal_nan=True)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_adam_param_is_rounded_master(oracle_lib):
    O = oracle_lib
    rng = np.random.default_rng(6)
    w = rng.normal(0, 0.02, 1000).astype(np.float32)
    m, v = np.zeros_like(w), np.zeros_like(w)
    g = rng.normal(0, 1e-3, 1000).astype(np.float32)
    for dt in (O.F16, O.BF16):
        ww, mm, vv = w.copy(), m.copy(), v.copy()
        p = O.adam(g, ww, mm, vv, O.adam_consts(LR, B1, B2, EPS, 1.0, 1), dt)
        assert np.array_equal(p, O.f32_to_16(ww, dt))


# ---------------------------------------------------------------------------
# Sharded == unsharded (brute force on tiny inputs)
# ---------------------------------------------------------------------------

def test_sharded_equals_unsharded(oracle_lib):
    """Running every rank's sharded step and concatenating the shards gives
    exactly the Adam step on the whole flat buffer, for every rank and step."""
    O = oracle_lib
    rng = np.random.default_rng(11)
    hp = O.Hyper(LR, B1, B2, EPS, 1.0)
    for n_d, align, sizes, cap in _random_plans(13, 60):
        psi = sum(sizes)
        gdt, pdt = (O.F16, O.BF16) if rng.random() < 0.5 else (O.BF16, O.F16)
        hp.grad_scale = 1.0 / n_d
        p = O.plan(psi, n_d, sizes, cap, align)
        tensors0 = [rng.normal(0, 0.02, n).astype(np.float32) for n in sizes]
        master_full = O.flatten(p, tensors0) if sizes else np.zeros(p.psi_pad, np.float32)
        mf, vf = np.zeros(p.psi_pad, np.float32), np.zeros(p.psi_pad, np.float32)
        wf = master_full.copy()
        shard_state = [[O.shard_of(p, r, master_full).copy(), np.zeros(p.shard_total, np.float32),
                        np.zeros(p.shard_total, np.float32)] for r in range(n_d)]
        for t in (1, 2, 3):
            # Each rank's full, flattened 16-bit gradient.
            fulls = []
            for q in range(n_d):
                gt = [_bits(rng.normal(0, 1e-3, n), gdt, O) for n in sizes]
                fulls.append(O.flatten(p, gt) if sizes else np.zeros(p.psi_pad, np.uint16))
            # Unsharded: reduce and update the whole flat buffer.
            c = O.adam_consts(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale, t)
            g_all = O.reduce(fulls, gdt, float(c[8]))
            p_all = O.adam(g_all, wf, mf, vf, c, pdt)
            # Sharded: every owner reduces its partition and updates its shard.
            full_params = np.zeros(p.psi_pad, np.uint16)
            for r in range(n_d):
                w, m, v = shard_state[r]
                ps = O.shard_step(O.owner_slices_from_full(p, r, fulls), gdt, hp, t, w, m, v, pdt)
                O.place_shard(p, r, ps, full_params)
            assert np.array_equal(full_params, p_all)
            assert np.array_equal(O.gather_pack(p, [s[0] for s in shard_state]).view(np.uint32),
                                  wf.view(np.uint32))
            assert np.array_equal(O.gather_pack(p, [s[1] for s in shard_state]), mf)


def test_single_rank_is_plain_mixed_precision_adam(oracle_lib):
    O = oracle_lib
    rng = np.random.default_rng(12)
    g = _bits(rng.normal(0, 1e-3, 999), O.F16, O)
    w = rng.normal(0, 0.02, 999).astype(np.float32)
    w1, m1, v1 = w.copy(), np.zeros_like(w), np.zeros_like(w)
    p1 = O.shard_step([g], O.F16, O.Hyper(LR, B1, B2, EPS, 1.0), 1, w1, m1, v1, O.F16)
    w2, m2, v2 = w.copy(), np.zeros_like(w), np.zeros_like(w)
    p2 = O.adam(O.value16(g, O.F16).astype(np.float32), w2, m2, v2,
                O.adam_consts(LR, B1, B2, EPS, 1.0, 1), O.F16)
    assert np.array_equal(p1, p2) and np.array_equal(w1, w2)


# ---------------------------------------------------------------------------
# Reshard (a sharded state laid out for another N_d / bucketing)
# ---------------------------------------------------------------------------

def test_reshard_invariants(oracle_lib):
    """Every tensor element keeps its value across a reshard, padding is
    zero, resharding back gives the original shards, and resharding onto the
    same plan is the identity."""
    O = oracle_lib
    rng = np.random.default_rng(41)
    for (n_d, align, sizes, cap), (n_d2, align2, _, cap2) in zip(_random_plans(43, 80), _random_plans(47, 80)):
        psi = sum(sizes)
        src = O.plan(psi, n_d, sizes, cap, align)
        dst = O.plan(psi, n_d2, sizes, cap2, align2)
        tensors = [rng.standard_normal(n).astype(np.float32) for n in sizes]
        flat = O.flatten(src, tensors) if sizes else np.zeros(src.psi_pad, np.float32)
        shards = [O.shard_of(src, r, flat) for r in range(n_d)]
        new = [O.reshard(src, dst, r, shards) for r in range(n_d2)]
        new_flat = O.gather_pack(dst, new)
        for t, x in enumerate(O.unflatten(dst, new_flat)):
            assert np.array_equal(x, tensors[t])
        for bk in dst.buckets:
            assert not np.any(new_flat[bk.flat_off + bk.numel: bk.flat_off + bk.padded])
        back = [O.reshard(dst, src, r, new) for r in range(n_d)]
        for a, b in zip(back, shards):
            assert np.array_equal(a, b)
        same = [O.reshard(src, src, r, shards) for r in range(n_d)]
        for a, b in zip(same, shards):
            assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# Stage 3: the per-layer sequence (gather the pre-step shards, step, the owner
# keeps its new 16-bit shard for the next gather)
# ---------------------------------------------------------------------------

def _stage3_expected_full(O, cfg, p, layer):
    """The full layer as every rank holds it before any step: the
    round-to-nearest-even 16-bit value of each initial master weight, zero in
    the padding.  Computed from the input definition and numpy's float16
    conversion, without the oracle's gather or its casts."""
    import synth
    pos = np.arange(p.psi_pad, dtype=np.int64)
    pad = np.zeros(p.psi_pad, bool)
    for bk in p.buckets:
        pad[bk.flat_off + bk.numel: bk.flat_off + bk.padded] = True
    w0 = synth.master_values(cfg.seed, pos + layer * p.psi_pad, cfg.sigma_w, pad)
    return w0.astype(np.float16).view(np.uint16)


def test_stage3_sequence(oracle_lib):
    """The oracle's Stage-3 layer step follows the pages' order (mind-map
    page, how a GPU that keeps a quarter computes: the layer's parameters are
    gathered for the computation, then the owner updates its part and keeps
    it; concept page, "three stages" table, Stage-3 row: parameters are
    gathered per layer and only the owner's shard stays resident).  Over three
    layers and two steps, with an owner other than rank 0 and several buckets:
    each layer's gathered buffer equals the layer as the shards stood before
    that layer's step -- at t = 1 the rounded initial masters, at t = 2 the
    same with the owner's block replaced by step 1's parameters -- the owner's
    shard after every step is the rounding of its master, and no other shard
    ever changes."""
    from oracle.runner import OracleRun
    from synth.workloads import Config, layer_sizes
    O = oracle_lib
    cfg = Config("stage3-tiny", tuple(layer_sizes(8)), n_d=4, gdt=O.BF16, pdt=O.F16, stage=3,
                 owner=2, bucket_cap=200, align=8, steps=2, layers=3, seed=9)
    run = OracleRun(cfg)
    p = run.plan
    assert len(p.buckets) > 1 and cfg.owner != 0
    expected = [_stage3_expected_full(O, cfg, p, layer) for layer in range(cfg.layers)]
    owner_pos = np.concatenate([np.arange(*p.owner_range(b, cfg.owner)) for b in range(len(p.buckets))])
    others0 = [[run.layers[layer]["shards"][q].copy() for q in range(cfg.n_d)] for layer in range(cfg.layers)]
    for t in (1, 2):
        for layer in range(cfg.layers):
            run.fill_grads(t, layer)
            run.step(t, layer)
            st = run.state(layer)
            assert np.array_equal(st["gathered"], expected[layer]), (t, layer)
            rounded = st["master"].astype(np.float16).view(np.uint16)
            assert np.array_equal(st["shards"][cfg.owner], rounded), (t, layer)
            for q in range(cfg.n_d):
                if q != cfg.owner:
                    assert np.array_equal(st["shards"][q], others0[layer][q]), (t, layer, q)
            # What the next gather of this layer must see.
            expected[layer] = expected[layer].copy()
            expected[layer][owner_pos] = rounded
    # Step 2 really changed the owner's block relative to the initial layer.
    assert not np.array_equal(expected[0], _stage3_expected_full(O, cfg, p, 0))
