"""GPU parity of the fused shard step (zero_adam_step), the unfused pair
(zero_shard_reduce + zero_adam_step from the reduced gradient), and the
Stage-3 layer loop, against the CPU oracle on the same seeded inputs.

Small workloads are compared element by element over the whole shard; they
still span many workgroups, several buckets and a ragged, padded tail."""
from dataclasses import replace

import numpy as np
import pytest

from synth import BF16, F16, F32
from synth.workloads import WORKLOADS, Config, GpuRun, small_config, with_owner
from tests.parity import assert_f32, assert_p16, assert_state

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _sync():
    import torch
    torch.cuda.synchronize()


SMALL_CASES = {
    "tiny-owner0": WORKLOADS["tiny"],
    "tiny-owner3-pad": with_owner(WORKLOADS["tiny"], 3),
    "tiny-bf16-owner2": replace(WORKLOADS["tiny"], gdt=BF16, pdt=BF16, owner=2),
    "tiny-align1-elem": replace(WORKLOADS["tiny"], align=1, owner=3),
    "nd3-generic": small_config(77_777, 3, BF16, F16, owner=1, steps=2, seed=7),
    "nd1": small_config(50_001, 1, F16, BF16, owner=0, steps=2, seed=8),
    "nd64-lastrank": small_config(300_000, 64, BF16, F16, owner=63, steps=2, seed=9),
    "stage1-nd16-allfull-mix": small_config(120_000, 16, F16, F16, owner=5, steps=3, seed=10, stage=1,
                                            mix=True, full_ranks=tuple(range(16))),
    "stage1-nd5-somefull": small_config(99_999, 5, BF16, BF16, owner=2, steps=2, seed=12, stage=1,
                                        mix=True, full_ranks=(0, 2, 4)),
    "multibucket-nd4": Config("multibucket", tuple([37, 0, 1000, 5, 12_345, 64, 7] * 9), n_d=4,
                              gdt=BF16, pdt=F16, owner=1, bucket_cap=2000, steps=2, seed=13),
    "manybuckets-nd4-align8": Config("manybuckets", tuple([37] * 150), n_d=4, gdt=F16, pdt=F16,
                                     owner=3, bucket_cap=37, align=8, steps=2, seed=14),
    "smaller-than-nd-align": small_config(10, 4, BF16, F16, owner=2, steps=2, seed=15),
    # Align 1: shard lengths and offsets not multiples of 4.  Owner 0 of the
    # tiny workload runs the vector kernel with a 1-element tail; the buckets
    # below mix pieces with leading elements, tails, and pieces whose offsets
    # disagree modulo 4 (element kernel).
    "align1-owner0-tail": replace(WORKLOADS["tiny"], align=1, owner=0),
    "align1-multibucket-heads": Config("a1mb", (1001, 2002, 3003, 4004, 5005, 6006, 7, 30_001), n_d=3,
                                       gdt=BF16, pdt=F16, owner=1, bucket_cap=5000, align=1, steps=2, seed=18),
    "align1-stage1-full": small_config(100_010, 2, F16, BF16, owner=1, steps=2, seed=19, stage=1, align=1,
                                       full_ranks=(0, 1)),
    "align2-nd5-heads": Config("a2", (999, 12_347, 5, 70_001), n_d=5, gdt=F16, pdt=F16, owner=3,
                               bucket_cap=13_000, align=2, steps=2, seed=20),
}


def run_pair(cfg, t_values=None):
    from oracle.runner import OracleRun
    run, ref = GpuRun(cfg), OracleRun(cfg)
    for t in (t_values or range(1, cfg.steps + 1)):
        run.fill_grads(t)
        ref.fill_grads(t)
        run.step(t)
        ref.step(t)
    _sync()
    return run, ref


@pytest.mark.parametrize("name", list(SMALL_CASES))
def test_fused_step_matches_oracle(gpu, oracle_lib, name):
    cfg = SMALL_CASES[name]
    say(f"[fused step] {name}: psi={cfg.psi} n_d={cfg.n_d} owner={cfg.owner} stage={cfg.stage} "
        f"align={cfg.align} steps={cfg.steps}")
    run, ref = run_pair(cfg)
    got, want = run.fetch(), ref.state()
    assert_state(got, want, cfg.pdt, name)


def test_large_step_numbers(gpu, oracle_lib):
    cfg = replace(WORKLOADS["tiny"], steps=3)
    say("[fused step] tiny at t = 998, 999, 1000")
    run, ref = run_pair(cfg, t_values=[998, 999, 1000])
    assert_state(run.fetch(), ref.state(), cfg.pdt, "t~1000")


def test_gpt2_small_ten_steps(gpu, oracle_lib):
    cfg = WORKLOADS["gpt2-small"]
    say(f"[fused step] gpt2-small: {len(cfg.sizes)} tensors, n_d={cfg.n_d}, 10 steps")
    run, ref = run_pair(cfg)
    got, want = run.fetch(), ref.state()
    r = assert_state(got, want, cfg.pdt, "gpt2")
    say(f"  {r}")


def test_gpt2_small_every_owner_one_step(gpu, oracle_lib):
    for owner in range(8):
        cfg = with_owner(replace(WORKLOADS["gpt2-small"], steps=1), owner)
        say(f"[fused step] gpt2-small owner {owner}")
        run, ref = run_pair(cfg)
        assert_state(run.fetch(), ref.state(), cfg.pdt, f"gpt2 owner {owner}")
        del run


@pytest.mark.parametrize("name", ["tiny-owner3-pad", "nd3-generic", "stage1-nd5-somefull",
                                  "manybuckets-nd4-align8", "tiny-align1-elem", "align1-owner0-tail",
                                  "align1-multibucket-heads", "align2-nd5-heads"])
def test_fused_equals_unfused(gpu, oracle_lib, name):
    """zero_shard_reduce then zero_adam_step(reduced) gives exactly the fused
    step; the reduced gradient itself matches the oracle's fold."""
    import torch
    import oracle as O
    from oracle.runner import OracleRun
    cfg = SMALL_CASES[name]
    say(f"[fused == unfused] {name}")
    fused, unfused, ref = GpuRun(cfg), GpuRun(cfg), OracleRun(cfg)
    red = torch.empty(unfused.S, dtype=torch.float32, device=gpu)
    for t in range(1, cfg.steps + 1):
        fused.fill_grads(t)
        unfused.fill_grads(t)
        ref.fill_grads(t)
        fused.step(t)
        unfused.reduce(red)
        unfused.step_from_reduced(t, red)
        _sync()
        want_red = O.reduce(ref.layers[0]["slices"], cfg.gdt, float(np.float32(cfg.grad_scale)))
        assert_f32(red.cpu().numpy(), want_red, "reduced", bitwise=True)
    a, b = fused.fetch(), unfused.fetch()
    for k in ("master", "m", "v"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    assert np.array_equal(a["full"], b["full"])


@pytest.mark.parametrize("name", ["multibucket-nd4", "manybuckets-nd4-align8", "stage1-nd5-somefull", "gpt2"])
def test_per_bucket_plans_equal_one_plan(gpu, name):
    """A step as one zero_adam_step per bucket, each with a plan of that
    bucket's tensors alone and pointers into the same buffers, equals the
    step with the whole multi-bucket plan, bit for bit (the concept page's
    trade-off 1: buckets are independent units of the step)."""
    cfg = WORKLOADS["gpt2-small"] if name == "gpt2" else SMALL_CASES[name]
    say(f"[per-bucket plans] {name}: {len(cfg.sizes)} tensors")
    whole, split = GpuRun(cfg), GpuRun(cfg)
    assert len(split.bucket_plans()) == whole.plan.n_buckets
    for t in (1, 2):
        whole.fill_grads(t)
        split.fill_grads(t)
        whole.step(t)
        split.step_per_bucket(t)
    _sync()
    a, b = whole.fetch(), split.fetch()
    for k in ("master", "m", "v"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k
    assert np.array_equal(a["full"], b["full"])


def test_reduce_more_ranks_than_one_launch(gpu, oracle_lib):
    """n_d = 200 > ZERO_MAX_RANKS: the reduction continues across launches in
    rank order; the fused path refuses, the reduced path is exact."""
    import torch
    import oracle as O
    import zero_sharded_mixed_02_amd as Z
    from oracle.runner import OracleRun
    cfg = small_config(100_000, 200, BF16, F16, owner=123, steps=2, seed=16, align=8)
    say("[reduce] n_d=200 over two launches")
    run, ref = GpuRun(cfg), OracleRun(cfg)
    red = torch.empty(run.S, dtype=torch.float32, device=gpu)
    for t in (1, 2):
        run.fill_grads(t)
        ref.fill_grads(t)
        run.reduce(red)
        run.step_from_reduced(t, red)
        ref.step(t)
        _sync()
        want_red = O.reduce(ref.layers[0]["slices"], cfg.gdt, float(np.float32(cfg.grad_scale)))
        assert_f32(red.cpu().numpy(), want_red, "reduced", bitwise=True)
    assert_state(run.fetch(), ref.state(), cfg.pdt, "n_d=200")
    with pytest.raises(Z.ZeroError) as ei:
        run.step(3)
    assert ei.value.status == Z.ZERO_EUNSUPPORTED


@pytest.mark.parametrize("window", [(0, 0), (50, 10), (300, 1), (-1, 0)])
def test_write_windows_change_nothing(gpu, oracle_lib, zero_lib, window):
    """The store timing of zero_set_write_window leaves every result bit
    unchanged: the fused step at n_d = 64 and 16 (compiled rank counts) and 5
    (runtime count), and the reduction at n_d = 200 (two launches), each equal
    to the oracle with windows off, forced (including a 10 ns opening in a
    3 us period) and automatic."""
    import torch
    import oracle as O
    from oracle.runner import OracleRun
    Z = zero_lib
    say(f"[write window] period/open = {window}")
    Z.zero_set_write_window(*window)
    try:
        for name in ("nd64-lastrank", "stage1-nd16-allfull-mix", "stage1-nd5-somefull"):
            cfg = SMALL_CASES[name]
            say(f"  fused {name}")
            run, ref = run_pair(cfg)
            assert_state(run.fetch(), ref.state(), cfg.pdt, f"{name} window {window}")
        cfg = small_config(100_000, 200, BF16, F16, owner=7, steps=1, seed=17, align=8)
        say("  reduce n_d=200")
        run, ref = GpuRun(cfg), OracleRun(cfg)
        red = torch.empty(run.S, dtype=torch.float32, device=gpu)
        run.fill_grads(1)
        ref.fill_grads(1)
        run.reduce(red)
        _sync()
        want = O.reduce(ref.layers[0]["slices"], cfg.gdt, float(np.float32(cfg.grad_scale)))
        assert_f32(red.cpu().numpy(), want, "reduced", bitwise=True)
    finally:
        Z.zero_set_write_window(-1)


def test_warm_read_changes_nothing(gpu, zero_lib):
    """zero_set_warm_read(1) adds a read of the state (or of the reduction's
    output) before fused steps and reductions that read >= 1 GiB of gradients
    (here 64 ranks x 8.5M elements, 1.09 GB) and leaves every result bit
    unchanged: two steps and a reduction from the same state with the warm-up
    on and off give identical master, m, v, parameters and reduced gradient,
    right after gradients written with ordinary stores (the case it is for).  The
    path without it is checked against the oracle by the other tests."""
    import torch
    Z = zero_lib
    cfg = small_config(64 * 8_500_000, 64, BF16, F16, owner=5, steps=2, seed=41, align=64)
    say("[warm read] 64 ranks x 8.5M, on and off, 2 steps")
    run = GpuRun(cfg)
    L0 = run.layers[0]
    start = [L0[k].clone() for k in ("master", "m", "v")]
    red = torch.empty(run.S, dtype=torch.float32, device=gpu)
    out = {}
    try:
        for warm in (False, True):
            Z.zero_set_warm_read(warm)
            for k, x in zip(("master", "m", "v"), start):
                L0[k].copy_(x)
            run.full.zero_()
            for t in (1, 2):
                run.fill_grads(t)
                run.step(t)
            run.fill_grads(3)
            red.fill_(-1.0)
            run.reduce(red)
            _sync()
            out[warm] = [L0[k].clone() for k in ("master", "m", "v")] + [run.full.clone(), red.clone()]
    finally:
        Z.zero_set_warm_read(False)
    for name, a, b in zip(("master", "m", "v", "params", "reduced"), out[False], out[True]):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), name


def test_stream_write_window_changes_nothing(gpu, oracle_lib, zero_lib):
    """A window set for one stream only (zero_set_stream_write_window) applies
    to launches on that stream and leaves every result bit unchanged; the
    stream's setting removed, the process default applies again."""
    import torch
    Z = zero_lib
    cfg = SMALL_CASES["nd64-lastrank"]
    stream = torch.cuda.current_stream().cuda_stream
    say("[stream window] forced 3 us / 10 ns on the current stream, default off")
    Z.zero_set_write_window(0, 0)
    Z.zero_set_stream_write_window(stream, 300, 1)
    try:
        run, ref = run_pair(cfg)
        assert_state(run.fetch(), ref.state(), cfg.pdt, "stream window")
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            run2, ref2 = run_pair(replace(cfg, seed=cfg.seed + 1))
        torch.cuda.synchronize()
        assert_state(run2.fetch(), ref2.state(), cfg.pdt, "other stream")
    finally:
        Z.zero_set_stream_write_window(stream, -2)
        Z.zero_set_write_window(-1)


def test_misaligned_buffers_take_element_path(gpu, oracle_lib, zero_lib):
    """Every buffer one element past a 16-byte boundary: the library must fall
    back to the element kernel and still match the oracle bit for bit."""
    import torch
    from oracle.runner import OracleRun
    Z = zero_lib
    cfg = small_config(40_003, 5, F16, BF16, owner=4, steps=3, seed=29)
    ref = OracleRun(cfg)
    plan = Z.zero_plan(cfg.psi, cfg.n_d, list(cfg.sizes), cfg.bucket_cap, cfg.align)
    S, P = plan.shard_total, plan.psi_pad

    def view(n, dtype):
        return torch.zeros(n + 8, dtype=dtype, device=gpu)[1:n + 1]

    g = [view(S, torch.int16) for _ in range(cfg.n_d)]
    w, m, v = view(S, torch.float32), view(S, torch.float32), view(S, torch.float32)
    full = view(P, torch.int16)
    w.copy_(torch.from_numpy(ref.layers[0]["master"]).to(gpu))
    src = Z.GradSrc(cfg.gdt, g)
    say("[misaligned] psi=40003 n_d=5 owner=4, all bases at +1 element")
    for t in range(1, cfg.steps + 1):
        ref.fill_grads(t)
        for q in range(cfg.n_d):
            g[q].copy_(torch.from_numpy(ref.layers[0]["slices"][q].view(np.int16)).to(gpu))
        Z.zero_adam_step(plan, cfg.owner, cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.grad_scale, t, src, None,
                         w, m, v, full, cfg.pdt, True)
        ref.step(t)
    _sync()
    got = {"master": w.cpu().numpy(), "m": m.cpu().numpy(), "v": v.cpu().numpy(),
           "full": full.cpu().numpy().view(np.uint16)}
    assert_state(got, ref.state(), cfg.pdt, "misaligned")


def test_empty_plan_is_a_no_op(gpu, zero_lib):
    import torch
    Z = zero_lib
    p = Z.zero_plan(0, 4, [], 0, 64)
    x = torch.zeros(16, dtype=torch.float32, device=gpu)
    src = Z.GradSrc(Z.ZERO_BF16, [0, 0, 0, 0])
    Z.zero_adam_step(p, 1, 1e-4, 0.9, 0.999, 1e-8, 0.25, 1, src, None, 0, 0, 0, 0, Z.ZERO_F16, True)
    Z.zero_shard_reduce(p, 1, src, 0.25, 0)
    Z.zero_gather_pack(p, [0, 0, 0, 0], Z.ZERO_F16, 0)
    Z.zero_flatten(p, [], Z.ZERO_F16, 0)
    _sync()
    assert not torch.any(x)


def test_owner_outside_range_untouched(gpu, oracle_lib):
    """The step writes the full parameter buffer only at the owner's ranges."""
    cfg = SMALL_CASES["multibucket-nd4"]
    run, ref = run_pair(cfg)
    full = run.fetch()["full"]
    mask = np.ones(full.size, bool)
    for b in range(len(ref.plan.buckets)):
        lo, hi = ref.plan.owner_range(b, cfg.owner)
        mask[lo:hi] = False
    assert not np.any(full[mask])


# ---------------------------------------------------------------------------
# Stage 3: per-layer gather_pack then the step into the resident shard
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("h,n_d,owner", [(256, 64, 0), (96, 8, 5)])
def test_stage3_layer_loop(gpu, oracle_lib, h, n_d, owner):
    from oracle.runner import OracleRun
    from synth.workloads import layer_sizes
    cfg = Config(f"stage3-h{h}", tuple(layer_sizes(h)), n_d=n_d, gdt=BF16, pdt=F16, stage=3,
                 owner=owner, steps=2, layers=3, seed=17)
    say(f"[stage3] h={h} n_d={n_d} owner={owner} layers=3 steps=2")
    run, ref = GpuRun(cfg), OracleRun(cfg)
    for t in range(1, cfg.steps + 1):
        for layer in range(cfg.layers):
            run.fill_grads(t, layer)
            ref.fill_grads(t, layer)
            run.step(t, layer)
            ref.step(t, layer)
            _sync()
            got, want = run.fetch(layer), ref.state(layer)
            assert np.array_equal(got["full"], want["gathered"]), ("gather", t, layer)
            assert_state({k: got[k] for k in ("master", "m", "v")}, want, cfg.pdt, f"L{layer}")
            for q in range(n_d):
                assert np.array_equal(got["shards"][q], want["shards"][q]), ("shard", q)


def test_stage3_pipelined_loop_matches_serial(gpu, oracle_lib):
    """The two-stream Stage-3 loop (gather of layer l+1 overlapping the step
    of layer l, double-buffered) leaves exactly the state of the serial loop,
    and its last two gathered buffers hold the oracle's materialised layers."""
    from oracle.runner import OracleRun
    from synth.workloads import layer_sizes
    cfg = Config("stage3-pipe", tuple(layer_sizes(128)), n_d=16, gdt=BF16, pdt=F16, stage=3,
                 owner=5, steps=2, layers=5, seed=23)
    say("[stage3] pipelined vs serial, h=128 n_d=16 layers=5 steps=2")
    serial, pipe, ref = GpuRun(cfg), GpuRun(cfg), OracleRun(cfg)
    for t in range(1, cfg.steps + 1):
        for layer in range(cfg.layers):
            serial.fill_grads(t, layer)
            pipe.fill_grads(t, layer)
            ref.fill_grads(t, layer)
        serial.layer_loop(t, pipelined=False)
        pipe.layer_loop(t, pipelined=True)
        for layer in range(cfg.layers):
            ref.step(t, layer)
        _sync()
        for layer in range(cfg.layers):
            a, b = serial.fetch(layer), pipe.fetch(layer)
            for k in ("master", "m", "v"):
                assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), (t, layer, k)
            assert np.array_equal(a["shards"], b["shards"]), (t, layer)
            assert_state({k: b[k] for k in ("master", "m", "v")}, ref.state(layer), cfg.pdt, f"L{layer}")
        last, prev = cfg.layers - 1, cfg.layers - 2
        bufs = [pipe.full.cpu().numpy().view(np.uint16), pipe.full2.cpu().numpy().view(np.uint16)]
        assert np.array_equal(bufs[last % 2], ref.state(last)["gathered"])
        assert np.array_equal(bufs[prev % 2], ref.state(prev)["gathered"])


def test_stage3_compute_sees_its_layer(gpu, oracle_lib):
    """With a layer compute between gather and step, every layer's compute
    reads exactly that layer's gathered weights (the pre-step shards), in the
    serial loop and in the prefetching two-stream loop, where the gather of
    layer l+1 runs during layer l's compute and step."""
    import torch
    from oracle.runner import OracleRun
    from synth.workloads import layer_sizes
    cfg = Config("stage3-compute", tuple(layer_sizes(128)), n_d=8, gdt=BF16, pdt=F16, stage=3,
                 owner=2, steps=2, layers=5, seed=29)
    say("[stage3] compute between gather and step, h=128 n_d=8 layers=5 steps=2")
    serial, pipe, ref = GpuRun(cfg), GpuRun(cfg), OracleRun(cfg)
    seen = {name: [torch.empty_like(serial.full) for _ in range(cfg.layers)] for name in ("serial", "pipe")}

    def recorder(name):
        def compute(layer, buf):
            seen[name][layer].copy_(buf)       # what this layer's compute read
        return compute

    for t in range(1, cfg.steps + 1):
        for layer in range(cfg.layers):
            serial.fill_grads(t, layer)
            pipe.fill_grads(t, layer)
            ref.fill_grads(t, layer)
        serial.layer_loop(t, pipelined=False, compute=recorder("serial"))
        pipe.layer_loop(t, pipelined=True, compute=recorder("pipe"))
        for layer in range(cfg.layers):
            ref.step(t, layer)
        _sync()
        for layer in range(cfg.layers):
            want = ref.state(layer)["gathered"]
            for name in ("serial", "pipe"):
                got = seen[name][layer].cpu().numpy().view(np.uint16)
                assert np.array_equal(got, want), (t, layer, name)
            a, b = serial.fetch(layer), pipe.fetch(layer)
            assert np.array_equal(a["shards"], b["shards"]), (t, layer)


@pytest.mark.parametrize("k", [16, 64])
def test_stage3_cu_split_loop_matches_serial(gpu, oracle_lib, k):
    """The prefetching loop with the compute units split between streams --
    layer compute and step on n - k CUs, the next layer's gather on the other
    k (the same share of every die) -- leaves exactly the serial loop's state,
    and every layer's compute reads that layer's gathered (pre-step)
    weights."""
    import torch
    from oracle.runner import OracleRun
    from synth import gpu as SG
    from synth.workloads import layer_sizes
    cfg = Config("stage3-cusplit", tuple(layer_sizes(128)), n_d=8, gdt=BF16, pdt=F16, stage=3,
                 owner=6, steps=2, layers=5, seed=31)
    n = SG.cu_count()
    say(f"[stage3] CU split k={k} of {n}, h=128 n_d=8 layers=5 steps=2")
    if n % 64:
        pytest.skip(f"{n} CUs do not split evenly over 8 dies")
    g_cus = SG.balanced_cus(k, n)
    serial, split, ref = GpuRun(cfg), GpuRun(cfg), OracleRun(cfg)
    ms_c = SG.MaskedStream(torch, sorted(set(range(n)) - set(g_cus)))
    ms_g = SG.MaskedStream(torch, g_cus)
    seen = {name: [torch.empty_like(serial.full) for _ in range(cfg.layers)] for name in ("serial", "split")}

    def recorder(name):
        def compute(layer, buf):
            seen[name][layer].copy_(buf)
        return compute

    try:
        for t in range(1, cfg.steps + 1):
            for layer in range(cfg.layers):
                serial.fill_grads(t, layer)
                split.fill_grads(t, layer)
                ref.fill_grads(t, layer)
            serial.layer_loop(t, pipelined=False, compute=recorder("serial"))
            cur = torch.cuda.current_stream()
            ms_c.torch.wait_stream(cur)
            with torch.cuda.stream(ms_c.torch):
                split.layer_loop(t, pipelined=True, compute=recorder("split"), side=ms_g.torch)
            cur.wait_stream(ms_c.torch)
            for layer in range(cfg.layers):
                ref.step(t, layer)
            _sync()
            for layer in range(cfg.layers):
                want = ref.state(layer)["gathered"]
                for name in ("serial", "split"):
                    got = seen[name][layer].cpu().numpy().view(np.uint16)
                    assert np.array_equal(got, want), (t, layer, name)
                a, b = serial.fetch(layer), split.fetch(layer)
                for key in ("master", "m", "v"):
                    assert np.array_equal(a[key].view(np.uint32), b[key].view(np.uint32)), (t, layer, key)
                assert np.array_equal(a["shards"], b["shards"]), (t, layer)
                assert_state({key: b[key] for key in ("master", "m", "v")}, ref.state(layer), cfg.pdt, f"L{layer}")
    finally:
        ms_c.close()
        ms_g.close()


# ---------------------------------------------------------------------------
# Special values and the output conversion
# ---------------------------------------------------------------------------

def _to_gpu(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def test_nan_inf_denormal_propagation(gpu, oracle_lib):
    import torch
    import oracle as O
    import zero_sharded_mixed_02_amd as Z
    n_d, S = 2, 4096
    p = Z.zero_plan(n_d * S, n_d, [n_d * S], 0, 8)
    assert p.shard_total == S
    specials16 = np.array([0x7C00, 0xFC00, 0x7E00, 0x0001, 0x8001, 0x03FF, 0x7BFF, 0xFBFF, 0, 0x8000],
                          np.uint16)
    rng = np.random.default_rng(3)
    g0 = rng.choice(specials16, S).astype(np.uint16)
    g1 = O.f32_to_16(rng.normal(0, 1e-3, S).astype(np.float32), O.F16)
    g1[::7] = rng.choice(specials16, g1[::7].size)
    w = rng.normal(0, 0.02, S).astype(np.float32)
    w[::11] = np.array([np.inf, -np.inf, np.nan, 1e-40, -1e-45, 0.0, -0.0, 3e38], np.float32)[
        np.arange(w[::11].size) % 8]
    m = np.zeros(S, np.float32)
    v = np.zeros(S, np.float32)
    m[::13] = 1e-30
    v[::13] = 1e-38
    dev = gpu
    tg = [_to_gpu(g0, dev), _to_gpu(g1, dev)]
    tw, tm, tv = _to_gpu(w, dev), _to_gpu(m, dev), _to_gpu(v, dev)
    full = torch.zeros(p.psi_pad, dtype=torch.int16, device=dev)
    owner = 1
    for t in (1, 2):
        Z.zero_adam_step(p, owner, 1e-4, 0.9, 0.999, 1e-8, 0.5, t, Z.GradSrc(Z.ZERO_F16, tg), None,
                         tw, tm, tv, full, Z.ZERO_BF16, True)
        O.shard_step([g0, g1], O.F16, O.Hyper(1e-4, 0.9, 0.999, 1e-8, 0.5), t, w, m, v, O.BF16)
    _sync()
    assert_f32(tw.cpu().numpy(), w, "master", bitwise=True)
    assert_f32(tm.cpu().numpy(), m, "m", bitwise=True)
    assert_f32(tv.cpu().numpy(), v, "v", bitwise=True)
    got = full.cpu().numpy().view(np.uint16)[owner * S:(owner + 1) * S]
    assert_p16(got, O.f32_to_16(w, O.BF16), O.BF16, "params", bitwise=True)


def _structured_f32_patterns():
    """fp32 bit patterns around every rounding boundary of both 16-bit
    formats: all sign/exponent/upper-mantissa combinations with the dropped
    bits at 0, 1, just below, at and just above the halfway point."""
    out = []
    hi16 = np.arange(1 << 16, dtype=np.uint32) << 16
    for low in (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF):
        out.append(hi16 | low)
    top = np.arange(1 << 19, dtype=np.uint32) << 13       # sign, exponent, 10 mantissa bits
    for low in (0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF):
        out.append(top | low)
    rng = np.random.default_rng(4)
    out.append(rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32))
    return np.concatenate(out)


@pytest.mark.parametrize("pdt", [F16, BF16])
def test_output_conversion_sweep(gpu, oracle_lib, pdt):
    """With lr = 0 and zero gradients the step leaves w unchanged, so the
    stored parameter is the conversion of the master weight: swept over ~7.5M
    fp32 patterns covering every exponent and rounding boundary."""
    import torch
    import oracle as O
    import zero_sharded_mixed_02_amd as Z
    bits = _structured_f32_patterns()
    S = bits.size - bits.size % 64
    bits = bits[:S]
    p = Z.zero_plan(S, 1, [S], 0, 64)
    dev = gpu
    w = _to_gpu(bits.view(np.float32), dev)
    m = torch.zeros(S, dtype=torch.float32, device=dev)
    v = torch.zeros(S, dtype=torch.float32, device=dev)
    g = torch.zeros(S, dtype=torch.int16, device=dev)
    out = torch.zeros(S, dtype=torch.int16, device=dev)
    Z.zero_adam_step(p, 0, 0.0, 0.9, 0.999, 1e-8, 1.0, 1, Z.GradSrc(Z.ZERO_BF16, [g]), None, w, m, v,
                     out, pdt, True)
    _sync()
    wn = w.cpu().numpy()
    assert np.array_equal(wn.view(np.uint32)[~np.isnan(wn)], bits[~np.isnan(wn)])
    assert_p16(out.cpu().numpy(), O.f32_to_16(bits.view(np.float32), pdt), pdt, "cast", bitwise=True)
