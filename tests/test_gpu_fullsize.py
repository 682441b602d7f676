"""Parity at the full workload sizes, in the launch configuration the
benchmark times: the GPU runs the whole shard; the oracle computes a sample of
its elements one by one (first and last 4096, every segment boundary, and
random positions), which is exact because every operation of the step is
elementwise in the shard index.  For the benchmark's own workload the oracle
also covers the whole shard (test_fused_7p5B_whole_shard)."""
import numpy as np
import pytest

from synth.workloads import WORKLOADS, GpuRun
from tests.parity import assert_p16, assert_state

pytestmark = [pytest.mark.gpu, pytest.mark.big]


def say(msg):
    print(msg, flush=True)


def sample_indices(S: int, seed: int, n_random: int = 65536) -> np.ndarray:
    rng = np.random.default_rng(seed)
    edges = [np.arange(min(4096, S)), np.arange(max(0, S - 4096), S)]
    seg = 1 << 28
    for b in range(seg, S, seg):            # pieces the host splits large shards into
        edges.append(np.arange(b - 64, min(S, b + 64)))
    edges.append(rng.integers(0, S, size=n_random))
    return np.unique(np.concatenate(edges))


def _free(run):
    import torch
    del run
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _full_size_config(name):
    from dataclasses import replace
    from synth.workloads import with_owner
    if name == "7.5B-stage2-align1-owner17":
        # The plain Psi/N_d layout: S = 117,187,500, offsets multiples of 4.
        return with_owner(replace(WORKLOADS["7.5B-stage2"], align=1, steps=2), 17)
    return WORKLOADS[name]


@pytest.mark.parametrize("name", ["7.5B-stage2", "13B-stage1", "7.5B-stage2-align1-owner17"])
def test_stage12_full_size(gpu, oracle_lib, name):
    import torch
    from oracle.runner import OracleRun
    cfg = _full_size_config(name)
    say(f"[full size] {cfg.name}: psi={cfg.psi} n_d={cfg.n_d} steps={cfg.steps}")
    run = GpuRun(cfg)
    say(f"  resident {run.bytes_resident() / 1e9:.1f} GB, S={run.S}")
    J = sample_indices(run.S, seed=cfg.seed)
    ref = OracleRun(cfg, sample=J)
    for t in range(1, cfg.steps + 1):
        run.fill_grads(t)
        ref.fill_grads(t)
        run.step(t)
        ref.step(t)
        torch.cuda.synchronize()
        say(f"  step {t} done")
    got = run.fetch_at(J, ref.pos)
    r = assert_state(got, ref.state(), cfg.pdt, cfg.name)
    say(f"  sample of {J.size}: {r}")
    _free(run)


def _oracle_whole_shard(cfg, S: int, steps: int, n_chunks: int = 64):
    """The oracle over the owner's whole shard: contiguous chunks of shard
    indices, each an OracleRun on that sample, on a thread pool.  Every
    operation of the step is elementwise in the shard index and the oracle's
    C calls release the GIL, so the concatenated chunks are the whole-shard
    result.  Returns (state dict over the whole shard, flat positions)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    from oracle.runner import OracleRun

    def one(J):
        ref = OracleRun(cfg, sample=J)
        for t in range(1, steps + 1):
            ref.fill_grads(t)
            ref.step(t)
            ref.layers[0]["slices"] = None
        st = ref.state()
        return {k: st[k] for k in ("master", "m", "v", "params")}, ref.pos

    chunks = np.array_split(np.arange(S, dtype=np.int64), n_chunks)
    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        parts = list(ex.map(one, chunks))
    state = {k: np.concatenate([p[0][k] for p in parts]) for k in ("master", "m", "v", "params")}
    return state, np.concatenate([p[1] for p in parts])


def test_fused_7p5B_whole_shard(gpu, oracle_lib):
    """The benchmark's workload (7.5B, N_d = 64, owner 0), two steps, compared
    over the WHOLE shard: every one of its 117,187,520 master, m, v and 16-bit
    parameter values equals the oracle's bit for bit, and the 7.5e9-element
    parameter buffer holds nothing but zeros outside the owner's range."""
    import torch
    from dataclasses import replace
    cfg = replace(WORKLOADS["7.5B-stage2"], steps=2)
    say(f"[whole shard] {cfg.name}: psi={cfg.psi} n_d={cfg.n_d} steps={cfg.steps}")
    run = GpuRun(cfg)
    S = run.S
    for t in range(1, cfg.steps + 1):
        run.fill_grads(t)
        run.step(t)
    torch.cuda.synchronize()
    say(f"  GPU done, S={S}; oracle over the whole shard ...")
    want, pos = _oracle_whole_shard(cfg, S, cfg.steps)
    lo, hi = int(pos.min()), int(pos.max()) + 1
    assert hi - lo == S, "owner 0 of a one-bucket plan owns one contiguous range"
    outside = int(torch.count_nonzero(run.full[:lo]).item()) + int(torch.count_nonzero(run.full[hi:]).item())
    assert outside == 0, f"{outside} parameter elements written outside the owner's range"
    got = run.fetch_at(np.arange(S, dtype=np.int64), pos)
    r = assert_state(got, want, cfg.pdt, cfg.name)
    say(f"  whole shard of {S}: {r}")
    _free(run)


def test_unfused_full_size(gpu, oracle_lib):
    """The 7.5B, N_d = 64 workload through zero_shard_reduce (its automatic
    write window included) and zero_adam_step from the reduced gradient: the
    sampled reduced gradient and state equal the oracle's."""
    import torch
    import oracle as O
    from oracle.runner import OracleRun
    from tests.parity import assert_f32
    cfg = WORKLOADS["7.5B-stage2"]
    say(f"[full size, unfused] {cfg.name}: psi={cfg.psi} n_d={cfg.n_d}, 2 steps")
    run = GpuRun(cfg)
    J = sample_indices(run.S, seed=33)
    ref = OracleRun(cfg, sample=J)
    red = torch.empty(run.S, dtype=torch.float32, device=gpu)
    j_t = torch.from_numpy(J).to(gpu)
    for t in (1, 2):
        run.fill_grads(t)
        ref.fill_grads(t)
        run.reduce(red)
        run.step_from_reduced(t, red)
        ref.step(t)
        torch.cuda.synchronize()
        want = O.reduce(ref.layers[0]["slices"], cfg.gdt, float(np.float32(cfg.grad_scale)))
        assert_f32(red[j_t].cpu().numpy(), want, "reduced", bitwise=True)
        say(f"  step {t} done")
    r = assert_state(run.fetch_at(J, ref.pos), ref.state(), cfg.pdt, cfg.name)
    say(f"  sample of {J.size}: {r}")
    del red
    _free(run)


def test_stage3_full_size(gpu, oracle_lib):
    import torch
    import synth
    from oracle.runner import OracleRun
    cfg = WORKLOADS["stage3-h8192x8"]
    say(f"[full size] {cfg.name}: {cfg.layers} layers of {cfg.psi} params, n_d={cfg.n_d}")
    run = GpuRun(cfg)
    say(f"  resident {run.bytes_resident() / 1e9:.1f} GB, S={run.S}")
    J = sample_indices(run.S, seed=cfg.seed)
    ref = OracleRun(cfg, sample=J)
    rng = np.random.default_rng(55)
    flat_sample = np.unique(np.concatenate([np.arange(4096), np.arange(run.P - 4096, run.P),
                                            rng.integers(0, run.P, 65536)]))
    # Expected gathered values: the rank owning each position holds the 16-bit
    # rounding of its master weight (how the resident shards were initialised).
    pad = np.zeros(flat_sample.size, bool)
    for bk in ref.plan.buckets:
        pad |= (flat_sample >= bk.flat_off + bk.numel) & (flat_sample < bk.flat_off + bk.padded)
    pos_t = torch.from_numpy(flat_sample).to(gpu)
    for t in range(1, cfg.steps + 1):
        for layer in range(cfg.layers):
            run.fill_grads(t, layer)
            ref.fill_grads(t, layer)
            run.step(t, layer)
            ref.step(t, layer)
            torch.cuda.synchronize()
            gathered = run.full[pos_t].cpu().numpy().view(np.uint16)
            want = synth.to_dtype_bits(
                synth.master_values(cfg.seed, flat_sample + layer * run.P, cfg.sigma_w, pad), cfg.pdt)
            assert np.array_equal(gathered, want), ("gather", layer)
            got = run.fetch_at(J, None, layer)
            r = assert_state(got, ref.state(layer), cfg.pdt, f"layer {layer}")
            say(f"  layer {layer}: gather ok, step {r['params']}")
    _free(run)
