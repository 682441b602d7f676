"""Randomised GPU parity: many small workloads drawn from a seeded generator
-- tensor lists with empty and odd-sized tensors, bucket caps, alignments
(vector and element kernels), rank counts from 1 to 130 (the fused kernel's
compiled and runtime rank counts, and the reduce-then-Adam path beyond 128),
every gradient/parameter dtype pair, Stage 1 full-buffer ranks, Stage 3 layer
loops, owners anywhere, write windows automatic, off or forced -- each run for
one or two steps and compared with the oracle over the whole shard, bit for
bit."""
import numpy as np
import pytest

from synth import BF16, F16
from synth.workloads import Config, GpuRun
from tests.parity import assert_state

pytestmark = pytest.mark.gpu

N_CASES = 120


def draw(seed: int):
    """(workload, write-window setting) of one seeded case."""
    rng = np.random.default_rng(1000 + seed)
    n_t = int(rng.integers(1, 12))
    sizes = tuple(int(x) for x in rng.choice([0, 1, 7, 64, 513, 4096, 20_000, 65_537], size=n_t))
    if sum(sizes) == 0:
        sizes = sizes + (1000,)
    n_d = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 64, 130]))
    stage = int(rng.choice([1, 2, 2, 3]))
    full = ()
    if stage == 1:
        full = tuple(sorted(int(q) for q in rng.choice(n_d, size=min(n_d, int(rng.integers(1, 4))),
                                                        replace=False)))
    cfg = Config(f"random-{seed}", sizes, n_d=n_d,
                 gdt=int(rng.choice([F16, BF16])), pdt=int(rng.choice([F16, BF16])),
                 stage=stage, owner=int(rng.integers(0, n_d)),
                 bucket_cap=int(rng.choice([0, 0, 5000, 30_000])), align=int(rng.choice([1, 8, 64])),
                 steps=int(rng.integers(1, 3)), layers=2 if stage == 3 else 1, seed=2000 + seed,
                 mix=bool(rng.integers(0, 2)), full_ranks=full)
    window = [(-1, 0), (0, 0), (40, 10), (300, 1)][int(rng.integers(0, 4))]
    return cfg, window


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_workload_matches_oracle(gpu, oracle_lib, zero_lib, seed):
    cfg, window = draw(seed)
    print(f"[random {seed}] sizes={cfg.sizes} n_d={cfg.n_d} stage={cfg.stage} owner={cfg.owner} "
          f"cap={cfg.bucket_cap} align={cfg.align} g/p={cfg.gdt}/{cfg.pdt} full={cfg.full_ranks} "
          f"steps={cfg.steps} window={window}", flush=True)
    Z = zero_lib
    Z.zero_set_write_window(*window)
    try:
        _run_case(gpu, cfg, seed)
    finally:
        Z.zero_set_write_window(-1)


def _run_case(gpu, cfg, seed):
    import torch
    from oracle.runner import OracleRun
    run, ref = GpuRun(cfg), OracleRun(cfg)
    red = torch.empty(max(1, run.S), dtype=torch.float32, device=gpu)
    for t in range(1, cfg.steps + 1):
        for layer in range(cfg.layers):
            run.fill_grads(t, layer)
            ref.fill_grads(t, layer)
            if cfg.n_d > 128:
                # Beyond one launch's rank table: reduce in rank groups, then Adam.
                if cfg.stage == 3:
                    run.Z.zero_gather_pack(run.plan, list(run.layers[layer]["shards"]), cfg.pdt, run.full)
                run.reduce(red, layer)
                run.step_from_reduced(t, red, layer)
            else:
                run.step(t, layer)
            ref.step(t, layer)
    torch.cuda.synchronize()
    for layer in range(cfg.layers):
        got, want = run.fetch(layer), ref.state(layer)
        assert_state(got, want, cfg.pdt, f"random {seed} layer {layer}", bitwise=True)
