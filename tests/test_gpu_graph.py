"""The step captured in a HIP graph: the library's launches take every table
in their kernel arguments and neither allocate nor synchronise, so a caller
can capture zero_adam_step (and the Stage-3 gather) once and replay it.

Kernel arguments are fixed at capture, the step number t included, so each
replay is the step at that t again.  The eager twin does the same calls the
same number of times; after every replay (with eager work and a device
synchronisation in between) the two states must agree bit for bit."""
from dataclasses import replace

import numpy as np
import pytest

from synth import BF16, F16
from synth.workloads import WORKLOADS, GpuRun, small_config

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def _same(a, b, what):
    for k in ("master", "m", "v"):
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), (what, k)
    assert np.array_equal(a["full"], b["full"]), (what, "full")
    if "shards" in a:
        assert np.array_equal(a["shards"], b["shards"]), (what, "shards")


@pytest.mark.parametrize("case,window", [
    ("nd64", None),            # automatic window (none at this size)
    ("nd64", (50, 10)),        # a forced window: the wait runs inside the graph
    ("stage3", None),          # gather_pack + step into the resident shard
])
def test_graph_replays_match_eager(gpu, zero_lib, case, window):
    import torch
    Z = zero_lib
    if case == "nd64":
        cfg = small_config(300_000, 64, BF16, F16, owner=5, steps=1, seed=41)
    else:
        cfg = replace(WORKLOADS["stage3-h8192x8"], sizes=(96, 96, 8192), n_d=8, owner=3, layers=2, seed=42)
    say(f"[graph] {case} window={window}")
    if window:
        Z.zero_set_write_window(*window)
    try:
        eager, graphed = GpuRun(cfg), GpuRun(cfg)
        for r in (eager, graphed):
            for layer in range(cfg.layers):
                r.fill_grads(1, layer)
        t = 3
        # Warm up on a side stream before capture (as torch requires), then capture.
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            graphed.step(t)
            eager.step(t)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            graphed.step(t)
        for rep in range(4):
            g.replay()
            eager.step(t)
            torch.cuda.synchronize()
            _same(graphed.fetch(), eager.fetch(), f"replay {rep}")
            # Eager work between replays: a throw-away reduction on the graphed run.
            tmp = torch.empty(graphed.S, dtype=torch.float32, device=gpu)
            graphed.reduce(tmp)
            torch.cuda.synchronize()
    finally:
        Z.zero_set_write_window(-1)
