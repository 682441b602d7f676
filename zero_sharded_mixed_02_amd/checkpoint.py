"""Rank-local checkpoints of the sharded optimizer state, restorable at a
different data-parallel degree.

The whole resumable state of one rank's shard step is the step counter t and
the fp32 master weights, first and second moments of its shard (the
mixed-precision Adam state of the ZeRO concept page, "why it is needed"); the
16-bit parameters are the rounding of the master weights and need not be
stored.  A checkpoint file holds those arrays plus the plan parameters, so a
job with another N_d (or bucketing) can rebuild its own shards with
``zero_reshard`` (concept page, design trade-off 4 and the checklist item on
restoring rank-local shards after the parallel degree changes).

Files are numpy ``.npz`` archives written and read with ``allow_pickle=False``.
"""
from __future__ import annotations

import json
from typing import Dict, Sequence

import numpy as np

from . import ZERO_F32, Plan, zero_plan, zero_reshard

FORMAT = "zero-shard-state-v1"


def _plan_meta(plan_args: Dict) -> Dict:
    return {k: (list(map(int, plan_args[k])) if k == "tensor_numel" else int(plan_args[k]))
            for k in ("psi", "n_d", "tensor_numel", "bucket_cap", "shard_align")}


def _check_state(name: str, a: np.ndarray, shard_total: int, where: str) -> None:
    if a.dtype != np.float32:
        raise ValueError(f"{where}: {name} is {a.dtype}, expected float32")
    if a.ndim != 1:
        raise ValueError(f"{where}: {name} has shape {a.shape}, expected one dimension")
    if a.size != shard_total:
        raise ValueError(f"{where}: {name} holds {a.size} elements, the plan's shard has {shard_total}")


def save_shard(path: str, plan_args: Dict, rank: int, t: int, master, m, v) -> None:
    """Write rank's state.  plan_args: dict(psi, n_d, tensor_numel, bucket_cap,
    shard_align) -- the arguments the shard's plan was built from.  master, m,
    v: one-dimensional fp32 tensors or arrays (any device) of exactly the
    plan's shard_total elements; anything else raises ValueError and writes
    nothing."""
    meta = {"format": FORMAT, "rank": int(rank), "t": int(t), "plan": _plan_meta(plan_args)}
    S = plan_from(meta["plan"]).shard_total
    if not 0 <= meta["rank"] < meta["plan"]["n_d"]:
        raise ValueError(f"rank {rank} outside [0, {meta['plan']['n_d']})")
    if meta["t"] < 0:
        raise ValueError(f"step {t} is negative")
    arrays = {}
    for name, x in (("master", master), ("m", m), ("v", v)):
        a = x.detach().cpu().numpy() if hasattr(x, "detach") else np.asarray(x)
        _check_state(name, a, S, path)
        arrays[name] = np.ascontiguousarray(a)
    np.savez(path, meta=np.frombuffer(json.dumps(meta).encode(), dtype=np.uint8), **arrays)


def load_shard(path: str) -> Dict:
    """Read one rank's file.  Its arrays must be one-dimensional float32 of
    the shard size its own plan gives; anything else raises ValueError."""
    with np.load(path, allow_pickle=False) as z:
        meta = json.loads(bytes(z["meta"]).decode())
        if meta.get("format") != FORMAT:
            raise ValueError(f"{path}: not a {FORMAT} file")
        meta["plan"] = _plan_meta(meta["plan"])
        S = plan_from(meta["plan"]).shard_total
        for k in ("master", "m", "v"):
            a = z[k]
            _check_state(k, a, S, path)
            meta[k] = a.copy()
    return meta


def plan_from(plan_args: Dict) -> Plan:
    return zero_plan(plan_args["psi"], plan_args["n_d"], plan_args["tensor_numel"],
                     plan_args["bucket_cap"], plan_args["shard_align"])


def restore(paths: Sequence[str], new_plan: Plan, new_rank: int, device="cuda"):
    """Rebuild (t, master, m, v) of new_rank under new_plan from the
    checkpoint files of every rank of the old plan (one file per old rank, any
    order).  Returns torch tensors on device."""
    import torch
    shards = [load_shard(p) for p in paths]
    old_args = shards[0]["plan"]
    if any(s["plan"] != old_args or s["t"] != shards[0]["t"] for s in shards):
        raise ValueError("checkpoint files come from different plans or steps")
    by_rank = {s["rank"]: s for s in shards}
    if sorted(by_rank) != list(range(old_args["n_d"])):
        raise ValueError(f"need one file per old rank 0..{old_args['n_d'] - 1}")
    old_plan = plan_from(old_args)
    for s in shards:   # already checked by load_shard; kept next to the GPU copies it guards
        for name in ("master", "m", "v"):
            _check_state(name, s[name], old_plan.shard_total, f"rank {s['rank']}")
    out = []
    for name in ("master", "m", "v"):
        src = [torch.from_numpy(by_rank[r][name]).to(device) for r in range(old_args["n_d"])]
        dst = torch.empty(new_plan.shard_total, dtype=torch.float32, device=device)
        zero_reshard(old_plan, new_plan, new_rank, src, ZERO_F32, dst)
        out.append(dst)
    torch.cuda.synchronize(device)
    return (shards[0]["t"], *out)
