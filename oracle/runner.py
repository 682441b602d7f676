"""Drives the CPU oracle over one workload (TEST INFRASTRUCTURE ONLY).

Inputs come from the seeded generator in ``synth`` (numpy half), laid out by
the oracle's own plan; nothing here reads anything the GPU produced.  Either
the whole owner's shard is computed (small workloads), or only a sample of its
elements: every operation of the step is elementwise in the shard index, so
the oracle run on the gathered sample gives exactly those elements of the full
result.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

import synth
from . import Hyper, gather_pack, place_shard, plan, shard_step


class OracleRun:
    def __init__(self, cfg, sample: Optional[np.ndarray] = None):
        self.cfg = cfg
        self.plan = plan(cfg.psi, cfg.n_d, list(cfg.sizes), cfg.bucket_cap, cfg.align)
        self.S, self.P = self.plan.shard_total, self.plan.psi_pad
        self.sample = None if sample is None else np.asarray(sample, dtype=np.int64)
        self.hp = Hyper(cfg.lr, cfg.beta1, cfg.beta2, cfg.eps, cfg.grad_scale)
        self.pos, self.pad = self.rank_positions(cfg.owner, self.sample)
        self.layers = []
        for layer in range(cfg.layers):
            L = {"master": synth.master_values(cfg.seed, self.pos + layer * self.P, cfg.sigma_w, self.pad),
                 "m": np.zeros(self.pos.size, np.float32),
                 "v": np.zeros(self.pos.size, np.float32),
                 "slices": None, "params": None}
            if cfg.stage == 3 and self.sample is None:
                L["shards"] = [self.initial_param_shard(q, layer) for q in range(cfg.n_d)]
            self.layers.append(L)

    def rank_positions(self, rank: int, sample=None):
        """Flat positions of rank's shard (shard-local order), and pad flags,
        from the oracle plan's owned ranges."""
        j = np.arange(self.plan.shard_total, dtype=np.int64) if sample is None else sample
        if not self.plan.buckets:
            return j.copy(), np.zeros(j.size, bool)
        starts = np.array([bk.shard_off for bk in self.plan.buckets], dtype=np.int64)
        b = np.searchsorted(starts, j, side="right") - 1          # bucket of each shard index
        lo = np.array([self.plan.owner_range(i, rank)[0] for i in range(len(starts))], np.int64)
        real_end = np.array([bk.flat_off + bk.numel for bk in self.plan.buckets], np.int64)
        pos = lo[b] + (j - starts[b])
        return pos, pos >= real_end[b]

    def initial_param_shard(self, q: int, layer: int) -> np.ndarray:
        pos, pad = self.rank_positions(q)
        w = synth.master_values(self.cfg.seed, pos + layer * self.P, self.cfg.sigma_w, pad)
        return synth.to_dtype_bits(w, self.cfg.pdt)

    def fill_grads(self, t: int, layer: int = 0):
        cfg = self.cfg
        self.layers[layer]["slices"] = [
            synth.grad_values(cfg.seed, q, t, self.pos + layer * self.P, cfg.sigma_g, cfg.gdt,
                              cfg.mix, self.pad)
            for q in range(cfg.n_d)]

    def step(self, t: int, layer: int = 0):
        L = self.layers[layer]
        if self.cfg.stage == 3 and self.sample is None:
            L["gathered"] = gather_pack(self.plan, L["shards"])
        L["params"] = shard_step(L["slices"], self.cfg.gdt, self.hp, t, L["master"], L["m"], L["v"],
                                 self.cfg.pdt)
        if self.cfg.stage == 3 and self.sample is None:
            L["shards"][self.cfg.owner] = L["params"]

    def state(self, layer: int = 0) -> dict:
        """master, m, v and params of the owner's shard (or of the sample)."""
        L = self.layers[layer]
        out = {"master": L["master"], "m": L["m"], "v": L["v"], "params": L["params"]}
        if self.sample is None and self.cfg.stage != 3:
            full = np.zeros(self.P, np.uint16)
            if L["params"] is not None:
                place_shard(self.plan, self.cfg.owner, L["params"], full)
            out["full"] = full
        if self.sample is None and self.cfg.stage == 3:
            out["shards"] = L["shards"]
            out["gathered"] = L.get("gathered")
        return out
