"""CPU oracle for one data-parallel rank's share of a ZeRO training step.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the GPU library (``zero_sharded_mixed_02_amd``) and neither imports the other.

Sources, cited by page and section (the pages are three web pages about ZeRO,
arXiv 1910.02054):

* ZeRO mind-map page (paperbridge.wiki):
  - "shrink the problem: four GPUs": state split into blocks A, B, C, D; GPU i
    keeps block i for the long term (ownership convention used by ``plan``);
  - "how does a GPU that stores a quarter compute": parameters of the current
    layer are exchanged so every GPU briefly holds them in full; gradients are
    split again and sent back to the GPU responsible for each part, which
    updates and keeps it;
  - "Stage 1/2/3": which of optimizer history, gradients and parameters are
    sharded; the 7.5B / 64-way memory figures 120 / 31.4 / 16.6 / 1.9 GB;
    parameter sharding communicates about 1.5x standard data parallelism;
  - "paper evidence": standard DP and gradient sharding move 2 Psi, parameter
    sharding 3 Psi (paper section 5);
  - glossary: all-gather and reduce-scatter.
* ZeRO concept page (papers.lqhl.me):
  - "why it is needed": the mixed-precision Adam state (16-bit parameters,
    fp32 master weights, first and second moments);
  - "three stages" table: resident sharded state and replicated state per stage;
    Stage 3 all-gathers parameters in forward/backward order and frees them;
  - "design trade-off 1": buckets (large buckets favour bandwidth, small
    ones release memory sooner).

The arithmetic (reduction fold, Adam, casts) lives in ``zero_oracle.c``; this
module holds the layout bookkeeping (plan, flatten, gather), the memory and
communication-volume analysis, and thin ctypes wrappers.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import List, Sequence

import numpy as np

from . import _build

F32, F16, BF16 = 0, 1, 2
_ESIZE = {F32: 4, F16: 2, BF16: 2}

_lib = None


def lib():
    """Load (building once if absent) the oracle's C library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        c_i64, c_i32, c_p = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f16_value.restype = ctypes.c_double
        L.orc_f16_value.argtypes = [ctypes.c_uint16]
        L.orc_bf16_value.restype = ctypes.c_double
        L.orc_bf16_value.argtypes = [ctypes.c_uint16]
        L.orc_cast_f32_to_16.argtypes = [c_p, c_p, c_i64, ctypes.c_int]
        L.orc_cast_bits_range_to_16.argtypes = [ctypes.c_uint32, c_i64, c_p, ctypes.c_int]
        L.orc_adam_consts.argtypes = [ctypes.c_double] * 5 + [c_i64, c_p]
        L.orc_reduce.argtypes = [c_i32, c_p, ctypes.c_int, c_i64, ctypes.c_float, c_p]
        L.orc_adam.argtypes = [c_i64, c_p, c_p, c_p, c_p, c_p, c_p, ctypes.c_int]
        L.orc_adam_f64.argtypes = [c_i64, c_p, c_p, c_p, c_p] + [ctypes.c_double] * 4 + [c_i64]
        L.orc_widen_to_f64.argtypes = [c_p, ctypes.c_int, c_i64, c_p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


# --------------------------------------------------------------------------
# Plan: buckets, padding, shard ownership
# --------------------------------------------------------------------------

@dataclass
class Bucket:
    flat_off: int      # first element of the bucket in the padded flat buffer
    numel: int         # real elements (sum of its tensors)
    padded: int        # numel rounded up to a multiple of n_d * align
    shard_numel: int   # padded / n_d, the slice each rank owns
    shard_off: int     # where this bucket's slice starts in a rank's shard


@dataclass
class Plan:
    psi: int
    n_d: int
    align: int
    bucket_cap: int
    buckets: List[Bucket] = field(default_factory=list)
    tensor_bucket: List[int] = field(default_factory=list)
    tensor_off: List[int] = field(default_factory=list)   # flat offset of each tensor
    tensor_numel: List[int] = field(default_factory=list)

    @property
    def psi_pad(self) -> int:
        return sum(b.padded for b in self.buckets)

    @property
    def shard_total(self) -> int:
        return sum(b.shard_numel for b in self.buckets)

    def owner_range(self, b: int, rank: int):
        """Flat range [lo, hi) of bucket b that rank owns."""
        bk = self.buckets[b]
        lo = bk.flat_off + rank * bk.shard_numel
        return lo, lo + bk.shard_numel

    def is_pad(self, flat_index: int) -> bool:
        for bk in self.buckets:
            if bk.flat_off <= flat_index < bk.flat_off + bk.padded:
                return flat_index >= bk.flat_off + bk.numel
        raise IndexError(flat_index)


def plan(psi: int, n_d: int, sizes: Sequence[int], bucket_cap: int = 0, align: int = 64) -> Plan:
    """Assign tensors to padded flat buckets and each bucket's slices to ranks.

    Tensors are taken in list order and never split.  A new bucket starts
    when the next tensor would push the current (non-empty) bucket past
    ``bucket_cap`` elements, so a tensor larger than the cap sits alone;
    ``bucket_cap == 0`` puts everything in one bucket.  Each bucket is padded at
    its end to a multiple of ``n_d * align``; rank r owns the r-th contiguous
    1/n_d of every bucket, as GPU i keeps block i in the mind-map page's
    four-GPU example.  A rank's shard is its slices of all buckets, in bucket
    order.
    """
    if n_d < 1 or align < 1 or bucket_cap < 0:
        raise ValueError("n_d >= 1, align >= 1, bucket_cap >= 0 required")
    if any(s < 0 for s in sizes) or sum(sizes) != psi:
        raise ValueError("tensor sizes must be >= 0 and sum to psi")
    groups: List[List[int]] = []
    cur: List[int] = []
    cur_n = 0
    for t, n in enumerate(sizes):
        if bucket_cap > 0 and cur and cur_n + n > bucket_cap:
            groups.append(cur)
            cur, cur_n = [], 0
        cur.append(t)
        cur_n += n
    if cur:
        groups.append(cur)

    p = Plan(psi=psi, n_d=n_d, align=align, bucket_cap=bucket_cap)
    p.tensor_bucket = [0] * len(sizes)
    p.tensor_off = [0] * len(sizes)
    p.tensor_numel = list(sizes)
    unit = n_d * align
    flat = 0
    shard = 0
    for b, g in enumerate(groups):
        numel = 0
        for t in g:
            p.tensor_bucket[t] = b
            p.tensor_off[t] = flat + numel
            numel += sizes[t]
        padded = ((numel + unit - 1) // unit) * unit
        sn = padded // n_d
        p.buckets.append(Bucket(flat, numel, padded, sn, shard))
        flat += padded
        shard += sn
    return p


# --------------------------------------------------------------------------
# Flatten / gather: bit copies
# --------------------------------------------------------------------------

def flatten(p: Plan, tensors: Sequence[np.ndarray]) -> np.ndarray:
    """Pack the tensors into the padded flat buffer; padding is zero."""
    dtype = tensors[0].dtype if tensors else np.uint16
    out = np.zeros(p.psi_pad, dtype=dtype)
    for t, x in enumerate(tensors):
        x = np.ascontiguousarray(x).reshape(-1)
        assert x.size == p.tensor_numel[t]
        o = p.tensor_off[t]
        out[o:o + x.size] = x
    return out


def unflatten(p: Plan, flat: np.ndarray) -> List[np.ndarray]:
    return [flat[o:o + n].copy() for o, n in zip(p.tensor_off, p.tensor_numel)]


def shard_of(p: Plan, rank: int, full: np.ndarray) -> np.ndarray:
    """The rank's shard: its owned slice of every bucket, concatenated."""
    parts = []
    for b in range(len(p.buckets)):
        lo, hi = p.owner_range(b, rank)
        parts.append(full[lo:hi])
    if not parts:
        return full[:0].copy()
    return np.concatenate(parts)


def place_shard(p: Plan, rank: int, shard: np.ndarray, full: np.ndarray) -> None:
    """Write a rank's shard into a full-size buffer at its owned ranges (the
    local half of all-gather)."""
    for b, bk in enumerate(p.buckets):
        lo, hi = p.owner_range(b, rank)
        full[lo:hi] = shard[bk.shard_off:bk.shard_off + bk.shard_numel]


def gather_pack(p: Plan, shards: Sequence[np.ndarray]) -> np.ndarray:
    """Materialise the full buffer from all n_d shards (the local layout of
    all-gather, and Stage 3's per-layer materialisation)."""
    assert len(shards) == p.n_d
    full = np.zeros(p.psi_pad, dtype=shards[0].dtype if len(shards) else np.uint16)
    for r, s in enumerate(shards):
        place_shard(p, r, s, full)
    return full


def reshard(src: Plan, dst: Plan, dst_rank: int, src_shards: Sequence[np.ndarray]) -> np.ndarray:
    """The shard of dst_rank under plan dst, from all shards under plan src
    (same tensor list): materialise the flat buffer, split it back into the
    tensors, flatten them with the new plan and take the rank's slices."""
    assert src.tensor_numel == dst.tensor_numel
    full = gather_pack(src, src_shards)
    tensors = unflatten(src, full)
    if tensors:
        flat = flatten(dst, tensors)
    else:
        flat = np.zeros(dst.psi_pad, dtype=full.dtype)
    return shard_of(dst, dst_rank, flat)


# --------------------------------------------------------------------------
# Arithmetic (through the C oracle)
# --------------------------------------------------------------------------

def f32_to_16(x: np.ndarray, dt: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_cast_f32_to_16(_ptr(x), _ptr(out), x.size, dt)
    return out


def value16(h: np.ndarray, dt: int) -> np.ndarray:
    """Exact value of 16-bit patterns as float64."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float64)
    lib().orc_widen_to_f64(_ptr(h), dt, h.size, _ptr(out))
    return out


def adam_consts(lr, beta1, beta2, eps, grad_scale, t) -> np.ndarray:
    out = np.empty(9, dtype=np.float32)
    lib().orc_adam_consts(lr, beta1, beta2, eps, grad_scale, t, _ptr(out))
    return out


def reduce(slices: Sequence[np.ndarray], dt: int, grad_scale: float) -> np.ndarray:
    """Fixed-order fp32 fold of the ranks' contributions, times grad_scale."""
    n = len(slices)
    count = slices[0].size
    arrs = [np.ascontiguousarray(s, dtype=np.uint16) for s in slices]
    for a in arrs:
        assert a.size == count
    ptrs = (ctypes.c_void_p * n)(*[a.ctypes.data for a in arrs])
    out = np.empty(count, dtype=np.float32)
    lib().orc_reduce(n, ptrs, dt, count, ctypes.c_float(np.float32(grad_scale)), _ptr(out))
    return out


def adam(g: np.ndarray, w: np.ndarray, m: np.ndarray, v: np.ndarray,
         consts: np.ndarray, pdt: int) -> np.ndarray:
    """One Adam step in place on fp32 (w, m, v); returns the 16-bit params."""
    for a in (g, w, m, v):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    p16 = np.empty(w.size, dtype=np.uint16)
    lib().orc_adam(w.size, _ptr(g), _ptr(w), _ptr(m), _ptr(v), _ptr(consts), _ptr(p16), pdt)
    return p16


def adam_f64(g, w, m, v, lr, beta1, beta2, eps, t):
    for a in (g, w, m, v):
        assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    lib().orc_adam_f64(w.size, _ptr(g), _ptr(w), _ptr(m), _ptr(v), lr, beta1, beta2, eps, t)


@dataclass
class Hyper:
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    grad_scale: float = 1.0


def shard_step(slices: Sequence[np.ndarray], gdt: int, hp: Hyper, t: int,
               w: np.ndarray, m: np.ndarray, v: np.ndarray, pdt: int) -> np.ndarray:
    """Reduce the owner's partition, then Adam on it (no fusion: the two
    steps one after the other)."""
    c = adam_consts(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.grad_scale, t)
    g = reduce(slices, gdt, float(c[8]))
    return adam(g, w, m, v, c, pdt)


def owner_slices_from_full(p: Plan, rank: int, fulls: Sequence[np.ndarray]) -> List[np.ndarray]:
    """What reduce-scatter delivers to the owner: each rank's gradient
    restricted to the owner's ranges, in shard-local layout."""
    return [shard_of(p, rank, f) for f in fulls]


# --------------------------------------------------------------------------
# Memory and communication analysis
# --------------------------------------------------------------------------

def memory_closed_form(psi: float, n_d: int, k: int = 12) -> dict:
    """Per-GPU model-state bytes with 2-byte params, 2-byte grads and K bytes
    of optimizer state per parameter, for standard data parallelism and the
    three sharding stages (the paper's Table 1 as quoted on the mind-map
    page, "Stage 1/2/3" section)."""
    return {
        "dp": (2 + 2 + k) * psi,
        "os": 4 * psi + k * psi / n_d,
        "os_g": 2 * psi + (2 + k) * psi / n_d,
        "os_g_p": (2 + 2 + k) * psi / n_d,
    }


# Which states each configuration keeps sharded (ZeRO concept page, "three
# stages" table; standard DP shards nothing).
STAGE_SHARDED = {
    "dp": set(),
    "os": {"optim"},
    "os_g": {"optim", "grads"},
    "os_g_p": {"optim", "grads", "params"},
}


def memory_from_layout(p: Plan, stage: str, k: int = 12) -> int:
    """Per-GPU model-state bytes counted from the buffers the layout keeps
    resident: each state is either the full padded flat buffer or one shard."""
    sharded = STAGE_SHARDED[stage]
    full, shard = p.psi_pad, p.shard_total
    params = 2 * (shard if "params" in sharded else full)
    grads = 2 * (shard if "grads" in sharded else full)
    optim = k * (shard if "optim" in sharded else full)
    return params + grads + optim


def comm_volume(p: Plan, stage: str, perspective: int = 0) -> dict:
    """Elements of the 16-bit buffers each collective spans, per rank per step,
    counted by walking the slice lists of the reduce and gather layouts: every
    rank's slice of every bucket, the rank's own slice included ("elements"),
    and without it ("off_rank_elements", what crosses a GPU boundary).

    Standard DP, Stage 1 and Stage 2: one reduce-scatter of the gradients plus
    one all-gather of the parameters (an all-reduce is exactly these two).
    Stage 3: parameters are all-gathered once in forward and once in backward,
    plus the gradient reduce-scatter ("three stages" table of the concept page).
    """
    def walk():
        total = off = 0
        for b in range(len(p.buckets)):
            for r in range(p.n_d):
                lo, hi = p.owner_range(b, r)
                total += hi - lo
                if r != perspective:
                    off += hi - lo
        return total, off

    if stage in ("dp", "os", "os_g"):
        ops = {"reduce_scatter": walk(), "all_gather": walk()}
    elif stage == "os_g_p":
        ops = {"reduce_scatter": walk(), "all_gather_fwd": walk(), "all_gather_bwd": walk()}
    else:
        raise ValueError(stage)
    total = sum(v[0] for v in ops.values())
    off = sum(v[1] for v in ops.values())
    return {"elements": total, "bytes": 2 * total, "off_rank_elements": off,
            "ops": {k: v[0] for k, v in ops.items()}}
