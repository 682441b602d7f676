"""GPU parity of the bit-copy entry points: zero_flatten (ragged tensors into
padded flat buckets) and zero_gather_pack (n_d shards into the full buffer),
bit-exact against the oracle, at aligned and misaligned element offsets."""
import numpy as np
import pytest

import synth
from synth.workloads import gpt2_small_sizes

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def rand_bits(seed, n, es):
    u = synth.draw_u64(synth.key_of(seed, 9, 0, 0), np.arange(n, dtype=np.uint64))
    return (u & np.uint64(0xFFFF)).astype(np.uint16) if es == 2 else (u & np.uint64(0xFFFFFFFF)).astype(np.uint32)


def _carve(torch, dev, host_arrays, offsets_mod, es):
    """Place each host array in one device buffer at an element offset with
    the given residue modulo 8, so tensor bases are not 16-byte aligned."""
    dt = torch.int16 if es == 2 else torch.int32
    total = sum(a.size + 16 for a in host_arrays) + 16
    buf = torch.zeros(total, dtype=dt, device=dev)
    views, pos = [], 0
    for a, r in zip(host_arrays, offsets_mod):
        pos = (pos + 7) // 8 * 8 + r
        v = buf[pos:pos + a.size]
        v.copy_(torch.from_numpy(a.view(np.int16 if es == 2 else np.int32)))
        views.append(v)
        pos += a.size
    return buf, views


@pytest.mark.parametrize("es,align,cap", [(2, 64, 1 << 24), (2, 1, 1 << 20), (4, 8, 1 << 22)])
def test_flatten_gpt2_list(gpu, oracle_lib, zero_lib, es, align, cap):
    import torch
    O, Z = oracle_lib, zero_lib
    sizes = gpt2_small_sizes() if es == 2 else gpt2_small_sizes(h=256, vocab=5000)
    say(f"[flatten] gpt2 list es={es} align={align} cap={cap}: {len(sizes)} tensors")
    rng = np.random.default_rng(es * 100 + align)
    data = [rand_bits(1000 + t, n, es) for t, n in enumerate(sizes)]
    mods = rng.integers(0, 8, size=len(sizes)) if align == 1 else np.zeros(len(sizes), int)
    _, views = _carve(torch, gpu, data, mods, es)
    zp = Z.zero_plan(sum(sizes), 8, sizes, cap, align)
    op = O.plan(sum(sizes), 8, sizes, cap, align)
    flat = torch.full((zp.psi_pad,), -1, dtype=torch.int16 if es == 2 else torch.int32, device=gpu)
    dt = Z.ZERO_BF16 if es == 2 else Z.ZERO_F32
    Z.zero_flatten(zp, views, dt, flat)
    torch.cuda.synchronize()
    got = flat.cpu().numpy().view(np.uint16 if es == 2 else np.uint32)
    want = O.flatten(op, data)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("es", [2, 4])
def test_flatten_ragged_misaligned(gpu, oracle_lib, zero_lib, es):
    import torch
    O, Z = oracle_lib, zero_lib
    rng = np.random.default_rng(77 + es)
    for trial in range(6):
        nt = int(rng.integers(1, 40))
        sizes = [int(x) for x in rng.choice([0, 1, 2, 3, 7, 8, 9, 15, 16, 17, 100, 1023, 4099, 70001],
                                            size=nt)]
        n_d = int(rng.choice([1, 2, 3, 4, 8]))
        align = int(rng.choice([1, 2, 8, 64]))
        cap = int(rng.choice([0, 50, 5000]))
        say(f"[flatten] ragged trial {trial}: {nt} tensors n_d={n_d} align={align} cap={cap} es={es}")
        data = [rand_bits(5000 + 97 * trial + t, n, es) for t, n in enumerate(sizes)]
        _, views = _carve(torch, gpu, data, rng.integers(0, 8, size=nt), es)
        psi = sum(sizes)
        zp = Z.zero_plan(psi, n_d, sizes, cap, align)
        op = O.plan(psi, n_d, sizes, cap, align)
        # Destination at an odd element offset too.
        off = int(rng.integers(0, 8))
        big = torch.full((zp.psi_pad + 16,), -1, dtype=torch.int16 if es == 2 else torch.int32, device=gpu)
        flat = big[off:off + zp.psi_pad]
        Z.zero_flatten(zp, [v if v.numel() else None for v in views],
                       Z.ZERO_F16 if es == 2 else Z.ZERO_F32, flat)
        torch.cuda.synchronize()
        got = big.cpu().numpy().view(np.uint16 if es == 2 else np.uint32)
        want = O.flatten(op, data) if data else np.zeros(0, np.uint16 if es == 2 else np.uint32)
        assert np.array_equal(got[off:off + zp.psi_pad], want.astype(got.dtype))
        fill = np.uint16(0xFFFF) if es == 2 else np.uint32(0xFFFFFFFF)
        assert np.all(got[:off] == fill) and np.all(got[off + zp.psi_pad:] == fill)


@pytest.mark.parametrize("es,align,n_d", [(2, 64, 64), (2, 1, 5), (4, 1, 3), (2, 8, 4)])
def test_gather_pack(gpu, oracle_lib, zero_lib, es, align, n_d):
    import torch
    O, Z = oracle_lib, zero_lib
    sizes = [12_345, 0, 999, 65_536, 7, 300_001]
    say(f"[gather_pack] es={es} align={align} n_d={n_d}")
    zp = Z.zero_plan(sum(sizes), n_d, sizes, 70_000, align)
    op = O.plan(sum(sizes), n_d, sizes, 70_000, align)
    shards = [rand_bits(9000 + q, op.shard_total, es) for q in range(n_d)]
    tdt = torch.int16 if es == 2 else torch.int32
    dev_shards = [torch.from_numpy(s.view(np.int16 if es == 2 else np.int32)).to(gpu) for s in shards]
    full = torch.full((zp.psi_pad,), -1, dtype=tdt, device=gpu)
    Z.zero_gather_pack(zp, dev_shards, Z.ZERO_F16 if es == 2 else Z.ZERO_F32, full)
    torch.cuda.synchronize()
    got = full.cpu().numpy().view(np.uint16 if es == 2 else np.uint32)
    assert np.array_equal(got, O.gather_pack(op, shards))


def _reshard_case(torch, gpu, O, Z, sizes, src_cfg, dst_cfg, es, seed):
    psi = sum(sizes)
    (n_d, cap, align), (n_d2, cap2, align2) = src_cfg, dst_cfg
    zs, zd = Z.zero_plan(psi, n_d, sizes, cap, align), Z.zero_plan(psi, n_d2, sizes, cap2, align2)
    os_, od = O.plan(psi, n_d, sizes, cap, align), O.plan(psi, n_d2, sizes, cap2, align2)
    # source shards: bits at real elements, zero padding (what a sharded state holds)
    tensors = [rand_bits(seed + t, n, es) for t, n in enumerate(sizes)]
    flat = O.flatten(os_, tensors)
    shards = [O.shard_of(os_, r, flat) for r in range(n_d)]
    npdt, tdt = (np.int16, torch.int16) if es == 2 else (np.int32, torch.int32)
    dev = [torch.from_numpy(s.view(npdt)).to(gpu) for s in shards]
    dt = Z.ZERO_BF16 if es == 2 else Z.ZERO_F32
    for r in range(n_d2):
        out = torch.full((zd.shard_total,), -1, dtype=tdt, device=gpu)
        Z.zero_reshard(zs, zd, r, dev, dt, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy().view(np.uint16 if es == 2 else np.uint32)
        assert np.array_equal(got, O.reshard(os_, od, r, shards)), (src_cfg, dst_cfg, r)


@pytest.mark.parametrize("es", [2, 4])
def test_reshard_random_plans(gpu, oracle_lib, zero_lib, es):
    import torch
    rng = np.random.default_rng(90 + es)
    for trial in range(8):
        nt = int(rng.integers(1, 25))
        sizes = [int(x) for x in rng.choice([0, 1, 5, 8, 63, 64, 100, 1000, 4097, 20000], size=nt)]
        src = (int(rng.choice([1, 2, 3, 4, 8])), int(rng.choice([0, 500, 5000])), int(rng.choice([1, 8, 64])))
        dst = (int(rng.choice([1, 2, 3, 5, 16])), int(rng.choice([0, 700, 9000])), int(rng.choice([1, 4, 64])))
        say(f"[reshard] trial {trial}: {nt} tensors {src} -> {dst} es={es}")
        _reshard_case(torch, gpu, oracle_lib, zero_lib, sizes, src, dst, es, 300 + trial)


@pytest.mark.parametrize("src,dst", [((8, 1 << 24, 64), (16, 1 << 24, 64)), ((8, 1 << 24, 64), (3, 1 << 22, 1))])
def test_reshard_gpt2_state(gpu, oracle_lib, zero_lib, src, dst):
    import torch
    say(f"[reshard] gpt2 fp32 state {src} -> {dst}")
    _reshard_case(torch, gpu, oracle_lib, zero_lib, gpt2_small_sizes(), src, dst, 4, 700)
