"""The seeded input generator: its three implementations agree bit for bit,
and its draws have the intended shape (mean, spread, bound, mix rates)."""
import numpy as np
import pytest

import synth


def _positions(n, seed):
    rng = np.random.default_rng(seed)
    return np.concatenate([np.arange(1000, dtype=np.int64),
                           rng.integers(0, 13_000_000_000, size=n, dtype=np.int64)])


@pytest.mark.parametrize("mix", [False, True])
def test_c_matches_numpy(mix):
    pos = _positions(2_000_000, 1)
    k, ks = synth.key_of(3, synth.STREAM_GRAD, 17, 6), synth.key_of(3, synth.STREAM_MIXSEL, 17, 6)
    a = synth.mix_f32(k, ks, pos, 1e-3) if mix else synth.normal_f32(k, pos, 1e-3)
    b = synth.mix_f32_np(k, ks, pos, 1e-3) if mix else synth.normal_f32_np(k, pos, 1e-3)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_draw_statistics():
    """The draws are N(0, sigma) as the workloads state (Box-Muller, tails to
    5.77 sigma): mean, spread, two- and three-sigma tail shares, kurtosis and
    the bound; and the zero/outlier mix rates of the 13B workload."""
    pos = np.arange(4_000_000, dtype=np.int64)
    x = synth.normal_f32(synth.key_of(1, synth.STREAM_GRAD, 0, 1), pos, 1e-3).astype(np.float64)
    assert abs(x.mean()) < 3e-6 and abs(x.std() - 1e-3) < 3e-6
    assert abs((np.abs(x) > 2e-3).mean() - 0.045500) < 5e-4        # 2 P(Z > 2)
    assert abs((np.abs(x) > 3e-3).mean() - 0.002700) < 1.5e-4      # 2 P(Z > 3)
    kurt = ((x - x.mean()) ** 4).mean() / x.var() ** 2
    assert abs(kurt - 3.0) < 0.02
    assert np.abs(x).max() <= 1e-3 * synth.Z_MAX * (1 + 1e-6)
    y = synth.mix_f32(synth.key_of(4, synth.STREAM_GRAD, 0, 1), synth.key_of(4, synth.STREAM_MIXSEL, 0, 1),
                      pos, 1e-3)
    assert abs((y == 0).mean() - 0.01) < 5e-4
    assert abs((np.abs(y) == 100).mean() - 0.001) < 1.5e-4


def test_unit_normal_follows_box_muller():
    """The fp32 sequence computes sqrt(-2 ln u1) cos(2 pi u2) of the hash's two
    24-bit uniforms to within 4e-7 of the radius (float64 reference with
    numpy's log and cos), including the extreme hashes."""
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64) << np.uint64(32)
    u |= rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64)
    edge = np.array([0, (2 ** 24 - 1) << 40, 0xFFFFFFFFFFFFFFFF, 0x3FFFFF00, 0x400000 << 8, 0xFFFFFF00],
                    dtype=np.uint64)
    u = np.concatenate([u, edge])
    z32 = synth.unit_normal_np(u).astype(np.float64)
    u1 = ((u >> np.uint64(40)) + np.uint64(1)).astype(np.float64) / 2 ** 24
    u2 = ((u & np.uint64(0xFFFFFFFF)) >> np.uint64(8)).astype(np.float64) / 2 ** 24
    r = np.sqrt(-2.0 * np.log(u1))
    z = r * np.cos(2.0 * np.pi * u2)
    assert np.all(np.abs(z32 - z) <= 4e-7 * r + 1e-30)
    assert z32[-6] == np.float32(synth.Z_MAX) or abs(z32[-6] - synth.Z_MAX) < 4e-6   # u1 = 2^-24, angle 0


def test_streams_are_distinct():
    pos = np.arange(100_000, dtype=np.int64)
    a = synth.normal_f32(synth.key_of(3, 1, 0, 1), pos, 1.0)
    b = synth.normal_f32(synth.key_of(3, 1, 1, 1), pos, 1.0)
    c = synth.normal_f32(synth.key_of(3, 1, 0, 2), pos, 1.0)
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.02 and abs(np.corrcoef(a, c)[0, 1]) < 0.02


@pytest.mark.gpu
@pytest.mark.parametrize("dt", [synth.F32, synth.F16, synth.BF16])
@pytest.mark.parametrize("mix", [False, True])
@pytest.mark.parametrize("nt", [False, True])
def test_gpu_fill_matches_host(gpu, dt, mix, nt):
    """The GPU fill, with ordinary or non-temporal stores, equals the numpy
    definition bit for bit."""
    import torch
    from synth import gpu as SG
    n, base = 3_000_001, 12_999_000_000
    k, ks = synth.key_of(5, synth.STREAM_GRAD, 3, 2), synth.key_of(5, synth.STREAM_MIXSEL, 3, 2)
    t = torch.empty(n, dtype=torch.float32 if dt == synth.F32 else torch.int16, device=gpu)
    SG.fill(t.data_ptr(), dt, n, k, base, 1e-3, torch.cuda.current_stream().cuda_stream, mix, ks, nt)
    torch.cuda.synchronize()
    got = t.cpu().numpy().view(np.uint32 if dt == synth.F32 else np.uint16)
    pos = np.arange(base, base + n, dtype=np.int64)
    x = synth.mix_f32(k, ks, pos, 1e-3) if mix else synth.normal_f32(k, pos, 1e-3)
    want = synth.to_dtype_bits(x, dt).view(np.uint32 if dt == synth.F32 else np.uint16)
    assert np.array_equal(got, want)


def test_cu_mask_words():
    """CU index sets -> 32-bit mask words (host logic of the CU-masked streams)."""
    from synth.gpu import cu_mask_words
    assert cu_mask_words(range(16), 256) == [0xFFFF, 0, 0, 0, 0, 0, 0, 0]
    assert cu_mask_words(range(16, 256), 256) == [0xFFFF0000] + [0xFFFFFFFF] * 7
    assert cu_mask_words([0, 33, 255], 256) == [1, 2, 0, 0, 0, 0, 0, 1 << 31]
    assert cu_mask_words([], 80) == [0, 0, 0]
    a, b = cu_mask_words(range(64), 256), cu_mask_words(range(64, 256), 256)
    assert all(x & y == 0 for x, y in zip(a, b)) and all(x | y == 0xFFFFFFFF for x, y in zip(a, b))
    with pytest.raises(ValueError):
        cu_mask_words([256], 256)
    with pytest.raises(ValueError):
        cu_mask_words([-1], 256)


@pytest.mark.parametrize("k", [8, 16, 32, 64, 128, 248])
def test_balanced_cus(k):
    """The CU set of a masked stream, and its complement, give every die the
    same number of CUs under both numberings (die-major and round-robin)."""
    from synth.gpu import balanced_cus
    n, dies = 256, 8
    a = balanced_cus(k, n, dies)
    b = sorted(set(range(n)) - set(a))
    assert len(a) == k and len(set(a)) == k and all(0 <= i < n for i in a)
    for cus, want in ((a, k // dies), (b, (n - k) // dies)):
        assert np.bincount([i // (n // dies) for i in cus], minlength=dies).tolist() == [want] * dies
        assert np.bincount([i % dies for i in cus], minlength=dies).tolist() == [want] * dies
    with pytest.raises(ValueError):
        balanced_cus(12, n, dies)


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [1 << 20, (1 << 20) + 16 * 777])
def test_calibration_probes(gpu, nbytes):
    """The HBM calibration probes do what they claim, also when the last
    workgroup is partial: the copy copies every byte, the write writes its
    pattern everywhere and nothing past the end, and both reads (non-temporal
    and cached) see the data (each workgroup's sink word is the xor of the
    16-byte units its first lane read)."""
    import torch
    from synth import gpu as SG
    n = nbytes // 4
    stream = torch.cuda.current_stream().cuda_stream
    src = torch.randint(-2**31, 2**31 - 1, (n + 64,), dtype=torch.int32, device=gpu)
    dst = torch.zeros(n + 64, dtype=torch.int32, device=gpu)
    SG.probe(SG.PROBE_COPY, dst.data_ptr(), src.data_ptr(), nbytes, 0, stream)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src[:n]) and not torch.any(dst[n:])
    SG.probe(SG.PROBE_WRITE, dst.data_ptr(), 0, nbytes, 0, stream)
    torch.cuda.synchronize()
    assert torch.all(dst[:n] == 0x3c003c00) and not torch.any(dst[n:])
    host = src[:n].cpu().numpy().view(np.uint32).reshape(-1, 4)   # 16-byte units
    words = SG.probe_sink_words(nbytes)
    for kind in (SG.PROBE_READ, SG.PROBE_READ_CACHED):
        sink = torch.zeros(words, dtype=torch.int32, device=gpu)
        SG.probe(kind, 0, src.data_ptr(), nbytes, sink.data_ptr(), stream)
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32)
        # Workgroup b's first lane (lane 0 of wave 0) reads units b*T*U + i*64 (i < U) on the
        # full-block path, units b*T*U + i*T on the last block's checked path.
        T, U = 1024, 8
        units = host.shape[0]
        for b in range(words):
            first = b * T * U
            idx = [first + i * 64 for i in range(U)] if first + T * U <= units else \
                  [first + i * T for i in range(U) if first + i * T < units]
            want = np.bitwise_xor.reduce(np.bitwise_xor.reduce(host[idx], axis=0)) if idx else 0
            assert got[b] == want, (kind, b)


@pytest.mark.gpu
@pytest.mark.parametrize("lds", [4, 32768])
def test_elastic_compute(gpu, lds):
    """The Stage-3 study's elastic compute stand-in computes what it says:
    per thread the affine recurrence x <- a x + b from its weight, which has
    the closed form a^k x0 + b (1 - a^k) / (1 - a), summed per workgroup;
    and it rejects an LDS size outside [4, 64 KiB]."""
    import torch
    from synth import gpu as SG
    n, blocks, iters = 700, 5, 300
    w = torch.randint(0, 65536, (n,), dtype=torch.int32).to(torch.int16).to(gpu)
    out = torch.zeros(blocks, dtype=torch.float32, device=gpu)
    stream = torch.cuda.current_stream().cuda_stream
    SG.elastic_compute(w.data_ptr(), n, iters, blocks, out.data_ptr(), stream, lds)
    torch.cuda.synchronize()
    a, b = np.float64(np.float32(0.999)), np.float64(np.float32(1e-3))
    x0 = w.cpu().numpy().view(np.uint16).astype(np.float64) * 2.0 ** -16
    idx = np.arange(blocks * 256) % n
    x = a ** iters * x0[idx] + b * (1 - a ** iters) / (1 - a)
    want = x.reshape(blocks, 256).sum(axis=1)
    np.testing.assert_allclose(out.cpu().numpy(), want, rtol=1e-4)
    for bad in (0, 65540):
        with pytest.raises(RuntimeError):
            SG.elastic_compute(w.data_ptr(), n, iters, blocks, out.data_ptr(), stream, bad)


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16 * 1023, 16 * (1024 * 37 + 5), 1 << 22])
@pytest.mark.parametrize("cap", [1, 3, 256])
def test_capped_copy_probe(gpu, nbytes, cap):
    """The capped-grid copy copies every byte and nothing past the end, with
    a ragged tail and with fewer workgroups than chunks."""
    import torch
    from synth import gpu as SG
    n = nbytes // 4
    src = torch.randint(-2**31, 2**31 - 1, (n + 64,), dtype=torch.int32, device=gpu)
    dst = torch.zeros(n + 64, dtype=torch.int32, device=gpu)
    SG.probe_copy_capped(dst.data_ptr(), src.data_ptr(), nbytes, cap, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src[:n]) and not torch.any(dst[n:])
