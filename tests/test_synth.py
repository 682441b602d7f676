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
    pos = _positions(500_000, 1)
    k, ks = synth.key_of(3, synth.STREAM_GRAD, 17, 6), synth.key_of(3, synth.STREAM_MIXSEL, 17, 6)
    a = synth.mix_f32(k, ks, pos, 1e-3) if mix else synth.normal_f32(k, pos, 1e-3)
    b = synth.mix_f32_np(k, ks, pos, 1e-3) if mix else synth.normal_f32_np(k, pos, 1e-3)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_draw_statistics():
    pos = np.arange(2_000_000, dtype=np.int64)
    x = synth.normal_f32(synth.key_of(1, synth.STREAM_GRAD, 0, 1), pos, 1e-3).astype(np.float64)
    assert abs(x.mean()) < 5e-6 and abs(x.std() - 1e-3) < 1e-5
    assert np.abs(x).max() <= 1e-3 * 3.47
    y = synth.mix_f32(synth.key_of(4, synth.STREAM_GRAD, 0, 1), synth.key_of(4, synth.STREAM_MIXSEL, 0, 1),
                      pos, 1e-3)
    assert abs((y == 0).mean() - 0.01) < 5e-4
    assert abs((np.abs(y) == 100).mean() - 0.001) < 1.5e-4


def test_streams_are_distinct():
    pos = np.arange(100_000, dtype=np.int64)
    a = synth.normal_f32(synth.key_of(3, 1, 0, 1), pos, 1.0)
    b = synth.normal_f32(synth.key_of(3, 1, 1, 1), pos, 1.0)
    c = synth.normal_f32(synth.key_of(3, 1, 0, 2), pos, 1.0)
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.02 and abs(np.corrcoef(a, c)[0, 1]) < 0.02


@pytest.mark.gpu
@pytest.mark.parametrize("dt", [synth.F32, synth.F16, synth.BF16])
@pytest.mark.parametrize("mix", [False, True])
def test_gpu_fill_matches_host(gpu, dt, mix):
    import torch
    from synth import gpu as SG
    n, base = 3_000_001, 12_999_000_000
    k, ks = synth.key_of(5, synth.STREAM_GRAD, 3, 2), synth.key_of(5, synth.STREAM_MIXSEL, 3, 2)
    t = torch.empty(n, dtype=torch.float32 if dt == synth.F32 else torch.int16, device=gpu)
    SG.fill(t.data_ptr(), dt, n, k, base, 1e-3, torch.cuda.current_stream().cuda_stream, mix, ks)
    torch.cuda.synchronize()
    got = t.cpu().numpy().view(np.uint32 if dt == synth.F32 else np.uint16)
    pos = np.arange(base, base + n, dtype=np.int64)
    x = synth.mix_f32(k, ks, pos, 1e-3) if mix else synth.normal_f32(k, pos, 1e-3)
    want = synth.to_dtype_bits(x, dt).view(np.uint32 if dt == synth.F32 else np.uint16)
    assert np.array_equal(got, want)
