"""The seeded input generator (shared by oracle-side and GPU-side tests).

Checks: a numpy re-implementation of the counter-based word stream
(splitmix64 output function, Steele/Lea/Flood 2014) matches bit for bit and
its Box-Muller normals to fp64 rounding; any slice equals the same slice of a
larger draw; heavy-hitter count and placement; bf16 rounding is the single
nearest-even rounding of the fp64 draw; moments of the draws.
"""
import numpy as np
import pytest

import tkvsynth

M64 = (1 << 64) - 1


def _mix64(z):
    z = (z + 0x9E3779B97F4A7C15) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _key(seed, tid):
    return _mix64(_mix64(seed) ^ ((tid * 0xD1B54A32D192ED03) & M64))


def test_word_stream_matches_python_mirror():
    for seed, tid in [(0, 1), (7, 5), (2**40 + 3, 3)]:
        got = tkvsynth.words(seed, tid, 123, 50)
        k = _key(seed, tid)
        ref = [_mix64((k + 123 + i) & M64) for i in range(50)]
        assert [int(x) for x in got] == ref


def test_normals_match_python_mirror():
    import math
    seed, tid, n0 = 3, 2, 1000
    got = tkvsynth.normals(seed, tid, n0, 64)
    k = _key(seed, tid)
    for i, g in enumerate(got):
        n = n0 + i
        x, y = _mix64((k + 2 * n) & M64), _mix64((k + 2 * n + 1) & M64)
        u1 = ((x >> 11) + 0.5) * 2.0 ** -53
        u2 = (y >> 11) * 2.0 ** -53
        ref = math.sqrt(-2.0 * math.log(u1)) * math.cos(2 * math.pi * u2)
        assert abs(g - ref) <= 4e-16 * max(1.0, abs(ref))


@pytest.mark.parametrize("name", ["tiny", "14b"])
def test_slices_agree(name):
    w = tkvsynth.CONFIGS[name].replace(layers=2, prefill=40, steps=8)
    full = w.kv(0, 0, w.n_final)
    part = w.kv(0, 17, 9)
    assert np.array_equal(full[:, :, 17:26], part)
    qa = w.q(0, 8)
    qb = w.q(5, 2)
    assert np.array_equal(qa[5:7], qb)
    assert np.array_equal(w.kv(1, 3, 4), w.kv(1, 3, 4))


def test_heavy_hitters():
    w = tkvsynth.CONFIGS["14b"]
    m = w.heavy_mask()
    nh = int(round(0.05 * w.n_final))
    assert m.shape == (w.batch, w.n_final)
    assert np.all(m.sum(axis=1) == nh)
    assert not np.array_equal(m[0], m[1])          # independent per sequence
    # heavy K rows carry the planted direction
    w2 = w.replace(layers=1)
    u = w2.unit_vector()
    K = w2.values(w2.kv(0, 0, 512)).astype(np.float64)
    proj = K[0, 0] @ u                              # [512, Hkv]
    heavy = m[0, :512].astype(bool)
    assert proj[heavy].mean() > 2.5 and abs(proj[~heavy].mean()) < 0.2


def test_bf16_is_nearest_even_of_fp64_draw():
    w = tkvsynth.CONFIGS["7b"].replace(layers=1, prefill=8, steps=0)
    bits = w.kv(1, 0, 8)                            # V: no planted shift, so it is the raw draw
    raw = tkvsynth.normals(w.seed, tkvsynth.TID_V, 0, bits.size)
    got = tkvsynth.bf16_to_f32(bits).ravel().astype(np.float64)
    b = got.astype(np.float32).view(np.uint32)
    up = (b + 0x10000).view(np.float32).astype(np.float64)
    dn = (b - 0x10000).view(np.float32).astype(np.float64)
    err = np.abs(raw - got)
    assert np.all(err <= np.abs(raw - up)) and np.all(err <= np.abs(raw - dn))
    assert np.all(err <= np.abs(got) * 2.0 ** -8)


def test_moments():
    g = tkvsynth.normals(11, 1, 0, 200000)
    assert abs(g.mean()) < 0.01 and abs(g.std() - 1) < 0.01
