"""Seeded input generator and the tolerance metric (no GPU)."""

import numpy as np

from metrics import bf16_excess_over_rms, half_ulp_bf16, max_abs_over_rms
from workloads import synth


def test_bf16_round_is_round_to_nearest_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 3.0e-3, 1 + 2 ** -8 + 2 ** -20], np.float32)
    y = synth.bf16_round(x.copy())
    np.testing.assert_array_equal(y, np.array([1.0, 1.0, 1 + 2 ** -6, -2.5, y[4], 1 + 2 ** -7], np.float32))
    assert np.all(y.view(np.uint32) & 0xFFFF == 0)
    rng = np.random.default_rng(0)
    z = (rng.standard_normal(100000) * 10).astype(np.float32)
    zr = synth.bf16_round(z.copy())
    assert np.all(np.abs(zr.astype(np.float64) - z) <= half_ulp_bf16(z) * (1 + 1e-12))


def test_generator_is_deterministic_and_thread_independent():
    a = synth.block_workload(T=40, d=64, N=3, S=3, H=1, rep_std_step=0.3, dtype="bf16", seed=4, with_dh=True)
    b = synth.block_workload(T=40, d=64, N=3, S=3, H=1, rep_std_step=0.3, dtype="bf16", seed=4, with_dh=True)
    for x, y in ((a.reps, b.reps), (a.partials, b.partials), (a.w, b.w), (a.gain, b.gain), (a.dh, b.dh)):
        np.testing.assert_array_equal(x, y)
    c = synth.block_workload(T=40, d=64, N=3, S=3, H=1, rep_std_step=0.3, dtype="bf16", seed=5)
    assert not np.array_equal(a.reps, c.reps)


def test_generator_distributions():
    wl = synth.block_workload(T=512, d=1024, N=8, S=4, H=1, rep_std_step=0.3, dtype="bf16", seed=0)
    for n in range(8):
        assert abs(wl.reps[n].std() / (1 + 0.3 * n) - 1) < 0.01
    # partials are running sums of unit-variance outputs
    for k in range(3):
        assert abs(wl.partials[k].std() / np.sqrt(k + 1) - 1) < 0.01
    assert abs(wl.w.std() * np.sqrt(1024) - 1) < 0.02
    assert abs((wl.gain - 1).std() / np.sqrt(0.02) - 1) < 0.03
    assert wl.w.dtype == np.float32 and np.any(wl.w.view(np.uint32) & 0xFFFF)  # parameters not rounded


def test_sample_tokens():
    idx = synth.sample_tokens(1000, 50)
    assert idx[0] == 0 and idx[-1] == 999 and len(idx) == 50 and np.all(np.diff(idx) > 0)
    assert np.array_equal(synth.sample_tokens(10, 50), np.arange(10))


def test_excess_metric():
    ref = np.array([4.0, -1.0, 0.25, 0.0])
    # a correctly rounded value has no excess; one ulp off at 4.0 leaves half an ulp
    assert bf16_excess_over_rms(ref + np.array([2 ** -6, 0, 0, 0]), ref) == 0.0
    e = bf16_excess_over_rms(ref + np.array([2 ** -5, 0, 0, 0]), ref)
    assert abs(e - 2 ** -6 / np.sqrt(np.mean(ref ** 2))) < 1e-15
    assert max_abs_over_rms(ref, ref) == 0.0
