"""Host checks of the GPU-vs-oracle comparison helpers."""
import numpy as np

from tests import parity


def test_close_applies_both_bounds():
    want = np.linspace(-1.0, 1.0, 1000)
    ok, mx, rel, _ = parity.close(want + 1e-3, want)
    assert ok and abs(mx - 1e-3) < 1e-12
    ok, _, rel, _ = parity.close(want * 1.015, want)     # max-abs 1.5e-2 but rel-L2 1.5e-2
    assert not ok and rel > 1e-2
    ok, mx, _, _ = parity.close(want + 3e-2, want)       # max-abs too large
    assert not ok and mx > 2e-2


def test_close_rejects_a_zero_output_below_the_absolute_tolerance():
    # a reference slice of size ~1e-2 (inside the max-abs bound everywhere): an all-zero
    # output meets max-abs 2e-2 but must fail on relative L2
    want = np.random.default_rng(0).uniform(-1e-2, 1e-2, 4096)
    ok, mx, rel, _ = parity.close(np.zeros_like(want), want)
    assert mx <= 2e-2 and rel == 1.0 and not ok
    ok, _, _, _ = parity.close(want * 1.005, want)     # 0.5 % relative error passes
    assert ok
    want = np.full(64, 5e-6)                            # above the vacuity level
    assert not parity.close(np.zeros_like(want), want)[0]


def test_close_rejects_non_finite_output():
    want = np.linspace(-1.0, 1.0, 64)
    got = want.copy()
    got[3] = np.nan
    assert not parity.close(got, want)[0]


def test_close_vanishing_reference_uses_max_abs_only():
    want = np.full(512, 1e-22)                           # a gradient that is zero in effect
    ok, _, rel, _ = parity.close(want + 1e-4, want)
    assert ok and rel > 1e10
    ok, _, _, _ = parity.close(want + 3e-2, want)
    assert not ok


def test_mask_rows_exemption_band():
    # one row of 4 blocks; the GPU keeps block 2 instead of block 1, whose probabilities
    # differ by less than the band around the threshold
    probs = np.array([0.5, 0.2500000004, 0.2499999998, 0.0], dtype=np.float64)
    order = np.array([0, 1, 2, 3])
    row = {"order": order, "sorted": probs[order], "tau": probs[1], "keep": np.array([0, 1]),
           "Lp": 2, "Lk": 1, "cum": np.cumsum(probs[order]), "L": 2}
    gpu_idx = np.array([[[[0, 2, -1, -1]]]], dtype=np.int32)
    gpu_cnt = np.array([[[2]]], dtype=np.int32)
    n, exempt, fails = parity.compare_mask_rows(gpu_idx, gpu_cnt, {(0, 0): [row]}, 0.75)
    assert n == 1 and not fails and len(exempt) == 1
    gpu_idx = np.array([[[[0, 3, -1, -1]]]], dtype=np.int32)   # block 3 is far from tau
    n, exempt, fails = parity.compare_mask_rows(gpu_idx, gpu_cnt, {(0, 0): [row]}, 0.75)
    assert fails
