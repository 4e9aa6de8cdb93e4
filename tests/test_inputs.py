"""The seeded input generators draw what the workload recipe states.

Checked on the CPU on samples: determinism per (workload, call, rank); the
N(0,1) moments; the outlier rate of the single-call workload; the two-sided
5% quantiles of Student-t with 4 and 3 degrees of freedom; the spread of the
per-channel lognormal(0, 0.5) scales, shared by all ranks of a call.
"""
import math

import numpy as np
import pytest
import torch

from error_compensated_bit_amd.inputs import WORKLOADS, Workload, draw, make_x

N = 1 << 18


def test_deterministic_and_distinct():
    w = WORKLOADS["chain56_p4_512x1024"]
    a = make_x(w, 3, 1)
    assert torch.equal(a, make_x(w, 3, 1))
    assert not torch.equal(a, make_x(w, 3, 2))
    assert not torch.equal(a, make_x(w, 4, 1))
    assert a.dtype == torch.bfloat16 and a.numel() == w.n


def test_normal_moments():
    x = draw("normal", (N,), "cpu", 9, 0, 0).double().numpy()
    assert abs(x.mean()) < 5 / math.sqrt(N)
    assert abs(x.var() - 1.0) < 0.02


def test_outlier_rate():
    """N(0,1), each element scaled by 20 with probability 1e-3: |x| > 6
    happens for about 1e-3 * P(|z| > 0.3) = 7.6e-4 of the elements (the
    unscaled tail adds 2e-9)."""
    x = draw("normal_outliers", (N,), "cpu", 9, 0, 1).numpy()
    expected = N * 1e-3 * 0.7642
    count = int(np.count_nonzero(np.abs(x) > 6.0))
    assert abs(count - expected) < 5 * math.sqrt(expected)


@pytest.mark.parametrize("dist,q975", [("t4", 2.7764451), ("t3", 3.1824463)])
def test_student_t_quantiles(dist, q975):
    """Two-sided 5% points of Student-t with 4 and 3 degrees of freedom."""
    x = draw(dist, (N,), "cpu", 9, 0, 2).numpy()
    frac = np.mean(np.abs(x) > q975)
    assert abs(frac - 0.05) < 5 * math.sqrt(0.05 * 0.95 / N)


def test_channel_scales_are_lognormal_and_shared():
    """x = t4 * exp(0.5 Z_c): the log of each channel's median |x| spreads
    with standard deviation about 0.5 across channels, and every rank of a
    call uses the same channel vector."""
    w = Workload("probe", 8, 2, (512, 1024), "t4_chan", 1)
    xs = [draw(w.dist, w.shape, "cpu", w.wid, 0, p).numpy() for p in range(2)]
    logs = [np.log(np.median(np.abs(x), axis=0)) for x in xs]
    for lg in logs:
        assert 0.42 < lg.std() < 0.58
    assert np.corrcoef(logs[0], logs[1])[0, 1] > 0.9
