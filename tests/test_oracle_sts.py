"""Pins of the oracle's sequential temperature scaling (definition in oracle/spec_oracle.c):
exactly calibrated data keeps T = 1, scaling every logit by 2 doubles every fitted temperature
(one octave of the grid), an overconfident head is recovered by Monte Carlo, the fit runs left to
right (a later position's data never moves an earlier temperature), and the fitted calibration
error never exceeds the uncalibrated one at position 0."""
import math

import numpy as np
import pytest

import oracle


def _calibrated_data():
    # position 0: sigmoid(log 3) = 0.75 and exactly 3/4 of the sequences pass it; position 1:
    # sigmoid(log 2) = 2/3, so the prefix probability is 1/2 and exactly half of all sequences pass both
    N, K = 400, 2
    z = np.empty((N, K), np.float32)
    z[:, 0] = math.log(3.0)
    z[:, 1] = math.log(2.0)
    a = np.zeros(N, np.int32)
    a[:300] = 1
    a[:200] = 2
    return z, np.full(N, K, np.int32), a


def test_exactly_calibrated_data_keeps_unit_temperature():
    z, L, a = _calibrated_data()
    grid = oracle.temperature_grid()
    r = oracle.temperature_scaling_ref(z, L, a, grid)
    assert np.all(r["T"] == 1.0)
    assert np.all(r["ece_after"] < 1e-6) and np.all(r["ece_before"] < 1e-6)


def _overconfident(seed, N=20000, K=4, scale=2.5):
    rng = np.random.default_rng(seed)
    zt = rng.normal(1.5, 1.0, (N, K))
    surv = rng.random((N, K)) < 1 / (1 + np.exp(-zt))
    a = np.where(surv.all(axis=1), K, surv.argmin(axis=1)).astype(np.int32)   # first failure
    return (scale * zt).astype(np.float32), np.full(N, K, np.int32), a


def test_overconfident_head_is_recovered():
    z, L, a = _overconfident(1)
    grid = oracle.temperature_grid()
    r = oracle.temperature_scaling_ref(z, L, a, grid)
    assert np.all(np.abs(np.log2(r["T"]) - math.log2(2.5)) < 0.3), r["T"]
    assert np.all(r["ece_after"] < r["ece_before"])


def test_doubling_the_logits_doubles_every_temperature():
    z, L, a = _overconfident(2, N=6000, K=3, scale=1.7)
    grid = oracle.temperature_grid()
    r1 = oracle.temperature_scaling_ref(z, L, a, grid)
    r2 = oracle.temperature_scaling_ref(2 * z, L, a, grid)
    assert np.array_equal(r2["T"], 2 * r1["T"])
    assert np.allclose(r2["ece_after"], r1["ece_after"], rtol=0, atol=1e-12)


def test_fit_runs_left_to_right():
    z, L, a = _overconfident(3, N=5000, K=4)
    grid = oracle.temperature_grid()
    r1 = oracle.temperature_scaling_ref(z, L, a, grid)
    z2 = z.copy()
    z2[:, 2:] = -z2[:, 2:]                  # later positions changed
    r2 = oracle.temperature_scaling_ref(z2, L, a, grid)
    assert np.array_equal(r1["T"][:2], r2["T"][:2])


def test_unverified_positions_and_invalid_sequences_carry_no_pair():
    z, L, a = _calibrated_data()
    grid = oracle.temperature_grid()
    L2 = L.copy()
    L2[::2] = 0                              # half the sequences verify nothing
    a2 = np.where(L2 == 0, 0, a).astype(np.int32)
    a2[1] = -1                               # an invalid sequence
    r = oracle.temperature_scaling_ref(z, L2, a2, grid)
    assert np.all(np.isfinite(r["T"]))
    # position 0 with unit temperature against the outcomes of the sequences that verify it
    keep = (L2 > 0) & (a2 >= 0)
    P = 1 / (1 + np.exp(-z[keep, 0].astype(np.float64)))
    e = abs(P.mean() - (a2[keep] >= 1).mean())   # all predictions share one bin
    assert abs(r["ece_before"][0] - e) < 1e-12
