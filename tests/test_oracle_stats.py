"""Pins of the oracle's acceptance statistics.

alpha_{b,j} = sum_v min(p_j, q_j) = 1 - TV(p_j, q_j) is the analytical acceptance rate of draft
position j ("The Speed Claim Nobody's Really Questioning", sections "The Semi-Autoregressive
Trick" and "The Real Innovation: Confidence-Scheduled Verification").  It is pinned to the
oracle's own rejection sampler by Monte Carlo (at position 0, and at position 1 given the drafted
token before it, which fixes which previous token the Markov bias uses), and to closed forms:
identical draft and target, a Markov bias that exactly closes the gap between them, disjoint
supports, a uniform draft against a one-peak target.  The calibration error is pinned to worked
values (tests/golden/calibration_cases.txt) and its extremes."""
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "calibration_cases.txt")


def _prefix_table(rows, V, K):
    """prefix table whose rows ignore the prefix: row of any prefix of length n = rows[n]"""
    n_rows = sum(V ** n for n in range(K + 1))
    table = np.empty((n_rows, V), np.float32)
    start = 0
    for n in range(K + 1):
        table[start:start + V ** n] = rows[n]
        start += V ** n
    return table


def _instance(seed, V=8, K=2, R=4, scale=0.8):
    rng = np.random.default_rng(seed)
    rows = (rng.standard_normal((K + 1, V)) * 1.3).astype(np.float32)
    base = (rows[:K] + rng.standard_normal((K, V)).astype(np.float32) * scale).astype(np.float32)
    A = (rng.standard_normal((V, R)) * 0.6).astype(np.float32)
    W = (rng.standard_normal((V, R)) * 0.6).astype(np.float32)
    return rows, base, A, W


def _alpha_at(rows, base, A, W, x0, draft, T):
    K, V = base.shape
    target = np.concatenate([rows[:K + 1]])[None]
    r = oracle.accept_stats_ref(base[None], target, A, W, np.array([x0], np.int32),
                                np.asarray(draft, np.int32)[None], np.array([T], np.float32))
    return r["alpha"][0]


def test_alpha_is_the_acceptance_rate_at_position_zero():
    rows, base, A, W = _instance(11)
    K, V = base.shape
    x0, T = 3, 0.9
    alpha0 = _alpha_at(rows, base, A, W, x0, [0, 0], T)[0]
    n = 200_000
    r = oracle.spec_cycle_ref_mc(base, _prefix_table(rows, V, K), A, W, x0, np.ones(K, np.float32), T, 0.5,
                                 seed=21, n_trials=n, noise=oracle.CHUNKED)
    rate = (r["accepted_len"] >= 1).mean()
    assert abs(rate - alpha0) < 4 * math.sqrt(alpha0 * (1 - alpha0) / n)


def test_alpha_at_position_one_uses_the_previous_draft_token():
    rows, base, A, W = _instance(12)
    K, V = base.shape
    x0, T = 5, 1.0
    n = 400_000
    r = oracle.spec_cycle_ref_mc(base, _prefix_table(rows, V, K), A, W, x0, np.ones(K, np.float32), T, 0.5,
                                 seed=22, n_trials=n, noise=oracle.FLAT)
    reached = r["accepted_len"] >= 1                  # position 1 is tested
    x_first = r["draft_tokens"][:, 0]
    checked = 0
    for v in range(V):
        sel = reached & (x_first == v)
        m = int(sel.sum())
        if m < 20_000:
            continue
        alpha1 = _alpha_at(rows, base, A, W, x0, [v, v], T)[1]   # prev of position 1 = v
        rate = (r["accepted_len"][sel] >= 2).mean()
        assert abs(rate - alpha1) < 4 * math.sqrt(alpha1 * (1 - alpha1) / m), v
        checked += 1
    assert checked >= 2


def test_alpha_is_one_for_identical_draft_and_target():
    rng = np.random.default_rng(4)
    B, K, V, R = 2, 3, 40, 8
    target = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    base = target[:, :K].copy()
    A = np.zeros((V, R), np.float32)
    W = np.zeros((V, R), np.float32)
    draft = rng.integers(0, V, (B, K)).astype(np.int32)
    r = oracle.accept_stats_ref(base, target, A, W, np.array([1, 2], np.int32), draft, np.array([0.7, 1.3], np.float32))
    assert np.all(np.abs(r["alpha"] - 1.0) < 1e-12)


def test_alpha_is_one_when_the_bias_closes_the_gap():
    # target row j = base row j + A[prev_j] . W exactly (fp64, then fp32): only the right previous
    # token (x0 at j = 0, the draft token at j - 1 after that) makes q equal p
    rng = np.random.default_rng(6)
    K, V, R = 3, 50, 8
    base = rng.standard_normal((1, K, V)).astype(np.float32)
    A = (rng.standard_normal((V, R)) * 0.5).astype(np.float32)
    W = (rng.standard_normal((V, R)) * 0.5).astype(np.float32)
    x0 = 7
    draft = np.array([[11, 23, 31]], np.int32)
    prevs = [x0, 11, 23]
    target = np.zeros((1, K + 1, V), np.float32)
    for j, pv in enumerate(prevs):
        bias = [math.fsum(float(A[pv, r]) * float(W[v, r]) for r in range(R)) for v in range(V)]
        target[0, j] = (base[0, j].astype(np.float64) + np.array(bias)).astype(np.float32)
    r = oracle.accept_stats_ref(base, target, A, W, np.array([x0], np.int32), draft, np.array([1.0], np.float32))
    assert np.all(np.abs(r["alpha"][0] - 1.0) < 1e-5)
    # position j reads the draft token of j - 1: changing one draft token moves only the next position
    for changed, draft2 in ((1, [[12, 23, 31]]), (2, [[11, 40, 31]])):
        r2 = oracle.accept_stats_ref(base, target, A, W, np.array([x0], np.int32), np.array(draft2, np.int32),
                                     np.array([1.0], np.float32))
        for j in range(K):
            if j == changed:
                assert r2["alpha"][0, j] < 0.999
            else:
                assert abs(r2["alpha"][0, j] - 1.0) < 1e-5


def test_alpha_is_zero_for_disjoint_supports():
    K, V, R = 2, 16, 4
    base = np.zeros((1, K, V), np.float32)
    target = np.zeros((1, K + 1, V), np.float32)
    base[:, :, V // 2:] = -np.inf
    target[:, :, :V // 2] = -np.inf
    A = np.zeros((V, R), np.float32)
    W = np.zeros((V, R), np.float32)
    r = oracle.accept_stats_ref(base, target, A, W, None, np.array([[1, 2]], np.int32), np.array([1.0], np.float32))
    assert np.all(r["alpha"] == 0.0)


@pytest.mark.parametrize("M,T", [(3.0, 1.0), (6.0, 0.6), (1.0, 2.0)])
def test_alpha_closed_form_uniform_draft_against_one_peak(M, T):
    # q uniform, p = e^{M/T} on one token and 1 elsewhere (normalised): as long as that token
    # holds more than 1/V, alpha = 1/V + (V - 1) / (e^{M/T} + V - 1)
    K, V, R = 1, 64, 4
    base = np.zeros((1, K, V), np.float32)
    target = np.zeros((1, K + 1, V), np.float32)
    target[0, :, 17] = M
    A = np.zeros((V, R), np.float32)
    W = np.zeros((V, R), np.float32)
    r = oracle.accept_stats_ref(base, target, A, W, None, np.array([[0]], np.int32), np.array([T], np.float32))
    e = math.exp(M / float(np.float32(T)))   # the temperature reaches the oracle as fp32
    assert abs(r["alpha"][0, 0] - (1 / V + (V - 1) / (e + V - 1))) < 1e-13


def test_alpha_is_nan_off_the_drafted_positions_and_for_bad_requests():
    rows, base, A, W = _instance(13, K=3)
    target = np.concatenate([rows])[None].repeat(3, axis=0)
    base3 = base[None].repeat(3, axis=0)
    draft = np.array([[1, 2, -1], [3, -1, -1], [1, 1, 1]], np.int32)
    temp = np.array([1.0, 0.8, -1.0], np.float32)
    r = oracle.accept_stats_ref(base3, target, A, W, np.array([0, 1, 2], np.int32), draft, temp)
    a = r["alpha"]
    assert np.isfinite(a[0, :2]).all() and np.isnan(a[0, 2])
    assert np.isfinite(a[1, 0]) and np.isnan(a[1, 1:]).all()
    assert np.isnan(a[2]).all()
    assert ((a[np.isfinite(a)] > 0) & (a[np.isfinite(a)] <= 1 + 1e-12)).all()


def _golden_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        head, conf, L, a, ece, n = [f.split() for f in line.split("|")]
        B, K = int(head[0]), int(head[1])
        cases.append((np.array(conf, np.float32).reshape(B, K), np.array(L, np.int32), np.array(a, np.int32),
                      float(ece[0]), int(n[0])))
    return cases


@pytest.mark.parametrize("case", range(2))
def test_calibration_error_worked_cases(case):
    conf, L, a, ece, n = _golden_cases()[case]
    got, got_n = oracle.calibration_error_ref(conf, L, a, nbins=10)
    assert got_n == n
    assert abs(got - ece) < 1e-6


def test_calibration_error_extremes():
    B, K = 4, 5
    conf = np.ones((B, K), np.float32)
    L = np.full(B, K, np.int32)
    # confident and always right: 0; confident and always wrong: 1; no pair: 0
    assert oracle.calibration_error_ref(conf, L, np.full(B, K, np.int32))[0] == 0.0
    assert oracle.calibration_error_ref(conf, L, np.zeros(B, np.int32))[0] == 1.0
    assert oracle.calibration_error_ref(conf, np.zeros(B, np.int32), np.zeros(B, np.int32)) == (0.0, 0)
