"""Pins for the oracle's primitives: counter hash, uniforms, Gumbel noise, log-sum-exp, Markov
bias and prefix cut -- each checked against something other than the oracle itself (published
values, closed forms, exact summation, independent library routines, worked cases)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_splitmix64_published_outputs():
    want = [int(x, 16) for x in _golden_lines("splitmix64_state0.txt")]
    assert oracle.splitmix64_outputs(0, 3) == want


def test_bits32_is_the_splitmix64_sequence_from_the_row_key():
    # index i uses the (i//2 + 1)-th output of a generator started at the row key:
    # high half for even i, low half for odd i
    for key in (0, 1, 0xDEADBEEFCAFEBABE, oracle.rowkey(7, 3, 2, 1)):
        seq = oracle.splitmix64_outputs(key, 6)
        for i in range(12):
            w = seq[i // 2]
            want = (w >> 32) if i % 2 == 0 else (w & 0xFFFFFFFF)
            assert oracle.bits32(key, i) == want


def test_rowkey_chains_first_outputs():
    # rowkey = first(first(first(first(seed) ^ request) ^ pos) ^ stream), first(x) = first
    # SplitMix64 output from state x (pinned above)
    def first(x):
        return oracle.splitmix64_outputs(x & (2**64 - 1), 1)[0]
    for seed, req, pos, st in [(1, 0, 0, 1), (123456789, 255, 15, 4), (2**63 + 5, 2**40, 3, 8)]:
        k = first(first(first(first(seed) ^ req) ^ pos) ^ st)
        assert oracle.rowkey(seed, req, pos, st) == k
    # a negative global request id is taken modulo 2^64
    assert oracle.rowkey(1, -1, 0, 1) == first(first(first(first(1) ^ (2**64 - 1)) ^ 0) ^ 1)


def test_uniform_exact_grid_and_uniformity():
    key = oracle.rowkey(11, 5, 2, 1)
    n = 200_000
    u = np.array([oracle.uniform(key, i) for i in range(n)])
    # U = (bits + 1/2) 2^-32 exactly
    grid = u * 2.0**32 - 0.5
    assert np.all(grid == np.round(grid))
    assert u.min() > 0.0 and u.max() < 1.0
    # equiprobable bins
    counts, _ = np.histogram(u, bins=64, range=(0, 1))
    assert stats.chisquare(counts).pvalue > 1e-4
    # adjacent indices (halves of one 64-bit word) are uncorrelated
    assert abs(np.corrcoef(u[0::2], u[1::2])[0, 1]) < 0.02


def test_gumbel_distribution_closed_form():
    key = oracle.rowkey(3, 1, 0, 4)
    n = 200_000
    g = np.array([oracle.gumbel(key, i) for i in range(n)])
    # standard Gumbel: CDF exp(-exp(-g)), mean = Euler-Mascheroni, variance pi^2/6
    assert stats.kstest(g, lambda x: np.exp(-np.exp(-x))).pvalue > 1e-4
    assert abs(g.mean() - 0.5772156649) < 4 * math.sqrt(math.pi**2 / 6 / n)
    assert abs(g.var() - math.pi**2 / 6) < 0.03
    # the largest noise value a 32-bit uniform can give: U = 2^-33 -> G = -log(-log1p(-2^-33))
    assert g.max() < 33 * math.log(2)


def test_gumbel_clz_bound():
    # G(v) <= (clz32(bits) + 1) ln 2: U >= 2^(31 - clz) 2^-32 and -log1p(-U) >= U
    key = oracle.rowkey(9, 9, 9, 1)
    for i in range(20_000):
        b = oracle.bits32(key, i)
        clz = 32 - b.bit_length()
        assert oracle.gumbel(key, i) <= (clz + 1) * math.log(2) + 1e-12


def test_lse_closed_forms_and_exact_sum():
    assert oracle.lse(np.zeros(7)) == pytest.approx(math.log(7), abs=1e-15)
    assert oracle.lse(np.array([0.0, math.log(3.0)])) == pytest.approx(math.log(4.0), abs=1e-15)
    assert oracle.lse(np.array([2.5, -np.inf])) == 2.5
    assert oracle.lse(np.array([-np.inf, -np.inf])) == -np.inf
    assert math.isnan(oracle.lse(np.array([1.0, np.nan])))
    assert oracle.lse(np.array([1.0, np.inf])) == np.inf
    rng = np.random.default_rng(5)
    for n in (2, 64, 1000, 151936):
        x = rng.standard_normal(n) * 3 + 8 * (rng.random(n) < 0.01)
        m = x.max()
        exact = m + math.log(math.fsum(math.exp(v - m) for v in x))   # exactly rounded sum
        assert abs(oracle.lse(x) - exact) <= 1e-13 * max(1.0, abs(exact))
        # shift invariance
        assert oracle.lse(x + 100.0) == pytest.approx(exact + 100.0, abs=1e-12)


def test_bias_matches_independent_matmul_and_special_cases():
    from draft_sampling_lossless_spec_amd.workloads import to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(2)
    V, R = 333, 32
    A32 = (rng.standard_normal((V, R)) * 0.05).astype(np.float32)
    W32 = (rng.standard_normal((V, R)) * 0.05).astype(np.float32)
    for prev in (0, 17, V - 1):
        want = W32.astype(np.float64) @ A32[prev].astype(np.float64)
        got = oracle.bias(A32, W32, prev)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)
    Ab, Wb = to_bf16_bits(A32), to_bf16_bits(W32)
    want = bf16_bits_to_f32(Wb).astype(np.float64) @ bf16_bits_to_f32(Ab)[17].astype(np.float64)
    np.testing.assert_allclose(oracle.bias(Ab, Wb, 17), want, rtol=0, atol=1e-15)
    # each product of two bf16 values is exact in fp64: compare with an exact rational sum
    a = bf16_bits_to_f32(Ab)[17].astype(np.float64)
    for v in (0, 100, V - 1):
        w = bf16_bits_to_f32(Wb)[v].astype(np.float64)
        exact = float(sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a, w)))
        assert abs(oracle.bias(Ab, Wb, 17)[v] - exact) <= 4e-16 * max(1e-300, abs(exact)) + 1e-20
    # no previous token -> zero bias; one-hot factors -> a single entry
    assert np.all(oracle.bias(A32, W32, -1) == 0.0)
    A1 = np.zeros((V, R), np.float32)
    W1 = np.zeros((V, R), np.float32)
    A1[5, 3] = 2.0
    W1[40, 3] = 1.5
    b = oracle.bias(A1, W1, 5)
    assert b[40] == 3.0 and np.count_nonzero(b) == 1


def test_cut_worked_cases():
    for line in _golden_lines("cut_cases.txt"):
        thr, confs, want = [p.strip() for p in line.split("|")]
        c = np.array([float(x) for x in confs.split()], dtype=np.float32)
        assert oracle.cut(c, float(thr)) == int(want), line


def test_cut_brute_force_against_exact_rationals():
    rng = np.random.default_rng(17)
    checked = 0
    for _ in range(3000):
        K = int(rng.integers(1, 17))
        c = rng.beta(3, 1.2, size=K).astype(np.float32)
        if rng.random() < 0.2:
            c[rng.integers(K)] = np.float32(rng.uniform(1.0, 3.0))   # non-monotone products
        thr = np.float32(rng.uniform(0.0, 0.9))
        P = Fraction(1)
        L = 0
        near = False
        for j in range(K):
            P *= Fraction(float(c[j]))
            if abs(float(P) - float(thr)) < 1e-12:
                near = True
            if not P >= Fraction(float(thr)):
                break
            L = j + 1
        if near:
            continue
        assert oracle.cut(c, float(thr)) == L
        checked += 1
    assert checked > 2500
