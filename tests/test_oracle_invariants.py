"""Invariants, determinism, sharding invariance and per-request error handling of the oracle on
the synthetic workloads (tiny config and a reduced ragged-vocabulary config)."""
import numpy as np
import pytest

import oracle
from draft_sampling_lossless_spec_amd import workloads as wl


def run(w, noise, request_offset=0, **kw):
    return oracle.spec_cycle_ref(w.base, w.target, w.A, w.W, w.x0, w.conf, w.temp, w.threshold, w.seed,
                                 noise=noise, request_offset=request_offset, **kw)


def check_invariants(w, r):
    B, K = w.conf.shape
    for b in range(B):
        L, a = r["verify_len"][b], r["accepted_len"][b]
        assert L == oracle.cut(w.conf[b], w.threshold)
        assert 0 <= a <= L
        assert np.all(r["tokens"][b, :a] == r["draft_tokens"][b, :a])
        assert 0 <= r["tokens"][b, a] < w.cfg.V
        assert np.all(r["tokens"][b, a + 1:] == -1)
        assert np.all(r["draft_tokens"][b, :L] >= 0) and np.all(r["draft_tokens"][b, L:] == -1)
        assert np.all(np.isfinite(r["logq"][b, :L])) and np.all(np.isnan(r["logq"][b, L:]))
        assert np.all(r["logq"][b, :L] <= 0)
        dec = min(a + 1, L)
        assert np.all(np.isfinite(r["logp"][b, :dec])) and np.all(np.isnan(r["logp"][b, dec:]))
        assert r["final_kind"][b] == (1 if a == L else r["final_kind"][b])
        if a < L:
            assert r["final_kind"][b] in (0, 2)
            assert not (r["u"][b, a] < r["ratio"][b, a])
        for j in range(a):
            assert r["u"][b, j] < r["ratio"][b, j]


@pytest.mark.parametrize("noise", [oracle.FLAT, oracle.CHUNKED])
def test_tiny_config_invariants(noise):
    w = wl.generate("tiny")
    r = run(w, noise)
    check_invariants(w, r)


@pytest.mark.parametrize("noise", [oracle.FLAT, oracle.CHUNKED])
def test_small_ragged_config_invariants_determinism_sharding(noise):
    cfg = wl.small_config(B=12, K=6, V=333, R=32, threshold=0.15)
    w = wl.generate(cfg)
    r1 = run(w, noise, nthreads=4)
    r2 = run(w, noise, nthreads=1)
    check_invariants(w, r1)
    for k in ("tokens", "accepted_len", "draft_tokens"):
        assert np.array_equal(r1[k], r2[k])
    np.testing.assert_array_equal(r1["logq"], r2["logq"])
    # sharding: the second half run on its own with request_offset = 6 reproduces the full run
    h = 6
    half = wl.Workload(w.cfg, w.base[h:], w.target[h:], w.A, w.W, w.x0[h:], w.conf[h:], w.temp[h:],
                       w.threshold, w.seed, w.request_ids[h:])
    r3 = run(half, noise, request_offset=h)
    for k in ("tokens", "accepted_len", "draft_tokens"):
        assert np.array_equal(r1[k][h:], r3[k])
    # a different seed changes the draws
    w2 = wl.Workload(w.cfg, w.base, w.target, w.A, w.W, w.x0, w.conf, w.temp, w.threshold, w.seed + 1,
                     w.request_ids)
    assert not np.array_equal(run(w2, noise)["draft_tokens"], r1["draft_tokens"])


def test_noise_schemes_agree_on_cut_and_differ_on_draws():
    cfg = wl.small_config(B=8, K=5, V=700, R=16)
    w = wl.generate(cfg)
    rf, rc = run(w, oracle.FLAT), run(w, oracle.CHUNKED)
    assert np.array_equal(rf["verify_len"], rc["verify_len"])
    assert not np.array_equal(rf["draft_tokens"], rc["draft_tokens"])
    # first-position q does not depend on the sampler's noise: logq of the same token agrees
    np.testing.assert_array_equal(rf["lse_q"][:, 0], rc["lse_q"][:, 0])


def test_invalid_requests_are_marked():
    cfg = wl.small_config(B=6, K=3, V=100, R=16, dtype=wl.FP32)
    w = wl.generate(cfg)
    w.temp[0] = 0.0
    w.temp[1] = np.nan
    w.x0[2] = cfg.V
    w.target[3, 0, 5] = np.nan
    w.conf[3] = 1.0
    w.base[4, 0, :] = -np.inf
    w.conf[4] = 1.0
    r = run(w, oracle.CHUNKED)
    for b in range(5):
        assert r["accepted_len"][b] == -1, b
        assert np.all(r["tokens"][b] == -1)
        assert r["final_kind"][b] == -1
    assert r["accepted_len"][5] >= 0
    # x0 = -1 means "no previous token": valid
    w.x0[5] = -1
    r = run(w, oracle.CHUNKED)
    assert r["accepted_len"][5] >= 0
    # a NaN threshold verifies nothing: one bonus token per request
    w2 = wl.generate(cfg)
    w2.threshold = float("nan")
    r = run(w2, oracle.FLAT)
    assert np.all(r["verify_len"] == 0) and np.all(r["accepted_len"] == 0) and np.all(r["final_kind"] == 1)


def test_bad_arguments_are_rejected():
    w = wl.generate(wl.small_config(B=2, K=2, V=50, R=8, dtype=wl.FP32))
    with pytest.raises(TypeError):
        oracle.spec_cycle_ref(w.base.astype(np.float64), w.target, w.A, w.W, w.x0, w.conf, w.temp, 0.2, 1)
    with pytest.raises(ValueError):
        oracle.spec_cycle_ref(w.base, w.target, w.A, w.W, w.x0, w.conf, w.temp, 0.2, 1, noise=3)
