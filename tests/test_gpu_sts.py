"""GPU parity of sequential temperature scaling (spec_temperature_scaling through the C ABI)
against the oracle on seeded held-out data.  Both sides evaluate the calibration errors in fp64
(order-independent bin sums on the GPU, bit-identical from run to run; the oracle sums in order;
the last bit of exp may differ), so the fitted temperatures must be equal and the errors agree to
1e-12."""
import math

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def held_out(seed, N, K, scale, mu=1.5):
    rng = np.random.default_rng(seed)
    zt = rng.normal(mu, 1.0, (N, K))
    surv = rng.random((N, K)) < 1 / (1 + np.exp(-zt))
    a = np.where(surv.all(axis=1), K, surv.argmin(axis=1)).astype(np.int32)
    L = rng.integers(1, K + 1, N).astype(np.int32)     # verified lengths vary
    a = np.minimum(a, L).astype(np.int32)
    a[:5] = -1                                         # left-out sequences
    return (scale * zt).astype(np.float32), L, a


def gpu_sts(z, L, a, grid, nbins):
    import torch
    from draft_sampling_lossless_spec_amd import spec_temperature_scaling
    c = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    out = spec_temperature_scaling(c(z), c(L), c(a), c(grid), nbins)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


CASES = [
    ("overconfident", 1, 20000, 4, 2.5, 10),
    ("underconfident", 2, 20000, 6, 0.5, 15),
    ("long_head", 3, 50000, 16, 1.8, 10),
    ("small", 4, 300, 3, 1.2, 5),
]


@pytest.mark.parametrize("name,seed,N,K,scale,nbins", CASES)
def test_sts_matches_oracle(name, seed, N, K, scale, nbins):
    print(f"sts {name} N={N} K={K}", flush=True)
    z, L, a = held_out(seed, N, K, scale)
    grid = oracle.temperature_grid()
    o = oracle.temperature_scaling_ref(z, L, a, grid, nbins)
    g = gpu_sts(z, L, a, grid, nbins)
    assert np.array_equal(g["T"], o["T"]), (g["T"], o["T"])
    for k in ("ece_before", "ece_after"):
        assert np.max(np.abs(g[k] - o[k])) < 1e-12, k
    g2 = gpu_sts(z, L, a, grid, nbins)
    for k in g:
        assert np.array_equal(g[k], g2[k]), f"{k} differs between runs"
    print(f"  T={np.round(g['T'], 3)} ece {o['ece_before'].mean():.4f} -> {o['ece_after'].mean():.4f}", flush=True)


def test_sts_recovers_overconfidence_on_gpu():
    z, L, a = held_out(7, 40000, 5, 2.0)
    g = gpu_sts(z, L, a, oracle.temperature_grid(), 10)
    assert np.all(np.abs(np.log2(g["T"]) - 1.0) < 0.3), g["T"]
