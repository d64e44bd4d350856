"""GPU parity of the acceptance statistics: spec_accept_stats (alpha = sum_v min(p_j, q_j) =
1 - TV(p_j, q_j) with both log-normalisers) and spec_calibration_error, through the C ABI,
against the fp64 oracle on the same seeded inputs.  The drafted tokens are a seeded input (a
random prefix length and random tokens per request), not an output of either side.

Tolerances (fp32 kernels against fp64): the log-normalisers within 1e-4 absolute, the cycle's own
bar on log-probabilities (|exp(error) - 1| <= 1e-4 on every probability built from them; fp32 sums
of up to 1.5e5 terms merged per 256 columns, fp32 Markov bias from exact bf16 products); alpha
within 1e-4 absolute (each term min(p, q) carries the relative error of its log-normaliser); the
calibration error is fp64 on both sides and summed in a fixed order: 1e-12.  Every request of the
full-size workloads is compared."""
import numpy as np
import pytest

import oracle
from draft_sampling_lossless_spec_amd import workloads as wl
from gpu_util import to_device

pytestmark = pytest.mark.gpu


def seeded_draft(B, K, V, seed):
    rng = np.random.default_rng(seed)
    L = rng.integers(0, K + 1, B)
    d = rng.integers(0, V, (B, K)).astype(np.int32)
    d[np.arange(K)[None, :] >= L[:, None]] = -1
    return d


def gpu_stats(w, draft, x0=True, temp=None, path=0):
    import torch
    from draft_sampling_lossless_spec_amd import spec_accept_stats
    d = to_device(w)
    t = d["temp"] if temp is None else torch.from_numpy(temp.astype(np.float32)).cuda()
    out = spec_accept_stats(d["base"], d["target"], d["A"], d["W"], torch.from_numpy(draft).cuda(), t,
                            x0=d["x0"] if x0 else None, path=path)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}


def ref_stats(w, draft, x0=True, temp=None):
    return oracle.accept_stats_ref(w.base, w.target, w.A, w.W, w.x0 if x0 else None, draft,
                                   w.temp if temp is None else temp)


def assert_stats_match(o, g):
    for k in ("alpha", "lse_q", "lse_p"):
        assert np.array_equal(np.isnan(o[k]), np.isnan(g[k])), f"{k}: NaN pattern differs"
    m = ~np.isnan(o["alpha"])
    for k in ("lse_q", "lse_p"):
        err = np.abs(o[k][m] - g[k][m])
        assert err.max(initial=0.0) < 1e-4, f"{k}: max error {err.max():.3g}"
    err = np.abs(o["alpha"][m] - g["alpha"][m])
    assert err.max(initial=0.0) < 1e-4, f"alpha: max error {err.max():.3g}"
    print(f"rows {int(m.sum())}: max |alpha err| {err.max(initial=0.0):.2e}", flush=True)


SMALL = {
    "tiny_fp32": lambda: wl.generate("tiny"),
    "ragged_v333_bf16": lambda: wl.generate(wl.small_config(B=12, K=6, V=333, R=32, threshold=0.15)),
    "v20000_bf16": lambda: wl.generate(wl.small_config(B=40, K=5, V=20000, R=64, threshold=0.1)),
    "b300_many_row_blocks": lambda: wl.generate(wl.small_config(B=300, K=3, V=2048, R=16, threshold=0.05)),
    "fp32_v1001": lambda: wl.generate(wl.small_config(B=5, K=4, V=1001, R=8, dtype=wl.FP32, threshold=0.1)),
    "k1_b1_r256": lambda: wl.generate(wl.small_config(B=1, K=1, V=4096, R=256, threshold=0.1)),
    "temp06_k8": lambda: wl.generate(wl.small_config(B=16, K=8, V=5000, R=32, threshold=0.05, temp=0.6,
                                                      sigma=(1.5,))),
    # whole 64-column chunks in bf16: the W-resident kernel takes these (AUTO and forced), the
    # sweep kernels are run on them too
    "v20032_bf16": lambda: wl.generate(wl.small_config(B=40, K=5, V=20032, R=64, threshold=0.1)),
    "temp06_k8_v4992": lambda: wl.generate(wl.small_config(B=16, K=8, V=4992, R=32, threshold=0.05, temp=0.6,
                                                            sigma=(1.5,))),
    "k32_b9_v64": lambda: wl.generate(wl.small_config(B=9, K=32, V=64, R=16, threshold=0.01)),
}
# cases on which both statistics paths run (the W-resident kernel needs bf16 and whole chunks)
BOTH = ("b300_many_row_blocks", "k1_b1_r256", "v20032_bf16", "temp06_k8_v4992", "k32_b9_v64")


@pytest.mark.parametrize("case", sorted(SMALL))
def test_small_stats_match_oracle(case):
    print(f"stats {case}", flush=True)
    w = SMALL[case]()
    draft = seeded_draft(w.cfg.B, w.cfg.K, w.cfg.V, 7)
    o = ref_stats(w, draft)
    for path in ((0, 1, 2) if case in BOTH else (0,)):
        print(f"  path {path}", flush=True)
        assert_stats_match(o, gpu_stats(w, draft, path=path))


def test_stats_edge_cases():
    print("stats edge cases", flush=True)
    w = wl.generate(wl.small_config(B=6, K=4, V=1000, R=32, threshold=0.1))
    B, K, V = w.cfg.B, w.cfg.K, w.cfg.V
    draft = seeded_draft(B, K, V, 3)
    draft[0] = -1                       # nothing drafted
    draft[1] = [4, 5, 6, 7]             # the whole block drafted
    temp = w.temp.copy()
    temp[2] = 0.0                       # invalid temperature: every position NaN
    for x0 in (True, False):
        assert_stats_match(ref_stats(w, draft, x0=x0, temp=temp), gpu_stats(w, draft, x0=x0, temp=temp))
    # the same on whole 64-column chunks, both paths
    wc = wl.generate(wl.small_config(B=6, K=4, V=1024, R=32, threshold=0.1))
    tc = wc.temp.copy()
    tc[2] = 0.0
    for x0 in (True, False):
        oc = ref_stats(wc, draft, x0=x0, temp=tc)
        for path in (1, 2):
            assert_stats_match(oc, gpu_stats(wc, draft, x0=x0, temp=tc, path=path))
    # identical draft and target rows and no bias: alpha = 1
    w2 = wl.Workload(w.cfg, w.target[:, :K].copy(), w.target, np.zeros_like(w.A), np.zeros_like(w.W), w.x0, w.conf,
                     w.temp, w.threshold, w.seed, w.request_ids)
    g = gpu_stats(w2, draft)
    a = g["alpha"][~np.isnan(g["alpha"])]
    assert np.all(np.abs(a - 1.0) < 1e-4)
    wc2 = wl.Workload(wc.cfg, wc.target[:, :K].copy(), wc.target, np.zeros_like(wc.A), np.zeros_like(wc.W), wc.x0,
                      wc.conf, wc.temp, wc.threshold, wc.seed, wc.request_ids)
    g = gpu_stats(wc2, draft, path=2)
    a = g["alpha"][~np.isnan(g["alpha"])]
    assert np.all(np.abs(a - 1.0) < 1e-4)


@pytest.mark.parametrize("name", ["longblock", "dspark5"])
def test_full_size_stats(name):
    print(f"stats full {name}", flush=True)
    w = wl.generate(name)
    B, K, V = w.cfg.B, w.cfg.K, w.cfg.V
    draft = seeded_draft(B, K, V, 11)
    g = gpu_stats(w, draft)
    o = ref_stats(w, draft)
    assert_stats_match(o, g)
    if V % 64 == 0:
        assert_stats_match(o, gpu_stats(w, draft, path=1))   # the sweep kernels as well
    # every drafted position is finite and a probability
    m = draft >= 0
    assert np.isfinite(g["alpha"][m]).all() and np.isnan(g["alpha"][~m]).all()
    assert (g["alpha"][m] > 0).all() and (g["alpha"][m] <= 1 + 1e-4).all()


@pytest.mark.parametrize("nbins", [1, 10, 15])
def test_calibration_error_matches_oracle(nbins):
    import torch
    from draft_sampling_lossless_spec_amd import spec_calibration_error
    print(f"calibration nbins={nbins}", flush=True)
    rng = np.random.default_rng(nbins)
    B, K = 1024, 32
    conf = rng.beta(6, 2, (B, K)).astype(np.float32)
    L = rng.integers(0, K + 1, B).astype(np.int32)
    a = np.minimum(rng.integers(0, K + 1, B), L).astype(np.int32)
    a[:7] = -1                          # invalid requests are skipped
    want, n = oracle.calibration_error_ref(conf, L, a, nbins)
    e, gn = spec_calibration_error(torch.from_numpy(conf).cuda(), torch.from_numpy(L).cuda(),
                                   torch.from_numpy(a).cuda(), nbins)
    torch.cuda.synchronize()
    assert int(gn.item()) == n
    assert abs(float(e.item()) - want) < 1e-12
    # order-independent bin sums: bit-identical from run to run
    e2, _ = spec_calibration_error(torch.from_numpy(conf).cuda(), torch.from_numpy(L).cuda(),
                                   torch.from_numpy(a).cuda(), nbins)
    torch.cuda.synchronize()
    assert float(e2.item()) == float(e.item())
