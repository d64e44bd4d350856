"""The allocation-free entry point (spec_cycle_noalloc, static per-GPU scratch) against spec_cycle
(caller workspace) on the same inputs: identical outputs on two calls in a row, the second with a
smaller batch and shorter block, so the second call runs on the first call's leftover scratch.
(Dimensions past the static array's size are rejected on the host: tests/test_abi.py.)"""
import numpy as np
import pytest

import oracle
from draft_sampling_lossless_spec_amd import workloads as wl
from gpu_util import PATH_AUTO, PATH_RESIDENT, PATH_STEPWISE, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _noalloc(w, noise, path):
    import torch
    from draft_sampling_lossless_spec_amd import spec_cycle_noalloc
    d = to_device(w)
    B, K = w.cfg.B, w.cfg.K
    out = {"accepted_len": torch.empty(B, dtype=torch.int32, device="cuda"),
           "tokens": torch.empty((B, K + 1), dtype=torch.int32, device="cuda"),
           "verify_len": torch.empty(B, dtype=torch.int32, device="cuda"),
           "draft_tokens": torch.empty((B, K), dtype=torch.int32, device="cuda"),
           "logq": torch.empty((B, K), dtype=torch.float32, device="cuda"),
           "logp": torch.empty((B, K), dtype=torch.float32, device="cuda")}
    torch.cuda.synchronize()
    spec_cycle_noalloc(d["base"], d["target"], d["A"], d["W"], d["conf"], d["temp"], w.threshold, w.seed, out,
                       x0=d["x0"], noise=noise, path=path)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _same(a, b):
    for k in a:
        if a[k].dtype.kind == "f":
            np.testing.assert_array_equal(np.isnan(a[k]), np.isnan(b[k]))
            m = ~np.isnan(a[k])
            np.testing.assert_array_equal(a[k][m], b[k][m])
        else:
            np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("noise,path", [(oracle.CHUNKED, PATH_RESIDENT), (oracle.CHUNKED, PATH_STEPWISE),
                                        (oracle.FLAT, PATH_AUTO)])
def test_noalloc_matches_workspace_entry_point(noise, path):
    print(f"noalloc noise={noise} path={path}", flush=True)
    # the resident cycle takes whole 64-column chunks only; the other paths also run a ragged tail
    big = wl.generate(wl.small_config(B=48, K=6, V=6016 if path == PATH_RESIDENT else 6000, R=64, threshold=0.05))
    small = wl.generate(wl.small_config(B=9, K=3, V=2048, R=32, threshold=0.1), gen_seed=2, cycle_seed=5)
    for w in (big, small):
        _same(run_gpu(w, noise, path=path), _noalloc(w, noise, path))
