"""The fail-loud path of the persistent kernels' bounded waits (the grid barrier and the lists' poll of
the words each merge publishes): a cooperative grid whose workgroups could not all run together
would wait forever, so every such wait gives up after a time limit, sets the workspace's error word,
and the call returns with every output marked invalid.  The limit is forced to zero from the host
(SPEC_RESIDENT_WAIT_TICKS, read at every launch), so a wait that does not end at its first poll
times out; every wave still leaves the kernel normally.  The next call, with the limit restored,
must be correct again (its nonce differs, so the error word of the failed call does not match)."""
import numpy as np
import pytest

import oracle
from draft_sampling_lossless_spec_amd import workloads as wl
from gpu_util import PATH_RESIDENT, run_gpu
from parity import compare

pytestmark = pytest.mark.gpu


def test_cycle_wait_timeout_marks_every_request_invalid_then_recovers(monkeypatch):
    # long drafts (low threshold) so that the cycle has several steps with merges and polls
    w = wl.generate(wl.small_config(B=48, K=6, V=2048, R=32, threshold=0.02))
    print("cycle: forced wait timeout, resident path", flush=True)
    monkeypatch.setenv("SPEC_RESIDENT_WAIT_TICKS", "0")
    g = run_gpu(w, oracle.CHUNKED, path=PATH_RESIDENT)
    assert np.all(g["accepted_len"] == -1)
    assert np.all(g["tokens"] == -1)
    monkeypatch.delenv("SPEC_RESIDENT_WAIT_TICKS")
    print("cycle: limit restored", flush=True)
    g = run_gpu(w, oracle.CHUNKED, path=PATH_RESIDENT)
    o = oracle.spec_cycle_ref(w.base, w.target, w.A, w.W, w.x0, w.conf, w.temp, w.threshold, w.seed,
                              noise=oracle.CHUNKED)
    rep = compare(o, g)
    print(rep.summary(), flush=True)
    assert not rep.failures, "\n".join(rep.failures[:10])


def test_stats_wait_timeout_gives_nan_then_recovers(monkeypatch):
    import torch
    from draft_sampling_lossless_spec_amd import spec_accept_stats
    from gpu_util import to_device
    w = wl.generate(wl.small_config(B=24, K=5, V=2048, R=32, threshold=0.1))
    rng = np.random.default_rng(5)
    draft = rng.integers(0, w.cfg.V, (w.cfg.B, w.cfg.K)).astype(np.int32)
    d = to_device(w)

    def run():
        out = spec_accept_stats(d["base"], d["target"], d["A"], d["W"], torch.from_numpy(draft).cuda(), d["temp"],
                                x0=d["x0"], path=PATH_RESIDENT)
        torch.cuda.synchronize()
        return {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}

    print("stats: forced wait timeout, W-resident kernel", flush=True)
    monkeypatch.setenv("SPEC_RESIDENT_WAIT_TICKS", "0")
    g = run()
    assert np.all(np.isnan(g["alpha"]))
    monkeypatch.delenv("SPEC_RESIDENT_WAIT_TICKS")
    print("stats: limit restored", flush=True)
    g = run()
    o = oracle.accept_stats_ref(w.base, w.target, w.A, w.W, w.x0, draft, w.temp)
    err = np.abs(o["alpha"] - g["alpha"])
    assert not np.isnan(g["alpha"]).any() and err.max() < 1e-4, f"alpha: max error {err.max():.3g}"
