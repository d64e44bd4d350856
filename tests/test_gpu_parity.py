"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on the same seeded
inputs.  Every case, the full-size workloads included, is compared request by request on every
output (tokens, accepted and verify lengths, drafted tokens, log q and log p); the full-size
workloads are also checked by the structural invariants.  Each compared case's counts (requests,
matched, excused near-ties, decisions, near-tie rate) are printed in the session summary."""
import numpy as np
import pytest

import oracle
from draft_sampling_lossless_spec_amd import workloads as wl
from gpu_util import PATH_AUTO, PATH_STEPWISE, paths_for, run_gpu, taken_path, to_device
from conftest import record_parity
from parity import Report, check_structure, compare

pytestmark = pytest.mark.gpu

NOISES = [oracle.FLAT, oracle.CHUNKED]


def ref(w, noise, request_offset=0, x0=True):
    return oracle.spec_cycle_ref(w.base, w.target, w.A, w.W, w.x0 if x0 else None, w.conf, w.temp, w.threshold,
                                 w.seed, noise=noise, request_offset=request_offset)


def assert_parity(rep: Report, case: str = ""):
    print(rep.summary(), flush=True)
    if case:
        record_parity(case, rep.summary())
    assert not rep.failures, "\n".join(rep.failures[:10])
    assert rep.near_tie_rate < 1e-3


def full_compare(w, noise, **kw):
    """Every path of this noise scheme against one oracle run; returns the last path's outputs."""
    o = ref(w, noise, **({"x0": kw["x0"]} if "x0" in kw else {}))
    for path in paths_for(w, noise):
        print(f"  path {taken_path(w, noise, path)}", flush=True)
        g = run_gpu(w, noise, path=path, **kw)
        assert_parity(compare(o, g))
    return g, o


SMALL = {
    "tiny_fp32": lambda: wl.generate("tiny"),
    "ragged_v333_bf16": lambda: wl.generate(wl.small_config(B=12, K=6, V=333, R=32, threshold=0.15)),
    "v20000_bf16_two_plain_items": lambda: wl.generate(wl.small_config(B=40, K=5, V=20000, R=64, threshold=0.1)),
    # the same on whole 64-column chunks, which the resident cycle also takes
    "v20032_bf16_five_plain_items": lambda: wl.generate(wl.small_config(B=40, K=5, V=20032, R=64, threshold=0.1)),
    "b300_two_row_blocks": lambda: wl.generate(wl.small_config(B=300, K=3, V=2048, R=16, threshold=0.05)),
    "fp32_v1001": lambda: wl.generate(wl.small_config(B=5, K=4, V=1001, R=8, dtype=wl.FP32, threshold=0.1)),
    "k1_b1": lambda: wl.generate(wl.small_config(B=1, K=1, V=4096, R=256, threshold=0.1)),
    "temp06_k8": lambda: wl.generate(wl.small_config(B=16, K=8, V=5000, R=32, threshold=0.05, temp=0.6,
                                                      sigma=(1.5,))),
    # the longest draft block the library takes (K = 32: 33 steps), close drafts so that requests
    # survive to late steps, full rank on the bf16 fast path
    "k32_max_positions": lambda: wl.generate(wl.small_config(B=8, K=32, V=3008, R=256, threshold=1e-6,
                                                              sigma=(0.3,))),
    # the largest batch (1024 requests): 224 slots staged on the fast path, most sub-blocks past them
    "b1024_small_v": lambda: wl.generate(wl.small_config(B=1024, K=2, V=1024, R=32, threshold=0.05)),
}


@pytest.mark.parametrize("noise", NOISES)
@pytest.mark.parametrize("case", sorted(SMALL))
def test_small_cases_match_oracle(case, noise):
    print(f"case {case} noise {noise}", flush=True)
    full_compare(SMALL[case](), noise)


@pytest.mark.parametrize("noise", NOISES)
def test_no_previous_token_and_cut_extremes(noise):
    w = wl.generate(wl.small_config(B=8, K=4, V=3008, R=32, threshold=0.2))
    full_compare(w, noise, x0=False)
    w.threshold = 2.0   # nothing survives the cut: one bonus token per request
    g, _ = full_compare(w, noise)
    assert np.all(g["verify_len"] == 0) and np.all(g["accepted_len"] == 0)
    w.threshold = 0.0   # everything is verified
    g, _ = full_compare(w, noise)
    assert np.all(g["verify_len"] == 4)


@pytest.mark.parametrize("noise", NOISES)
def test_identical_draft_and_target_accept_all(noise):
    w = wl.generate(wl.small_config(B=8, K=5, V=2048, R=16, threshold=0.05))
    w.base[:] = w.target[:, :5]
    w.A[:] = 0
    w.W[:] = 0
    g, _ = full_compare(w, noise)
    assert np.array_equal(g["accepted_len"], g["verify_len"])


@pytest.mark.parametrize("noise", NOISES)
def test_invalid_requests(noise):
    w = wl.generate(wl.small_config(B=6, K=3, V=600, R=16, dtype=wl.FP32, threshold=0.05))
    w.temp[0] = 0.0
    w.temp[1] = np.nan
    w.x0[2] = w.cfg.V
    w.target[3, 0, 5] = np.nan
    w.conf[3] = 1.0
    w.base[4, 1, :] = -np.inf
    w.conf[4] = 1.0
    g, o = full_compare(w, noise)
    assert np.all(g["accepted_len"][:5] == -1) and g["accepted_len"][5] >= 0


@pytest.mark.parametrize("noise", NOISES)
def test_determinism_and_sharding(noise):
    w = wl.generate(wl.small_config(B=20, K=5, V=4032, R=32, threshold=0.1))
    h = 7
    half = wl.Workload(w.cfg, w.base[h:], w.target[h:], w.A, w.W, w.x0[h:], w.conf[h:], w.temp[h:], w.threshold,
                       w.seed, w.request_ids[h:])
    for path in paths_for(w, noise):
        print(f"  path {taken_path(w, noise, path)}", flush=True)
        g1 = run_gpu(w, noise, path=path)
        g2 = run_gpu(w, noise, path=path)
        for k in g1:
            np.testing.assert_array_equal(g1[k], g2[k])
        g3 = run_gpu(half, noise, request_offset=h, path=path)
        for k in g1:
            np.testing.assert_array_equal(g1[k][h:], g3[k])


# (workload, threshold or None for its own, generator and cycle seed); cases of one workload and
# seed are adjacent so that its generated inputs are reused
FULL = [("dspark5", None, 1), ("dspark5", None, 2), ("dspark5", None, 3),
        ("longblock", None, 1), ("longblock", None, 2), ("longblock", None, 3),
        ("mixed", None, 1),
        ("highconc", 0.05, 1), ("highconc", 0.2, 1), ("highconc", 0.5, 1), ("highconc", 0.8, 1)]
FULL_CASES = [(n, t, sd, nz) for (n, t, sd) in FULL for nz in NOISES]

_cache = {}


def _full_workload(name, seed):
    key = (name, seed)
    if key not in _cache:
        _cache.clear()
        _cache[key] = wl.generate(name, gen_seed=seed, cycle_seed=seed)
    return _cache[key]


@pytest.mark.parametrize("name,thr,seed,noise", FULL_CASES)
def test_full_size_workloads(name, thr, seed, noise):
    case = f"{name} thr={thr} seed={seed} noise={'chunked' if noise == oracle.CHUNKED else 'flat'}"
    print(f"full {case}", flush=True)
    w = _full_workload(name, seed)
    w.threshold = w.cfg.threshold if thr is None else thr
    paths = paths_for(w, noise)
    if noise == oracle.CHUNKED:
        # the full-size chunked workloads are what the one-launch resident cycle is for
        assert len(paths) == 2
    # every request of the batch against the oracle, on every path of this noise scheme
    o = ref(w, noise)
    for path in paths:
        pname = taken_path(w, noise, path)
        g = run_gpu(w, noise, path=path)
        errs = check_structure(w, g, oracle.cut)
        assert not errs, "\n".join(errs[:10])
        assert_parity(compare(o, g), f"{case} path={pname}")
        print(f"{name} {pname}: sum L={int(g['verify_len'].sum())} sum a={int(g['accepted_len'].sum())}", flush=True)


def test_side_stream_matches_default_stream():
    """A call enqueued on a side stream gives the default-stream results; the tensors the binding
    allocates for it stay reserved for that stream while other work allocates on the default one."""
    import torch
    from draft_sampling_lossless_spec_amd import spec_cycle
    print("side stream", flush=True)
    w = wl.generate(wl.small_config(B=20, K=5, V=4032, R=32, threshold=0.1))
    g1 = run_gpu(w, oracle.CHUNKED)
    d = to_device(w)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    out = spec_cycle(d["base"], d["target"], d["A"], d["W"], d["conf"], d["temp"], w.threshold, w.seed, x0=d["x0"],
                     noise=oracle.CHUNKED, diag=True, stream=side)
    # default-stream allocations and writes while the side-stream call may still run
    junk = [torch.full((1 << 20,), 7, dtype=torch.int32, device="cuda") for _ in range(16)]
    side.synchronize()
    torch.cuda.synchronize()
    g2 = {k: v.cpu().numpy() for k, v in out.items()}
    for k in g1:
        np.testing.assert_array_equal(g1[k], g2[k])
    assert all(int(j[0].item()) == 7 for j in junk)


def test_resident_workspace_reused_across_shapes():
    """One workspace for consecutive resident calls of different shapes (the same bytes hold one
    call's records where the next call keeps its published per-request words, and the reverse):
    every call matches the oracle, so no word left by an earlier call is taken for a live one."""
    import torch
    from draft_sampling_lossless_spec_amd import spec_workspace_bytes
    from gpu_util import PATH_RESIDENT
    shapes = [dict(B=64, K=6, V=2048, R=32, threshold=0.02), dict(B=32, K=3, V=1024, R=16, threshold=0.05),
              dict(B=96, K=8, V=2048, R=32, threshold=0.01), dict(B=64, K=6, V=2048, R=32, threshold=0.02)]
    ws_bytes = max(spec_workspace_bytes(c["B"], c["K"], c["V"], c["R"], path=PATH_RESIDENT) for c in shapes)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    for i, cfg in enumerate(shapes):
        w = wl.generate(wl.small_config(**cfg), gen_seed=i + 1)
        print(f"shared workspace call {i}: {cfg}", flush=True)
        g = run_gpu(w, oracle.CHUNKED, workspace=ws, path=PATH_RESIDENT)
        assert_parity(compare(ref(w, oracle.CHUNKED), g))
