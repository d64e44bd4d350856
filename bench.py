"""Benchmark of one batched speculation cycle on one MI355X.

A step is one full cycle (prefix cut, Markov-biased draft of every verified position, rejection
verification, correction / bonus) over one batch of synthetic inputs already resident in HBM.
Default workload: the 16-position long-block cycle, B=256, K=16, V=151936, rank 256, bf16.

Prints one JSON line: throughput in verified draft tokens/s (sum of per-request verify lengths
per second, wall clock of back-to-back cycles), the per-cycle p10/p50/p90 and the same with the
last-level cache flushed between cycles, the roofline of the dominant kernel from HIP events
attached to its dispatches, the fp64 CPU oracle on the whole batch (all host threads, plus one
thread on a sample) with the parity counts of the GPU's first cycle against it, and the same
figures for the other four synthetic workloads under `configs`.
"""
import argparse
import ctypes as C
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12        # MI355X HBM3E, bytes/s
MFMA_PEAK = 2.5e15       # MI355X dense bf16 matrix peak, flop/s
METRIC = "verified draft tokens/sec per MI355X + % HBM roofline (B=256,K=16,V=151936)"


def hip_runtime():
    hip = C.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
    hip.hipEventCreate.restype = C.c_int
    hip.hipEventDestroy.argtypes = [C.c_void_p]
    hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
    hip.hipEventElapsedTime.restype = C.c_int
    return hip


def compulsory_bytes(cfg, L, a):
    """Bytes the method must move at least once: draft rows of every verified position, target rows
    of every decided position plus the correction/bonus row, W once, the gathered A rows, and the
    small per-request inputs and outputs."""
    e = 2 if cfg.dtype == 1 else 4
    V, R, K = cfg.V, cfg.R, cfg.K
    B = len(L)
    sL = int(L.sum())
    sa1 = int((a + 1).sum())
    return (e * V * (sL + sa1) + e * R * V + e * R * sL + 4 * B * K + 12 * B + 4 * B * (K + 1))


def bias_flops(cfg, L, a):
    """Flops of the Markov-bias contraction the cycle must do: one [R] x [R, V] product per draft
    row of a verified position and per correction row (a request rejected before its last
    position)."""
    rows = int(L.sum()) + int((a < L).sum())
    return 2 * cfg.R * cfg.V * rows


def measured_traffic(kernel, workload, noise):
    """HBM bytes per launch of `kernel` from the rocprofv3 FETCH_SIZE / WRITE_SIZE record committed
    under profiles/, scaled by a plain copy's readings; None unless the record was taken on the
    current kernel source and on this workload."""
    import re
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if noise != "chunked" or not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return int(rec["traffic_bytes_per_launch"])


def kernel_source_hash(kernel):
    """SHA-256 over the sources a kernel is built from (a traffic record holds only while they are
    unchanged)."""
    import hashlib
    csrc = os.path.join(ROOT, "draft_sampling_lossless_spec_amd", "csrc")
    files = (["cycle_resident.hip", "resident.h", "device_common.h"] if kernel == "k_resident"
             else ["spec_cycle.hip"])
    h = hashlib.sha256()
    for fn in files:
        h.update(open(os.path.join(csrc, fn), "rb").read())
    return h.hexdigest()


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def pct(x, q):
    return float(np.percentile(np.asarray(x, dtype=np.float64), q))


def parity_counts(orc, diag):
    """The oracle's outputs against the GPU's first cycle under the parity rule of the tests."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity import compare
    rep = compare(orc, diag)
    return {"requests": rep.requests, "matched": rep.matched, "excused": rep.excused,
            "failures": len(rep.failures), "decisions": rep.decisions, "near_ties": rep.near_ties,
            "near_tie_rate": rep.near_tie_rate, "max_prob_err": rep.max_prob_err,
            "first_failures": rep.failures[:3]}


def measure(name, threshold, steps, warmup, noise, with_oracle, flush_only=False, seed=1, events=True, path=0,
            oracle_requests=0):
    """One workload: timed cycles (back to back and with the cache flushed between cycles), the
    dominant kernel's event-timed launches, and the oracle beside it with the parity counts of the
    first cycle.  Returns (summary dict, diagnostics for the main line)."""
    import torch
    from draft_sampling_lossless_spec_amd import (spec_cycle, spec_cycle_kernel_count, spec_cycle_path,
                                                  spec_workspace_bytes)
    from draft_sampling_lossless_spec_amd import workloads as wl

    t0 = time.time()
    w = wl.generate(name, gen_seed=seed, cycle_seed=seed, threshold=threshold)
    cfg = w.cfg
    from draft_sampling_lossless_spec_amd import SpecError
    try:
        spec_cycle_path(cfg.B, cfg.K, cfg.V, cfg.R, cfg.dtype, noise, path)
    except SpecError:
        path = 0   # a workload the requested path does not take (fp32 rows, say): the automatic choice
    print(f"[bench] {name} thr={w.threshold}: generated in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    base, target, A, W = t(w.base), t(w.target), t(w.A), t(w.W)
    x0, conf, temp = t(w.x0), t(w.conf), t(w.temp)
    B, K = cfg.B, cfg.K
    ws = torch.empty(spec_workspace_bytes(B, K, cfg.V, cfg.R, cfg.dtype, noise, path), dtype=torch.uint8, device=dev)
    out = {"accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
           "tokens": torch.empty((B, K + 1), dtype=torch.int32, device=dev)}
    run = lambda **kw: spec_cycle(base, target, A, W, conf, temp, w.threshold, w.seed, x0=x0, noise=noise,
                                  workspace=ws, out=out, path=path, **kw)
    dg = spec_cycle(base, target, A, W, conf, temp, w.threshold, w.seed, x0=x0, noise=noise, workspace=ws,
                    diag=True, path=path)
    torch.cuda.synchronize()
    diag = {k: v.cpu().numpy() for k, v in dg.items()}
    L, a = diag["verify_len"], diag["accepted_len"]
    assert np.all(a >= 0), "synthetic workload produced invalid requests"
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    taken = spec_cycle_path(B, K, cfg.V, cfg.R, cfg.dtype, noise, path)
    res = {"B": B, "K": K, "V": cfg.V, "R": cfg.R, "threshold": w.threshold, "sum_verify_len": int(L.sum()),
           "sum_emitted": int((a + 1).sum()), "max_verify_len": int(L.max()),
           "path": {1: "stepwise", 2: "resident"}[taken]}
    cb = compulsory_bytes(cfg, L, a)
    res["compulsory_bytes"] = cb

    ms = None
    if not flush_only:
        # back to back: the wall clock of `steps` plain calls is the figure; an event pair between
        # calls gives the per-cycle spread
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ts = time.perf_counter()
        evs[0].record()
        for i in range(steps):
            run()
            evs[i + 1].record()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - ts) * 1e3 / steps
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        res.update({"us_per_cycle": ms * 1e3, "p10_us": pct(per, 10) * 1e3, "p50_us": pct(per, 50) * 1e3,
                    "p90_us": pct(per, 90) * 1e3, "value": int(L.sum()) / (ms * 1e-3),
                    "hbm_frac_cycle": cb / (ms * 1e-3) / HBM_PEAK})
    # flushed: a 1 GiB write between cycles evicts the 256 MB last-level cache; only the cycle is timed
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    fl = []
    for i in range(steps):
        scratch.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        e1.synchronize()
        fl.append(e0.elapsed_time(e1))
    del scratch
    res.update({"flushed_p10_us": pct(fl, 10) * 1e3, "flushed_p50_us": pct(fl, 50) * 1e3,
                "flushed_p90_us": pct(fl, 90) * 1e3,
                "flushed_value": int(L.sum()) / (pct(fl, 50) * 1e-3),
                "flushed_hbm_frac_cycle": cb / (pct(fl, 50) * 1e-3) / HBM_PEAK})

    kern = None
    if events:
        # start/stop events attached to every kernel dispatch of the cycle (same work, own pass)
        hip = hip_runtime()
        nk = spec_cycle_kernel_count(B, K, cfg.V, cfg.R, cfg.dtype, noise, path)
        nrep = max(3, min(steps, 10))
        ev = [(C.c_void_p * (2 * nk))() for _ in range(nrep)]
        for arr in ev:
            for i in range(2 * nk):
                h = C.c_void_p()
                assert hip.hipEventCreate(C.byref(h)) == 0
                arr[i] = h.value
        torch.cuda.synchronize()
        for i in range(nrep):
            run(_events=ev[i])
        torch.cuda.synchronize()

        def el(e0, e1):
            f = C.c_float()
            assert hip.hipEventElapsedTime(C.byref(f), C.c_void_p(e0), C.c_void_p(e1)) == 0
            return f.value

        d = np.array([[el(arr[2 * k], arr[2 * k + 1]) for k in range(nk)] for arr in ev])   # ms [rep, kernel]
        for arr in ev:
            for i in range(2 * nk):
                hip.hipEventDestroy(C.c_void_p(arr[i]))
        kern = kernel_breakdown(cfg, L, a, d, nk)
        res["kernels"] = {k: {kk: vv for kk, vv in v.items() if kk != "per_step_us"} for k, v in kern.items()}

    if with_oracle:
        # the oracle on the whole batch, or on its first oracle_requests requests (request ids, and so
        # the noise, are those of the whole batch)
        import oracle
        n = B if not oracle_requests else min(B, oracle_requests)
        tc = time.perf_counter()
        r = oracle.spec_cycle_ref(w.base[:n], w.target[:n], w.A, w.W, w.x0[:n], w.conf[:n], w.temp[:n], w.threshold,
                                  w.seed, noise=noise)
        dt = time.perf_counter() - tc
        res["oracle"] = {"seconds": dt, "threads": oracle.max_threads(), "requests": n,
                         "value": float(r["verify_len"][r["verify_len"] > 0].sum() / dt)}
        dn = {k: (v[:n] if hasattr(v, "shape") and v.ndim >= 1 and v.shape[0] == B else v) for k, v in diag.items()}
        res["parity"] = parity_counts(r, dn)
    return res, (w, cfg, L, a, kern)


def kernel_breakdown(cfg, L, a, d, nk):
    """Per-kernel times (us per cycle) from the event-timed pass, and the algorithmic bytes of the
    kernels that stream rows.  d: [repetitions, dispatch] milliseconds."""
    e = 2 if cfg.dtype == 1 else 4
    sL, sa1 = int(L.sum()), int((a + 1).sum())
    bias_bytes = e * cfg.V * sL + e * cfg.R * cfg.V + e * cfg.R * sL      # draft rows, W once, gathered A rows
    plain_bytes = e * cfg.V * sa1                                        # decided target rows + bonus rows
    mean = d.mean(axis=0) * 1e3                                          # us per dispatch
    if nk == 1:
        # one persistent launch runs the whole cycle
        cb = compulsory_bytes(cfg, L, a)
        return {"k_resident": {"us_per_cycle": float(mean[0]), "algorithmic_bytes": cb, "launches_per_cycle": 1,
                               "achieved_GBps": cb / (mean[0] * 1e-6) / 1e9,
                               "bias_flops": bias_flops(cfg, L, a)}}
    K = cfg.K
    steps = np.arange(K + 1)
    kb, kp, km = mean[1 + 3 * steps], mean[2 + 3 * steps], mean[3 + 3 * steps]
    fused = cfg.dtype == 1 and cfg.V % 8 == 0
    out = {"k_init": {"us_per_cycle": float(mean[0]), "launches_per_cycle": 1}}
    if fused:
        sb = bias_bytes + plain_bytes
        out["k_sweep"] = {"us_per_cycle": float(kb.sum()), "algorithmic_bytes": sb, "launches_per_cycle": K + 1,
                          "achieved_GBps": sb / (kb.sum() * 1e-6) / 1e9, "per_step_us": kb.tolist()}
    else:
        out["k_bias"] = {"us_per_cycle": float(kb.sum()), "algorithmic_bytes": bias_bytes,
                         "launches_per_cycle": K + 1, "achieved_GBps": bias_bytes / (kb.sum() * 1e-6) / 1e9}
        out["k_plain"] = {"us_per_cycle": float(kp.sum()), "algorithmic_bytes": plain_bytes,
                          "launches_per_cycle": K + 1, "achieved_GBps": plain_bytes / (kp.sum() * 1e-6) / 1e9}
    out["k_merge"] = {"us_per_cycle": float(km.sum()), "launches_per_cycle": K + 1, "per_step_us": km.tolist()}
    return out


# the five synthetic workloads; the long-block one is the headline line, the others go into `configs`
OTHER_CONFIGS = [("tiny", None), ("dspark5", None), ("highconc", 0.05), ("highconc", 0.2), ("highconc", 0.5),
                 ("highconc", 0.8), ("mixed", None)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="longblock")
    ap.add_argument("--threshold", type=float, default=None)
    ap.add_argument("--noise", choices=["chunked", "flat"], default="chunked")
    ap.add_argument("--path", choices=["auto", "stepwise", "resident"], default="auto",
                    help="execution path of the cycle (auto: the resident one whenever the call qualifies)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true", help="measure the headline workload only (no `configs`)")
    ap.add_argument("--cpu-sample", type=int, default=16,
                    help="requests in the single-threaded oracle sample of the headline workload")
    ap.add_argument("--stats", action="store_true",
                    help="measure the acceptance-statistics call (alpha = 1 - TV per drafted position) on the drafts "
                         "of one cycle of the workload instead of the cycle itself; prints its own JSON line")
    ap.add_argument("--schedule", action="store_true",
                    help="measure the prefix scheduler on the workload's confidences against a synthetic target "
                         "step-time curve at several loads; prints its own JSON line")
    ap.add_argument("--sts", action="store_true",
                    help="measure sequential temperature scaling on synthetic held-out confidences (an "
                         "overconfident head); prints its own JSON line")
    ap.add_argument("--decode", type=int, default=0,
                    help="chain this many scheduled cycles (scheduler, cycle, next context, all on the device) over "
                         "two alternating row sets and report tokens per cycle and the modelled latency per token")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (5 times) and exit: the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    ap.add_argument("--cpu-requests", type=int, default=0,
                    help="(--stats) requests in the oracle's timed sample (0 = the whole batch)")
    args = ap.parse_args()
    if args.copy_bytes > 0:
        import torch
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4, "copies": 5}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (requests shard with "
              "request_offset and no collective; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.stats:
        return bench_stats(args)
    if args.schedule:
        return bench_schedule(args)
    if args.sts:
        return bench_sts(args)
    if args.decode > 0:
        return bench_decode(args)

    from draft_sampling_lossless_spec_amd import CHUNKED, FLAT
    noise = CHUNKED if args.noise == "chunked" else FLAT
    with_oracle = not args.no_cpu_baseline
    path = {"auto": 0, "stepwise": 1, "resident": 2}[args.path]
    res, (w, cfg, L, a, kern) = measure(args.config, args.threshold, args.steps, args.warmup, noise, with_oracle,
                                        path=path)
    ms_per_step = res["us_per_cycle"] * 1e-3
    print(f"[bench] {args.config}: sum L={res['sum_verify_len']} sum(a+1)={res['sum_emitted']} "
          f"max L={res['max_verify_len']} compulsory={res['compulsory_bytes'] / 1e6:.1f} MB; wall "
          f"{res['us_per_cycle']:.1f} us/cycle (p10/p50/p90 {res['p10_us']:.1f}/{res['p50_us']:.1f}/"
          f"{res['p90_us']:.1f}); flushed p50 {res['flushed_p50_us']:.1f} us", file=sys.stderr, flush=True)
    for k, v in kern.items():
        extra = f" per-step {' '.join(f'{x:.1f}' for x in v['per_step_us'])}" if "per_step_us" in v else ""
        print(f"[bench]   {k}: {v['us_per_cycle']:.1f} us/cycle{extra}", file=sys.stderr, flush=True)

    dom = max((k for k in kern if "algorithmic_bytes" in kern[k]), key=lambda k: kern[k]["us_per_cycle"])
    nl = kern[dom]["launches_per_cycle"]
    achieved = kern[dom]["achieved_GBps"] * 1e9
    traffic = measured_traffic(dom, cfg.name, args.noise) if cfg.dtype == 1 else None

    cpu = None
    if with_oracle:
        import oracle
        n = max(1, min(args.cpu_sample, cfg.B))
        tc = time.perf_counter()
        r1 = oracle.spec_cycle_ref(w.base[:n], w.target[:n], w.A, w.W, w.x0[:n], w.conf[:n], w.temp[:n],
                                   w.threshold, w.seed, noise=noise, nthreads=1)
        dt1 = time.perf_counter() - tc
        o = res["oracle"]
        cpu = {"value": o["value"], "unit": "verified draft tokens/s", "cores": o["threads"], "kind": "oracle",
               "sample": f"the whole batch of one cycle of the same workload ({cfg.B} requests, "
                         f"{res['sum_verify_len']} verified draft tokens, {o['seconds']:.1f} s wall, fp64 C + "
                         f"OpenMP over requests)",
               "value_1thread": float(r1["verify_len"].sum() / dt1),
               "sample_1thread": f"first {n} requests ({int(r1['verify_len'].sum())} verified draft tokens, "
                                 f"{dt1:.1f} s wall, one thread)",
               "cpu_model": cpu_model(), "host_threads": os.cpu_count()}

    configs = {}
    if not args.only and args.config == "longblock":
        for name, thr in OTHER_CONFIGS:
            steps = max(5, min(args.steps, 10))
            # every request of these workloads is compared with the oracle by the GPU parity tests;
            # here the first 128 of each, so that the whole run stays within a few minutes
            r, _ = measure(name, thr, steps, 2, noise, with_oracle, flush_only=(name == "dspark5"), events=False,
                           path=path, oracle_requests=128)
            key = name if thr is None else f"{name}_tau{thr}"
            configs[key] = r
            print(f"[bench] {key}: " + json.dumps({k: r.get(k) for k in ("us_per_cycle", "flushed_p50_us",
                                                                            "hbm_frac_cycle",
                                                                            "flushed_hbm_frac_cycle")})
                  + (f" parity {r['parity']['matched']}/{r['parity']['requests']}" if "parity" in r else ""),
                  file=sys.stderr, flush=True)

    line = {
        "metric": METRIC, "value": res["value"], "unit": "verified draft tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if cfg.dtype == 1 else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "K": cfg.K, "V": cfg.V, "R": cfg.R, "threshold": w.threshold,
                   "noise": args.noise, "path": res["path"], "sum_verify_len": res["sum_verify_len"],
                   "sum_emitted": res["sum_emitted"],
                   "max_verify_len": res["max_verify_len"]},
        "hbm_frac_cycle": res["hbm_frac_cycle"],
        "cycle_us": {k: res[k] for k in ("us_per_cycle", "p10_us", "p50_us", "p90_us", "flushed_p10_us",
                                        "flushed_p50_us", "flushed_p90_us")},
        "flushed_value": res["flushed_value"], "flushed_hbm_frac_cycle": res["flushed_hbm_frac_cycle"],
        "roofline": roofline_obj(kern, dom, nl, achieved, traffic),
        "kernels": res["kernels"],
        "parity": res.get("parity"),
        "cpu_baseline": cpu,
        "configs": configs,
    }
    print(json.dumps(line), flush=True)


def roofline_obj(kern, dom, nl, achieved, traffic):
    """The dominant kernel against its roofline.  For the one-launch cycle both floors are given: the
    HBM floor of its algorithmic bytes and the MFMA floor of its bias contraction; `bound` names the
    larger one."""
    k = kern[dom]
    r = {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
         "frac": achieved / HBM_PEAK, "traffic": traffic, "kernel": dom, "launches_per_cycle": nl,
         "traffic_unit": "HBM bytes per launch", "algorithmic_bytes_per_launch": k["algorithmic_bytes"] / nl}
    if "bias_flops" in k:
        t = k["us_per_cycle"] * 1e-6
        hbm_floor, mfma_floor = k["algorithmic_bytes"] / HBM_PEAK, k["bias_flops"] / MFMA_PEAK
        r["floors_us"] = {"hbm": hbm_floor * 1e6, "mfma": mfma_floor * 1e6}
        mf = {"achieved": k["bias_flops"] / t / 1e12, "peak": MFMA_PEAK / 1e12, "unit": "TFLOP/s",
              "frac": k["bias_flops"] / t / MFMA_PEAK, "flops_per_launch": k["bias_flops"]}
        if mfma_floor > hbm_floor:
            # the contraction's floor is the higher one: the primary fields are the MFMA figures
            r["hbm"] = {kk: r[kk] for kk in ("achieved", "peak", "unit", "frac")}
            r.update({kk: mf[kk] for kk in ("achieved", "peak", "unit", "frac")})
            r["bound"] = "mfma"
        else:
            r["mfma"] = mf
    return r


def bench_decode(args):
    """Multi-cycle decode: per cycle the scheduler picks verify lengths from the confidences and
    the target step-time curve t(n) = 20 ms + 2 us n, the cycle runs with them, and each request's
    last emitted token becomes the next cycle's context; two synthetic row sets alternate and the
    seed advances per cycle.  Reports tokens per request per cycle (tau), the measured cycle time
    and the modelled latency per token (cycle + target step) / tau."""
    import torch
    from draft_sampling_lossless_spec_amd import (spec_advance, spec_cycle_lengths, spec_schedule,
                                                  spec_workspace_bytes)
    from draft_sampling_lossless_spec_amd import workloads as wl
    sets = [wl.generate(args.config, gen_seed=s, threshold=args.threshold) for s in (1, 2)]
    w = sets[0]
    B, K = w.cfg.B, w.cfg.K

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    rows = [(t(s.base), t(s.target), t(s.conf.astype(np.float32))) for s in sets]
    A, W, temp = t(w.A), t(w.W), t(w.temp)
    x0 = t(w.x0.astype(np.int32))
    emitted = torch.zeros(B, dtype=torch.int64, device="cuda")
    T = torch.from_numpy(0.02 + 2e-6 * np.arange(B * K + 1, dtype=np.float64)).cuda()
    L = torch.empty(B, dtype=torch.int32, device="cuda")
    so = torch.empty(4, dtype=torch.float64, device="cuda")
    ws = torch.empty(spec_workspace_bytes(B, K, w.cfg.V, w.cfg.R, w.cfg.dtype), dtype=torch.uint8, device="cuda")
    out = {"accepted_len": torch.empty(B, dtype=torch.int32, device="cuda"),
           "tokens": torch.empty((B, K + 1), dtype=torch.int32, device="cuda")}
    verify = torch.zeros(B, dtype=torch.int64, device="cuda")

    def cycle(c):
        base, target, conf = rows[c % 2]
        spec_schedule(conf, T, 4096, verify_len=L, out=so)
        spec_cycle_lengths(base, target, A, W, L, temp, w.seed + c, x0=x0, workspace=ws, out=out)
        spec_advance(out["tokens"], out["accepted_len"], x0, emitted)
        verify.add_(L.to(torch.int64))

    for c in range(2):
        cycle(c)
    torch.cuda.synchronize()
    emitted.zero_()
    verify.zero_()
    n = args.decode
    ts = time.perf_counter()
    for c in range(n):
        cycle(c)
    torch.cuda.synchronize()
    t_cycle = (time.perf_counter() - ts) / n
    tau = float(emitted.sum().item()) / (n * B)
    n_verify = float(verify.sum().item()) / n
    t_target = 0.02 + 2e-6 * n_verify
    line = {
        "metric": "scheduled decode: emitted tokens per request per cycle (tau)", "value": tau,
        "unit": "tokens/request/cycle", "n_gpus": 1, "steps": n, "warmup": 2, "ms_per_step": t_cycle * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.cfg.name, "B": B, "K": K, "row_sets": 2, "target_step_model": "20 ms + 2 us per draft token"},
        "decode": {"verify_tokens_per_cycle": n_verify, "cycle_us": t_cycle * 1e6,
                   "modelled_target_step_ms": t_target * 1e3,
                   "latency_per_token_ms": (t_cycle + t_target) / tau * 1e3,
                   "emitted_tokens_per_s_modelled": tau * B / (t_cycle + t_target),
                   "speculation_overhead_frac": t_cycle / (t_cycle + t_target)},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def bench_sts(args):
    """Sequential temperature scaling of a synthetic overconfident head: N = 100000 held-out
    sequences of K = 16 positions (true logits N(1.5, 1), raw logits 2x, survival drawn from the
    true probabilities, random verified lengths), 61-entry octave grid, 10 bins; timed with events
    on its stream, the oracle beside it."""
    import torch
    from draft_sampling_lossless_spec_amd import spec_temperature_scaling
    N, K = 100000, 16
    rng = np.random.default_rng(1)
    zt = rng.normal(1.5, 1.0, (N, K))
    surv = rng.random((N, K)) < 1 / (1 + np.exp(-zt))
    a = np.where(surv.all(axis=1), K, surv.argmin(axis=1)).astype(np.int32)
    L = rng.integers(1, K + 1, N).astype(np.int32)
    a = np.minimum(a, L).astype(np.int32)
    z = (2.0 * zt).astype(np.float32)
    grid = np.exp2(np.arange(-24, 37) / 12)   # 2^(m/12): a quarter to eight, T = 1 included
    c = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    zd, Ld, ad, gd = c(z), c(L), c(a), c(grid)
    for _ in range(args.warmup):
        out = spec_temperature_scaling(zd, Ld, ad, gd, 10)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        out = spec_temperature_scaling(zd, Ld, ad, gd, 10)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        tc = time.perf_counter()
        oracle.temperature_scaling_ref(z, L, a, grid, 10)
        dt = time.perf_counter() - tc
        cpu = {"value": 1.0 / dt, "unit": "fits/s", "cores": 1, "kind": "oracle",
               "sample": f"the same fit ({dt:.1f} s wall, fp64 C, one thread)"}
    pairs = int(np.minimum(L, K).sum())
    byt = 2 * (len(grid) + 1) * (4 * N * K + 8 * N + 8 * N)   # per evaluation: z column, lengths, running product
    line = {
        "metric": "sequential temperature scaling: fits/s", "value": 1e3 / ms, "unit": "fits/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": "held-out confidences, overconfident head x2", "N": N, "K": K, "grid": len(grid),
                   "nbins": 10, "pairs": pairs,
                   "T": [round(float(t), 3) for t in out["T"].cpu().numpy()],
                   "ece_before": float(out["ece_before"].mean().item()),
                   "ece_after": float(out["ece_after"].mean().item())},
        "roofline": {"bound": "alu", "achieved": None, "peak": None, "unit": None, "frac": None, "traffic": None,
                     "kernel": "k_sts_eval",
                     "note": "fp64 sigmoid per (sequence, grid entry, position); byte count for the record: "
                             f"{byt / 1e9:.2f} GB of L2-resident reads per fit"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_schedule(args):
    """Prefix scheduler: spec_schedule on the workload's confidences, timed with events on its
    stream, against the target step-time curve t(n) = t0 + t1 n (seconds per verification step with
    n draft tokens; t0 = the measured speculation cycle plus a fixed target cost, t1 the per-token
    cost at a few loads), with the oracle beside it."""
    import torch
    from draft_sampling_lossless_spec_amd import spec_schedule
    from draft_sampling_lossless_spec_amd import workloads as wl

    w = wl.generate(args.config, threshold=args.threshold)
    B, K = w.cfg.B, w.cfg.K
    conf = torch.from_numpy(w.conf.astype(np.float32)).cuda()
    n = np.arange(B * K + 1, dtype=np.float64)
    loads = {}
    for name, t1 in (("idle", 2e-7), ("moderate", 2e-6), ("busy", 2e-5)):
        T = torch.from_numpy(0.02 + t1 * n).cuda()      # 20 ms per target step plus t1 per draft token
        L, out = spec_schedule(conf, T, 4096)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        loads[name] = {"t1_s_per_token": t1, "verify_tokens": int(o[1]), "threshold": float(o[0]),
                       "mean_verify_len": float(L.float().mean().item()), "expected_tokens": float(o[2])}
    T = torch.from_numpy(0.02 + 2e-6 * n).cuda()
    Lb = torch.empty(B, dtype=torch.int32, device="cuda")
    ob = torch.empty(4, dtype=torch.float64, device="cuda")
    for _ in range(args.warmup):
        spec_schedule(conf, T, 4096, verify_len=Lb, out=ob)
    torch.cuda.synchronize()
    # one launch is a few microseconds, less than the Python call around it: the timed calls are
    # captured into one graph and replayed once between events
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(args.steps):
                spec_schedule(conf, T, 4096, verify_len=Lb, out=ob)
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    # the scheduled cycle at moderate load: scheduler -> cycle with its verify lengths, all on the device
    from draft_sampling_lossless_spec_amd import spec_cycle_lengths, spec_workspace_bytes

    def t_(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    base, target, A, W, x0, temp = (t_(a) for a in (w.base, w.target, w.A, w.W, w.x0, w.temp))
    ws = torch.empty(spec_workspace_bytes(B, K, w.cfg.V, w.cfg.R, w.cfg.dtype), dtype=torch.uint8, device="cuda")
    cyc_out = {"accepted_len": torch.empty(B, dtype=torch.int32, device="cuda"),
               "tokens": torch.empty((B, K + 1), dtype=torch.int32, device="cuda")}

    def scheduled():
        spec_schedule(conf, T, 4096, verify_len=Lb, out=ob)
        spec_cycle_lengths(base, target, A, W, Lb, temp, w.seed, x0=x0, workspace=ws, out=cyc_out)

    for _ in range(3):
        scheduled()
    torch.cuda.synchronize()
    tsc = time.perf_counter()
    for _ in range(10):
        scheduled()
    torch.cuda.synchronize()
    us_cycle = (time.perf_counter() - tsc) / 10 * 1e6
    n_sched = int(Lb.sum().item())
    sched_cycle = {"load": "moderate", "verify_tokens": n_sched, "us_per_cycle": us_cycle,
                   "verified_draft_tokens_per_s": n_sched / (us_cycle * 1e-6),
                   "emitted_tokens_per_cycle": int((cyc_out["accepted_len"] + 1).sum().item())}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        Tn = 0.02 + 2e-6 * n
        reps = 0
        tc = time.perf_counter()
        while time.perf_counter() - tc < 2.0:
            oracle.schedule_ref(w.conf.astype(np.float32), Tn, 4096)
            reps += 1
        dt = (time.perf_counter() - tc) / reps
        cpu = {"value": 1.0 / dt, "unit": "schedules/s", "cores": 1, "kind": "oracle",
               "sample": f"the whole batch, {reps} calls in {dt * reps:.1f} s (fp64 C, one thread)"}
    byt = 4 * B * K + 8 * (B * K + 1) + 4 * B + 32
    line = {
        "metric": "prefix scheduler: schedules/s", "value": 1e6 / us, "unit": "schedules/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": us * 1e-3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "config": {"workload": w.cfg.name, "B": B, "K": K, "nbins": 4096, "loads": loads},
        "scheduled_cycle": sched_cycle,
        "roofline": {"bound": "hbm", "achieved": byt / (us * 1e-6) / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": byt / (us * 1e-6) / HBM_PEAK, "traffic": None, "kernel": "k_schedule",
                     "note": "one workgroup over a few tens of KB: latency-bound, the HBM figure is for the record"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def bench_stats(args):
    """Acceptance statistics of one cycle's drafted positions: spec_accept_stats timed on its own
    (plain calls, wall clock), HBM roofline of the whole call, the oracle beside it on a sample."""
    import torch
    from draft_sampling_lossless_spec_amd import CHUNKED, spec_accept_stats, spec_cycle, spec_stats_workspace_bytes
    from draft_sampling_lossless_spec_amd import workloads as wl

    w = wl.generate(args.config, threshold=args.threshold)
    cfg = w.cfg
    dev = torch.device("cuda:0")

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    base, target, A, W = t(w.base), t(w.target), t(w.A), t(w.W)
    x0, conf, temp = t(w.x0), t(w.conf), t(w.temp)
    B, K = cfg.B, cfg.K
    diag = spec_cycle(base, target, A, W, conf, temp, w.threshold, w.seed, x0=x0, noise=CHUNKED, diag=True)
    draft = diag["draft_tokens"]
    torch.cuda.synchronize()
    rows = int((draft >= 0).sum().item())
    ws = torch.empty(spec_stats_workspace_bytes(B, K, cfg.V, cfg.R, cfg.dtype), dtype=torch.uint8, device=dev)
    out = {k: torch.empty((B, K), dtype=torch.float32, device=dev) for k in ("alpha", "lse_q", "lse_p")}
    run = lambda: spec_accept_stats(base, target, A, W, draft, temp, x0=x0, workspace=ws, out=out)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ts = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - ts) * 1e3 / args.steps
    # the same calls again between events on the stream they run on: the call-level roofline
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms_ev = e0.elapsed_time(e1) / args.steps
    e = 2 if cfg.dtype == 1 else 4
    alg = e * cfg.V * 2 * rows + e * cfg.R * cfg.V + e * cfg.R * rows + 4 * 3 * B * K
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        d_np = draft.cpu().numpy()
        n = max(1, min(B, args.cpu_requests or B))
        tc = time.perf_counter()
        oracle.accept_stats_ref(w.base[:n], w.target[:n], w.A, w.W, w.x0[:n], d_np[:n], w.temp[:n])
        dt = time.perf_counter() - tc
        cpu = {"value": float((d_np[:n] >= 0).sum() / dt), "unit": "drafted positions/s", "cores": oracle.max_threads(),
               "kind": "oracle", "sample": f"first {n} of {B} requests ({int((d_np[:n] >= 0).sum())} positions, "
                                           f"{dt:.1f} s wall, fp64 C + OpenMP)"}
    line = {
        "metric": "acceptance statistics: drafted positions/s (alpha = 1 - TV per position)", "value": rows / (ms * 1e-3),
        "unit": "drafted positions/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == 1 else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "K": K, "V": cfg.V, "R": cfg.R, "rows": rows},
        "roofline": {"bound": "hbm", "achieved": alg / (ms_ev * 1e-3) / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": alg / (ms_ev * 1e-3) / HBM_PEAK, "traffic": None,
                     "kernel": "spec_accept_stats (prep, 2 sweeps, 2 merges)", "algorithmic_bytes_per_call": alg},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
