"""Helpers for GPU tests: move a workload to the device and run the library through its binding."""
import numpy as np


def to_device(w):
    import torch
    dev = "cuda"

    def arr(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    return dict(base=arr(w.base), target=arr(w.target), A=arr(w.A), W=arr(w.W),
                x0=torch.from_numpy(w.x0.astype(np.int32)).to(dev),
                conf=torch.from_numpy(w.conf.astype(np.float32)).to(dev),
                temp=torch.from_numpy(w.temp.astype(np.float32)).to(dev))


# execution paths compared with the oracle per noise scheme: chunked noise has both the
# stepwise kernels and the one-launch resident cycle (the automatic choice where it qualifies)
PATH_AUTO, PATH_STEPWISE, PATH_RESIDENT = 0, 1, 2
PATH_NAMES = {PATH_AUTO: "auto", PATH_STEPWISE: "stepwise", PATH_RESIDENT: "resident"}


def taken_path(w, noise, path=PATH_AUTO):
    from draft_sampling_lossless_spec_amd import spec_cycle_path
    c = w.cfg
    return PATH_NAMES[spec_cycle_path(c.B, c.K, c.V, c.R, c.dtype, noise, path)]


def paths_for(w, noise):
    """The explicit paths a case runs on: the automatic one, and for chunked noise both the
    stepwise kernels and the one-launch resident cycle wherever the call qualifies for it."""
    from draft_sampling_lossless_spec_amd import SpecError, spec_cycle_path
    if noise == 0:
        return [PATH_AUTO]
    c = w.cfg
    out = [PATH_STEPWISE]
    try:
        spec_cycle_path(c.B, c.K, c.V, c.R, c.dtype, noise, PATH_RESIDENT)
        out.append(PATH_RESIDENT)
    except SpecError:
        pass
    return out


def run_gpu(w, noise, dev_inputs=None, request_offset=0, x0=True, workspace=None, path=PATH_AUTO):
    import torch
    from draft_sampling_lossless_spec_amd import spec_cycle
    d = dev_inputs or to_device(w)
    out = spec_cycle(d["base"], d["target"], d["A"], d["W"], d["conf"], d["temp"], w.threshold, w.seed,
                     x0=d["x0"] if x0 else None, request_offset=request_offset, noise=noise, diag=True,
                     workspace=workspace, path=path)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}
