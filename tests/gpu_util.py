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


def run_gpu(w, noise, dev_inputs=None, request_offset=0, x0=True, workspace=None):
    import torch
    from draft_sampling_lossless_spec_amd import spec_cycle
    d = dev_inputs or to_device(w)
    out = spec_cycle(d["base"], d["target"], d["A"], d["W"], d["conf"], d["temp"], w.threshold, w.seed,
                     x0=d["x0"] if x0 else None, request_offset=request_offset, noise=noise, diag=True,
                     workspace=workspace)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}
