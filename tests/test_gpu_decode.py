"""GPU decode loop against the oracle's: cycles chained on the device (spec_cycle, then
spec_advance feeding each request's last emitted token to the next cycle, seed + c per cycle,
two row sets alternating) compared cycle by cycle with the oracle's chain.  A request whose
outputs part ways at a near-tie (excused by the parity rule) continues from a different context,
so it leaves the comparison of later cycles."""
import numpy as np
import pytest

import oracle
from draft_sampling_lossless_spec_amd import workloads as wl
from gpu_util import PATH_AUTO, PATH_RESIDENT, PATH_STEPWISE, to_device
from parity import Report, compare

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("noise,path", [(oracle.FLAT, PATH_AUTO), (oracle.CHUNKED, PATH_STEPWISE),
                                        (oracle.CHUNKED, PATH_RESIDENT)])
def test_decode_chain_matches_oracle(noise, path):
    import torch
    from draft_sampling_lossless_spec_amd import spec_advance, spec_cycle
    print(f"decode chain noise={noise} path={path}", flush=True)
    V = 3008 if path == PATH_RESIDENT else 3000   # the resident cycle takes whole 64-column chunks only
    sets = [wl.generate(wl.small_config(B=32, K=6, V=V, R=32, threshold=0.1), gen_seed=s) for s in (1, 2)]
    w = sets[0]
    n_cycles, seed = 5, 11
    outs = oracle.decode_ref([s.base for s in sets], [s.target for s in sets], w.A, w.W, w.x0,
                             [s.conf for s in sets], w.temp, w.threshold, seed, n_cycles, noise=noise)
    devs = [to_device(s) for s in sets]
    A, W = devs[0]["A"], devs[0]["W"]
    x0 = torch.from_numpy(w.x0.astype(np.int32)).cuda()
    emitted = torch.zeros(w.cfg.B, dtype=torch.int64, device="cuda")
    synced = list(range(w.cfg.B))
    for c in range(n_cycles):
        d = devs[c % 2]
        g = spec_cycle(d["base"], d["target"], A, W, d["conf"], d["temp"], w.threshold, seed + c, x0=x0, noise=noise,
                       diag=True, path=path)
        spec_advance(g["tokens"], g["accepted_len"], x0, emitted)
        torch.cuda.synchronize()
        gn = {k: v.cpu().numpy() for k, v in g.items()}
        rep = compare(outs[c], gn, rows=synced)
        print(f"cycle {c}: {rep.summary()}", flush=True)
        assert not rep.failures, "\n".join(rep.failures[:10])
        same = [b for b in synced if gn["accepted_len"][b] == outs[c]["accepted_len"][b]
                and np.array_equal(gn["tokens"][b], outs[c]["tokens"][b])]
        nxt = oracle.advance_ref(outs[c]["tokens"], outs[c]["accepted_len"], outs[c]["x0"])
        assert np.array_equal(x0.cpu().numpy()[same], nxt[same])
        synced = same
    assert len(synced) >= w.cfg.B - 2
    total = sum((o["accepted_len"] + 1)[o["accepted_len"] >= 0].sum() for o in outs)
    print(f"emitted over {n_cycles} cycles: gpu {int(emitted.sum().item())}, oracle {int(total)}", flush=True)
