"""Parity comparator between the HIP library and the fp64 oracle (test-side helper).

Rule (per request): tokens and accepted length must equal the oracle's, except where the first
decision at which the two runs part ways is a near-tie in the oracle's own trace -- an argmax whose
top-2 perturbed-score margin is below 1e-4 (either level of the CHUNKED sampler), or an accept
test with |u - p/q| below 1e-5.  Such a request is excused from that decision on.  Before that
point every sampled token's q and p must agree to 1e-4 relative: |exp(log_gpu - log_ref) - 1|.
Near-ties are counted over every decision the oracle takes and must stay below 0.1 %.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

ARGMAX_TIE = 1e-4
ACCEPT_TIE = 1e-5
PROB_TOL = 1e-4


@dataclass
class Report:
    requests: int = 0
    matched: int = 0
    excused: int = 0
    failures: list = field(default_factory=list)
    decisions: int = 0
    near_ties: int = 0
    prob_checks: int = 0
    max_prob_err: float = 0.0

    @property
    def near_tie_rate(self):
        return self.near_ties / max(1, self.decisions)

    def summary(self):
        return (f"requests={self.requests} matched={self.matched} excused={self.excused} "
                f"failures={len(self.failures)} decisions={self.decisions} near_ties={self.near_ties} "
                f"rate={self.near_tie_rate:.2e} prob_checks={self.prob_checks} max_prob_err={self.max_prob_err:.2e}")


def _tie(m1, m2):
    return (np.isfinite(m1) and m1 < ARGMAX_TIE) or (np.isfinite(m2) and m2 < ARGMAX_TIE)


def _prob_err(lg, lr):
    return abs(math.expm1(float(lg) - float(lr)))


def compare(orc: dict, gpu: dict, rows=None, report: Report | None = None) -> Report:
    """orc: oracle output dict; gpu: dict of numpy arrays (accepted_len, tokens, verify_len,
    draft_tokens, logq, logp) for the same requests in the same order."""
    rep = report or Report()
    B, K = orc["draft_tokens"].shape
    for b in range(B) if rows is None else rows:
        rep.requests += 1
        tag = f"request {b}"
        a_o, a_g = int(orc["accepted_len"][b]), int(gpu["accepted_len"][b])
        if a_o < 0:
            if a_g == -1 and np.all(gpu["tokens"][b] == -1):
                rep.matched += 1
            else:
                rep.failures.append(f"{tag}: oracle marks it invalid, gpu accepted_len={a_g}")
            continue
        L = int(orc["verify_len"][b])
        if int(gpu["verify_len"][b]) != L:
            rep.failures.append(f"{tag}: verify length {gpu['verify_len'][b]} != {L}")
            continue
        # decision counts and near-ties over the oracle's own trace
        m1, m2 = orc["draft_margin1"][b], orc["draft_margin2"][b]
        dec_acc = min(a_o + 1, L)
        rep.decisions += L + dec_acc + 1
        rep.near_ties += sum(bool(_tie(m1[j], m2[j])) for j in range(L))
        rep.near_ties += sum(bool(abs(orc["u"][b, j] - orc["ratio"][b, j]) < ACCEPT_TIE) for j in range(dec_acc))
        rep.near_ties += int(bool(_tie(orc["final_margin1"][b], orc["final_margin2"][b])))

        excused = False
        failed = None
        # draft decisions, in order
        for j in range(L):
            if gpu["draft_tokens"][b, j] != orc["draft_tokens"][b, j]:
                if _tie(m1[j], m2[j]):
                    excused = True
                else:
                    failed = (f"{tag}: draft x_{j} gpu={gpu['draft_tokens'][b, j]} oracle={orc['draft_tokens'][b, j]} "
                              f"margins={m1[j]:.3g},{m2[j]:.3g}")
                break
            e = _prob_err(gpu["logq"][b, j], orc["logq"][b, j])
            rep.prob_checks += 1
            rep.max_prob_err = max(rep.max_prob_err, e)
            if e > PROB_TOL:
                failed = f"{tag}: logq_{j} gpu={gpu['logq'][b, j]} oracle={orc['logq'][b, j]}"
                break
        if failed is None and not excused and np.any(gpu["draft_tokens"][b, L:] != -1):
            failed = f"{tag}: draft tokens beyond L are not -1"
        # accept decisions
        if failed is None and not excused:
            for j in range(dec_acc):
                acc_o, acc_g = j < a_o, j < a_g
                gdec = j <= a_g and j < L
                if gdec:
                    e = _prob_err(gpu["logp"][b, j], orc["logp"][b, j])
                    rep.prob_checks += 1
                    rep.max_prob_err = max(rep.max_prob_err, e)
                    if e > PROB_TOL:
                        failed = f"{tag}: logp_{j} gpu={gpu['logp'][b, j]} oracle={orc['logp'][b, j]}"
                        break
                if acc_o != acc_g:
                    if abs(orc["u"][b, j] - orc["ratio"][b, j]) < ACCEPT_TIE:
                        excused = True
                    else:
                        failed = (f"{tag}: accept at {j}: gpu={acc_g} oracle={acc_o} u={orc['u'][b, j]:.6g} "
                                  f"ratio={orc['ratio'][b, j]:.6g}")
                    break
        # final draw and token layout
        if failed is None and not excused:
            if a_g != a_o:
                failed = f"{tag}: accepted_len gpu={a_g} oracle={a_o}"
            elif gpu["tokens"][b, a_o] != orc["tokens"][b, a_o]:
                if _tie(orc["final_margin1"][b], orc["final_margin2"][b]):
                    excused = True
                else:
                    failed = (f"{tag}: final token gpu={gpu['tokens'][b, a_o]} oracle={orc['tokens'][b, a_o]} "
                              f"kind={orc['final_kind'][b]} margins={orc['final_margin1'][b]:.3g},"
                              f"{orc['final_margin2'][b]:.3g}")
            elif not np.array_equal(gpu["tokens"][b], orc["tokens"][b]):
                failed = f"{tag}: token rows differ: gpu={gpu['tokens'][b]} oracle={orc['tokens'][b]}"
        if failed is not None:
            rep.failures.append(failed)
        elif excused:
            rep.excused += 1
        else:
            rep.matched += 1
    return rep


def check_structure(w, gpu: dict, cut_fn) -> list:
    """Invariants that hold at any size: L from the fp64 cut, 0 <= a <= L, accepted tokens are the
    drafts, one emitted token after them, -1 padding."""
    errs = []
    B, K = w.conf.shape
    for b in range(B):
        a = int(gpu["accepted_len"][b])
        L = int(gpu["verify_len"][b])
        if a < 0:
            errs.append(f"request {b} unexpectedly invalid")
            continue
        if L != cut_fn(w.conf[b], w.threshold):
            errs.append(f"request {b}: L={L} != cut")
        if not 0 <= a <= L:
            errs.append(f"request {b}: a={a} L={L}")
            continue
        t = gpu["tokens"][b]
        d = gpu["draft_tokens"][b]
        if not (np.array_equal(t[:a], d[:a]) and 0 <= t[a] < w.cfg.V and np.all(t[a + 1:] == -1)):
            errs.append(f"request {b}: bad token row {t}")
        if not (np.all(d[:L] >= 0) and np.all(d[:L] < w.cfg.V) and np.all(d[L:] == -1)):
            errs.append(f"request {b}: bad draft row {d}")
        if not (np.all(np.isfinite(gpu["logq"][b, :L])) and np.all(gpu["logq"][b, :L] <= 1e-6)):
            errs.append(f"request {b}: bad logq")
    return errs
