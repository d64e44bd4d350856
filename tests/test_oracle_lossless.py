"""Statistical and brute-force pins for the oracle's cycle.

(a) per-position acceptance = 1 - TV(p, q) (Monte Carlo) and E[accepted | L] in closed form;
(b) losslessness on a brute-force instance: V=8, K=3, target logits a lookup table over every
    prefix, Markov bias active -- the exact distribution of what one cycle emits, continued by
    target draws, equals the target's autoregressive distribution, and the oracle's hashed
    samplers reproduce that exact emission distribution (chi-square over many request ids);
plus the Gumbel-max samplers against softmax and the special cases that reduce to textbook
sampling.  The exact enumeration below is an independent statement of the rejection-sampling
mathematics ("DSpark turns speculation into a scheduler", opening section: accept, or reject at
the first bad position and sample a correction from the target; "The Speed Claim Nobody's Really
Questioning", section "Speculative Decoding in Two Sentences": accept the longest valid prefix
and append one bonus token; with this accept/reject rule the emitted tokens follow the target's own distribution)."""
import itertools
import math
from collections import Counter

import numpy as np
import pytest
from scipy import stats

import oracle

V8, K3 = 8, 3


def softmax(x):
    x = np.asarray(x, dtype=np.float64)
    m = x.max()
    e = np.exp(x - m)
    return e / e.sum()


def prefix_rows(V, K):
    return sum(V ** n for n in range(K + 1))


def pooled_chisquare(observed: dict, expected_p: dict, n: int):
    """chi-square of observed counts against expected probabilities, pooling cells with
    expected count < 5 into one cell; returns the p-value."""
    obs, exp_ = [], []
    pool_o, pool_e = 0.0, 0.0
    for key, p in expected_p.items():
        e = p * n
        o = observed.get(key, 0)
        if e < 5:
            pool_o += o
            pool_e += e
        else:
            obs.append(o)
            exp_.append(e)
    extra = sum(v for k, v in observed.items() if k not in expected_p)
    assert extra == 0, f"{extra} draws landed on zero-probability outcomes"
    if pool_e > 0:
        obs.append(pool_o)
        exp_.append(pool_e)
    obs = np.array(obs, dtype=np.float64)
    exp_ = np.array(exp_, dtype=np.float64)
    exp_ *= obs.sum() / exp_.sum()
    return stats.chisquare(obs, exp_).pvalue


@pytest.mark.parametrize("noise", [oracle.FLAT, oracle.CHUNKED])
@pytest.mark.parametrize("V,T", [(8, 1.0), (200, 1.0), (200, 0.6)])
def test_gumbel_max_draws_follow_softmax(noise, V, T):
    # L = 0 (every confidence 0): the cycle emits one bonus draw from p = softmax(target row/T)
    rng = np.random.default_rng(V * 10 + noise)
    K = 1
    table = (rng.standard_normal((prefix_rows(V, K), V)) * 1.5).astype(np.float32)
    base = rng.standard_normal((K, V)).astype(np.float32)
    A = np.zeros((V, 4), np.float32)
    W = np.zeros((V, 4), np.float32)
    n = 200_000
    r = oracle.spec_cycle_ref_mc(base, table, A, W, -1, np.zeros(K, np.float32), T, 0.5, seed=77,
                                 n_trials=n, noise=noise)
    assert np.all(r["accepted_len"] == 0) and np.all(r["verify_len"] == 0)
    assert np.all(r["final_kind"] == 1)
    p = softmax(table[0] / T)
    obs = Counter(r["tokens"][:, 0].tolist())
    assert pooled_chisquare(obs, {v: p[v] for v in range(V)}, n) > 1e-5


def tiny_instance(seed, markov=True, T=1.0):
    rng = np.random.default_rng(seed)
    table = (rng.standard_normal((prefix_rows(V8, K3), V8)) * 1.3).astype(np.float32)
    base = (rng.standard_normal((K3, V8)) * 1.3).astype(np.float32)
    R = 4
    if markov:
        A = rng.standard_normal((V8, R)).astype(np.float32)
        W = rng.standard_normal((V8, R)).astype(np.float32) * np.float32(0.7)
    else:
        A = np.zeros((V8, R), np.float32)
        W = np.zeros((V8, R), np.float32)
    x0 = 3
    return table, base, A, W, x0, T


def exact_emission(table, base, A, W, x0, T, L):
    """Exact distribution of (accepted_len a, emitted tokens) for verify length L, by
    enumerating every draft path.  q_j(.|prev) = softmax((base_j + A[prev] W^T)/T),
    p(.|prefix) = softmax(table[prefix]/T)."""
    V = table.shape[1]
    A64, W64 = A.astype(np.float64), W.astype(np.float64)

    def q(j, prev):
        bias = W64 @ A64[prev] if prev >= 0 else np.zeros(V)
        return softmax((base[j].astype(np.float64) + bias) / T)

    def p(prefix):
        return softmax(table[oracle.table_index(prefix, V)].astype(np.float64) / T)

    out = Counter()
    for xs in itertools.product(range(V), repeat=L):
        # probability of this draft path
        Q = 1.0
        qs = []
        prev = x0
        for j, x in enumerate(xs):
            qj = q(j, prev)
            qs.append(qj)
            Q *= qj[x]
            prev = x
        if Q == 0.0:
            continue
        surv = 1.0
        for j in range(L):
            pj = p(xs[:j])
            acc = min(1.0, pj[xs[j]] / qs[j][xs[j]])
            rej = surv * (1.0 - acc)
            if rej > 0:
                res = np.maximum(pj - qs[j], 0.0)
                res = res / res.sum() if res.sum() > 0 else pj
                for y in range(V):
                    if res[y] > 0:
                        out[(j, xs[:j] + (y,))] += Q * rej * res[y]
            surv *= acc
        pb = p(xs)
        for y in range(V):
            out[(L, xs + (y,))] += Q * surv * pb[y]
    return out


@pytest.mark.parametrize("L", [0, 1, 2, 3])
def test_exact_emission_is_lossless(L):
    # the enumerated emission distribution continued by target draws is the target's
    # autoregressive distribution over sequences of length L + 1
    table, base, A, W, x0, T = tiny_instance(1, T=0.8)
    em = exact_emission(table, base, A, W, x0, T, L)
    assert abs(sum(em.values()) - 1.0) < 1e-12

    def p(prefix):
        return softmax(table[oracle.table_index(prefix, V8)].astype(np.float64) / T)

    for z in itertools.product(range(V8), repeat=L + 1):
        target = 1.0
        for i in range(L + 1):
            target *= p(z[:i])[z[i]]
        got = 0.0
        for a in range(L + 1):
            e = em.get((a, z[:a + 1]), 0.0)
            if e:
                cont = 1.0
                for i in range(a + 1, L + 1):
                    cont *= p(z[:i])[z[i]]
                got += e * cont
        assert abs(got - target) < 1e-12


def _conf_for(L, K):
    # confidences 1 for the first L positions then 0; threshold 0.5 cuts at exactly L
    return np.array([1.0] * L + [0.0] * (K - L), np.float32)


@pytest.mark.parametrize("noise", [oracle.FLAT, oracle.CHUNKED])
@pytest.mark.parametrize("L", [0, 1, 2, 3])
def test_oracle_emission_matches_exact_distribution(noise, L):
    table, base, A, W, x0, T = tiny_instance(1, T=0.8)
    em = exact_emission(table, base, A, W, x0, T, L)
    n = 400_000
    r = oracle.spec_cycle_ref_mc(base, table, A, W, x0, _conf_for(L, K3), T, 0.5, seed=2024 + L,
                                 n_trials=n, noise=noise)
    assert np.all(r["verify_len"] == L)
    a = r["accepted_len"]
    toks = r["tokens"]
    obs = Counter((int(a[i]), tuple(toks[i, :a[i] + 1].tolist())) for i in range(n))
    assert pooled_chisquare(obs, dict(em), n) > 1e-5


@pytest.mark.parametrize("noise", [oracle.FLAT, oracle.CHUNKED])
def test_acceptance_rate_is_one_minus_tv(noise):
    # check (a): P(accept at position 0) = sum_v min(p_0, q_0) = 1 - TV(p_0, q_0)
    table, base, A, W, x0, T = tiny_instance(4, T=1.0)
    L = 1
    n = 400_000
    r = oracle.spec_cycle_ref_mc(base, table, A, W, x0, _conf_for(L, K3), T, 0.5, seed=99,
                                 n_trials=n, noise=noise)
    q0 = softmax((base[0].astype(np.float64) + W.astype(np.float64) @ A[x0].astype(np.float64)) / T)
    p0 = softmax(table[0].astype(np.float64) / T)
    alpha = np.minimum(p0, q0).sum()
    assert abs(alpha - (1 - 0.5 * np.abs(p0 - q0).sum())) < 1e-12
    rate = (r["accepted_len"] == 1).mean()
    se = math.sqrt(alpha * (1 - alpha) / n)
    assert abs(rate - alpha) < 4 * se


def test_expected_accepted_length_closed_form():
    # with no Markov bias and a prefix-independent target, positions are independent:
    # E[a | L] = sum_{k=1..L} prod_{i<k} alpha_i, alpha_i = 1 - TV(p_i, q_i)
    rng = np.random.default_rng(8)
    table = np.empty((prefix_rows(V8, K3), V8), np.float32)
    rows = (rng.standard_normal((K3 + 1, V8)) * 1.2).astype(np.float32)
    for n in range(K3 + 1):
        for pre in itertools.product(range(V8), repeat=n):
            table[oracle.table_index(pre, V8)] = rows[n]
    base = (rows[:K3] + rng.standard_normal((K3, V8)).astype(np.float32) * 0.7).astype(np.float32)
    A = np.zeros((V8, 4), np.float32)
    W = np.zeros((V8, 4), np.float32)
    alphas = [np.minimum(softmax(rows[i]), softmax(base[i])).sum() for i in range(K3)]
    want = sum(np.prod(alphas[:k]) for k in range(1, K3 + 1))
    n = 400_000
    r = oracle.spec_cycle_ref_mc(base, table, A, W, 5, np.ones(K3, np.float32), 1.0, 0.5, seed=5,
                                 n_trials=n, noise=oracle.CHUNKED)
    a = r["accepted_len"].astype(np.float64)
    assert abs(a.mean() - want) < 4 * a.std() / math.sqrt(n)


@pytest.mark.parametrize("noise", [oracle.FLAT, oracle.CHUNKED])
def test_identical_draft_and_target_accept_everything(noise):
    # base = target and no Markov bias: p/q = 1 exactly, so every verified draft is accepted
    rng = np.random.default_rng(3)
    V, K = 300, 4
    rows = (rng.standard_normal((K + 1, V)) * 2).astype(np.float32)
    table = np.empty((1, V), np.float32)   # unused rows are never read for this check
    B = 64
    base = np.broadcast_to(rows[:K], (B, K, V)).copy()
    target = np.broadcast_to(rows, (B, K + 1, V)).copy()
    A = np.zeros((V, 8), np.float32)
    W = np.zeros((V, 8), np.float32)
    conf = rng.uniform(0.6, 1.0, size=(B, K)).astype(np.float32)
    r = oracle.spec_cycle_ref(base, target, A, W, None, conf, np.full(B, 0.9, np.float32), 0.3, 11,
                              noise=noise)
    assert np.all(r["accepted_len"] == r["verify_len"])
    assert np.all(r["final_kind"] == 1)
    del table


@pytest.mark.parametrize("noise", [oracle.FLAT, oracle.CHUNKED])
def test_one_hot_target_emits_only_its_token(noise):
    V, K, B = 130, 3, 200
    rng = np.random.default_rng(6)
    target = np.full((B, K + 1, V), -np.inf, np.float32)
    target[:, :, 77] = 0.0
    base = rng.standard_normal((B, K, V)).astype(np.float32)
    base[:, :, 77] += 2.0
    A = np.zeros((V, 4), np.float32)
    W = np.zeros((V, 4), np.float32)
    conf = np.ones((B, K), np.float32)
    r = oracle.spec_cycle_ref(base, target, A, W, None, conf, np.ones(B, np.float32), 0.5, 3, noise=noise)
    for b in range(B):
        a = r["accepted_len"][b]
        assert np.all(r["tokens"][b, :a + 1] == 77)
        assert np.all(r["tokens"][b, a + 1:] == -1)


@pytest.mark.parametrize("noise", [oracle.FLAT, oracle.CHUNKED])
def test_draft_on_a_zero_probability_token_is_always_rejected(noise):
    # draft puts all mass on token 4, which the target forbids: reject at position 0, and the
    # correction is a draw from norm(max(0, p - q)) = p
    V, K = 8, 2
    rng = np.random.default_rng(12)
    trow = (rng.standard_normal(V) * 1.0).astype(np.float32)
    trow[4] = -np.inf
    table = np.tile(trow, (prefix_rows(V, K), 1)).astype(np.float32)
    base = np.full((K, V), -np.inf, np.float32)
    base[:, 4] = 0.0
    A = np.zeros((V, 4), np.float32)
    W = np.zeros((V, 4), np.float32)
    n = 100_000
    r = oracle.spec_cycle_ref_mc(base, table, A, W, -1, np.ones(K, np.float32), 1.0, 0.5, seed=4,
                                 n_trials=n, noise=noise)
    assert np.all(r["accepted_len"] == 0)
    assert np.all(r["final_kind"] == 0)
    p = softmax(trow)
    obs = Counter(r["tokens"][:, 0].tolist())
    assert obs.get(4, 0) == 0
    assert pooled_chisquare(obs, {v: p[v] for v in range(V) if p[v] > 0}, n) > 1e-5
