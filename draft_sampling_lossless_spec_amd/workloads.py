"""Seeded synthetic inputs for the speculation cycle.

This module only draws inputs: it holds none of the cycle's arithmetic and imports neither the
oracle nor the HIP library, so both sides can be fed the same arrays.

The pages measure on live DeepSeek-V4 traffic and on offline math / code / chat suites that are
not available here; these generators stand in for them with the shapes, value distributions and
structure of the workloads the pages discuss:

* ``tiny``       -- B=2, K=4, V=1024, R=32, fp32.  Target ~N(0,1) with +6 on one uniform token
                    per row; draft base = target + N(0,1); A, W ~ N(0, 0.05^2); conf ~ U(0.5, 1);
                    threshold 0.3; temperature 1.0.
* ``dspark5``    -- the shipped five-token block ("The Speed Claim Nobody's Really Questioning",
                    section "What the Numbers Actually Say"): B=64, K=5, V=151936, R=256, bf16.
                    Target ~N(0,1) with +8 on one favoured token per row; base = target + N(0,1);
                    A, W ~ N(0, 0.02^2); conf ~ Beta(8,2); threshold 0.2; temperature 1.0.
* ``longblock``  -- 16-position blocks (same page, section "The Semi-Autoregressive Trick": draft
                    length 4 -> 16): B=256, K=16, same generators, draft noise sigma rising
                    linearly from 0.5 at position 0 to 2.0 at position 15 (suffix decay);
                    conf ~ Beta(6,3); threshold 0.1; temperature 1.0.
* ``highconc``   -- high concurrency with a shrinking verify budget ("DSpark turns speculation
                    into a scheduler", section "Confidence is a serving primitive"): B=1024,
                    K=5, V=129280, sigma 1.0, conf ~ Beta(5,2), threshold in {0.05, 0.2, 0.5, 0.8},
                    temperature 0.6.
* ``mixed``      -- code-like / math-like / chat-like thirds (per-domain acceptance differences on
                    "The Speed Claim...", section "What the Numbers Actually Say"): B=512, K=16,
                    sigma 0.3 / 1.0 / 2.0 and conf ~ Beta(12,2) / Beta(6,2) / Beta(3,2) by third,
                    threshold 0.3, temperature 0.6 or 1.0 per request.

Every request has its own numpy PCG64 stream (SeedSequence([gen_seed, config id, 0, b])), so a
subset of requests can be regenerated bit-identically without drawing the whole batch; A and W
have streams of their own (one per block of 4096 vocabulary rows).  bf16 arrays are returned as uint16 bit patterns (round to nearest
even from the fp32 draw).  x0[b] (the last committed token) is uniform over the vocabulary.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

FP32, BF16 = 0, 1


@dataclass(frozen=True)
class Config:
    name: str
    cid: int
    B: int
    K: int
    V: int
    R: int
    dtype: int
    fav: float
    aw_sigma: float
    threshold: float
    temp: float | None                   # None: per request 0.6 / 1.0
    conf_kind: str                       # "uniform" or "beta"
    conf_params: tuple                   # (lo, hi) or per-third Beta a-values with b fixed
    sigma: tuple                         # per third (or one entry); "ramp" handled by sigma_ramp
    sigma_ramp: tuple | None = None      # (start, end) linear over positions
    thresholds: tuple = field(default_factory=tuple)


CONFIGS = {
    "tiny": Config("tiny", 0, B=2, K=4, V=1024, R=32, dtype=FP32, fav=6.0, aw_sigma=0.05,
                   threshold=0.3, temp=1.0, conf_kind="uniform", conf_params=(0.5, 1.0), sigma=(1.0,)),
    "dspark5": Config("dspark5", 1, B=64, K=5, V=151936, R=256, dtype=BF16, fav=8.0, aw_sigma=0.02,
                      threshold=0.2, temp=1.0, conf_kind="beta", conf_params=((8.0, 2.0),), sigma=(1.0,)),
    "longblock": Config("longblock", 2, B=256, K=16, V=151936, R=256, dtype=BF16, fav=8.0, aw_sigma=0.02,
                        threshold=0.1, temp=1.0, conf_kind="beta", conf_params=((6.0, 3.0),), sigma=(1.0,),
                        sigma_ramp=(0.5, 2.0)),
    "highconc": Config("highconc", 3, B=1024, K=5, V=129280, R=256, dtype=BF16, fav=8.0, aw_sigma=0.02,
                       threshold=0.2, temp=0.6, conf_kind="beta", conf_params=((5.0, 2.0),), sigma=(1.0,),
                       thresholds=(0.05, 0.2, 0.5, 0.8)),
    "mixed": Config("mixed", 4, B=512, K=16, V=151936, R=256, dtype=BF16, fav=8.0, aw_sigma=0.02,
                    threshold=0.3, temp=None, conf_kind="beta",
                    conf_params=((12.0, 2.0), (6.0, 2.0), (3.0, 2.0)), sigma=(0.3, 1.0, 2.0)),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs here are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    cfg: Config
    base: np.ndarray          # [B, K, V]   float32 or uint16 (bf16 bits)
    target: np.ndarray        # [B, K+1, V]
    A: np.ndarray             # [V, R]
    W: np.ndarray             # [V, R]  vocabulary-major: row v = column v of the R x V factor
    x0: np.ndarray            # [B] int32
    conf: np.ndarray          # [B, K] float32
    temp: np.ndarray          # [B] float32
    threshold: float
    seed: int                 # cycle seed (noise hash)
    request_ids: np.ndarray   # [B] which requests of the full batch these rows are

    @property
    def dims(self):
        c = self.cfg
        return dict(B=len(self.request_ids), K=c.K, V=c.V, R=c.R, dtype=c.dtype)


def _third(cfg: Config, b: int) -> int:
    if len(cfg.sigma) == 1:
        return 0
    per = -(-cfg.B // 3)
    return min(2, b // per)


def _request_rows(cfg: Config, gen_seed: int, b: int, V: int | None = None):
    """Draw one request's rows; returns (target [K+1,V] f32, base [K,V] f32, conf [K], x0, temp)."""
    V = cfg.V if V is None else V
    K = cfg.K
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([gen_seed, cfg.cid, 0, b])))
    target = rng.standard_normal((K + 1, V), dtype=np.float32)
    fav = rng.integers(0, V, size=K + 1)
    target[np.arange(K + 1), fav] += np.float32(cfg.fav)
    t = _third(cfg, b)
    if cfg.sigma_ramp is not None:
        s0, s1 = cfg.sigma_ramp
        sig = np.array([s0 + (s1 - s0) * j / max(K - 1, 1) for j in range(K)], dtype=np.float32)
    else:
        sig = np.full(K, cfg.sigma[t], dtype=np.float32)
    noise = rng.standard_normal((K, V), dtype=np.float32)
    base = target[:K] + sig[:, None] * noise
    if cfg.conf_kind == "uniform":
        lo, hi = cfg.conf_params
        conf = rng.uniform(lo, hi, size=K).astype(np.float32)
    else:
        a, bb = cfg.conf_params[t if len(cfg.conf_params) > 1 else 0]
        conf = rng.beta(a, bb, size=K).astype(np.float32)
    x0 = int(rng.integers(0, V))
    temp = cfg.temp if cfg.temp is not None else (0.6 if rng.random() < 0.5 else 1.0)
    return target, base, conf, x0, np.float32(temp)


FACTOR_BLOCK = 4096   # rows of A / W drawn from one stream


def markov_factors(cfg: Config, gen_seed: int, threads: int | None = None):
    """A [V,R], W [V,R] ~ N(0, aw_sigma^2) in the config dtype; every block of 4096 rows has its
    own stream (SeedSequence([gen_seed, config id, 1 for A / 2 for W, block]))."""
    out = []
    nblk = -(-cfg.V // FACTOR_BLOCK)
    for kind in (1, 2):
        m = np.empty((cfg.V, cfg.R), dtype=np.uint16 if cfg.dtype == BF16 else np.float32)

        def one(blk, kind=kind, m=m):
            lo, hi = blk * FACTOR_BLOCK, min(cfg.V, (blk + 1) * FACTOR_BLOCK)
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([gen_seed, cfg.cid, kind, blk])))
            x = rng.standard_normal((hi - lo, cfg.R), dtype=np.float32) * np.float32(cfg.aw_sigma)
            m[lo:hi] = to_bf16_bits(x) if cfg.dtype == BF16 else x

        nthreads = threads or min(16, os.cpu_count() or 1)
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(nblk)))
        out.append(m)
    return out[0], out[1]


def generate(name_or_cfg, gen_seed: int = 1, cycle_seed: int = 1, requests=None, threshold=None,
             threads: int | None = None, factors=None) -> Workload:
    """Generate a workload (all requests, or the listed request ids of the full batch)."""
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    ids = np.arange(cfg.B) if requests is None else np.asarray(requests, dtype=np.int64)
    n = len(ids)
    K, V = cfg.K, cfg.V
    edt = np.uint16 if cfg.dtype == BF16 else np.float32
    base = np.empty((n, K, V), dtype=edt)
    target = np.empty((n, K + 1, V), dtype=edt)
    conf = np.empty((n, K), dtype=np.float32)
    x0 = np.empty(n, dtype=np.int32)
    temp = np.empty(n, dtype=np.float32)

    def one(i):
        t, b, c, x, tp = _request_rows(cfg, gen_seed, int(ids[i]))
        if cfg.dtype == BF16:
            target[i] = to_bf16_bits(t)
            base[i] = to_bf16_bits(b)
        else:
            target[i] = t
            base[i] = b
        conf[i] = c
        x0[i] = x
        temp[i] = tp

    nthreads = threads or min(16, os.cpu_count() or 1)
    if n > 1 and nthreads > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, range(n)))
    else:
        for i in range(n):
            one(i)
    A, W = factors if factors is not None else markov_factors(cfg, gen_seed)
    thr = cfg.threshold if threshold is None else float(threshold)
    return Workload(cfg, base, target, A, W, x0, conf, temp, thr, cycle_seed, ids)


def small_config(name: str = "small", B=3, K=4, V=333, R=32, dtype=BF16, **kw) -> Config:
    """A reduced config with the generators of ``dspark5`` (ragged V, several tiles) for tests."""
    base = dict(name=name, cid=100, B=B, K=K, V=V, R=R, dtype=dtype, fav=8.0, aw_sigma=0.02,
                threshold=0.2, temp=1.0, conf_kind="beta", conf_params=((8.0, 2.0),), sigma=(1.0,))
    base.update(kw)
    return Config(**base)
