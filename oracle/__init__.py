"""fp64 CPU oracle for the speculation cycle -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product path (the HIP library and its binding) never touches it.

This module is a ctypes loader around ``liboracle.so`` (built from ``spec_oracle.c`` by
``oracle/build.py``): argument marshalling from numpy arrays.  Every arithmetic step of the cycle
and of the statistics lives in the C file, which cites the passages of the DSpark pages it
follows.  Three small pieces are Python here: ``temperature_grid`` (the candidate temperatures,
powers of two on an even grid), ``advance_ref`` (the next cycle's context: the last token a
request emitted) and ``decode_ref`` (the loop that chains oracle cycles with them).
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SPEC_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

FLAT, CHUNKED = 0, 1
FP32, BF16 = 0, 1
STREAMS = {"DRAFT": 1, "ACCEPT": 2, "RESIDUAL": 3, "BONUS": 4,
           "DRAFT_C": 5, "RESIDUAL_C": 7, "BONUS_C": 8}
CHUNK = 64


class Dims(C.Structure):
    _fields_ = [("B", C.c_int32), ("K", C.c_int32), ("V", C.c_int32), ("R", C.c_int32),
                ("dtype", C.c_int32), ("noise", C.c_int32)]


_OUT_FIELDS = [
    ("accepted_len", C.c_int32, "B"), ("tokens", C.c_int32, "BK1"), ("verify_len", C.c_int32, "B"),
    ("draft_tokens", C.c_int32, "BK"), ("final_kind", C.c_int32, "B"),
    ("logq", C.c_double, "BK"), ("logp", C.c_double, "BK"), ("lse_q", C.c_double, "BK"),
    ("lse_p", C.c_double, "BK1"), ("u", C.c_double, "BK"), ("ratio", C.c_double, "BK"),
    ("draft_margin1", C.c_double, "BK"), ("draft_margin2", C.c_double, "BK"),
    ("final_margin1", C.c_double, "B"), ("final_margin2", C.c_double, "B"),
]


class Out(C.Structure):
    _fields_ = [(name, C.POINTER(ct)) for name, ct, _ in _OUT_FIELDS]


_lib = None


def load(build_if_missing: bool = True) -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise FileNotFoundError(LIB_PATH)
        from oracle import build as _b
        _b.build()
    lib = C.CDLL(LIB_PATH)
    lib.oracle_splitmix64_next.restype = C.c_uint64
    lib.oracle_splitmix64_next.argtypes = [C.POINTER(C.c_uint64)]
    lib.oracle_rowkey.restype = C.c_uint64
    lib.oracle_rowkey.argtypes = [C.c_uint64] * 4
    lib.oracle_bits32.restype = C.c_uint32
    lib.oracle_bits32.argtypes = [C.c_uint64, C.c_uint64]
    lib.oracle_uniform.restype = C.c_double
    lib.oracle_uniform.argtypes = [C.c_uint64, C.c_uint64]
    lib.oracle_gumbel.restype = C.c_double
    lib.oracle_gumbel.argtypes = [C.c_uint64, C.c_uint64]
    lib.oracle_lse.restype = C.c_double
    lib.oracle_lse.argtypes = [C.c_void_p, C.c_int64]
    lib.oracle_cut.restype = C.c_int32
    lib.oracle_cut.argtypes = [C.c_void_p, C.c_int32, C.c_float]
    lib.oracle_bias.restype = None
    lib.oracle_bias.argtypes = [C.c_void_p, C.c_void_p, C.c_int, C.c_int32, C.c_int32, C.c_int32, C.c_void_p]
    lib.oracle_max_threads.restype = C.c_int
    lib.oracle_max_threads.argtypes = []
    common = [C.POINTER(Dims), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    for fn in (lib.spec_cycle_ref, lib.spec_cycle_ref_table):
        fn.restype = C.c_int
        fn.argtypes = common + [C.c_void_p, C.c_void_p, C.c_void_p, C.c_float, C.c_uint64, C.c_int64,
                                C.POINTER(Out), C.c_int]
    lib.spec_cycle_ref_lengths.restype = C.c_int
    lib.spec_cycle_ref_lengths.argtypes = common + [C.c_void_p, C.c_void_p, C.c_void_p, C.c_uint64, C.c_int64,
                                                    C.POINTER(Out), C.c_int]
    lib.spec_cycle_ref_mc.restype = C.c_int
    lib.spec_cycle_ref_mc.argtypes = common + [C.c_int32, C.c_void_p, C.c_float, C.c_float, C.c_uint64,
                                               C.c_int64, C.c_int64, C.POINTER(Out), C.c_int]
    lib.spec_accept_stats_ref.restype = C.c_int
    lib.spec_accept_stats_ref.argtypes = common + [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                                   C.c_void_p, C.c_int]
    lib.spec_calibration_error_ref.restype = C.c_double
    lib.spec_calibration_error_ref.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                               C.POINTER(C.c_int64)]
    lib.spec_temperature_scaling_ref.restype = C.c_int
    lib.spec_temperature_scaling_ref.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p,
                                                 C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.spec_schedule_ref.restype = C.c_int
    lib.spec_schedule_ref.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]
    _lib = lib
    return lib


# ----------------------------------------------------------------------------------------
# scalar helpers (used by the pins)
# ----------------------------------------------------------------------------------------
def splitmix64_outputs(state: int, n: int) -> list[int]:
    lib = load()
    s = C.c_uint64(state)
    return [int(lib.oracle_splitmix64_next(C.byref(s))) for _ in range(n)]


def rowkey(seed: int, request: int, pos: int, stream: int) -> int:
    m = (1 << 64) - 1
    return int(load().oracle_rowkey(seed & m, request & m, pos & m, stream & m))


def bits32(key: int, i: int) -> int:
    return int(load().oracle_bits32(key, i))


def uniform(key: int, i: int) -> float:
    return float(load().oracle_uniform(key, i))


def gumbel(key: int, i: int) -> float:
    return float(load().oracle_gumbel(key, i))


def lse(x: np.ndarray) -> float:
    x = np.ascontiguousarray(x, dtype=np.float64)
    return float(load().oracle_lse(x.ctypes.data, x.size))


def cut(conf, threshold: float) -> int:
    c = np.ascontiguousarray(conf, dtype=np.float32)
    return int(load().oracle_cut(c.ctypes.data, c.size, C.c_float(threshold)))


def bias(A: np.ndarray, W: np.ndarray, prev: int) -> np.ndarray:
    dt = _dtype_code(A)
    V, R = A.shape
    out = np.empty(V, dtype=np.float64)
    Ac, Wc = np.ascontiguousarray(A), np.ascontiguousarray(W)
    load().oracle_bias(Ac.ctypes.data, Wc.ctypes.data, dt, V, R, prev, out.ctypes.data)
    return out


def max_threads() -> int:
    return int(load().oracle_max_threads())


# ----------------------------------------------------------------------------------------
# the cycle
# ----------------------------------------------------------------------------------------
def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return FP32
    if a.dtype == np.uint16:   # bf16 bit patterns
        return BF16
    raise TypeError(f"oracle inputs must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _alloc_out(B: int, K: int):
    arrays = {}
    kw = {}
    for name, ct, shape in _OUT_FIELDS:
        shp = {"B": (B,), "BK": (B, K), "BK1": (B, K + 1)}[shape]
        a = np.empty(shp, dtype=np.int32 if ct is C.c_int32 else np.float64)
        arrays[name] = a
        kw[name] = a.ctypes.data_as(C.POINTER(ct))
    return arrays, Out(**kw)


def spec_cycle_ref(base, target, A, W, x0, conf, temp, threshold, seed, noise=CHUNKED,
                   request_offset=0, nthreads=0, target_is_table=False) -> dict:
    """Run the oracle cycle.  base [B,K,V], target [B,K+1,V] (or a prefix table when
    target_is_table), A [V,R], W [V,R] as float32 or uint16 bf16 bits; x0 [B] int32 or None;
    conf [B,K] float32; temp [B] float32.  Returns a dict of numpy arrays."""
    lib = load()
    dt = _dtype_code(base)
    B, K, V = base.shape
    R = A.shape[1]
    for a in (target, A, W):
        if _dtype_code(a) != dt:
            raise TypeError("all logit / factor arrays must share one dtype")
    base = np.ascontiguousarray(base)
    target = np.ascontiguousarray(target)
    A = np.ascontiguousarray(A)
    W = np.ascontiguousarray(W)
    conf = np.ascontiguousarray(conf, dtype=np.float32).reshape(B, K)
    temp = np.ascontiguousarray(temp, dtype=np.float32).reshape(B)
    x0p = None
    if x0 is not None:
        x0 = np.ascontiguousarray(x0, dtype=np.int32).reshape(B)
        x0p = x0.ctypes.data
    d = Dims(B, K, V, R, dt, noise)
    arrays, out = _alloc_out(B, K)
    fn = lib.spec_cycle_ref_table if target_is_table else lib.spec_cycle_ref
    rc = fn(C.byref(d), base.ctypes.data, target.ctypes.data, A.ctypes.data, W.ctypes.data, x0p,
            conf.ctypes.data, temp.ctypes.data, C.c_float(threshold), C.c_uint64(seed),
            C.c_int64(request_offset), C.byref(out), nthreads)
    if rc != 0:
        raise ValueError(f"spec_cycle_ref rejected its arguments (code {rc})")
    return arrays


def spec_cycle_ref_lengths(base, target, A, W, x0, verify_len, temp, seed, noise=CHUNKED, request_offset=0,
                           nthreads=0) -> dict:
    """The oracle cycle with given verify lengths [B] (0..K; others mark the request invalid)
    instead of the prefix cut."""
    lib = load()
    dt = _dtype_code(base)
    B, K, V = base.shape
    R = A.shape[1]
    base, target, A, W = (np.ascontiguousarray(a) for a in (base, target, A, W))
    L = np.ascontiguousarray(verify_len, dtype=np.int32).reshape(B)
    temp = np.ascontiguousarray(temp, dtype=np.float32).reshape(B)
    x0p = None
    if x0 is not None:
        x0 = np.ascontiguousarray(x0, dtype=np.int32).reshape(B)
        x0p = x0.ctypes.data
    d = Dims(B, K, V, R, dt, noise)
    arrays, out = _alloc_out(B, K)
    rc = lib.spec_cycle_ref_lengths(C.byref(d), base.ctypes.data, target.ctypes.data, A.ctypes.data, W.ctypes.data,
                                    x0p, L.ctypes.data, temp.ctypes.data, C.c_uint64(seed),
                                    C.c_int64(request_offset), C.byref(out), nthreads)
    if rc != 0:
        raise ValueError(f"spec_cycle_ref_lengths rejected its arguments (code {rc})")
    return arrays


def spec_cycle_ref_mc(base, target_table, A, W, x0, conf, temp, threshold, seed, n_trials,
                      noise=CHUNKED, request_offset=0, nthreads=0) -> dict:
    """One request's inputs (base [K,V], prefix table target) repeated over n_trials request
    ids; returns per-trial outputs."""
    lib = load()
    dt = _dtype_code(base)
    K, V = base.shape
    R = A.shape[1]
    base = np.ascontiguousarray(base)
    target_table = np.ascontiguousarray(target_table)
    A = np.ascontiguousarray(A)
    W = np.ascontiguousarray(W)
    conf = np.ascontiguousarray(conf, dtype=np.float32).reshape(K)
    d = Dims(1, K, V, R, dt, noise)
    arrays, out = _alloc_out(int(n_trials), K)
    rc = lib.spec_cycle_ref_mc(C.byref(d), base.ctypes.data, target_table.ctypes.data, A.ctypes.data,
                               W.ctypes.data, C.c_int32(x0), conf.ctypes.data, C.c_float(temp),
                               C.c_float(threshold), C.c_uint64(seed), C.c_int64(request_offset),
                               C.c_int64(n_trials), C.byref(out), nthreads)
    if rc != 0:
        raise ValueError(f"spec_cycle_ref_mc rejected its arguments (code {rc})")
    return arrays


def table_index(prefix, V: int) -> int:
    """Row of a prefix in the prefix table (layout defined in spec_oracle.c)."""
    n = len(prefix)
    off = (V ** n - 1) // (V - 1)
    idx = 0
    for y in prefix:
        idx = idx * V + int(y)
    return off + idx


# ----------------------------------------------------------------------------------------
# acceptance statistics
# ----------------------------------------------------------------------------------------
def accept_stats_ref(base, target, A, W, x0, draft_tokens, temp, nthreads=0) -> dict:
    """alpha [B,K] = sum_v min(p_j, q_j) = 1 - TV(p_j, q_j) at every drafted position (NaN
    elsewhere), with the two log-normalisers lse_q and lse_p [B,K]; fp64."""
    lib = load()
    dt = _dtype_code(base)
    B, K, V = base.shape
    R = A.shape[1]
    base, target, A, W = (np.ascontiguousarray(a) for a in (base, target, A, W))
    draft = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, K)
    temp = np.ascontiguousarray(temp, dtype=np.float32).reshape(B)
    x0p = None
    if x0 is not None:
        x0 = np.ascontiguousarray(x0, dtype=np.int32).reshape(B)
        x0p = x0.ctypes.data
    out = {k: np.empty((B, K), dtype=np.float64) for k in ("alpha", "lse_q", "lse_p")}
    d = Dims(B, K, V, R, dt, CHUNKED)
    rc = lib.spec_accept_stats_ref(C.byref(d), base.ctypes.data, target.ctypes.data, A.ctypes.data, W.ctypes.data,
                                   x0p, draft.ctypes.data, temp.ctypes.data, out["alpha"].ctypes.data,
                                   out["lse_q"].ctypes.data, out["lse_p"].ctypes.data, nthreads)
    if rc != 0:
        raise ValueError(f"spec_accept_stats_ref rejected its arguments (code {rc})")
    return out


def calibration_error_ref(conf, verify_len, accepted_len, nbins=10):
    """(ECE, number of pairs) of the confidences' prefix-survival product against realised
    survival over every verified position of every valid request."""
    lib = load()
    conf = np.ascontiguousarray(conf, dtype=np.float32)
    B, K = conf.shape
    L = np.ascontiguousarray(verify_len, dtype=np.int32).reshape(B)
    a = np.ascontiguousarray(accepted_len, dtype=np.int32).reshape(B)
    n = C.c_int64(0)
    e = lib.spec_calibration_error_ref(conf.ctypes.data, L.ctypes.data, a.ctypes.data, B, K, int(nbins), C.byref(n))
    return float(e), int(n.value)


# ----------------------------------------------------------------------------------------
# prefix scheduler
# ----------------------------------------------------------------------------------------
def schedule_ref(conf, step_time, nbins=4096) -> dict:
    """Hardware-aware prefix scheduler (definition in spec_oracle.c): per-request verify lengths
    maximising expected emitted tokens per second of target step time."""
    lib = load()
    conf = np.ascontiguousarray(conf, dtype=np.float32)
    B, K = conf.shape
    T = np.ascontiguousarray(step_time, dtype=np.float64)
    if T.shape != (B * K + 1,):
        raise ValueError(f"step_time must have B*K+1 = {B * K + 1} entries")
    L = np.empty(B, np.int32)
    out = np.empty(4, np.float64)
    rc = lib.spec_schedule_ref(conf.ctypes.data, B, K, T.ctypes.data, int(nbins), L.ctypes.data, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"spec_schedule_ref rejected its arguments (code {rc})")
    return {"verify_len": L, "threshold": float(out[0]), "n": int(out[1]), "expected_tokens": float(out[2]),
            "goodput": float(out[3])}


# ----------------------------------------------------------------------------------------
# sequential temperature scaling
# ----------------------------------------------------------------------------------------
def temperature_grid(steps_per_octave=12, lo_octaves=-2, hi_octaves=3) -> np.ndarray:
    """ascending grid T = 2^(m / steps_per_octave), m from lo_octaves to hi_octaves octaves: it holds
    T = 1 exactly and doubling T moves exactly steps_per_octave entries"""
    m = np.arange(lo_octaves * steps_per_octave, hi_octaves * steps_per_octave + 1)
    return np.exp2(m / steps_per_octave)


def temperature_scaling_ref(z, verify_len, accepted_len, grid, nbins=10) -> dict:
    """Left-to-right per-position temperatures of the confidence logits z [N,K] minimising the
    calibration error of the cumulative prefix probability (definition in spec_oracle.c)."""
    lib = load()
    z = np.ascontiguousarray(z, dtype=np.float32)
    N, K = z.shape
    L = np.ascontiguousarray(verify_len, dtype=np.int32).reshape(N)
    a = np.ascontiguousarray(accepted_len, dtype=np.int32).reshape(N)
    g = np.ascontiguousarray(grid, dtype=np.float64)
    out = {k: np.empty(K, np.float64) for k in ("T", "ece_before", "ece_after")}
    rc = lib.spec_temperature_scaling_ref(z.ctypes.data, L.ctypes.data, a.ctypes.data, N, K, g.ctypes.data, len(g),
                                          int(nbins), out["T"].ctypes.data, out["ece_before"].ctypes.data,
                                          out["ece_after"].ctypes.data)
    if rc != 0:
        raise ValueError(f"spec_temperature_scaling_ref rejected its arguments (code {rc})")
    return out


# ----------------------------------------------------------------------------------------
# decode loop
# ----------------------------------------------------------------------------------------
def advance_ref(tokens, accepted_len, x0):
    """next context: the last token each valid request emitted (tokens[b, a_b]); invalid keep x0"""
    x = np.array(x0, dtype=np.int32, copy=True)
    for b, a in enumerate(accepted_len):
        if 0 <= a < tokens.shape[1]:
            x[b] = tokens[b, a]
    return x


def decode_ref(base_sets, target_sets, A, W, x0, conf_sets, temp, threshold, seed, n_cycles, noise=CHUNKED):
    """the oracle's decode loop: cycle c reads row set c % len(base_sets), seed + c, and the
    previous cycle's last emitted tokens as x0"""
    x = np.array(x0, dtype=np.int32, copy=True)
    outs = []
    for c in range(n_cycles):
        i = c % len(base_sets)
        r = spec_cycle_ref(base_sets[i], target_sets[i], A, W, x, conf_sets[i], temp, threshold, seed + c, noise=noise)
        r["x0"] = x.copy()
        outs.append(r)
        x = advance_ref(r["tokens"], r["accepted_len"], x)
    return outs
