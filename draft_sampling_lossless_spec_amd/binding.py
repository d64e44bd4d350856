"""ctypes binding of libspeccycle.so.  Argument marshalling only: shapes and dtypes of torch
device tensors are checked, pointers and the current HIP stream are passed to the C ABI
(include/spec_cycle.h), and the C return code is turned into an exception."""
from __future__ import annotations

import ctypes as C
import os

FP32, BF16 = 0, 1
FLAT, CHUNKED = 0, 1
PATH_AUTO, PATH_STEPWISE, PATH_RESIDENT = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libspeccycle.so")
_lib = None


class SpecError(RuntimeError):
    pass


class _Dims(C.Structure):
    _fields_ = [("B", C.c_int32), ("K", C.c_int32), ("V", C.c_int32), ("R", C.c_int32),
                ("dtype", C.c_int32), ("noise", C.c_int32), ("path", C.c_int32)]


class _Diag(C.Structure):
    _fields_ = [("verify_len", C.c_void_p), ("draft_tokens", C.c_void_p), ("logq", C.c_void_p),
                ("logp", C.c_void_p)]


def lib_path() -> str:
    return _LIB_PATH


def _held(stream, *tensors):
    """Tensors this binding allocated for a call enqueued on `stream`: the caching allocator must
    not hand their blocks to another stream's allocation while the call's kernels still use them,
    so every one is recorded as in use on `stream` (a no-op cost when it is the current stream)."""
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # torch ships a HIP runtime with the same soname; loading it first keeps one runtime per process
    import torch  # noqa: F401
    if not os.path.exists(_LIB_PATH):
        raise SpecError(f"{_LIB_PATH} is missing: build it with `python -m draft_sampling_lossless_spec_amd.build`")
    lib = C.CDLL(_LIB_PATH)
    lib.spec_workspace_bytes.restype = C.c_size_t
    lib.spec_workspace_bytes.argtypes = [C.POINTER(_Dims)]
    lib.spec_error_string.restype = C.c_char_p
    lib.spec_error_string.argtypes = [C.c_int]
    lib.spec_version.restype = C.c_int
    lib.spec_version.argtypes = []
    cycle_args = [C.POINTER(_Dims), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                  C.c_void_p, C.c_float, C.c_uint64, C.c_int64, C.c_void_p, C.c_void_p, C.POINTER(_Diag),
                  C.c_void_p, C.c_size_t, C.c_void_p]
    lib.spec_cycle.restype = C.c_int
    lib.spec_cycle.argtypes = cycle_args
    lib.spec_cycle_lengths.restype = C.c_int
    lib.spec_cycle_lengths.argtypes = [C.POINTER(_Dims), C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p, C.c_uint64, C.c_int64, C.c_void_p, C.c_void_p,
                                       C.POINTER(_Diag), C.c_void_p, C.c_size_t, C.c_void_p]
    lib.spec_cycle_noalloc.restype = C.c_int
    lib.spec_cycle_noalloc.argtypes = cycle_args[:14] + [C.c_void_p]
    lib.spec_cycle_timed.restype = C.c_int
    lib.spec_cycle_timed.argtypes = cycle_args + [C.c_void_p, C.c_int]
    lib.spec_cycle_kernel_count.restype = C.c_int
    lib.spec_cycle_kernel_count.argtypes = [C.POINTER(_Dims)]
    lib.spec_cycle_path.restype = C.c_int
    lib.spec_cycle_path.argtypes = [C.POINTER(_Dims)]
    lib.spec_stats_workspace_bytes.restype = C.c_size_t
    lib.spec_stats_workspace_bytes.argtypes = [C.POINTER(_Dims)]
    lib.spec_accept_stats.restype = C.c_int
    lib.spec_accept_stats.argtypes = [C.POINTER(_Dims)] + [C.c_void_p] * 10 + [C.c_void_p, C.c_size_t, C.c_void_p]
    lib.spec_temperature_scaling_workspace_bytes.restype = C.c_size_t
    lib.spec_temperature_scaling_workspace_bytes.argtypes = [C.c_int32, C.c_int32]
    lib.spec_temperature_scaling.restype = C.c_int
    lib.spec_temperature_scaling.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p,
                                             C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                             C.c_size_t, C.c_void_p]
    lib.spec_advance.restype = C.c_int
    lib.spec_advance.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p]
    lib.spec_schedule.restype = C.c_int
    lib.spec_schedule.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                  C.c_void_p]
    lib.spec_calibration_error.restype = C.c_int
    lib.spec_calibration_error.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32,
                                           C.c_void_p, C.c_void_p, C.c_void_p]
    _lib = lib
    return lib


def spec_version() -> int:
    return int(_load().spec_version())


def spec_error_string(code: int) -> str:
    return _load().spec_error_string(code).decode()


def spec_workspace_bytes(B: int, K: int, V: int, R: int, dtype: int = BF16, noise: int = CHUNKED,
                         path: int = PATH_AUTO) -> int:
    d = _Dims(B, K, V, R, dtype, noise, path)
    return int(_load().spec_workspace_bytes(C.byref(d)))


def spec_cycle_path(B: int, K: int, V: int, R: int, dtype: int = BF16, noise: int = CHUNKED,
                    path: int = PATH_AUTO) -> int:
    """The path (PATH_STEPWISE or PATH_RESIDENT) spec_cycle takes for these dims on the current
    device; raises on a negative code."""
    rc = int(_load().spec_cycle_path(C.byref(_Dims(B, K, V, R, dtype, noise, path))))
    if rc < 0:
        raise SpecError(f"spec_cycle_path: {spec_error_string(rc)} (code {rc})")
    return rc


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FP32
    if t.dtype == torch.bfloat16:
        return BF16
    raise SpecError(f"logits / factors must be float32 or bfloat16, got {t.dtype}")


def _check(t, name, shape, dtype=None):
    if not t.is_cuda:
        raise SpecError(f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise SpecError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise SpecError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise SpecError(f"{name} must be {dtype}, got {t.dtype}")


def spec_cycle_kernel_count(B: int, K: int, V: int, R: int, dtype: int = BF16, noise: int = CHUNKED,
                            path: int = PATH_AUTO) -> int:
    d = _Dims(B, K, V, R, dtype, noise, path)
    return int(_load().spec_cycle_kernel_count(C.byref(d)))


def spec_cycle_timed(*args, events, **kw) -> dict:
    """spec_cycle with a start/stop event pair on every kernel; `events` is a ctypes array of
    hipEvent_t handles (2 per kernel, see spec_cycle_kernel_count)."""
    return spec_cycle(*args, _events=events, **kw)


def spec_cycle(base_logits, target_logits, A, W, conf, temp, threshold: float, seed: int, x0=None,
               request_offset: int = 0, noise: int = CHUNKED, diag: bool = False, workspace=None,
               out=None, stream=None, path: int = PATH_AUTO, _events=None) -> dict:
    """Run one speculation cycle on the current HIP stream (or `stream`).  Returns a dict with
    'accepted_len' [B] and 'tokens' [B, K+1] (int32 device tensors) and, with diag=True,
    'verify_len', 'draft_tokens', 'logq', 'logp'.  `path` selects the execution path (PATH_AUTO,
    PATH_STEPWISE, PATH_RESIDENT; results are the same).  Asynchronous like the C call."""
    import torch
    B, K, V = base_logits.shape
    R = A.shape[1]
    dt = _dtype_code(base_logits)
    _check(base_logits, "base_logits", (B, K, V))
    _check(target_logits, "target_logits", (B, K + 1, V), base_logits.dtype)
    _check(A, "A", (V, R), base_logits.dtype)
    _check(W, "W", (V, R), base_logits.dtype)
    _check(conf, "conf", (B, K), torch.float32)
    _check(temp, "temp", (B,), torch.float32)
    if x0 is not None:
        _check(x0, "x0", (B,), torch.int32)
    dev = base_logits.device
    lib = _load()
    d = _Dims(B, K, V, R, dt, noise, path)
    need = int(lib.spec_workspace_bytes(C.byref(d)))
    if need == 0:
        raise SpecError(f"unsupported dimensions B={B} K={K} V={V} R={R} dtype={dt} noise={noise} path={path}")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    made = []
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        made.append(workspace)
    if out is None:
        out = {"accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
               "tokens": torch.empty((B, K + 1), dtype=torch.int32, device=dev)}
        made += [out["accepted_len"], out["tokens"]]
    dg = None
    if diag:
        for k, shp, ty in (("verify_len", (B,), torch.int32), ("draft_tokens", (B, K), torch.int32),
                           ("logq", (B, K), torch.float32), ("logp", (B, K), torch.float32)):
            if k not in out:
                out[k] = torch.empty(shp, dtype=ty, device=dev)
                made.append(out[k])
        dg = _Diag(out["verify_len"].data_ptr(), out["draft_tokens"].data_ptr(), out["logq"].data_ptr(),
                   out["logp"].data_ptr())
    _held(stream, *made)
    args = (C.byref(d), base_logits.data_ptr(), target_logits.data_ptr(), A.data_ptr(), W.data_ptr(),
            x0.data_ptr() if x0 is not None else None, conf.data_ptr(), temp.data_ptr(),
            C.c_float(threshold), C.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), C.c_int64(request_offset),
            out["accepted_len"].data_ptr(), out["tokens"].data_ptr(),
            C.byref(dg) if dg is not None else None, workspace.data_ptr(), workspace.numel(),
            C.c_void_p(stream.cuda_stream))
    if _events is None:
        rc = lib.spec_cycle(*args)
    else:
        rc = lib.spec_cycle_timed(*args, C.cast(_events, C.c_void_p), len(_events))
    if rc != 0:
        raise SpecError(f"spec_cycle failed: {spec_error_string(rc)} (code {rc})")
    return out


SPEC_SCRATCH_BYTES = 64 << 20


def spec_cycle_noalloc(base_logits, target_logits, A, W, conf, temp, threshold: float, seed: int, out: dict,
                       x0=None, request_offset: int = 0, noise: int = CHUNKED, stream=None,
                       path: int = PATH_AUTO) -> dict:
    """spec_cycle through the allocation-free entry point: the library's static per-GPU scratch
    array replaces the workspace, and the caller passes every output tensor in `out`
    ('accepted_len', 'tokens', and optionally 'verify_len', 'draft_tokens', 'logq', 'logp' for the
    diagnostics).  Neither this function nor the library allocates device memory.  Calls that
    overlap on one GPU race on the shared array."""
    import torch
    B, K, V = base_logits.shape
    R = A.shape[1]
    dt = _dtype_code(base_logits)
    _check(base_logits, "base_logits", (B, K, V))
    _check(target_logits, "target_logits", (B, K + 1, V), base_logits.dtype)
    _check(A, "A", (V, R), base_logits.dtype)
    _check(W, "W", (V, R), base_logits.dtype)
    _check(conf, "conf", (B, K), torch.float32)
    _check(temp, "temp", (B,), torch.float32)
    if x0 is not None:
        _check(x0, "x0", (B,), torch.int32)
    _check(out["accepted_len"], "accepted_len", (B,), torch.int32)
    _check(out["tokens"], "tokens", (B, K + 1), torch.int32)
    dg = None
    if "verify_len" in out:
        for k, shp, ty in (("verify_len", (B,), torch.int32), ("draft_tokens", (B, K), torch.int32),
                           ("logq", (B, K), torch.float32), ("logp", (B, K), torch.float32)):
            _check(out[k], k, shp, ty)
        dg = _Diag(out["verify_len"].data_ptr(), out["draft_tokens"].data_ptr(), out["logq"].data_ptr(),
                   out["logp"].data_ptr())
    lib = _load()
    d = _Dims(B, K, V, R, dt, noise, path)
    if stream is None:
        stream = torch.cuda.current_stream(base_logits.device)
    rc = lib.spec_cycle_noalloc(C.byref(d), base_logits.data_ptr(), target_logits.data_ptr(), A.data_ptr(),
                                W.data_ptr(), x0.data_ptr() if x0 is not None else None, conf.data_ptr(),
                                temp.data_ptr(), C.c_float(threshold), C.c_uint64(seed & 0xFFFFFFFFFFFFFFFF),
                                C.c_int64(request_offset), out["accepted_len"].data_ptr(), out["tokens"].data_ptr(),
                                C.byref(dg) if dg is not None else None, C.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise SpecError(f"spec_cycle_noalloc failed: {spec_error_string(rc)} (code {rc})")
    return out


def spec_stats_workspace_bytes(B: int, K: int, V: int, R: int, dtype: int = BF16) -> int:
    return int(_load().spec_stats_workspace_bytes(C.byref(_Dims(B, K, V, R, dtype, CHUNKED))))


def spec_accept_stats(base_logits, target_logits, A, W, draft_tokens, temp, x0=None, workspace=None,
                      out=None, stream=None, path: int = 0) -> dict:
    """Analytical acceptance rate alpha = sum_v min(p_j, q_j) = 1 - TV(p_j, q_j) of every drafted
    position (draft_tokens [B, K] int32, -1 past the drafted prefix, as the cycle's diagnostics
    give it), with the log-normalisers 'lse_q' and 'lse_p'; NaN elsewhere.  path: 0 picks (the
    W-resident kernel where the shape allows it), 1 the sweep kernels, 2 the W-resident kernel.
    Asynchronous."""
    import torch
    B, K, V = base_logits.shape
    R = A.shape[1]
    dt = _dtype_code(base_logits)
    _check(base_logits, "base_logits", (B, K, V))
    _check(target_logits, "target_logits", (B, K + 1, V), base_logits.dtype)
    _check(A, "A", (V, R), base_logits.dtype)
    _check(W, "W", (V, R), base_logits.dtype)
    _check(draft_tokens, "draft_tokens", (B, K), torch.int32)
    _check(temp, "temp", (B,), torch.float32)
    if x0 is not None:
        _check(x0, "x0", (B,), torch.int32)
    dev = base_logits.device
    lib = _load()
    d = _Dims(B, K, V, R, dt, CHUNKED, path)
    need = int(lib.spec_stats_workspace_bytes(C.byref(d)))
    if need == 0:
        raise SpecError(f"unsupported dimensions B={B} K={K} V={V} R={R} dtype={dt}")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _held(stream, workspace)
    if out is None:
        out = {k: torch.empty((B, K), dtype=torch.float32, device=dev) for k in ("alpha", "lse_q", "lse_p")}
        _held(stream, *out.values())
    rc = lib.spec_accept_stats(C.byref(d), base_logits.data_ptr(), target_logits.data_ptr(), A.data_ptr(),
                               W.data_ptr(), x0.data_ptr() if x0 is not None else None, draft_tokens.data_ptr(),
                               temp.data_ptr(), out["alpha"].data_ptr(),
                               out["lse_q"].data_ptr() if "lse_q" in out else None,
                               out["lse_p"].data_ptr() if "lse_p" in out else None,
                               workspace.data_ptr(), workspace.numel(), C.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise SpecError(f"spec_accept_stats failed: {spec_error_string(rc)} (code {rc})")
    return out


def spec_calibration_error(conf, verify_len, accepted_len, nbins: int = 10, stream=None):
    """Expected calibration error of the confidences' prefix-survival product against realised
    survival, and the number of (request, position) pairs; returns two device tensors (fp64 [1],
    int64 [1]).  Asynchronous."""
    import torch
    B, K = conf.shape
    _check(conf, "conf", (B, K), torch.float32)
    _check(verify_len, "verify_len", (B,), torch.int32)
    _check(accepted_len, "accepted_len", (B,), torch.int32)
    dev = conf.device
    ece = torch.empty(1, dtype=torch.float64, device=dev)
    n = torch.empty(1, dtype=torch.int64, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    _held(stream, ece, n)
    rc = _load().spec_calibration_error(conf.data_ptr(), verify_len.data_ptr(), accepted_len.data_ptr(), B, K,
                                        int(nbins), ece.data_ptr(), n.data_ptr(), C.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise SpecError(f"spec_calibration_error failed: {spec_error_string(rc)} (code {rc})")
    return ece, n


def spec_schedule(conf, step_time, nbins: int = 4096, verify_len=None, out=None, stream=None):
    """Hardware-aware prefix scheduler: per-request verify lengths ([B] int32 device tensor) and a
    [4] fp64 device tensor (threshold, kept positions, expected emitted tokens, goodput) for the
    confidences conf [B, K] fp32 and the target step-time curve step_time [B K + 1] fp64 (seconds
    per verification step with n draft tokens).  Asynchronous."""
    import torch
    B, K = conf.shape
    _check(conf, "conf", (B, K), torch.float32)
    _check(step_time, "step_time", (B * K + 1,), torch.float64)
    dev = conf.device
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if verify_len is None:
        verify_len = torch.empty(B, dtype=torch.int32, device=dev)
        _held(stream, verify_len)
    if out is None:
        out = torch.empty(4, dtype=torch.float64, device=dev)
        _held(stream, out)
    rc = _load().spec_schedule(conf.data_ptr(), B, K, step_time.data_ptr(), int(nbins), verify_len.data_ptr(),
                               out.data_ptr(), C.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise SpecError(f"spec_schedule failed: {spec_error_string(rc)} (code {rc})")
    return verify_len, out


def spec_cycle_lengths(base_logits, target_logits, A, W, verify_len, temp, seed: int, x0=None,
                       request_offset: int = 0, noise: int = CHUNKED, diag: bool = False, workspace=None,
                       out=None, stream=None, path: int = PATH_AUTO) -> dict:
    """One speculation cycle with per-request verify lengths (verify_len [B] int32 device tensor,
    e.g. from spec_schedule) in place of the prefix cut.  Returns what spec_cycle returns."""
    import torch
    B, K, V = base_logits.shape
    R = A.shape[1]
    dt = _dtype_code(base_logits)
    _check(base_logits, "base_logits", (B, K, V))
    _check(target_logits, "target_logits", (B, K + 1, V), base_logits.dtype)
    _check(A, "A", (V, R), base_logits.dtype)
    _check(W, "W", (V, R), base_logits.dtype)
    _check(verify_len, "verify_len", (B,), torch.int32)
    _check(temp, "temp", (B,), torch.float32)
    if x0 is not None:
        _check(x0, "x0", (B,), torch.int32)
    dev = base_logits.device
    lib = _load()
    d = _Dims(B, K, V, R, dt, noise, path)
    need = int(lib.spec_workspace_bytes(C.byref(d)))
    if need == 0:
        raise SpecError(f"unsupported dimensions B={B} K={K} V={V} R={R} dtype={dt} noise={noise} path={path}")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    made = []
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        made.append(workspace)
    if out is None:
        out = {"accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
               "tokens": torch.empty((B, K + 1), dtype=torch.int32, device=dev)}
        made += [out["accepted_len"], out["tokens"]]
    dg = None
    if diag:
        for k, shp, ty in (("verify_len", (B,), torch.int32), ("draft_tokens", (B, K), torch.int32),
                           ("logq", (B, K), torch.float32), ("logp", (B, K), torch.float32)):
            if k not in out:
                out[k] = torch.empty(shp, dtype=ty, device=dev)
                made.append(out[k])
        dg = _Diag(out["verify_len"].data_ptr(), out["draft_tokens"].data_ptr(), out["logq"].data_ptr(),
                   out["logp"].data_ptr())
    _held(stream, *made)
    rc = lib.spec_cycle_lengths(C.byref(d), base_logits.data_ptr(), target_logits.data_ptr(), A.data_ptr(),
                                W.data_ptr(), x0.data_ptr() if x0 is not None else None, verify_len.data_ptr(),
                                temp.data_ptr(), C.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), C.c_int64(request_offset),
                                out["accepted_len"].data_ptr(), out["tokens"].data_ptr(),
                                C.byref(dg) if dg is not None else None, workspace.data_ptr(), workspace.numel(),
                                C.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise SpecError(f"spec_cycle_lengths failed: {spec_error_string(rc)} (code {rc})")
    return out


def spec_temperature_scaling(z, verify_len, accepted_len, grid, nbins: int = 10, workspace=None, stream=None) -> dict:
    """Sequential temperature scaling: z [N, K] fp32 logits, verify_len / accepted_len [N] int32,
    grid [G] fp64 ascending temperatures (device tensors).  Returns device tensors 'T',
    'ece_before', 'ece_after' ([K] fp64).  Asynchronous."""
    import torch
    N, K = z.shape
    _check(z, "z", (N, K), torch.float32)
    _check(verify_len, "verify_len", (N,), torch.int32)
    _check(accepted_len, "accepted_len", (N,), torch.int32)
    G = grid.shape[0]
    _check(grid, "grid", (G,), torch.float64)
    dev = z.device
    lib = _load()
    need = int(lib.spec_temperature_scaling_workspace_bytes(N, G))
    if need == 0:
        raise SpecError(f"unsupported sizes N={N} G={G}")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _held(stream, workspace)
    out = {k: torch.empty(K, dtype=torch.float64, device=dev) for k in ("T", "ece_before", "ece_after")}
    _held(stream, *out.values())
    rc = lib.spec_temperature_scaling(z.data_ptr(), verify_len.data_ptr(), accepted_len.data_ptr(), N, K,
                                      grid.data_ptr(), G, int(nbins), out["T"].data_ptr(),
                                      out["ece_before"].data_ptr(), out["ece_after"].data_ptr(), workspace.data_ptr(),
                                      workspace.numel(), C.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise SpecError(f"spec_temperature_scaling failed: {spec_error_string(rc)} (code {rc})")
    return out


def spec_advance(tokens, accepted_len, x0, emitted=None, stream=None):
    """Next cycle's context in place: x0 [B] int32 <- the last token each valid request emitted;
    emitted [B] int64 (optional) += accepted_len + 1.  Asynchronous."""
    import torch
    B, K1 = tokens.shape
    _check(tokens, "tokens", (B, K1), torch.int32)
    _check(accepted_len, "accepted_len", (B,), torch.int32)
    _check(x0, "x0", (B,), torch.int32)
    if emitted is not None:
        _check(emitted, "emitted", (B,), torch.int64)
    if stream is None:
        stream = torch.cuda.current_stream(tokens.device)
    rc = _load().spec_advance(tokens.data_ptr(), accepted_len.data_ptr(), B, K1 - 1, x0.data_ptr(),
                              emitted.data_ptr() if emitted is not None else None, C.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise SpecError(f"spec_advance failed: {spec_error_string(rc)} (code {rc})")
