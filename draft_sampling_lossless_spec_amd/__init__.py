"""MI355X-native batched speculation cycle (DSpark-style confidence-scheduled speculative
decoding): a HIP library with a C ABI (include/spec_cycle.h) and this thin ctypes binding.

    from draft_sampling_lossless_spec_amd import spec_cycle, spec_workspace_bytes

Every step of the cycle runs in the library's gfx950 kernels; this package only marshals
device tensors into the C call.  It raises if the library has not been built
(``python -m draft_sampling_lossless_spec_amd.build``) -- there is no CPU fallback.
"""
from .binding import (  # noqa: F401
    BF16, CHUNKED, FLAT, FP32, PATH_AUTO, PATH_RESIDENT, PATH_STEPWISE, SpecError, spec_cycle_path, lib_path, spec_accept_stats, spec_advance, spec_calibration_error, spec_cycle,
    spec_cycle_lengths, spec_cycle_noalloc, SPEC_SCRATCH_BYTES,
    spec_cycle_kernel_count, spec_cycle_timed, spec_error_string, spec_schedule, spec_stats_workspace_bytes,
    spec_temperature_scaling, spec_version, spec_workspace_bytes,
)
