"""MI355X-native backward pass of top-k sparse flash attention (and the forward
pass that produces its out / softmaxMax / softmaxSum inputs).

The compute runs in libsfag (hand-written HIP kernels for gfx950, C ABI in
include/sfag.h); this package only marshals arguments to it.
"""
from ._binding import (BAD_INDEX_RANGE, BAD_LENGTH_NEGATIVE, BAD_LENGTH_SUM_KV, BAD_LENGTH_SUM_Q,  # noqa: F401
                       ERR_NULLPTR, ERR_PARAM_INVALID, ERR_RUNTIME, ERR_TILING, KERNEL_GROUPS, LIB_PATH, OK,
                       STATIC_SCRATCH_BYTES, SfagError, SfagRuntimeError, SfagValueError, backward,
                       backward_static, band_entries, band_indices, build_index, destroy, forward, lib,
                       make_options, plan, profile_enable, profile_read, profile_reset, validation_read,
                       workspace_size)
