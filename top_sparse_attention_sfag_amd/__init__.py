"""MI355X-native backward pass of top-k sparse flash attention (and the forward
pass that produces its out / softmaxMax / softmaxSum inputs).

The compute runs in libsfag (hand-written HIP kernels for gfx950, C ABI in
include/sfag.h); this package only marshals arguments to it.
"""
from ._binding import (ERR_NULLPTR, ERR_PARAM_INVALID, ERR_RUNTIME, ERR_TILING, LIB_PATH, OK,  # noqa: F401
                       KERNEL_GROUPS, SfagError, SfagRuntimeError, SfagValueError, backward, band_entries, band_indices,
                       build_index, destroy, forward,
                       lib,
                       plan, profile_enable, profile_read, profile_reset, workspace_size)
