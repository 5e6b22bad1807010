"""MI355X-native verification step of lossless greedy speculative decoding.

The compute path is the C-ABI library libspec.so (hand-written gfx950 HIP
kernels); this package holds its build script, a ctypes binding with the
same function names and a small `Engine` wrapper that owns the torch-
allocated device workspace and stream.  PyTorch is used only for device
memory and streams.
"""

from ._lib import (  # noqa: F401
    SpecError, spec_config, spec_workspace_bytes, spec_create,
    spec_load_weights, spec_prefill, spec_verify, spec_commit, spec_release,
    spec_request_state, spec_force_root, spec_set_fault, spec_timing_enable, spec_timing_read,
    spec_destroy, spec_last_error, spec_acceptance_update, spec_plan_drafts,
    spec_probe_read_bandwidth, spec_probe_read_bandwidth_noalloc,
    EXPORTS, LIB_PATH, lib,
    SPEC_DTYPE_BF16, SPEC_DTYPE_FP32, SPEC_LAYER_ATTN, SPEC_LAYER_LR,
    SPEC_E_INVAL, SPEC_E_STATE, SPEC_E_CAPACITY, SPEC_E_HIP,
    SPEC_E_UNSUPPORTED, SPEC_MAX_LAYERS, SPEC_WEIGHTS_NATIVE, SPEC_WEIGHTS_W12,
    SPEC_WEIGHTS_W12_LOWP,
)
from .engine import Engine, make_config  # noqa: F401
