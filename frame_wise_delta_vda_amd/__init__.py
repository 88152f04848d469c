"""MI355X (gfx950) Video Delta Attention forward: a HIP library behind a C ABI
(include/vda.h) and its Python binding.  Build with
``python -m frame_wise_delta_vda_amd.build``."""
from .vda import (  # noqa: F401
    Plan, VdaError, load_library, declared_functions,
    vda_plan_create, vda_forward, vda_forward_stages, vda_forward_gated, vda_backward,
    vda_plan_destroy, vda_plan_workspace_bytes, vda_status_string, vda_debug_workspace,
    vda_plan_enable_timing, vda_plan_timings, vda_plan_set_timed_stages, vda_forward_noalloc, vda_plan_set_scan_chunk, vda_plan_get_scan_chunk, VDA_SCAN_CHUNK_AUTO,
    VDA_DTYPE_F32, VDA_DTYPE_BF16, VDA_DTYPE_FP8_E4M3, DTYPES,
    VDA_STAGE_STATS, VDA_STAGE_SCAN, VDA_STAGE_READOUT, VDA_STAGE_ALL, STATUS,
    VDA_SUCCESS, VDA_ERROR_INVALID_VALUE, VDA_ERROR_NOT_SUPPORTED, VDA_ERROR_MISALIGNED,
    VDA_ERROR_OUT_OF_MEMORY, VDA_ERROR_DEVICE, VDA_ERROR_TOO_LARGE,
    VDA_NOALLOC_SCRATCH_BYTES,
)
