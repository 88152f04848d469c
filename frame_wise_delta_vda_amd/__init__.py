"""MI355X (gfx950) Video Delta Attention forward: a HIP library behind a C ABI
(include/vda.h) and its Python binding.  Build with
``python -m frame_wise_delta_vda_amd.build``."""
from .vda import (  # noqa: F401
    Plan, VdaError, load_library, declared_functions,
    vda_plan_create, vda_forward, vda_forward_stages, vda_plan_destroy,
    vda_plan_workspace_bytes, vda_status_string, vda_debug_workspace,
    VDA_DTYPE_F32, VDA_DTYPE_BF16, VDA_STAGE_STATS, VDA_STAGE_SCAN, VDA_STAGE_READOUT,
    VDA_STAGE_ALL, STATUS,
)
