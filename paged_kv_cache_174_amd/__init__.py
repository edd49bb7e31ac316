"""pkv: paged K/V write, history-staging gather and piecewise paged attention
for AR-diffusion on AMD MI355X (gfx950).

The compute lives in ``libpkv.so`` (HIP kernels behind the C ABI of
``include/pkv.h``); this package is its ctypes binding plus the once-per-forward
metadata plan.  Build with ``python -m paged_kv_cache_174_amd.build``.
"""

from ._lib import (  # noqa: F401
    EXPORTED,
    PKV_BF16,
    PKV_F32,
    PKV_FP8_E4M3,
    PKV_SEG_CAUSAL,
    PKV_SEG_FULL,
    PkvError,
    PkvValueError,
    Pools,
    lib,
    pkv_action_table,
    pkv_build_segments,
    pkv_gather,
    pkv_last_attn_plan,
    pkv_last_error,
    pkv_paged_attn,
    pkv_paged_attn_main,
    pkv_paged_attn_merge,
    pkv_paged_attn_noalloc,
    pkv_paged_attn_workspace_size,
    pkv_paged_write,
    pkv_paged_write_attn,
    pkv_probe_mfma,
    pkv_probe_stream,
    pkv_slot_mapping,
    pkv_validate_metadata_host,
    pkv_version,
    pkv_window_capacity,
    pkv_window_table,
)
from .plan import ForwardPlan, HistoryStaging, StagingDecision  # noqa: F401
from .window import WindowConfig, WindowManager  # noqa: F401
