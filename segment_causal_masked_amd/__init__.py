"""Action-aware causal attention (Hy-Nomas) for MI355X / gfx950.

The computation lives in libnomas_attn.so (hand-written HIP kernels behind the
C ABI of include/nomas_attn.h); this package is its Python binding plus the
seeded workload descriptions.  Importing the package does not load the
library; the first call does, and fails loudly if it is not built.
"""
from ._lib import (  # noqa: F401
    CameraPlan, KVCache, KVCacheInt8, NomasError, Plan, load,
    nomas_kvcache_adopt, nomas_kvcache_int8_adopt, nomas_kvcache_int8_append, nomas_kvcache_int8_create, nomas_kvcache_int8_destroy,
    nomas_kvcache_int8_expand, nomas_kvcache_int8_len, nomas_kvcache_int8_truncate,
    nomas_camera_attn_fwd, nomas_camera_attn_plan, nomas_camera_plan_destroy,
    nomas_camera_plan_export_ranges, nomas_camera_plan_get_info,
    nomas_action_latent_window, nomas_attn_bwd, nomas_attn_bwd_workspace_size, nomas_attn_fwd, nomas_attn_fwd_noalloc,
    nomas_attn_fwd_workspace_size, nomas_attn_plan, nomas_kvcache_append,
    nomas_kvcache_create, nomas_kvcache_destroy, nomas_kvcache_len, nomas_kvcache_reset,
    nomas_kvcache_truncate, nomas_last_error, nomas_plan_destroy, nomas_plan_export_classes,
    nomas_plan_get_info, nomas_status_string,
)
