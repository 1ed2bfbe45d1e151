"""io_aware_exact_22_amd -- exact attention forward for MI355X (gfx950).

``libfa_mi355x.so`` holds the hand-written HIP kernels and a C ABI
(``include/fa_mi355x.h``); this package is a thin ctypes binding over it.
PyTorch supplies device memory and streams only: every arithmetic step of the
forward pass runs in the library's kernels, and the binding raises if the
library is missing rather than falling back to anything else.
"""
from .fa import (FA_DTYPE_BF16, FA_DTYPE_FP16, FA_DTYPE_FP32, FA_ERR_SCRATCH, FA_MAX_KV_SPLITS,
                 FA_MAX_SPLITS, fa_fwd_kvcache, fa_fwd_kvcache_auto_splits,
                 fa_fwd_kvcache_workspace_size, flash_attn_fwd_kvcache,
                 FA_NOALLOC_SCRATCH_BYTES, FaError, fa_bwd,
                 fa_bwd_workspace_size, fa_fwd, fa_fwd_blocksparse,
                 fa_fwd_blocksparse_workspace_size, fa_fwd_check_args, fa_fwd_paged, fa_fwd_splitkv,
                 fa_fwd_splitkv_auto_splits, fa_fwd_splitkv_noalloc, fa_fwd_splitkv_workgroup_tile,
                 fa_fwd_splitkv_workspace_size, fa_fwd_tile_schedule, fa_fwd_workgroup_tile,
                 fa_fwd_launch_order, fa_status_string, flash_attn_bwd, flash_attn_fwd,
                 flash_attn_fwd_blocksparse, flash_attn_fwd_paged, flash_attn_fwd_splitkv,
                 library_path)

__all__ = [
    "FA_DTYPE_BF16", "FA_DTYPE_FP16", "FA_DTYPE_FP32", "FA_ERR_SCRATCH", "FA_MAX_SPLITS",
    "FA_NOALLOC_SCRATCH_BYTES", "FA_MAX_KV_SPLITS", "FaError", "fa_bwd", "fa_fwd_kvcache",
    "fa_fwd_kvcache_auto_splits", "fa_fwd_kvcache_workspace_size", "flash_attn_fwd_kvcache",
    "fa_bwd_workspace_size", "fa_fwd", "fa_fwd_blocksparse", "fa_fwd_blocksparse_workspace_size",
    "fa_fwd_check_args", "fa_fwd_paged", "fa_fwd_splitkv", "fa_fwd_splitkv_auto_splits",
    "fa_fwd_splitkv_noalloc",
    "fa_fwd_splitkv_workgroup_tile", "fa_fwd_splitkv_workspace_size", "fa_fwd_tile_schedule",
    "fa_fwd_workgroup_tile", "fa_fwd_launch_order",
    "fa_status_string", "flash_attn_bwd", "flash_attn_fwd", "flash_attn_fwd_blocksparse",
    "flash_attn_fwd_paged", "flash_attn_fwd_splitkv", "library_path",
]
