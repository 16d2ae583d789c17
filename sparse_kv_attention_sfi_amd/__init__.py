"""MI355X (gfx950) decode-attention path of Slow-Fast Inference (SFI).

The compute lives in ``libsfi.so`` (HIP kernels behind the C ABI declared in
``include/sfi.h``); this package is its thin Python binding.
"""
from .binding import (  # noqa: F401
    KVDesc, Scheduler, SFIError, alloc_workspace, lib, support_params,
    sfi_debug_support, sfi_fast_plan, sfi_fast_step, sfi_fast_step_pack, sfi_fast_step_packed, sfi_fast_step_packed_noalloc, sfi_kv_append, sfi_pack_support, sfi_profile_enable, sfi_profile_read,
    sfi_profile_reset, sfi_select, sfi_slow_plan, sfi_slow_step, sfi_slow_step_select, sfi_slow_step_select_async, sfi_status_str, sfi_version,
    sfi_workspace_bytes, sfi_workspace_init,
    SFI_OP_SLOW, SFI_OP_SELECT, SFI_OP_FAST, SFI_OP_SLOW_SELECT, SFI_K_SLOW_PARTIAL, SFI_K_SLOW_COMBINE,
    SFI_K_SELECT, SFI_K_FAST, SFI_K_APPEND, SFI_K_PACK, SFI_K_FAST_MERGE, SFI_K_FAST_PACK, KERNEL_NAMES,
)
