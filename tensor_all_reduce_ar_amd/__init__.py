"""MI355X (gfx950) all-reduce core: the rank-partial sum and the sum fused
with bias, residual and RMSNorm, as hand-written HIP kernels behind a C ABI
(include/ar.h, built into libar.so).

Importing this package does not touch the GPU; the library is loaded on the
first call and its absence is an error.
"""
from .ar import (AR_BF16, AR_FP16, AR_FP32, AR_FUSION_NONE, AR_FUSION_RESIDUAL_RMS_NORM, AR_MAX_RANKS, AR_OK,
                 AR_SLOT_ALIGN_BYTES, AR_SLOT_STAGGER_BYTES, ArError, Params, PreparedCall, Workspace,
                 allocate_workspace, ar_configuration_supported, ar_last_hip_error, ar_partials_layout,
                 ar_residual_rmsnorm, ar_residual_rmsnorm_slice, ar_rmsnorm, ar_slice_range, ar_status_string,
                 ar_sum, ar_sum_slice, ar_workspace_size, make_params, prepare_residual_rmsnorm,
                 prepare_residual_rmsnorm_slice, prepare_rmsnorm, prepare_sum, prepare_sum_slice)

__all__ = ["ar_sum", "ar_residual_rmsnorm", "ar_rmsnorm", "ar_sum_slice", "ar_residual_rmsnorm_slice",
           "ar_slice_range", "ar_configuration_supported", "ar_workspace_size", "ar_partials_layout",
           "ar_status_string", "ar_last_hip_error", "allocate_workspace", "Workspace", "prepare_sum",
           "prepare_residual_rmsnorm", "prepare_rmsnorm", "prepare_sum_slice", "prepare_residual_rmsnorm_slice",
           "PreparedCall", "Params", "make_params", "ArError", "AR_FP32", "AR_FP16", "AR_BF16",
           "AR_FUSION_NONE", "AR_FUSION_RESIDUAL_RMS_NORM", "AR_MAX_RANKS", "AR_OK", "AR_SLOT_ALIGN_BYTES",
           "AR_SLOT_STAGGER_BYTES"]
