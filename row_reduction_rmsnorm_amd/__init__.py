"""Row-wise reduce-then-rescale kernels for AMD MI355X (gfx950).

RMSNorm, fused residual-add + RMSNorm, LayerNorm and row softmax on the
online (m, d) normaliser, as hand-written HIP kernels behind the C ABI of
``librowreduce.so`` (declared in ``include/rowreduce.h``).  This package is
the thin Python binding: it marshals torch tensors' device pointers and the
current stream into that ABI and nothing else.
"""
from .binding import (  # noqa: F401
    BF16, EXPORTS, F32, RR_BF16, RR_ERR_HIP, RR_ERR_INVALID_ARG, RR_ERR_UNSUPPORTED,
    RR_ERR_WORKSPACE, RR_F32, RR_OK, RR_OP_FUSED_ADD_RMSNORM, RR_OP_LAYERNORM, RR_OP_RMSNORM,
    RR_OP_SOFTMAX, RR_OP_SOFTMAX_CAUSAL,
    RR_VARIANT_AUTO, RR_VARIANT_BLOCK, RR_VARIANT_LOOP, RR_VARIANT_SPLIT, RR_VARIANT_SPLIT_ONE_KERNEL,
    RR_VARIANT_SUBWAVE, RR_VARIANT_WAVE, RR_VARIANT_SPLIT_TWO_KERNELS,
    RowReduceError, VARIANT_NAMES, check, dtype_code, fused_add_rmsnorm, last_error_message,
    layernorm, lib, raw_layernorm, rr_layernorm,
    raw_fused_add_rmsnorm, raw_rmsnorm, raw_softmax_rows, rmsnorm, rr_fused_add_rmsnorm,
    rr_query_plan, rr_rmsnorm, rr_selftest_wave_allreduce, rr_stream_copy,
    load_library, diag_lib, forced_variant, DIAG_EXPORTS, split_fallbacks, split_wait,
    SPLIT_WAIT_TICKS_DEFAULT,
    rr_softmax_rows, rr_softmax_rows_workspace_bytes, softmax_rows, softmax_workspace,
    status_string, rr_softmax_opts, make_softmax_opts, raw_softmax_rows_ex, rr_softmax_rows_ex,
    rr_softmax_rows_ex_workspace_bytes, softmax_rows_ex, raw_rmsnorm_strided,
    raw_fused_add_rmsnorm_strided, raw_layernorm_strided, raw_softmax_rows_strided,
    rr_rmsnorm_strided, rr_fused_add_rmsnorm_strided, rr_layernorm_strided,
    rr_softmax_rows_strided, raw_softmax_rows_strided_noalloc, rr_softmax_rows_strided_noalloc,
)
