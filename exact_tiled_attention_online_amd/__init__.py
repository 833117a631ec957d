"""Exact tiled attention for MI355X (gfx950): online-softmax forward and
recompute backward as hand-written HIP kernels behind a C ABI (libfa.so).

The Python layer only marshals arguments; see ``_lib`` for the entry points
(fa_fwd, fa_bwd, fa_bwd_workspace_bytes, fa_bwd_workspace_size,
fa_bwd_dq_method, the three backward stages, the FP8 forward, the
split-key-range forward, the dropout forward and backward, fa_strerror) and
the torch-tensor conveniences ``forward`` / ``backward`` /
``forward_fp8`` / ``forward_splitkv`` / ``forward_dropout`` /
``backward_dropout``.
"""
from ._lib import (  # noqa: F401
    FA_BF16, FA_DQ_ATOMIC, FA_DQ_HANDOFF, FA_DQ_RECOMPUTE, FA_FP32, FA_LAYOUT_BHND, FA_LAYOUT_BNHD, FAError,
    LIB_PATH, backward, fa_bwd, fa_bwd_dq_method, fa_bwd_workspace_size,
    backward_dropout, drop_threshold, fa_bwd_dropout, fa_fwd_dropout, forward_dropout,
    fa_bwd_dkdv, fa_bwd_dq, fa_bwd_preprocess, fa_bwd_workspace_bytes, fa_fwd, fa_fwd_fp8, fa_fwd_splitkv,
    fa_fwd_splitkv_workspace_bytes, fa_fwd_splitkv_fp8, fa_fwd_splitkv_fp8_workspace_bytes, fa_strerror,
    fa_fwd_splitkv_noalloc, FA_SPLITKV_NOALLOC_MAX_BYTES, FA_ERR_SCRATCH,
    fa_fwd_strided, fa_bwd_strided, forward_strided, backward_strided,
    forward, forward_fp8, forward_splitkv, forward_splitkv_fp8, load, workspace,
)
