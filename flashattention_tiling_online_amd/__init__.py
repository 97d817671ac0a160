"""MI355X-native fused FlashAttention forward: gfx950 HIP kernels behind a C-ABI.

``fa_fwd`` computes O = softmax(scale * Q K^T [+ causal mask]) V and the row
logsumexp L for [B, H, N, d] tensors in one fused kernel (``fa_fwd_masked``: with a
caller's boolean mask on the scores); ``fa_fwd_split`` computes
the same over key ranges in parallel and merges the partial states
(``fa_fwd_split_static_raw``: the same without a workspace, for callers that cannot
allocate), and ``fa_merge`` folds partial states computed elsewhere; ``fa_bwd``
computes the gradients dQ, dK, dV by recomputation from the forward's O and L
(``fa_bwd_masked`` for the masked forward);
``fa_fwd_dropout`` / ``fa_bwd_dropout`` are the two with dropout on P (see include/fa.h).
"""
from .binding import (FA_DTYPE_BF16, FA_DTYPE_F16, FA_DTYPE_F32, FA_ERR_INVALID_ARG,
                      FA_ERR_LAUNCH, FA_ERR_SCRATCH, FA_ERR_UNSUPPORTED, FA_OK,
                      FA_STATIC_SCRATCH_BYTES, FAError, fa_bwd, fa_bwd_masked, fa_bwd_masked_raw, fa_bwd_raw,
                      fa_bwd_dropout, fa_bwd_dropout_raw, fa_bwd_workspace, fa_fwd,
                      fa_fwd_dropout, fa_fwd_dropout_raw, fa_fwd_masked, fa_fwd_masked_raw, fa_fwd_raw,
                      fa_fwd_split, fa_fwd_split_raw, fa_fwd_split_static_raw,
                      fa_fwd_split_workspace, fa_merge, fa_merge_raw, fa_split_hint,
                      fa_status_str, fa_tile_rows)

__all__ = ["fa_fwd", "fa_fwd_raw", "fa_fwd_masked", "fa_fwd_masked_raw", "fa_bwd", "fa_bwd_raw",
           "fa_bwd_masked", "fa_bwd_masked_raw", "fa_bwd_workspace",
           "fa_fwd_dropout", "fa_fwd_dropout_raw", "fa_bwd_dropout", "fa_bwd_dropout_raw",
           "fa_fwd_split", "fa_fwd_split_raw", "fa_fwd_split_static_raw",
           "fa_fwd_split_workspace", "fa_merge", "fa_merge_raw", "fa_split_hint",
           "fa_status_str", "fa_tile_rows", "FAError", "FA_OK", "FA_ERR_INVALID_ARG",
           "FA_ERR_UNSUPPORTED", "FA_ERR_LAUNCH", "FA_ERR_SCRATCH", "FA_STATIC_SCRATCH_BYTES",
           "FA_DTYPE_F32", "FA_DTYPE_F16", "FA_DTYPE_BF16"]
