"""MI355X-native fused FlashAttention forward: gfx950 HIP kernels behind a C-ABI.

``fa_fwd`` computes O = softmax(scale * Q K^T [+ causal mask]) V and the row
logsumexp L for [B, H, N, d] tensors in one fused kernel (see include/fa.h).
"""
from .binding import (FA_DTYPE_BF16, FA_DTYPE_F16, FA_DTYPE_F32, FA_ERR_INVALID_ARG,
                      FA_ERR_LAUNCH, FA_ERR_UNSUPPORTED, FA_OK, FAError, fa_fwd, fa_fwd_raw,
                      fa_status_str, fa_tile_rows)

__all__ = ["fa_fwd", "fa_fwd_raw", "fa_status_str", "fa_tile_rows", "FAError", "FA_OK",
           "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_LAUNCH", "FA_DTYPE_F32",
           "FA_DTYPE_F16", "FA_DTYPE_BF16"]
