"""MI355X-native fused FlashAttention forward (gfx950 HIP kernels behind a C-ABI)."""
