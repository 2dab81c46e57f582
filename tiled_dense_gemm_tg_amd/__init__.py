"""MI355X-native tiled half-precision GEMM (gfx950), behind a C-ABI library."""
