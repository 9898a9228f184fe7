"""Q4_0 block-quantized weight dequant, GEMV and GEMM on AMD MI355X (gfx950)."""
