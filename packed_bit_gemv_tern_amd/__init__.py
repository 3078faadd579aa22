"""Ternary packed-bit GEMV / small-M GEMM for AMD MI355X (gfx950)."""
