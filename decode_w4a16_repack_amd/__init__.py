"""MI355X-native W4A16 group-quantized GEMM/GEMV (binding package)."""
