"""MI355X-native dense GEMM: hand-written gfx950 HIP kernels behind a C ABI."""
