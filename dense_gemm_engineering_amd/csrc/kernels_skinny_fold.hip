// Tall-skinny fused-epilogue GEMM instances for alpha = 1, beta = 0 and fp16
// output (the bias starts the accumulators; the epilogue is GELU or nothing
// and the rounding).
#include "skinny_launch.h"

namespace dge {

hipError_t skinny_fold_init() { return skinny_optin<true>(); }

hipError_t launch_skinny_fold(int dt, int nt, int trans_b, const SkinnyArgs& a, int grid,
                              int waves, size_t lds, hipStream_t s) {
    return skinny_launch<true>(dt, nt, trans_b, a, grid, waves, lds, s);
}

}  // namespace dge
