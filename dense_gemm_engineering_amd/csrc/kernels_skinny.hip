// Tall-skinny fused-epilogue GEMM instances (fp16 and bf16 inputs), general
// epilogue; the alpha = 1, beta = 0, fp16-output instances are in
// kernels_skinny_fold.hip.
#include "skinny_launch.h"

namespace dge {

hipError_t skinny_init() {
    hipError_t e = skinny_optin<false>();
    return e == hipSuccess ? skinny_fold_init() : e;
}

hipError_t launch_skinny(int dt, int nt, int trans_b, const SkinnyArgs& a, int grid, int waves,
                         size_t lds, hipStream_t s) {
    if (a.ep.alpha == 1.0f && a.ep.beta == 0.0f && a.c_type == OUT_F16)
        return launch_skinny_fold(dt, nt, trans_b, a, grid, waves, lds, s);
    return skinny_launch<false>(dt, nt, trans_b, a, grid, waves, lds, s);
}

}  // namespace dge
