// Fused q4-weight GEMM instances: C = A * dequant(q)^T with fp16 A and N x K
// weights as 18-byte q4 blocks, through the direct-to-LDS kernel whose B
// tile is decoded from the blocks in registers.
#include "launch.h"
#include "mfma_direct.h"

namespace dge {

template <int BM, int BN, int WM, int WN>
static hipError_t launch_q4_one(const MfmaArgs& a, int nwg, hipStream_t s) {
    constexpr int MS = WM * WN == 8 ? 16 : 32;
    hipLaunchKernelGGL((gemm_direct_kernel<IN_F16, BM, BN, WM, WN, true, MS, true>), dim3(nwg),
                       dim3(WM * WN * 64), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_mfma_q4_f16(int tile, const MfmaArgs& a, int nwg, hipStream_t s) {
    switch (tile) {
        case TILE_256x256: return launch_q4_one<256, 256, 2, 2>(a, nwg, s);
        case TILE_256x128: return launch_q4_one<256, 128, 2, 2>(a, nwg, s);
        case TILE_128x128: return launch_q4_one<128, 128, 2, 2>(a, nwg, s);
        case TILE_128x64: return launch_q4_one<128, 64, 2, 2>(a, nwg, s);
        case TILE_256x256_W8: return launch_q4_one<256, 256, 2, 4>(a, nwg, s);
        case TILE_256x128_W8: return launch_q4_one<256, 128, 4, 2>(a, nwg, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace dge
