// Decode-shaped GEMM instances (M <= 64 input rows, N x K weight, 16-bit).
#include "launch.h"
#include "decode.h"

namespace dge {

template <int DT>
static hipError_t decode_dt(const DecodeArgs& a, int grid, hipStream_t s) {
    const dim3 block(DECODE_WAVES * 64);
    switch ((a.M + 15) / 16) {
        case 1:
            if (a.M == 1)
                hipLaunchKernelGGL((gemm_decode_kernel<DT, 1, false>), dim3(grid), block, 0, s, a);
            else
                hipLaunchKernelGGL((gemm_decode_kernel<DT, 1>), dim3(grid), block, 0, s, a);
            break;
        case 2: hipLaunchKernelGGL((gemm_decode_kernel<DT, 2>), dim3(grid), block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((gemm_decode_kernel<DT, 3>), dim3(grid), block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((gemm_decode_kernel<DT, 4>), dim3(grid), block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int DT>
static hipError_t decode_split_dt(const DecodeArgs& a, int grid, hipStream_t s) {
    const dim3 block(DECODE_WAVES * 64);
    switch ((a.M + 15) / 16) {
        case 2: hipLaunchKernelGGL((gemm_decode_split_kernel<DT, 2>), dim3(grid), block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((gemm_decode_split_kernel<DT, 3>), dim3(grid), block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((gemm_decode_split_kernel<DT, 4>), dim3(grid), block, 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_decode_split(int dt, const DecodeArgs& a, hipStream_t s) {
    const int grid = a.N / DSPLIT_ROWS * a.ksplit;
    return dt == IN_BF16 ? decode_split_dt<IN_BF16>(a, grid, s) : decode_split_dt<IN_F16>(a, grid, s);
}

hipError_t launch_decode(int dt, const DecodeArgs& a, hipStream_t s) {
    const int grid = (a.N + 15) / 16;
    return dt == IN_BF16 ? decode_dt<IN_BF16>(a, grid, s) : decode_dt<IN_F16>(a, grid, s);
}

}  // namespace dge
