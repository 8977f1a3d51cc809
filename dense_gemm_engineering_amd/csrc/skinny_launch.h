// Launch and LDS opt-in of the tall-skinny instances for one value of FOLD
// (the epilogue with alpha = 1, beta = 0 and fp16 output, whose kernels carry
// no other epilogue, or the general one); each of the two translation units
// that include this instantiates one of them.
#pragma once

#include "launch.h"
#include "skinny.h"

namespace dge {

template <int DT, int NT, bool FOLD>
static hipError_t skinny_nt(int trans_b, const SkinnyArgs& a, int grid, int waves, size_t lds,
                            hipStream_t s) {
    if (trans_b)
        hipLaunchKernelGGL((gemm_skinny_kernel<DT, NT, true, FOLD>), dim3(grid), dim3(waves * 64),
                           lds, s, a);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<DT, NT, false, FOLD>), dim3(grid), dim3(waves * 64),
                           lds, s, a);
    return hipGetLastError();
}

template <int DT, bool FOLD>
static hipError_t skinny_dt(int nt, int trans_b, const SkinnyArgs& a, int grid, int waves,
                            size_t lds, hipStream_t s) {
    switch (nt) {
        case 2: return skinny_nt<DT, 2, FOLD>(trans_b, a, grid, waves, lds, s);
        case 4: return skinny_nt<DT, 4, FOLD>(trans_b, a, grid, waves, lds, s);
        case 6: return skinny_nt<DT, 6, FOLD>(trans_b, a, grid, waves, lds, s);
        case 8: return skinny_nt<DT, 8, FOLD>(trans_b, a, grid, waves, lds, s);
        case 10: return skinny_nt<DT, 10, FOLD>(trans_b, a, grid, waves, lds, s);
        case 12: return skinny_nt<DT, 12, FOLD>(trans_b, a, grid, waves, lds, s);
        case 14: return skinny_nt<DT, 14, FOLD>(trans_b, a, grid, waves, lds, s);
        case 16: return skinny_nt<DT, 16, FOLD>(trans_b, a, grid, waves, lds, s);
        default: return hipErrorInvalidValue;
    }
}

template <int DT, int NT, bool FOLD>
static hipError_t optin_nt() {
    const int bytes = 160 * 1024;
    hipError_t e = hipFuncSetAttribute((const void*)gemm_skinny_kernel<DT, NT, false, FOLD>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)gemm_skinny_kernel<DT, NT, true, FOLD>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int DT, bool FOLD>
static hipError_t optin_dt() {
    hipError_t e;
    if ((e = optin_nt<DT, 2, FOLD>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 4, FOLD>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 6, FOLD>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 8, FOLD>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 10, FOLD>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 12, FOLD>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 14, FOLD>()) != hipSuccess) return e;
    return optin_nt<DT, 16, FOLD>();
}

template <bool FOLD>
static hipError_t skinny_optin() {
    hipError_t e = optin_dt<IN_F16, FOLD>();
    return e == hipSuccess ? optin_dt<IN_BF16, FOLD>() : e;
}

template <bool FOLD>
static hipError_t skinny_launch(int dt, int nt, int trans_b, const SkinnyArgs& a, int grid,
                                int waves, size_t lds, hipStream_t s) {
    return dt == IN_BF16 ? skinny_dt<IN_BF16, FOLD>(nt, trans_b, a, grid, waves, lds, s)
                         : skinny_dt<IN_F16, FOLD>(nt, trans_b, a, grid, waves, lds, s);
}

}  // namespace dge
