// Tall-skinny fused-epilogue GEMM instances (fp16 and bf16 inputs).
#include "launch.h"
#include "skinny.h"

namespace dge {

template <int DT, int NT>
static hipError_t skinny_nt(int trans_b, const SkinnyArgs& a, int grid, int waves, size_t lds,
                            hipStream_t s) {
    if (trans_b)
        hipLaunchKernelGGL((gemm_skinny_kernel<DT, NT, true>), dim3(grid), dim3(waves * 64), lds,
                           s, a);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<DT, NT, false>), dim3(grid), dim3(waves * 64), lds,
                           s, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t skinny_dt(int nt, int trans_b, const SkinnyArgs& a, int grid, int waves,
                            size_t lds, hipStream_t s) {
    switch (nt) {
        case 2: return skinny_nt<DT, 2>(trans_b, a, grid, waves, lds, s);
        case 4: return skinny_nt<DT, 4>(trans_b, a, grid, waves, lds, s);
        case 6: return skinny_nt<DT, 6>(trans_b, a, grid, waves, lds, s);
        case 8: return skinny_nt<DT, 8>(trans_b, a, grid, waves, lds, s);
        case 10: return skinny_nt<DT, 10>(trans_b, a, grid, waves, lds, s);
        case 12: return skinny_nt<DT, 12>(trans_b, a, grid, waves, lds, s);
        case 14: return skinny_nt<DT, 14>(trans_b, a, grid, waves, lds, s);
        case 16: return skinny_nt<DT, 16>(trans_b, a, grid, waves, lds, s);
        default: return hipErrorInvalidValue;
    }
}

template <int DT, int NT>
static hipError_t optin_nt() {
    const int bytes = 160 * 1024;
    hipError_t e = hipFuncSetAttribute((const void*)gemm_skinny_kernel<DT, NT, false>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)gemm_skinny_kernel<DT, NT, true>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int DT>
static hipError_t optin_dt() {
    hipError_t e;
    if ((e = optin_nt<DT, 2>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 4>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 6>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 8>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 10>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 12>()) != hipSuccess) return e;
    if ((e = optin_nt<DT, 14>()) != hipSuccess) return e;
    return optin_nt<DT, 16>();
}

hipError_t skinny_init() {
    hipError_t e = optin_dt<IN_F16>();
    return e == hipSuccess ? optin_dt<IN_BF16>() : e;
}

hipError_t launch_skinny(int dt, int nt, int trans_b, const SkinnyArgs& a, int grid, int waves,
                         size_t lds, hipStream_t s) {
    return dt == IN_BF16 ? skinny_dt<IN_BF16>(nt, trans_b, a, grid, waves, lds, s)
                         : skinny_dt<IN_F16>(nt, trans_b, a, grid, waves, lds, s);
}

}  // namespace dge
