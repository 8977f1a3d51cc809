// Launchers for the vector-ALU ladder kernels, the split-K fixup and the q4
// dequant.
#include "dequant.h"
#include "launch.h"

namespace dge {

template <int DT>
static hipError_t naive_dt(const SimpleArgs& a, hipStream_t s) {
    dim3 block(64, 4);
    dim3 grid((a.N + 63) / 64, (a.M + 3) / 4);
    hipLaunchKernelGGL((gemm_naive_kernel<DT>), grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_naive(int dt, const SimpleArgs& a, hipStream_t s) {
    switch (dt) {
        case IN_F16: return naive_dt<IN_F16>(a, s);
        case IN_BF16: return naive_dt<IN_BF16>(a, s);
        default: return naive_dt<IN_F32>(a, s);
    }
}

template <int DT>
static hipError_t tiled_dt(const SimpleArgs& a, hipStream_t s) {
    dim3 grid((a.N + 63) / 64, (a.M + 63) / 64);
    hipLaunchKernelGGL((gemm_lds_tiled_kernel<DT>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_lds_tiled(int dt, const SimpleArgs& a, hipStream_t s) {
    switch (dt) {
        case IN_F16: return tiled_dt<IN_F16>(a, s);
        case IN_BF16: return tiled_dt<IN_BF16>(a, s);
        default: return tiled_dt<IN_F32>(a, s);
    }
}

template <int DT>
static hipError_t fixup_dt(const SimpleArgs& a, const float* ws, int splits, hipStream_t s) {
    const int64_t total = (int64_t)a.M * a.N;
    const int ob = a.c_type == OUT_F32 ? 4 : 2;
    if (a.N % 4 == 0 && ((uintptr_t)ws & 15) == 0 && ((uintptr_t)a.C & (4 * ob - 1)) == 0 &&
        (a.ldc * ob) % (4 * ob) == 0) {
        int64_t blocks = (total / 4 + 255) / 256;
        if (blocks > 65536) blocks = 65536;
        const dim3 g((unsigned)blocks), b(256);
        if (a.c_type == OUT_F16)
            hipLaunchKernelGGL((splitk_fixup4_kernel<DT, OUT_F16>), g, b, 0, s, a, ws, splits);
        else if (a.c_type == OUT_BF16)
            hipLaunchKernelGGL((splitk_fixup4_kernel<DT, OUT_BF16>), g, b, 0, s, a, ws, splits);
        else
            hipLaunchKernelGGL((splitk_fixup4_kernel<DT, OUT_F32>), g, b, 0, s, a, ws, splits);
        return hipGetLastError();
    }
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((splitk_fixup_kernel<DT>), dim3((unsigned)blocks), dim3(256), 0, s, a, ws,
                       splits);
    return hipGetLastError();
}

hipError_t launch_splitk_fixup(int dt, const SimpleArgs& a, const float* ws, int splits,
                               hipStream_t s) {
    switch (dt) {
        case IN_F16: return fixup_dt<IN_F16>(a, ws, splits, s);
        case IN_BF16: return fixup_dt<IN_BF16>(a, ws, splits, s);
        default: return fixup_dt<IN_F32>(a, ws, splits, s);
    }
}

__global__ __launch_bounds__(256) void clear_u32_kernel(unsigned* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = 0u;
}

hipError_t launch_clear_u32(unsigned* p, int64_t n, hipStream_t s) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(clear_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_dequant_q4(const void* q, void* out, int64_t rows, int64_t cols, int64_t ldo,
                             int vec_out, hipStream_t s) {
    if (cols % 256 == 0) return launch_dequant_kq(KQ_Q4_0_256, q, out, rows, cols, ldo, vec_out, s);
    const int64_t total = rows * (cols / 32);
    int64_t blocks = (total + DQ_BLOCKS - 1) / DQ_BLOCKS;
    if (blocks > 1 << 20) blocks = 1 << 20;
    const int flags = (((uintptr_t)q & 15) == 0 ? 1 : 0) | (vec_out ? 2 : 0);
    hipLaunchKernelGGL(dequant_q4_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       (const uint8_t*)q, (uint16_t*)out, rows, cols, ldo, flags);
    return hipGetLastError();
}

hipError_t launch_dequant_kq(int qtype, const void* q, void* out, int64_t rows, int64_t cols,
                             int64_t ldo, int vec_out, hipStream_t s) {
    constexpr int SB = KQ_STEP;
    const int64_t total = rows * (cols / 256);
    int64_t blocks = (total + SB - 1) / SB;
    // 8 resident workgroups per CU of a 256-CU part: each takes several
    // steps, so its register prefetch of the next step overlaps the decode
    if (blocks > KQ_GRID) blocks = KQ_GRID;
    const int flags = (((uintptr_t)q & 15) == 0 ? 1 : 0) | (vec_out ? 2 : 0) |
                      ((int64_t)(SB + 1) * ldo * 2 < ((int64_t)1 << 31) ? 4 : 0);
    if (qtype == KQ_Q6_K)
        hipLaunchKernelGGL((dequant_kq_f16_kernel<KQ_Q6_K, SB>), dim3((unsigned)blocks), dim3(256), 0,
                           s, (const uint8_t*)q, (uint16_t*)out, rows, cols, ldo, flags);
    else if (qtype == KQ_Q4_0_256)
        hipLaunchKernelGGL((dequant_kq_f16_kernel<KQ_Q4_0_256, SB>), dim3((unsigned)blocks), dim3(256),
                           0, s, (const uint8_t*)q, (uint16_t*)out, rows, cols, ldo, flags);
    else if (qtype == KQ_Q6_K_224)
        hipLaunchKernelGGL((dequant_kq_f16_kernel<KQ_Q6_K_224, SB>), dim3((unsigned)blocks), dim3(256),
                           0, s, (const uint8_t*)q, (uint16_t*)out, rows, cols, ldo, flags);
    else
        hipLaunchKernelGGL((dequant_kq_f16_kernel<KQ_Q4_K, SB>), dim3((unsigned)blocks), dim3(256), 0,
                           s, (const uint8_t*)q, (uint16_t*)out, rows, cols, ldo, flags);
    return hipGetLastError();
}

}  // namespace dge
