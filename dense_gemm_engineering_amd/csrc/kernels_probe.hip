// Measurement probes: the ceilings the GEMM path is judged against, measured
// on the device itself rather than taken from the data sheet.
//
//  * probe_mfma_kernel: the headline kernel's matrix work and nothing else.
//    256 workgroups of 8 waves; each wave takes two k-blocks of operand
//    fragments from the real A and B (the workload's value distribution, so
//    the matrix units toggle as many bits as in the GEMM: their power, and
//    so the clock, depends on the data) and issues the same 16x16x32 MFMAs
//    over the same 8 x 4 blocks of accumulators in the same serpentine order,
//    k_blocks times, with no loads, LDS traffic or stores in the loop.  At
//    k_blocks = 128 it does the 2 x 4096^3 FLOPs of the 4096^3 product.
//    It records the shader and real-time clocks like the GEMM does.
//  * probe_read_kernel / probe_copy_kernel: streaming 16-byte reads (and
//    writes) over a buffer larger than the 256 MB Infinity Cache: the HBM
//    bandwidth a kernel of this library can reach.
#include "launch.h"

namespace dge {

typedef unsigned long long u64;

template <int DT>
__global__ __launch_bounds__(512, 1) void probe_mfma_kernel(const void* A, const void* B,
                                                            int64_t lda, int64_t ldb,
                                                            int k_blocks, float* out, u64* clk) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    u64 clk0 = 0, rt0 = 0;
    if (clk) {
        clk0 = __builtin_amdgcn_s_memtime();
        rt0 = __builtin_amdgcn_s_memrealtime();
    }
    // the workgroup's 256 x 256 tile of a 4096 x 4096 output; the wave's
    // 128 x 64 part (2 x 4 waves), as in the 8-wave GEMM tile
    const int tm = blockIdx.x / 16, tn = blockIdx.x % 16;
    const int r0 = tm * 256 + (wave / 4) * 128, c0 = tn * 256 + (wave % 4) * 64;
    u32x4 fa[2][8], fb[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int k = kb * 32 + (lane / 16) * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            fa[kb][i] = *(const u32x4*)((const uint16_t*)A + (int64_t)(r0 + 16 * i + lane % 16) * lda + k);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            fb[kb][j] = *(const u32x4*)((const uint16_t*)B + (int64_t)(c0 + 16 * j + lane % 16) * ldb + k);
    }
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
    // k-block `it` uses fragment set it % 2 (the set is a compile-time index:
    // a run-time one would move the fragments through memory)
    auto kblock = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < 32; ++x) {
            const int i = x / 4, j = (i & 1) ? 3 - x % 4 : x % 4;
            mma_chunk<DT>(acc[i][j], fb[kb][j], fa[kb][i]);
        }
    };
    int it = 0;
    for (; it + 1 < k_blocks; it += 2) {
        kblock(0);
        kblock(1);
    }
    if (it < k_blocks) kblock(0);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s += acc[i][j];
    out[(int64_t)blockIdx.x * 512 + tid] = s[0] + s[1] + s[2] + s[3];
    if (clk) {
        const u64 clk1 = __builtin_amdgcn_s_memtime(), rt1 = __builtin_amdgcn_s_memrealtime();
        if (tid == 0) {
            u64* c = clk + 4 * (int64_t)blockIdx.x;
            c[0] = clk0;
            c[1] = rt0;
            c[2] = clk1;
            c[3] = rt1;
        }
    }
}

// Reads n16 16-byte chunks, eight independent loads in flight per thread;
// one 32-bit digest per thread keeps the loads alive.
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* src, int64_t n16,
                                                         unsigned* out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    u32x4 x = {0, 0, 0, 0};
    for (; i + 7 * stride < n16; i += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) x ^= v[u];
    }
    for (; i < n16; i += stride) x ^= __builtin_nontemporal_load(src + i);
    out[(int64_t)blockIdx.x * 256 + threadIdx.x] = x[0] ^ x[1] ^ x[2] ^ x[3];
}

// Copies n16 16-byte chunks (non-temporal loads and stores, as the GEMM's
// output), four chunks in flight per thread.
__global__ __launch_bounds__(256) void probe_copy_kernel(const u32x4* src, u32x4* dst,
                                                         int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

hipError_t launch_probe_mfma(int dt, const void* A, const void* B, int64_t lda, int64_t ldb,
                             int k_blocks, float* out, unsigned long long* clk, hipStream_t s) {
    if (dt == IN_F16)
        hipLaunchKernelGGL(probe_mfma_kernel<IN_F16>, dim3(PROBE_MFMA_GRID), dim3(512), 0, s, A, B,
                           lda, ldb, k_blocks, out, clk);
    else
        hipLaunchKernelGGL(probe_mfma_kernel<IN_BF16>, dim3(PROBE_MFMA_GRID), dim3(512), 0, s, A,
                           B, lda, ldb, k_blocks, out, clk);
    return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, int64_t n16, unsigned* out, int grid,
                             hipStream_t s) {
    hipLaunchKernelGGL(probe_read_kernel, dim3(grid), dim3(256), 0, s,
                       (const u32x4*)src, n16, out);
    return hipGetLastError();
}

hipError_t launch_probe_copy(const void* src, void* dst, int64_t n16, int grid, hipStream_t s) {
    hipLaunchKernelGGL(probe_copy_kernel, dim3(grid), dim3(256), 0, s,
                       (const u32x4*)src, (u32x4*)dst, n16);
    return hipGetLastError();
}

}  // namespace dge
