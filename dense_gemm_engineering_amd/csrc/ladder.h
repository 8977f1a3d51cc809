// The vector-ALU rungs of the GEMM ladder ("Matrix Multiplication: The
// Operation Behind Modern AI", sections "The naive kernel", "Tiling: choosing
// your own intensity" and "Registers: the same trick, one level higher"):
//
//  * gemm_naive_kernel: one thread per output element, walking all of K with
//    one FMA per k.  threadIdx.x runs along the columns of C, so a wave reads
//    64 consecutive elements of a B row and broadcasts one A element — the
//    coalesced mapping of that section.  No reuse is collected: every A and B
//    element is fetched from the cache hierarchy once per output that needs it.
//  * gemm_lds_tiled_kernel: 64 x 64 output tiles, K in steps of 16 staged
//    through LDS, each thread accumulating a 4 x 4 register patch; each LDS
//    value read feeds 4 FMAs.  fp32 FMA only, no matrix cores.
//
// Both take any input type (converted to fp32 on load), any output type and
// the full epilogue, so they double as the reference-shaped fallbacks for
// tiny or oddly aligned problems.
#pragma once

#include "device_common.h"

namespace dge {

struct SimpleArgs {
    const void* A;
    const void* B;
    void* C;
    int64_t lda, ldb, ldc;
    int M, N, K;
    int trans_b;
    int c_type;
    Epilogue ep;
};

template <int DT>
__device__ inline float load_b(const SimpleArgs& p, int k, int n) {
    return p.trans_b ? load_elem<DT>(p.B, (int64_t)n * p.ldb + k)
                     : load_elem<DT>(p.B, (int64_t)k * p.ldb + n);
}

template <int DT>
__device__ inline void finish_one(const SimpleArgs& p, int row, int col, float acc) {
    float old = 0.0f;
    const int64_t idx = (int64_t)row * p.ldc + col;
    if (p.ep.beta != 0.0f) {
        if (p.c_type == OUT_F32)
            old = ((const float*)p.C)[idx];
        else if (p.c_type == OUT_F16)
            old = (float)((const _Float16*)p.C)[idx];
        else
            old = (float)((const __bf16*)p.C)[idx];
    }
    const float t = apply_epilogue<DT>(p.ep, acc, old, col);
    if (p.c_type == OUT_F32)
        ((float*)p.C)[idx] = t;
    else if (p.c_type == OUT_F16)
        ((_Float16*)p.C)[idx] = (_Float16)t;
    else
        ((__bf16*)p.C)[idx] = (__bf16)t;
}

template <int DT>
__global__ __launch_bounds__(256) void gemm_naive_kernel(SimpleArgs p) {
    const int col = blockIdx.x * blockDim.x + threadIdx.x;
    const int row = blockIdx.y * blockDim.y + threadIdx.y;
    if (row >= p.M || col >= p.N) return;
    float acc = 0.0f;
    for (int k = 0; k < p.K; ++k)
        acc = fmaf(load_elem<DT>(p.A, (int64_t)row * p.lda + k), load_b<DT>(p, k, col), acc);
    finish_one<DT>(p, row, col, acc);
}

template <int DT>
__global__ __launch_bounds__(256) void gemm_lds_tiled_kernel(SimpleArgs p) {
    constexpr int BM = 64, BN = 64, BK = 16;
    // K-major staging so the inner loop reads a column of A and a row of B
    // as broadcasts/consecutive words; +1 pad against bank conflicts on the
    // transposing stores.
    __shared__ float As[BK][BM + 1];
    __shared__ float Bs[BK][BN + 1];
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += BK) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid + 256 * i;  // 1024 elements per tile
            // A tile: 64 rows x 16 k, k fastest
            const int ar = e / BK, ak = e % BK;
            const int gr = m0 + ar, gk = k0 + ak;
            As[ak][ar] = (gr < p.M && gk < p.K) ? load_elem<DT>(p.A, (int64_t)gr * p.lda + gk) : 0.0f;
            // B tile: 16 k x 64 columns, n fastest
            const int bk = e / BN, bn = e % BN;
            const int gk2 = k0 + bk, gn = n0 + bn;
            Bs[bk][bn] = (gk2 < p.K && gn < p.N) ? load_b<DT>(p, gk2, gn) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[k][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx + 16 * j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = m0 + ty + 16 * i, col = n0 + tx + 16 * j;
            if (row < p.M && col < p.N) finish_one<DT>(p, row, col, acc[i][j]);
        }
}

// Split-K fixup: C = epi(sum_s ws[s]) with the slices summed in order
// s = 0, 1, ..., so the result does not depend on launch timing.
template <int DT>
__global__ __launch_bounds__(256) void splitk_fixup_kernel(SimpleArgs p, const float* ws,
                                                           int splits) {
    const int64_t total = (int64_t)p.M * p.N;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total; idx += stride) {
        float s = 0.0f;
        for (int sp = 0; sp < splits; ++sp) s += ws[sp * total + idx];
        const int row = (int)(idx / p.N), col = (int)(idx % p.N);
        finish_one<DT>(p, row, col, s);
    }
}

// The same fixup, four consecutive columns per thread: 16-byte partial
// loads, one 8- or 16-byte store (N % 4 == 0, the workspace 16-byte aligned,
// C rows and the 4-column groups aligned to their store size).  Each group
// is summed in the same slice order as above.  A thread requests up to
// FIXUP_BATCH slices' partials (and its bias and old C values) before it
// adds any of them: loaded one at a time, each slice cost a whole memory
// round trip.
constexpr int FIXUP_BATCH = 8;

template <int DT, int OT>
__global__ __launch_bounds__(256) void splitk_fixup4_kernel(SimpleArgs p, const float* ws,
                                                            int splits) {
    typedef typename OutType<OT>::T T;
    const int64_t total = (int64_t)p.M * p.N, groups = total / 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const bool small = total <= 0xFFFFFFFFll;  // 32-bit row / column arithmetic
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
        const int64_t idx = 4 * g;
        const float* w = ws + idx;
        f32x4 s = *(const f32x4*)w;
        for (int sp0 = 1; sp0 < splits; sp0 += FIXUP_BATCH) {
            f32x4 v[FIXUP_BATCH];
#pragma unroll
            for (int j = 0; j < FIXUP_BATCH; ++j)
                if (sp0 + j < splits) v[j] = *(const f32x4*)(w + (int64_t)(sp0 + j) * total);
#pragma unroll
            for (int j = 0; j < FIXUP_BATCH; ++j)
                if (sp0 + j < splits) s += v[j];
        }
        int row, col;
        if (small) {
            row = (int)((uint32_t)idx / (uint32_t)p.N);
            col = (int)((uint32_t)idx - (uint32_t)row * (uint32_t)p.N);
        } else {
            row = (int)(idx / p.N);
            col = (int)(idx - (int64_t)row * p.N);
        }
        T* c = (T*)p.C + (int64_t)row * p.ldc + col;
        float old[4] = {0.f, 0.f, 0.f, 0.f}, bias[4] = {0.f, 0.f, 0.f, 0.f};
        if (p.ep.beta != 0.0f) {
#pragma unroll
            for (int e = 0; e < 4; ++e) old[e] = OutType<OT>::to_f32(c[e]);
        }
        if (p.ep.epi != EPI_NONE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) bias[e] = load_elem<DT>(p.ep.bias, col + e);
        }
        T o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            o[e] = OutType<OT>::from_f32(epilogue_value(p.ep, s[e], old[e], bias[e]));
        if constexpr (OutType<OT>::BYTES == 4)
            *(f32x4*)c = (f32x4){o[0], o[1], o[2], o[3]};
        else
            *(uint2*)c = make_uint2((uint32_t)__builtin_bit_cast(uint16_t, o[0]) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, o[1]) << 16),
                                    (uint32_t)__builtin_bit_cast(uint16_t, o[2]) |
                                        ((uint32_t)__builtin_bit_cast(uint16_t, o[3]) << 16));
    }
}

}  // namespace dge
