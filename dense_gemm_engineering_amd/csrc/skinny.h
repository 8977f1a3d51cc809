// Tall-skinny GEMM with the fused epilogue: C = epi(alpha X W + beta C) for
// M >> N, K with N <= 256 and K <= 256 (the window-transformer projections,
// K = 160 with N = 160 or 32).  At these shapes the product is HBM-bound
// (X is read once, C written once; W is 51 KB), so the kernel is built around
// streaming X:
//
//  * W is small enough to sit in LDS for the whole kernel, stored transposed
//    ([n][k], k-contiguous, rows padded by 16 bytes) so that it can serve as
//    the MFMA "A" operand of C^T = W^T X^T.
//  * X needs no LDS: the MFMA "B" operand of X^T is 8 consecutive k of one
//    row of X per lane, i.e. a 16-byte load straight from memory into the
//    operand registers.  Each wave issues all the loads of its 32 rows
//    (K / 32 k-blocks x 2 row blocks; 16 rows for N > 160) before its first
//    MFMA, and the next rows' loads before its epilogue, so many bytes are
//    in flight per CU.
//  * In C^T each lane holds 4 consecutive columns n of one row m of C, so the
//    epilogue (alpha/beta, per-column bias, tanh-GELU, rounding) works on 4
//    adjacent outputs; the rounded tile goes through the wave's LDS staging
//    area and leaves as whole rows, 16 bytes per lane (stores of 32-byte
//    fragments into 16 rows at a time left HBM with partial lines).
#pragma once

#include "device_common.h"
#include "mfma_gemm.h"

namespace dge {

struct SkinnyArgs {
    const void* X;  // M x K, row-major, 16-byte aligned rows
    const void* W;  // K x N (trans_b = 0) or N x K (trans_b = 1)
    void* C;
    int64_t ldx, ldw, ldc;
    int M, N, K;
    int pitch;   // LDS row pitch of W^T in elements (K + 8)
    int c_type;
    int vec_c;   // bit 1: W rows allow aligned 16-byte loads; bit 2: C rows are
                 // 16-byte aligned and N fills whole 16-byte chunks
    Epilogue ep;
};

constexpr int SKINNY_KBMAX = 8;   // K <= 256
constexpr int SKINNY_WAVES = 4;
// 16-row blocks per wave: two while the accumulators of N <= 160 leave room,
// one for wider N (keeps every instance free of register spills)
__host__ __device__ constexpr int skinny_rb(int nt) { return nt <= 10 ? 2 : 1; }

template <int OT>
__device__ inline void skinny_load4(const SkinnyArgs& p, int m, int n0, float* t) {
    typedef typename OutType<OT>::T T;
    const T* c = (const T*)p.C + (int64_t)m * p.ldc + n0;
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = n0 + e < p.N ? OutType<OT>::to_f32(c[e]) : 0.0f;
}

// Epilogue of one wave's RB x 16 rows: alpha/beta, bias, GELU and rounding
// in registers (4 consecutive columns per lane), the rounded values staged in
// the wave's LDS tile (rows of pitch_o bytes), then written out row by row
// with 16-byte stores so that a wave writes whole rows of C.
template <int DT, int OT, int NT, int RB>
__device__ inline void skinny_finish(const SkinnyArgs& p, f32x4 (&acc)[RB][NT], int base,
                                     int lane, char* stage) {
    typedef typename OutType<OT>::T T;
    constexpr int OB = OutType<OT>::BYTES;
    const int pitch_o = NT * 16 * OB + 16;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int ml = rb * 16 + (lane & 15);
        const int m = base + ml;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n0 = nt * 16 + 4 * (lane >> 4);
            float old[4] = {0.f, 0.f, 0.f, 0.f};
            if (p.ep.beta != 0.0f && m < p.M && n0 < p.N) skinny_load4<OT>(p, m, n0, old);
            float t[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = n0 + e < p.N ? n0 + e : p.N - 1;
                t[e] = apply_epilogue<DT>(p.ep, acc[rb][nt][e], old[e], n);
            }
            char* dst = stage + ml * pitch_o + n0 * OB;
            if constexpr (OB == 2) {
                const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, OutType<OT>::from_f32(t[0])) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, OutType<OT>::from_f32(t[1])) << 16);
                const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, OutType<OT>::from_f32(t[2])) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, OutType<OT>::from_f32(t[3])) << 16);
                *(uint2*)dst = make_uint2(lo, hi);
            } else {
                *(f32x4*)dst = (f32x4){t[0], t[1], t[2], t[3]};
            }
        }
    }
    // the wave reads back what it wrote: wave-scope ordering is enough
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const int row_bytes = p.N * OB;
    const int cpr = (row_bytes + 15) / 16;  // 16-byte chunks per row
    const bool vec = (p.vec_c & 4) != 0;    // rows of C are 16-byte aligned and whole chunks
    for (int q = lane; q < RB * 16 * cpr; q += 64) {
        const int ml = q / cpr, c = q - ml * cpr;
        const int m = base + ml;
        if (m >= p.M) continue;
        const char* src = stage + ml * pitch_o + c * 16;
        char* dst = (char*)p.C + ((int64_t)m * p.ldc) * OB + c * 16;
        if (vec) {
            *(u32x4*)dst = *(const u32x4*)src;
        } else {
            for (int e = 0; e < 16 / OB; ++e)
                if (c * 16 + e * OB < row_bytes) ((T*)dst)[e] = ((const T*)src)[e];
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

// W^T into LDS ([n][k], rows n >= N zero-filled).
// N x K W: a task is 8 consecutive k of one n, stored as one 16-byte LDS
// write.  K x N W: a task is a pair of k-rows x 8 consecutive n (two 16-byte
// loads), stored as eight 32-bit LDS writes of (k, k+1) pairs; consecutive
// lanes take consecutive k-pairs, so the transposing writes of a wave fall
// in consecutive dwords (a one-element-per-lane transpose put every lane of
// a wave on the same bank).  Eight tasks per lane are loaded before any is
// stored, so their latencies overlap.
template <int DT, int NT, bool TRANS_B>
__device__ inline void skinny_load_w(const SkinnyArgs& p, uint16_t* wt, int tid) {
    constexpr int NP = NT * 16;
    constexpr int NTH = SKINNY_WAVES * 64;
    const bool vec_w = (p.vec_c & 2) != 0;  // W rows allow aligned 16-byte loads
    if constexpr (TRANS_B) {
        const int per_line = p.K / 8;
        const int ntask = NP * per_line;
        for (int t0 = 0; t0 < ntask; t0 += 8 * NTH) {
            u32x4 v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = t0 + i * NTH + tid;
                v[i] = (u32x4){0, 0, 0, 0};
                const int n = t / per_line, k8 = (t - n * per_line) * 8;
                if (t < ntask && n < p.N) {
                    const int64_t idx = (int64_t)n * p.ldw + k8;
                    v[i] = vec_w ? load16((const char*)p.W + idx * 2) : load_chunk_masked<DT>(p.W, idx, 8);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = t0 + i * NTH + tid;
                const int n = t / per_line, k8 = (t - n * per_line) * 8;
                if (t < ntask) *(u32x4*)(wt + n * p.pitch + k8) = v[i];
            }
        }
    } else {
        const int kp_count = p.K / 2;
        const int ntask = kp_count * (NP / 8);
        for (int t0 = 0; t0 < ntask; t0 += 4 * NTH) {
            u32x4 v0[4], v1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + i * NTH + tid;
                v0[i] = v1[i] = (u32x4){0, 0, 0, 0};
                const int n8 = (t / kp_count) * 8, kp = t - (t / kp_count) * kp_count;
                if (t >= ntask || n8 >= p.N) continue;
                const int64_t i0 = (int64_t)(2 * kp) * p.ldw + n8, i1 = i0 + p.ldw;
                if (vec_w && n8 + 8 <= p.N) {
                    v0[i] = load16((const char*)p.W + i0 * 2);
                    v1[i] = load16((const char*)p.W + i1 * 2);
                } else {
                    v0[i] = load_chunk_masked<DT>(p.W, i0, p.N - n8);
                    v1[i] = load_chunk_masked<DT>(p.W, i1, p.N - n8);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + i * NTH + tid;
                if (t >= ntask) continue;
                const int n8 = (t / kp_count) * 8, kp = t - (t / kp_count) * kp_count;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t lo = (v0[i][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    const uint32_t hi = (v1[i][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    *(uint32_t*)(wt + (n8 + e) * p.pitch + 2 * kp) = lo | (hi << 16);
                }
            }
        }
    }
}

// The X operand registers of one wave's RB x 16 rows starting at row base.
template <int RB>
__device__ inline void skinny_load_x(const SkinnyArgs& p, int base, int lane,
                                     u32x4 (&xf)[RB][SKINNY_KBMAX]) {
    const int KB = p.K / 32;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int m = base + rb * 16 + (lane & 15);
        if (m >= p.M) m = p.M - 1;  // rows past the end: valid memory, never stored
        const char* row = (const char*)p.X + ((int64_t)m * p.ldx + 8 * (lane >> 4)) * 2;
#pragma unroll
        for (int kb = 0; kb < SKINNY_KBMAX; ++kb)
            if (kb < KB) xf[rb][kb] = load16(row + kb * 64);
    }
}

// Dynamic LDS: W^T (NT*16 rows x pitch elements), then one output staging
// tile per wave (RB*16 rows x (NT*16*out_bytes + 16) bytes).
__host__ __device__ inline size_t skinny_lds_bytes(int nt, int pitch, int out_bytes) {
    return (size_t)nt * 16 * pitch * 2 +
           (size_t)SKINNY_WAVES * skinny_rb(nt) * 16 * (nt * 16 * out_bytes + 16);
}

template <int DT, int NT, bool TRANS_B>
__global__ __launch_bounds__(SKINNY_WAVES * 64, 2) void gemm_skinny_kernel(SkinnyArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint16_t wt[];  // NT*16 rows x pitch
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int RB = skinny_rb(NT);
    const int KB = p.K / 32;
    const int rows_per_step = SKINNY_WAVES * RB * 16 * gridDim.x;
    int base = (blockIdx.x * SKINNY_WAVES + wave) * RB * 16;

    // The first rows' X loads go out before W is staged, so the two overlap.
    u32x4 xf[RB][SKINNY_KBMAX];
    if (base < p.M) skinny_load_x(p, base, lane, xf);
    skinny_load_w<DT, NT, TRANS_B>(p, wt, tid);
    __syncthreads();

    const uint16_t* wrow = wt + (lane & 15) * p.pitch + 8 * (lane >> 4);
    const int ob = p.c_type == OUT_F32 ? 4 : 2;
    char* stage = (char*)(wt + NT * 16 * p.pitch) + wave * (RB * 16 * (NT * 16 * ob + 16));
    for (; base < p.M; base += rows_per_step) {
        f32x4 acc[RB][NT];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[rb][nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < SKINNY_KBMAX; ++kb) {
            if (kb >= KB) break;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const u32x4 wf = *(const u32x4*)(wrow + nt * 16 * p.pitch + kb * 32);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) mma_chunk<DT>(acc[rb][nt], wf, xf[rb][kb]);
            }
        }
        // the next rows' loads overlap this epilogue's stores
        if (base + rows_per_step < p.M) skinny_load_x(p, base + rows_per_step, lane, xf);
        if (p.c_type == OUT_F16)
            skinny_finish<DT, OUT_F16, NT, RB>(p, acc, base, lane, stage);
        else if (p.c_type == OUT_BF16)
            skinny_finish<DT, OUT_BF16, NT, RB>(p, acc, base, lane, stage);
        else
            skinny_finish<DT, OUT_F32, NT, RB>(p, acc, base, lane, stage);
    }
}

}  // namespace dge
