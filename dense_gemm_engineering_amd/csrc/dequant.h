// q4 -> binary16 weight expansion ("02 · 8m/8m② — Tiled wmma f16 prefill
// GEMM", §2.3 and its q4_0 dequant kernel in §3.2).
//
// Block (r, b) of an N x K weight is 18 bytes at 18 * (r * K/32 + b): a
// little-endian binary16 scale d, then 16 code bytes; byte i carries element
// i in its low nibble and element i + 16 in its high nibble, and code q
// stands for d * (q - 8).
//
// The pass is HBM-bound (2.5625 bytes per weight: 0.5625 read, 2 written).
// A workgroup takes 256 consecutive blocks (4608 contiguous bytes, 16-byte
// aligned when q is, since 256 * 18 is a multiple of 16), brings them into
// LDS with coalesced 16-byte loads, and then each thread produces 16-byte
// output chunks (8 weights) from LDS, consecutive threads writing consecutive
// chunks.  Chunk p (0..3) of a block holds elements 8p..8p+7: the low
// (p < 2) or high (p >= 2) nibbles of code bytes 8 (p & 1) .. 8 (p & 1) + 7.
// Reading the raw bytes from LDS avoids the 2-byte scattered global loads a
// thread-per-chunk decode would need (blocks start at 2-byte boundaries, so
// no wide global load can address a block's fields directly; cf. the
// misaligned-load pitfall of §3.3).
//
// d * (q - 8) is exact in fp32 (11-bit significand times a 4-bit integer),
// and the conversion to binary16 rounds to nearest-even with subnormals kept,
// so the result is bit-identical to a single rounding of the exact product.
#pragma once

#include "device_common.h"

namespace dge {

constexpr int DQ_BLOCKS = 256;  // q4 blocks per workgroup step

__global__ __launch_bounds__(256) void dequant_q4_f16_kernel(const uint8_t* __restrict__ q,
                                                             uint16_t* __restrict__ out,
                                                             int64_t rows, int64_t cols,
                                                             int64_t ldo, int flags) {
    __shared__ __attribute__((aligned(16))) uint8_t raw[DQ_BLOCKS * 18];
    const bool vec_in = (flags & 1) != 0, vec_out = (flags & 2) != 0;
    const int tid = threadIdx.x;
    const int64_t nb = cols / 32;
    const int64_t total = rows * nb;
    for (int64_t b0 = (int64_t)blockIdx.x * DQ_BLOCKS; b0 < total;
         b0 += (int64_t)gridDim.x * DQ_BLOCKS) {
        const int nblk = (int)(total - b0 < DQ_BLOCKS ? total - b0 : DQ_BLOCKS);
        const int bytes = nblk * 18;
        const uint8_t* src = q + 18 * b0;
        int done = 0;
        if (vec_in) {
            for (int c = tid; c < bytes / 16; c += 256) *(u32x4*)(raw + 16 * c) = *(const u32x4*)(src + 16 * c);
            done = bytes / 16 * 16;
        }
        for (int i = done + tid; i < bytes; i += 256) raw[i] = src[i];
        // first block of the step: row r0, block column c0 (one 64-bit division per step)
        const int64_t r0 = b0 / nb;
        const uint32_t c0 = (uint32_t)(b0 - r0 * nb), unb = (uint32_t)nb;
        __syncthreads();
        for (int j = tid; j < nblk * 4; j += 256) {
            const int blk = j >> 2, part = j & 3;
            const uint8_t* bb = raw + 18 * blk;
            const float d = (float)__builtin_bit_cast(_Float16, *(const uint16_t*)bb);
            const uint16_t* qs = (const uint16_t*)(bb + 2 + 8 * (part & 1));
            const int shift = (part >> 1) * 4;
            uint32_t o[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t two = qs[w];  // code bytes 2w (low half) and 2w + 1 (high half)
                const int q0 = (int)((two >> shift) & 15u);
                const int q1 = (int)((two >> (8 + shift)) & 15u);
                const uint16_t h0 = __builtin_bit_cast(uint16_t, (_Float16)(d * (float)(q0 - 8)));
                const uint16_t h1 = __builtin_bit_cast(uint16_t, (_Float16)(d * (float)(q1 - 8)));
                o[w] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            }
            const uint32_t cc = c0 + (uint32_t)blk;   // < nb + 256
            const uint32_t dr = cc / unb;
            uint16_t* dst = out + (r0 + dr) * ldo + 32 * (cc - dr * unb) + 8 * part;
            if (vec_out) {
                *(u32x4*)dst = (u32x4){o[0], o[1], o[2], o[3]};
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    dst[2 * w] = (uint16_t)(o[w] & 0xffff);
                    dst[2 * w + 1] = (uint16_t)(o[w] >> 16);
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace dge
