// q4 -> binary16 weight expansion ("02 · 8m/8m② — Tiled wmma f16 prefill
// GEMM", §2.3 and its q4_0 dequant kernel in §3.2).
//
// Block (r, b) of an N x K weight is 18 bytes at 18 * (r * K/32 + b): a
// little-endian binary16 scale d, then 16 code bytes; byte i carries element
// i in its low nibble and element i + 16 in its high nibble, and code q
// stands for d * (q - 8).
//
// The pass is HBM-bound (2.5625 bytes per weight: 0.5625 read, 2 written), so
// the thread mapping is chosen for the stores: one thread produces one
// 16-byte chunk of output (8 consecutive weights), so consecutive lanes write
// consecutive 16-byte chunks and a wave writes 1 KB of contiguous row.  Chunk
// p (0..3) of a block holds elements 8p..8p+7: the low (p < 2) or high
// (p >= 2) nibbles of code bytes 8 (p & 1) .. 8 (p & 1) + 7.  The four lanes
// of a block read the same 18 bytes, which the L1/L2 serve after the first;
// every load is 2-byte aligned because blocks start at even offsets (a wide
// load at block + 2 would not be, cf. the misaligned-load pitfall of §3.3).
//
// d * (q - 8) is exact in fp32 (11-bit significand times a 4-bit integer),
// and the conversion to binary16 rounds to nearest-even with subnormals kept,
// so the result is bit-identical to a single rounding of the exact product.
#pragma once

#include "device_common.h"

namespace dge {

__global__ __launch_bounds__(256) void dequant_q4_f16_kernel(const uint8_t* __restrict__ q,
                                                             uint16_t* __restrict__ out,
                                                             int64_t rows, int64_t cols,
                                                             int64_t ldo, int vec_out) {
    const int64_t cpr = cols / 8;  // output chunks per row
    const int64_t total = rows * cpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += stride) {
        const int64_t r = c / cpr;
        const int64_t cc = c - r * cpr;
        const int64_t b = cc >> 2;
        const int part = (int)(cc & 3);
        const uint8_t* blk = q + 18 * (r * (cols / 32) + b);
        const float d = (float)__builtin_bit_cast(_Float16, *(const uint16_t*)blk);
        const uint16_t* qs = (const uint16_t*)(blk + 2 + 8 * (part & 1));
        const int shift = (part >> 1) * 4;
        uint32_t o[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t two = qs[w];  // code bytes 2w (low half) and 2w + 1 (high half)
            const int c0 = (int)((two >> shift) & 15u);
            const int c1 = (int)((two >> (8 + shift)) & 15u);
            const uint16_t h0 = __builtin_bit_cast(uint16_t, (_Float16)(d * (float)(c0 - 8)));
            const uint16_t h1 = __builtin_bit_cast(uint16_t, (_Float16)(d * (float)(c1 - 8)));
            o[w] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        }
        uint16_t* dst = out + r * ldo + 32 * b + 8 * part;
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
}

}  // namespace dge
