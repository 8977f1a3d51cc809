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


// K-quant super-blocks (256 weights) -> binary16, same page, §3.2 (one
// dequant kernel per weight type, float arithmetic then one conversion to
// binary16).
//   q6_K (QT = KQ_Q6_K, or KQ_Q6_K_224 for the same bytes padded to a
//     224-byte stride), 210 bytes: ql[128] low 4 bits, qh[64] high 2 bits,
//     int8 scales sc[16] at byte 192, binary16 d at 208.  Weight e = 128 h +
//     32 tt + l takes the low (tt < 2) or high nibble of ql[64 h + 32 (tt & 1)
//     + l], the 2 bits (qh[32 h + l] >> 2 tt) & 3 and sc[8 h + 2 tt + l / 16];
//     value d * sc * (q - 32), exact in fp32 (<= 24 significant bits), rounded
//     once to binary16.
//   q4_K (QT = KQ_Q4_K), 144 bytes: binary16 d and dmin, 12 bytes of 6-bit
//     scales and mins for 8 sub-blocks of 32, qs[128]; sub-blocks 2p and 2p + 1
//     take the low and high nibbles of qs[32 p .. 32 p + 31]; value d sc q -
//     dmin m in fp32 (both products exact, the difference rounded once), then
//     rounded to binary16: two roundings, which differ from one rounding of
//     the exact value when the binary32 result is a binary16 tie.
//   q4_0 rows of a multiple of 256 weights (QT = KQ_Q4_0_256) take the same
//     path as groups of eight 18-byte blocks, 144 bytes per 256 weights:
//     persistent workgroups with the next group prefetched into registers
//     move them faster than the one-step-per-workgroup q4_0 kernel above.
// A workgroup stages SB consecutive super-blocks (SB a multiple of 8: 1680,
// 1792 or 1152 bytes per 8, multiples of 16) into LDS with coalesced loads; task c
// then decodes the 16-byte output chunk c % 32 (weights 8 (c % 32) .. + 7) of
// super-block c / 32, consecutive threads writing consecutive chunks.
constexpr int KQ_STEP = 16;    // super-blocks per workgroup step
constexpr int KQ_GRID = 2048;  // most workgroups a launch uses

template <int QT> struct KQuant;
// BYTES: block stride; Q6: the q6_K fields (the 224-byte layout is the 210
// bytes of a q6_K super-block followed by 14 unused bytes)
template <> struct KQuant<KQ_Q4_K> { static constexpr int BYTES = 144; static constexpr bool Q6 = false; };
template <> struct KQuant<KQ_Q6_K> { static constexpr int BYTES = 210; static constexpr bool Q6 = true; };
template <> struct KQuant<KQ_Q6_K_224> { static constexpr int BYTES = 224; static constexpr bool Q6 = true; };
template <> struct KQuant<KQ_Q4_0_256> { static constexpr int BYTES = 144; static constexpr bool Q6 = false; };

template <int QT, int SB>
__global__ __launch_bounds__(256) void dequant_kq_f16_kernel(const uint8_t* __restrict__ q,
                                                             uint16_t* __restrict__ out,
                                                             int64_t rows, int64_t cols,
                                                             int64_t ldo, int flags) {
    constexpr int BYTES = KQuant<QT>::BYTES;
    static_assert(SB % 8 == 0, "groups of 8 super-blocks keep 16-byte alignment");
    // (16 spare bytes: the q4_0 decode reads whole dwords past a block's end)
    __shared__ __attribute__((aligned(16))) uint8_t raw[SB * BYTES + 16];
    const bool vec_in = (flags & 1) != 0, vec_out = (flags & 2) != 0;
    const bool off32 = (flags & 4) != 0;  // (SB + 1) rows of out span < 2^31 bytes
    const int tid = threadIdx.x;
    const int64_t nsb = cols / 256;
    const int64_t total = rows * nsb;
    // 16-byte input chunks per thread per step; with aligned input the next
    // step's chunks are loaded into registers while this step is decoded
    constexpr int NCH = (SB * BYTES + 16 * 256 - 1) / (16 * 256);
    u32x4 pre[NCH];
    auto fetch = [&](int64_t g) {
        const int nb = (int)(total - g < SB ? total - g : SB);
        const uint8_t* src = q + BYTES * g;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int c = tid + 256 * i;
            if (c < nb * BYTES / 16) pre[i] = *(const u32x4*)(src + 16 * c);
        }
    };
    const int64_t gstep = (int64_t)gridDim.x * SB;
    if (vec_in && (int64_t)blockIdx.x * SB < total) fetch((int64_t)blockIdx.x * SB);
    for (int64_t g0 = (int64_t)blockIdx.x * SB; g0 < total; g0 += gstep) {
        const int nblk = (int)(total - g0 < SB ? total - g0 : SB);
        const int bytes = nblk * BYTES;
        const uint8_t* src = q + BYTES * g0;
        int done = 0;
        if (vec_in) {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int c = tid + 256 * i;
                if (c < bytes / 16) *(u32x4*)(raw + 16 * c) = pre[i];
            }
            done = bytes / 16 * 16;
        }
        for (int i = done + tid; i < bytes; i += 256) raw[i] = src[i];
        // first super-block of the step: row r0, column c0 (one 64-bit division per step)
        const int64_t r0 = g0 / nsb;
        const uint32_t c0 = (uint32_t)(g0 - r0 * nsb), unsb = (uint32_t)nsb;
        uint16_t* orow = out + r0 * ldo;  // row r0 of the output
        const bool wide = nsb >= SB;      // a step then crosses at most one row end
        const uint32_t ldo32 = (uint32_t)ldo;
        __syncthreads();
        if (vec_in && g0 + gstep < total) fetch(g0 + gstep);
        for (int task = tid; task < 32 * nblk; task += 256) {
            const int sbl = task >> 5, c = task & 31;
            const uint8_t* blk = raw + BYTES * sbl;
            const int e0 = 8 * c;
            uint16_t h[8];
            uint32_t hw[4];  // the eight results as pairs (the q4_0 path)
            if constexpr (QT == KQ_Q4_0_256) {
                // chunk c % 4 of q4_0 block c / 4 of the group: the low (chunk
                // < 2) or high nibbles of code bytes 8 (chunk & 1) .. + 7.
                // The block starts at an even byte o; its fields are read as
                // whole dwords from o rounded down to 4 and aligned with
                // alignbit.  Each code becomes the binary16 1024 + q by
                // placing the byte 0x64 above it, minus 1032 is q - 8 exactly,
                // and one packed multiply by d rounds d (q - 8) once: the same
                // bits as the binary32 product rounded to binary16.
                const int p = c & 3;
                const int o = BYTES * sbl + 18 * (c >> 2);
                const uint32_t* rw = (const uint32_t*)(raw + (o & ~3));
                const uint32_t hs = (uint32_t)(o & 2) * 8;  // 0 or 16 bits
                const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)(rw[0] >> hs));
                const int rel = (o & 2) + 2 + 8 * (p & 1);  // code bytes past o & ~3
                const uint32_t w0 = rw[rel >> 2], w1 = rw[(rel >> 2) + 1], w2 = rw[(rel >> 2) + 2];
                const uint32_t bs = (uint32_t)(rel & 3) * 8;
                uint32_t c03 = __builtin_amdgcn_alignbit(w1, w0, bs);  // code bytes 0-3
                uint32_t c47 = __builtin_amdgcn_alignbit(w2, w1, bs);  // code bytes 4-7
                if (p >= 2) {
                    c03 >>= 4;
                    c47 >>= 4;
                }
                c03 &= 0x0F0F0F0Fu;
                c47 &= 0x0F0F0F0Fu;
                typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
                const h2_t off = {(_Float16)1032.0f, (_Float16)1032.0f}, d2 = {d, d};
                // perm selectors: 0-3 pick bytes of the codes, 4 the byte 0x64
                const uint32_t v[4] = {__builtin_amdgcn_perm(0x64646464u, c03, 0x04010400u),
                                       __builtin_amdgcn_perm(0x64646464u, c03, 0x04030402u),
                                       __builtin_amdgcn_perm(0x64646464u, c47, 0x04010400u),
                                       __builtin_amdgcn_perm(0x64646464u, c47, 0x04030402u)};
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    hw[i] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(h2_t, v[i]) - off) * d2);
            } else if constexpr (KQuant<QT>::Q6) {
                // eight consecutive weights share tt, hh and the scale: their
                // low bits are 8 consecutive ql bytes and their high bits 8
                // consecutive qh bytes, read as dwords (the block starts at an
                // even byte o) and combined four codes to a dword
                const int hh = e0 / 128, tt = (e0 % 128) / 32, l0 = e0 % 32;
                const int o = BYTES * sbl;
                const uint32_t* rw = (const uint32_t*)(raw + (o & ~3));
                const uint32_t bs = (uint32_t)(o & 2) * 8;  // 0 or 16 bits
                const int rl = (o & 2) + 64 * hh + 32 * (tt & 1) + l0;  // ql bytes past o & ~3
                const int rh = (o & 2) + 128 + 32 * hh + l0;            // qh bytes
                const int rd = (o & 2) + 208;                           // d
                uint32_t lo03 = __builtin_amdgcn_alignbit(rw[(rl >> 2) + 1], rw[rl >> 2], bs);
                uint32_t lo47 = __builtin_amdgcn_alignbit(rw[(rl >> 2) + 2], rw[(rl >> 2) + 1], bs);
                const uint32_t hi03 = __builtin_amdgcn_alignbit(rw[(rh >> 2) + 1], rw[rh >> 2], bs);
                const uint32_t hi47 = __builtin_amdgcn_alignbit(rw[(rh >> 2) + 2], rw[(rh >> 2) + 1], bs);
                if (tt >= 2) {
                    lo03 >>= 4;
                    lo47 >>= 4;
                }
                const uint32_t q03 = (lo03 & 0x0F0F0F0Fu) | (((hi03 >> (2 * tt)) & 0x03030303u) << 4);
                const uint32_t q47 = (lo47 & 0x0F0F0F0Fu) | (((hi47 >> (2 * tt)) & 0x03030303u) << 4);
                const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(rw[rd >> 2] >> bs));
                const float dsc = d * (float)(int8_t)blk[192 + 8 * hh + 2 * tt + l0 / 16];  // exact
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t qw = i < 4 ? q03 : q47;
                    const float code = (float)((qw >> (8 * (i & 3))) & 0xFFu) - 32.0f;  // exact
                    // exact product, one rounding; the empty asm keeps the
                    // multiply a multiply (folded into a mixed-precision FMA it
                    // adds +0, which turns a -0 product into +0)
                    float v = dsc * code;
                    __asm__("" : "+v"(v));
                    h[i] = __builtin_bit_cast(uint16_t, (_Float16)v);
                }
            } else {
                const int p = e0 / 64, w0 = e0 % 64, j = 2 * p + (w0 >= 32);
                const float d = (float)__builtin_bit_cast(_Float16, (uint16_t)(blk[0] | (blk[1] << 8)));
                const float dmin = (float)__builtin_bit_cast(_Float16, (uint16_t)(blk[2] | (blk[3] << 8)));
                const uint8_t* s12 = blk + 4;
                int sc, m;
                if (j < 4) {
                    sc = s12[j] & 63;
                    m = s12[j + 4] & 63;
                } else {
                    sc = (s12[j + 4] & 15) | ((s12[j - 4] >> 6) << 4);
                    m = (s12[j + 4] >> 4) | ((s12[j] >> 6) << 4);
                }
                const float a = d * (float)sc, u = dmin * (float)m;  // both exact
                // the 8 code bytes (16-byte-aligned block, 8-aligned bytes): one
                // 8-byte read, the low or high nibbles of each byte
                uint2 qw = *(const uint2*)(blk + 16 + 32 * p + (w0 & 31));
                if (w0 >= 32) {
                    qw.x >>= 4;
                    qw.y >>= 4;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t code = ((i < 4 ? qw.x : qw.y) >> (8 * (i & 3))) & 15u;
                    // a * code is exact, so the fused form rounds the difference
                    // once, to binary32; the empty asm keeps that binary32 value
                    // (otherwise the compiler folds fma and conversion into one
                    // mixed-precision FMA that rounds straight to binary16, which
                    // differs at binary16 ties)
                    float v = __builtin_fmaf(a, (float)code, -u);
                    __asm__("" : "+v"(v));
                    h[i] = __builtin_bit_cast(uint16_t, (_Float16)v);
                }
            }
            if constexpr (QT != KQ_Q4_0_256) {
#pragma unroll
                for (int i = 0; i < 4; ++i) hw[i] = (uint32_t)h[2 * i] | ((uint32_t)h[2 * i + 1] << 16);
            }
            const uint32_t cc = c0 + (uint32_t)sbl;  // < nsb + SB
            uint16_t* dst;
            if (off32 && wide) {
                // row r0 or r0 + 1: a 32-bit offset from row r0
                const uint32_t off = cc >= unsb ? ldo32 + 256u * (cc - unsb) : 256u * cc;
                dst = orow + (off + (uint32_t)e0);
            } else {
                const uint32_t dr = cc / unsb;
                dst = out + (r0 + dr) * ldo + 256 * (cc - dr * unsb) + e0;
            }
            if (vec_out) {
                *(u32x4*)dst = (u32x4){hw[0], hw[1], hw[2], hw[3]};
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dst[2 * i] = (uint16_t)(hw[i] & 0xFFFFu);
                    dst[2 * i + 1] = (uint16_t)(hw[i] >> 16);
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace dge
