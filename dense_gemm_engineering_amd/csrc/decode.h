// Decode-shaped GEMM: C = epi(alpha X W^T + beta C) for a few input rows
// (M <= 64) against an N x K weight ("Matrix Multiplication: The Operation
// Behind Modern AI", "The shape a language model actually runs": at M = 1
// the best possible intensity is ~1 FLOP per byte, so the time is the time
// to read W once).  Everything is arranged around streaming W from HBM:
//
//  * A workgroup owns 16 weight rows and all M input rows; its 8 waves split
//    K into 8 slices of whole 32-deep k-blocks.  Within a wave, the MFMA "A"
//    operand is 8 consecutive k of one weight row per lane and the "B"
//    operand 8 consecutive k of one row of X (L2-resident: X is at most 64 x
//    K).  Both are loaded in a coalesced layout and moved into the operand
//    layout through small per-wave LDS slots: the weight as whole rows (4
//    rows x 256 bytes per load, for whole batches inside K; the ragged end
//    of a slice loads in operand layout), X for M > 1 as 64-byte row pieces
//    per lane quad.  The product is C^T = W X^T in 16 x 16 blocks, MT =
//    ceil(M / 16) of them.
//  * Loads for 16 k-blocks (8 for M > 32) are issued before their MFMAs, so
//    each lane keeps up to 256 bytes of W (and of X) in flight; with 8 waves
//    per CU that is ~128 KB of W per CU, and a 4096-deep K costs each wave a
//    single round trip to memory.
//  * The 8 partial blocks are summed through LDS in a fixed order (slice 0
//    first), so results do not depend on timing, and the fused epilogue
//    writes 16 consecutive columns per output row.
#pragma once

#include "device_common.h"
#include "mfma_gemm.h"

namespace dge {

struct DecodeArgs {
    const void* X;  // M x K, row-major
    const void* W;  // N x K, row-major
    void* C;        // M x N
    int64_t ldx, ldw, ldc;
    int M, N, K;
    int c_type;
    Epilogue ep;
    // split schedule (gemm_decode_split_kernel): K slices and the fp32
    // partial sums (ksplit x M x N, ld N); rec (may be null): 4 real-time
    // counter values per workgroup
    int ksplit;
    float* ws;
    unsigned long long* rec;
};

constexpr int DECODE_WAVES = 8;
constexpr int DPAD = 17;  // floats per 16-wide row of a partial block in LDS
// k-blocks whose loads are issued together: 16 (a 4096-deep K in one round
// trip per wave) while the registers allow, 8 for M > 32
__host__ __device__ constexpr int decode_batch(int mt) { return mt <= 2 ? 16 : 8; }
// k-blocks per coalesced weight-load span: each load instruction then covers
// 4 whole rows x 256 bytes
constexpr int DSPAN = 4;

// XT: X goes through the per-wave transpose slot (below); off for M = 1,
// whose clamped rows make every quad read one address anyway.
template <int DT, int MT, bool XT = true>
__global__ __launch_bounds__(DECODE_WAVES * 64) void gemm_decode_kernel(DecodeArgs p) {
    // partial C^T blocks of every wave: [wave][mt][16 n][16 m] fp32, each n
    // row padded to DPAD floats so that the summation's reads (16 rows of one
    // column) fall in different banks
    __shared__ __attribute__((aligned(16))) float part[DECODE_WAVES][MT][16 * DPAD];
    // each wave's X transpose slot: MT blocks of 16 rows x 4 16-byte chunks
    __shared__ __attribute__((aligned(16))) u32x4 xslot[XT ? DECODE_WAVES : 1][MT][64];
    // each wave's weight transpose slot: 16 rows x 16 16-byte units
    __shared__ __attribute__((aligned(16))) u32x4 wslot[DECODE_WAVES][256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 16;
    const int nkb = (p.K + 31) / 32;
    const int kb0 = wave * nkb / DECODE_WAVES, kb1 = (wave + 1) * nkb / DECODE_WAVES;

    // this lane's weight row: n0 + (lane & 15) (clamped to the last row:
    // valid memory, never stored); input rows are clamped to M - 1 the same way
    const int nr = min(n0 + (lane & 15), p.N - 1);
    const char* wrow = (const char*)p.W + ((int64_t)nr * p.ldw + 8 * (lane >> 4)) * 2;
    // X is loaded with the four lanes of a quad on one row's 64 contiguous
    // bytes (lane L: row 16 mt + L / 4, chunk L % 4): in the MFMA operand
    // layout (row L % 16) every quad would touch four rows, and the address
    // unit spends a cycle per row (M = 64: 24.4 -> 19.1 us for the loads
    // alone).  Each k-block's X then goes through the wave's LDS slot into
    // the operand layout; chunk c of row r sits at r * 4 + (c ^ ((r >> 2) & 3)),
    // so the sixteen rows of one chunk fall in different bank groups.
    const int xrl = XT ? lane >> 2 : lane & 15, xcl = XT ? lane & 3 : lane >> 4;  // row, chunk
    const char* xrow[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int mr = min(16 * mt + xrl, p.M - 1);
        xrow[mt] = (const char*)p.X + ((int64_t)mr * p.ldx + 8 * xcl) * 2;
    }
    const int xw = 4 * (lane >> 2) + ((lane & 3) ^ ((lane >> 4) & 3));  // where this lane's load goes
    const int xr = 4 * (lane & 15) + ((lane >> 4) ^ ((lane >> 2) & 3));  // where its operand comes from
    const int kchunk = 8 * (lane >> 4);  // this lane's k offset within a k-block

    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    constexpr int DECODE_BATCH = decode_batch(MT);
    // the k-block's MFMAs on one weight fragment and the batch's X operands
    auto mma_kblock = [&](const u32x4& wfr, const u32x4 (&xfr)[MT]) __attribute__((always_inline)) {
        // the wave's own LDS operations complete in order: the reads see
        // these writes, and the next k-block's writes land after them
        u32x4 xo[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if constexpr (XT)
                xslot[wave][mt][xw] = xfr[mt];
            else
                xo[mt] = xfr[mt];
        }
        if constexpr (XT) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xo[mt] = xslot[wave][mt][xr];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) mma_chunk<DT>(acc[mt], wfr, xo[mt]);
    };

    // Whole batches inside K: the weight rows load as whole rows (load j of
    // a span: row n0 + 4 j + lane / 16, 16-byte unit lane % 16; rows past N
    // clamped, never stored) and each span's 16 rows go through the wave's
    // slot into operand layout (unit u of row r at r * 16 + (u ^ r):
    // conflict-free both ways).  In operand layout every load puts 16 rows
    // under one instruction and 4 under every lane quad, which the memory
    // pipeline moves at about half the rate.
    constexpr int NSP = DECODE_BATCH / DSPAN;  // spans per batch
    const int lr = lane >> 4, lu = lane & 15, orow = lane & 15, ochunk = lane >> 4;
    const char* wtile = (const char*)p.W + (int64_t)n0 * p.ldw * 2;
    uint32_t woff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        woff[j] = (uint32_t)((min(n0 + 4 * j + lr, p.N - 1) - n0) * p.ldw * 2 + 16 * lu);
    int kb = kb0;
    for (; kb + DECODE_BATCH <= kb1 && (kb + DECODE_BATCH) * 32 <= p.K; kb += DECODE_BATCH) {
        u32x4 raw[NSP][4], xf[DECODE_BATCH][MT];
#pragma unroll
        for (int sp = 0; sp < NSP; ++sp)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                raw[sp][j] = load16(wtile + (int64_t)(kb + DSPAN * sp) * 64 + woff[j]);
#pragma unroll
        for (int i = 0; i < DECODE_BATCH; ++i)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) xf[i][mt] = load16(xrow[mt] + (int64_t)(kb + i) * 64);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int sp = 0; sp < NSP; ++sp) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * j + lr;
                wslot[wave][r * 16 + (lu ^ r)] = raw[sp][j];
            }
            u32x4 wf[DSPAN];
#pragma unroll
            for (int i = 0; i < DSPAN; ++i) wf[i] = wslot[wave][orow * 16 + ((4 * i + ochunk) ^ orow)];
#pragma unroll
            for (int i = 0; i < DSPAN; ++i) mma_kblock(wf[i], xf[DSPAN * sp + i]);
        }
    }
    // the rest (a short or ragged end of the wave's k-blocks): fragments in
    // operand layout, masked by k
    for (; kb < kb1; kb += DECODE_BATCH) {
        u32x4 wf[DECODE_BATCH], xf[DECODE_BATCH][MT];
#pragma unroll
        for (int i = 0; i < DECODE_BATCH; ++i) {
            // K % 8 == 0: a chunk is all in or all out (W and X lanes hold
            // different chunks, each masked by its own k)
            const int k = (kb + i) * 32 + kchunk, kx = (kb + i) * 32 + 8 * xcl;
            const bool in = kb + i < kb1 && k < p.K, inx = kb + i < kb1 && kx < p.K;
            wf[i] = in ? load16(wrow + (int64_t)(kb + i) * 64) : (u32x4){0, 0, 0, 0};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                xf[i][mt] = inx ? load16(xrow[mt] + (int64_t)(kb + i) * 64) : (u32x4){0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < DECODE_BATCH; ++i) mma_kblock(wf[i], xf[i]);
    }

    // lane holds C^T rows n = 4 (lane / 16) + e, column m = lane % 16 of each block
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[wave][mt][(4 * (lane >> 4) + e) * DPAD + (lane & 15)] = acc[mt][e];
    __syncthreads();

    // output (m, n0 + j) for t = 16 m + j: 16 consecutive columns per row
    for (int t = tid; t < 16 * p.M; t += DECODE_WAVES * 64) {
        const int m = t >> 4, j = t & 15, n = n0 + j;
        if (n >= p.N) continue;
        const int mt = m >> 4, ml = m & 15;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < DECODE_WAVES; ++w) s += part[w][mt][j * DPAD + ml];  // m < 16 MT
        const int64_t idx = (int64_t)m * p.ldc + n;
        if (p.c_type == OUT_F32) {
            float* c = (float*)p.C + idx;
            *c = apply_epilogue<DT>(p.ep, s, p.ep.beta != 0.0f ? *c : 0.0f, n);
        } else if (p.c_type == OUT_F16) {
            _Float16* c = (_Float16*)p.C + idx;
            *c = (_Float16)apply_epilogue<DT>(p.ep, s, p.ep.beta != 0.0f ? (float)*c : 0.0f, n);
        } else {
            __bf16* c = (__bf16*)p.C + idx;
            *c = (__bf16)apply_epilogue<DT>(p.ep, s, p.ep.beta != 0.0f ? (float)*c : 0.0f, n);
        }
    }
}

// Split schedule for 17 <= M <= 64 rows (the kernel above re-reads all of X
// for every 16 weight rows: at M = 64 that is four times the weight's own
// bytes).  A workgroup owns DSPLIT_ROWS = 64 weight rows and one of ksplit
// K slices (grid (N / 64) x ksplit, 256 workgroups for N = 4096 with ksplit
// = 4), so X crosses from L2 once per workgroup and slice: as many bytes as
// the weight.  Its 8 waves split the slice's k-blocks.
//
//  * Weight loads are coalesced: a wave takes its k-blocks in spans of
//    DSPAN = 4 (128 k, 256 bytes of a row), and each 16-byte load
//    instruction covers 4 whole rows x 256 bytes (lane L: row L / 16,
//    16-byte unit L % 16).  The MFMA operand layout (lane L: row L % 16) puts
//    16 rows under every instruction and 4 rows under every lane quad, and
//    the memory pipeline then moves the same bytes at about half the rate
//    (M = 64 on a 4096 x 4096 weight: 7.7 -> 4.4 us median for a wave's
//    loads).  Each 16-row group goes through a 4 KB slot of the wave's own
//    LDS (16-byte unit u of row r at r * 16 + (u ^ r): conflict-free both
//    ways) into operand layout.
//  * The 8 waves' partial C^T blocks are summed through LDS in wave order
//    (the slots alias each wave's own part of that buffer) and written to
//    ws[slice][m][n]; the split-K fixup sums the slices in slice order and
//    applies the epilogue, so the result does not depend on timing.  (A
//    last-arriving workgroup finishing C in this launch was slower here: the
//    device-scope stores, counter and loads it needs cost ~4 round trips of
//    ~1.5 us to the memory side, against ~2.7 us for the fixup launch.)
constexpr int DSPLIT_ROWS = 64;

template <int DT, int MT>
__global__ __launch_bounds__(DECODE_WAVES * 64) void gemm_decode_split_kernel(DecodeArgs p) {
    constexpr int NB = DSPLIT_ROWS / 16;  // weight blocks per workgroup
    // each wave's partial rows of C: row m (of 16 MT) holds the slice's
    // DSPLIT_ROWS columns at a pitch of DROW floats, so that a lane's 4
    // consecutive columns of one block leave as one 16-byte write and the
    // summation reads 16 bytes per wave (written as single floats, the
    // reduction took ~1 us at M = 64).  The 272-byte pitch puts the 16 rows
    // one write instruction covers on different banks.  During the main loop
    // each wave's part holds its transpose slot.
    constexpr int DROW = DSPLIT_ROWS + 4;
    constexpr int PWORDS = 16 * MT * DROW > 1024 ? 16 * MT * DROW : 1024;
    __shared__ __attribute__((aligned(16))) float part[DECODE_WAVES][PWORDS];
    static_assert(PWORDS * 4 >= 16 * 16 * 16, "transpose slot fits a wave's part");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    unsigned long long t_start = 0, t_land = 0;
    if (p.rec && tid == 0) t_start = __builtin_amdgcn_s_memrealtime();
    const int ntile = p.N / DSPLIT_ROWS;
    const int nb_i = blockIdx.x % ntile, ks = blockIdx.x / ntile;
    const int n0 = nb_i * DSPLIT_ROWS;
    const int nkb = p.K / 32;
    const int s0 = ks * nkb / p.ksplit, s1 = (ks + 1) * nkb / p.ksplit;  // the slice's k-blocks
    const int kb0 = s0 + wave * (s1 - s0) / DECODE_WAVES;
    const int kb1 = s0 + (wave + 1) * (s1 - s0) / DECODE_WAVES;
    const int lr = lane >> 4, lu = lane & 15;  // load layout: row within 4, 16-byte unit
    const int orow = lane & 15, ochunk = lane >> 4;  // operand layout: row, 8-element chunk
    u32x4* slot = (u32x4*)&part[wave][0];

    f32x4 acc[NB][MT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[b][mt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // per-lane byte offsets: W row n0 + 16 g + 4 j + lr is the uniform
    // (16 g + 4 j) x ldw on top of lr x ldw.  X (L2-resident, shared by the
    // slice's workgroups) is loaded straight in operand layout: a coalesced
    // load and transpose measured the same.  Its rows are clamped to M - 1
    // (rows past M feed only outputs that are never stored).
    const uint32_t wlane = (uint32_t)(lr * p.ldw * 2 + 16 * lu);
    uint32_t xlane[MT];
#pragma unroll
    for (int g = 0; g < MT; ++g)
        xlane[g] = (uint32_t)((min(16 * g + orow, p.M - 1) * p.ldx + 8 * ochunk) * 2);
    const char* wtile = (const char*)p.W + (int64_t)n0 * p.ldw * 2;

    // whole spans
    int kbs = kb0;
    for (; kbs + DSPAN <= kb1; kbs += DSPAN) {
        u32x4 rw[NB][4], xf[MT][DSPAN];
        const char* wk = wtile + (int64_t)kbs * 64;
        const char* xk = (const char*)p.X + (int64_t)kbs * 64;
#pragma unroll
        for (int g = 0; g < NB; ++g) {
#pragma unroll
            for (int j = 0; j < 4; ++j) rw[g][j] = load16(wk + (int64_t)(16 * g + 4 * j) * p.ldw * 2 + wlane);
            if (g < MT) {
#pragma unroll
                for (int kb = 0; kb < DSPAN; ++kb) xf[g][kb] = load16(xk + xlane[g] + kb * 64);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if (p.rec && tid == 0 && kbs == kb0) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            t_land = __builtin_amdgcn_s_memrealtime();
        }
        // 16-row group -> operand fragments of its DSPAN k-blocks; the wave's
        // LDS operations complete in order, so a slot's next writes land
        // after its reads
        u32x4 wf[NB][DSPAN];
        auto transpose = [&](const u32x4(&raw)[4], u32x4(&fr)[DSPAN]) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * j + lr;
                slot[r * 16 + (lu ^ r)] = raw[j];
            }
#pragma unroll
            for (int kb = 0; kb < DSPAN; ++kb) fr[kb] = slot[orow * 16 + ((4 * kb + ochunk) ^ orow)];
        };
#pragma unroll
        for (int g = 0; g < NB; ++g) {
            transpose(rw[g], wf[g]);
            // the blocks groups 0..g complete: (g, mt <= g) and (b < g, g)
#pragma unroll
            for (int kb = 0; kb < DSPAN; ++kb) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    if (mt <= g) mma_chunk<DT>(acc[g][mt], wf[g][kb], xf[mt][kb]);
                if (g < MT) {
#pragma unroll
                    for (int b = 0; b < g; ++b) mma_chunk<DT>(acc[b][g], wf[b][kb], xf[g][kb]);
                }
            }
        }
    }
    // the last 1..3 k-blocks (a slice that is not whole spans): fragments
    // loaded straight in operand layout
    for (; kbs < kb1; ++kbs) {
        u32x4 wf[NB], xf[MT];
#pragma unroll
        for (int b = 0; b < NB; ++b)
            wf[b] = load16(wtile + ((int64_t)(16 * b + orow) * p.ldw + kbs * 32 + 8 * ochunk) * 2);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            xf[mt] = load16((const char*)p.X +
                            ((int64_t)min(16 * mt + orow, p.M - 1) * p.ldx + kbs * 32 + 8 * ochunk) * 2);
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) mma_chunk<DT>(acc[b][mt], wf[b], xf[mt]);
    }
    // lane holds C^T rows n = 4 (lane / 16) + e, column m = lane % 16 of each
    // block: columns 16 b + 4 (lane / 16) .. + 3 of row 16 mt + lane % 16
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            *(f32x4*)&part[wave][(mt * 16 + (lane & 15)) * DROW + b * 16 + 4 * (lane >> 4)] = acc[b][mt];
    __syncthreads();
    unsigned long long t_loop = 0;
    if (p.rec && tid == 0) t_loop = __builtin_amdgcn_s_memrealtime();

    // the slice's partial, 4 columns per thread (t = 16 m + q: columns
    // n0 + 4 q .. + 3 of row m): a wave stores 4 rows x 256 contiguous bytes
    float* ws = p.ws + (int64_t)ks * p.M * p.N + n0;
    for (int t = tid; t < 16 * p.M; t += DECODE_WAVES * 64) {
        const int m = t >> 4, q = t & 15;
        // the waves' partials added in wave order
        f32x4 sum = *(const f32x4*)&part[0][m * DROW + 4 * q];
#pragma unroll
        for (int w = 1; w < DECODE_WAVES; ++w) sum += *(const f32x4*)&part[w][m * DROW + 4 * q];
        *(f32x4*)(ws + (int64_t)m * p.N + 4 * q) = sum;
    }
    if (p.rec && tid == 0) {
        // per workgroup: start, loads of the first whole span landed in
        // wave 0, loads and MFMAs of all waves done, partial issued (100 MHz
        // real-time counter)
        unsigned long long* r = p.rec + 4 * (int64_t)blockIdx.x;
        r[0] = t_start;
        r[1] = t_land;
        r[2] = t_loop;
        r[3] = __builtin_amdgcn_s_memrealtime();
    }
}

}  // namespace dge
