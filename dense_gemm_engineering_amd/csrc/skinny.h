// Tall-skinny GEMM with the fused epilogue: C = epi(alpha X W + beta C) for
// M >> N, K with N <= 256 and K <= 256 (the window-transformer projections,
// K = 160 with N = 160 or 32).  At these shapes the product is HBM-bound
// (X is read once, C written once; W is 51 KB), so the kernel is built around
// streaming X:
//
//  * One workgroup per CU with 8 waves.  W sits in LDS once per workgroup
//    for the whole kernel and serves as the MFMA "A" operand of C^T = W^T
//    X^T; the bias is staged next to it as fp32.  An N x K W is stored as it
//    is ([n][k], rows padded by 16 bytes) and its fragments are plain
//    16-byte reads.  A K x N W is also stored as it is ([k][n] in blocks of
//    64 columns, 16-byte chunks XOR-swizzled by k-row) and its W^T
//    fragments are read with ds_read_b64_tr_b16, as the GEMM reads a K x N
//    B: its loads are then whole rows of W, 16 bytes per lane, and its LDS
//    writes plain 16-byte stores.  (Transposing on the way in instead needs
//    each lane on a pair of k-rows, so that every load of a wave touched 64
//    cache lines: staging 51 KB took ~3 us at N = K = 160.)  A wave reads
//    all the W^T fragments of a 32-deep k-block at once (so their LDS
//    latencies overlap) and, up to N = 64, applies each to two 16-row blocks.
//  * X needs no LDS: the MFMA "B" operand of X^T is 8 consecutive k of one
//    row of X per lane, i.e. a 16-byte load straight from memory into the
//    operand registers.  Each wave owns 16 rows (32 for N <= 64) at a time
//    and issues their loads (K / 32 per lane and row block) before its first
//    MFMA, and the next rows' loads before its epilogue.  The prologue asks
//    for W and the bias before X and publishes W with an LDS-only barrier,
//    so each wave starts as soon as its own rows arrive.
//  * In C^T each lane holds 4 consecutive columns n of one row m of C, so the
//    epilogue (alpha/beta, per-column bias, tanh-GELU, rounding) works on 4
//    adjacent outputs; the rounded tile goes through the wave's LDS staging
//    area and leaves as whole rows, 16 bytes per lane.
//  * The vector ALU, not HBM, turned out to bound it: at N = K = 160 a wave
//    issued ~1870 VALU instructions (the GELU's exp and reciprocal per
//    output, but also per-chunk index arithmetic for W, zeroing and bias
//    adds, conversions, 64-bit store addresses, and hoisted masks of the
//    unused epilogue kinds spilling scalar registers), ~65% of each SIMD's
//    time, and the cache-warm time was within 3% of the HBM-cold one.  So
//    W is staged in uniform-stride passes with 32-bit offsets; with alpha =
//    1, beta = 0 and fp16 output the bias starts the accumulators (separate
//    instances carrying only that epilogue); pairs are converted with one
//    packed instruction; and a wave whose rows are one contiguous block of
//    C stores it at a uniform base plus a 32-bit offset.  N = 160: 14.1 ->
//    12.4 us (graph replays, HBM-cold X and C, same machine, alternating
//    processes).
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
    int pitch;   // LDS row pitch of W in elements (skinny_pitch)
    int c_type;
    int vec_c;   // bit 1: W rows allow aligned 16-byte loads; bit 2: C rows are
                 // 16-byte aligned and N fills whole 16-byte chunks
    Epilogue ep;
    // phase records (may be null): 4 real-time counter values per workgroup,
    // taken by its first thread
    unsigned long long* rec;
};

constexpr int SKINNY_KBMAX = 8;        // K <= 256
// 16-row blocks per wave and step: two for N <= 64, else one.  For N = 160
// one block per step gives each wave two steps at 65536 rows, so one step's
// stores overlap the next step's loads (measured 19.7 -> 18.3 us HBM-cold);
// for N = 32 the two ways measure the same.
__host__ __device__ constexpr int skinny_rb(int nt) { return nt <= 4 ? 2 : 1; }
// k-blocks of X (32 k each) held in registers at a time: all of K <= 256
// (with one row block per step the registers allow it for every N).
__host__ __device__ constexpr int skinny_kch(int) { return 8; }
// Waves per workgroup at most (256 registers per lane).
__host__ __device__ constexpr int skinny_max_waves(int) { return 8; }

// A K x N W sits in LDS in column blocks of SKINNY_CB = 64 columns, each K
// rows of 128 bytes (8 chunks of 16 bytes), as many blocks as NT*16 columns
// need.  With the fixed 128-byte row every k-row offset a k-block's fragment
// reads need stays well below 64 KB, an immediate of the read.
constexpr int SKINNY_CB = 64;
__host__ __device__ constexpr int skinny_cblocks(int nt) { return (nt * 16 + SKINNY_CB - 1) / SKINNY_CB; }
// LDS row pitch in elements: K + 8 for an N x K W ([n][k]), SKINNY_CB for a
// K x N W ([block][k][n % 64])
__host__ __device__ inline int skinny_pitch(int trans_b, int K) {
    return trans_b ? K + 8 : SKINNY_CB;
}
__host__ __device__ inline size_t skinny_w_bytes(int trans_b, int nt, int K) {
    return trans_b ? (size_t)nt * 16 * (K + 8) * 2 : (size_t)skinny_cblocks(nt) * K * SKINNY_CB * 2;
}
// Dynamic LDS: W, the bias (NT*16 fp32), the accumulators' starting row
// (NT*16 fp32), then one output staging tile per wave (RB*16 rows x
// (NT*16*out_bytes + 16) bytes).
__host__ __device__ inline size_t skinny_stage_bytes(int nt, int out_bytes) {
    return (size_t)16 * skinny_rb(nt) * (nt * 16 * out_bytes + 16);
}
__host__ __device__ inline size_t skinny_lds_bytes(int trans_b, int nt, int K, int out_bytes,
                                                   int waves) {
    return skinny_w_bytes(trans_b, nt, K) + (size_t)nt * 16 * 8 +
           (size_t)waves * skinny_stage_bytes(nt, out_bytes);
}
// Waves per workgroup: the most (8, 4, 2 or 1) whose staging fits 160 KB.
inline int skinny_waves(int trans_b, int nt, int K, int out_bytes) {
    int w = skinny_max_waves(nt);
    while (w > 1 && skinny_lds_bytes(trans_b, nt, K, out_bytes, w) > 160 * 1024) w /= 2;
    return w;
}
// XOR swizzle of the 16-byte chunks of k-row k of a K x N W (8 chunks a
// row): a transposed fragment read covers 16 k-rows (k % 4 = 0..3 from each
// of the 4 lane groups, 8 apart) x 32 bytes.  With 128-byte rows, k-rows of
// one parity share bank groups unless bit 1 of k moves them, and lane
// groups 0 / 1 (and 2 / 3) unless bit 3 does: the 32-byte pair index is
// XORed with those two bits, so each half of the read (32 lanes) covers 8
// different 32-byte bank groups.
__device__ inline int swz_kn(int k) { return (((k >> 1) & 1) << 1) | (((k >> 3) & 1) << 2); }
typedef __attribute__((address_space(3))) uint16_t lds_u16;
__device__ inline uint2 skinny_read_tr(const lds_u16* p) {
    typedef short s16x4_t __attribute__((ext_vector_type(4)));
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)p);
    return __builtin_bit_cast(uint2, v);
}

template <int OT>
__device__ inline void skinny_load4(const SkinnyArgs& p, int m, int n0, float* t) {
    typedef typename OutType<OT>::T T;
    const T* c = (const T*)p.C + (int64_t)m * p.ldc + n0;
#pragma unroll
    for (int e = 0; e < 4; ++e) t[e] = n0 + e < p.N ? OutType<OT>::to_f32(c[e]) : 0.0f;
}

// Epilogue of one wave's RB x 16 rows starting at row base: alpha/beta,
// bias, GELU and rounding in registers (4 consecutive columns per lane), the
// rounded values staged in the wave's LDS tile (rows of pitch_o bytes), then
// written out row by row with 16-byte non-temporal stores so that a wave writes whole
// rows of C.
// The epilogue kind is a template argument (EPI): with it a runtime flag,
// the compiler evaluated bias and GELU for every output and selected.
// GEN = false is the case alpha = 1, beta = 0: the accumulators started from
// the bias (or zero), so the value before GELU is the accumulator itself.
template <int OT, int NT, int RB, int EPI, bool GEN>
__device__ inline void skinny_finish(const SkinnyArgs& p, const f32x4 (&acc)[RB][NT],
                                     const float* bias_s, int base, int lane, char* stage) {
    typedef typename OutType<OT>::T T;
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    constexpr int OB = OutType<OT>::BYTES;
    constexpr int pitch_o = NT * 16 * OB + 16;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int ml = rb * 16 + (lane & 15);
        const int m = base + ml;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n0 = nt * 16 + 4 * (lane >> 4);
            float t[4];
            if constexpr (GEN) {
                f32x4 b = {0.f, 0.f, 0.f, 0.f};
                if constexpr (EPI != EPI_NONE) b = *(const f32x4*)(bias_s + n0);  // zero past N
                if (p.ep.beta != 0.0f) {  // wave-uniform; a branch around loads of C
                    float old[4] = {0.f, 0.f, 0.f, 0.f};
                    if (m < p.M && n0 < p.N) skinny_load4<OT>(p, m, n0, old);
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[e] = p.ep.alpha * acc[rb][nt][e] + p.ep.beta * old[e] + b[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) t[e] = __builtin_fmaf(p.ep.alpha, acc[rb][nt][e], b[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = acc[rb][nt][e];
            }
            if constexpr (EPI == EPI_BIAS_GELU) {
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] = gelu_tanh(t[e]);
            }
            char* dst = stage + ml * pitch_o + n0 * OB;
            if constexpr (OT == OUT_F16) {
                // one packed conversion per pair (round to nearest even)
                const h2_t lo = {(_Float16)t[0], (_Float16)t[1]};
                const h2_t hi = {(_Float16)t[2], (_Float16)t[3]};
                *(uint2*)dst = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
            } else if constexpr (OB == 2) {
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
    // chunk q = lane + 64 i of the RB*16 x cpr chunks is (row q / cpr, chunk
    // q % cpr); stepped without a division per chunk
    const int d_row = 64 / cpr, d_chunk = 64 - d_row * cpr;
    int r = lane / cpr, c = lane - r * cpr;
    if (vec && p.ldc == p.N && base + RB * 16 <= p.M) {
        // the wave's rows are one contiguous block of C: chunk q sits q * 16
        // bytes past the block's start (a uniform address, a 32-bit offset)
        constexpr int QMAX = (RB * 16 * NT * 16 * OB / 16 + 63) / 64;  // chunks per lane at most
        const int total = RB * 16 * cpr;
        char* blk = (char*)p.C + (int64_t)base * p.ldc * OB;
#pragma unroll
        for (int i = 0; i < QMAX; ++i) {
            const int q = lane + 64 * i;
            if (q < total)
                __builtin_nontemporal_store(*(const u32x4*)(stage + r * pitch_o + c * 16),
                                            (u32x4*)(blk + (uint32_t)q * 16u));
            r += d_row;
            c += d_chunk;
            if (c >= cpr) {
                c -= cpr;
                ++r;
            }
        }
    } else {
        while (r < RB * 16) {
            const int mm = base + r;
            if (mm < p.M) {
                const char* src = stage + r * pitch_o + c * 16;
                char* dst = (char*)p.C + ((int64_t)mm * p.ldc) * OB + c * 16;
                if (vec) {
                    __builtin_nontemporal_store(*(const u32x4*)src, (u32x4*)dst);
                } else {
                    for (int e = 0; e < 16 / OB; ++e)
                        if (c * 16 + e * OB < row_bytes) ((T*)dst)[e] = ((const T*)src)[e];
                }
            }
            r += d_row;
            c += d_chunk;
            if (c >= cpr) {
                c -= cpr;
                ++r;
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
}

template <int NT, int RB, int EPI>
__device__ inline void skinny_finish_ot(const SkinnyArgs& p, const f32x4 (&acc)[RB][NT],
                                        const float* bias_s, int base, int lane, char* stage) {
    if (p.c_type == OUT_F16)
        skinny_finish<OUT_F16, NT, RB, EPI, true>(p, acc, bias_s, base, lane, stage);
    else if (p.c_type == OUT_BF16)
        skinny_finish<OUT_BF16, NT, RB, EPI, true>(p, acc, bias_s, base, lane, stage);
    else
        skinny_finish<OUT_F32, NT, RB, EPI, true>(p, acc, bias_s, base, lane, stage);
}

// W into LDS by nth threads, one batch (BT tasks per thread) at a time:
// load() brings a batch into registers, store() writes it to LDS, so that
// other loads can be issued in between.  A task is one 16-byte chunk: 8
// consecutive k of one n-row of an N x K W, or 8 consecutive n of one k-row
// of a K x N W (chunks past N zero-filled up to NT*16 columns); consecutive
// lanes take consecutive chunks of a row, so the loads of a wave cover
// whole rows.
template <int DT, int NT, bool TRANS_B>
struct WStage {
    static constexpr int NP = NT * 16;
    static constexpr int BT = 8;  // tasks per thread per batch: one batch at N = K = 160
    u32x4 v[BT];

    __device__ static inline int per_row(const SkinnyArgs& p) { return TRANS_B ? p.K / 8 : NP / 8; }
    __device__ static inline int ntask(const SkinnyArgs& p) {
        return TRANS_B ? NP * (p.K / 8) : p.K * (NP / 8);
    }
    // Task t of this workgroup is task (t + rot) mod ntask: every workgroup
    // wants all of W at the same moment, and rotating the order spreads the
    // requests over the cache channels.
    __device__ static inline int rotated(int t, int rot, int nt_all) {
        const int r = t + rot;
        return r >= nt_all ? r - nt_all : r;
    }
    __device__ inline void load(const SkinnyArgs& p, int t0, int tid, int nth, int rot) {
        const bool vec_w = (p.vec_c & 2) != 0;  // W rows allow aligned 16-byte loads
        const int nt_all = ntask(p), pr = per_row(p);
#pragma unroll
        for (int i = 0; i < BT; ++i) {
            const int tt = t0 + i * nth + tid;
            v[i] = (u32x4){0, 0, 0, 0};
            if (tt >= nt_all) continue;
            const int t = rotated(tt, rot, nt_all);
            const int row = t / pr, c8 = (t - row * pr) * 8;
            if constexpr (TRANS_B) {
                if (row >= p.N) continue;
                const int64_t idx = (int64_t)row * p.ldw + c8;
                v[i] = vec_w ? load16((const char*)p.W + idx * 2) : load_chunk_masked<DT>(p.W, idx, 8);
            } else {
                if (c8 >= p.N) continue;
                const int64_t idx = (int64_t)row * p.ldw + c8;
                v[i] = vec_w && c8 + 8 <= p.N ? load16((const char*)p.W + idx * 2)
                                              : load_chunk_masked<DT>(p.W, idx, p.N - c8);
            }
        }
    }
    __device__ inline void store(const SkinnyArgs& p, uint16_t* wt, int t0, int tid, int nth,
                                 int rot) const {
        const int nt_all = ntask(p), pr = per_row(p);
#pragma unroll
        for (int i = 0; i < BT; ++i) {
            const int tt = t0 + i * nth + tid;
            if (tt >= nt_all) continue;
            const int t = rotated(tt, rot, nt_all);
            const int row = t / pr, c = t - row * pr;
            if constexpr (TRANS_B)
                *(u32x4*)(wt + row * p.pitch + 8 * c) = v[i];
            else
                *(u32x4*)(wt + (c >> 3) * p.K * SKINNY_CB + row * SKINNY_CB +
                          8 * ((c & 7) ^ swz_kn(row))) = v[i];
        }
    }
};

// A K x N W with N a multiple of 8, 16-byte aligned rows and byte offsets
// below 2^32: thread tid owns chunk column c = tid % PR (PR = NT * 2 chunks
// of the NT*16 staged columns, zeros past N) of k-rows r0 + RP i (r0 = tid /
// PR, RP = nth / PR rows a pass; threads past RP * PR stage nothing).  The
// passes, and the threads' rows within a pass, run in a per-workgroup
// rotated order (every workgroup wants all of W at the same moment;
// starting at different rows spreads the requests over the cache channels),
// so a pass's row and offsets are a uniform shift of the thread's first: a
// few VALU instructions per 16-byte chunk, against several dozen with a
// division and 64-bit addresses per chunk.
template <int NT>
__device__ inline void skinny_stage_w_kn(const SkinnyArgs& p, uint16_t* wt, int tid, int nth) {
    constexpr int PR = NT * 2, BT = 8;
    const int RP = nth / PR, K = p.K;
    const int c = tid % PR;
    int r0 = tid / PR;
    if (r0 >= RP) return;
    r0 += (int)((blockIdx.x * 13u) % (unsigned)RP);  // first rows rotated too
    if (r0 >= RP) r0 -= RP;
    const bool live = c * 8 < p.N;
    const int NI = (K + RP - 1) / RP;  // passes
    const int irot = (int)(blockIdx.x % (unsigned)NI);
    const uint32_t ldw2 = (uint32_t)p.ldw * 2u;
    const uint32_t goff0 = (uint32_t)r0 * ldw2 + (uint32_t)c * 16u;
    char* lblk = (char*)wt + (c >> 3) * K * SKINNY_CB * 2;
    for (int i0 = 0; i0 < NI; i0 += BT) {
        u32x4 v[BT];
#pragma unroll
        for (int j = 0; j < BT; ++j) {
            v[j] = (u32x4){0, 0, 0, 0};
            int ip = i0 + j + irot;
            if (ip >= NI) ip -= NI;
            if (i0 + j < NI && live && r0 + ip * RP < K)
                v[j] = load16((const char*)p.W + (goff0 + (uint32_t)(ip * RP) * ldw2));
        }
#pragma unroll
        for (int j = 0; j < BT; ++j) {
            int ip = i0 + j + irot;
            if (ip >= NI) ip -= NI;
            const int row = r0 + ip * RP;
            if (i0 + j < NI && row < K)
                *(u32x4*)(lblk + row * (SKINNY_CB * 2) + 16 * ((c & 7) ^ swz_kn(row))) = v[j];
        }
    }
}

// The X operand registers of k-blocks kb0 .. kb0 + KCH - 1 of one wave's
// RB x 16 rows starting at row base.  (Loading whole rows and moving them
// into operand layout through LDS, as the decode kernel does for its
// weight, measured slower here: 14.6 -> 16.8 us at N = K = 160.)
template <int RB, int KCH>
__device__ inline void skinny_load_x(const SkinnyArgs& p, int base, int kb0, int lane,
                                     u32x4 (&xf)[RB][KCH]) {
    const int KB = p.K / 32;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int m = base + rb * 16 + (lane & 15);
        if (m >= p.M) m = p.M - 1;  // rows past the end: valid memory, never stored
        const char* row = (const char*)p.X + ((int64_t)m * p.ldx + 8 * (lane >> 4) + 32 * kb0) * 2;
#pragma unroll
        for (int kb = 0; kb < KCH; ++kb)
            if (kb0 + kb < KB) xf[rb][kb] = load16(row + kb * 64);
    }
}

// FOLD: alpha = 1, beta = 0 and fp16 output (the launcher's choice), the
// bias starting the accumulators; the other instances take any epilogue.
template <int DT, int NT, bool TRANS_B, bool FOLD>
__global__ __launch_bounds__(skinny_max_waves(NT) * 64) void gemm_skinny_kernel(SkinnyArgs p) {
    extern __shared__ __attribute__((aligned(16))) uint16_t wt[];  // NT*16 rows x pitch
    constexpr int RB = skinny_rb(NT);
    constexpr int KCH = skinny_kch(NT);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int KB = p.K / 32;
    const int rows_per_step = nwaves * RB * 16 * gridDim.x;
    int base = (blockIdx.x * nwaves + wave) * RB * 16;
    const bool rec = p.rec && tid == 0;
    unsigned long long t_start = 0, t_w = 0, t_x = 0;
    if (rec) t_start = __builtin_amdgcn_s_memrealtime();

    // Prologue: W and the bias are staged before any X is requested (issued
    // together, X would flood the memory system and W, which every wave
    // needs, would come back last: measured ~4.5 us instead of ~1-2 us), and
    // the barrier that publishes W waits for LDS traffic only; then each
    // wave requests its rows of X and starts its MFMAs as soon as they
    // arrive, so later rows' loads overlap earlier rows' stores.
    const int nth = blockDim.x;
    uint32_t bias_bits[4];  // NT * 16 <= 256 values over at least 64 threads
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = tid + i * nth;
        bias_bits[i] = p.ep.epi != EPI_NONE && n < p.N ? load_elem_bits<DT>(p.ep.bias, n) : 0u;
    }
    bool fast_w = false;
    if constexpr (!TRANS_B)
        fast_w = (p.vec_c & 2) != 0 && p.N % 8 == 0 && p.K * p.ldw * 2 < (int64_t)1 << 32;
    if (fast_w) {
        skinny_stage_w_kn<NT>(p, wt, tid, nth);
    } else {
        WStage<DT, NT, TRANS_B> wst;
        const int w_tasks = WStage<DT, NT, TRANS_B>::ntask(p);
        const int rot = (int)(((int64_t)blockIdx.x * 97 * 64) % w_tasks);
        const int w_batch = WStage<DT, NT, TRANS_B>::BT * nth;
        for (int t0 = 0; t0 < w_tasks; t0 += w_batch) {
            wst.load(p, t0, tid, nth, rot);
            wst.store(p, wt, t0, tid, nth, rot);
        }
    }
    // FOLD: the accumulators start from the bias (init_s), and the epilogue
    // adds nothing; otherwise they start from zero and the epilogue applies
    // alpha, beta and the bias (bias_s)
    constexpr bool fold = FOLD;
    float* bias_s = (float*)((char*)wt + skinny_w_bytes(TRANS_B, NT, p.K));
    float* init_s = bias_s + NT * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (tid + i * nth < NT * 16) {
            const float b = InType<DT>::to_f32(bias_bits[i]);
            bias_s[tid + i * nth] = b;
            init_s[tid + i * nth] = fold ? b : 0.0f;
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this thread's LDS writes are done
    __builtin_amdgcn_s_barrier();
    if (rec) t_w = __builtin_amdgcn_s_memrealtime();
    u32x4 xf[RB][KCH];
    if (base < p.M) skinny_load_x<RB, KCH>(p, base, 0, lane, xf);
    if (rec) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the first rows have landed
        t_x = __builtin_amdgcn_s_memrealtime();
    }

    const uint16_t* wrow = wt + (lane & 15) * p.pitch + 8 * (lane >> 4);
    // K x N W: transposed fragment reads.  Lane group g = lane / 16 covers
    // k-rows 32 kb + 8 g + 4 h + t / 4 (t = lane % 16) and columns 16 nt +
    // 4 (t % 4); lane t receives column 16 nt + t, 4 k per read, 8 for the
    // two halves h.  The k-row's swizzle depends only on t / 4 and g % 2
    // (k % 4 and bit 3 of k), so each lane's offsets within a k-block are
    // fixed: tr_off[nt] elements past the k-block's uniform row.
    const lds_u16* wt3 = (const lds_u16*)wt;
    int tr_off[TRANS_B ? 1 : NT];
    if constexpr (!TRANS_B) {
        const int t = lane & 15, g = lane >> 4;
        const int sw = (((t >> 3) & 1) << 1) | ((g & 1) << 2);  // swz_kn of those k-rows
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int n = nt * 16 + 4 * (t & 3), nb = n % SKINNY_CB;
            tr_off[nt] = (n / SKINNY_CB) * p.K * SKINNY_CB + (8 * g + (t >> 2)) * SKINNY_CB +
                         8 * ((nb >> 3) ^ sw) + (n & 7);
        }
    }
    const int ob = p.c_type == OUT_F32 ? 4 : 2;
    char* stage = (char*)(init_s + NT * 16) + wave * skinny_stage_bytes(NT, ob);
    for (; base < p.M; base += rows_per_step) {
        f32x4 acc[RB][NT];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                acc[rb][nt] = *(const f32x4*)(init_s + nt * 16 + 4 * (lane >> 4));
#pragma unroll
        for (int c0 = 0; c0 < SKINNY_KBMAX; c0 += KCH) {
            if (c0 >= KB) break;
#pragma unroll
            for (int kb = 0; kb < KCH; ++kb) {
                if (c0 + kb >= KB) break;
                // all of this k-block's W^T fragments first, then the MFMAs
                u32x4 wf[NT];
                if constexpr (TRANS_B) {
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        wf[nt] = *(const u32x4*)(wrow + nt * 16 * p.pitch + (c0 + kb) * 32);
                } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        // uniform, and with the fixed row pitch an immediate
                        // offset (a runtime pitch made the compiler hold an
                        // address per (k-block, h, nt) across steps)
                        const lds_u16* kp = wt3 + ((c0 + kb) * 32 + 4 * h) * SKINNY_CB;
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) {
                            const uint2 v = skinny_read_tr(kp + tr_off[nt]);
                            wf[nt][2 * h] = v.x;
                            wf[nt][2 * h + 1] = v.y;
                        }
                    }
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) mma_chunk<DT>(acc[rb][nt], wf[nt], xf[rb][kb]);
                // keep the next k-block's fragment reads after these MFMAs
                // (hoisted, they hold NT more registers per k-block)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the next rows' loads overlap this epilogue's stores
        if (base + rows_per_step < p.M) skinny_load_x<RB, KCH>(p, base + rows_per_step, 0, lane, xf);
        if constexpr (FOLD) {
            // alpha = 1, beta = 0, fp16 out: the bias is already in acc
            if (p.ep.epi == EPI_BIAS_GELU)
                skinny_finish<OUT_F16, NT, RB, EPI_BIAS_GELU, false>(p, acc, bias_s, base, lane, stage);
            else
                skinny_finish<OUT_F16, NT, RB, EPI_NONE, false>(p, acc, bias_s, base, lane, stage);
        } else if (p.ep.epi == EPI_BIAS_GELU) {
            skinny_finish_ot<NT, RB, EPI_BIAS_GELU>(p, acc, bias_s, base, lane, stage);
        } else if (p.ep.epi == EPI_BIAS) {
            skinny_finish_ot<NT, RB, EPI_BIAS>(p, acc, bias_s, base, lane, stage);
        } else {
            skinny_finish_ot<NT, RB, EPI_NONE>(p, acc, bias_s, base, lane, stage);
        }
    }
    if (rec) {
        // start, W staged (barrier passed), wave 0's first rows landed, wave 0's
        // last stores issued
        unsigned long long* r = p.rec + 4 * (int64_t)blockIdx.x;
        r[0] = t_start;
        r[1] = t_w;
        r[2] = t_x;
        r[3] = __builtin_amdgcn_s_memrealtime();
    }
}

}  // namespace dge
