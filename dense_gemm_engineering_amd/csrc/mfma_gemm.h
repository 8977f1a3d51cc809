// LDS-staged macro-tile GEMM on the gfx950 matrix cores.
//
// One workgroup computes a BM x BN tile of C = A * B with fp32 accumulation;
// its WM x WN waves each own a (BM/WM) x (BN/WN) sub-tile held in
// registers as 16x16 MFMA accumulator blocks.  K advances in stages of 128
// bytes per row (64 fp16/bf16 or 32 fp32 elements).  Design points, with the
// prior art they answer:
//
//  * Staging through a double-buffered LDS ring: the next stage's global
//    loads are issued before the current stage's MFMAs and written to the
//    other buffer afterwards, one barrier per stage (the overlap that the
//    cp.async double buffer of "02 · 8m/8m② — Tiled wmma f16 prefill GEMM"
//    §2.4 and the TMA ring of "Optimizing GEMMs using tcgen05 - Part 2" §5.1
//    buy on their hardware).
//  * A 128-byte K stage per row, i.e. 64 half-precision elements: the fixed
//    per-stage cost (barrier, address math) is paid once per 2 x 16 MFMA
//    k-steps of 32 ("Optimizing GEMMs using tcgen05 - Part 2", §7.3 makes
//    the same trade with BK = 64).
//  * LDS rows hold 8 chunks of 16 bytes; chunk c of row r is stored at
//    position c ^ (r & 7), so the 16 lanes that read one MFMA operand (16
//    rows, same chunk) touch 8 distinct 16-byte bank groups.
//  * Both operands sit in LDS K-contiguous ([row][k]), the order the MFMA
//    operand registers want (8 consecutive k per lane).  A K x N row-major B
//    is transposed on its way in: each thread loads an 8 x 8 (fp32: 4 x 4)
//    block with 16-byte row loads and writes its transpose as 16-byte LDS
//    stores.
//  * Large per-wave tiles (up to 128 x 128, 256 fp32 accumulators per lane)
//    so each LDS byte feeds many MFMAs ("Matrix Multiplication: The Operation
//    Behind Modern AI", section "Registers: the same trick, one level
//    higher"; the A-fragment reuse of the prefill page, §3.2).
//  * The epilogue stages each wave's accumulators through LDS so that every
//    lane writes 8 consecutive output columns and a wave writes whole rows
//    ("Optimizing GEMMs using tcgen05 - Part 2", §7.2-7.3: full-line stores
//    after a transpose through shared memory; the prefill page masks the
//    tails in that one place, §3.1).
//  * Workgroup ids are remapped so each XCD's workgroups cover a compact
//    block of tiles (the L2 panel sharing of the prefill page, §2.2,
//    adjusted for 8 XCDs with separate L2s).
#pragma once

#include "device_common.h"

namespace dge {

// MFMA operand layout (16x16 blocks): lane l supplies row (l & 15) of A and
// column (l & 15) of B, each with the 16 bytes of K chunk (l >> 4) of the
// current 4-chunk k-block; lane l receives C rows 4 * (l >> 4) + e,
// e = 0..3, of column (l & 15).
// One of the four 16x16x4 fp32 products of a chunk pair (element e).  The
// element is copied to a scalar before the bit cast: a bit cast applied
// directly to a vector-element lvalue reads element 0 whatever the index.
__device__ inline void mma_f32_elem(f32x4& acc, const u32x4& a, const u32x4& b, int e) {
    const uint32_t ae = a[e], be = b[e];
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, ae),
                                               __builtin_bit_cast(float, be), acc, 0, 0, 0);
}

template <int DT>
__device__ inline void mma_chunk(f32x4& acc, const u32x4& a, const u32x4& b) {
    if constexpr (DT == IN_F16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                     __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    } else if constexpr (DT == IN_BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                      __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    } else {
        // fp32: a 16-byte chunk is 4 consecutive k; element e of every lane
        // group forms one 16x16x4 product, and the 4 products cover all 16 k
        // of the k-block (A and B use the same (lane group, element) -> k
        // assignment, so the sum is unchanged).
#pragma unroll
        for (int e = 0; e < 4; ++e) mma_f32_elem(acc, a, b, e);
    }
}


constexpr int CH = 8;  // 16-byte chunks per LDS row: 128 bytes of K per stage

__device__ inline int swz(int row) { return row & 7; }

enum : int { LOAD_FAST = 0, LOAD_EDGE = 1 };

// Kernel arguments (by value).
struct MfmaArgs {
    const void* A;
    const void* B;
    void* C;
    float* ws;  // split-K partials: splits x M x N fp32, or null
    int64_t lda, ldb, ldc;
    int M, N, K;
    int tiles_m, tiles_n, splits, k_per_split;  // k_per_split: multiple of the stage depth
    int group_m;
    int c_type;
    int vec_ok;  // 1 when A, B, C (and the loads' 16-byte chunks) are 16-byte aligned
    Epilogue ep;
    // persistent stream-K schedule (direct-to-LDS kernel): stages per tile,
    // partial-tile slots (2 x grid x BM x BN fp32) and per-tile arrival
    // counters (zero at launch)
    int sk_stages;
    int sk_rounds;  // rounds of whole tiles before the stream-K tail
    float* sk_ws;
    unsigned* sk_cnt;
    // measurement only (direct-to-LDS kernels, data-parallel schedule): when
    // set, each workgroup records its shader-clock and 100 MHz real-time
    // counters at its start and end, 4 values at clk + 4 blockIdx.x
    unsigned long long* clk;
};

// Pack KPL elements loaded one by one (with a bound) into a 16-byte chunk.
template <int DT>
__device__ inline u32x4 load_chunk_masked(const void* base, int64_t idx, int valid) {
    u32x4 v = {0, 0, 0, 0};
    if constexpr (InType<DT>::BYTES == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t x = e < valid ? load_elem_bits<DT>(base, idx + e) : 0u;
            v[e >> 1] |= x << (16 * (e & 1));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = e < valid ? load_elem_bits<DT>(base, idx + e) : 0u;
    }
    return v;
}

__device__ inline u32x4 load16(const void* p) { return *(const u32x4*)p; }

// Row panel of a K-contiguous operand (A, or B when trans_b): ROWS rows x one
// 128-byte K stage, PER 16-byte chunks per thread.
template <int DT, int ROWS, int NT, int MODE>
struct RowPanel {
    static constexpr int BYTES = InType<DT>::BYTES;
    static constexpr int KPL = 16 / BYTES;
    static constexpr int PER = ROWS * CH / NT;
    static_assert(PER * NT == ROWS * CH, "row panel must split evenly over the threads");
    u32x4 v[PER];

    __device__ inline void load(const void* base, int64_t ld, int r0, int nrows, int k0, int kend,
                                int tid, int vec_ok) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + i * NT;
            const int row = c / CH, ch = c % CH;
            int gr = r0 + row;
            const int gk = k0 + ch * KPL;
            if constexpr (MODE == LOAD_FAST) {
                v[i] = load16((const char*)base + ((int64_t)gr * ld + gk) * BYTES);
            } else {
                if (gr >= nrows) gr = nrows - 1;  // rows past the edge: valid memory, output discarded
                const int64_t idx = (int64_t)gr * ld + gk;
                if (vec_ok && gk + KPL <= kend)
                    v[i] = load16((const char*)base + idx * BYTES);
                else
                    v[i] = load_chunk_masked<DT>(base, idx, kend - gk);
            }
        }
    }

    __device__ inline void store(u32x4* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + i * NT;
            const int row = c / CH, ch = c % CH;
            lds[row * CH + (ch ^ swz(row))] = v[i];
        }
    }
};

// Column panel of a K x N row-major B: one stage of K (CH blocks of KPL rows)
// x COLS columns, loaded as KPL x KPL blocks and transposed into [n][k].
template <int DT, int COLS, int NT, int MODE>
struct ColPanel {
    static constexpr int BYTES = InType<DT>::BYTES;
    static constexpr int KPL = 16 / BYTES;
    static constexpr int NB = COLS / KPL;
    static constexpr int TOTAL = CH * NB;               // KPL x KPL blocks per stage
    static constexpr int PER = (TOTAL + NT - 1) / NT;   // blocks per thread (the last may be idle)
    static_assert(TOTAL % NT == 0 || TOTAL < NT, "column panel must split evenly over the threads");
    u32x4 v[PER][KPL];

    __device__ inline void load(const void* base, int64_t ld, int n0, int ncols, int k0, int kend,
                                int tid, int vec_ok) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = tid + i * NT;
            if (TOTAL < NT && b >= TOTAL) break;
            const int kb = b / NB, nb = b % NB;
            const int gn = n0 + nb * KPL;
#pragma unroll
            for (int r = 0; r < KPL; ++r) {
                const int gk = k0 + kb * KPL + r;
                if constexpr (MODE == LOAD_FAST) {
                    v[i][r] = load16((const char*)base + ((int64_t)gk * ld + gn) * BYTES);
                } else {
                    if (gk >= kend || gn >= ncols) {
                        v[i][r] = (u32x4){0, 0, 0, 0};
                    } else {
                        const int64_t idx = (int64_t)gk * ld + gn;
                        if (vec_ok && gn + KPL <= ncols)
                            v[i][r] = load16((const char*)base + idx * BYTES);
                        else
                            v[i][r] = load_chunk_masked<DT>(base, idx, ncols - gn);
                    }
                }
            }
        }
    }

    __device__ inline void store(u32x4* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int b = tid + i * NT;
            if (TOTAL < NT && b >= TOTAL) break;
            const int kb = b / NB, nb = b % NB;
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                u32x4 o;
                if constexpr (BYTES == 2) {
                    // o[d] = (k = 2d, n = j) | (k = 2d + 1, n = j) << 16
                    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
                    for (int d = 0; d < 4; ++d)
                        o[d] = __builtin_amdgcn_perm(v[i][2 * d + 1][j >> 1], v[i][2 * d][j >> 1], sel);
                } else {
#pragma unroll
                    for (int d = 0; d < 4; ++d) o[d] = v[i][d][j];
                }
                const int row = nb * KPL + j;
                lds[row * CH + (kb ^ swz(row))] = o;
            }
        }
    }
};

template <int OT>
__device__ inline void store_row8(void* C, int64_t ldc, int row, int col, int N, const float* t,
                                  bool vec) {
    typedef typename OutType<OT>::T T;
    T* p = (T*)C + (int64_t)row * ldc + col;
    if (vec && col + 8 <= N) {
        if constexpr (OutType<OT>::BYTES == 2) {
            u32x4 o;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                uint16_t lo = __builtin_bit_cast(uint16_t, OutType<OT>::from_f32(t[2 * d]));
                uint16_t hi = __builtin_bit_cast(uint16_t, OutType<OT>::from_f32(t[2 * d + 1]));
                o[d] = (uint32_t)lo | ((uint32_t)hi << 16);
            }
            *(u32x4*)p = o;
        } else {
            *(f32x4*)p = (f32x4){t[0], t[1], t[2], t[3]};
            *(f32x4*)(p + 4) = (f32x4){t[4], t[5], t[6], t[7]};
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (col + e < N) p[e] = OutType<OT>::from_f32(t[e]);
    }
}

template <int OT>
__device__ inline void load_row8(const void* C, int64_t ldc, int row, int col, int N, float* t,
                                 bool vec) {
    typedef typename OutType<OT>::T T;
    const T* p = (const T*)C + (int64_t)row * ldc + col;
    if (vec && col + 8 <= N) {
        if constexpr (OutType<OT>::BYTES == 2) {
            u32x4 o = *(const u32x4*)p;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                t[2 * d] = OutType<OT>::to_f32(__builtin_bit_cast(T, (uint16_t)(o[d] & 0xffff)));
                t[2 * d + 1] = OutType<OT>::to_f32(__builtin_bit_cast(T, (uint16_t)(o[d] >> 16)));
            }
        } else {
            f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                t[e] = a[e];
                t[4 + e] = b[e];
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = col + e < N ? OutType<OT>::to_f32(p[e]) : 0.0f;
    }
}

// Epilogue for 8 consecutive columns of one row: alpha/beta/bias/GELU, one
// rounding to the output type, store.
template <int DT, int OT>
__device__ __attribute__((always_inline)) inline void finish_row8(const MfmaArgs& p, int row, int col, const float* acc) {
    const bool vec = p.vec_ok != 0;
    float old[8];
    if (p.ep.beta != 0.0f) load_row8<OT>(p.C, p.ldc, row, col, p.N, old, vec);
    float t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int c = col + e < p.N ? col + e : p.N - 1;
        t[e] = apply_epilogue<DT>(p.ep, acc[e], p.ep.beta != 0.0f ? old[e] : 0.0f, c);
    }
    store_row8<OT>(p.C, p.ldc, row, col, p.N, t, vec);
}

// ---- a4: the fused epilogue.  Each wave stages its accumulators through
// LDS one strip of SM rows at a time and then writes 8 consecutive columns
// per lane, so a wave stores whole rows; with a split-K workspace the raw
// fp32 partials go there instead.  drain_strip writes one staged strip
// (SM rows x WTN columns, row pitch PITCH floats) whose first element is
// C[grow0][gcol0].
template <int DT, int MODE, int WTN, int SM, int PITCH>
__device__ __attribute__((always_inline)) inline void drain_strip(const MfmaArgs& p, const float* stg, int grow0, int gcol0,
                                   int split, int lane) {
    constexpr int LPR = WTN / 8;   // lanes per row, 8 columns each
    constexpr int RPP = 64 / LPR;  // rows per pass
    static_assert(LPR * 8 == WTN && RPP * LPR == 64 && SM % RPP == 0, "epilogue lane map");
    // The read-back loop does not touch the accumulators; keeping it rolled
    // keeps the strip loop small enough to unroll fully, so the accumulator
    // array is only ever indexed statically (no scratch).
#pragma nounroll
    for (int pass = 0; pass < SM / RPP; ++pass) {
        const int r = pass * RPP + lane / LPR;
        const int c8 = (lane % LPR) * 8;
        const int grow = grow0 + r;
        const int gcol = gcol0 + c8;
        float v[8];
        const f32x4 lo = *(const f32x4*)&stg[r * PITCH + c8];
        const f32x4 hi = *(const f32x4*)&stg[r * PITCH + c8 + 4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = lo[e];
            v[4 + e] = hi[e];
        }
        if (MODE == LOAD_EDGE && (grow >= p.M || gcol >= p.N)) continue;
        if (p.ws) {
            float* w = p.ws + ((int64_t)split * p.M + grow) * p.N + gcol;
            if (p.vec_ok && gcol + 8 <= p.N && (p.N & 3) == 0) {
                *(f32x4*)w = lo;
                *(f32x4*)(w + 4) = hi;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (gcol + e < p.N) w[e] = v[e];
            }
        } else if (p.c_type == OUT_F16) {
            finish_row8<DT, OUT_F16>(p, grow, gcol, v);
        } else if (p.c_type == OUT_BF16) {
            finish_row8<DT, OUT_BF16>(p, grow, gcol, v);
        } else {
            finish_row8<DT, OUT_F32>(p, grow, gcol, v);
        }
    }
}

// Epilogue of a tile held as 16x16 accumulator blocks (16-row strips,
// stg: NW x 16 x (WTN + 4) fp32).
template <int DT, int BM, int BN, int WM, int WN, int MODE, int TM, int TN>
__device__ __attribute__((always_inline)) inline void epilogue_tile(const MfmaArgs& p, f32x4 (&acc)[TM][TN], float* stg_all,
                                     int m0, int n0, int split) {
    constexpr int WTM = BM / WM, WTN = BN / WN;
    static_assert(TM * 16 == WTM && TN * 16 == WTN, "wave tile");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;
    constexpr int PITCH = WTN + 4;  // floats; the pad staggers rows across banks
    float* stg = stg_all + wave * (16 * PITCH);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                stg[(4 * (lane >> 4) + e) * PITCH + 16 * j + (lane & 15)] = acc[i][j][e];
        __syncthreads();
        drain_strip<DT, MODE, WTN, 16, PITCH>(p, stg, m0 + wm0 + 16 * i, n0 + wn0, split, lane);
        __syncthreads();
    }
}

template <int DT, int BM, int BN, int WM, int WN, bool TRANS_B, int MODE>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_mfma_kernel(MfmaArgs p) {
    constexpr int NT = WM * WN * 64;
    constexpr int KPL = 16 / InType<DT>::BYTES;
    constexpr int BK = CH * KPL;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 16, TN = WTN / 16;
    static_assert(TM * 16 == WTM && TN * 16 == WTN, "wave tile must be a multiple of 16");

    __shared__ u32x4 lds[2][(BM + BN) * CH];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / WN) * WTM, wn0 = (wave % WN) * WTN;

    // ---- a1: tile scheduling
    const int ntiles = p.tiles_m * p.tiles_n;
    const int nwg = ntiles * p.splits;
    const int lin = remap_xcd(blockIdx.x, nwg);
    const int split = lin / ntiles;
    int tm, tn;
    grouped_tile(lin % ntiles, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = split * p.k_per_split;
    int kend = kbeg + p.k_per_split;
    if (kend > p.K) kend = p.K;
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    RowPanel<DT, BM, NT, MODE> pa;
    using BPanel = typename std::conditional<TRANS_B, RowPanel<DT, BN, NT, MODE>,
                                             ColPanel<DT, BN, NT, MODE>>::type;
    BPanel pb;

    auto load_stage = [&](int k0) {
        pa.load(p.A, p.lda, m0, p.M, k0, kend, tid, p.vec_ok);
        pb.load(p.B, p.ldb, n0, p.N, k0, kend, tid, p.vec_ok);
    };
    auto store_stage = [&](int st) {
        pa.store(&lds[st][0], tid);
        pb.store(&lds[st][BM * CH], tid);
    };

    // Fragments of one 4-chunk k-block: TM A operands and TN B operands.
    auto read_frags = [&](int st, int kb, u32x4* fa, u32x4* fb) {
        const u32x4* la = &lds[st][0];
        const u32x4* lb = &lds[st][BM * CH];
        const int ch = kb * 4 + (lane >> 4);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm0 + 16 * i + (lane & 15);
            fa[i] = la[row * CH + (ch ^ swz(row))];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn0 + 16 * j + (lane & 15);
            fb[j] = lb[row * CH + (ch ^ swz(row))];
        }
    };
    auto mma_all = [&](const u32x4* fa, const u32x4* fb) {
        if constexpr (DT == IN_F32) {
            // element e of every chunk in turn: consecutive MFMAs then never
            // feed one another, and each accumulator is updated in place
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) mma_f32_elem(acc[i][j], fa[i], fb[j], e);
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) mma_chunk<DT>(acc[i][j], fa[i], fb[j]);
        }
    };
    static_assert(CH == 8, "two 4-chunk k-blocks per stage");
    u32x4 fa0[TM], fb0[TN], fa1[TM], fb1[TN];

    static_assert(WM * WN * 16 * (WTN + 4) * 4 <= (int)sizeof(lds), "epilogue staging must fit");

    // ---- a2: prologue.  Stage 0 goes to LDS buffer 0; stage 1 waits in
    // registers.  In the steady state the registers always hold the stage
    // after the one being computed, so every global load has a whole stage
    // of MFMA work to land before its LDS write.
    if (nk > 0) {
        load_stage(kbeg);
        store_stage(0);
    }
    if (nk > 1) load_stage(kbeg + BK);
    __syncthreads();

    // ---- a2 + a3: main loop.  Stage kt: read k-block 0 of buffer kt&1, put
    // stage kt+1 (in registers) into the other buffer, issue the global
    // loads of stage kt+2, read k-block 1, then the MFMAs; one barrier.
    int kt = 0;
    for (; kt + 2 < nk; ++kt) {
        const int st = kt & 1;
        read_frags(st, 0, fa0, fb0);
        store_stage(st ^ 1);
        load_stage(kbeg + (kt + 2) * BK);
        read_frags(st, 1, fa1, fb1);
        mma_all(fa0, fb0);
        mma_all(fa1, fb1);
        __syncthreads();
    }
    if (kt + 1 < nk) {  // next to last stage: the last one is already in registers
        const int st = kt & 1;
        read_frags(st, 0, fa0, fb0);
        store_stage(st ^ 1);
        read_frags(st, 1, fa1, fb1);
        mma_all(fa0, fb0);
        mma_all(fa1, fb1);
        __syncthreads();
        ++kt;
    }
    if (kt < nk) {  // last stage
        const int st = kt & 1;
        read_frags(st, 0, fa0, fb0);
        read_frags(st, 1, fa1, fb1);
        mma_all(fa0, fb0);
        mma_all(fa1, fb1);
    }
    __syncthreads();

    epilogue_tile<DT, BM, BN, WM, WN, MODE>(p, acc, (float*)&lds[0][0], m0, n0, split);
}

}  // namespace dge
