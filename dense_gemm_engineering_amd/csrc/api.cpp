// C ABI of the gfx950 dense-GEMM library: argument validation, kernel and
// schedule selection, launches on the caller's stream.  Declarations and the
// contract of every entry point are in include/gemm.h.
#include "gemm.h"
#include "gemm_probe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "launch.h"

// Scratch of gemm_ex_noalloc: its split-K partial sums and its stream-K
// partial tiles and arrival counters live here instead of in a caller
// workspace.  Each device holds one copy from the library's load until the
// process ends.  In host code the name is only a handle: the device address
// is looked up once per device at initialisation and kept per device.
static __device__ __align__(256) unsigned char scratch[GEMM_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace dge;

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    int ok;         // 1 = gfx950, usable
    int cus;        // compute units
    void* scratch;  // this device's copy of `scratch` (null if it could not be resolved)
};

std::once_flag g_dev_once[kMaxDevices];
DeviceInfo g_dev[kMaxDevices];

gemm_status_t current_device(DeviceInfo* out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return GEMM_ERR_DEVICE;
    }
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        DeviceInfo info{0, 0, nullptr};
        if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
            std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 && skinny_init() == hipSuccess) {
            info.ok = 1;
            info.cus = prop.multiProcessorCount;
            // with `dev` current: its copy of the no-allocation scratch
            void* sp = nullptr;
            if (hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch)) == hipSuccess) info.scratch = sp;
        }
        (void)hipGetLastError();
        g_dev[dev] = info;
    });
    if (!g_dev[dev].ok) return GEMM_ERR_DEVICE;
    *out = g_dev[dev];
    return GEMM_OK;
}

// GEMM_TEST_FAIL=<site>: force an error after validation, before any launch.
gemm_status_t forced_failure() {
    const char* f = std::getenv("GEMM_TEST_FAIL");
    if (!f || !*f) return GEMM_OK;
    if (!std::strcmp(f, "launch")) return GEMM_ERR_LAUNCH;
    if (!std::strcmp(f, "device")) return GEMM_ERR_DEVICE;
    if (!std::strcmp(f, "workspace")) return GEMM_ERR_WORKSPACE;
    return GEMM_OK;
}

int in_bytes(int dt) { return dt == IN_F32 ? 4 : 2; }
int out_bytes(int ct) { return ct == OUT_F32 ? 4 : 2; }

// Byte range [lo, hi) spanned by a rows x cols matrix with leading dimension ld.
struct Range {
    uintptr_t lo, hi;
};
Range span(const void* p, int64_t rows, int64_t cols, int64_t ld, int elem) {
    if (!p || rows <= 0 || cols <= 0) return {0, 0};
    uintptr_t lo = (uintptr_t)p;
    return {lo, lo + (uintptr_t)(((rows - 1) * ld + cols) * elem)};
}
bool overlaps(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

struct Gemm {
    int dt;
    int64_t M, N, K;
    float alpha, beta;
    const void* A;
    int64_t lda;
    const void* B;
    int64_t ldb;
    int trans_b;
    void* C;
    int64_t ldc;
    int c_type;
    int epi;
    const void* bias;
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
    int b_q4;  // B is an N x K weight as q4 blocks (18 bytes per 32 weights)
    // measurement only (gemm_probe_clock): per-workgroup clock records, and
    // how many workgroups they can hold
    unsigned long long* clk;
    int64_t clk_cap;
};

constexpr int64_t kMaxDim = (int64_t)1 << 30;

gemm_status_t validate(const Gemm& g) {
    if (g.dt < IN_F16 || g.dt > IN_F32) return GEMM_ERR_INVALID_VALUE;
    if (g.c_type < OUT_F32 || g.c_type > OUT_BF16) return GEMM_ERR_INVALID_VALUE;
    if (g.dt == IN_F32 && g.c_type != OUT_F32) return GEMM_ERR_INVALID_VALUE;
    if (g.epi < EPI_NONE || g.epi > EPI_BIAS_GELU) return GEMM_ERR_INVALID_VALUE;
    if (g.trans_b != 0 && g.trans_b != 1) return GEMM_ERR_INVALID_VALUE;
    if (g.M < 0 || g.N < 0 || g.K < 0) return GEMM_ERR_INVALID_VALUE;
    if (g.M > kMaxDim || g.N > kMaxDim || g.K > kMaxDim) return GEMM_ERR_INVALID_VALUE;
    if (!std::isfinite(g.alpha) || !std::isfinite(g.beta)) return GEMM_ERR_INVALID_VALUE;
    if (g.M == 0 || g.N == 0) return GEMM_OK;
    if (g.ldc < g.N || g.ldc > kMaxDim * 64) return GEMM_ERR_INVALID_VALUE;
    if (g.lda < std::max<int64_t>(1, g.K) || g.lda > kMaxDim * 64) return GEMM_ERR_INVALID_VALUE;
    const int64_t ldb_min = g.trans_b ? std::max<int64_t>(1, g.K) : g.N;
    if (g.ldb < ldb_min || g.ldb > kMaxDim * 64) return GEMM_ERR_INVALID_VALUE;
    // offsets must fit the kernels' 64-bit element indexing with margin
    if ((double)g.M * (double)g.ldc > 9e15 || (double)g.M * (double)g.lda > 9e15 ||
        (double)(g.trans_b ? g.N : g.K) * (double)g.ldb > 9e15)
        return GEMM_ERR_INVALID_VALUE;
    if (!g.C) return GEMM_ERR_INVALID_VALUE;
    if (g.K > 0 && (!g.A || !g.B)) return GEMM_ERR_INVALID_VALUE;
    if (g.epi != EPI_NONE && !g.bias) return GEMM_ERR_INVALID_VALUE;
    const Range rc = span(g.C, g.M, g.N, g.ldc, out_bytes(g.c_type));
    const Range ra = g.K > 0 ? span(g.A, g.M, g.K, g.lda, in_bytes(g.dt)) : Range{0, 0};
    const Range rb = g.K <= 0 ? Range{0, 0}
                     : g.b_q4 ? Range{(uintptr_t)g.B, (uintptr_t)g.B + (uintptr_t)(g.N * (g.K / 32) * 18)}
                     : g.trans_b ? span(g.B, g.N, g.K, g.ldb, in_bytes(g.dt))
                                 : span(g.B, g.K, g.N, g.ldb, in_bytes(g.dt));
    const Range rbias = g.epi != EPI_NONE ? span(g.bias, 1, g.N, g.N, in_bytes(g.dt)) : Range{0, 0};
    if (overlaps(rc, ra) || overlaps(rc, rb) || overlaps(rc, rbias)) return GEMM_ERR_INVALID_VALUE;
    return GEMM_OK;
}

Epilogue make_epilogue(const Gemm& g) {
    Epilogue e;
    e.alpha = g.alpha;
    e.beta = g.beta;
    e.epi = g.epi;
    e.bias = g.bias;
    return e;
}

SimpleArgs simple_args(const Gemm& g) {
    SimpleArgs a;
    a.A = g.A;
    a.B = g.B;
    a.C = g.C;
    a.lda = g.lda;
    a.ldb = g.ldb;
    a.ldc = g.ldc;
    a.M = (int)g.M;
    a.N = (int)g.N;
    a.K = (int)g.K;
    a.trans_b = g.trans_b;
    a.c_type = g.c_type;
    a.ep = make_epilogue(g);
    return a;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int env_int(const char* name, int dflt) {
    const char* v = std::getenv(name);
    if (!v || !*v) return dflt;
    return std::atoi(v);
}

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Workgroups of a tile that run on one CU at once: the 256-row tiles' two
// LDS stages (96 or 128 KB) leave room for one; 128 x 128 and 128 x 64 run
// two.
int tile_occupancy(int tile) {
    return tile == TILE_256x256 || tile == TILE_256x128 || tile == TILE_256x256_W8 ||
                   tile == TILE_256x128_W8
               ? 1
               : 2;
}

// Time model of one round (every CU running tile_occupancy tiles at once) of
// a tile shape: fixed_us (prologue, epilogue, launch) + us_per_k * K.
// Calibrated on 16-bit 4096^3 and 2048 x {4096, 11008} x {4096, 11008}
// products with the direct-to-LDS kernels (4096^3: the 8-wave 256 x 256 tile
// takes ~116 us, the 4-wave one ~130 us, 256 x 128 and 128 x 128 ~146-151 us
// over two rounds); the 8-wave 256 x 128 tile on 2048 x 4096 x K, K = 1024
// .. 11008 (one round: 24.0, 37.3, 64.6, 120.3, 160.2 us for K = 1024, 2048,
// 4096, 8192, 11008).
struct TileCost {
    double fixed_us, us_per_k;
};
TileCost tile_cost(int tile) {
    switch (tile) {
        case TILE_256x256_W8: return {15.0, 0.0246};
        case TILE_256x256: return {17.0, 0.0276};
        case TILE_256x128: return {10.0, 0.0160};
        case TILE_256x128_W8: return {9.0, 0.0136};
        case TILE_128x128: return {10.0, 0.0160};
        default: return {8.0, 0.0110};  // 128 x 64
    }
}

size_t ws_bytes_for(int64_t M, int64_t N, int splits);

// Modelled time of a (tile, splits) schedule: rounds of the tile grid times
// the per-round cost of its K slice, plus for a split the fixup pass that
// re-reads the fp32 partials (at ~5 TB/s).  A partly filled last round runs
// faster per tile (fewer CUs share power and bandwidth): measured ~0.75-0.8x
// of a full round at a third to a half of the CUs, modelled as 0.65 + 0.35 f
// for a fill fraction f.
double schedule_us(int64_t M, int64_t N, int64_t K, int tile, int splits, int bk, int cus) {
    const TileShape ts = tile_shape(tile);
    const TileCost c = tile_cost(tile);
    const int64_t work = (int64_t)ceil_div(M, ts.bm) * ceil_div(N, ts.bn) * splits;
    const int64_t slots = (int64_t)cus * tile_occupancy(tile);
    const int64_t full = work / slots, rest = work - full * slots;
    const int64_t k_slice = (int64_t)ceil_div(ceil_div(K, bk), splits) * bk;
    const double round_us = c.fixed_us + c.us_per_k * (double)k_slice;
    double us = (double)full * round_us;
    if (rest > 0) us += round_us * (0.65 + 0.35 * (double)rest / (double)slots);
    if (splits > 1) us += (double)(4 * splits + 4) * (double)M * (double)N / 5.0e6;
    return us;
}

// fp32 inputs: the fp32 MFMA rate bounds every tile (16x16x4 blocks at a
// sixteenth of the 16-bit rate), so a schedule takes the busiest CU's FLOPs
// at the tile's per-CU rate, plus a fixed cost per launch and, for a split,
// the fixup pass.  Per-CU rates fitted on MI355X to M = N = K = 1024, 2048
// and 4096 over every tile and split (e.g. 4096^3: 8-wave 256 x 256 982 us,
// 128 x 64 1127 us; 2048^3: 128 x 64 154 us, 8-wave 256 x 256 split 4 156
// us; 1024^3: 128 x 64 split 2 34 us); the 16-bit model above, whose partly
// filled rounds run faster for power, picked half-filled grids here (2048^3
// in 299 us).
double tile_rate_f32(int tile) {  // TFLOP/s per CU
    switch (tile) {
        case TILE_256x256_W8: return 0.554;
        case TILE_256x256: return 0.41;
        case TILE_128x128: return 0.47;
        case TILE_128x64: return 0.48;
        default: return 0.46;  // 256 x 128 (both ids run the 4-wave kernel)
    }
}
double schedule_us_f32(int64_t M, int64_t N, int64_t K, int tile, int splits, int bk, int cus) {
    const TileShape ts = tile_shape(tile);
    const int64_t work = (int64_t)ceil_div(M, ts.bm) * ceil_div(N, ts.bn) * splits;
    const int64_t per_cu = (work + cus - 1) / cus;
    const int64_t k_slice = (int64_t)ceil_div(ceil_div(K, bk), splits) * bk;
    const double flops = 2.0 * ts.bm * ts.bn * (double)k_slice * (double)per_cu;
    double us = 12.0 + flops / (tile_rate_f32(tile) * 1e6);
    // the fixup's partial traffic at ~4 TB/s (2048^3 split 4: ~23 us)
    if (splits > 1) us += (double)(4 * splits + 4) * (double)M * (double)N / 4.0e6;
    return us;
}

// Persistent schedule with a stream-K tail (direct-to-LDS kernels): the grid
// is every CU slot the tile allows (at most one workgroup per iteration).
// Its time is R whole-tile rounds plus the tail's ceil(I / G) stages, plus
// per extra segment a share of the prologue and epilogue the overlap does
// not hide, plus, when tail tiles are split, the fp32 partial stores and the
// reduction (measured on MI355X: ~45 us per launch for 256 x 256 tiles,
// scaling with the tile area).
constexpr double kSkSegmentUs = 3.0, kSkPartialUs = 45.0;

int64_t sk_grid(int tile, int64_t iters, int cus) {
    return std::min<int64_t>((int64_t)cus * tile_occupancy(tile), iters);
}

// Whole-tile rounds before the stream-K tail: as many full rounds of the
// grid as fit, less one while the tail would have fewer iterations than
// workgroups (every workgroup's tail range must be non-empty, or a split
// tile would count a workgroup that never arrives).
int64_t sk_rounds(int64_t tiles, int64_t S, int64_t G) {
    int64_t R = tiles / G;
    while (R > 0 && tiles > R * G && (tiles - R * G) * S < G) --R;
    return R;
}

// Workspace of the stream-K schedule: 2 fp32 partial tiles per workgroup,
// then one 32-bit counter per tile (256-byte aligned).
size_t sk_counter_offset(int tile, int64_t grid) {
    const TileShape ts = tile_shape(tile);
    return (size_t)2 * grid * ts.bm * ts.bn * sizeof(float);
}
size_t sk_ws_bytes(int tile, int64_t grid, int64_t tiles) {
    return sk_counter_offset(tile, grid) + ((size_t)tiles * 4 + 255) / 256 * 256;
}

double sk_schedule_us(int64_t M, int64_t N, int64_t K, int tile, int bk, int cus) {
    const TileShape ts = tile_shape(tile);
    const TileCost c = tile_cost(tile);
    const int64_t tiles = (int64_t)ceil_div(M, ts.bm) * ceil_div(N, ts.bn);
    const int64_t S = ceil_div(K, bk), G = sk_grid(tile, tiles * S, cus);
    const int64_t R = sk_rounds(tiles, S, G), I = (tiles - R * G) * S;
    const int64_t per = I > 0 ? (I + G - 1) / G : 0;  // tail stages per workgroup
    double us = c.fixed_us + c.us_per_k * (double)((R * S + per) * bk);
    const int64_t segments = R + (per + S - 1) / S + (I % G != 0 ? 1 : 0);
    us += kSkSegmentUs * (double)std::max<int64_t>(segments - 1, 0);
    if (I > 0 && (I % G != 0 || (I / G) % S != 0))
        us += kSkPartialUs * (double)(ts.bm * ts.bn) / 65536.0;
    return us;
}

// Joint choice of tile shape and K split.  tile / splits: the caller's
// request (GEMM_TILE_AUTO / 0 = free); allowed: bit t set for each tile id
// that may be chosen.  A split is only considered while ws_bytes covers its
// partials; each K slice keeps at least 16 stages.
// sk_allowed: bit t set where the stream-K schedule may run tile t; with
// sk_only, only those are considered.  *sk = 1 when stream-K wins.
void choose_schedule(int64_t M, int64_t N, int64_t K, int dt, int cus, size_t ws_bytes,
                     int* tile, int* splits, unsigned allowed = ~0u, unsigned sk_allowed = 0,
                     bool sk_only = false, int* sk = nullptr) {
    const int bk = stage_k(dt);
    const int t_lo = *tile == GEMM_TILE_AUTO ? TILE_256x256 : *tile;
    const int t_hi = *tile == GEMM_TILE_AUTO ? TILE_LAST : *tile;
    int best_t = t_lo, best_s = 1, best_sk = 0;
    double best = 1e300;
    for (int t = t_lo; t <= t_hi; ++t) {
        if ((sk_allowed >> t & 1u) && *splits <= 1) {
            const TileShape ts = tile_shape(t);
            const int64_t tiles = (int64_t)ceil_div(M, ts.bm) * ceil_div(N, ts.bn);
            const int64_t I = tiles * ceil_div(K, bk);
            if (ws_bytes >= sk_ws_bytes(t, sk_grid(t, I, cus), tiles)) {
                const double us = sk_schedule_us(M, N, K, t, bk, cus);
                if (us < best * 0.999) {
                    best = us;
                    best_t = t;
                    best_s = 1;
                    best_sk = 1;
                }
            }
        }
        if (sk_only || !(allowed >> t & 1u)) continue;
        for (int sp = 1; sp <= 8; ++sp) {
            if (*splits > 0 && sp != *splits) continue;
            if (sp > 1 && (K / sp < 16 * (int64_t)bk || ws_bytes < ws_bytes_for(M, N, sp)))
                continue;
            const double us = dt == IN_F32 ? schedule_us_f32(M, N, K, t, sp, bk, cus)
                                           : schedule_us(M, N, K, t, sp, bk, cus);
            if (us < best * 0.999) {
                best = us;
                best_t = t;
                best_s = sp;
                best_sk = 0;
            }
        }
    }
    *tile = best_t;
    if (*splits == 0) *splits = best_s;
    if (sk) *sk = best_sk;
}

size_t ws_bytes_for(int64_t M, int64_t N, int splits) {
    return splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// Column split: the first n1 columns as whole rounds of tile `tile` (every
// CU slot busy for the full K), the other N - n1 columns as a problem of
// their own with their best schedule (tile2, splits2).  It pays where the
// plain schedule's last round is mostly empty but costs a full K: 2048 x
// 11008 x 4096 has 344 tiles of 256 x 256 for 256 CUs, 1.34 rounds; as
// 8192 columns (one round) + 2816 columns (smaller tiles, one short round)
// it saves the empty part of the second round.  allowed2(n) gives the tiles
// the rest may use.  Chosen only when the model says 3% or more.
struct ColumnSplit {
    int64_t n1;
    int tile, tile2, splits2;
};
template <typename AllowedFn>
bool choose_column_split(int64_t M, int64_t N, int64_t K, int dt, int cus, size_t ws_bytes,
                         unsigned allowed, AllowedFn allowed2, ColumnSplit* cs) {
    const int bk = stage_k(dt);
    int t0 = GEMM_TILE_AUTO, s0 = 0;
    choose_schedule(M, N, K, dt, cus, ws_bytes, &t0, &s0, allowed);
    double best = schedule_us(M, N, K, t0, s0, bk, cus) * 0.97;
    bool found = false;
    for (int t = TILE_256x256; t <= TILE_LAST; ++t) {
        if (!(allowed >> t & 1u)) continue;
        const TileShape ts = tile_shape(t);
        const int64_t tm = ceil_div(M, ts.bm), slots = (int64_t)cus * tile_occupancy(t);
        if (M % ts.bm != 0 || slots % tm != 0) continue;
        const int64_t cols = slots / tm;  // tile columns of one full round
        const int64_t n1 = (N / ts.bn) / cols * cols * ts.bn;
        if (n1 <= 0 || n1 >= N) continue;
        const unsigned a2 = allowed2(N - n1);
        if (!a2) continue;
        int t2 = GEMM_TILE_AUTO, s2 = 0;
        choose_schedule(M, N - n1, K, dt, cus, ws_bytes, &t2, &s2, a2);
        const double us = schedule_us(M, n1, K, t, 1, bk, cus) + schedule_us(M, N - n1, K, t2, s2, bk, cus);
        if (us < best) {
            best = us;
            found = true;
            *cs = ColumnSplit{n1, t, t2, s2};
        }
    }
    return found;
}

gemm_status_t launch_status(hipError_t e) {
    if (e == hipSuccess) return GEMM_OK;
    return GEMM_ERR_LAUNCH;
}

// direct: 0 = register-staged kernel only, 1 = direct-to-LDS kernel when the
// problem qualifies (full tiles, 16-bit inputs, aligned operands).
// The direct-to-LDS kernels address each load, and each 16-bit output store,
// as a wave-uniform base plus a 32-bit per-lane byte offset of up to 32 rows:
// leading dimensions below 2^24 elements keep it under 2^31.
bool direct_ld_ok(const Gemm& g) {
    return g.lda < ((int64_t)1 << 24) && (g.b_q4 || g.ldb < ((int64_t)1 << 24)) &&
           g.ldc < ((int64_t)1 << 24);
}

// Tiles whose stream-K schedule can run this problem: the direct-to-LDS
// kernel's conditions (16-bit inputs, full tiles, whole stages, aligned
// operands, and for a K x N B at least 128 columns).
unsigned streamk_tiles(const Gemm& g) {
    if (g.b_q4 || g.dt == IN_F32 || g.K <= 0 || g.K % stage_k(g.dt) != 0 || !direct_ld_ok(g))
        return 0;
    if (env_int("GEMM_DIRECT", 1) == 0 || env_int("GEMM_STREAMK", 1) == 0) return 0;
    const int vec_el = 16 / in_bytes(g.dt);
    const bool vec = aligned16(g.A) && aligned16(g.B) && aligned16(g.C) && g.lda % vec_el == 0 &&
                     g.ldb % vec_el == 0 && (g.ldc * out_bytes(g.c_type)) % 16 == 0;
    if (!vec) return 0;
    unsigned m = 0;
    for (int t = TILE_256x256; t <= TILE_LAST; ++t) {
        const TileShape s = tile_shape(t);
        if (g.M % s.bm == 0 && g.N % s.bn == 0 && (g.trans_b || s.bn >= 128)) m |= 1u << t;
    }
    return m;
}

// The fused q4 kernel's tiles: full tiles of an M x N problem.
unsigned q4_tiles(int64_t M, int64_t N) {
    unsigned m = 0;
    for (int t = TILE_256x256; t <= TILE_LAST; ++t) {
        const TileShape s = tile_shape(t);
        if (M % s.bm == 0 && N % s.bn == 0) m |= 1u << t;
    }
    return m;
}

// Columns [c0, c0 + n) of g as a problem of its own (same A; B, C and the
// bias offset to column c0).
Gemm column_range(const Gemm& g, int64_t c0, int64_t n) {
    Gemm h = g;
    h.N = n;
    if (g.b_q4)
        h.B = (const char*)g.B + c0 * (g.K / 32) * 18;
    else
        h.B = (const char*)g.B + (g.trans_b ? c0 * g.ldb : c0) * in_bytes(g.dt);
    h.C = (char*)g.C + c0 * out_bytes(g.c_type);
    if (g.bias) h.bias = (const char*)g.bias + c0 * in_bytes(g.dt);
    return h;
}

// streamk: 1 = the stream-K schedule was asked for (it runs where eligible);
// colsplit: the automatic schedule may split the columns (not within a part)
gemm_status_t run_mfma(const Gemm& g, int tile, int splits, int cus, int direct,
                       int streamk = 0, bool colsplit = true) {
    if (tile != GEMM_TILE_AUTO && (tile < TILE_256x256 || tile > TILE_LAST))
        return GEMM_ERR_INVALID_VALUE;
    if (colsplit && tile == GEMM_TILE_AUTO && splits == 0 && !streamk && direct &&
        g.dt != IN_F32 && env_int("GEMM_COLSPLIT", 1) != 0) {
        const unsigned all = g.b_q4 ? q4_tiles(g.M, g.N) : ~0u;
        auto allowed2 = [&](int64_t n2) { return g.b_q4 ? q4_tiles(g.M, n2) : ~0u; };
        ColumnSplit cs;
        if (all && choose_column_split(g.M, g.N, g.K, g.dt, cus, g.ws ? g.ws_bytes : 0, all,
                                       allowed2, &cs)) {
            if (g.clk) return GEMM_ERR_NOT_SUPPORTED;  // clock records cover one launch
            gemm_status_t st = run_mfma(column_range(g, 0, cs.n1), cs.tile, 1, cus, direct, 0, false);
            if (st != GEMM_OK) return st;
            // the rest with its tile; its split is chosen again against the
            // workspace (the same choice, unless the workspace is misaligned)
            return run_mfma(column_range(g, cs.n1, g.N - cs.n1), cs.tile2, 0, cus, direct, 0, false);
        }
    }
    const bool explicit_split = splits > 1;
    unsigned allowed = ~0u;
    if (g.b_q4) {
        // the fused q4 kernel takes full tiles, whole 64-deep stages, a 4-byte
        // aligned block array and the direct-load alignment of A and C
        allowed = 0;
        for (int t = TILE_256x256; t <= TILE_LAST; ++t) {
            const TileShape s = tile_shape(t);
            if (g.M % s.bm == 0 && g.N % s.bn == 0) allowed |= 1u << t;
        }
        if (tile != GEMM_TILE_AUTO) allowed &= 1u << tile;
        const bool ok = allowed && g.K % 64 == 0 && direct_ld_ok(g) && ((uintptr_t)g.B & 3) == 0 && aligned16(g.A) &&
                        aligned16(g.C) && g.lda % 8 == 0 && (g.ldc * out_bytes(g.c_type)) % 16 == 0;
        if (!ok) return GEMM_ERR_NOT_SUPPORTED;
    }
    // the stream-K schedule only runs when asked for: measured on MI355X it
    // does not beat the data-parallel and split schedules on any workload
    // here (the workgroups of an XCD sit at different K stages, so its 4 MB
    // L2 no longer shares A/B stage blocks between them; split tiles move
    // BM x BN fp32 partials through memory twice)
    unsigned sk_allowed = direct && streamk ? streamk_tiles(g) : 0;
    if (tile != GEMM_TILE_AUTO) sk_allowed &= 1u << tile;
    const bool sk_only = streamk && sk_allowed != 0;
    int sk = 0;
    if (tile == GEMM_TILE_AUTO || splits == 0 || sk_only)
        choose_schedule(g.M, g.N, g.K, g.dt, cus, g.ws ? g.ws_bytes : 0, &tile, &splits, allowed,
                        sk_allowed, sk_only, &sk);
    if (sk_only && !sk) return GEMM_ERR_WORKSPACE;  // stream-K was asked for and does not fit
    const TileShape ts = tile_shape(tile);
    const int bk = stage_k(g.dt);
    const int max_splits = std::max(1, ceil_div(g.K, bk));
    if (splits > max_splits) splits = max_splits;
    if (splits > 1) {
        const size_t need = ws_bytes_for(g.M, g.N, splits);
        if (!g.ws || g.ws_bytes < need || !aligned16(g.ws)) {
            if (explicit_split) return GEMM_ERR_WORKSPACE;
            splits = 1;
        }
    }
    MfmaArgs a{};
    a.A = g.A;
    a.B = g.B;
    a.C = g.C;
    a.ws = splits > 1 ? (float*)g.ws : nullptr;
    a.lda = g.lda;
    a.ldb = g.ldb;
    a.ldc = g.ldc;
    a.M = (int)g.M;
    a.N = (int)g.N;
    a.K = (int)g.K;
    a.tiles_m = ceil_div(g.M, ts.bm);
    a.tiles_n = ceil_div(g.N, ts.bn);
    a.splits = splits;
    // K slices are whole stages
    const int stages = ceil_div(g.K, bk);
    a.k_per_split = splits > 1 ? ceil_div(stages, splits) * bk : (int)std::max<int64_t>(g.K, 1);
    if (splits > 1) a.splits = ceil_div(g.K, a.k_per_split);
    splits = a.splits;
    const int per_xcd = std::max(1, (a.tiles_m * a.tiles_n) / 8);
    int gm = 1;
    while (gm * gm * 2 < per_xcd) gm *= 2;
    a.group_m = std::max(1, std::min(env_int("GEMM_GROUP_M", gm), a.tiles_m));
    a.c_type = g.c_type;
    const int vec_el = 16 / in_bytes(g.dt);
    const bool vec = aligned16(g.A) && (g.b_q4 || aligned16(g.B)) && aligned16(g.C) &&
                     g.lda % vec_el == 0 && (g.b_q4 || g.ldb % vec_el == 0) &&
                     (g.ldc * out_bytes(g.c_type)) % 16 == 0;
    a.vec_ok = vec ? 1 : 0;
    a.ep = make_epilogue(g);
    // (K = 0 takes the bounds-checked loads: the unchecked kernels load their
    // first stages before looking at the stage count)
    const bool fast = vec && g.K > 0 && g.M % ts.bm == 0 && g.N % ts.bn == 0 && g.K % bk == 0 &&
                      (splits == 1 || a.k_per_split % bk == 0);
    const int64_t nwg = (int64_t)a.tiles_m * a.tiles_n * splits;
    if (nwg > 0x7fffffff) return GEMM_ERR_NOT_SUPPORTED;
    hipError_t e;
    if (g.b_q4) {
        if (!fast) return GEMM_ERR_NOT_SUPPORTED;
        e = launch_mfma_q4_f16(tile, a, (int)nwg, g.stream);
        if (e == hipSuccess && splits > 1)
            e = launch_splitk_fixup(g.dt, simple_args(g), (const float*)g.ws, splits, g.stream);
        return launch_status(e);
    }
    const bool use_direct = direct && fast && g.dt != IN_F32 && direct_ld_ok(g) &&
                            (g.trans_b || ts.bn >= 128) && env_int("GEMM_DIRECT", 1) != 0;
    if (g.clk) {
        // clock records: one data-parallel launch of a direct-to-LDS kernel
        if (g.b_q4 || !use_direct || sk || splits > 1 || nwg > g.clk_cap)
            return GEMM_ERR_NOT_SUPPORTED;
        a.clk = g.clk;
    }
    if (sk && use_direct && aligned16(g.ws)) {
        const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n, S = g.K / bk;
        const int64_t G = sk_grid(tile, tiles * S, cus);
        a.ws = nullptr;
        a.splits = 1;
        a.k_per_split = (int)g.K;
        a.sk_stages = (int)S;
        a.sk_rounds = (int)sk_rounds(tiles, S, G);
        a.sk_ws = (float*)g.ws;
        a.sk_cnt = (unsigned*)((char*)g.ws + sk_counter_offset(tile, G));
        // the arrival counters are only read when a tail tile is split
        const int64_t I = (tiles - (int64_t)a.sk_rounds * G) * S;
        const bool split_tail = I > 0 && (I % G != 0 || (I / G) % S != 0);
        e = split_tail ? launch_clear_u32(a.sk_cnt, tiles, g.stream) : hipSuccess;
        if (e == hipSuccess)
            e = g.dt == IN_F16 ? launch_mfma_direct_f16(tile, g.trans_b, a, (int)G, 1, g.stream)
                               : launch_mfma_direct_bf16(tile, g.trans_b, a, (int)G, 1, g.stream);
        return launch_status(e);
    }
    if (use_direct) {
        e = g.dt == IN_F16 ? launch_mfma_direct_f16(tile, g.trans_b, a, (int)nwg, 0, g.stream)
                           : launch_mfma_direct_bf16(tile, g.trans_b, a, (int)nwg, 0, g.stream);
        if (e != hipSuccess) return launch_status(e);
        if (splits > 1)
            e = launch_splitk_fixup(g.dt, simple_args(g), (const float*)g.ws, splits, g.stream);
        return launch_status(e);
    }
    switch (g.dt) {
        case IN_F16: e = launch_mfma_f16(tile, g.trans_b, fast, a, (int)nwg, g.stream); break;
        case IN_BF16: e = launch_mfma_bf16(tile, g.trans_b, fast, a, (int)nwg, g.stream); break;
        default: e = launch_mfma_f32(tile, g.trans_b, fast, a, (int)nwg, g.stream); break;
    }
    if (e != hipSuccess) return launch_status(e);
    if (splits > 1) e = launch_splitk_fixup(g.dt, simple_args(g), (const float*)g.ws, splits, g.stream);
    return launch_status(e);
}

// The tall-skinny kernel: 16-bit inputs, K a multiple of 32 up to 256,
// N up to 256, X rows 16-byte aligned, W^T and the staging of at least two
// waves fitting 160 KB of LDS.
bool skinny_eligible(const Gemm& g) {
    if (g.dt == IN_F32 || g.K < 32 || g.K > 256 || g.K % 32 != 0 || g.N > 256) return false;
    if (!aligned16(g.A) || g.lda % 8 != 0) return false;
    const int nt = (ceil_div(g.N, 16) + 1) / 2 * 2;
    return skinny_lds_bytes(g.trans_b, nt, (int)g.K, out_bytes(g.c_type), 2) <= 160 * 1024;
}

// The automatic schedule takes the tall-skinny kernel for M >> N.
bool skinny_auto(const Gemm& g) {
    return skinny_eligible(g) && g.M >= 8 * g.N && g.M >= 4096 && env_int("GEMM_SKINNY", 1) != 0;
}

gemm_status_t run_skinny(const Gemm& g, int cus) {
    SkinnyArgs a;
    a.X = g.A;
    a.W = g.B;
    a.C = g.C;
    a.ldx = g.lda;
    a.ldw = g.ldb;
    a.ldc = g.ldc;
    a.M = (int)g.M;
    a.N = (int)g.N;
    a.K = (int)g.K;
    const int nt = (ceil_div(g.N, 16) + 1) / 2 * 2;
    a.pitch = skinny_pitch(g.trans_b, (int)g.K);
    a.c_type = g.c_type;
    const int cb = out_bytes(g.c_type);
    a.vec_c = (aligned16(g.B) && g.ldb % 8 == 0 ? 2 : 0) |
              (aligned16(g.C) && (g.ldc * cb) % 16 == 0 && (g.N * cb) % 16 == 0 ? 4 : 0);
    a.ep = make_epilogue(g);
    a.rec = g.clk;
    const int waves = skinny_waves(g.trans_b, nt, (int)g.K, cb);
    const size_t lds = skinny_lds_bytes(g.trans_b, nt, (int)g.K, cb, waves);
    // one workgroup per CU: W is staged once per CU and amortised over the
    // CU's share of the rows (16 * skinny_rb per wave per step)
    const int grid = std::max(1, std::min(ceil_div(g.M, waves * 16 * skinny_rb(nt)), cus));
    if (g.clk && g.clk_cap < grid) return GEMM_ERR_NOT_SUPPORTED;
    return launch_status(launch_skinny(g.dt, nt, g.trans_b, a, grid, waves, lds, g.stream));
}

// The decode-shaped kernel: a few rows of 16-bit X against an N x K weight.
bool decode_eligible(const Gemm& g) {
    return g.dt != IN_F32 && g.trans_b == 1 && !g.b_q4 && g.M >= 1 && g.M <= 64 &&
           g.K % 8 == 0 && aligned16(g.A) && aligned16(g.B) && g.lda % 8 == 0 && g.ldb % 8 == 0;
}

// K slices of the split decode schedule for 17 <= M <= 64 rows (0: the
// one-pass kernel): about one workgroup per CU, each wave of a slice keeping
// at least one whole k-block.  Measured on a 4096 x 4096 weight (graph
// replays, HBM-cold), split + fixup against one pass: M = 17 12.0 / 12.6 us,
// M = 32 12.8 / 15.3, M = 48 12.5 / 18.9, M = 64 14.6 / 21.8; M <= 16 keeps
// the one-pass kernel (its X traffic is no larger than the weight's).
int decode_ksplit(int64_t M, int64_t N, int64_t K, int cus) {
    if (M <= 16 || M > 64 || N % DSPLIT_ROWS != 0 || K % 32 != 0 ||
        env_int("GEMM_DECODE_SPLIT", 1) == 0)
        return 0;
    const int64_t tiles = N / DSPLIT_ROWS;
    int ks = (int)std::max<int64_t>(1, std::min<int64_t>(8, (cus + tiles / 2) / tiles));
    while (ks > 1 && K / 32 / ks < DECODE_WAVES) --ks;
    return ks > 1 ? ks : 0;
}

size_t decode_ws_bytes(int64_t M, int64_t N, int ks) {
    return ks > 1 ? (size_t)ks * (size_t)M * (size_t)N * sizeof(float) : 0;
}

DecodeArgs decode_args(const Gemm& g) {
    DecodeArgs a{};
    a.X = g.A;
    a.W = g.B;
    a.C = g.C;
    a.ldx = g.lda;
    a.ldw = g.ldb;
    a.ldc = g.ldc;
    a.M = (int)g.M;
    a.N = (int)g.N;
    a.K = (int)g.K;
    a.c_type = g.c_type;
    a.ep = make_epilogue(g);
    return a;
}

gemm_status_t run_decode(const Gemm& g, int cus) {
    const int ks = decode_ksplit(g.M, g.N, g.K, cus);
    if (ks > 1 && g.ws && aligned16(g.ws) && g.ws_bytes >= decode_ws_bytes(g.M, g.N, ks)) {
        DecodeArgs a = decode_args(g);
        a.ksplit = ks;
        a.ws = (float*)g.ws;
        if (g.clk && g.clk_cap < g.N / DSPLIT_ROWS * ks) return GEMM_ERR_NOT_SUPPORTED;
        a.rec = g.clk;
        hipError_t e = launch_decode_split(g.dt, a, g.stream);
        if (e == hipSuccess) e = launch_splitk_fixup(g.dt, simple_args(g), a.ws, ks, g.stream);
        return launch_status(e);
    }
    if (g.clk) return GEMM_ERR_NOT_SUPPORTED;
    return launch_status(launch_decode(g.dt, decode_args(g), g.stream));
}

gemm_status_t run_gemm(const Gemm& g, const gemm_tuning_t* tuning) {
    gemm_status_t st = validate(g);
    if (st != GEMM_OK) return st;
    gemm_tuning_t tn{GEMM_ALGO_AUTO, GEMM_TILE_AUTO, 0};
    if (tuning) tn = *tuning;
    if (tn.algo < GEMM_ALGO_AUTO || tn.algo > GEMM_ALGO_STREAMK) return GEMM_ERR_INVALID_VALUE;
    if (tn.tile < GEMM_TILE_AUTO || tn.tile > GEMM_TILE_256x128_W8) return GEMM_ERR_INVALID_VALUE;
    if (tn.splits < 0) return GEMM_ERR_INVALID_VALUE;
    if (g.M == 0 || g.N == 0) return GEMM_OK;
    if ((st = forced_failure()) != GEMM_OK) return st;
    DeviceInfo dev;
    if ((st = current_device(&dev)) != GEMM_OK) return st;
    switch (tn.algo) {
        case GEMM_ALGO_NAIVE:
            if (tn.splits > 1) return GEMM_ERR_INVALID_VALUE;
            return launch_status(launch_naive(g.dt, simple_args(g), g.stream));
        case GEMM_ALGO_LDS_TILED:
            if (tn.splits > 1) return GEMM_ERR_INVALID_VALUE;
            return launch_status(launch_lds_tiled(g.dt, simple_args(g), g.stream));
        case GEMM_ALGO_MFMA:
            return run_mfma(g, tn.tile, tn.splits, dev.cus, 0);
        case GEMM_ALGO_SKINNY:
            if (tn.splits > 1) return GEMM_ERR_INVALID_VALUE;
            if (skinny_eligible(g)) return run_skinny(g, dev.cus);
            return run_mfma(g, tn.tile, 1, dev.cus, 1);
        case GEMM_ALGO_DECODE:
            if (tn.splits > 1) return GEMM_ERR_INVALID_VALUE;
            if (g.K > 0 && decode_eligible(g)) return run_decode(g, dev.cus);
            return run_mfma(g, tn.tile, 1, dev.cus, 1);
        case GEMM_ALGO_STREAMK:
            if (tn.splits > 1) return GEMM_ERR_INVALID_VALUE;
            return run_mfma(g, tn.tile, 0, dev.cus, 1, 1);
        case GEMM_ALGO_AUTO:
            if (tn.tile == GEMM_TILE_AUTO && tn.splits <= 1 && g.K > 0 && decode_eligible(g))
                return run_decode(g, dev.cus);
            if (tn.tile == GEMM_TILE_AUTO && tn.splits <= 1 && skinny_auto(g))
                return run_skinny(g, dev.cus);
            return run_mfma(g, tn.tile, tn.splits, dev.cus, 1);
        default:
            return run_mfma(g, tn.tile, tn.splits, dev.cus, 1);
    }
}

Gemm make_gemm(int dt, int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
               const void* B, int64_t ldb, int trans_b, float beta, void* C, int64_t ldc,
               gemm_out_t c_type, gemm_epilogue_t epi, const void* bias, void* workspace,
               size_t workspace_bytes, void* stream) {
    Gemm g;
    g.dt = dt;
    g.M = M;
    g.N = N;
    g.K = K;
    g.alpha = alpha;
    g.beta = beta;
    g.A = A;
    g.lda = lda;
    g.B = B;
    g.ldb = ldb;
    g.trans_b = trans_b;
    g.C = C;
    g.ldc = ldc;
    g.c_type = (int)c_type;
    g.epi = (int)epi;
    g.bias = bias;
    g.ws = workspace;
    g.ws_bytes = workspace_bytes;
    g.stream = (hipStream_t)stream;
    g.b_q4 = 0;
    g.clk = nullptr;
    g.clk_cap = 0;
    return g;
}

}  // namespace

extern "C" {

gemm_status_t gemm_f16(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                       const void* B, int64_t ldb, int trans_b, float beta, void* C, int64_t ldc,
                       gemm_out_t c_type, gemm_epilogue_t epi, const void* bias, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return run_gemm(make_gemm(IN_F16, M, N, K, alpha, A, lda, B, ldb, trans_b, beta, C, ldc, c_type,
                              epi, bias, workspace, workspace_bytes, stream),
                    nullptr);
}

gemm_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                        const void* B, int64_t ldb, int trans_b, float beta, void* C, int64_t ldc,
                        gemm_out_t c_type, gemm_epilogue_t epi, const void* bias, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return run_gemm(make_gemm(IN_BF16, M, N, K, alpha, A, lda, B, ldb, trans_b, beta, C, ldc,
                              c_type, epi, bias, workspace, workspace_bytes, stream),
                    nullptr);
}

gemm_status_t gemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                       const void* B, int64_t ldb, int trans_b, float beta, void* C, int64_t ldc,
                       gemm_out_t c_type, gemm_epilogue_t epi, const void* bias, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return run_gemm(make_gemm(IN_F32, M, N, K, alpha, A, lda, B, ldb, trans_b, beta, C, ldc, c_type,
                              epi, bias, workspace, workspace_bytes, stream),
                    nullptr);
}

gemm_status_t gemm_ex(gemm_in_t in_type, int64_t M, int64_t N, int64_t K, float alpha,
                      const void* A, int64_t lda, const void* B, int64_t ldb, int trans_b,
                      float beta, void* C, int64_t ldc, gemm_out_t c_type, gemm_epilogue_t epi,
                      const void* bias, void* workspace, size_t workspace_bytes,
                      const gemm_tuning_t* tuning, void* stream) {
    return run_gemm(make_gemm((int)in_type, M, N, K, alpha, A, lda, B, ldb, trans_b, beta, C, ldc,
                              c_type, epi, bias, workspace, workspace_bytes, stream),
                    tuning);
}

gemm_status_t gemm_ex_noalloc(gemm_in_t in_type, int64_t M, int64_t N, int64_t K, float alpha,
                              const void* A, int64_t lda, const void* B, int64_t ldb,
                              int trans_b, float beta, void* C, int64_t ldc, gemm_out_t c_type,
                              gemm_epilogue_t epi, const void* bias, const gemm_tuning_t* tuning,
                              void* stream) {
    Gemm g = make_gemm((int)in_type, M, N, K, alpha, A, lda, B, ldb, trans_b, beta, C, ldc,
                       c_type, epi, bias, nullptr, 0, stream);
    gemm_status_t st = validate(g);
    if (st != GEMM_OK || g.M == 0 || g.N == 0) return st;
    DeviceInfo dev;
    if ((st = current_device(&dev)) != GEMM_OK) return st;
    if (!dev.scratch) return GEMM_ERR_DEVICE;
    // the schedule is chosen as for a caller workspace of the scratch's size;
    // a request that needs more (an explicit split or stream-K) is rejected
    g.ws = dev.scratch;
    g.ws_bytes = GEMM_NOALLOC_SCRATCH_BYTES;
    st = run_gemm(g, tuning);
    return st == GEMM_ERR_WORKSPACE ? GEMM_ERR_SCRATCH : st;
}

gemm_status_t gemm_probe_clock(gemm_in_t in_type, int64_t M, int64_t N, int64_t K, float alpha,
                               const void* A, int64_t lda, const void* B, int64_t ldb,
                               int trans_b, float beta, void* C, int64_t ldc, gemm_out_t c_type,
                               gemm_epilogue_t epi, const void* bias, unsigned long long* clk,
                               int64_t clk_entries, void* stream) {
    if (!clk || clk_entries <= 0 || ((uintptr_t)clk & 15)) return GEMM_ERR_INVALID_VALUE;
    Gemm g = make_gemm((int)in_type, M, N, K, alpha, A, lda, B, ldb, trans_b, beta, C, ldc,
                       c_type, epi, bias, nullptr, 0, stream);
    g.clk = clk;
    g.clk_cap = clk_entries;
    gemm_status_t st = validate(g);
    if (st != GEMM_OK || g.M == 0 || g.N == 0) return st;
    if (g.K == 0 || g.dt == IN_F32) return GEMM_ERR_NOT_SUPPORTED;
    DeviceInfo dev;
    if ((st = current_device(&dev)) != GEMM_OK) return st;
    return run_mfma(g, GEMM_TILE_AUTO, 0, dev.cus, 1);
}

gemm_status_t gemm_probe_phases(gemm_in_t in_type, int64_t M, int64_t N, int64_t K,
                                const void* A, int64_t lda, const void* B, int64_t ldb,
                                int trans_b, void* C, int64_t ldc, gemm_out_t c_type,
                                gemm_epilogue_t epi, const void* bias, void* workspace,
                                size_t workspace_bytes, unsigned long long* rec,
                                int64_t rec_entries, void* stream) {
    if (!rec || rec_entries <= 0 || ((uintptr_t)rec & 15)) return GEMM_ERR_INVALID_VALUE;
    Gemm g = make_gemm((int)in_type, M, N, K, 1.0f, A, lda, B, ldb, trans_b, 0.0f, C, ldc,
                       c_type, epi, bias, workspace, workspace_bytes, stream);
    g.clk = rec;
    g.clk_cap = rec_entries;
    gemm_status_t st = validate(g);
    if (st != GEMM_OK || g.M == 0 || g.N == 0) return st;
    if (g.K == 0) return GEMM_ERR_NOT_SUPPORTED;
    DeviceInfo dev;
    if ((st = current_device(&dev)) != GEMM_OK) return st;
    if (decode_eligible(g) && decode_ksplit(g.M, g.N, g.K, dev.cus) > 1) return run_decode(g, dev.cus);
    if (skinny_auto(g)) return run_skinny(g, dev.cus);
    return GEMM_ERR_NOT_SUPPORTED;
}

gemm_status_t gemm_probe_mfma(gemm_in_t in_type, const void* A, int64_t lda, const void* B,
                              int64_t ldb, int64_t rows, int64_t cols, int k_blocks, float* out,
                              unsigned long long* clk, void* stream) {
    if ((in_type != GEMM_IN_F16 && in_type != GEMM_IN_BF16) || !A || !B || !out ||
        !aligned16(A) || !aligned16(B) || rows < 4096 || cols < 64 || lda < cols || ldb < cols ||
        lda % 8 != 0 || ldb % 8 != 0 || lda > kMaxDim || ldb > kMaxDim || k_blocks < 1 ||
        ((uintptr_t)clk & 15))
        return GEMM_ERR_INVALID_VALUE;
    DeviceInfo dev;
    gemm_status_t st = current_device(&dev);
    if (st != GEMM_OK) return st;
    return launch_status(launch_probe_mfma((int)in_type, A, B, lda, ldb, k_blocks, out, clk,
                                           (hipStream_t)stream));
}

gemm_status_t gemm_probe_read(const void* src, size_t bytes, int grid, unsigned* out,
                              void* stream) {
    if (!src || !out || !aligned16(src) || bytes % 16 != 0 || grid < 1 || grid > 65536)
        return GEMM_ERR_INVALID_VALUE;
    if (bytes == 0) return GEMM_OK;
    DeviceInfo dev;
    gemm_status_t st = current_device(&dev);
    if (st != GEMM_OK) return st;
    return launch_status(
        launch_probe_read(src, (int64_t)(bytes / 16), out, grid, (hipStream_t)stream));
}

gemm_status_t gemm_probe_copy(const void* src, void* dst, size_t bytes, int grid, void* stream) {
    if (!src || !dst || !aligned16(src) || !aligned16(dst) || bytes % 16 != 0 || grid < 1 ||
        grid > 65536)
        return GEMM_ERR_INVALID_VALUE;
    if (bytes == 0) return GEMM_OK;
    if (overlaps(Range{(uintptr_t)src, (uintptr_t)src + bytes},
                 Range{(uintptr_t)dst, (uintptr_t)dst + bytes}))
        return GEMM_ERR_INVALID_VALUE;
    DeviceInfo dev;
    gemm_status_t st = current_device(&dev);
    if (st != GEMM_OK) return st;
    return launch_status(
        launch_probe_copy(src, dst, (int64_t)(bytes / 16), grid, (hipStream_t)stream));
}

gemm_status_t dequant_q4_f16(const void* q, void* out, int64_t rows, int64_t cols, int64_t ldo,
                             void* stream) {
    if (rows < 0 || cols < 0 || cols % 32 != 0 || ldo < cols) return GEMM_ERR_INVALID_VALUE;
    if (rows > kMaxDim || cols > kMaxDim || ldo > kMaxDim * 64) return GEMM_ERR_INVALID_VALUE;
    if (rows == 0 || cols == 0) return GEMM_OK;
    if (!q || !out || ((uintptr_t)q & 1) || ((uintptr_t)out & 1)) return GEMM_ERR_INVALID_VALUE;
    const Range rq = {(uintptr_t)q, (uintptr_t)q + (uintptr_t)(rows * (cols / 32) * 18)};
    if (overlaps(rq, span(out, rows, cols, ldo, 2))) return GEMM_ERR_INVALID_VALUE;
    gemm_status_t st = forced_failure();
    if (st != GEMM_OK) return st;
    DeviceInfo dev;
    if ((st = current_device(&dev)) != GEMM_OK) return st;
    const int vec_out = aligned16(out) && ldo % 8 == 0;
    return launch_status(
        launch_dequant_q4(q, out, rows, cols, ldo, vec_out, (hipStream_t)stream));
}

// Block width (weights) and size (bytes) of a gemm_qtype_t; false if unknown.
static bool qformat(int qtype, int64_t* width, int64_t* bytes) {
    switch (qtype) {
        case GEMM_Q4_0: *width = 32; *bytes = 18; return true;
        case GEMM_Q4_K: *width = 256; *bytes = 144; return true;
        case GEMM_Q6_K: *width = 256; *bytes = 210; return true;
        case GEMM_Q6_K_224: *width = 256; *bytes = 224; return true;
        default: return false;
    }
}

gemm_status_t dequant_f16(gemm_qtype_t qtype, const void* q, void* out, int64_t rows,
                          int64_t cols, int64_t ldo, void* stream) {
    int64_t w = 0, nb = 0;
    if (!qformat((int)qtype, &w, &nb)) return GEMM_ERR_INVALID_VALUE;
    if (qtype == GEMM_Q4_0) return dequant_q4_f16(q, out, rows, cols, ldo, stream);
    if (rows < 0 || cols < 0 || cols % w != 0 || ldo < cols) return GEMM_ERR_INVALID_VALUE;
    if (rows > kMaxDim || cols > kMaxDim || ldo > kMaxDim * 64) return GEMM_ERR_INVALID_VALUE;
    if (rows == 0 || cols == 0) return GEMM_OK;
    if (!q || !out || ((uintptr_t)out & 1)) return GEMM_ERR_INVALID_VALUE;
    const Range rq = {(uintptr_t)q, (uintptr_t)q + (uintptr_t)(rows * (cols / w) * nb)};
    if (overlaps(rq, span(out, rows, cols, ldo, 2))) return GEMM_ERR_INVALID_VALUE;
    gemm_status_t st = forced_failure();
    if (st != GEMM_OK) return st;
    DeviceInfo dev;
    if ((st = current_device(&dev)) != GEMM_OK) return st;
    const int vec_out = aligned16(out) && ldo % 8 == 0;
    const int kq = qtype == GEMM_Q6_K ? KQ_Q6_K : qtype == GEMM_Q6_K_224 ? KQ_Q6_K_224 : KQ_Q4_K;
    return launch_status(
        launch_dequant_kq(kq, q, out, rows, cols, ldo, vec_out, (hipStream_t)stream));
}

gemm_status_t prefill_f16(gemm_qtype_t qtype, int64_t M, int64_t N, int64_t K, const void* A,
                          int64_t lda, const void* q, void* w16, void* C, int64_t ldc,
                          gemm_out_t c_type, gemm_epilogue_t epi, const void* bias,
                          void* workspace, size_t workspace_bytes, void* stream) {
    int64_t w = 0, nb = 0;
    if (!qformat((int)qtype, &w, &nb)) return GEMM_ERR_INVALID_VALUE;
    if (M < 0 || N < 0 || K < 0 || K % w != 0) return GEMM_ERR_INVALID_VALUE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMM_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return GEMM_OK;
    if (K > 0 && (!q || !w16)) return GEMM_ERR_INVALID_VALUE;
    // validate the GEMM half before enqueueing the dequant
    Gemm g = make_gemm(IN_F16, M, N, K, 1.0f, A, lda, w16, std::max<int64_t>(K, 1), 1, 0.0f, C, ldc,
                       c_type, epi, bias, workspace, workspace_bytes, stream);
    gemm_status_t st = validate(g);
    if (st != GEMM_OK) return st;
    if (K > 0) {
        const Range rw = span(w16, N, K, K, 2);
        const Range rq = {(uintptr_t)q, (uintptr_t)q + (uintptr_t)(N * (K / w) * nb)};
        if (overlaps(rw, rq) || overlaps(rw, span(A, M, K, lda, 2)) ||
            overlaps(rw, span(C, M, N, ldc, out_bytes((int)c_type))))
            return GEMM_ERR_INVALID_VALUE;
        st = dequant_f16(qtype, q, w16, N, K, K, stream);
        if (st != GEMM_OK) return st;
    }
    return run_gemm(g, nullptr);
}

gemm_status_t prefill_q4_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                             const void* q, void* w16, void* C, int64_t ldc, gemm_out_t c_type,
                             gemm_epilogue_t epi, const void* bias, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return prefill_f16(GEMM_Q4_0, M, N, K, A, lda, q, w16, C, ldc, c_type, epi, bias, workspace,
                       workspace_bytes, stream);
}

gemm_status_t gemm_q4_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                          const void* q, void* C, int64_t ldc, gemm_out_t c_type,
                          gemm_epilogue_t epi, const void* bias, void* workspace,
                          size_t workspace_bytes, const gemm_tuning_t* tuning, void* stream) {
    gemm_tuning_t tn{GEMM_ALGO_AUTO, GEMM_TILE_AUTO, 0};
    if (tuning) tn = *tuning;
    if ((tn.algo != GEMM_ALGO_AUTO && tn.algo != GEMM_ALGO_MFMA_DIRECT) ||
        tn.tile < GEMM_TILE_AUTO || tn.tile > GEMM_TILE_256x128_W8 || tn.splits < 0)
        return GEMM_ERR_INVALID_VALUE;
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return GEMM_ERR_INVALID_VALUE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return GEMM_ERR_INVALID_VALUE;
    if (M == 0 || N == 0) return GEMM_OK;
    if (K > 0 && (!q || ((uintptr_t)q & 1) != 0)) return GEMM_ERR_INVALID_VALUE;
    Gemm g = make_gemm(IN_F16, M, N, K, 1.0f, A, lda, q, std::max<int64_t>(K, 1), 1, 0.0f, C, ldc,
                       c_type, epi, bias, workspace, workspace_bytes, stream);
    g.b_q4 = 1;
    gemm_status_t st = validate(g);
    if (st != GEMM_OK) return st;
    if ((st = forced_failure()) != GEMM_OK) return st;
    DeviceInfo dev;
    if ((st = current_device(&dev)) != GEMM_OK) return st;
    if (K > 0) {
        st = run_mfma(g, tn.tile, tn.splits, dev.cus, 1);
        if (st != GEMM_ERR_NOT_SUPPORTED) return st;
        if (tn.algo == GEMM_ALGO_MFMA_DIRECT) return st;  // the fused kernel was required
    }
    // Shapes the fused kernel does not take: expand the weights into the
    // workspace (N x K fp16) and run the two-pass path.
    const size_t need = (size_t)N * (size_t)K * 2;
    if (K > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
        return GEMM_ERR_WORKSPACE;
    g.b_q4 = 0;
    if (K > 0) {
        const Range rw = span(workspace, N, K, K, 2);
        const Range rq = {(uintptr_t)q, (uintptr_t)q + (uintptr_t)(N * (K / 32) * 18)};
        if (overlaps(rw, rq) || overlaps(rw, span(A, M, K, lda, 2)) ||
            overlaps(rw, span(C, M, N, ldc, out_bytes((int)c_type))))
            return GEMM_ERR_INVALID_VALUE;
        st = dequant_q4_f16(q, workspace, N, K, K, stream);
        if (st != GEMM_OK) return st;
        g.B = workspace;
        g.ldb = K;
    }
    g.ws = nullptr;
    g.ws_bytes = 0;
    gemm_tuning_t two_pass{GEMM_ALGO_AUTO, tn.tile, tn.splits > 1 ? 1 : 0};
    return run_gemm(g, &two_pass);
}

size_t gemm_workspace_size(int64_t M, int64_t N, int64_t K, int dtype) {
    if (M <= 0 || N <= 0 || K <= 0 || dtype < IN_F16 || dtype > IN_F32) return 0;
    DeviceInfo dev{1, 256, nullptr};
    if (current_device(&dev) != GEMM_OK) dev.cus = 256;
    // decode shapes (the split decode schedule, used with an N x K weight)
    if (dtype != IN_F32 && M <= 64) {
        const int ks = decode_ksplit(M, N, K, dev.cus);
        if (ks > 1) return decode_ws_bytes(M, N, ks);
    }
    if (dtype != IN_F32) {
        ColumnSplit cs;
        if (choose_column_split(M, N, K, dtype, dev.cus, (size_t)-1, ~0u,
                                [](int64_t) { return ~0u; }, &cs))
            return ws_bytes_for(M, N - cs.n1, cs.splits2);
    }
    int tile = GEMM_TILE_AUTO, s = 0;
    choose_schedule(M, N, K, dtype, dev.cus, (size_t)-1, &tile, &s);
    return ws_bytes_for(M, N, s);
}

size_t gemm_workspace_size_streamk(int64_t M, int64_t N, int64_t K, int tile) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    if (tile != GEMM_TILE_AUTO && (tile < TILE_256x256 || tile > TILE_LAST)) return 0;
    DeviceInfo dev{1, 256, nullptr};
    if (current_device(&dev) != GEMM_OK) dev.cus = 256;
    size_t need = 0;
    for (int t = TILE_256x256; t <= TILE_LAST; ++t) {
        if (tile != GEMM_TILE_AUTO && t != tile) continue;
        const TileShape ts = tile_shape(t);
        const int64_t tiles = (int64_t)ceil_div(M, ts.bm) * ceil_div(N, ts.bn);
        need = std::max(need, sk_ws_bytes(t, sk_grid(t, tiles * ceil_div(K, 64), dev.cus), tiles));
    }
    return need;
}

size_t gemm_workspace_size_splits(int64_t M, int64_t N, int splits) {
    if (M <= 0 || N <= 0 || splits <= 1) return 0;
    return ws_bytes_for(M, N, splits);
}

const char* gemm_status_string(gemm_status_t s) {
    switch (s) {
        case GEMM_OK: return "GEMM_OK";
        case GEMM_ERR_INVALID_VALUE: return "GEMM_ERR_INVALID_VALUE: invalid argument";
        case GEMM_ERR_NOT_SUPPORTED: return "GEMM_ERR_NOT_SUPPORTED: request not supported";
        case GEMM_ERR_WORKSPACE: return "GEMM_ERR_WORKSPACE: workspace too small for the split";
        case GEMM_ERR_LAUNCH: return "GEMM_ERR_LAUNCH: kernel launch failed";
        case GEMM_ERR_DEVICE: return "GEMM_ERR_DEVICE: no usable gfx950 device";
        case GEMM_ERR_SCRATCH:
            return "GEMM_ERR_SCRATCH: the request needs more than the 32 MiB static scratch";
        default: return "unknown gemm_status_t";
    }
}

gemm_status_t gemm_init(void) {
    DeviceInfo dev;
    return current_device(&dev);
}

}  // extern "C"
