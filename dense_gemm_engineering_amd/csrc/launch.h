// Host-side launchers for the gfx950 kernels (C++ linkage; the C ABI in
// api.cpp validates arguments and calls these).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "ladder.h"
#include "mfma_gemm.h"
#include "skinny.h"
#include "decode.h"

namespace dge {

// Tile configurations (values match gemm_tile_t).
enum : int { TILE_256x256 = 1, TILE_256x128 = 2, TILE_128x128 = 3, TILE_128x64 = 4,
              TILE_256x256_W8 = 5, TILE_256x128_W8 = 6, TILE_LAST = 6 };

struct TileShape {
    int bm, bn;
};
inline TileShape tile_shape(int tile) {
    switch (tile) {
        case TILE_256x256: return {256, 256};
        case TILE_256x128: return {256, 128};
        case TILE_128x128: return {128, 128};
        case TILE_256x256_W8: return {256, 256};
        case TILE_256x128_W8: return {256, 128};
        default: return {128, 64};
    }
}

// Stage depth in elements: 128 bytes of K.
inline int stage_k(int dt) { return dt == IN_F32 ? 32 : 64; }

// Per-dtype MFMA launchers (one translation unit each).  `fast` selects the
// unchecked load path (every tile full, K a multiple of the stage depth,
// everything 16-byte aligned).
hipError_t launch_mfma_f16(int tile, int trans_b, int fast, const MfmaArgs& a, int nwg,
                           hipStream_t s);
hipError_t launch_mfma_bf16(int tile, int trans_b, int fast, const MfmaArgs& a, int nwg,
                            hipStream_t s);
hipError_t launch_mfma_f32(int tile, int trans_b, int fast, const MfmaArgs& a, int nwg,
                           hipStream_t s);

// Direct-to-LDS variant (16-bit inputs, full tiles, 16-byte aligned operands).
// Returns hipErrorInvalidValue for a tile it does not provide.
// sk = 1: the persistent stream-K schedule, nwg = its grid (a.sk_* set, the
// arrival counters zeroed on the same stream first).
// One entry per input type and B layout (nn: K x N, nt: N x K), each built in
// a translation unit of its own.
hipError_t launch_mfma_direct_f16_nn(int tile, const MfmaArgs& a, int nwg, int sk, hipStream_t s);
hipError_t launch_mfma_direct_f16_nt(int tile, const MfmaArgs& a, int nwg, int sk, hipStream_t s);
hipError_t launch_mfma_direct_bf16_nn(int tile, const MfmaArgs& a, int nwg, int sk, hipStream_t s);
hipError_t launch_mfma_direct_bf16_nt(int tile, const MfmaArgs& a, int nwg, int sk, hipStream_t s);
inline hipError_t launch_mfma_direct_f16(int tile, int trans_b, const MfmaArgs& a, int nwg, int sk,
                                         hipStream_t s) {
    return trans_b ? launch_mfma_direct_f16_nt(tile, a, nwg, sk, s)
                   : launch_mfma_direct_f16_nn(tile, a, nwg, sk, s);
}
inline hipError_t launch_mfma_direct_bf16(int tile, int trans_b, const MfmaArgs& a, int nwg, int sk,
                                          hipStream_t s) {
    return trans_b ? launch_mfma_direct_bf16_nt(tile, a, nwg, sk, s)
                   : launch_mfma_direct_bf16_nn(tile, a, nwg, sk, s);
}
// Fused q4-weight GEMM (p.B = q4 blocks of an N x K weight, 4-byte aligned;
// K % 64 == 0; full tiles of the given shape only).
hipError_t launch_mfma_q4_f16(int tile, const MfmaArgs& a, int nwg, hipStream_t s);

// Tall-skinny kernel: nt = 16-column tiles of N (even, 2..16), waves per
// workgroup (1..16), lds = dynamic LDS bytes (skinny_lds_bytes).
hipError_t launch_skinny(int dt, int nt, int trans_b, const SkinnyArgs& a, int grid, int waves,
                         size_t lds, hipStream_t s);
// The instances for alpha = 1, beta = 0 and fp16 output, which
// launch_skinny picks for such arguments (kernels_skinny_fold.hip).
hipError_t launch_skinny_fold(int dt, int nt, int trans_b, const SkinnyArgs& a, int grid,
                              int waves, size_t lds, hipStream_t s);
// Allows every skinny instance up to 160 KB of dynamic LDS.  Called once per
// device at library initialisation, never from inside a launch sequence.
hipError_t skinny_init();
hipError_t skinny_fold_init();
// Decode-shaped kernel: 1 <= M <= 64, N x K 16-bit weight, one workgroup per
// 16 weight rows.
hipError_t launch_decode(int dt, const DecodeArgs& a, hipStream_t s);
// Split schedule: 17 <= M <= 64, N % 64 == 0, K % 32 == 0, every wave of a
// slice with at least one k-block; a.ws receives a.ksplit x M x N fp32
// partials (the split-K fixup finishes C).
hipError_t launch_decode_split(int dt, const DecodeArgs& a, hipStream_t s);

hipError_t launch_naive(int dt, const SimpleArgs& a, hipStream_t s);
hipError_t launch_lds_tiled(int dt, const SimpleArgs& a, hipStream_t s);
// n 32-bit zeros at p (a fill kernel: no memset node if the stream is captured).
hipError_t launch_clear_u32(unsigned* p, int64_t n, hipStream_t s);
hipError_t launch_splitk_fixup(int dt, const SimpleArgs& a, const float* ws, int splits,
                               hipStream_t s);
hipError_t launch_dequant_q4(const void* q, void* out, int64_t rows, int64_t cols, int64_t ldo,
                             int vec_out, hipStream_t s);
// K-quant super-blocks (qtype KQ_Q4_K, KQ_Q6_K or KQ_Q6_K_224), cols % 256 == 0.
hipError_t launch_dequant_kq(int qtype, const void* q, void* out, int64_t rows, int64_t cols,
                             int64_t ldo, int vec_out, hipStream_t s);

// Measurement probes (kernels_probe.hip).  The MFMA probe runs
// PROBE_MFMA_GRID workgroups of 8 waves over the 4096 x 4096 output of the
// headline product (A and B need 4096 rows of at least 64 elements, 16-byte
// aligned, leading dimensions a multiple of 8); out receives
// PROBE_MFMA_GRID x 512 floats, clk (if set) 4 values per workgroup.  The
// streaming probes take 16-byte chunks on `grid` workgroups of 256 threads;
// out receives grid x 256 digests.
constexpr int PROBE_MFMA_GRID = 256;
hipError_t launch_probe_mfma(int dt, const void* A, const void* B, int64_t lda, int64_t ldb,
                             int k_blocks, float* out, unsigned long long* clk, hipStream_t s);
hipError_t launch_probe_read(const void* src, int64_t n16, unsigned* out, int grid,
                             hipStream_t s);
hipError_t launch_probe_copy(const void* src, void* dst, int64_t n16, int grid, hipStream_t s);

}  // namespace dge
