/*
 * gemm_probe.h — measurement probes of the MI355X (gfx950) dense-GEMM
 * library.  They are not part of the GEMM path: they measure the ceilings
 * that path is judged against on the device itself, and the engine clock
 * it runs at, so that a fraction of the data-sheet peak can be split into
 * clock and issue ("Matrix Multiplication: The Operation Behind Modern AI",
 * the measured roofs of "The Tesla T4, measured" and the power-limited
 * clock of "What the precision buys").
 *
 * Conventions as in gemm.h: device pointers owned by the caller, work
 * enqueued on `stream` (a hipStream_t as void*, NULL = default stream), no
 * allocation, no host synchronisation, arguments checked on the host
 * (GEMM_ERR_INVALID_VALUE) before anything is enqueued.
 *
 * Clock records (gemm_probe_clock, gemm_probe_mfma): 4 unsigned 64-bit
 * values per workgroup at clk[4 w .. 4 w + 3]: the shader-clock counter and
 * the 100 MHz real-time counter when workgroup w starts, then both again
 * when it has issued its last store.  clk must be 16-byte aligned.
 */
#ifndef DGE_GEMM_PROBE_H
#define DGE_GEMM_PROBE_H

#include "gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups of gemm_probe_mfma. */
#define GEMM_PROBE_MFMA_GRID 256

/* The GEMM of gemm_ex (automatic schedule, no workspace) with per-workgroup
 * clock records.  Only schedules that are one data-parallel launch of a
 * direct-to-LDS kernel can be recorded (the 4096^3 product is one);
 * others return GEMM_ERR_NOT_SUPPORTED and enqueue nothing, as does a grid
 * larger than clk_entries workgroups.  C receives the same result as
 * gemm_ex. */
gemm_status_t gemm_probe_clock(gemm_in_t in_type, int64_t M, int64_t N, int64_t K, float alpha,
                               const void* A, int64_t lda, const void* B, int64_t ldb,
                               int trans_b, float beta, void* C, int64_t ldc, gemm_out_t c_type,
                               gemm_epilogue_t epi, const void* bias, unsigned long long* clk,
                               int64_t clk_entries, void* stream);

/* Phase records of the schedules whose time is not in their MFMA work:
 * C = A B (trans_b = 0) or A B^T (trans_b = 1) with the epilogue `epi`
 * (alpha = 1, beta = 0), run as gemm_ex runs it with this workspace, plus 4
 * unsigned 64-bit values of the 100 MHz real-time counter per workgroup at
 * rec[4 w .. 4 w + 3].  Supported schedules and their records:
 *   - split decode (M <= 64 rows against an N x K weight, a workspace of
 *     gemm_workspace_size bytes; the records cover its first kernel, not
 *     the fixup): start, the first 128-deep span's loads landed in wave 0,
 *     loads and MFMAs of all 8 waves done, partial issued;
 *   - tall-skinny (M >= 4096, M >= 8 N, N and K <= 256): start, W staged in
 *     LDS, wave 0's first rows of A landed, wave 0's last stores issued.
 * Other schedules return GEMM_ERR_NOT_SUPPORTED and enqueue nothing, as does
 * a grid of more than rec_entries workgroups.  The waits that take the
 * "landed" records delay wave 0 slightly.  rec must be 16-byte aligned; C
 * receives the same result as gemm_ex. */
gemm_status_t gemm_probe_phases(gemm_in_t in_type, int64_t M, int64_t N, int64_t K,
                                const void* A, int64_t lda, const void* B, int64_t ldb,
                                int trans_b, void* C, int64_t ldc, gemm_out_t c_type,
                                gemm_epilogue_t epi, const void* bias, void* workspace,
                                size_t workspace_bytes, unsigned long long* rec,
                                int64_t rec_entries, void* stream);

/* Matrix work of the 8-wave 256 x 256 GEMM tile without its loads, LDS
 * traffic or stores: GEMM_PROBE_MFMA_GRID workgroups; each of their 8 waves
 * reads two 32-deep k-blocks of fp16 (in_type GEMM_IN_F16) or bf16
 * (GEMM_IN_BF16) operand fragments from the rows of its 128 x 64 part of a
 * 4096 x 4096 output (A: rows of A; B: rows of B, read as the N x K layout)
 * and issues k_blocks x 32 v_mfma 16x16x32 in the GEMM's order.
 * k_blocks = 128 is the 2 x 4096^3 FLOPs of the 4096^3 product.  A and B
 * need rows >= 4096 rows of cols >= 64 elements, leading dimensions lda,
 * ldb >= cols and a multiple of 8, 16-byte alignment.  out receives
 * GEMM_PROBE_MFMA_GRID x 512 floats (per-lane sums, so nothing is
 * discarded); clk may be NULL or hold 4 x GEMM_PROBE_MFMA_GRID records. */
gemm_status_t gemm_probe_mfma(gemm_in_t in_type, const void* A, int64_t lda, const void* B,
                              int64_t ldb, int64_t rows, int64_t cols, int k_blocks, float* out,
                              unsigned long long* clk, void* stream);

/* Streaming read of `bytes` (a multiple of 16, src 16-byte aligned) with
 * 16-byte non-temporal loads, eight in flight per thread, on `grid`
 * (1..65536) workgroups of 256 threads; out receives grid x 256 32-bit
 * digests (their XOR is the XOR of every 32-bit word read). */
gemm_status_t gemm_probe_read(const void* src, size_t bytes, int grid, unsigned* out,
                              void* stream);

/* Streaming copy of `bytes` (a multiple of 16) from src to dst (16-byte
 * aligned, disjoint) with 16-byte non-temporal loads and stores, four in
 * flight per thread, on `grid` (1..65536) workgroups of 256 threads. */
gemm_status_t gemm_probe_copy(const void* src, void* dst, size_t bytes, int grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DGE_GEMM_PROBE_H */
