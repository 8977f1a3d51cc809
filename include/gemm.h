/*
 * gemm.h — C ABI of the MI355X (gfx950) dense-GEMM library.
 *
 * Operations
 *   gemm_f16 / gemm_bf16 / gemm_f32:
 *       C = epi(alpha * A * B + beta * C)
 *     The dense product C_ij = sum_k A_ik B_kj, 2MNK FLOPs ("Matrix
 *     Multiplication: The Operation Behind Modern AI", section "The operation
 *     everything is made of"), accumulated in fp32 on the matrix cores
 *     ("Optimizing GEMMs using tcgen05 - Part 2": fp16 in, fp32 accumulate).
 *     epi adds one value per output column and optionally applies the tanh
 *     form of GELU, 0.5 t (1 + tanh(sqrt(2/pi) (t + 0.044715 t^3))).
 *   dequant_q4_f16:
 *     expands 4-bit weight blocks into binary16 ("02 · 8m/8m② — Tiled wmma
 *     f16 prefill GEMM", §2.3 and the q4_0 dequant kernel in §3.2).
 *   prefill_q4_f16:
 *     the prefill projection of the same page: dequantise an N x K q4 weight
 *     into a caller-supplied binary16 scratch, then C = A * W^T on the same
 *     stream (§1 route 2, §3.2 host routing).
 *   gemm_q4_f16:
 *     the same projection with the dequantisation fused into the GEMM's
 *     B-tile producer, so the binary16 weight is never written to memory:
 *     the dequant-in-GEMM successor that §2.3 of the same page names for
 *     the three-pass cost of the dequant-then-GEMM route.
 *   dequant_f16 / prefill_f16:
 *     the same two entry points for any of the page's block formats: q4_0
 *     and the 256-weight super-block formats q4_K and q6_K, one dequant
 *     kernel per format in front of the same GEMM (same page, §2.3 and §3.1
 *     name the formats and the per-format kernel; §3.2 prints the q6_K one).
 *
 * Conventions (all entry points)
 *   - Row-major throughout; leading dimensions are in elements.
 *       A: M x K, lda >= K.
 *       B: K x N with ldb >= N (trans_b = 0), or N x K with ldb >= K
 *          (trans_b = 1, the weight layout of the prefill page).
 *       C: M x N, ldc >= N.
 *   - Every pointer argument is a DEVICE pointer owned by the caller; the
 *     library never allocates, frees or retains memory, and never
 *     synchronises the host.  `stream` is a hipStream_t passed as void*
 *     (NULL = the default stream); all work is enqueued on it.
 *   - Arguments are validated on the host before any device call; a
 *     rejected call enqueues nothing and returns a non-zero status.  No entry
 *     point calls exit() or prints.
 *   - M == 0 or N == 0 is a successful no-op.  K == 0 gives
 *     C = epi(beta * C) (the product of empty sums is zero).
 *   - beta == 0: C is write-only (its old contents, NaN included, are never
 *     read).
 *   - epi != GEMM_EPI_NONE requires bias != NULL: N values of the input type
 *     (fp16 for gemm_f16, bf16 for gemm_bf16, fp32 for gemm_f32).
 *   - C must not overlap A, B or bias (GEMM_ERR_INVALID_VALUE).
 *   - Output rounding: one round-to-nearest-even from fp32 to c_type;
 *     overflow gives +-inf; subnormals are kept.
 *   - Unaligned pointers or leading dimensions that are not a multiple of
 *     16 bytes take a slower element-wise load path; they are not errors.
 *   - workspace: caller-owned device scratch for split-K and stream-K
 *     partial sums (and the stream-K arrival counters, which each call
 *     clears itself).  If it is NULL or smaller than gemm_workspace_size(),
 *     the call runs a schedule that fits (at worst without splitting K; it
 *     does not fail).  Calls that share a workspace must not overlap.
 *   - Split-K and stream-K partial sums are reduced in fixed order (K slice
 *     0, 1, ...), so results are bitwise reproducible run to run.
 *   - Thread safety: calls may be issued concurrently from several host
 *     threads (distinct streams or not); the only shared state is a
 *     once-initialised device-property cache.
 *
 * Fault injection (tests): the environment variable GEMM_TEST_FAIL makes
 * every entry point return a chosen error after validation and before any
 * launch: "launch" -> GEMM_ERR_LAUNCH, "device" -> GEMM_ERR_DEVICE,
 * "workspace" -> GEMM_ERR_WORKSPACE.  Nothing is enqueued in that case.
 */
#ifndef DGE_GEMM_H
#define DGE_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_VALUE = 1, /* bad size, leading dimension, pointer, enum or overlap */
    GEMM_ERR_NOT_SUPPORTED = 2, /* valid request the library does not implement */
    GEMM_ERR_WORKSPACE = 3,     /* explicit split request without enough workspace */
    GEMM_ERR_LAUNCH = 4,        /* the HIP runtime rejected a launch */
    GEMM_ERR_DEVICE = 5,        /* no usable gfx950 device is current */
    GEMM_ERR_SCRATCH = 6        /* gemm_ex_noalloc: the request needs more scratch than
                                   GEMM_NOALLOC_SCRATCH_BYTES */
} gemm_status_t;

/* Size of the static per-device scratch of gemm_ex_noalloc (32 MiB). */
#define GEMM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

typedef enum { GEMM_EPI_NONE = 0, GEMM_EPI_BIAS = 1, GEMM_EPI_BIAS_GELU = 2 } gemm_epilogue_t;

typedef enum { GEMM_OUT_F32 = 0, GEMM_OUT_F16 = 1, GEMM_OUT_BF16 = 2 } gemm_out_t;

typedef enum { GEMM_IN_F16 = 0, GEMM_IN_BF16 = 1, GEMM_IN_F32 = 2 } gemm_in_t;

/* Block-quantised weight formats of dequant_f16 / prefill_f16 (layouts at
 * dequant_f16). */
typedef enum {
    GEMM_Q4_0 = 0, /* 32 weights in 18 bytes */
    GEMM_Q4_K = 1, /* 256 weights in 144 bytes */
    GEMM_Q6_K = 2, /* 256 weights in 210 bytes */
    GEMM_Q6_K_224 = 3 /* GEMM_Q6_K blocks padded to a 224-byte stride */
} gemm_qtype_t;

/* Kernel families, for gemm_ex's explicit selection. */
typedef enum {
    GEMM_ALGO_AUTO = 0,      /* library's choice by shape */
    GEMM_ALGO_NAIVE = 1,     /* one thread per output element, no reuse (the floor) */
    GEMM_ALGO_LDS_TILED = 2, /* LDS tiles + register-blocked fp32 FMA, no matrix cores */
    GEMM_ALGO_MFMA = 3,      /* LDS-staged macro tiles on the matrix cores, operands
                                staged through registers (any shape and alignment) */
    GEMM_ALGO_MFMA_DIRECT = 4, /* macro tiles fed by direct global->LDS loads (fp16/bf16,
                                  full tiles, 16-byte aligned operands); other problems
                                  run as GEMM_ALGO_MFMA.  AUTO uses it when eligible. */
    GEMM_ALGO_SKINNY = 5,     /* tall-skinny kernel: W resident in LDS, X streamed into
                                 the MFMA operands (fp16/bf16, K a multiple of 32 up to
                                 256, N <= 256, A 16-byte aligned with lda % 8 == 0);
                                 other problems run as GEMM_ALGO_MFMA_DIRECT.  AUTO uses
                                 it for M >= 4096 and M >= 8N when eligible. */
    GEMM_ALGO_DECODE = 6,     /* decode shape: 1 <= M <= 64 input rows against an N x K
                                 weight (trans_b = 1, fp16/bf16, K % 8 == 0, A and B
                                 16-byte aligned with lda, ldb % 8 == 0), W streamed
                                 from memory straight into the MFMA operands, K split
                                 over 8 waves and summed in a fixed order; other
                                 problems run as GEMM_ALGO_MFMA_DIRECT.  AUTO uses it
                                 whenever eligible ("Matrix Multiplication: The
                                 Operation Behind Modern AI", "The shape a language
                                 model actually runs").  For 17 <= M <= 64 with
                                 N % 64 == 0 and K % 32 == 0 it also splits K over
                                 workgroups (64 weight rows each, X read once per
                                 workgroup) when the workspace holds the fp32
                                 partials (gemm_workspace_size gives the bytes); the
                                 split-K fixup sums them in slice order. */
    GEMM_ALGO_STREAMK = 7     /* persistent stream-K schedule of the direct-to-LDS
                                 kernels ("Optimizing GEMMs using tcgen05 - Part 2",
                                 §8: stream-K for the tail and a persistent kernel
                                 whose next tile's loads overlap this tile's
                                 epilogue): one workgroup per CU slot, each taking an
                                 equal contiguous share of the (tile, K stage)
                                 iterations; partial tiles are summed in K order by
                                 the segment that completes them.  Needs fp16/bf16,
                                 full tiles, K % 64 == 0, aligned operands and
                                 gemm_workspace_size_streamk() bytes of 16-byte
                                 aligned workspace (GEMM_ERR_WORKSPACE with less);
                                 other problems, and the 128 x 64 tile with a K x N
                                 B, run as GEMM_ALGO_MFMA_DIRECT.  AUTO
                                 does not choose it: on MI355X it measured no faster
                                 than the data-parallel and split-K schedules on
                                 the square and prefill shapes (an XCD's workgroups
                                 at different K stages share less of its L2, and
                                 split tiles move fp32 partials through memory). */
} gemm_algo_t;

/* Tile configurations of the MFMA family (macro tile BM x BN, waves). */
typedef enum {
    GEMM_TILE_AUTO = 0,
    GEMM_TILE_256x256 = 1, /* 4 waves, 128 x 128 per wave */
    GEMM_TILE_256x128 = 2, /* 4 waves, 128 x 64 per wave */
    GEMM_TILE_128x128 = 3, /* 4 waves, 64 x 64 per wave */
    GEMM_TILE_128x64 = 4,  /* 4 waves, 64 x 32 per wave */
    GEMM_TILE_256x256_W8 = 5, /* 8 waves (two per SIMD), 128 x 64 per wave */
    GEMM_TILE_256x128_W8 = 6  /* 8 waves (4 x 2), 64 x 64 per wave; the register-staged
                                 family runs it as GEMM_TILE_256x128 */
} gemm_tile_t;

typedef struct {
    int algo;   /* gemm_algo_t */
    int tile;   /* gemm_tile_t; MFMA family only */
    int splits; /* 0 = auto, 1 = never split, s > 1 = split K into s slices
                   (needs gemm_workspace_size_splits(M, N, s) bytes) */
} gemm_tuning_t;

/* fp16 A/B/bias, fp32 accumulate, c_type output. */
gemm_status_t gemm_f16(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                       const void* B, int64_t ldb, int trans_b, float beta, void* C, int64_t ldc,
                       gemm_out_t c_type, gemm_epilogue_t epi, const void* bias, void* workspace,
                       size_t workspace_bytes, void* stream);

/* bf16 A/B/bias, fp32 accumulate, c_type output. */
gemm_status_t gemm_bf16(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                        const void* B, int64_t ldb, int trans_b, float beta, void* C, int64_t ldc,
                        gemm_out_t c_type, gemm_epilogue_t epi, const void* bias, void* workspace,
                        size_t workspace_bytes, void* stream);

/* fp32 A/B/bias, fp32 accumulate (fp32 matrix-core path by default);
 * c_type must be GEMM_OUT_F32. */
gemm_status_t gemm_f32(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                       const void* B, int64_t ldb, int trans_b, float beta, void* C, int64_t ldc,
                       gemm_out_t c_type, gemm_epilogue_t epi, const void* bias, void* workspace,
                       size_t workspace_bytes, void* stream);

/* The same operation with the input type and the kernel family, tile and
 * split chosen explicitly (tuning may be NULL = all automatic).  Used by the
 * fp32 ladder (naive -> LDS-tiled -> MFMA) and by tile and split sweeps.  A
 * split request (splits > 1) with too little workspace returns
 * GEMM_ERR_WORKSPACE; the naive and LDS-tiled families never split. */
gemm_status_t gemm_ex(gemm_in_t in_type, int64_t M, int64_t N, int64_t K, float alpha,
                      const void* A, int64_t lda, const void* B, int64_t ldb, int trans_b,
                      float beta, void* C, int64_t ldc, gemm_out_t c_type, gemm_epilogue_t epi,
                      const void* bias, void* workspace, size_t workspace_bytes,
                      const gemm_tuning_t* tuning, void* stream);

/* gemm_ex without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The split-K partial sums and the
 * stream-K partial tiles and arrival counters go to a static scratch array
 * of GEMM_NOALLOC_SCRATCH_BYTES that the library holds on each device from
 * its load until the process ends; the call itself allocates nothing.  The
 * schedule is the one gemm_ex picks with a workspace of that size; a request
 * that needs more (an explicit split whose partials exceed it, or stream-K
 * on a grid whose partial tiles exceed it) returns GEMM_ERR_SCRATCH and
 * enqueues nothing.  The caller still passes A, B, C and bias, with the
 * conventions above.  Every call on one device shares that device's
 * scratch: calls that overlap in time on one device (concurrent streams, or
 * host threads on different streams) race and give undefined results; calls
 * ordered on one stream are safe (each clears the counters it needs and
 * writes every partial it reads). */
gemm_status_t gemm_ex_noalloc(gemm_in_t in_type, int64_t M, int64_t N, int64_t K, float alpha,
                              const void* A, int64_t lda, const void* B, int64_t ldb,
                              int trans_b, float beta, void* C, int64_t ldc, gemm_out_t c_type,
                              gemm_epilogue_t epi, const void* bias, const gemm_tuning_t* tuning,
                              void* stream);

/* q4 -> binary16.  q holds rows * (cols/32) blocks of 18 bytes, row-major
 * (block (r, b) at byte 18 * (r * cols/32 + b)): a little-endian binary16
 * scale d, then 16 bytes whose low nibble is element i and high nibble
 * element i + 16 of the block.  out[r * ldo + 32 b + e] = RNE16(d * (code - 8)).
 * Requires cols % 32 == 0, ldo >= cols, q 2-byte aligned and out 2-byte
 * aligned (GEMM_ERR_INVALID_VALUE otherwise).  The result is bit-exact
 * (the product is exact in fp32). */
gemm_status_t dequant_q4_f16(const void* q, void* out, int64_t rows, int64_t cols, int64_t ldo,
                             void* stream);

/* Prefill projection: w16 (caller scratch, N x K binary16, >= 2*N*K bytes)
 * = dequant(q); then C = epi(A * w16^T), A M x K fp16 (lda), C M x N (ldc,
 * c_type), alpha = 1, beta = 0.  K % 32 == 0 is required.  Both steps are
 * enqueued on `stream`; w16 holds the dequantised weight afterwards. */
gemm_status_t prefill_q4_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                             const void* q, void* w16, void* C, int64_t ldc, gemm_out_t c_type,
                             gemm_epilogue_t epi, const void* bias, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Fused prefill projection: C = epi(A * dequant(q)^T), A M x K fp16 (lda),
 * q the N x K weight as q4 blocks (layout of dequant_q4_f16, 2-byte aligned),
 * C M x N (ldc, c_type), alpha = 1, beta = 0, bias as for gemm_f16.  K % 32
 * == 0 is required (GEMM_ERR_INVALID_VALUE otherwise).  The weights are
 * decoded inside the GEMM kernel with one RNE rounding of d * (code - 8), the
 * same binary16 values dequant_q4_f16 writes, so the result equals
 * prefill_q4_f16's up to the GEMM's own summation order.  The fused kernel
 * takes shapes whose M and N are multiples of a 128 x 64 (or larger) tile,
 * K % 64 == 0, q 4-byte aligned, A, C 16-byte aligned with lda % 8 == 0
 * and lda, ldc below 2^24;
 * the workspace then only serves a K split (gemm_workspace_size with
 * GEMM_IN_F16 gives its size; less workspace = no split).  Any other shape
 * expands the weights into the workspace first, which must then hold
 * 2 * N * K bytes, 16-byte aligned (GEMM_ERR_WORKSPACE otherwise).
 * tuning (may be NULL): algo GEMM_ALGO_AUTO or GEMM_ALGO_MFMA_DIRECT (= the
 * fused kernel is required: GEMM_ERR_NOT_SUPPORTED for a shape it cannot
 * take), tile and splits as for gemm_ex; other algos are
 * GEMM_ERR_INVALID_VALUE. */
gemm_status_t gemm_q4_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                          const void* q, void* C, int64_t ldc, gemm_out_t c_type,
                          gemm_epilogue_t epi, const void* bias, void* workspace,
                          size_t workspace_bytes, const gemm_tuning_t* tuning, void* stream);

/* Block-quantised weight -> binary16, for every gemm_qtype_t.  q holds the
 * rows x cols weight as consecutive blocks, row-major (block b of row r is
 * block number r * (cols / W) + b, W weights per block), with no padding;
 * out[r * ldo + c] receives weight (r, c).  Multi-byte fields are
 * little-endian; "binary16" fields are IEEE half precision.
 *   GEMM_Q4_0 (W = 32, 18 bytes): as dequant_q4_f16.
 *   GEMM_Q6_K (W = 256, 210 bytes): ql[128] at 0, qh[64] at 128, 16 int8
 *     scales sc at 192, binary16 d at 208.  Weight e = 128 h + 32 t + l
 *     (h < 2, t < 4, l < 32) has the 6-bit code q whose low 4 bits are the
 *     low (t < 2) or high (t >= 2) nibble of ql[64 h + 32 (t & 1) + l] and
 *     whose high 2 bits are bits 2t, 2t + 1 of qh[32 h + l]; its value is
 *     RNE16(d * sc[8 h + 2 t + l / 16] * (q - 32)), computed exactly (a
 *     zero product keeps the IEEE sign: -0 when d * sc < 0).
 *   GEMM_Q6_K_224 (W = 256, 224 bytes): a GEMM_Q6_K block followed by 14
 *     bytes that are not read (the padded layout the page's q6_K kernel
 *     takes through its block stride, §3.2).
 *   GEMM_Q4_K (W = 256, 144 bytes): binary16 d at 0, binary16 dmin at 2,
 *     12 bytes of packed 6-bit scales at 4, 128 code bytes qs at 16.  The
 *     256 weights form 8 sub-blocks of 32 with a 6-bit scale s_j and min
 *     m_j: for j < 4, s_j = byte[j] & 63 and m_j = byte[j + 4] & 63; for
 *     j >= 4, s_j = (byte[j + 4] & 15) | (byte[j - 4] >> 6) << 4 and m_j =
 *     (byte[j + 4] >> 4) | (byte[j] >> 6) << 4 (byte[] = the 12 bytes).
 *     Weight e = 64 p + w (p < 4, w < 64) is in sub-block j = 2p + (w >= 32)
 *     and has the code q = low (w < 32) or high nibble of qs[32 p + w % 32];
 *     its value is RNE16(RNE32(d s_j q - dmin m_j)) (both products exact in
 *     binary32, the difference rounded once to binary32, then to binary16).
 * Requires cols % W == 0, ldo >= cols, out 2-byte aligned, q 2-byte aligned
 * for GEMM_Q4_0 (any alignment for the K formats), q and out disjoint, and a
 * known qtype; GEMM_ERR_INVALID_VALUE otherwise.  The results are
 * bit-exact.  rows == 0 or cols == 0 is a successful no-op. */
gemm_status_t dequant_f16(gemm_qtype_t qtype, const void* q, void* out, int64_t rows,
                          int64_t cols, int64_t ldo, void* stream);

/* Prefill projection for every gemm_qtype_t: w16 (caller scratch, N x K
 * binary16, >= 2*N*K bytes) = dequant_f16(qtype, q); then C = epi(A *
 * w16^T), A M x K fp16 (lda), C M x N (ldc, c_type), alpha = 1, beta = 0,
 * bias as for gemm_f16.  K must be a multiple of the format's block width
 * (32 for GEMM_Q4_0, 256 for the K formats).  Both steps are enqueued on
 * `stream`; w16 holds the dequantised weight afterwards. */
gemm_status_t prefill_f16(gemm_qtype_t qtype, int64_t M, int64_t N, int64_t K, const void* A,
                          int64_t lda, const void* q, void* w16, void* C, int64_t ldc,
                          gemm_out_t c_type, gemm_epilogue_t epi, const void* bias,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes the automatic schedule of this shape would use (0 if it
 * would not split K).  dtype is a gemm_in_t. */
size_t gemm_workspace_size(int64_t M, int64_t N, int64_t K, int dtype);

/* Workspace bytes an explicit split into `splits` slices needs. */
size_t gemm_workspace_size_splits(int64_t M, int64_t N, int splits);

/* Workspace bytes the stream-K schedule (GEMM_ALGO_STREAMK) needs for this
 * shape and tile (a gemm_tile_t; GEMM_TILE_AUTO = the largest over tiles) on
 * the current device: two fp32 partial tiles per workgroup of the persistent
 * grid, then one 32-bit arrival counter per tile.  0 for an empty problem. */
size_t gemm_workspace_size_streamk(int64_t M, int64_t N, int64_t K, int tile);

/* Static, NUL-terminated description of a status code. */
const char* gemm_status_string(gemm_status_t s);

/* Checks that the current device is a gfx950 and caches its properties.
 * Called implicitly by every compute entry point; may be called first to
 * pay the one-time cost outside a timed region. */
gemm_status_t gemm_init(void);

#ifdef __cplusplus
}
#endif

#endif /* DGE_GEMM_H */
