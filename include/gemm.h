/*
 * libgemm -- dense row-major GEMM on AMD Instinct MI355X (gfx950).
 *
 * Operation (every compute entry point):
 *     C[i][j] = sum_{k=0}^{K-1} A[i][k] * B[k][j],   0 <= i < M, 0 <= j < N
 * i.e. C[M x N] = A[M x K] x B[K x N] in row-major storage, 2*M*N*K flops.
 * This is the problem statement of "GEMM: from naive to shared memory tiling
 * and register blocking" (quant67.com, introduction) and of the naive kernel
 * in "sgemm - beyond cuBLAS" (wingedge777.com, section 1); the FP16 variant
 * is the HGEMM of "hgemm_naive_kernel explained" (yuyanqi.com, section 1.1),
 * here with FP32 accumulation instead of the page's FP16 accumulator.
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * Layout     Row-major.  Element (i, k) of A is A[i*lda + k], (k, j) of B is
 *            B[k*ldb + j], (i, j) of C is C[i*ldc + j].  Leading dimensions
 *            are counted in elements.
 * Memory     A, B and C are device pointers owned by the caller.  The library
 *            never allocates, frees or retains them.  C is overwritten (no
 *            alpha/beta); its columns [N, ldc) are never written.
 * Streams    `stream` is a hipStream_t passed as void* (NULL = the default
 *            stream).  Calls only enqueue work and return; the caller
 *            synchronises.  Concurrent calls on different streams are safe.
 * Degenerate M == 0 or N == 0: no work, GEMM_OK.  K == 0: C[0:M, 0:N] = 0
 *            (the empty sum).
 * Alignment  None required.  Operands whose pointers are 16-byte aligned and
 *            whose K, N and leading dimensions are multiples of 4 (FP32) or 8
 *            (FP16) take the 128-bit vector path; others a scalar path with
 *            the same results.
 * Rounding   FP32: products and sums in FP32 on the matrix cores; the order
 *            of the K-sum is the kernel's (results agree with the exact sum
 *            within |C - C_exact| <= 1e-5 * sum_k |A_ik||B_kj| for the
 *            supported sizes).  FP16: FP16 inputs, FP32 accumulation, one
 *            round-to-nearest-even conversion to FP16 per output.  BF16:
 *            the same with bfloat16 inputs and output (8 significant bits:
 *            |C - C_exact| <= 5e-3 * sum_k |A_ik||B_kj|).
 * Errors     No exception or abort crosses this interface.  Argument errors
 *            are detected on the host before any GPU work is enqueued:
 *              M, N or K < 0                              -> INVALID_ARG
 *              lda < max(1,K), ldb < max(1,N), ldc < max(1,N) -> INVALID_ARG
 *              NULL A (M,K > 0), B (K,N > 0) or C (M,N > 0) -> INVALID_ARG
 *              M, N or K above 2^31-1, C of more than 2^31-1
 *              64 x 64 tiles, or an operand whose byte range
 *              (leading dimension included) reaches 2^63     -> INVALID_ARG
 *              byte range of C overlapping that of A or B   -> ALIAS
 *              forced configuration unknown / wrong dtype   -> UNSUPPORTED
 *              launch failure reported by the HIP runtime   -> HIP
 *            gemm_last_error() returns a message for the calling thread's
 *            most recent failure.
 */
#ifndef DENSE_GEMM_ROW_AMD_GEMM_H
#define DENSE_GEMM_ROW_AMD_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = -1,
    GEMM_ERR_UNSUPPORTED = -2,
    GEMM_ERR_HIP = -3,
    GEMM_ERR_ALIAS = -4
} gemm_status_t;

/* IEEE 754 binary16 bit pattern. */
typedef uint16_t gemm_f16_t;
/* bfloat16 bit pattern: the upper 16 bits of an IEEE 754 binary32. */
typedef uint16_t gemm_bf16_t;
/* FP8 E4M3 byte (OCP 8-bit floating point: 1 sign, 4 exponent bits with
 * bias 7, 3 fraction bits, no infinities, largest finite 448). */
typedef uint8_t gemm_f8_t;
/* FP8 E5M2 byte (OCP 8-bit floating point: 1 sign, 5 exponent bits with
 * bias 15, 2 fraction bits, infinities and NaN in exponent 31, largest
 * finite 57344). */
typedef uint8_t gemm_e5m2_t;

typedef enum gemm_dtype {
    GEMM_DTYPE_F32 = 0,
    GEMM_DTYPE_F16 = 1,
    GEMM_DTYPE_BF16 = 2,
    GEMM_DTYPE_F8 = 3,  /* E4M3 A and B, bfloat16 C */
    GEMM_DTYPE_E5M2 = 4 /* E5M2 A and B, bfloat16 C */
} gemm_dtype_t;

/* Kernel families. */
typedef enum gemm_family {
    GEMM_FAMILY_MFMA = 0, /* matrix-core kernels (v_mfma_f32_32x32x2_f32,
                             v_mfma_f32_32x32x16_f16 / _bf16,
                             v_mfma_f32_32x32x64_f8f6f4)                  */
    GEMM_FAMILY_SIMT = 1  /* vector-FMA kernel, kept as an ablation (FP32) */
} gemm_family_t;

/* Workgroup-to-tile order. */
typedef enum gemm_order {
    GEMM_ORDER_ROW = 0,     /* tile (bid / tiles_n, bid % tiles_n)             */
    GEMM_ORDER_GROUPED = 1, /* column sweep inside bands of group_m tile rows  */
    GEMM_ORDER_XCD = 2      /* GROUPED after gathering the workgroups that the
                               dispatcher sends to one XCD (round robin over
                               8) into one contiguous run of tiles            */
} gemm_order_t;

/*
 * One compiled kernel variant plus its launch order.  gemm_get_config fills
 * every field; gemm_*_ex reads `id` (which variant) and `order`/`group_m`
 * (how workgroups map to tiles) and ignores the descriptive fields.
 */
typedef struct gemm_config {
    int32_t id;         /* index in the variant table of this dtype          */
    int32_t dtype;      /* gemm_dtype_t                                      */
    int32_t family;     /* gemm_family_t                                     */
    int32_t bm, bn, bk; /* macro tile: rows, columns, K-slice depth          */
    int32_t wm, wn;     /* per-wave tile (SIMT: per-thread tile rows, cols)  */
    int32_t threads;    /* workgroup size (multiple of the 64-lane wave)     */
    int32_t stages;     /* LDS buffers in the K pipeline                     */
    int32_t lds_bytes;  /* LDS per workgroup                                 */
    int32_t order;      /* gemm_order_t                                      */
    int32_t group_m;    /* band height in tile rows for GROUPED/XCD orders   */
    int32_t splits;     /* K chunks for gemm_*_splitk (1 = no split); the
                           plain and _ex entry points ignore it             */
    char name[48];      /* e.g. "mfma_f32_128x128x32_w64x64"                 */
} gemm_config_t;

/*
 * FP32 GEMM, C = A x B (FP32 in, FP32 out).  Chooses the variant from the
 * tuning table (gemm_load_tuning) or a shape heuristic.
 */
gemm_status_t gemm_f32(int64_t M, int64_t N, int64_t K,
                       const float *A, int64_t lda,
                       const float *B, int64_t ldb,
                       float *C, int64_t ldc, void *stream);

/*
 * FP16 GEMM, C = A x B: binary16 inputs, FP32 accumulation, binary16 output
 * rounded to nearest even (overflow gives +-Inf, subnormals are kept).
 */
gemm_status_t gemm_f16(int64_t M, int64_t N, int64_t K,
                       const gemm_f16_t *A, int64_t lda,
                       const gemm_f16_t *B, int64_t ldb,
                       gemm_f16_t *C, int64_t ldc, void *stream);

/*
 * BF16 GEMM, C = A x B: bfloat16 inputs, FP32 accumulation, bfloat16 output
 * rounded to nearest even.  BF16 is the 16-bit type the GB300 GEMM article
 * lists beside FP16 for the matrix units (sections 1.1 and 5.1); it keeps
 * FP32's exponent range with 8 significant bits.  Same kernels as FP16 with
 * the bf16 matrix instruction; every gemm_f16_* entry point has a gemm_bf16_*
 * counterpart with the same contract.
 */
gemm_status_t gemm_bf16(int64_t M, int64_t N, int64_t K,
                        const gemm_bf16_t *A, int64_t lda,
                        const gemm_bf16_t *B, int64_t ldb,
                        gemm_bf16_t *C, int64_t ldc, void *stream);

/*
 * FP8 GEMM, C = A x B: FP8 E4M3 inputs, FP32 accumulation, bfloat16 output
 * rounded to nearest even (E4M3 products reach 448^2 * K, past FP16's
 * range; bfloat16 keeps FP32's).  FP8 is the tier above FP16 that the
 * GB300 GEMM article names for the matrix units (section 1.1).  Inputs are
 * taken as they are (no scale factors; the fused-epilogue form's alpha
 * applies a per-tensor scale).  Any shape and alignment is accepted: the
 * vector layout (A, B, C 16-byte aligned, K, N, lda, ldb multiples of 16,
 * ldc a multiple of 8) runs on the 8-bit matrix instruction, anything else
 * on the general kernel, which widens each FP8 element to its (exactly
 * equal) bfloat16 value and computes on the bf16 instruction.  Every
 * gemm_f16_* entry point has a gemm_f8_* counterpart with gemm_f8_t A and B
 * and gemm_bf16_t C, with the same layout rules (the INT8 epilogue and A
 * transposed need the vector layout, as for every type);
 * gemm_splitk_workspace_bytes takes GEMM_DTYPE_F8.
 */
gemm_status_t gemm_f8(int64_t M, int64_t N, int64_t K,
                      const gemm_f8_t *A, int64_t lda,
                      const gemm_f8_t *B, int64_t ldb,
                      gemm_bf16_t *C, int64_t ldc, void *stream);

/* As gemm_f32 / gemm_f16 / gemm_bf16 / gemm_f8 with a forced variant and tile order
 * (tests, tuner, ablation).  cfg->id must name a variant of the matching
 * dtype. */
gemm_status_t gemm_f32_ex(int64_t M, int64_t N, int64_t K,
                          const float *A, int64_t lda,
                          const float *B, int64_t ldb,
                          float *C, int64_t ldc, void *stream,
                          const gemm_config_t *cfg);
gemm_status_t gemm_f16_ex(int64_t M, int64_t N, int64_t K,
                          const gemm_f16_t *A, int64_t lda,
                          const gemm_f16_t *B, int64_t ldb,
                          gemm_f16_t *C, int64_t ldc, void *stream,
                          const gemm_config_t *cfg);
gemm_status_t gemm_bf16_ex(int64_t M, int64_t N, int64_t K,
                           const gemm_bf16_t *A, int64_t lda,
                           const gemm_bf16_t *B, int64_t ldb,
                           gemm_bf16_t *C, int64_t ldc, void *stream,
                           const gemm_config_t *cfg);
gemm_status_t gemm_f8_ex(int64_t M, int64_t N, int64_t K,
                         const gemm_f8_t *A, int64_t lda,
                         const gemm_f8_t *B, int64_t ldb,
                         gemm_bf16_t *C, int64_t ldc, void *stream,
                         const gemm_config_t *cfg);

/*
 * Split-K GEMM: the same results contract as gemm_f32 / gemm_f16, for shapes
 * with too few output tiles to fill the GPU (e.g. M = N = 1024, K = 8192).
 * The K range is cut into S chunks of Kc = roundup(ceil(K / splits), a)
 * with a = 64, or 128 for the 8-bit types (a multiple of every variant's
 * K slice), and S = ceil(K / Kc) <= splits; one launch computes every chunk's FP32
 * partial product into `workspace` (S x M x N floats, row-major), and a
 * second launch sums the S partials of each element in chunk order and
 * writes C (FP32, or FP16 / BF16 rounded to nearest even once, after the
 * sum).
 * The order of the sum is fixed, so results are bit-reproducible for a
 * given configuration.  Splitting the K sum of the pages' C = A x B
 * changes only the order of its additions ("nxbn.cn GB300 GEMM",
 * section 6.2, on split-K and summation order).
 *
 * cfg      NULL: variant and split count from gemm_select_config.  Else
 *          cfg->id / order / group_m pick the variant for the partial
 *          products and cfg->splits the requested S (0 = choose).
 * workspace  Caller-owned device memory of at least
 *          gemm_splitk_workspace_bytes(dtype, M, N, K, splits) bytes,
 *          16-byte aligned, not overlapping A, B or C (-> ALIAS).  Too small
 *          or NULL (when a split happens) -> INVALID_ARG.  The library does
 *          not allocate.  Its contents on return are unspecified.
 * Falls back to the unsplit path (no workspace use) when S comes out as 1,
 * when the operands do not take the vector path (alignment as above), or
 * when the chosen variant has no split-K form.  Concurrent calls must not
 * share a workspace.
 */
gemm_status_t gemm_f32_splitk(int64_t M, int64_t N, int64_t K,
                              const float *A, int64_t lda,
                              const float *B, int64_t ldb,
                              float *C, int64_t ldc,
                              void *workspace, int64_t workspace_bytes,
                              void *stream, const gemm_config_t *cfg);
gemm_status_t gemm_f16_splitk(int64_t M, int64_t N, int64_t K,
                              const gemm_f16_t *A, int64_t lda,
                              const gemm_f16_t *B, int64_t ldb,
                              gemm_f16_t *C, int64_t ldc,
                              void *workspace, int64_t workspace_bytes,
                              void *stream, const gemm_config_t *cfg);
gemm_status_t gemm_bf16_splitk(int64_t M, int64_t N, int64_t K,
                               const gemm_bf16_t *A, int64_t lda,
                               const gemm_bf16_t *B, int64_t ldb,
                               gemm_bf16_t *C, int64_t ldc,
                               void *workspace, int64_t workspace_bytes,
                               void *stream, const gemm_config_t *cfg);
gemm_status_t gemm_f8_splitk(int64_t M, int64_t N, int64_t K,
                             const gemm_f8_t *A, int64_t lda,
                             const gemm_f8_t *B, int64_t ldb,
                             gemm_bf16_t *C, int64_t ldc,
                             void *workspace, int64_t workspace_bytes,
                             void *stream, const gemm_config_t *cfg);

/*
 * Per-workgroup timestamps of the GEMM launches that follow on the calling
 * thread (the "trace" of a launch; tracing and profiling).  While `stamps`
 * is set, every launch of the two LDS-direct kernel families (the default
 * variants: names "dl_f32_*" and "tr_*") makes workgroup w =
 * blockIdx.y * gridDim.x + blockIdx.x, for w < `workgroups`, write eight
 * uint64 into stamps[8w .. 8w+7]: pairs (shader-cycle counter s_memtime,
 * 100 MHz constant clock s_memrealtime) at four points: 0 kernel entry,
 * 1 first K slice in LDS, 2 K loop done, 3 C stores issued.  The
 * workgroup's clock over an interval is d(cycles) / d(constant clock) x
 * 100 MHz.  Each launch overwrites the entries of its workgroups; other
 * kernels write nothing.  `stamps` is a device buffer of at least
 * 8 x `workgroups` uint64, owned by the caller, who keeps it alive while
 * set; NULL stops tracing.  Bad capacity (negative, above 2^31-1, or 0
 * with a buffer) -> GEMM_ERR_INVALID_ARG.  Tracing is not a result of the
 * GEMM: outputs are unchanged.
 */
gemm_status_t gemm_trace_set(uint64_t *stamps, int64_t workgroups);

/*
 * Split-K that allocates nothing and takes no workspace: for callers that
 * cannot allocate device memory (code under HIP graph capture, serving
 * loops and harnesses that forbid hipMalloc).  The same computation and
 * results as gemm_<dtype>_splitk with the same cfg (bit for bit: same
 * variant, chunks and reduction order), for dtype GEMM_DTYPE_F32 / F16 /
 * BF16 / F8 / E5M2 with A, B and C of that dtype's gemm_<dtype>_splitk
 * types (device pointers; FP8 products are BF16).  The FP32 partial planes
 * live in a static device array of GEMM_SPLITK_STATIC_MAX_BYTES that each
 * GPU the library runs on holds until the process ends; the call itself
 * calls no allocator.
 * Errors: as gemm_<dtype>_splitk; an unknown dtype, or a split whose
 * partials (S x M x N x 4 bytes) exceed GEMM_SPLITK_STATIC_MAX_BYTES
 * -> GEMM_ERR_INVALID_ARG before any launch (pass cfg with fewer splits,
 * or use the workspace form).  Calls that run unsplit touch no scratch.
 * Every call on one GPU shares that GPU's array and leaves its last
 * partials there: calls that overlap in time on one GPU (two streams,
 * two threads) race and must be serialised by the caller.
 */
#define GEMM_SPLITK_STATIC_MAX_BYTES (64ll << 20)
gemm_status_t gemm_splitk_static(int32_t dtype, int64_t M, int64_t N, int64_t K,
                                 const void *A, int64_t lda,
                                 const void *B, int64_t ldb,
                                 void *C, int64_t ldc,
                                 void *stream, const gemm_config_t *cfg);

/* Workspace bytes a split-K call with `splits` requested chunks needs
 * (0 when it would not split; splits <= 0 means the library's choice for
 * the shape).  An unknown dtype, negative sizes or sizes that the GEMM
 * calls refuse (above 2^31-1, or C of more than 2^31-1 64 x 64 tiles)
 * give -1, and so does a workspace size beyond 2^63-1 bytes (a split-K
 * call then returns GEMM_ERR_INVALID_ARG). */
int64_t gemm_splitk_workspace_bytes(int32_t dtype, int64_t M, int64_t N, int64_t K,
                                    int32_t splits);

/*
 * GEMM with B given transposed: C = A x B where B is passed as Bt, the
 * N x K row-major matrix with Bt[j*ldbt + k] = B[k][j] (column-major B, the
 * layout of the baseline kernel in the lqnn.cn SGEMM article, section 3.1;
 * the page transposes it before its GEMM, here the matrix cores read its
 * k-contiguous columns directly).  Same conventions as gemm_f32 / gemm_f16
 * with ldbt >= max(1, K) in place of ldb >= max(1, N); the vector path needs
 * ldbt a multiple of 4 (FP32) or 8 (FP16).  cfg NULL: the selection for the
 * shape among the variants with a transposed-B form; a forced variant
 * without one -> UNSUPPORTED.
 */
gemm_status_t gemm_f32_bt(int64_t M, int64_t N, int64_t K,
                          const float *A, int64_t lda,
                          const float *Bt, int64_t ldbt,
                          float *C, int64_t ldc, void *stream,
                          const gemm_config_t *cfg);
gemm_status_t gemm_f16_bt(int64_t M, int64_t N, int64_t K,
                          const gemm_f16_t *A, int64_t lda,
                          const gemm_f16_t *Bt, int64_t ldbt,
                          gemm_f16_t *C, int64_t ldc, void *stream,
                          const gemm_config_t *cfg);
gemm_status_t gemm_bf16_bt(int64_t M, int64_t N, int64_t K,
                           const gemm_bf16_t *A, int64_t lda,
                           const gemm_bf16_t *Bt, int64_t ldbt,
                           gemm_bf16_t *C, int64_t ldc, void *stream,
                           const gemm_config_t *cfg);
gemm_status_t gemm_f8_bt(int64_t M, int64_t N, int64_t K,
                         const gemm_f8_t *A, int64_t lda,
                         const gemm_f8_t *Bt, int64_t ldbt,
                         gemm_bf16_t *C, int64_t ldc, void *stream,
                         const gemm_config_t *cfg);

/*
 * GEMM in any of the four layouts: C = op(A) x op(B), op(X) = X^T when its
 * flag is 1.  trans_a = 1: A is passed as its K x M transpose, row-major
 * (column-major A; element (i, k) at A[k*lda + i], lda >= max(1, M));
 * trans_b = 1: B as its N x K transpose (element (k, j) at B[j*ldb + k],
 * ldb >= max(1, K), as gemm_*_bt).  C is M x N row-major as always.  These
 * are the column-major operand layouts of the lqnn.cn SGEMM article
 * (section 3.1), read directly by the matrix cores instead of transposed
 * beforehand.  trans_a = 0 forms are the same calls as gemm_* / gemm_*_bt.
 * trans_a = 1 runs on the LDS-direct kernels only and needs the vector
 * layout: A, B, C 16-byte aligned; M, lda, ldb and N (K instead of N when
 * trans_b) multiples of 16 bytes' worth of elements; ldc likewise for C;
 * else UNSUPPORTED before any launch.  Flags other than 0 / 1 ->
 * INVALID_ARG.  cfg NULL: the selection among the variants with the form.
 */
gemm_status_t gemm_f32_trans(int64_t M, int64_t N, int64_t K,
                             const float *A, int64_t lda,
                             const float *B, int64_t ldb,
                             float *C, int64_t ldc, void *stream,
                             const gemm_config_t *cfg, int32_t trans_a, int32_t trans_b);
gemm_status_t gemm_f16_trans(int64_t M, int64_t N, int64_t K,
                             const gemm_f16_t *A, int64_t lda,
                             const gemm_f16_t *B, int64_t ldb,
                             gemm_f16_t *C, int64_t ldc, void *stream,
                             const gemm_config_t *cfg, int32_t trans_a, int32_t trans_b);
gemm_status_t gemm_bf16_trans(int64_t M, int64_t N, int64_t K,
                              const gemm_bf16_t *A, int64_t lda,
                              const gemm_bf16_t *B, int64_t ldb,
                              gemm_bf16_t *C, int64_t ldc, void *stream,
                              const gemm_config_t *cfg, int32_t trans_a, int32_t trans_b);
gemm_status_t gemm_f8_trans(int64_t M, int64_t N, int64_t K,
                            const gemm_f8_t *A, int64_t lda,
                            const gemm_f8_t *B, int64_t ldb,
                            gemm_bf16_t *C, int64_t ldc, void *stream,
                            const gemm_config_t *cfg, int32_t trans_a, int32_t trans_b);

/* Activation applied by the fused epilogue. */
typedef enum gemm_act {
    GEMM_ACT_NONE = 0,
    GEMM_ACT_RELU = 1 /* max(x, 0) */
} gemm_act_t;

/*
 * Fused epilogue: C = act(alpha * (A x B) + beta * C + bias[j]).
 * alpha and beta are the scaling parameters of the tiled SGEMM kernel in
 * the lqnn.cn SGEMM article (section 3.3; the page leaves beta unapplied,
 * here it has its BLAS meaning); bias and activation are the post-GEMM
 * operations that the GB300 GEMM article (section 7.1) fuses into the
 * epilogue instead of a second pass over C.
 */
typedef struct gemm_epilogue {
    float alpha;       /* scales the product A x B                            */
    float beta;        /* scales the old C; 0: C is not read (may hold NaN)   */
    const float *bias; /* NULL, or N device floats added per column j         */
    int32_t act;       /* gemm_act_t                                          */
} gemm_epilogue_t;

/*
 * GEMM with the fused epilogue, computed in FP32 from the FP32 accumulator
 * (and, for FP16 / BF16, from the 16-bit old C) and rounded once to the output
 * type.  Same layout, stream, alignment and error conventions as gemm_f32 /
 * gemm_f16, plus:
 *   epi NULL or epi->act unknown                       -> INVALID_ARG
 *   bias overlapping C                                 -> ALIAS
 *   forced variant without a fused-epilogue form       -> UNSUPPORTED
 * cfg NULL: the same selection as gemm_f32 / gemm_f16 (among the variants
 * with a fused-epilogue form).  K == 0 gives C = act(beta * C + bias).
 */
gemm_status_t gemm_f32_epi(int64_t M, int64_t N, int64_t K,
                           const float *A, int64_t lda,
                           const float *B, int64_t ldb,
                           float *C, int64_t ldc, void *stream,
                           const gemm_config_t *cfg, const gemm_epilogue_t *epi);
gemm_status_t gemm_f16_epi(int64_t M, int64_t N, int64_t K,
                           const gemm_f16_t *A, int64_t lda,
                           const gemm_f16_t *B, int64_t ldb,
                           gemm_f16_t *C, int64_t ldc, void *stream,
                           const gemm_config_t *cfg, const gemm_epilogue_t *epi);
gemm_status_t gemm_bf16_epi(int64_t M, int64_t N, int64_t K,
                            const gemm_bf16_t *A, int64_t lda,
                            const gemm_bf16_t *B, int64_t ldb,
                            gemm_bf16_t *C, int64_t ldc, void *stream,
                            const gemm_config_t *cfg, const gemm_epilogue_t *epi);
gemm_status_t gemm_f8_epi(int64_t M, int64_t N, int64_t K,
                          const gemm_f8_t *A, int64_t lda,
                          const gemm_f8_t *B, int64_t ldb,
                          gemm_bf16_t *C, int64_t ldc, void *stream,
                          const gemm_config_t *cfg, const gemm_epilogue_t *epi);

/*
 * GEMM with the INT8-quantising epilogue: the fused epilogue's value,
 * computed in FP32 from the accumulator, is rounded to the nearest integer
 * (ties to even) and saturated to [-128, 127]:
 *     Q[i][j] = sat8(rne(act(alpha * (A x B)[i][j] + bias[j])))
 * so the FP32 result becomes INT8 with its scaling inside the GEMM instead
 * of a separate quantisation pass over C (the epilogue fusion of the GB300
 * GEMM article, section 7.1).  alpha is the per-tensor quantisation scale
 * (1 / step); epi->beta must be 0 (an INT8 old C has no meaning here:
 * INVALID_ARG otherwise).  Q is M x N int8, row-major, leading dimension ldq
 * (>= max(1, N)); its columns [N, ldq) are never written; it must not
 * overlap A, B or the bias (-> ALIAS).  A NaN value gives 0.
 * Supported on the vector layout only: A, B, Q and bias 16-byte aligned, K,
 * N, lda, ldb multiples of 16 bytes' worth of A/B elements, ldq a multiple
 * of 16 (else UNSUPPORTED before any launch).  cfg NULL: the selection
 * among the variants with an INT8 form; a forced variant without one ->
 * UNSUPPORTED.
 */
gemm_status_t gemm_f32_epi_q8(int64_t M, int64_t N, int64_t K,
                              const float *A, int64_t lda,
                              const float *B, int64_t ldb,
                              int8_t *Q, int64_t ldq, void *stream,
                              const gemm_config_t *cfg, const gemm_epilogue_t *epi);
gemm_status_t gemm_f16_epi_q8(int64_t M, int64_t N, int64_t K,
                              const gemm_f16_t *A, int64_t lda,
                              const gemm_f16_t *B, int64_t ldb,
                              int8_t *Q, int64_t ldq, void *stream,
                              const gemm_config_t *cfg, const gemm_epilogue_t *epi);
gemm_status_t gemm_bf16_epi_q8(int64_t M, int64_t N, int64_t K,
                               const gemm_bf16_t *A, int64_t lda,
                               const gemm_bf16_t *B, int64_t ldb,
                               int8_t *Q, int64_t ldq, void *stream,
                               const gemm_config_t *cfg, const gemm_epilogue_t *epi);
gemm_status_t gemm_f8_epi_q8(int64_t M, int64_t N, int64_t K,
                             const gemm_f8_t *A, int64_t lda,
                             const gemm_f8_t *B, int64_t ldb,
                             int8_t *Q, int64_t ldq, void *stream,
                             const gemm_config_t *cfg, const gemm_epilogue_t *epi);

/*
 * FP8 E5M2 GEMM: the other OCP 8-bit encoding (5 exponent bits, 2 fraction
 * bits: FP16's exponent range, one fraction bit fewer than E4M3).  FP32
 * accumulation, bfloat16 output rounded to nearest even; the same kernels
 * as FP8 E4M3 with the E5M2 operand format of the matrix instruction.  Each
 * entry point has the contract of its gemm_f8_* counterpart (the same
 * forms, layouts, sizes and errors), with gemm_e5m2_t A and B;
 * gemm_splitk_workspace_bytes takes GEMM_DTYPE_E5M2.
 */
gemm_status_t gemm_e5m2(int64_t M, int64_t N, int64_t K,
                        const gemm_e5m2_t *A, int64_t lda,
                        const gemm_e5m2_t *B, int64_t ldb,
                        gemm_bf16_t *C, int64_t ldc, void *stream);
gemm_status_t gemm_e5m2_ex(int64_t M, int64_t N, int64_t K,
                           const gemm_e5m2_t *A, int64_t lda,
                           const gemm_e5m2_t *B, int64_t ldb,
                           gemm_bf16_t *C, int64_t ldc, void *stream,
                           const gemm_config_t *cfg);
gemm_status_t gemm_e5m2_splitk(int64_t M, int64_t N, int64_t K,
                               const gemm_e5m2_t *A, int64_t lda,
                               const gemm_e5m2_t *B, int64_t ldb,
                               gemm_bf16_t *C, int64_t ldc,
                               void *workspace, int64_t workspace_bytes,
                               void *stream, const gemm_config_t *cfg);
gemm_status_t gemm_e5m2_bt(int64_t M, int64_t N, int64_t K,
                           const gemm_e5m2_t *A, int64_t lda,
                           const gemm_e5m2_t *Bt, int64_t ldbt,
                           gemm_bf16_t *C, int64_t ldc, void *stream,
                           const gemm_config_t *cfg);
gemm_status_t gemm_e5m2_trans(int64_t M, int64_t N, int64_t K,
                              const gemm_e5m2_t *A, int64_t lda,
                              const gemm_e5m2_t *B, int64_t ldb,
                              gemm_bf16_t *C, int64_t ldc, void *stream,
                              const gemm_config_t *cfg, int32_t trans_a, int32_t trans_b);
gemm_status_t gemm_e5m2_epi(int64_t M, int64_t N, int64_t K,
                            const gemm_e5m2_t *A, int64_t lda,
                            const gemm_e5m2_t *B, int64_t ldb,
                            gemm_bf16_t *C, int64_t ldc, void *stream,
                            const gemm_config_t *cfg, const gemm_epilogue_t *epi);
gemm_status_t gemm_e5m2_epi_q8(int64_t M, int64_t N, int64_t K,
                               const gemm_e5m2_t *A, int64_t lda,
                               const gemm_e5m2_t *B, int64_t ldb,
                               int8_t *Q, int64_t ldq, void *stream,
                               const gemm_config_t *cfg, const gemm_epilogue_t *epi);

/* Variant table: count per dtype, and the description of variant idx. */
int32_t gemm_num_configs(int32_t dtype);
gemm_status_t gemm_get_config(int32_t dtype, int32_t idx, gemm_config_t *out);

/* The configuration gemm_f32 / gemm_f16 would use for this shape (host
 * only; no GPU work; splits = 1). */
gemm_status_t gemm_select_config(int32_t dtype, int64_t M, int64_t N, int64_t K,
                                 gemm_config_t *out);

/* The configuration gemm_f32_splitk / gemm_f16_splitk would use with
 * cfg = NULL: variant, tile order and split count (1 when splitting does not
 * pay for this shape).  Host only. */
gemm_status_t gemm_select_splitk_config(int32_t dtype, int64_t M, int64_t N, int64_t K,
                                        gemm_config_t *out);

/* Workgroup-to-tile map of a configuration (host only): the tile
 * (tile_m, tile_n) that workgroup `block` computes for an M x N output.
 * The kernels use the same function on the device. */
gemm_status_t gemm_tile_of_block(const gemm_config_t *cfg, int64_t M, int64_t N,
                                 int64_t block, int64_t *tile_m, int64_t *tile_n);

/* Host check of a variant's LDS layouts: every staging write and fragment
 * read stays inside the stage, writes cover the stage exactly once, and the
 * bank-conflict count under `banks` 4-byte banks is reported per access
 * class (out[0] staging writes, out[1] fragment reads, in extra passes over
 * the minimum).  Returns GEMM_OK when the layout is a bijection in bounds. */
gemm_status_t gemm_layout_check(int32_t dtype, int32_t idx, int32_t banks,
                                int64_t out[2]);

/* Environment, read at the first call: GEMM_FORCE_CONFIG=<variant name>
 * makes calls of that variant's element type that pass no cfg use it (where
 * it has the call's form; split-K calls take the model's best split count
 * for it), as if given to the *_ex form; gemm_select_config and
 * gemm_select_splitk_config still report the library's own choice.
 * GEMM_LOG (any value but "0") prints one line per call to stderr: type,
 * shape, form and the configuration used. */

/* Tuning table: a text file of lines "dtype M N K name order group_m
 * [splits]" (dtype f32|f16|bf16|f8|e5m2; splits defaults to 1).  Exact-shape matches
 * override the heuristic.  Loading replaces the previous table; NULL clears
 * it.  Not safe to call concurrently with GEMM calls. */
gemm_status_t gemm_load_tuning(const char *path);

const char *gemm_status_string(gemm_status_t status);
const char *gemm_last_error(void); /* thread-local; "" when none */
/* The same thread-local message under a second name: for GEMM_ERR_HIP it
 * holds the HIP runtime's error text (hipGetErrorString of the launch
 * error), for the other statuses the argument check that failed. */
const char *gemm_last_hip_error(void);
const char *gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_ROW_AMD_GEMM_H */
