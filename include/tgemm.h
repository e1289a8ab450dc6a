/*
 * tgemm -- dense GEMM for LLM linear layers on AMD Instinct MI355X (gfx950).
 *
 * C ABI of the shared library libtgemm.so.  Every entry point takes plain
 * device pointers and sizes; no framework types cross this boundary.
 *
 * Sources cited by short name:
 *   "GEMM compute-cost page"  kwkr.cn/news/191298 (why GEMM dominates LLM
 *                             compute; the linear layer Y = X W + b of its
 *                             section 3.1, the fused bias+activation
 *                             epilogue of section 5.1, the LM head of 7.2).
 *   "DeepGEMM page"           zwxr.cn/news/240083 (a DeepGEMM-style kernel
 *                             library: simple callable interface in section
 *                             1.3, row-major naive reference in 3.2, FP8
 *                             group scales in 2.4, fusion hooks in 5.1).
 *
 * Conventions shared by all calls
 * -------------------------------
 * Layout.   Matrices are row-major: element (i, j) of a matrix with row
 *           stride ld sits at ptr[i * ld + j] (the A[m*K + k], B[k*N + n]
 *           indexing of the DeepGEMM page, section 3.2).  The inner stride is
 *           always 1.
 * Memory.   All pointers are device pointers owned by the caller.  The
 *           library never allocates or frees device memory and keeps no
 *           buffers between calls.  Paths that need scratch (the K splits
 *           of the small-M bf16 kernel, of the integer-weight heads and of
 *           the FP8 tile scheduler; the log-softmax heads' statistics) take
 *           it from the caller as a `workspace` pointer and its size in
 *           bytes, with a *_workspace_size query for the size a call needs.
 *           A NULL workspace runs the unsplit kernels (the log-softmax heads
 *           require one).  A non-NULL workspace must be 16-byte aligned and
 *           at least the queried size, else TGEMM_ERR_INVALID.  Calls that
 *           may run at the same time must not share a workspace.  C must
 *           not overlap A, B, bias, the scale arrays or the workspace (not
 *           checked).
 * Threads.  The library holds no mutable state, so calls from several host
 *           threads are independent (each with its own workspace).
 * Streams.  `stream` is a hipStream_t passed as void*; NULL is the default
 *           stream.  Calls only enqueue work on it and return; they never
 *           synchronise.  Results are visible to later work on that stream.
 * Errors.   Every call returns a tgemm_status_t.  Argument errors are found
 *           before anything is enqueued, and C is then left untouched.
 *           TGEMM_ERR_LAUNCH reports a HIP error raised by the launch itself;
 *           faults inside a kernel surface at the caller's next
 *           synchronisation, as usual for asynchronous HIP work.
 * Sizes.    M, N, K >= 0.  M == 0 or N == 0 is a no-op returning TGEMM_OK.
 *           K == 0 is an empty sum: C = epilogue(0 + bias).  Each of M, N, K
 *           must be below 2^31, and every element offset (i * ld + j) must
 *           fit in 63 bits.
 */
#ifndef TGEMM_H
#define TGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TGEMM_ABI_VERSION 2

typedef enum {
    TGEMM_OK = 0,
    TGEMM_ERR_INVALID = 1,      /* bad pointer, size, stride or enum value      */
    TGEMM_ERR_UNSUPPORTED = 2,  /* valid request the kernels do not support      */
    TGEMM_ERR_LAUNCH = 3,       /* the HIP runtime refused the kernel launch    */
    TGEMM_ERR_SCRATCH = 4       /* gemm_bf16_noalloc: the split needs more than
                                   its fixed scratch (TGEMM_NOALLOC_SCRATCH_BYTES) */
} tgemm_status_t;

/* Epilogue applied to the fp32 accumulator before the single output rounding.
 * Order follows the GEMM compute-cost page, section 5.1: add the bias, then
 * the activation, then write back.  The activation is the tanh form of GeLU,
 * 0.5*y*(1 + tanh(sqrt(2/pi)*(y + 0.044715*y^3))).  The DeepGEMM page
 * (section 5.1) asks for a hook before the output is written; an enum is the
 * ahead-of-time-compiled form of that hook. */
typedef enum {
    TGEMM_EPI_NONE = 0,
    TGEMM_EPI_BIAS = 1,            /* y = acc + bias[j]                          */
    TGEMM_EPI_BIAS_GELU_TANH = 2   /* y = gelu_tanh(acc + bias[j])               */
} tgemm_epilogue_t;

typedef enum {
    TGEMM_OUT_F32 = 0,   /* C holds float32                                     */
    TGEMM_OUT_BF16 = 1   /* C holds bfloat16, rounded to nearest even            */
} tgemm_out_t;

/* Kernel family choice for gemm_bf16_ex. */
typedef enum {
    TGEMM_ALGO_AUTO = 0,   /* thin-M kernel for M <= 64, tiled kernel otherwise */
    TGEMM_ALGO_TILED = 1,  /* LDS-tiled MFMA kernel, any shape                  */
    TGEMM_ALGO_THIN = 2,   /* bandwidth-bound small-M kernel, requires M <= 64  */
    /* The tiled kernel with a fixed tile shape (the offline autotune sweep
     * times each against the automatic choice). */
    TGEMM_ALGO_TILED_256x256 = 3,
    TGEMM_ALGO_TILED_256x128 = 4,
    TGEMM_ALGO_TILED_128x128 = 5
} tgemm_algo_t;

/*
 * gemm_bf16 -- C[M,N] = epilogue(A[M,K] . B[K,N] + bias[N])
 *
 * The linear layer of the GEMM compute-cost page (section 3.1, Y = X W + b;
 * section 2.1 lists its uses: Q/K/V/O projections, the FFN pair, the LM
 * head) with bf16 inputs and fp32 accumulation.
 *
 *   A      bf16 [M, K], row stride lda (elements), lda >= K
 *   B      bf16 [K, N], row stride ldb, ldb >= N   (N-contiguous, "row-major B")
 *   bias   bf16 [N], contiguous; required (non-NULL) for the two bias
 *          epilogues and ignored for TGEMM_EPI_NONE
 *   C      out_dtype [M, N], row stride ldc, ldc >= N
 *   epilogue   a tgemm_epilogue_t value
 *   out_dtype  a tgemm_out_t value
 *   stream     hipStream_t or NULL
 *
 * Pointers must be non-NULL when the matrix they point to is non-empty.
 * Any alignment is accepted; 16-byte aligned base pointers with strides that
 * are multiples of 8 elements take the vectorised load path.  No workspace
 * is used (gemm_bf16_ex with a workspace may split small-M problems along
 * K).  Operands are used exactly as the bf16 values they hold, subnormals
 * included (no flush to zero); a NaN in A[i, k] makes row i of C NaN, one in
 * B[k, j] or bias[j] column j.  Returns TGEMM_OK, TGEMM_ERR_INVALID or
 * TGEMM_ERR_LAUNCH.
 */
int gemm_bf16(const void* A, const void* B, const void* bias, void* C,
              int64_t M, int64_t N, int64_t K,
              int64_t lda, int64_t ldb, int64_t ldc,
              int epilogue, int out_dtype, void* stream);

/* Layout of the B operand of gemm_bf16_strided_batched. */
typedef enum {
  TGEMM_B_KN = 0, /* B [K, N], row stride ldb >= N (as gemm_bf16) */
  TGEMM_B_NK = 1  /* B [N, K], row stride ldb >= K (as gemm_bf16_nt) */
} tgemm_b_layout_t;

/*
 * gemm_bf16_strided_batched -- C_z = epilogue(A_z . B_z + bias), z < batch,
 * with A_z = A + z*stride_a, B_z = B + z*stride_b, C_z = C + z*stride_c
 * (strides in elements; 0 shares an operand across the batch).
 *
 * Many same-shaped GEMMs in one launch, so that small problems together fill
 * the GPU (the GEMM compute-cost page, section 5.3: packing independent
 * small GEMMs into one batched call raised utilisation where single
 * small-M calls left it low).  One bias [N] serves every problem.  Each
 * problem follows gemm_bf16 (b_layout TGEMM_B_KN) or gemm_bf16_nt
 * (TGEMM_B_NK) and gives the same result as that call.
 * Invalid (TGEMM_ERR_INVALID): negative batch or strides, an unknown
 * b_layout, batch > 1 with stride_c < (M-1)*ldc + N (outputs would
 * overlap), and the per-problem errors.  batch > 65535, and for TGEMM_B_NK
 * the operands gemm_bf16_nt does not support, return TGEMM_ERR_UNSUPPORTED.
 * Vector loads are used only when strides keep every problem 16-byte
 * aligned.  Returns TGEMM_OK, TGEMM_ERR_INVALID, TGEMM_ERR_UNSUPPORTED or
 * TGEMM_ERR_LAUNCH.
 */
int gemm_bf16_strided_batched(const void* A, const void* B, const void* bias, void* C,
                              int64_t M, int64_t N, int64_t K,
                              int64_t lda, int64_t ldb, int64_t ldc,
                              int64_t stride_a, int64_t stride_b, int64_t stride_c, int64_t batch,
                              int b_layout, int epilogue, int out_dtype, void* stream);

/*
 * gemm_bf16_nt -- C = epilogue(A . Bt^T + bias): gemm_bf16 with the weight
 * given K-contiguous, Bt [N, K] row-major (row stride ldb >= K elements),
 * the layout nn.Linear keeps its weight in ([out_features, in_features]).
 *
 * The GEMM compute-cost page (section 5.2) asks that operands be laid out
 * the way the kernel reads them, so that no implicit transpose (an extra
 * pass and copy) precedes the product; this entry point reads [N, K] weights
 * as they are.  Everything else (A, bias, C, epilogue, out_dtype, numerics,
 * stream) as gemm_bf16.
 * Supported: K % 8 == 0, A and Bt 16-byte aligned with lda, ldb multiples of
 * 8 (others return TGEMM_ERR_UNSUPPORTED; N is free).  Returns TGEMM_OK,
 * TGEMM_ERR_INVALID, TGEMM_ERR_UNSUPPORTED or TGEMM_ERR_LAUNCH.
 */
int gemm_bf16_nt(const void* A, const void* Bt, const void* bias, void* C,
                 int64_t M, int64_t N, int64_t K,
                 int64_t lda, int64_t ldb, int64_t ldc,
                 int epilogue, int out_dtype, void* stream);

/* Name of the kernel gemm_bf16_nt launches for aligned operands of these
 * sizes, or NULL when they are unsupported or invalid.  No launch. */
const char* gemm_bf16_nt_kernel_name(int64_t M, int64_t N, int64_t K);

/*
 * gemm_bf16_ex -- gemm_bf16 with an explicit kernel family (tgemm_algo_t)
 * and an optional workspace for the small-M K split.
 *
 * For M <= 64 (the thin kernel) and a weight with few 512-column stripes
 * (N <= 65536) the thin kernel leaves most compute units idle; with a
 * workspace it cuts K into chunks run by separate workgroups (the DeepGEMM
 * page, section 2.1: a grid too small for the machine leaves units unused),
 * writes each chunk's fp32 partial sums to the workspace, and a second
 * kernel adds them in chunk order, applies bias and epilogue and rounds
 * once (deterministic; only the fp32 summation order differs from the
 * unsplit call).
 *
 *   algo             a tgemm_algo_t value
 *   workspace        NULL (never split) or device memory of at least
 *                    gemm_bf16_workspace_size(M, N, K, algo) bytes, 16-byte
 *                    aligned, owned by the caller; contents on entry do not
 *                    matter and are clobbered
 *   workspace_bytes  its size
 *
 * TGEMM_ALGO_THIN with M > 64 returns TGEMM_ERR_UNSUPPORTED; a non-NULL
 * workspace that is unaligned or short returns TGEMM_ERR_INVALID.  Other
 * arguments and errors as gemm_bf16.
 */
int gemm_bf16_ex(const void* A, const void* B, const void* bias, void* C,
                 int64_t M, int64_t N, int64_t K,
                 int64_t lda, int64_t ldb, int64_t ldc,
                 int epilogue, int out_dtype, int algo,
                 void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes gemm_bf16_ex needs to split this problem (a multiple of
 * 256; 0 when it would not split); -1 for negative or oversized sizes or an
 * unknown algo.  No GPU call. */
int64_t gemm_bf16_workspace_size(int64_t M, int64_t N, int64_t K, int algo);

/*
 * gemm_bf16_noalloc -- gemm_bf16_ex with its small-M K split in a fixed
 * device scratch array of the library instead of a caller workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * Arguments and results as gemm_bf16_ex with a sufficient workspace (the
 * same kernels, split plan and bits).  The call allocates and frees
 * nothing.  The scratch is TGEMM_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU,
 * held by every GPU the library runs on until the process ends; its address
 * on a device is looked up on the first call made with that device current.
 * A problem whose split needs more (gemm_bf16_workspace_size above the
 * limit) returns TGEMM_ERR_SCRATCH before anything is enqueued; problems
 * that do not split use no scratch.  All calls on one GPU share that GPU's
 * array and it keeps the last call's partials (no part of it needs to start
 * at zero): calls that may overlap on one GPU (other streams, other host
 * threads) race on it and must be serialised by the caller.  Returns
 * TGEMM_OK, TGEMM_ERR_INVALID, TGEMM_ERR_UNSUPPORTED, TGEMM_ERR_SCRATCH or
 * TGEMM_ERR_LAUNCH.
 */
#define TGEMM_NOALLOC_SCRATCH_BYTES (INT64_C(32) << 20)
int gemm_bf16_noalloc(const void* A, const void* B, const void* bias, void* C,
                      int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc,
                      int epilogue, int out_dtype, int algo, void* stream);

/*
 * gemm_fp8_blockscaled -- C[i,j] = sum_g sA[i,g] * sB[g, j/128] *
 *                                  sum_{k in group g} A[i,k] * B[k,j]
 *
 * FP8 inputs with per-group fp32 scale factors and fp32 accumulation, the
 * low-precision scheme of the DeepGEMM page, section 2.4: groups of 128
 * elements along K for each row of A, 128 x 128 blocks for B, products
 * accumulated in fp32, scales applied per K group, bf16 output.
 *
 *   A    OCP e4m3fn bytes [M, K], packed row-major (row stride K)
 *   sA   fp32 [M, ceil(K/128)], packed row-major; group g covers columns
 *        [128g, min(K, 128g+128))
 *   B    e4m3fn bytes [K, N], packed row-major (row stride N)
 *   sB   fp32 [ceil(K/128), ceil(N/128)], packed row-major
 *   C    bf16 [M, N], packed row-major
 *
 * Dequantised value = decode(code) * scale.  Scales must be finite; NaN
 * codes (0x7F, 0xFF) propagate to the outputs they touch.  Output tiles
 * are 256 x 256; when the last round of tiles would occupy at most half of
 * the compute units (one tile per unit), each of its tiles runs as two
 * 128-row halves over all of K, which gives bit-identical results
 * (gemm_fp8_blockscaled_ex with a workspace splits small grids along K
 * instead).  Returns TGEMM_OK, TGEMM_ERR_INVALID or TGEMM_ERR_LAUNCH.
 */
int gemm_fp8_blockscaled(const void* A, const float* sA, const void* B, const float* sB,
                         void* C, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * gemm_fp8_blockscaled_ex -- gemm_fp8_blockscaled with the tile scheduler's
 * K split, in a caller workspace.
 *
 * The direct kernel gives each 256 x 256 output tile to one workgroup, one
 * workgroup per compute unit at a time.  When the tiles would leave compute
 * units idle (the DeepGEMM page, section 2.1: a grid too small for the
 * machine leaves SMs unused), each tile of the last round is split along K
 * into P ranges of whole scale groups, run by P workgroups; their fp32
 * partial tiles go to the workspace and the workgroup that finishes last
 * adds them in range order and writes C.
 *
 *   split_parts      0: automatic (only when the tiles would keep at most a
 *                    quarter of the compute units busy: P = compute units /
 *                    tiles, at most 8, at least eight scale groups per range;
 *                    measured on MI355X, a fuller grid runs faster unsplit;
 *                    otherwise the 128-row halves of gemm_fp8_blockscaled);
 *                    1: never split, whole 256 x 256 tiles only (no halves
 *                    either); 2 .. 8: split the last round's tiles into that
 *                    many ranges (at most one per scale group), whatever the
 *                    grid
 *   workspace        NULL (never split) or device memory of at least
 *                    gemm_fp8_workspace_size(M, N, K, split_parts) bytes,
 *                    16-byte aligned, owned by the caller.  Layout: one
 *                    32-bit arrival counter per split tile (the region
 *                    rounded up to 256 bytes), then the fp32 partial tiles.
 *                    The counters must be zero before the workspace is
 *                    first used (allocate it zero-filled); every call
 *                    returns them to zero when it completes, so a workspace
 *                    kept for these calls needs no clearing between them.
 *                    The partial tiles' contents on entry do not matter.
 *   workspace_bytes  its size
 *
 * The result differs from the unsplit one only by fp32 summation order;
 * it does not depend on which workgroup finishes first.  Operands the
 * direct kernel does not take run unsplit on the general kernel.
 * split_parts outside 0 .. 8, or a non-NULL workspace that is unaligned or
 * short, returns TGEMM_ERR_INVALID; otherwise as gemm_fp8_blockscaled.
 */
int gemm_fp8_blockscaled_ex(const void* A, const float* sA, const void* B, const float* sB,
                            void* C, int64_t M, int64_t N, int64_t K, int split_parts,
                            void* workspace, int64_t workspace_bytes, void* stream);

/* Workspace bytes gemm_fp8_blockscaled_ex needs on the current device (the
 * plan depends on its compute-unit count): 0 when it would not split; -1
 * for negative or oversized sizes or split_parts outside 0 .. 8. */
int64_t gemm_fp8_workspace_size(int64_t M, int64_t N, int64_t K, int split_parts);

/*
 * gemm_fp8_blockscaled_nt -- gemm_fp8_blockscaled with the weight stored
 * K-contiguous: C[i,j] = sum_g sA[i,g] * sB[g, j/128] * sum_{k in g} A[i,k] * Bt[j,k]
 *
 * The layout nn.Linear keeps its weight in ([out, in] = [N, K]), in which
 * FP8 checkpoints are usually stored; the GEMM compute-cost page (section
 * 5.2) asks for operands in the layout the kernel reads, so no transpose
 * pass is needed.  Same scales and rounding as gemm_fp8_blockscaled:
 *
 *   A    e4m3fn bytes [M, K], packed row-major
 *   sA   fp32 [M, ceil(K/128)]
 *   Bt   e4m3fn bytes [N, K], packed row-major (row j = column j of B)
 *   sB   fp32 [ceil(K/128), ceil(N/128)] (block (g, h) covers K rows
 *        [128g, 128g+128) and columns [128h, 128h+128) of B), as before
 *   C    bf16 [M, N], packed row-major
 *
 * The Bt tile is read like A's, so every MFMA operand holds the same bytes
 * as in gemm_fp8_blockscaled on the transposed weight, and the results are
 * equal bit for bit (same kernel schedule and tile split).  Supported:
 * K % 16 == 0 (else TGEMM_ERR_UNSUPPORTED); any M, N, alignment.  Other
 * errors as gemm_fp8_blockscaled.
 */
int gemm_fp8_blockscaled_nt(const void* A, const float* sA, const void* Bt, const float* sB,
                            void* C, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * gemm_fp8_split_plan -- the tile split gemm_fp8_blockscaled_ex would use
 * (host only, no GPU call): for C [M, N] with K and `cus` compute units,
 * *whole tiles run whole and the last *split_tiles tiles run in *parts K
 * ranges each (*parts == 1: no split).  Returns TGEMM_OK, or
 * TGEMM_ERR_INVALID for negative or oversized sizes, cus < 0, split_parts
 * outside 0 .. 8 or a NULL output.
 */
int gemm_fp8_split_plan(int64_t M, int64_t N, int64_t K, int cus, int split_parts, int* whole,
                        int* split_tiles, int* parts);

/*
 * gemm_bf16_logsoftmax -- C[i,n] = y[i,n] - log sum_n' exp(y[i,n']),
 *                         y = X W + bias
 *
 * The LM head with its bias add and the LogSoftmax that follows it fused
 * (the GEMM compute-cost page, section 7.2: merging the output projection,
 * the bias and LogSoftmax so no separate passes read the logits back):
 * each row of C is the log-probability distribution over the N columns.
 * Shapes and strides as gemm_bf16 (X in place of A, W of B); bias bf16 [N]
 * or NULL (no bias); C bf16 or fp32 (out_dtype).
 *
 *   workspace        device memory of at least
 *                    gemm_logsoftmax_workspace_size(M, N, out_dtype) bytes,
 *                    16-byte aligned, owned by the caller; scratch (its
 *                    contents on entry do not matter and are clobbered)
 *   workspace_bytes  its size
 *
 * Two kernels on the stream: the thin GEMM, whose epilogue adds the bias,
 * forms per 512-column stripe each row's maximum and sum of exponentials
 * and writes the fp32 logits (into C for fp32 output, else into the
 * workspace); then a normalisation that merges each row's stripe pairs into
 * log sum exp and writes logit - lse.  Logits and the row statistics are
 * fp32 and each output is rounded once.  Calls on one stream serialise;
 * concurrent calls must not share a workspace.
 * Supported: M <= 64, K % 8 == 0, N % 8 == 0, X and W 16-byte aligned with
 * ldx, ldw multiples of 8 (others return TGEMM_ERR_UNSUPPORTED).  N == 0
 * with M > 0, a NULL or short workspace return TGEMM_ERR_INVALID.
 * Returns TGEMM_OK, TGEMM_ERR_INVALID, TGEMM_ERR_UNSUPPORTED or
 * TGEMM_ERR_LAUNCH.
 */
int gemm_bf16_logsoftmax(const void* X, const void* W, const void* bias, void* C,
                         int64_t M, int64_t N, int64_t K,
                         int64_t ldx, int64_t ldw, int64_t ldc, int out_dtype,
                         void* workspace, int64_t workspace_bytes, void* stream);

/*
 * gemm_bf16_w8_logsoftmax, gemm_bf16_w4_logsoftmax -- the weight-only int8 /
 * int4 LM head with bias and log-softmax over each row:
 *   C[i,n] = y[i,n] - log sum_n' exp(y[i,n']),  y = X (q s) + bias
 *
 * The GEMM compute-cost page's two remedies for the LM head (section 7.2)
 * together: the integer weight of gemm_bf16_w8 / gemm_bf16_w4 (plan A) and
 * the fused bias + LogSoftmax of gemm_bf16_logsoftmax (plan B).  Weight
 * codes, scales and their layouts as gemm_bf16_w8 / gemm_bf16_w4; bias,
 * output, workspace (gemm_logsoftmax_workspace_size(M, N, out_dtype) bytes)
 * and the two-pass scheme as gemm_bf16_logsoftmax.  Supported: the integer
 * heads' shapes (M <= 64, K % 8 == 0, N % 4 == 0, ldq % 4 == 0); others
 * return TGEMM_ERR_UNSUPPORTED.  N == 0 with M > 0, a NULL or short
 * workspace and the gemm_bf16_w8 argument errors return TGEMM_ERR_INVALID.
 * Returns TGEMM_OK, TGEMM_ERR_INVALID, TGEMM_ERR_UNSUPPORTED or
 * TGEMM_ERR_LAUNCH.
 */
int gemm_bf16_w8_logsoftmax(const void* X, const void* Q, const float* S, const void* bias, void* C,
                            int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq, int64_t ldc,
                            int out_dtype, void* workspace, int64_t workspace_bytes, void* stream);
int gemm_bf16_w4_logsoftmax(const void* X, const void* Q, const float* S, const void* bias, void* C,
                            int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq, int64_t ldc,
                            int out_dtype, void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of workspace gemm_bf16_logsoftmax needs: M * ceil(N/512) * 8
 * rounded up to a multiple of 256, plus M * N * 4 when out_dtype is
 * TGEMM_OUT_BF16; -1 for negative or oversized sizes or an unknown
 * out_dtype. */
int64_t gemm_logsoftmax_workspace_size(int64_t M, int64_t N, int out_dtype);

/*
 * gemm_bf16_w8 -- C[i,n] = epilogue( sum_k X[i,k] * (Q[k,n] * S[k/128, n]) + bias[n] )
 *
 * Weight-only int8 GEMM for the small-M, memory-bound case: the LM head of
 * the GEMM compute-cost page (section 7.2, its first remedy: keep the large
 * weight in a low-precision integer format so fewer bytes are streamed).
 * Scales follow the per-group scheme of the DeepGEMM page, section 2.4: one
 * fp32 scale per (group of 128 consecutive rows of Q, column).
 *
 *   X     bf16 [M, K], row stride ldx >= K (elements)
 *   Q     int8 [K, N] two's-complement codes, row stride ldq >= N (bytes)
 *   S     fp32 [ceil(K/128), N], packed row-major; row g scales Q rows
 *         [128g, min(K, 128g+128))
 *   bias  bf16 [N] or NULL (required when epilogue != TGEMM_EPI_NONE)
 *   C     [M, N] bf16 or fp32 (out_dtype), row stride ldc >= N
 *
 *   workspace        NULL (never split) or device memory of at least
 *                    gemm_wq_workspace_size(M, N, K) bytes, 16-byte
 *                    aligned, owned by the caller (contents irrelevant)
 *   workspace_bytes  its size
 *
 * Epilogue, output rounding and conventions as gemm_bf16.  Products X * Q
 * are exact and summed in fp32 per 128-row group, and each group's sum is
 * scaled by S in fp32 (no weight is rounded), so the result carries the
 * rounding of an fp32-accumulated GEMM.  With a workspace, a narrow weight
 * (N <= 65536) is cut along K into chunks of whole 128-row groups when that
 * fills more of the device; the chunks' fp32 partials go to the workspace
 * and are summed in chunk order, then the bias and epilogue are applied and
 * the result rounded once (deterministic; the summation order, so the last
 * bits, differ from the unsplit call).
 * X is used exactly as the bf16 values it holds, subnormals included (no
 * flush to zero); a NaN in X[i, k] makes row i of C NaN, a NaN in S[g, n]
 * or bias[n] column n.
 * Supported: M <= 64, K % 8 == 0, N % 4 == 0, ldq % 4 == 0 (others return
 * TGEMM_ERR_UNSUPPORTED).  An unaligned or short non-NULL workspace returns
 * TGEMM_ERR_INVALID.  Returns TGEMM_OK, TGEMM_ERR_INVALID,
 * TGEMM_ERR_UNSUPPORTED or TGEMM_ERR_LAUNCH.
 */
int gemm_bf16_w8(const void* X, const void* Q, const float* S, const void* bias, void* C,
                 int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq, int64_t ldc,
                 int epilogue, int out_dtype, void* workspace, int64_t workspace_bytes,
                 void* stream);

/* Workspace bytes gemm_bf16_w8 / gemm_bf16_w4 need to split this problem
 * along K (a multiple of 256; 0 when they would not split) on the current
 * device; -1 for negative or oversized sizes. */
int64_t gemm_wq_workspace_size(int64_t M, int64_t N, int64_t K);

/* Name of the kernel (or kernel pair, "split+reduction") gemm_bf16_w8
 * launches for packed operands of these sizes, with a sufficient workspace
 * (with_workspace != 0) or without one; NULL when they are unsupported or
 * invalid.  No launch. */
const char* gemm_w8_kernel_name(int64_t M, int64_t N, int64_t K, int with_workspace);

/*
 * gemm_bf16_w4 -- C[i,n] = epilogue( sum_k X[i,k] * (q[k,n] * S[k/128, n]) + bias[n] )
 *
 * Weight-only int4 GEMM: gemm_bf16_w8 with 4-bit codes, a quarter of the
 * bf16 weight's bytes (the GEMM compute-cost page, section 4.3, lists int4
 * beside int8 as the low-precision integer weight formats; section 7.2 is
 * the LM-head use).
 *
 *   X     bf16 [M, K], row stride ldx >= K (elements)
 *   Q     bytes [K/2, N], row stride ldq >= N (bytes): byte (r, n) holds
 *         q[2r, n] in bits 0-3 and q[2r+1, n] in bits 4-7, each a 4-bit
 *         two's-complement code in [-8, 7]
 *   S     fp32 [ceil(K/128), N], packed row-major; row g scales K rows
 *         [128g, min(K, 128g+128)) (Q byte rows [64g, 64g+64))
 *   bias, C, epilogue, out_dtype, workspace, stream as gemm_bf16_w8
 *
 * Numerics as gemm_bf16_w8: products are exact and each 128-row group's
 * fp32 sum is scaled once.  Supported: M <= 64, K % 8 == 0, N % 4 == 0,
 * ldq % 4 == 0 (others return TGEMM_ERR_UNSUPPORTED).  Returns TGEMM_OK,
 * TGEMM_ERR_INVALID, TGEMM_ERR_UNSUPPORTED or TGEMM_ERR_LAUNCH.
 */
int gemm_bf16_w4(const void* X, const void* Q, const float* S, const void* bias, void* C,
                 int64_t M, int64_t N, int64_t K, int64_t ldx, int64_t ldq, int64_t ldc,
                 int epilogue, int out_dtype, void* workspace, int64_t workspace_bytes,
                 void* stream);

/* As gemm_w8_kernel_name for gemm_bf16_w4. */
const char* gemm_w4_kernel_name(int64_t M, int64_t N, int64_t K, int with_workspace);

/*
 * quantize_fp8_1x128 -- FP8 codes and scales for the A operand of
 * gemm_fp8_blockscaled: one scale per (row, 128-wide column group).
 *
 * The producer side of the DeepGEMM page's low-precision scheme (section
 * 2.4): each group of consecutive values shares one fp32 scale that maps it
 * into the e4m3 range.  For the group of row i, columns [128g, min(K,128g+128)):
 *
 *   scale     = amax / 448 in fp32 (rounded to nearest), amax = max |x| over
 *               the group; 1 when the group is all zero
 *   Q[i, k]   = e4m3fn( clamp(X[i, k] / scale, -448, 448) ), the division in
 *               fp32 (rounded to nearest), the cast to nearest, ties to even;
 *               zero keeps its sign
 *
 *   X    bf16 [M, K], row-major with row stride ldx >= K
 *   Q    e4m3fn bytes [M, K], packed row-major (row stride K); may be passed
 *        straight to gemm_fp8_blockscaled as A
 *   S    fp32 [M, ceil(K/128)], packed row-major (gemm_fp8_blockscaled's sA)
 *
 * X must be finite (a NaN or infinity gives unspecified codes and scales in
 * its group).  Q and S must not overlap X.  M == 0 or K == 0 is a no-op.
 * Returns TGEMM_OK, TGEMM_ERR_INVALID (null pointer, negative size,
 * ldx < K), TGEMM_ERR_UNSUPPORTED (more than 2^33 rows x 512-column
 * chunks) or TGEMM_ERR_LAUNCH.
 */
int quantize_fp8_1x128(const void* X, void* Q, float* S, int64_t M, int64_t K, int64_t ldx,
                       void* stream);

/*
 * gemm_bf16_quant_fp8 -- Q, S = quantize_1x128( bf16( epilogue(A B + bias) ) )
 *
 * The bf16 GEMM with the activation quantiser welded into its epilogue (the
 * DeepGEMM page, section 1.2: activation, quantisation and scaling in one
 * kernel; section 2.4 for the 1 x 128 groups): each output is computed and
 * rounded to bf16 exactly as gemm_bf16 with bf16 output computes it, and
 * instead of being stored it is quantised as quantize_fp8_1x128 quantises
 * X -- per row, groups of 128 consecutive columns, scale = amax / 448 (1
 * for an all-zero group), code = e4m3fn(clamp(value / scale, -448, 448)).
 * The bf16 output is never written.  Q and S are the A operand and sA of a
 * following gemm_fp8_blockscaled (an FFN up-projection feeding an FP8
 * down-projection).  Codes and scales equal, bit for bit, gemm_bf16_ex on
 * the same tiled kernel followed by quantize_fp8_1x128 on its output.
 *
 *   A, B, bias, M, N, K, lda, ldb, epilogue   as gemm_bf16 (B is [K, N])
 *   Q     e4m3fn bytes [M, N], packed row-major (row stride N)
 *   S     fp32 [M, ceil(N/128)], packed row-major
 *   algo  TGEMM_ALGO_AUTO / TGEMM_ALGO_TILED (the tiled kernel's shape table)
 *         or TGEMM_ALGO_TILED_256x256 / _256x128 / _128x128
 *
 * Supported: the direct tiled kernel's operands -- A and B 16-byte aligned,
 * lda and ldb multiples of 8, K and N multiples of 8.  Others, and
 * TGEMM_ALGO_THIN, return TGEMM_ERR_UNSUPPORTED.  NULL Q or S (with M, N >
 * 0) and the gemm_bf16 argument errors return TGEMM_ERR_INVALID.  Q and S
 * must not overlap the inputs.  Returns TGEMM_OK, TGEMM_ERR_INVALID,
 * TGEMM_ERR_UNSUPPORTED or TGEMM_ERR_LAUNCH.
 */
int gemm_bf16_quant_fp8(const void* A, const void* B, const void* bias, void* Q, float* S,
                        int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int epilogue,
                        int algo, void* stream);

/*
 * quantize_fp8_128x128 -- FP8 codes and scales for the B operand of
 * gemm_fp8_blockscaled: one scale per 128 x 128 block.
 *
 * Same rule as quantize_fp8_1x128 with the group being the block of rows
 * [128g, min(K,128g+128)) and columns [128h, min(N,128h+128)) (DeepGEMM
 * page, section 2.4: a small block of the weight matrix shares one scale).
 *
 *   W    bf16 [K, N], row-major with row stride ldw >= N
 *   Q    e4m3fn bytes [K, N], packed row-major (gemm_fp8_blockscaled's B)
 *   S    fp32 [ceil(K/128), ceil(N/128)], packed row-major (its sB)
 *
 * Same error behaviour as quantize_fp8_1x128 (TGEMM_ERR_UNSUPPORTED beyond
 * 2^31 - 1 blocks).
 */
int quantize_fp8_128x128(const void* W, void* Q, float* S, int64_t K, int64_t N, int64_t ldw,
                         void* stream);

/* Name of the kernel configuration (or kernel pair, "split+reduction")
 * gemm_bf16_ex would launch for a problem with 16-byte aligned operands,
 * given a sufficient workspace (with_workspace != 0) or none (as gemm_bf16
 * always runs).  No launch, no validation of pointers; operands that are
 * not 16-byte aligned, or whose row strides are not multiples of 8, run the
 * register-staged kernel of the same tile shape.  Returns a static string,
 * or NULL when the request is invalid. */
const char* gemm_bf16_kernel_name(int64_t M, int64_t N, int64_t K, int epilogue,
                                  int out_dtype, int algo, int with_workspace);

/* Name of the kernel configuration gemm_fp8_blockscaled launches for these
 * sizes (the direct-to-LDS kernel when K is a multiple of 16 and N >= 4, the
 * general kernel otherwise).  No launch. */
const char* gemm_fp8_kernel_name(int64_t M, int64_t N, int64_t K);

/* Static, human-readable text for a status code. */
const char* gemm_status_string(int status);

/* TGEMM_ABI_VERSION of the built library. */
int gemm_abi_version(void);

/*
 * Attainable-ceiling probes -- measurement kernels, not part of any GEMM.
 *
 * The published peaks (2.5 PFLOP/s dense bf16, 5 PFLOP/s fp8, 8 TB/s HBM)
 * are not what this part sustains under load: the matrix-heavy kernels run
 * power-bound below the peak clock, and a plain streaming read does not
 * reach the HBM spec.  These probes measure what the hardware delivers with
 * nothing else in the way, so a kernel's fraction of them can be reported
 * next to its fraction of the published peak (the DeepGEMM page, section
 * 3.4: time, fraction of peak, bandwidth).
 *
 *   TGEMM_PROBE_MFMA_BF16 / _FP8: one 512-thread workgroup per compute unit;
 *       every wave issues 32 MFMAs per iteration (v_mfma_f32_32x32x16_bf16,
 *       or v_mfma_scale_f32_16x16x128_f8f6f4 on e4m3 operands) on seeded
 *       pseudo-random operands held in registers and rotated between
 *       instructions, into four independent accumulators; each thread
 *       writes one float (the sum of its accumulators) to out.  FLOP per
 *       call: gemm_probe_mfma_flop(probe, iters).
 *   TGEMM_PROBE_STREAM_READ: a streaming read of src (bytes, a multiple of
 *       16, src 16-byte aligned) taken as rows of (compute units) KiB, one
 *       workgroup per compute unit reading its KiB of every row with
 *       non-temporal 16-byte loads (the fastest read pattern measured on this
 *       part), plus a grid-stride tail; each thread writes the XOR of the
 *       32-bit words it read, so the XOR of all of out equals the XOR of all
 *       words of src.
 *
 * gemm_probe_out_elems(probe): the number of 32-bit outputs the probe
 * writes on the current device (-1 for an unknown probe or device).
 * Returns TGEMM_OK, TGEMM_ERR_INVALID (unknown probe, negative or oversized
 * iters, NULL or short out, bytes not a multiple of 16, unaligned src),
 * TGEMM_ERR_UNSUPPORTED (device properties unavailable) or TGEMM_ERR_LAUNCH.
 */
typedef enum {
    TGEMM_PROBE_MFMA_BF16 = 0,
    TGEMM_PROBE_MFMA_FP8 = 1,
    TGEMM_PROBE_STREAM_READ = 2
} tgemm_probe_t;

int64_t gemm_probe_out_elems(int probe);
double gemm_probe_mfma_flop(int probe, int64_t iters);
int gemm_probe_mfma(int probe, int64_t iters, float* out, int64_t out_elems, uint64_t seed, void* stream);
int gemm_probe_stream_read(const void* src, int64_t bytes, uint32_t* out, int64_t out_elems, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H */
