/*
 * mgemm.h -- dense GEMM for AMD MI355X (gfx950): C = alpha * op(A) * op(B) + beta * C.
 *
 * The operation is the one the GEMM pages define: "SGEMM CUDA代码学习" (leetCUDA
 * 15-sgemm), section 问题定义与记号 (C[m][n] = sum_k A[m][k] * B[k][n], row-major),
 * with the alpha/beta update of "CUDA GEMM：从基础写法到工程优化" (opening
 * definition) and of the worklog "如何优化一个 CUDA Matmul Kernel", Kernel 1.  The
 * "TN" layout of "HGEMM SMEM Swizzle 代码学习" (kernel comment) and of "Warp
 * Specialization HGEMM" section 6 (A row-major M x K, B stored N x K) is
 * (ta = MG_N, tb = MG_T) here.
 *
 * Storage.  Every matrix is row-major: element (r, c) of a stored matrix X is
 * at X + r * ldx + c (in elements).
 *   op(A) is M x K: stored M x K (lda >= K) when ta == MG_N,
 *                   stored K x M (lda >= M) when ta == MG_T.
 *   op(B) is K x N: stored K x N (ldb >= N) when tb == MG_N,
 *                   stored N x K (ldb >= K) when tb == MG_T.
 *   C is M x N with ldc >= N; it is read (when beta != 0) and written.
 *
 * Arithmetic.  Products and sums are fp32 (fp16/bf16 inputs are multiplied
 * exactly and accumulated in fp32); the epilogue computes alpha*acc + beta*C
 * in fp32 and rounds once (nearest-even) to the C type.  Summation order is
 * unspecified.  No TF32-style input rounding, no fast-math.
 *
 * Special cases (BLAS conventions):
 *   M == 0 or N == 0       no-op, nothing is read or written.
 *   K == 0 or alpha == 0   C = beta * C; A and B are not read.
 *   beta == 0              C is write-only: C's old contents (even NaN) are
 *                          never read.
 *
 * Pointers and ownership.  A, B, C are device pointers (HBM) owned by the
 * caller; the library never allocates, frees or retains them, never writes
 * A or B, and needs only element alignment (16-byte alignment of pointers and
 * leading dimensions selects faster load/store paths).  C must not overlap A
 * or B.  The call is asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream): device-side faults appear at the caller's next synchronisation.
 *
 * Errors.  Every argument is validated before anything is launched; on an
 * error C is untouched and the status says why:
 *   MG_EINVAL        negative dimension, leading dimension too small, NULL
 *                    pointer with a non-empty extent, unknown enum value,
 *                    C overlapping A or B.
 *   MG_EUNSUPPORTED  valid but outside what the kernels address: a dimension
 *                    >= 2^31, or a leading dimension above 2^21 elements.
 *   MG_EHIP          the launch failed; mg_last_hip_error() gives the code.
 *   MG_ESCRATCH      (gemm_ex_noalloc only) a forced split count needs more
 *                    than the library's fixed scratch array.
 * Functions never throw and never print.  Calls are reentrant and thread
 * safe; a GEMM call plans with the tuning table loaded when it starts, even
 * while another thread loads a new one.
 */
#ifndef MGEMM_H
#define MGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MG_OK = 0, MG_EINVAL = 1, MG_EUNSUPPORTED = 2, MG_EHIP = 3, MG_ESCRATCH = 4 } mg_status;
typedef enum { MG_N = 0, MG_T = 1 } mg_op;
typedef enum { MG_F32 = 0, MG_F16 = 1, MG_BF16 = 2 } mg_dtype;

/* fp32 SGEMM.  A, B, C are fp32. */
mg_status gemm_f32(mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K, float alpha,
                   const float *A, int64_t lda, const float *B, int64_t ldb, float beta,
                   float *C, int64_t ldc, void *stream);

/* fp16-input GEMM with fp32 accumulation.  A, B hold IEEE binary16 bit
 * patterns; C is fp16 (c_type = MG_F16) or fp32 (c_type = MG_F32). */
mg_status gemm_f16(mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K, float alpha,
                   const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, float beta,
                   void *C, mg_dtype c_type, int64_t ldc, void *stream);

/* bf16-input GEMM with fp32 accumulation.  A, B hold bfloat16 bit patterns;
 * C is bf16 (c_type = MG_BF16) or fp32 (c_type = MG_F32). */
mg_status gemm_bf16(mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K, float alpha,
                    const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, float beta,
                    void *C, mg_dtype c_type, int64_t ldc, void *stream);

/* The same three operations with the kernel configuration forced: `config`
 * is an id in [0, mg_num_configs(in_type)) or -1 for the planner's choice.
 * A configuration that cannot run the given problem (e.g. a fast-path
 * variant on misaligned data) returns MG_EUNSUPPORTED.  Used by the
 * autotuner and the profiling harness. */
mg_status gemm_f32_cfg(int config, mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K,
                       float alpha, const float *A, int64_t lda, const float *B, int64_t ldb,
                       float beta, float *C, int64_t ldc, void *stream);
mg_status gemm_f16_cfg(int config, mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K,
                       float alpha, const uint16_t *A, int64_t lda, const uint16_t *B,
                       int64_t ldb, float beta, void *C, mg_dtype c_type, int64_t ldc,
                       void *stream);
mg_status gemm_bf16_cfg(int config, mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K,
                        float alpha, const uint16_t *A, int64_t lda, const uint16_t *B,
                        int64_t ldb, float beta, void *C, mg_dtype c_type, int64_t ldc,
                        void *stream);

/* Split-K GEMM with a caller-provided workspace: any of the three operations
 * (in_type MG_F32 with c_type MG_F32; MG_F16 or MG_BF16 with their own type or
 * MG_F32 as c_type), with A, B, C and the arguments as above.
 *
 * The K dimension is cut into `splits` contiguous ranges.  Each range's
 * partial product is written in fp32 to `workspace`; a second kernel, on the
 * same stream, sums the partials in range order and applies alpha and beta
 * with one rounding to the C type.  This is the split of "如何优化一个 CUDA
 * Matmul Kernel" (the worklog), section Kernel 10: Warptiling (its look at the
 * kernels cuBLAS picks for small shapes: a matmul kernel followed by a
 * reduction kernel over extra memory), also named in "SGEMM CUDA代码学习",
 * 第6步 (cuBLAS gap review).  It fills the GPU when M x N gives few tiles and K
 * is long.  Results are deterministic (identical bits on every run with the
 * same arguments) and within the same error bound as the unsplit call, whose
 * last bits they may not match.
 *
 *   splits     0: the planner's choice: a single range (the plain kernel)
 *                 when the tiles already fill the GPU, else enough ranges to
 *                 give every CU work, each at least two K slices deep, and no
 *                 more than workspace_bytes holds; 1: no split; 2..64: at most
 *                 that many ranges (the ranges are whole K slices, so fewer
 *                 may result).
 *   workspace  device memory owned by the caller, 16-byte aligned, not
 *              overlapping A, B or C, of at least splits * M * N * 4 bytes
 *              when splits >= 2 (see mg_workspace_size); may be NULL when
 *              workspace_bytes is 0.  Its contents on entry are ignored; it
 *              is scratch until the call's kernels have finished.
 *   config     as for the _cfg entry points (-1: the planner's choice).
 *
 * With a workspace, an operand that 16-byte loads cannot read (base or
 * leading dimension not 16-byte aligned, or a contiguous extent that is not a
 * multiple of 16 bytes) is first copied into the workspace with its rows
 * padded with zeros to a 16-byte multiple, so the fast tiles run on it; the
 * copies are placed first, then the split partials.  mg_workspace_size
 * counts both (for 16-byte-aligned base pointers).
 * Errors: as above, plus MG_EINVAL for splits outside 0..64, a misaligned or
 * overlapping workspace, or one smaller than a forced split count needs. */
mg_status gemm_ex(mg_dtype in_type, mg_dtype c_type, mg_op ta, mg_op tb, int64_t M, int64_t N,
                  int64_t K, float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                  float beta, void *C, int64_t ldc, void *workspace, size_t workspace_bytes,
                  int config, int splits, void *stream);

/* gemm_ex without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Arguments, results and errors are gemm_ex's, with
 * the workspace replaced by a fixed scratch array of MG_NOALLOC_SCRATCH_BYTES
 * (32 MiB) that the library holds in device memory on every GPU it runs on,
 * from the first call on that GPU until the process ends.  The call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * The GPU is the stream's (the current device for the null stream).
 *
 * The planner (splits = 0) splits and repacks only within the scratch, so any
 * problem runs; a forced split count whose fp32 partials need more than the
 * scratch (splits * M * N * 4 > MG_NOALLOC_SCRATCH_BYTES) returns MG_ESCRATCH
 * before anything is launched.  Every call on one GPU uses that GPU's single
 * array: calls that overlap in time on one GPU (different streams, or
 * threads) race on it and give wrong results; serialize them.  The array
 * keeps the last call's contents, which no call relies on. */
#define MG_NOALLOC_SCRATCH_BYTES (32u << 20)
mg_status gemm_ex_noalloc(mg_dtype in_type, mg_dtype c_type, mg_op ta, mg_op tb, int64_t M, int64_t N,
                          int64_t K, float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                          float beta, void *C, int64_t ldc, int config, int splits, void *stream);

/* Workspace bytes that gemm_ex with splits = 0 uses for this problem when
 * given enough (operand copies plus split partials; 0 when it would neither
 * repack nor split), for 16-byte-aligned base pointers with these leading
 * dimensions. */
size_t mg_workspace_size(mg_dtype in_type, mg_dtype c_type, mg_op ta, mg_op tb, int64_t M, int64_t N,
                         int64_t K, int64_t lda, int64_t ldb);

/* fp32 GEMM through the fp16 matrix cores (C = alpha * op(A) * op(B) + beta * C,
 * fp32 A, B, C, arguments and special cases as for gemm_f32), for callers
 * who want fp32 results faster than the fp32 MFMA peak allows.
 *
 * "SGEMM CUDA代码学习", 第5步, trades accuracy for speed by rounding fp32 inputs
 * to TF32 for the tensor cores.  This entry keeps fp32-level accuracy
 * instead: each row of op(A) and column of op(B) is scaled by a power of two
 * that brings its largest magnitude into [2^14, 2^15), every scaled value v
 * is split into hi = fp16(v) and lo = fp16(v - hi), and
 *   op(A) op(B) ~ A_hi B_hi + A_hi B_lo + A_lo B_hi
 * runs as one fp16 GEMM with fp32 accumulation over 3 K (the split of
 * Markidis et al., 2018, with the scaling of Ootomo and Yokota, 2022); the
 * epilogue undoes the scaling exactly.  Each product is represented to about
 * 2^-21 relative, so the result meets the fp32 bound 1e-5 * |a_i| * |b_j|
 * (row and column 2-norms) by a wide margin; it is not bitwise equal to
 * gemm_f32.  Non-finite inputs give NaN or Inf but not necessarily the same
 * ones as gemm_f32.
 *
 *   workspace  device memory owned by the caller, 16-byte aligned, not
 *              overlapping A, B or C, of at least
 *              mg_split16_workspace_size(M, N, K) bytes (about 12 (M + N) K
 *              bytes: the split operands); contents on entry are ignored.
 * Errors: as for gemm_f32, plus MG_EINVAL for a missing, misaligned,
 * overlapping or too small workspace, and MG_EUNSUPPORTED for M, N or K
 * above 2^22, or K above 699040 (the split operands' row pitch). */
mg_status gemm_f32_split16(mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K, float alpha,
                           const float *A, int64_t lda, const float *B, int64_t ldb, float beta,
                           float *C, int64_t ldc, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Workspace bytes gemm_f32_split16 needs (0 for an empty problem). */
size_t mg_split16_workspace_size(int64_t M, int64_t N, int64_t K);

/* Kernel configurations available for an input type, and their names
 * (static strings).  A name reads
 * <staging>_<type>_<BM>x<BN>x<BK>[_s<stages>][_w<waves along M>x<waves along N>][_pp],
 * e.g. "dma_f16_256x256x64_s2_w2x4":
 *   dma     direct-to-LDS loads (both operands must be 16-byte loadable);
 *   ws      direct-to-LDS loads issued by four dedicated producer waves for
 *           the consumer waves (_w gives the consumer waves) that only read
 *           fragments and issue matrix instructions (same requirement);
 *   mfma    16-byte loads staged through registers (same requirement);
 *   elemA / elemB / elemAB   element loads for A / B / both (any alignment);
 *   valu    fp32 on the vector ALUs (fp32 C only);
 *   _pp     the ping-pong schedule (two wave groups alternating between
 *           matrix instructions and memory instructions);
 *   _sk     the stream-K schedule: one round of persistent workgroups share
 *           the problem's slice iterations in equal ranges, and a tile split
 *           between workgroups is finished by the last one to reach it, from
 *           fp32 partials in the workspace, summed in k order (deterministic).
 *           These run only through gemm_ex with a workspace of at least
 *           2 x 256 x BM x BN x 4 bytes plus 4 bytes per tile (a smaller one:
 *           MG_EUNSUPPORTED when forced; the planner then takes another
 *           configuration). */
int mg_num_configs(mg_dtype in_type);
const char *mg_config_name(mg_dtype in_type, int config);

/* The configuration the planner picks for a problem (or -1 if none fits). */
int mg_chosen_config(mg_dtype in_type, mg_dtype c_type, mg_op ta, mg_op tb, int64_t M, int64_t N,
                     int64_t K);

/* The configuration gemm_ex with a large enough workspace picks (after any
 * operand repacking), for 16-byte-aligned base pointers with these leading
 * dimensions; -1 if none fits. */
int mg_chosen_config_ws(mg_dtype in_type, mg_dtype c_type, mg_op ta, mg_op tb, int64_t M, int64_t N,
                        int64_t K, int64_t lda, int64_t ldb);

/* Load a shape-keyed tuning table (text, one rule per line:
 * "<in> <c> <ta> <tb> <M> <N> <K> <config-name> [ws [s=<splits>]]", e.g.
 * "f16 f16 N T 4096 4096 4096 dma_f16_256x256x64_s2_w2x4"); lines starting with
 * '#' are comments.  A rule tagged "ws" applies only to gemm_ex calls with a
 * workspace (it was tuned with split-K and operand repacking available), and
 * its "s=" count (1..64) replaces the planner's fill rule when gemm_ex is
 * called with splits = 0; untagged rules apply to every call.  Lines
 * "rate <in> <config> <fraction> <workgroups per CU>" record, per
 * configuration, the best fraction of the type's peak it reached where the
 * table was tuned and its occupancy there.
 *
 * Planning (plain calls): a problem takes the nearest rule of the same type
 * and layout class by log-distance of M, N, K, if one is near enough (sum of
 * |log2| ratios <= 1.5).  A rule for another shape is dropped when a cost
 * model expects it to be more than 10 % slower than the model's own pick.
 * The model charges each configuration ceil(tiles / (256 x occupancy))
 * rounds of (occupancy) tile times at its rate; it also decides for shapes no
 * rule is near.  Rules naming an element-load variant are skipped for
 * operands 16-byte loads can read.
 * Replaces any table loaded before.  Returns MG_EINVAL if the file cannot be
 * read or a line names an unknown config or tag (the previous table is then
 * kept).  The new table is published atomically: calls already planning keep
 * the table they started with. */
mg_status mg_load_tune_table(const char *path);
/* Number of rules in the loaded table (0 if none). */
int mg_tune_table_size(void);

/* Workgroups of a configuration that fit on one CU of the current device at
 * once, as the HIP runtime computes it from the kernel's registers, LDS and
 * workgroup size (one representative layout); -1 for an unknown config or
 * when the runtime cannot say (no device).  Used by the autotuner to record
 * the figure in the tuning table. */
int mg_config_occupancy(mg_dtype in_type, int config);

/* Human-readable status text (static string). */
const char *mg_status_str(mg_status s);
/* The hipError_t of the most recent MG_EHIP on the calling thread (0 if none). */
int mg_last_hip_error(void);
/* Library version string. */
const char *mg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MGEMM_H */
