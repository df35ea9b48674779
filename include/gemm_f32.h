/*
 * gemm_f32.h -- dense single-precision matrix multiply on AMD MI355X (gfx950).
 *
 * The operation is the one the UIUC ECE408 Lecture 12 final-project page
 * (project_template.cu, section 2, "tiledMatMulKernel") computes:
 *
 *     C[M x N] = A[M x K] . B[K x N]        row-major, binary32 in and out,
 *
 * i.e. C(i,j) = sum over k of A(i,k) * B(k,j), for any M, N, K >= 0, including
 * sizes that are not multiples of any tile and the 1 x 1 x 1 case the page
 * lists among its boundary runs.  As on the page there is no alpha/beta, no
 * transpose and no column-major form: C is overwritten.  The page addresses
 * packed operands; this interface adds the usual row-major leading dimensions:
 *
 *     A(i,k) = A[(size_t)i * lda + k]     lda >= max(1, K)
 *     B(k,j) = B[(size_t)k * ldb + j]     ldb >= max(1, N)
 *     C(i,j) = C[(size_t)i * ldc + j]     ldc >= max(1, N)
 *
 * Precision: products and sums are binary32 on the FP32 matrix cores
 * (v_mfma_f32_*_f32; no reduced-precision xf32 forms) or the FP32 vector
 * unit.  The summation order over k is the kernel's own, so on general
 * inputs the result differs from the exactly rounded sum by ordinary binary32
 * accumulation error; when every partial sum is representable in binary32
 * (e.g. operands that are small multiples of 0.25) the result is exact.
 *
 * Memory and ownership: A, B and C are DEVICE pointers owned by the caller,
 * 4-byte aligned (16-byte alignment of the base and of lda/ldb/ldc*4 lets the
 * kernels use 128-bit loads, but is not required).  C must not overlap A or
 * B, and must be ordinary device memory (hipMalloc): on shapes whose tile
 * count would leave most compute units idle in the last round, the library
 * splits the K range of some output tiles between two workgroups, first
 * clears those tiles and then adds both partial sums into C with hardware
 * atomic float adds.  Exactly two addends on +0.0 commute, so the result is
 * the same whichever lands first: every configuration is deterministic
 * (gemm_f32_describe() marks such plans).  The library allocates no device
 * memory.  Its only state is each device's compute-unit count, read once
 * (hipDeviceGetAttribute) on the first call that plans work for the current
 * device and used to size the tile rounds; without a usable device the
 * 256 compute units of a whole MI355X are assumed.  It is safe to call from
 * several host threads.
 *
 * Asynchrony: every call only enqueues work on `stream` (a hipStream_t; 0 is
 * the null stream) and returns.  Errors detected while the kernels run are
 * reported by the caller's next synchronising HIP call, not by the return
 * value.
 *
 * Degenerate shapes (as the harness of the UIUC ECE408 Lecture 12
 * final-project page treats them, project_template.cu section 7: negative
 * sizes are an error, an empty output returns at once, K = 0 leaves the sum
 * empty):
 *   M < 0, N < 0 or K < 0  -> GEMM_F32_ERR_DIM, nothing is enqueued;
 *   M == 0 or N == 0       -> GEMM_F32_OK, nothing is enqueued, any pointer
 *                             may be NULL;
 *   K == 0                 -> the M x N window of C is set to +0.0; A and B
 *                             may be NULL.
 * Only the M x N window of C is written; C[i*ldc + j] for j >= N is left
 * untouched.
 */
#ifndef GEMM_F32_H
#define GEMM_F32_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

/* Exported from libgemm_f32.so (the library is built with hidden visibility). */
#define GEMM_F32_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define GEMM_F32_OK          0  /* work enqueued (or nothing to do)            */
#define GEMM_F32_ERR_DIM     1  /* M, N or K negative, or too large to tile     */
#define GEMM_F32_ERR_LD      2  /* lda < max(1,K), ldb < max(1,N) or
                                   ldc < max(1,N)                              */
#define GEMM_F32_ERR_NULL    3  /* a pointer the shape needs is NULL            */
#define GEMM_F32_ERR_LAUNCH  4  /* the HIP runtime refused the kernel launch    */
#define GEMM_F32_ERR_CONFIG  5  /* unknown configuration index                 */
#define GEMM_F32_ERR_ALIGN   6  /* a pointer is not 4-byte aligned              */
#define GEMM_F32_ERR_SCRATCH 7  /* gemm_f32_ws_noalloc: the split plan needs
                                   more than GEMM_F32_SCRATCH_BYTES            */

/*
 * C := A . B on `stream`, with the kernel configuration chosen for the shape
 * and operand alignment (gemm_f32_describe() names the choice).  Arguments
 * are validated in this order: sizes (GEMM_F32_ERR_DIM), leading dimensions
 * (GEMM_F32_ERR_LD), the configuration index where one is passed
 * (GEMM_F32_ERR_CONFIG), NULL pointers (GEMM_F32_ERR_NULL), alignment
 * (GEMM_F32_ERR_ALIGN); the first failure is returned and nothing is
 * enqueued.  An empty output (M or N == 0) returns GEMM_F32_OK after the
 * size, leading-dimension and configuration checks, whatever the pointers.
 */
GEMM_F32_API int gemm_f32(int M, int N, int K,
             const float *A, int lda,
             const float *B, int ldb,
             float *C, int ldc,
             hipStream_t stream);

/*
 * As gemm_f32(), but with the kernel configuration forced to `config`
 * (0 <= config < gemm_f32_num_configs(); -1 selects automatically).  Every
 * configuration handles every shape and alignment, so this exists to test and
 * to time each kernel on any problem; unknown indices return
 * GEMM_F32_ERR_CONFIG.
 */
GEMM_F32_API int gemm_f32_with_config(int config, int M, int N, int K,
                         const float *A, int lda,
                         const float *B, int ldb,
                         float *C, int ldc,
                         hipStream_t stream);

/*
 * Split-K with a caller-provided workspace, for problems with few output
 * tiles and a long K (e.g. 200 x 200 x 20000, whose 64 x 64 tiles would
 * occupy 16 of the 256 compute units).  The K range is cut into slices that
 * run as independent workgroups, each writing its partial product into the
 * workspace; a second kernel then adds the slices in slice order (0, 1, ...)
 * into C, so the result is deterministic (and bit-exact whenever every
 * partial sum is representable, as with the other entry points).
 *
 * gemm_f32_ws_size() returns the workspace bytes the split plan for this
 * shape needs, or 0 when the shape is not split (enough tiles already, or K
 * too short).  gemm_f32_ws() computes C := A . B like gemm_f32(); it uses
 * the split plan when gemm_f32_ws_size(M, N, K) > 0, `workspace` is a
 * 16-byte aligned device buffer of at least that many bytes that overlaps
 * none of A, B and C, and the leading dimensions allow 32-bit panel
 * offsets; otherwise it runs exactly what gemm_f32() runs and leaves the
 * workspace untouched.  The caller owns the workspace; its contents on
 * return are unspecified.  Validation and return codes are gemm_f32()'s.
 * Calls that share a workspace must not run concurrently.
 */
GEMM_F32_API size_t gemm_f32_ws_size(int M, int N, int K);
GEMM_F32_API int gemm_f32_ws(int M, int N, int K,
                             const float *A, int lda,
                             const float *B, int ldb,
                             float *C, int ldc,
                             void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * product and split-K plan as gemm_f32_ws(), with the workspace taken from a
 * scratch array the library holds in device memory, GEMM_F32_SCRATCH_BYTES
 * per GPU (a static __device__ array, resident on each GPU the library runs
 * on until the process ends).  The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine.  Its address on the current device
 * is resolved once, on the first call on that device.
 *
 * 4 MiB holds every split plan on a whole MI355X (at most one 64 x 64 slab
 * per compute unit); a plan that needs more (a device with more compute
 * units) returns GEMM_F32_ERR_SCRATCH and enqueues nothing.  Shapes that are
 * not split run exactly what gemm_f32() runs.  Validation and the other
 * return codes are gemm_f32()'s.
 *
 * All calls on one GPU share its scratch array, which keeps the last call's
 * partial products (every slab element is written before it is read, so
 * nothing needs clearing): calls that overlap in time on one GPU (several
 * streams, or several host threads) race and give wrong results.  Order
 * them on one stream, or use gemm_f32_ws() with a workspace per stream.
 */
#define GEMM_F32_SCRATCH_BYTES ((size_t)4 << 20)
GEMM_F32_API int gemm_f32_ws_noalloc(int M, int N, int K,
                                     const float *A, int lda,
                                     const float *B, int ldb,
                                     float *C, int ldc,
                                     hipStream_t stream);

/* Number of kernel configurations, and the name of one ("" if unknown). */
GEMM_F32_API int gemm_f32_num_configs(void);
GEMM_F32_API const char *gemm_f32_config_name(int config);

/*
 * Shape of a configuration: output tile bm x bn, K-panel depth bk, threads
 * per workgroup; any output pointer may be NULL.  If blocks_per_cu is not
 * NULL it receives how many of its workgroups one compute unit holds at once
 * (from the HIP occupancy calculator, which needs a GPU; without one the call
 * returns GEMM_F32_ERR_LAUNCH).  Unknown configurations return
 * GEMM_F32_ERR_CONFIG.
 */
GEMM_F32_API int gemm_f32_config_info(int config, int *bm, int *bn, int *bk,
                                      int *threads, int *blocks_per_cu);

/*
 * Writes into buf (NUL-terminated, at most buflen bytes) a one-line
 * description of what gemm_f32_with_config(config, ...) would enqueue for
 * these arguments (config -1: what gemm_f32() would enqueue): the
 * configuration name first ("none" for an empty output, "fill_zero" for
 * K == 0), then tile grid, workgroup count and load widths, and, when the
 * last 1-4 rows or columns (or both) are computed as strips beside the tile
 * grid, " strip_rows=R" and/or " strip_cols=C"; when C has at least 2^23 elements and
 * rows that are not 16-byte aligned (C's address or ldc * 4 not a multiple
 * of 16) and the configuration has such a variant, " c_store=write_back"
 * (C written with ordinary rather than streaming stores); last, when a
 * stream-K plan splits some tiles' K range between two workgroups, which
 * then add their partial sums into C with atomic adds (C must be ordinary
 * device memory), " c_accumulate=atomic_add".
 * Pointers are only inspected for alignment, never dereferenced.  Returns the
 * status the call would return for the same arguments.
 */
GEMM_F32_API int gemm_f32_describe(int config, int M, int N, int K,
                                   const float *A, int lda,
                                   const float *B, int ldb,
                                   const float *C, int ldc,
                                   char *buf, int buflen);

/*
 * The FP32 matrix-core peak of HIP device `device` derived from its
 * properties: compute units x 256 FLOP per clock (four SIMDs, each finishing
 * one 32x32x2 FP32 MFMA, 4096 FLOP, every 64 cycles) x the peak engine clock
 * the runtime reports.  Any output pointer may be NULL.  Without a usable
 * device the call returns GEMM_F32_ERR_LAUNCH and writes nothing.
 */
GEMM_F32_API int gemm_f32_device_peak(int device, int *compute_units, int *clock_khz,
                                      double *tflops);

/* Static text for a return code. */
GEMM_F32_API const char *gemm_f32_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_F32_H */
