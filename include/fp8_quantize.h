/*
 * fp8_quantize.h -- C ABI of the MI355X (gfx950) dynamic FP8 quantiser.
 *
 * The operation (the gist "matmul_fp8.py" (a-r-r-o-w), functions `get_scale`
 * and `benchmark`: the bf16 operands are quantised before the scaled
 * multiply, with scale = amax / finfo(float8_e4m3fn).max, a division, a clamp
 * and a cast; pytorch PR #130422 "Inductor lowering for `torch._scaled_mm`",
 * Testing, treats this amax/cast as the producer fused into the preceding op):
 *
 *     scale    = amax / 448                      (fp32)
 *     q[r][c]  = e4m3fn_RNE( clamp( x[r][c] / scale, -448, 448 ) )
 *
 *   amax is max |x| over the whole matrix (FP8Q_PER_TENSOR, one scale) or
 *   over each row (FP8Q_ROWWISE, one scale per row).  The division is the
 *   correctly rounded fp32 one; the cast rounds to nearest, ties to even.  A
 *   row (per-tensor: a matrix) whose amax is 0 gets scale 0 and codes 0x00.
 *   The outputs are exactly what fp8_scaled_mm takes as A and scale_a (or, for
 *   B stored N x K, as B and scale_b).
 *
 *   x      rows x cols bf16, row-major (row stride cols elements), finite.
 *          (Outside that contract: a NaN element is skipped by the amax and
 *          comes out as a NaN code.)
 *   q      rows x cols e4m3fn codes (uint8), row-major.  Written in full.
 *   scale  1 (per-tensor) or rows (row-wise) fp32 values.  Written in full.
 *
 * Pointers are DEVICE pointers on the current HIP device; the caller owns them
 * and the library keeps none after the call.  The library allocates nothing.
 * Execution is asynchronous on `stream` (a hipStream_t; NULL = default).  The
 * per-tensor mode of fp8_quantize_e4m3 / _e5m2 reads x twice (a maximum pass,
 * then the conversion); while its kernels run, the first 4 bytes per
 * workgroup of q hold the workgroups' partial maxima, which the conversion
 * then overwrites.  The _ws entry points below read x once.
 *
 * Preconditions (checked on the host before anything is enqueued):
 *   0 <= rows, cols <= 2^31, cols % 16 == 0; x and q 16-byte aligned, scale
 *   4-byte aligned; x, q, scale non-NULL, except that x and q may be NULL
 *   when rows or cols is 0 (then only the scales, all 0, are written) and
 *   scale may be NULL for a row-wise call with no rows (nothing is written).
 *   q must not overlap x.
 * Errors: FP8Q_OK (0) or an FP8Q_ERR_* code; on a validation error nothing is
 * enqueued.
 */
#ifndef FP8_QUANTIZE_H
#define FP8_QUANTIZE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t*` */

enum fp8q_scaling_mode { FP8Q_PER_TENSOR = 0, FP8Q_ROWWISE = 1 };

enum fp8q_status {
    FP8Q_OK = 0,
    FP8Q_ERR_NULL = 1,   /* a required pointer is NULL */
    FP8Q_ERR_SHAPE = 2,  /* rows/cols out of range or cols % 16 != 0 */
    FP8Q_ERR_ALIGN = 3,  /* a pointer is not aligned as required */
    FP8Q_ERR_MODE = 4,   /* unknown scaling_mode */
    FP8Q_ERR_DEVICE = 5, /* no usable HIP device */
    FP8Q_ERR_LAUNCH = 6, /* a kernel launch failed */
    FP8Q_ERR_WORKSPACE = 7 /* workspace smaller than fp8_quantize_workspace_size() */
};

/* Quantise x into (q, scale) as described above. */
int fp8_quantize_e4m3(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                      int scaling_mode, struct ihipStream_t* stream);

/* The same for float8 e5m2 codes (the gist's `benchmark` quantises for
 * float8_e5m2 the same way, with finfo(float8_e5m2).max = 57344):
 *     scale = amax / 57344;  q = e5m2_RNE( clamp( x / scale, -57344, 57344 ) )
 * Arguments, preconditions and errors as for fp8_quantize_e4m3; the codes are
 * what fp8_scaled_mm_typed takes with FP8MM_E5M2. */
int fp8_quantize_e5m2(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                      int scaling_mode, struct ihipStream_t* stream);

/* Bytes of workspace the _ws entry points need for these arguments: 67840
 * for a per-tensor call with elements, else 0 (row-wise mode and empty matrices
 * use none). */
int64_t fp8_quantize_workspace_size(int64_t rows, int64_t cols, int scaling_mode);

/* The same operation as fp8_quantize_e4m3 / fp8_quantize_e5m2 (same results,
 * bit for bit), with a caller workspace that lets the per-tensor mode read x
 * once: one workgroup per CU holds its share of x in registers and LDS while
 * the maximum is formed across the grid, then converts it.
 *
 *   workspace        device memory, 4-byte aligned, at least
 *                    fp8_quantize_workspace_size() bytes, ZERO-FILLED before
 *                    its first use.  Every call sets its counters and flags
 *                    back to zero once the stream has run it, so one buffer
 *                    serves all calls ordered on one stream; calls that may
 *                    run at the same time need separate buffers.  NULL: the two-pass path
 *                    of fp8_quantize_e4m3 (no workspace is used).
 *   workspace_bytes  its size in bytes.
 *
 * The grid-wide wait of the one-pass kernel is bounded: if other work holds
 * CUs so that the kernel's workgroups cannot all run at once, a workgroup that
 * has waited 1 ms (see fp8_quantize_set_wait_limit_us) leaves its share to the
 * last workgroup to reach the wait, which re-reads and converts it.  Only the
 * time changes.
 * Errors: as fp8_quantize_e4m3, plus FP8Q_ERR_WORKSPACE (workspace non-NULL
 * and smaller than needed) and FP8Q_ERR_ALIGN (workspace not 4-byte aligned);
 * nothing is enqueued then.  Row-wise calls ignore the workspace. */
int fp8_quantize_e4m3_ws(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                         int scaling_mode, void* workspace, int64_t workspace_bytes,
                         struct ihipStream_t* stream);
int fp8_quantize_e5m2_ws(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                         int scaling_mode, void* workspace, int64_t workspace_bytes,
                         struct ihipStream_t* stream);

/* Test hook: the one-pass kernel's wait limit, in microseconds, for calls
 * enqueued after this one (process-wide, not thread-safe).  0 makes every
 * workgroup but the last to arrive leave its share to that one; a negative
 * value restores the default of 1000.  Returns the previous limit. */
int64_t fp8_quantize_set_wait_limit_us(int64_t us);

/* Static, NUL-terminated text for a status code. */
const char* fp8_quantize_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8_QUANTIZE_H */
