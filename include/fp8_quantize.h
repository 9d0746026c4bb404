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
 * per-tensor mode uses scale[0] as its running maximum while the call's
 * kernels run.
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
    FP8Q_ERR_LAUNCH = 6  /* a kernel launch failed */
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

/* Static, NUL-terminated text for a status code. */
const char* fp8_quantize_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8_QUANTIZE_H */
