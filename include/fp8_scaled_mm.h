/*
 * fp8_scaled_mm.h -- C ABI of the MI355X (gfx950) FP8 scaled matrix multiply.
 *
 * The operation (the scaled-mm semantics of the gist "matmul_fp8.py"
 * (a-r-r-o-w), kernel `matmul_fp8_kernel`, and of pytorch PR #125204
 * "rowwise scaling kernel", Summary):
 *
 *     out[m][n] = bf16_rne( s[m][n] * sum_{k<K} A[m][k] * B[n][k]  (+ bias[n]) )
 *
 *   A    M x K float8 e4m3fn (OCP), row-major, row stride K bytes.
 *   B    N x K float8 e4m3fn, row-major, row stride K bytes.
 *        (fp8_scaled_mm_typed also takes e5m2 for either operand.)  This is the
 *        "TN" right operand: the K x N column-major matrix of the pages,
 *        handed over as its N x K transpose (PR #125204 Summary: only TN is
 *        supported and the scale of B runs along its fast dimension).
 *   s    FP8MM_PER_TENSOR: scale_a[0] * scale_b[0]   (one fp32 each)
 *        FP8MM_ROWWISE:    scale_a[m] * scale_b[n]   (M and N fp32 values;
 *        PR #125204 Summary: the scale of x has length M, that of y length N).
 *        The product of the two scales is formed in fp32 in both modes.
 *   The products are accumulated in fp32 (the gist's accumulator is fp32).
 *   bias optional bf16 vector of length N, added after scaling and not
 *        scaled (PR #142045 Summary: scaling and bias are to be applied as
 *        epilogues).
 *   out  M x N bf16, row-major, row stride N elements, rounded to nearest
 *        even.  Every element is written; `out` is never read.
 *
 * Pointers: A, B, scale_a, scale_b, bias and out are DEVICE pointers on the
 * current HIP device.  The library never dereferences them on the host, so
 * scales may be produced by an earlier kernel on the same stream.  The
 * caller owns every buffer and the library keeps no pointer to them after the
 * call returns; it may be called from several host threads.
 *
 * Workspace: when the output has too few tiles to occupy the GPU, the K
 * reduction can be split over several workgroups whose fp32 partial tiles
 * meet in a workspace (the split-K of the gist "matmul_fp8.py", autotune
 * parameter SPLIT_K, done with a deterministic in-order sum instead of
 * atomics).  The library never allocates one: fp8_scaled_mm and
 * fp8_scaled_mm_with_config never split K (they pick tiles that fill the GPU
 * without it), and fp8_scaled_mm_with_plan / fp8_scaled_mm_typed split K
 * only with a caller workspace.
 *
 * Execution: asynchronous on `stream` (a hipStream_t; NULL = the default
 * stream).  Every entry point only enqueues kernels: no allocation, no
 * memset, no host synchronisation, so a call can be captured into a HIP
 * graph, the first call on a stream included.  The first call on a device
 * reads the device's properties once (CU count, architecture).
 *
 * Preconditions (checked on the host, before anything is enqueued):
 *   - 0 <= M, N <= 2^31 - 1; 16 <= K <= 2^23 and K % 16 == 0 (whole 16-byte
 *     row chunks: the pages' TMA path likewise needs K * itemsize to be a
 *     multiple of 16, PR #142101 review discussion).  M == 0 or N == 0 is a
 *     successful no-op that touches no pointer (any of them may be NULL).
 *   - Otherwise A, B, scale_a, scale_b, out non-NULL; bias may be NULL.
 *   - A and B 16-byte aligned; scales 4-byte aligned; bias and out 2-byte
 *     aligned.  out must not overlap any input.
 * Errors: the return value is FP8MM_OK (0) or one of the FP8MM_ERR_* codes;
 * on a validation error nothing is enqueued and `out` is untouched.  A
 * device that is not a gfx950 gives FP8MM_ERR_DEVICE; a launch failure
 * reported by the runtime gives FP8MM_ERR_LAUNCH.
 */
#ifndef FP8_SCALED_MM_H
#define FP8_SCALED_MM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t; /* hipStream_t is `struct ihipStream_t*` */

enum fp8mm_scaling_mode {
    FP8MM_PER_TENSOR = 0,
    FP8MM_ROWWISE = 1
};

enum fp8mm_status {
    FP8MM_OK = 0,
    FP8MM_ERR_NULL = 1,    /* a required pointer is NULL */
    FP8MM_ERR_SHAPE = 2,   /* M, N or K out of range, or K % 16 != 0 */
    FP8MM_ERR_ALIGN = 3,   /* a pointer is not aligned as required */
    FP8MM_ERR_MODE = 4,    /* unknown scaling_mode */
    FP8MM_ERR_DEVICE = 5,  /* no usable HIP device, or not a gfx950 */
    FP8MM_ERR_LAUNCH = 6,  /* the kernel launch failed */
    FP8MM_ERR_CONFIG = 7,  /* unknown tile configuration id or split count */
    FP8MM_ERR_WORKSPACE = 8, /* caller workspace smaller than required */
    FP8MM_ERR_FORMAT = 9,    /* unknown operand format */
    FP8MM_ERR_SCRATCH = 10   /* fp8_scaled_mm_noalloc: plan larger than its scratch */
};

/* Operand formats (OCP 8-bit floating point).  The gist "matmul_fp8.py",
 * function `benchmark`, accepts float8_e4m3fn or float8_e5m2 operands. */
enum fp8mm_format {
    FP8MM_E4M3FN = 0,   /* bias 7, no infinities, NaN = S.1111.111, max 448 */
    FP8MM_E5M2 = 1      /* bias 15, IEEE-style inf/NaN, max 57344 */
};

/* The scaled multiply described above, with the tile configuration chosen
 * from (M, N, K, scaling_mode, bias present). */
int fp8_scaled_mm(const void* A, const void* B, const float* scale_a, const float* scale_b,
                  const void* bias_or_null, void* out, int64_t M, int64_t N, int64_t K,
                  int scaling_mode, struct ihipStream_t* stream);

/* The same, with an explicit tile configuration (0 <= config_id <
 * fp8_scaled_mm_num_configs()), or the automatic choice for config_id < 0.
 * Every configuration computes the same function; they differ in speed. */
int fp8_scaled_mm_with_config(const void* A, const void* B, const float* scale_a,
                              const float* scale_b, const void* bias_or_null, void* out,
                              int64_t M, int64_t N, int64_t K, int scaling_mode,
                              struct ihipStream_t* stream, int config_id);

/* splits value that asks for a stream-K plan (see fp8_scaled_mm_with_plan). */
#define FP8MM_SPLITS_STREAM_K (-1)

/* The most general form: explicit tile configuration (config_id < 0: chosen
 * from the shape), split-K factor (splits == 0: chosen; 1: no split; at most
 * 64, clamped to the number of K slices; FP8MM_SPLITS_STREAM_K: stream-K,
 * below), and workspace.  K is split only
 * with a non-NULL `workspace`: 256-byte aligned, at least
 * fp8_scaled_mm_workspace_size() bytes, zero-filled before its first use (its
 * first 256 KiB are arrival counters, which every call leaves at zero again;
 * the partial tiles after them need no initial value).  The caller owns it.
 * With a NULL workspace the automatic plan does not split, and an explicit
 * splits > 1 returns FP8MM_ERR_WORKSPACE.  A workspace must not be used by
 * two calls that can run at the same time.  Results do not depend on which
 * workgroup finishes first: partial tiles are summed in split order.
 *
 * Stream-K (splits == FP8MM_SPLITS_STREAM_K; a generic configuration that can
 * split K, else FP8MM_ERR_CONFIG; a workspace, else FP8MM_ERR_WORKSPACE):
 * the grid fills every workgroup slot of the GPU and each workgroup takes an
 * equal share of the tiles' (tile, K slice) iterations in tile-major order, so
 * the work is balanced however the tile count compares with the CU count; a
 * tile shared by several workgroups is finished through partial tiles summed
 * in workgroup order.  Its workspace (fp8_scaled_mm_workspace_size with the
 * same arguments) is bounded for any device; results are deterministic on a
 * given device (the split points depend on its CU count). */
int fp8_scaled_mm_with_plan(const void* A, const void* B, const float* scale_a,
                            const float* scale_b, const void* bias_or_null, void* out,
                            int64_t M, int64_t N, int64_t K, int scaling_mode,
                            struct ihipStream_t* stream, int config_id, int splits,
                            void* workspace, int64_t workspace_bytes);

/* fp8_scaled_mm_with_plan with the operand formats given: A holds a_format
 * codes and B b_format codes (FP8MM_E4M3FN or FP8MM_E5M2 each; mixed pairs
 * allowed).  The products of two float8 values are exact in fp32 for every
 * pair, so only the format decode differs; the rest of the contract, the
 * configurations and the workspace rules are those of fp8_scaled_mm_with_plan
 * (which is this call with both formats FP8MM_E4M3FN).  Infinite or NaN
 * inputs give IEEE results of the fp32 accumulation (not otherwise checked).
 * Returns FP8MM_ERR_FORMAT for any other format value. */
int fp8_scaled_mm_typed(const void* A, int a_format, const void* B, int b_format,
                        const float* scale_a, const float* scale_b, const void* bias_or_null,
                        void* out, int64_t M, int64_t N, int64_t K, int scaling_mode,
                        struct ihipStream_t* stream, int config_id, int splits, void* workspace,
                        int64_t workspace_bytes);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): fp8_scaled_mm_with_plan
 * (config_id < 0 / splits == 0: automatic, as there) whose split-K counters
 * and partial tiles live in a 64 MiB static device array of the library
 * instead of a caller workspace.  Each GPU the library runs on holds its own
 * copy from module load until the process ends; the call allocates nothing
 * and only enqueues kernels (a small kernel that zeroes the counters its plan
 * uses, then the multiply).  The array's device address is looked up once
 * per device, on the first call there.  The automatic plan splits only as
 * far as its partial tiles fit in the array; an explicit split count whose
 * plan does not fit returns FP8MM_ERR_SCRATCH with nothing enqueued.  Every
 * call on a GPU shares that GPU's array: calls that can overlap on one GPU
 * (different streams, or several host threads) race and may give wrong
 * results; calls on one stream are ordered and safe.  Operand formats are
 * e4m3fn; the rest of the contract is fp8_scaled_mm_with_plan's. */
int fp8_scaled_mm_noalloc(const void* A, const void* B, const float* scale_a,
                          const float* scale_b, const void* bias_or_null, void* out, int64_t M,
                          int64_t N, int64_t K, int scaling_mode, struct ihipStream_t* stream,
                          int config_id, int splits);

/* Workspace bytes the plan (config_id < 0 / splits == 0: automatic;
 * splits == FP8MM_SPLITS_STREAM_K: stream-K, an upper bound for any device)
 * needs for this problem when the call has a workspace; 0 when it does not
 * split K, -1 for a bad mode.  Host logic only. */
int64_t fp8_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K, int scaling_mode,
                                     int has_bias, int config_id, int splits);

/* The split-K factor the automatic plan uses when the call has a workspace
 * (host logic only; -1 for an invalid problem).  Without a workspace it is 1. */
int fp8_scaled_mm_select_splits(int64_t M, int64_t N, int64_t K, int scaling_mode, int has_bias,
                                int config_id);

/* Number of tile configurations compiled into the library. */
int fp8_scaled_mm_num_configs(void);

/* Static, NUL-terminated description of a configuration ("" if unknown). */
const char* fp8_scaled_mm_config_name(int config_id);

/* The configuration the automatic plan uses for this problem: without a
 * workspace (with_workspace == 0: fp8_scaled_mm, or a NULL workspace) or with
 * one (fp8_scaled_mm_with_plan with a workspace).  The plan comes from fixed
 * rules where 256 x 256 tiles fill the GPU and from a cost model fitted to
 * measurements of every plan elsewhere; each host thread keeps the model's
 * last answers for 64 shapes.  Pure host logic: no device access.  Returns
 * -1 for an invalid problem. */
int fp8_scaled_mm_select_config(int64_t M, int64_t N, int64_t K, int scaling_mode, int has_bias,
                                int with_workspace);

/* Grid size (workgroups) a launch of `config_id` without split-K uses on a
 * device with `num_cus` compute units for an M x N output (host logic only). */
int64_t fp8_scaled_mm_grid_size(int config_id, int64_t M, int64_t N, int num_cus);

/* Static, NUL-terminated text for a status code (fp8mm_status_string is the
 * same function under the short name). */
const char* fp8_scaled_mm_status_string(int status);
const char* fp8mm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FP8_SCALED_MM_H */
