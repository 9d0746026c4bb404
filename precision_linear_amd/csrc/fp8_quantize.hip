// Dynamic FP8 (e4m3fn or e5m2) quantisation of a bf16 matrix for gfx950 (MI355X).
//
//   scale = amax / qmax           (fp32; amax over the matrix or over each row)
//   q     = RNE( clamp( x / scale, -qmax, qmax ) )          (x / scale in fp32)
//
// qmax = 448 for e4m3fn, 57344 for e5m2.  The quantisation of the gist
// "matmul_fp8.py" (a-r-r-o-w), functions `get_scale` and `benchmark`
// (scale = amax / finfo(dtype).max, divide, clamp, cast, for either float8
// dtype): the producer of A and scale_a for the scaled multiply, which
// pytorch PR #130422, Testing, notes can be fused with the preceding op.
// A row (or matrix) whose amax is 0 gets scale 0 and codes 0 (the division
// would be 0/0).
//
// HBM-bound: every element is read once (twice for the per-tensor mode, whose
// second pass usually hits the 256 MB MALL) and written once.
//   * Row-wise: one workgroup per row (grid-stride over rows beyond 128 per
//     CU).  A row of up to 8 x 4096 elements stays in registers between the
//     amax and the quantisation (16 bf16 = 32 bytes per thread and chunk,
//     loaded as two 16-byte vectors); longer rows are read a second time
//     (from L2).
//   * Per-tensor: a grid-stride amax pass whose workgroups each write their
//     maximum to a slot of their own, one workgroup that reduces the slots
//     and writes the scale, and a quantisation pass.  The slots are the first
//     4 * (workgroups) bytes of q, which the quantisation pass then
//     overwrites (every workgroup covers at least 4096 elements, so they fit):
//     the library allocates nothing.  (An atomic maximum on one word instead
//     serialised about 9 ns per workgroup at the end of the pass.)
//   * x / scale must be the correctly rounded fp32 quotient (the fp8 rounding
//     that follows turns a one-ulp difference at a tie into another code).
//     The IEEE division sequence is a dozen VALU instructions per element,
//     which made both modes VALU-bound.  The scale is the same for a whole
//     row (or matrix), so its correctly rounded reciprocal r is computed once
//     and each element takes a multiply and two residual corrections (Div
//     below: 5 VALU operations and a sign copy).
//   * The conversion is v_cvt_pk_fp8_f32 (e4m3) or v_cvt_pk_bf8_f32 (e5m2),
//     round to nearest even; its inputs are within +-qmax (1 + 2^-23).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8_quantize.h"

namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 16;                      // elements per thread per chunk
constexpr int kChunkElems = kThreads * kGroup;  // 4096
// Per-tensor passes: groups of 16 elements each thread keeps in flight per
// loop step, and workgroups per CU (measured on MI355X, 8192 x 8192: 4, 8,
// 16 and 32 per CU within 4% of each other, 8 the fastest).
constexpr int kAmaxUnroll = 4;
constexpr int kQuantUnroll = 2;
constexpr int kTensorBlocksPerCu = 8;

// Format parameters: FMT 0 = e4m3fn, 1 = e5m2.
template <int FMT> struct Fp8Fmt;
template <> struct Fp8Fmt<0> {
    static constexpr float kMax = 448.f;
    template <bool HI>
    __device__ static __forceinline__ int cvt_pk(float a, float b, int old) {
        return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
    }
};
template <> struct Fp8Fmt<1> {
    static constexpr float kMax = 57344.f;
    template <bool HI>
    __device__ static __forceinline__ int cvt_pk(float a, float b, int old) {
        return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
    }
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16 bf16 values (two 16-byte vectors) -> max |x|.
__device__ __forceinline__ float absmax16(const uint4 (&v)[2]) {
    float m = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m = fmaxf(m, fabsf(bf16_lo(w[i])));
            m = fmaxf(m, fabsf(bf16_hi(w[i])));
        }
    }
    return m;
}

// Correctly rounded x / s for many x and one s.
//
// r = RN(1/s) (IEEE division, once).  q0 = RN(x r) is within two ulps of x/s;
// the residual e0 = x - s q0 (one fma) and q1 = RN(q0 + e0 r) bring the
// quotient within one ulp; then, with r within half an ulp of 1/s and q1
// within one ulp of x/s, the residual e1 = x - s q1 is exact and
// RN(q1 + e1 r) = RN(x/s) (P. Markstein, "Computation of elementary functions
// on the IBM RISC System/6000 processor", IBM J. Res. Dev. 34(1), 1990; the
// final step of the IA-64 division sequences).  The argument needs the
// residuals clear of the fp32 subnormal range and r finite, so the sequence
// is taken only for 2^-60 <= s <= FLT_MAX.  There, every x that can reach a
// nonzero float8 code (|x/s| >= 2^-17, half the smallest e5m2 subnormal) has
// |x| >= 2^-77 and normal residuals, so its quotient is RN(x/s) exactly;
// smaller quotients (subnormal x) may be off in the last fp32 bits but round
// to +-0 in both formats either way.  Checked exhaustively on MI355X against
// the IEEE division: every positive finite bf16 amax (s = amax / qmax) times
// every finite bf16 x with |x| <= amax, both formats: no quotient with
// |x/s| >= 2^-17 and no float8 code differs.  Elsewhere (s tiny, infinite or
// NaN) the IEEE division is used.  The residuals are formed negated,
// e = s q - x, and subtracted, q - e r: the same values (rounding is
// symmetric), but x = -0 then gives -0 where x - s q would give +0.
//
// On this path the clamp to +-qmax is not needed: |x| <= amax, so the
// correctly rounded |x/s| is at most qmax (1 + 2^-23), which the float8
// conversion rounds to qmax (checked in the same exhaustive run, against the
// clamped IEEE quotient).  A NaN input (amax skips it) stays NaN, as it does
// through the clamp of the gist's torch code.
struct Div {
    float s, r;
    bool fast;
};

__device__ __forceinline__ Div make_div(float s) {
    Div d;
    d.s = s;
    d.r = 1.f / s;
    d.fast = s >= 0x1p-60f && s <= 3.4028234663852886e38f;
    return d;
}

__device__ __forceinline__ float div_fast(float x, const Div& d) {
    float q = x * d.r;
    float e = fmaf(d.s, q, -x);
    q = fmaf(-e, d.r, q);
    e = fmaf(d.s, q, -x);
    return fmaf(-e, d.r, q);
}

template <int FMT, bool FAST>
__device__ __forceinline__ float quant1(float x, const Div& d) {
    constexpr float kMax = Fp8Fmt<FMT>::kMax;
    if constexpr (FAST) {
        return div_fast(x, d);
    } else {
        const float y = x / d.s;
        return y != y ? y : fminf(fmaxf(y, -kMax), kMax);   // NaN passes, like torch's clamp
    }
}

// 16 bf16 values -> 16 float8 codes (one 16-byte vector).
template <int FMT, bool FAST>
__device__ __forceinline__ uint4 quant16_impl(const uint4 (&v)[2], const Div& d) {
    uint32_t out[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t w[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            int packed = Fp8Fmt<FMT>::template cvt_pk<false>(
                quant1<FMT, FAST>(bf16_lo(w[2 * p]), d), quant1<FMT, FAST>(bf16_hi(w[2 * p]), d), 0);
            packed = Fp8Fmt<FMT>::template cvt_pk<true>(quant1<FMT, FAST>(bf16_lo(w[2 * p + 1]), d),
                                                        quant1<FMT, FAST>(bf16_hi(w[2 * p + 1]), d),
                                                        packed);
            out[2 * h + p] = (uint32_t)packed;
        }
    }
    return uint4{out[0], out[1], out[2], out[3]};
}

// A row (or matrix) whose amax is 0 gets codes 0.
template <int FMT>
__device__ __forceinline__ uint4 quant16(const uint4 (&v)[2], const Div& d) {
    if (d.s == 0.f) return uint4{0u, 0u, 0u, 0u};
    return d.fast ? quant16_impl<FMT, true>(v, d) : quant16_impl<FMT, false>(v, d);
}

__device__ __forceinline__ void load16(const uint16_t* p, uint4 (&v)[2]) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
    v[0] = q[0];
    v[1] = q[1];
}

// Maximum over the workgroup (all lanes return it).
__device__ __forceinline__ float block_max(float m, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const int wave = threadIdx.x / 64;
    __syncthreads();   // red[] may still be read by the previous row's reduction
    if (threadIdx.x % 64 == 0) red[wave] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red[w]);
    return m;
}

// Row-wise.  CHUNKS > 0: the row (at most CHUNKS * 4096 elements) is held in
// registers, and the workgroup's next row is loaded before the current one is
// reduced and written (its load latency hides under that work); CHUNKS == 0:
// any length, read twice.
template <int CHUNKS, int FMT>
__global__ void __launch_bounds__(kThreads)
quant_rowwise_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ scale,
                     int64_t rows, int64_t cols) {
    __shared__ float red[kThreads / 64];
    const int64_t groups = cols / kGroup;
    if constexpr (CHUNKS > 0) {
        auto load_row = [&](int64_t r, uint4 (&w)[CHUNKS][2]) {
            const uint16_t* xr = x + r * cols;
#pragma unroll
            for (int c = 0; c < CHUNKS; ++c) {
                const int64_t g = threadIdx.x + (int64_t)c * kThreads;
                if (g < groups) load16(xr + g * kGroup, w[c]);
            }
        };
        uint4 v[CHUNKS][2];
        int64_t r = blockIdx.x;
        if (r < rows) load_row(r, v);
        for (; r < rows; r += gridDim.x) {
            uint4 vn[CHUNKS][2];
            const int64_t rn = r + gridDim.x;
            if (rn < rows) load_row(rn, vn);
            float m = 0.f;
#pragma unroll
            for (int c = 0; c < CHUNKS; ++c)
                if (threadIdx.x + (int64_t)c * kThreads < groups) m = fmaxf(m, absmax16(v[c]));
            const float s = block_max(m, red) / Fp8Fmt<FMT>::kMax;
            if (threadIdx.x == 0) scale[r] = s;
            const Div d = make_div(s);
            uint8_t* qr = q + r * cols;
#pragma unroll
            for (int c = 0; c < CHUNKS; ++c) {
                const int64_t g = threadIdx.x + (int64_t)c * kThreads;
                if (g < groups) *reinterpret_cast<uint4*>(qr + g * kGroup) = quant16<FMT>(v[c], d);
            }
#pragma unroll
            for (int c = 0; c < CHUNKS; ++c) {
                v[c][0] = vn[c][0];
                v[c][1] = vn[c][1];
            }
        }
    } else {
        for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
            const uint16_t* xr = x + r * cols;
            uint8_t* qr = q + r * cols;
            float m = 0.f;
            for (int64_t g = threadIdx.x; g < groups; g += kThreads) {
                uint4 v[2];
                load16(xr + g * kGroup, v);
                m = fmaxf(m, absmax16(v));
            }
            const float s = block_max(m, red) / Fp8Fmt<FMT>::kMax;
            if (threadIdx.x == 0) scale[r] = s;
            const Div d = make_div(s);
            for (int64_t g = threadIdx.x; g < groups; g += kThreads) {
                uint4 v[2];
                load16(xr + g * kGroup, v);
                *reinterpret_cast<uint4*>(qr + g * kGroup) = quant16<FMT>(v, d);
            }
        }
    }
}

// n floats of 0 (the scales of rows without elements).
__global__ void __launch_bounds__(kThreads) zero_kernel(float* p, int64_t n) {
    for (int64_t i = blockIdx.x * (int64_t)kThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kThreads)
        p[i] = 0.f;
}

// Per-tensor pass 1: this workgroup's maximum of |x| over its grid-stride
// share of the elements, into partial[blockIdx.x].
__global__ void __launch_bounds__(kThreads)
amax_kernel(const uint16_t* __restrict__ x, int64_t groups, float* partial) {
    __shared__ float red[kThreads / 64];
    constexpr int U = kAmaxUnroll;   // groups in flight per thread
    float m = 0.f;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t g = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    for (; g + (U - 1) * stride < groups; g += U * stride) {
        uint4 v[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) load16(x + (g + u * stride) * kGroup, v[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) m = fmaxf(m, absmax16(v[u]));
    }
    for (; g < groups; g += stride) {
        uint4 v[2];
        load16(x + g * kGroup, v);
        m = fmaxf(m, absmax16(v));
    }
    m = block_max(m, red);
    if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// Per-tensor pass 2 (one workgroup): amax = the maximum of the n partial
// maxima (n <= kReduceMax: at most kReducePerThread per thread, all loaded
// before any is used, so the pass costs one memory latency); scale[0] =
// amax / qmax.
constexpr int kReducePerThread = 16;
constexpr int kReduceMax = kThreads * kReducePerThread;

template <int FMT>
__global__ void __launch_bounds__(kThreads)
amax_reduce_kernel(const float* __restrict__ partial, int n, float* scale) {
    __shared__ float red[kThreads / 64];
    float v[kReducePerThread];
#pragma unroll
    for (int j = 0; j < kReducePerThread; ++j) {
        const int i = threadIdx.x + j * kThreads;
        v[j] = i < n ? partial[i] : 0.f;
    }
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < kReducePerThread; ++j) m = fmaxf(m, v[j]);
    m = block_max(m, red);
    if (threadIdx.x == 0) scale[0] = m / Fp8Fmt<FMT>::kMax;
}

// Per-tensor pass 3: quantise with the scale of pass 2.
template <int FMT>
__global__ void __launch_bounds__(kThreads)
quant_tensor_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ q, int64_t groups,
                    const float* scale) {
    const Div d = make_div(scale[0]);
    constexpr int U = kQuantUnroll;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t g = blockIdx.x * (int64_t)kThreads + threadIdx.x;
    for (; g + (U - 1) * stride < groups; g += U * stride) {
        uint4 v[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) load16(x + (g + u * stride) * kGroup, v[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            *reinterpret_cast<uint4*>(q + (g + u * stride) * kGroup) = quant16<FMT>(v[u], d);
    }
    for (; g < groups; g += stride) {
        uint4 v[2];
        load16(x + g * kGroup, v);
        *reinterpret_cast<uint4*>(q + g * kGroup) = quant16<FMT>(v, d);
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int device_cus_q() {
    int dev = -1, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
}

template <int FMT>
int quantize_impl(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                  int scaling_mode, struct ihipStream_t* stream) {
    if (scaling_mode != FP8Q_PER_TENSOR && scaling_mode != FP8Q_ROWWISE) return FP8Q_ERR_MODE;
    if (rows < 0 || cols < 0 || cols % kGroup != 0 || cols > (int64_t(1) << 31) ||
        rows > (int64_t(1) << 31))
        return FP8Q_ERR_SHAPE;
    const bool empty = rows == 0 || cols == 0;
    const int64_t n_scales = scaling_mode == FP8Q_PER_TENSOR ? 1 : rows;
    if ((n_scales > 0 && !scale) || (!empty && (!x || !q))) return FP8Q_ERR_NULL;
    if ((uintptr_t)scale & 3) return FP8Q_ERR_ALIGN;
    if (!empty && (!aligned16(x) || !aligned16(q))) return FP8Q_ERR_ALIGN;
    if (n_scales == 0) return FP8Q_OK;   // row-wise without rows: nothing to write
    const int cus = device_cus_q();
    if (cus <= 0) return FP8Q_ERR_DEVICE;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    uint8_t* qb = static_cast<uint8_t*>(q);
    (void)hipGetLastError();
    if (empty) {
        // No element: amax is 0, so every scale is 0.
        const int64_t blocks = (n_scales + kThreads - 1) / kThreads;
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                           dim3(kThreads), 0, hs, scale, n_scales);
    } else if (scaling_mode == FP8Q_ROWWISE) {
        const int64_t chunks = (cols + kChunkElems - 1) / kChunkElems;
        // One workgroup per row (up to 128 per CU, then grid-stride with the
        // next row prefetched): the hardware keeps 8 resident per CU and starts
        // the next as one finishes, which beat fewer workgroups that each
        // prefetch their next row (MI355X, 8192 x 8192: 41.4 -> 34.2 us).
        const int64_t cap = (int64_t)cus * 128;
        const unsigned grid = (unsigned)(rows < cap ? rows : cap);
        if (chunks <= 1)
            hipLaunchKernelGGL((quant_rowwise_kernel<1, FMT>), dim3(grid), dim3(kThreads), 0, hs, xb, qb,
                               scale, rows, cols);
        else if (chunks <= 2)
            hipLaunchKernelGGL((quant_rowwise_kernel<2, FMT>), dim3(grid), dim3(kThreads), 0, hs, xb, qb,
                               scale, rows, cols);
        else if (chunks <= 4)
            hipLaunchKernelGGL((quant_rowwise_kernel<4, FMT>), dim3(grid), dim3(kThreads), 0, hs, xb, qb,
                               scale, rows, cols);
        else if (chunks <= 8)
            hipLaunchKernelGGL((quant_rowwise_kernel<8, FMT>), dim3(grid), dim3(kThreads), 0, hs, xb, qb,
                               scale, rows, cols);
        else
            hipLaunchKernelGGL((quant_rowwise_kernel<0, FMT>), dim3(grid), dim3(kThreads), 0, hs, xb, qb,
                               scale, rows, cols);
    } else {
        const int64_t groups = rows * cols / kGroup;
        const int64_t want = (groups + kThreads - 1) / kThreads;
        int64_t cap = (int64_t)cus * kTensorBlocksPerCu;
        if (cap > kReduceMax) cap = kReduceMax;   // one partial per thread slot of pass 2
        const unsigned grid = (unsigned)(want < cap ? want : cap);
        // The partial maxima go to the start of q (grid <= ceil(n / 4096)
        // workgroups, 4 bytes each, within q's n bytes), which pass 3 overwrites.
        float* partial = reinterpret_cast<float*>(qb);
        hipLaunchKernelGGL(amax_kernel, dim3(grid), dim3(kThreads), 0, hs, xb, groups, partial);
        hipLaunchKernelGGL(amax_reduce_kernel<FMT>, dim3(1), dim3(kThreads), 0, hs, partial, (int)grid,
                           scale);
        hipLaunchKernelGGL(quant_tensor_kernel<FMT>, dim3(grid), dim3(kThreads), 0, hs, xb, qb, groups,
                           scale);
    }
    if (hipGetLastError() != hipSuccess) return FP8Q_ERR_LAUNCH;
    return FP8Q_OK;
}

}  // namespace

extern "C" {

int fp8_quantize_e4m3(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                      int scaling_mode, struct ihipStream_t* stream) {
    return quantize_impl<0>(x, q, scale, rows, cols, scaling_mode, stream);
}

int fp8_quantize_e5m2(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                      int scaling_mode, struct ihipStream_t* stream) {
    return quantize_impl<1>(x, q, scale, rows, cols, scaling_mode, stream);
}

const char* fp8_quantize_status_string(int s) {
    switch (s) {
        case FP8Q_OK: return "ok";
        case FP8Q_ERR_NULL: return "a required pointer is NULL";
        case FP8Q_ERR_SHAPE: return "rows or cols out of range (need cols % 16 == 0, both < 2^31)";
        case FP8Q_ERR_ALIGN: return "misaligned pointer (x, q: 16 B; scale: 4 B)";
        case FP8Q_ERR_MODE: return "unknown scaling mode";
        case FP8Q_ERR_DEVICE: return "no usable HIP device";
        case FP8Q_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

}  // extern "C"
