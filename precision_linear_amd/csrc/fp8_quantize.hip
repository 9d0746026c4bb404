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
// HBM-bound: every element is read once and written once (read twice by the
// per-tensor mode's two-pass path; the MALL keeps little of the first read for
// the second: re-reading 128 MiB right after reading it is 11% faster than
// reading it cold).
//   * Row-wise: one workgroup per row (grid-stride over rows beyond 128 per
//     CU).  A row of up to 8 x 4096 elements stays in registers between the
//     amax and the quantisation (16 bf16 = 32 bytes per thread and chunk,
//     loaded as two 16-byte vectors); longer rows are read a second time
//     (from L2).
//   * Per-tensor, two passes (no workspace, or a matrix below the one-pass
//     threshold): a grid-stride amax pass whose workgroups each write their
//     maximum to a slot of their own, one workgroup that reduces the slots
//     and writes the scale, and a quantisation pass.  The slots are the first
//     4 * (workgroups) bytes of q, which the quantisation pass then
//     overwrites (every workgroup covers at least 4096 elements, so they fit):
//     the library allocates nothing.  (An atomic maximum on one word instead
//     serialised about 9 ns per workgroup at the end of the pass.)
//   * Per-tensor, one pass (with a caller workspace): see
//     quant_tensor_onepass_kernel.
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

// ---------------------------------------------------------------------------
// Per-tensor mode in one pass over x (with a caller workspace).
//
// One workgroup of 1024 threads per CU.  Pass 1 reads the whole matrix in
// grid-stride steps of 1024 groups per workgroup (32 KiB of x); the first
// kHoldRegs steps stay in registers and the next kHoldLds in LDS (8192 x 8192
// on 256 CUs is 16 steps, 15 of them held), later ones are only reduced.
// Each workgroup publishes its maximum and counts itself in; the last to
// arrive reduces the maxima and hands the scale to every workgroup through a
// word of its own (one 128-byte line each, so no line is polled by more than
// one workgroup, nor by anyone while the count is raised); each waits for its
// word, then converts what it holds, re-reading only the steps it did not
// hold.  x is read once, not twice.
//
// The wait needs every workgroup of the grid to reach pass 1's end while the
// others wait, i.e. all of them resident at once.  One per CU with the CU
// count as the grid is that, but not when other kernels hold CUs (another
// stream, another process).  So the wait is bounded: a workgroup that has
// waited 1 ms of the constant-rate wall clock (or the limit set by
// fp8_quantize_set_wait_limit_us) claims its word by exchanging kGaveUp into
// it.  If the exchange returns 0 it leaves, freeing its CU for the workgroups
// not yet started, and its share is left to the last to arrive, whose own
// exchange of that word returns kGaveUp: after its own pass 2 it converts
// every share so left (re-reading x).  If the exchange returns the scale, the
// scale had just arrived: the workgroup sets the word back to 0 and goes on.
// Each word thus has one owner at every moment, and the result never depends
// on which path a share took.
//
// Workspace (32-bit words; zero-filled before its first use, and every call
// sets them back to zero: the last to arrive resets the counter, the maxima
// and the words of shares left to it, every other workgroup its own word once
// read):
//   [0] arrivals   [kWsPartial + b] ~(workgroup b's maximum's bits), 0 until stored
//   [kWsGo + 32 b] ~(the scale's bits) for workgroup b, 0 until it is known,
//                  kGaveUp once b has left its share (a scale's bits are never
//                  all ones, nor kGaveUp's complement: the maximum skips NaN)
constexpr int kOneThreads = 1024;
constexpr int kOneWaves = kOneThreads / 64;
constexpr int kHoldRegs = 11;                    // steps held in registers (88 VGPRs)
constexpr int kHoldLds = 4;                      // steps held in LDS (128 KiB)
constexpr int kOneMaxGrid = 512;
constexpr int kWsPartial = 64;
constexpr int kWsGo = kWsPartial + kOneMaxGrid;
constexpr int kGoStride = 32;                    // words: one 128-byte line per workgroup
constexpr int64_t kOneWorkspaceBytes = 4 * (kWsGo + kGoStride * kOneMaxGrid);
constexpr uint32_t kGaveUp = 0x00400001u;        // ~ of a NaN pattern
// The grid-wide wait costs a few memory round trips plus the spread of the
// workgroups' pass-1 end times (MI355X: 6-8 us); below about 6 steps per
// workgroup (25M elements on 256 CUs) reading x twice is faster: 4096 x 4096
// one pass 23.4 us, two passes 20.2 us; 8192 x 4096 31.9 us against 34.7 us.
constexpr int64_t kOnePassMinSteps = 6;
constexpr int64_t kWaitUsDefault = 1000;
constexpr uint32_t kMaxPolls = 1u << 20;
constexpr uint32_t kBufferWord3 = 0x00020000u;   // raw buffer, 32-bit data format

int64_t g_wait_us = kWaitUsDefault;

// Workspace words are read and written with device-scope atomics (coherent
// across the XCDs' L2s), relaxed.  No fence is needed: the only data that
// passes between workgroups is in those words themselves, and each word says
// by its own value whether it has been written (a maximum and a scale word
// are nonzero once stored), so a reader waits for the value, not for an
// ordering.  (An acquire at this scope would also invalidate the XCD's L2:
// one per workgroup cost 2.5 us per 8192 x 8192 call.)
__device__ __forceinline__ uint32_t ws_load(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ws_store(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes per lane from x into LDS: lane l's bytes at byte offset voff land
// at lds + 16 l (lds is wave-uniform, in M0).  Inline asm: the compiler does
// not track these loads, so their consumer waits with an explicit vmcnt(0).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, const void* lds, uint32_t voff) {
    const uint32_t m0 = (uint32_t)(uintptr_t)lds;
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "{m0}"(m0)
                 : "memory");
}

// Maximum over a workgroup of W waves (all lanes return it).
template <int W>
__device__ __forceinline__ float block_max_w(float m, float* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __syncthreads();
    if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < W; ++w) m = fmaxf(m, red[w]);
    return m;
}

template <int FMT>
__global__ void __launch_bounds__(kOneThreads)
quant_tensor_onepass_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ q, float* __restrict__ scale,
                            int64_t groups, uint32_t* ws, int64_t wait_ticks) {
    __shared__ __attribute__((aligned(1024))) uint4 held[kHoldLds][2][kOneThreads];
    __shared__ float red[kOneWaves];
    __shared__ uint32_t left[kOneMaxGrid];   // the last to arrive: shares left to it
    __shared__ float s_scale;
    __shared__ int s_last, s_gave, s_any_left;
    const int tid = threadIdx.x;
    const int64_t T = (int64_t)gridDim.x * kOneThreads;
    const int64_t g0 = blockIdx.x * (int64_t)kOneThreads + tid;
    const int64_t steps = (groups + T - 1) / T;
    // The held steps in 32-bit byte offsets from x and q (at most
    // (kHoldRegs + kHoldLds) * 2^19 groups of 32 bytes: under 2^31), with
    // step s present when s * T < groups - g0.
    const uint32_t t32 = (uint32_t)T;
    const int64_t rem = groups - g0;
    const uint32_t lim = rem <= 0 ? 0u : rem >= 0x7fffffff ? 0x7fffffffu : (uint32_t)rem;
    const uint32_t off0 = (uint32_t)g0 * 32u;
    const char* xc = reinterpret_cast<const char*>(x);
    char* qc = reinterpret_cast<char*>(q);
    auto held_store = [&](uint32_t s, const uint4& c) {
        *reinterpret_cast<uint4*>(qc + (off0 / 2u + s * t32 * 16u)) = c;
    };
    uint32_t* go = ws + kWsGo + kGoStride * blockIdx.x;

    // Pass 1: issue every held step's loads (registers, then LDS), then the
    // rest; reduce once they are in.
    uint4 v[kHoldRegs][2];
#pragma unroll
    for (uint32_t s = 0; s < kHoldRegs; ++s) {
        if (s * t32 < lim) {
            const uint4* p = reinterpret_cast<const uint4*>(xc + (off0 + s * t32 * 32u));
            v[s][0] = p[0];
            v[s][1] = p[1];
        }
    }
    {
        const int64_t xbytes = groups * 32;
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(xc), (short)0, (int)(xbytes < 0xffffffffll ? xbytes : 0xffffffffll),
            (int)kBufferWord3);
        const int wave = tid / 64;
#pragma unroll
        for (uint32_t s = 0; s < kHoldLds; ++s) {
            if ((kHoldRegs + s) * t32 < lim) {
                const uint32_t o = off0 + (kHoldRegs + s) * t32 * 32u;
                dma16(rx, &held[s][0][wave * 64], o);
                dma16(rx, &held[s][1][wave * 64], o + 16u);
            }
        }
    }
    float m = 0.f;
    for (int64_t s = kHoldRegs + kHoldLds; s < steps; ++s) {
        const int64_t g = s * T + g0;
        if (g < groups) {
            uint4 w[2];
            load16(x + g * kGroup, w);
            m = fmaxf(m, absmax16(w));
        }
    }
#pragma unroll
    for (uint32_t s = 0; s < kHoldRegs; ++s)
        if (s * t32 < lim) m = fmaxf(m, absmax16(v[s]));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the LDS loads (each lane reads its own)
#pragma unroll
    for (uint32_t s = 0; s < kHoldLds; ++s) {
        if ((kHoldRegs + s) * t32 < lim) {
            const uint4 w[2] = {held[s][0][tid], held[s][1][tid]};
            m = fmaxf(m, absmax16(w));
        }
    }
    m = block_max_w<kOneWaves>(m, red);

    // Count in.  The maximum goes out as ~bits (never 0: the maximum is not
    // NaN) without waiting for it to land; the last to arrive waits for every
    // word to be nonzero, makes the scale, and hands it out.
    if (tid == 0) {
        ws_store(ws + kWsPartial + blockIdx.x, ~__float_as_uint(m));
        s_last = __hip_atomic_fetch_add(ws, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 gridDim.x - 1;
    }
    __syncthreads();
    const bool last = s_last != 0;
    uint32_t was = 0u;   // the last to arrive: what workgroup tid's word held
    if (last) {
        float a = 0.f;
        int missing = 0;
        if (tid < (int)gridDim.x) {
            // Every count is in, so every maximum has been stored; one still
            // in flight lands within a memory round trip.  (Bounded all the
            // same: should one never land, the scale is NaN and every code
            // NaN, rather than a wrong scale.)
            uint32_t* pw = ws + kWsPartial + tid;
            uint32_t w = ws_load(pw);
            for (uint32_t polls = 0; w == 0u && polls < kMaxPolls; ++polls) {
                __builtin_amdgcn_s_sleep(1);
                w = ws_load(pw);
            }
            missing = w == 0u;
            a = __uint_as_float(~w);
            ws_store(pw, 0u);
        }
        float sc = block_max_w<kOneWaves>(a, red) / Fp8Fmt<FMT>::kMax;
        if (__syncthreads_or(missing)) sc = __uint_as_float(0x7fc00000u);
        if (tid < (int)gridDim.x && tid != (int)blockIdx.x)   // (its own word stays 0)
            was = __hip_atomic_exchange(ws + kWsGo + kGoStride * tid, ~__float_as_uint(sc),
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) {
            ws_store(ws, 0u);   // every count is in
            s_scale = sc;
            s_gave = 0;
        }
    } else if (tid == 0) {
        // Wait for this workgroup's word (bounded by the clock and, should it
        // not advance, by the number of polls, each about 500 cycles apart).
        int gave_up = 0;
        const uint64_t t0 = wall_clock64();
        uint32_t w = ws_load(go);
        for (uint32_t polls = 0; w == 0u; ++polls) {
            if ((int64_t)(wall_clock64() - t0) >= wait_ticks || polls >= kMaxPolls) {
                w = __hip_atomic_exchange(go, kGaveUp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (w == 0u) {
                    gave_up = 1;          // claimed: the share is left to the last to arrive
                } else {
                    ws_store(go, 0u);     // the scale came first: undo the claim
                }
                break;
            }
            __builtin_amdgcn_s_sleep(8);
            w = ws_load(go);
        }
        if (!gave_up) ws_store(go, 0u);
        s_scale = __uint_as_float(~w);
        s_gave = gave_up;
    }
    __syncthreads();
    if (s_gave) return;
    const float sc = s_scale;
    if (blockIdx.x == 0 && tid == 0) scale[0] = sc;

    // Pass 2: convert what is held, re-read the rest (the first re-read step
    // is loaded before the LDS-held steps are converted, once the registers
    // of the others are free).
    const Div d = make_div(sc);
#pragma unroll
    for (uint32_t k = 0; k < kHoldRegs; ++k)
        if (k * t32 < lim) held_store(k, quant16<FMT>(v[k], d));
    int64_t s = kHoldRegs + kHoldLds;
    uint4 nx[2];
    if (s < steps && s * T + g0 < groups) load16(x + (s * T + g0) * kGroup, nx);
#pragma unroll
    for (uint32_t k = 0; k < kHoldLds; ++k) {
        if ((kHoldRegs + k) * t32 < lim) {
            const uint4 w[2] = {held[k][0][tid], held[k][1][tid]};
            held_store(kHoldRegs + k, quant16<FMT>(w, d));
        }
    }
    for (; s < steps; ++s) {
        const int64_t g = s * T + g0;
        if (g < groups) {
            const uint4 w[2] = {nx[0], nx[1]};
            const int64_t gn = g + T;
            if (gn < groups) load16(x + gn * kGroup, nx);
            *reinterpret_cast<uint4*>(q + g * kGroup) = quant16<FMT>(w, d);
        }
    }
    if (!last) return;

    // The last to arrive: convert the shares left to it, and set their words
    // back to zero.
    if (tid < (int)gridDim.x) left[tid] = was == kGaveUp;
    if (__syncthreads_or(was == kGaveUp)) {
        for (uint32_t b = 0; b < gridDim.x; ++b) {
            if (!left[b]) continue;
            if (b == 0 && tid == 0) scale[0] = sc;
            for (int64_t g = b * (int64_t)kOneThreads + tid; g < groups; g += T) {
                uint4 w[2];
                load16(x + g * kGroup, w);
                *reinterpret_cast<uint4*>(q + g * kGroup) = quant16<FMT>(w, d);
            }
        }
        if (tid < (int)gridDim.x && was == kGaveUp) ws_store(ws + kWsGo + kGoStride * tid, 0u);
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

// Ticks of the device's wall clock in `us` microseconds (0 if unknown).
int64_t wait_ticks(int64_t us) {
    int dev = -1, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return 0;
    return us * (int64_t)khz / 1000;
}

template <int FMT>
int quantize_impl(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                  int scaling_mode, void* workspace, int64_t workspace_bytes,
                  struct ihipStream_t* stream) {
    if (scaling_mode != FP8Q_PER_TENSOR && scaling_mode != FP8Q_ROWWISE) return FP8Q_ERR_MODE;
    if (rows < 0 || cols < 0 || cols % kGroup != 0 || cols > (int64_t(1) << 31) ||
        rows > (int64_t(1) << 31))
        return FP8Q_ERR_SHAPE;
    const bool empty = rows == 0 || cols == 0;
    const int64_t n_scales = scaling_mode == FP8Q_PER_TENSOR ? 1 : rows;
    if ((n_scales > 0 && !scale) || (!empty && (!x || !q))) return FP8Q_ERR_NULL;
    if ((uintptr_t)scale & 3) return FP8Q_ERR_ALIGN;
    if (!empty && (!aligned16(x) || !aligned16(q))) return FP8Q_ERR_ALIGN;
    if (workspace && ((uintptr_t)workspace & 3)) return FP8Q_ERR_ALIGN;
    const bool onepass = workspace && !empty && scaling_mode == FP8Q_PER_TENSOR;
    if (onepass && workspace_bytes < kOneWorkspaceBytes) return FP8Q_ERR_WORKSPACE;
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
    } else if (onepass && rows * cols / kGroup >= kOnePassMinSteps * (int64_t)(cus < kOneMaxGrid ? cus : kOneMaxGrid) *
                                                   kOneThreads) {
        const int64_t groups = rows * cols / kGroup;
        const int64_t want = (groups + kOneThreads - 1) / kOneThreads;
        const int64_t cap = cus < kOneMaxGrid ? cus : kOneMaxGrid;
        const unsigned grid = (unsigned)(want < cap ? want : cap);
        const int64_t ticks = wait_ticks(g_wait_us);
        uint32_t* ws = static_cast<uint32_t*>(workspace);
        hipLaunchKernelGGL(quant_tensor_onepass_kernel<FMT>, dim3(grid), dim3(kOneThreads), 0, hs, xb, qb,
                           scale, groups, ws, ticks);
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
    return quantize_impl<0>(x, q, scale, rows, cols, scaling_mode, nullptr, 0, stream);
}

int fp8_quantize_e5m2(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                      int scaling_mode, struct ihipStream_t* stream) {
    return quantize_impl<1>(x, q, scale, rows, cols, scaling_mode, nullptr, 0, stream);
}

int64_t fp8_quantize_workspace_size(int64_t rows, int64_t cols, int scaling_mode) {
    if (scaling_mode != FP8Q_PER_TENSOR || rows <= 0 || cols <= 0) return 0;
    return kOneWorkspaceBytes;
}

int fp8_quantize_e4m3_ws(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                         int scaling_mode, void* workspace, int64_t workspace_bytes,
                         struct ihipStream_t* stream) {
    return quantize_impl<0>(x, q, scale, rows, cols, scaling_mode, workspace, workspace_bytes, stream);
}

int fp8_quantize_e5m2_ws(const void* x, void* q, float* scale, int64_t rows, int64_t cols,
                         int scaling_mode, void* workspace, int64_t workspace_bytes,
                         struct ihipStream_t* stream) {
    return quantize_impl<1>(x, q, scale, rows, cols, scaling_mode, workspace, workspace_bytes, stream);
}

int64_t fp8_quantize_set_wait_limit_us(int64_t us) {
    const int64_t before = g_wait_us;
    g_wait_us = us < 0 ? kWaitUsDefault : us;
    return before;
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
        case FP8Q_ERR_WORKSPACE: return "workspace smaller than fp8_quantize_workspace_size()";
        default: return "unknown status";
    }
}

}  // extern "C"
