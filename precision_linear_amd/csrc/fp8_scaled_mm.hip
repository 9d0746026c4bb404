// FP8 (e4m3fn) scaled matrix multiply for gfx950 (MI355X, CDNA4).
//
//   out[m][n] = bf16_rne( s[m][n] * sum_k A[m][k] * B[n][k] (+ bias[n]) )
//
// Semantics: the gist "matmul_fp8.py" (a-r-r-o-w), `matmul_fp8_kernel`
// (fp32 accumulation over K, one multiply by the scale after the K loop, then
// the cast to the output type); row-wise scales and the TN operand layout from
// pytorch PR #125204, Summary; the bias epilogue from PR #142045, Summary.
//
// Structure of one launch (all of it gfx950-specific):
//   * Persistent grid: at most one workgroup per CU walks the output tiles in
//     grouped order (GROUP_M tile rows per band, the L2-reuse order the gist
//     cites from the Triton matmul tutorial), with workgroup ids renumbered so
//     that the workgroups of one XCD take neighbouring tiles and share that
//     XCD's L2.
//   * Staging: A and B K-slices go global -> LDS with 16-byte buffer loads that
//     write LDS directly (no VGPR round trip).  Rows outside the matrix and the
//     K tail read as zero: the buffer's record limit covers the rows, and K-tail
//     chunks get an offset past that limit.  The 16-byte chunks of each LDS row
//     are XOR-permuted by row so that the MFMA operand reads hit distinct banks.
//     STAGES buffers rotate so the loads for later K slices run under the MFMAs.
//   * Inner loop: v_mfma_f32_32x32x64_f8f6f4 (or 16x16x128) with e4m3 operands
//     and fp32 accumulators held in registers for the whole K loop.
//   * Epilogue: scale (fp32 sa*sb in both modes), optional bias, RNE to bf16,
//     stores of 4 consecutive bf16 per lane (8 bytes) where the row allows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8_scaled_mm.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWave = 64;
constexpr uint32_t kBufferWord3 = 0x00020000u;   // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;    // any offset >= num_records reads zero
constexpr int kXcds = 8;                         // gfx950: 8 XCDs, round-robin dispatch

struct Params {
    const uint8_t* A;
    const uint8_t* B;
    const float* scale_a;
    const float* scale_b;
    const uint16_t* bias;  // may be null
    uint16_t* out;
    int M, N, K;
    int tiles_m, tiles_n, num_tiles, k_iters;
    int rowwise;
    int vec_store;         // N % 4 == 0 and out 8-byte aligned
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)kBufferWord3);
}

// fp32 -> bf16, round to nearest even; NaN -> quiet NaN with the sign kept.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

template <int CPR>
__device__ __forceinline__ int chunk_swizzle(int r) {
    // CPR = 16-byte chunks per LDS row (a power of two).  Consecutive rows get
    // distinct XOR masks over every aligned run of CPR rows.
    constexpr int LOG = CPR == 4 ? 2 : CPR == 8 ? 3 : CPR == 16 ? 4 : 5;
    return (r ^ (r >> LOG)) & (CPR - 1);
}

template <int MI>
struct Mfma;

template <>
struct Mfma<32> {
    static constexpr int KSTEP = 64;      // bytes of K per instruction
    typedef v16f acc_t;
    static constexpr int NACC = 16;
    __device__ static __forceinline__ acc_t run(v8i a, v8i b, acc_t c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

template <>
struct Mfma<16> {
    static constexpr int KSTEP = 128;
    typedef v4f acc_t;
    static constexpr int NACC = 4;
    __device__ static __forceinline__ acc_t run(v8i a, v8i b, acc_t c) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    }
};

__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int group_m,
                                            int& pm, int& pn) {
    // Bands of group_m tile rows; inside a band, tiles go down the band's rows
    // first, then across the columns.
    const int band = group_m * tiles_n;
    const int g = t / band;
    const int first = g * group_m;
    const int rows = min(tiles_m - first, group_m);
    const int w = t - g * band;
    pm = first + w % rows;
    pn = w / rows;
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int MI, int GROUP_M>
struct Cfg {
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = WAVES * kWave;
    static constexpr int WTM = BM / WAVES_M;     // wave tile rows (m)
    static constexpr int WTN = BN / WAVES_N;     // wave tile cols (n)
    static constexpr int FM = WTM / MI;
    static constexpr int FN = WTN / MI;
    static constexpr int CPR = BK / 16;          // 16-byte chunks per LDS row
    static constexpr int A_BYTES = BM * BK;
    static constexpr int B_BYTES = BN * BK;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static constexpr int A_BLOCKS = A_BYTES / 1024;  // 1 KiB = one wave-wide 16-byte load
    static constexpr int B_BLOCKS = B_BYTES / 1024;
    static constexpr int A_LOADS = A_BLOCKS / WAVES; // per wave per stage
    static constexpr int B_LOADS = B_BLOCKS / WAVES;
    static constexpr int LOADS = A_LOADS + B_LOADS;
    static constexpr int KSTEP = Mfma<MI>::KSTEP;
    static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile must hold whole MFMA tiles");
    static_assert(BK % KSTEP == 0, "BK must be a multiple of the MFMA K step");
    static_assert(CPR == 4 || CPR == 8 || CPR == 16 || CPR == 32, "BK must be 64..512");
    static_assert(A_BLOCKS % WAVES == 0 && B_BLOCKS % WAVES == 0, "loads must split evenly");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS is 160 KiB per workgroup");
    static_assert(STAGES >= 2, "at least double buffering");
    static_assert(LOADS * (STAGES - 1) <= 63, "vmcnt counts up to 63");
};

// Issue the direct-to-LDS loads of one K slice (k0) for this wave.
template <class C>
__device__ __forceinline__ void load_stage(uint8_t* lds_stage, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, int K, int k0, int wave,
                                           int lane) {
    constexpr int RPB = 1024 / (C::CPR * 16);    // LDS rows per 1 KiB block
    const int rr = lane / C::CPR;
    const int pos = lane % C::CPR;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
        const int blk = wave + i * C::WAVES;
        const int r = blk * RPB + rr;
        const int c = pos ^ chunk_swizzle<C::CPR>(r);
        const int k = k0 + c * 16;
        const uint32_t off = k < K ? (uint32_t)(r * K + k) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            ra, (lds_void_t*)(lds_stage + blk * 1024), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
        const int blk = wave + i * C::WAVES;
        const int r = blk * RPB + rr;
        const int c = pos ^ chunk_swizzle<C::CPR>(r);
        const int k = k0 + c * 16;
        const uint32_t off = k < K ? (uint32_t)(r * K + k) : kOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rb, (lds_void_t*)(lds_stage + C::A_BYTES + blk * 1024), 16, off, 0, 0, 0);
    }
}

// 32 operand bytes for one MFMA: row `r` of an LDS operand tile, logical
// chunks c0 and c0+1.
template <int CPR>
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int r, int c0) {
    const int sw = chunk_swizzle<CPR>(r);
    const uint8_t* row = tile + r * (CPR * 16);
    v4i lo = *reinterpret_cast<const v4i*>(row + ((c0 ^ sw) << 4));
    v4i hi = *reinterpret_cast<const v4i*>(row + (((c0 + 1) ^ sw) << 4));
    v8i f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    return f;
}

// Workgroup barrier without the memory-model fence of __syncthreads(): the
// waits it needs (LDS reads done, own LDS-DMA loads landed) are explicit.
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt untouched
    __builtin_amdgcn_s_barrier();
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt encoding on gfx9: vmcnt low bits [3:0], high bits [15:14];
    // expcnt [6:4] and lgkmcnt [11:8] left at their maxima (no wait).
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int MI, int GROUP_M>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * kWave)
fp8_gemm_kernel(Params p) {
    using C = Cfg<BM, BN, BK, WAVES_M, WAVES_N, STAGES, MI, GROUP_M>;
    using F = Mfma<MI>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int wm = wave / WAVES_N;
    const int wn = wave % WAVES_N;

    // Renumber workgroups so that the ones on one XCD get consecutive ids.
    const int G = gridDim.x;
    int wg = blockIdx.x;
    if (G % kXcds == 0) wg = (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds;

    const float s_pt = p.rowwise ? 0.f : p.scale_a[0] * p.scale_b[0];

    for (int t = wg; t < p.num_tiles; t += G) {
        int pm, pn;
        tile_coords(t, p.tiles_m, p.tiles_n, GROUP_M, pm, pn);
        const int row0 = pm * BM;
        const int col0 = pn * BN;
        const uint32_t rows_a = (uint32_t)min(BM, p.M - row0);
        const uint32_t rows_b = (uint32_t)min(BN, p.N - col0);
        const __amdgpu_buffer_rsrc_t ra =
            make_rsrc(p.A + (size_t)row0 * p.K, rows_a * (uint32_t)p.K);
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(p.B + (size_t)col0 * p.K, rows_b * (uint32_t)p.K);

        typename F::acc_t acc[C::FN][C::FM];
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
            for (int j = 0; j < C::FM; ++j)
#pragma unroll
                for (int v = 0; v < F::NACC; ++v) acc[i][j][v] = 0.f;

        // Every wave must be done with the LDS of the previous tile (and its
        // own epilogue stores must have left) before this tile's loads start.
        wait_vmcnt<0>();
        barrier_lds();
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s)
            if (s < p.k_iters) load_stage<C>(smem + s * C::STAGE_BYTES, ra, rb, p.K, s * BK, wave, lane);

        for (int kt = 0; kt < p.k_iters; ++kt) {
            // Stage kt is complete once at most (loads issued after it) remain.
            if (kt + STAGES - 2 < p.k_iters) wait_vmcnt<C::LOADS * (STAGES - 2)>();
            else wait_vmcnt<0>();
            barrier_lds();
            const int nk = kt + STAGES - 1;
            if (nk < p.k_iters)
                load_stage<C>(smem + (nk % STAGES) * C::STAGE_BYTES, ra, rb, p.K, nk * BK, wave,
                              lane);
            const uint8_t* sa_t = smem + (kt % STAGES) * C::STAGE_BYTES;
            const uint8_t* sb_t = sa_t + C::A_BYTES;
#pragma unroll
            for (int ks = 0; ks < BK / C::KSTEP; ++ks) {
                // operand k chunks: MI=32 -> lanes 0-31 chunks {0,1}, 32-63 {2,3};
                // MI=16 -> four lane groups of 16 take chunk pairs 0..3.
                const int c0 = ks * (C::KSTEP / 16) + (lane / MI) * 2;
                v8i af[C::FM], bfr[C::FN];
#pragma unroll
                for (int j = 0; j < C::FM; ++j)
                    af[j] = read_frag<C::CPR>(sa_t, wm * C::WTM + j * MI + lane % MI, c0);
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
                    bfr[i] = read_frag<C::CPR>(sb_t, wn * C::WTN + i * MI + lane % MI, c0);
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
#pragma unroll
                    for (int j = 0; j < C::FM; ++j) acc[i][j] = F::run(bfr[i], af[j], acc[i][j]);
            }
        }

        // Epilogue.  The MFMA was fed B as its first operand, so lane l holds
        // output row m = l % MI of each sub-tile and runs of 4 consecutive
        // columns n.
#pragma unroll
        for (int j = 0; j < C::FM; ++j) {
            const int m = row0 + wm * C::WTM + j * MI + lane % MI;
            if (m >= p.M) continue;
            const float sa_m = p.rowwise ? p.scale_a[m] : 0.f;
            uint16_t* orow = p.out + (size_t)m * p.N;
#pragma unroll
            for (int i = 0; i < C::FN; ++i) {
#pragma unroll
                for (int g = 0; g < F::NACC / 4; ++g) {
                    const int n = col0 + wn * C::WTN + i * MI +
                                  (MI == 32 ? 8 * g + 4 * (lane / 32) : 4 * (lane / 16));
                    if (n >= p.N) continue;
                    uint32_t h[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int nc = min(n + c, p.N - 1);
                        const float s = p.rowwise ? sa_m * p.scale_b[nc] : s_pt;
                        float y = acc[i][j][4 * g + c];
                        if (p.bias) {
                            const float b = __uint_as_float((uint32_t)p.bias[nc] << 16);
                            y = __builtin_fmaf(y, s, b);
                        } else {
                            y = y * s;
                        }
                        h[c] = f32_to_bf16_rne(y);
                    }
                    if (p.vec_store && n + 3 < p.N) {
                        uint2 w;
                        w.x = h[0] | (h[1] << 16);
                        w.y = h[2] | (h[3] << 16);
                        *reinterpret_cast<uint2*>(orow + n) = w;
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            if (n + c < p.N) orow[n + c] = (uint16_t)h[c];
                    }
                }
            }
        }
    }
}

// ------------------------------------------------------------------ host ---

struct ConfigInfo {
    const char* name;
    int bm, bn, bk;
    int threads;
    int lds_bytes;
    int occupancy;   // workgroups per CU the persistent grid assumes
    void (*launch)(const Params&, dim3, hipStream_t);
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int MI, int GROUP_M>
void launch_cfg(const Params& p, dim3 grid, hipStream_t stream) {
    using C = Cfg<BM, BN, BK, WAVES_M, WAVES_N, STAGES, MI, GROUP_M>;
    hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, BK, WAVES_M, WAVES_N, STAGES, MI, GROUP_M>), grid,
                       dim3(C::THREADS), 0, stream, p);
}

#define FP8MM_CFG(name, BM, BN, BK, WMW, WNW, ST, MI, GM)                                      \
    ConfigInfo {                                                                               \
        name, BM, BN, BK, Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::THREADS,                          \
            Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::LDS_BYTES, 1,                               \
            &launch_cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>                                      \
    }

const ConfigInfo kConfigs[] = {
    FP8MM_CFG("bm256_bn256_bk128_w2x2_s2_mfma32", 256, 256, 128, 2, 2, 2, 32, 8),
    FP8MM_CFG("bm128_bn128_bk128_w2x2_s3_mfma32", 128, 128, 128, 2, 2, 3, 32, 8),
    FP8MM_CFG("bm32_bn64_bk256_w1x2_s4_mfma32", 32, 64, 256, 1, 2, 4, 32, 8),
    FP8MM_CFG("bm16_bn64_bk256_w1x4_s4_mfma16", 16, 64, 256, 1, 4, 4, 16, 8),
};
constexpr int kNumConfigs = sizeof(kConfigs) / sizeof(kConfigs[0]);

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int choose_config(int64_t M, int64_t N, int64_t K, int mode, int has_bias) {
    (void)K; (void)mode; (void)has_bias;
    if (M <= 16) return 3;
    if (M <= 64) return 2;
    const int64_t big_tiles = cdiv(M, 256) * cdiv(N, 256);
    if (big_tiles >= 256) return 0;
    return 1;
}

int device_cus(int dev) {
    // Per-device compute-unit count, read once.
    static int cache[64] = {0};
    if (dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        __atomic_store_n(&cache[dev], cus, __ATOMIC_RELAXED);
    }
    return __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int validate(const void* A, const void* B, const float* sa, const float* sb, const void* bias,
             void* out, int64_t M, int64_t N, int64_t K, int mode) {
    if (mode != FP8MM_PER_TENSOR && mode != FP8MM_ROWWISE) return FP8MM_ERR_MODE;
    if (M < 0 || N < 0 || M > INT32_MAX || N > INT32_MAX) return FP8MM_ERR_SHAPE;
    if (K < 16 || K > (int64_t(1) << 23) || K % 16 != 0) return FP8MM_ERR_SHAPE;
    if (M == 0 || N == 0) return FP8MM_OK;  // empty output: nothing is read or written
    if (!A || !B || !sa || !sb || !out) return FP8MM_ERR_NULL;
    if (!aligned(A, 16) || !aligned(B, 16)) return FP8MM_ERR_ALIGN;
    if (!aligned(sa, 4) || !aligned(sb, 4)) return FP8MM_ERR_ALIGN;
    if (!aligned(out, 2) || (bias && !aligned(bias, 2))) return FP8MM_ERR_ALIGN;
    return FP8MM_OK;
}

int64_t grid_for(int cfg, int64_t M, int64_t N, int cus) {
    const ConfigInfo& c = kConfigs[cfg];
    const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
    const int64_t slots = (int64_t)cus * c.occupancy;
    return tiles < slots ? tiles : slots;
}

}  // namespace

extern "C" {

int fp8_scaled_mm_num_configs(void) { return kNumConfigs; }

const char* fp8_scaled_mm_config_name(int id) {
    return (id >= 0 && id < kNumConfigs) ? kConfigs[id].name : "";
}

int fp8_scaled_mm_select_config(int64_t M, int64_t N, int64_t K, int mode, int has_bias) {
    if (mode != FP8MM_PER_TENSOR && mode != FP8MM_ROWWISE) return -1;
    if (M < 0 || N < 0 || K < 16 || K % 16 != 0) return -1;
    return choose_config(M, N, K, mode, has_bias);
}

int64_t fp8_scaled_mm_grid_size(int id, int64_t M, int64_t N, int num_cus) {
    if (id < 0 || id >= kNumConfigs || M <= 0 || N <= 0 || num_cus <= 0) return 0;
    return grid_for(id, M, N, num_cus);
}

const char* fp8_scaled_mm_status_string(int s) {
    switch (s) {
        case FP8MM_OK: return "ok";
        case FP8MM_ERR_NULL: return "a required pointer is NULL";
        case FP8MM_ERR_SHAPE: return "M, N or K out of range (need 0<=M,N<2^31, 16<=K<=2^23, K%16==0)";
        case FP8MM_ERR_ALIGN: return "misaligned pointer (A,B: 16 B; scales: 4 B; bias,out: 2 B)";
        case FP8MM_ERR_MODE: return "unknown scaling mode";
        case FP8MM_ERR_DEVICE: return "no usable gfx950 device";
        case FP8MM_ERR_LAUNCH: return "kernel launch failed";
        case FP8MM_ERR_CONFIG: return "unknown tile configuration";
        default: return "unknown status";
    }
}

int fp8_scaled_mm_with_config(const void* A, const void* B, const float* scale_a,
                              const float* scale_b, const void* bias, void* out, int64_t M,
                              int64_t N, int64_t K, int mode, struct ihipStream_t* stream,
                              int config_id) {
    int st = validate(A, B, scale_a, scale_b, bias, out, M, N, K, mode);
    if (st != FP8MM_OK) return st;
    if (config_id >= kNumConfigs) return FP8MM_ERR_CONFIG;
    if (M == 0 || N == 0) return FP8MM_OK;
    const int cfg = config_id >= 0 ? config_id : choose_config(M, N, K, mode, bias != nullptr);

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FP8MM_ERR_DEVICE;
    const int cus = device_cus(dev);
    if (cus <= 0) return FP8MM_ERR_DEVICE;

    Params p;
    p.A = static_cast<const uint8_t*>(A);
    p.B = static_cast<const uint8_t*>(B);
    p.scale_a = scale_a;
    p.scale_b = scale_b;
    p.bias = static_cast<const uint16_t*>(bias);
    p.out = static_cast<uint16_t*>(out);
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    const ConfigInfo& c = kConfigs[cfg];
    p.tiles_m = (int)cdiv(M, c.bm);
    p.tiles_n = (int)cdiv(N, c.bn);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    if (tiles > INT32_MAX) return FP8MM_ERR_SHAPE;
    p.num_tiles = (int)tiles;
    p.k_iters = (int)cdiv(K, c.bk);
    p.rowwise = mode == FP8MM_ROWWISE;
    p.vec_store = (N % 4 == 0) && aligned(out, 8);

    const dim3 grid((unsigned)grid_for(cfg, M, N, cus));
    (void)hipGetLastError();  // clear a stale error from earlier, unrelated calls
    c.launch(p, grid, reinterpret_cast<hipStream_t>(stream));
    if (hipGetLastError() != hipSuccess) return FP8MM_ERR_LAUNCH;
    return FP8MM_OK;
}

int fp8_scaled_mm(const void* A, const void* B, const float* scale_a, const float* scale_b,
                  const void* bias, void* out, int64_t M, int64_t N, int64_t K, int mode,
                  struct ihipStream_t* stream) {
    return fp8_scaled_mm_with_config(A, B, scale_a, scale_b, bias, out, M, N, K, mode, stream, -1);
}

}  // extern "C"
