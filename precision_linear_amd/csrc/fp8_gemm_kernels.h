// FP8 (e4m3fn / e5m2) scaled matrix multiply for gfx950 (MI355X, CDNA4): the kernels.
//
//   out[m][n] = bf16_rne( s[m][n] * sum_k A[m][k] * B[n][k] (+ bias[n]) )
//
// Semantics: the gist "matmul_fp8.py" (a-r-r-o-w), `matmul_fp8_kernel`
// (fp32 accumulation over K, one multiply by the scale after the K loop, then
// the cast to the output type); row-wise scales and the TN operand layout from
// pytorch PR #125204, Summary; the bias epilogue from PR #142045, Summary.
//
// Structure of one launch (all of it gfx950-specific):
//   * Persistent grid: one workgroup per CU (two where the tile's LDS allows)
//     walks the output tiles in grouped order (GROUP_M tile rows per band, the
//     L2-reuse order the gist cites from the Triton matmul tutorial), with
//     workgroup ids renumbered so that the workgroups of one XCD take
//     neighbouring tiles and share that XCD's L2.
//   * Staging: A and B K-slices go global -> LDS with 16-byte buffer loads that
//     write LDS directly (no VGPR round trip).  Rows outside the matrix and the
//     K tail read as zero: the buffer's record limit covers the rows, and K-tail
//     chunks get an offset past that limit.  The 16-byte chunks of each LDS row
//     are XOR-permuted by row so that the MFMA operand reads hit distinct banks.
//     STAGES buffers rotate so the loads for later K slices run under the MFMAs.
//   * Inner loop: v_mfma_f32_16x16x128_f8f6f4 (ping-pong kernel, skinny and
//     narrow tiles) or 32x32x64 (the other tiles) with e4m3 / e5m2 operands and
//     fp32 accumulators held in registers for the whole K loop.
//   * Epilogue: scale (fp32 sa*sb in both modes), optional bias, RNE to bf16,
//     then the bf16 tile goes through LDS so that the stores to the output
//     write whole runs of its rows (16, 4 or 2 bytes per lane, as wide as the
//     row alignment allows).
//
// This header holds the device code and the launch wrappers.  Each operand
// format pair is instantiated in a translation unit of its own
// (fp8_gemm_f<k>.hip, which only expands FP8MM_DEFINE_LAUNCH_TABLE), so the
// four compile in parallel; fp8_scaled_mm.hip holds the host logic and the
// C ABI and reaches the kernels through those launch tables.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8mm {

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
    int vec16;             // N % 8 == 0 and out 16-byte aligned
    // Split-K: each output tile is computed by `splits` work units, unit s
    // covering K slices [s*k_chunk, (s+1)*k_chunk).  With splits > 1 the fp32
    // partial tiles go to `partials` and the unit that arrives last at the
    // tile's counter adds them up in split order and runs the epilogue.
    int splits, k_chunk;
    float* partials;       // num_tiles * splits * BM * BN floats (splits > 1)
    unsigned* counters;    // num_tiles arrival counters (splits > 1)
    // Stream-K (the generic kernel's SK instantiation): the num_tiles * k_iters
    // (tile, K slice) iterations, tile-major, are cut into gridDim.x equal
    // ranges, workgroup w taking [w * total / G, (w + 1) * total / G); a tile
    // is finished by the one workgroup that covers it whole, or by the
    // segments (the workgroups whose ranges meet it) through partials and
    // counters as in split-K, `splits` then being the room per tile for
    // segments (an upper bound on their number).
};

typedef void (*Launch)(const Params&, dim3, hipStream_t);
struct LaunchPair {
    Launch plain;
    // The same tiles with B loaded non-temporally, for grids with a single row
    // of tiles (B is then read once); null where not compiled.
    Launch stream;
    // The stream-K form (Cfg::STREAM_K_OK configurations only, else null).
    Launch stream_k;
};

// Operand formats, as a kernel template parameter FMT: bit 0 set = A is e5m2,
// bit 1 set = B is e5m2 (else e4m3fn).
constexpr int kFormats = 4;

// The generic kernel's tile configurations, in config-id order:
// X(name, BM, BN, BK, WAVES_M, WAVES_N, STAGES, MFMA size, GROUP_M); the
// ping-pong kernel follows them (id kPingPongId).
//   * few rows (M <= 16, 64, 128) and many columns: tiles as tall as M, 112
//     or 64 wide, or 128 x 128, streaming B from HBM;
//   * few rows and few columns (a column shard of a skinny problem): narrow
//     tiles, split over K (the last unit of a tile reads every partial, so
//     smaller tiles make that fix-up cheaper) or, without a workspace, enough
//     of them to fill the CUs;
//   * 128 x 128 on 8 waves (mid-size grids) and on 4 waves with two
//     workgroups per CU (one's output stores overlap the other's loads);
//   * 64 x 128 on 4 waves, three workgroups per CU: output-write-bound grids
//     (K of one slice) whose rows are not 16-byte aligned.
#define FP8MM_GENERIC_CONFIGS(X)                                                   \
    X("bm16_bn32_bk512_w1x2_s6_mfma16", 16, 32, 512, 1, 2, 6, 16, 8)               \
    X("bm16_bn64_bk256_w1x4_s4_mfma16", 16, 64, 256, 1, 4, 4, 16, 8)               \
    X("bm16_bn112_bk256_w1x7_s4_mfma16", 16, 112, 256, 1, 7, 4, 16, 8)             \
    X("bm64_bn32_bk256_w4x2_s4_mfma16", 64, 32, 256, 4, 2, 4, 16, 8)               \
    X("bm64_bn64_bk256_w1x4_s4_mfma16", 64, 64, 256, 1, 4, 4, 16, 8)               \
    X("bm64_bn112_bk256_w1x7_s3_mfma16", 64, 112, 256, 1, 7, 3, 16, 8)             \
    X("bm128_bn32_bk256_w4x2_s3_mfma16", 128, 32, 256, 4, 2, 3, 16, 8)             \
    X("bm128_bn64_bk256_w4x2_s3_mfma16", 128, 64, 256, 4, 2, 3, 16, 8)             \
    X("bm128_bn128_bk128_w2x4_s4_mfma32", 128, 128, 128, 2, 4, 4, 32, 8)           \
    X("bm128_bn128_bk128_w2x2_s2_mfma32", 128, 128, 128, 2, 2, 2, 32, 8)           \
    X("bm64_bn128_bk128_w2x2_s2_mfma32", 64, 128, 128, 2, 2, 2, 32, 8)
constexpr int kNumGenericConfigs = 11;
constexpr int kPingPongId = kNumGenericConfigs;
constexpr int kNumConfigs = kNumGenericConfigs + 1;

// One table per format pair, defined in fp8_gemm_f<k>.hip.  Not const: a
// const namespace-scope variable would also be emitted for the device, where
// host function addresses do not exist.
extern LaunchPair kLaunchF0[kNumConfigs];
extern LaunchPair kLaunchF1[kNumConfigs];
extern LaunchPair kLaunchF2[kNumConfigs];
extern LaunchPair kLaunchF3[kNumConfigs];

}  // namespace fp8mm

namespace {

using namespace fp8mm;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef v4i v4i_a2 __attribute__((aligned(2)));   // 16 bytes at any even LDS address
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWave = 64;
constexpr uint32_t kBufferWord3 = 0x00020000u;   // raw buffer, 32-bit data format (gfx9 family)
constexpr uint32_t kOutOfRange = 0x80000000u;    // any offset >= num_records reads zero
constexpr int kXcds = 8;                         // gfx950: 8 XCDs, round-robin dispatch



__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             (int)kBufferWord3);
}

// One 16-byte-per-lane buffer load that writes LDS directly: lane l's 16
// bytes from rsrc + voff + soff land at LDS byte address lds + 16*l (lds is
// wave-uniform and goes to M0).  Written as inline asm so that the compiler
// does not treat later LDS reads as dependent on it: every wait on these loads
// is an explicit vmcnt wait placed by the code that issues them.  NT marks the
// load non-temporal (data read once: it should not displace reused lines from
// the L2).
template <bool NT = false>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, const void* lds, uint32_t voff,
                                      uint32_t soff) {
    const uint32_t m0 = (uint32_t)(uintptr_t)lds;
    if constexpr (NT)
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds"
                     :
                     : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0)
                     : "memory");
    else
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                     :
                     : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0)
                     : "memory");
}

// Position of 16-byte chunk c of LDS row r is c ^ chunk_swizzle(r).  The MFMA
// operand reads have 8 (or 16) consecutive lanes read the same logical chunk
// of 8 (16) consecutive rows; the mask makes those land in distinct banks
// whether the LDS serves 128 or 256 bytes per cycle.  It uses row bits 0..3
// only, so every 16-row-aligned block of rows shares one pattern.
template <int CPR>
__device__ __forceinline__ int chunk_swizzle(int r) {
    if constexpr (CPR == 4) return ((r >> 1) ^ (r >> 2)) & 3;   // 4 rows per 256 B
    if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);    // 2 rows per 256 B
    return r & 15;                                              // >= 256-byte rows
}

// Operand formats, as a kernel template parameter FMT: bit 0 set = A is e5m2,
// bit 1 set = B is e5m2 (else e4m3fn).  The f8f6f4 MFMAs take the format of
// each source as an immediate (0 = e4m3, 1 = e5m2); the kernels feed the B
// fragment as the first source, so its format goes in the first selector.
template <int FMT> constexpr int fmt_src0() { return (FMT >> 1) & 1; }   // B
template <int FMT> constexpr int fmt_src1() { return FMT & 1; }          // A

template <int MI>
struct Mfma;

template <>
struct Mfma<32> {
    static constexpr int KSTEP = 64;      // bytes of K per instruction
    typedef v16f acc_t;
    static constexpr int NACC = 16;
    // c += b_frag^T-contracted-with a_frag: the output block's lane l holds row
    // l % 32 of B's fragment and columns from A's.
    template <int FMT>
    __device__ static __forceinline__ acc_t run(v8i b_frag, v8i a_frag, acc_t c) {
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b_frag, a_frag, c, fmt_src0<FMT>(),
                                                               fmt_src1<FMT>(), 0, 0, 0, 0);
    }
};

template <>
struct Mfma<16> {
    static constexpr int KSTEP = 128;
    typedef v4f acc_t;
    static constexpr int NACC = 4;
    template <int FMT>
    __device__ static __forceinline__ acc_t run(v8i b_frag, v8i a_frag, acc_t c) {
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b_frag, a_frag, c, fmt_src0<FMT>(),
                                                                fmt_src1<FMT>(), 0, 0, 0, 0);
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

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int MI, int GROUP_M,
          bool NT_B = false, int FMT_ = 0>
struct Cfg {
    static constexpr int FMT = FMT_;     // operand formats (see kFormats)
    // B is read by one tile row only (the grid has a single row of tiles):
    // its loads are marked non-temporal so that they do not evict A, which
    // every tile reads.
    static constexpr bool STREAM_B = NT_B;
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
    static constexpr int MAIN_BYTES = STAGES * STAGE_BYTES;
    // Epilogue parameters of the current tile: BM row scales, BN column
    // scales (fp32) and BN bias values (bf16).
    static constexpr int EPI_BYTES = BM * 4 + BN * 4 + BN * 2;
    static constexpr int LDS_BYTES = MAIN_BYTES + ((EPI_BYTES + 15) / 16) * 16;
    static constexpr int NSA = (BM + THREADS - 1) / THREADS;   // staged per thread
    static constexpr int NSB = (BN + THREADS - 1) / THREADS;
    static constexpr int A_BLOCKS = A_BYTES / 1024;  // 1 KiB = one wave-wide 16-byte load
    static constexpr int B_BLOCKS = B_BYTES / 1024;
    // Loads per wave per stage.  When the blocks do not split evenly over the
    // waves, the surplus loads repeat the last block: the same bytes land at
    // the same LDS address twice, and every wave keeps the same load count
    // (which the vmcnt arithmetic relies on).
    static constexpr int A_LOADS = (A_BLOCKS + WAVES - 1) / WAVES;
    static constexpr int B_LOADS = (B_BLOCKS + WAVES - 1) / WAVES;
    static constexpr int LOADS = A_LOADS + B_LOADS;
    static constexpr int KSTEP = Mfma<MI>::KSTEP;
    static constexpr int NKS = BK / KSTEP;        // MFMA K steps per stage
    static constexpr int MI_ = MI;
    // Split-K keeps a second copy of the accumulators while it sums the
    // partials, so it is compiled only where both fit in registers.
    static constexpr int PER_LANE_ACC = FM * FN * (MI == 32 ? 16 : 4);
    static constexpr bool SPLIT_OK = PER_LANE_ACC <= 64;
    // A stream-K form is compiled for the 128 x 128 tiles only (a second
    // instantiation of the kernel; the others would double the library for a
    // plan that measured slower on every workload here).
    static constexpr bool STREAM_K_OK = SPLIT_OK && BM == 128 && BN == 128;
    // Spread a stage's loads between MFMAs only where a K step has enough
    // MFMAs to hide them (the big, MFMA-bound tiles).
    static constexpr bool INTERLEAVE = MI == 32 && FM * FN >= 8;
    static constexpr int BK_ = BK;
    static constexpr int BM_ = BM;
    static constexpr int BN_ = BN;
    static constexpr int STAGES_ = STAGES;
    // The epilogue stages the finished bf16 tile (rows of BN * 2 bytes, whole
    // 16-byte chunks) in the stage buffers.
    static constexpr int STG_CHUNKS = BN * 2 / 16;
    static_assert(WTM % MI == 0 && WTN % MI == 0, "wave tile must hold whole MFMA tiles");
    static_assert(MI % 16 == 0, "fragment row blocks must be 16-row aligned for the swizzle");
    static_assert(BK % KSTEP == 0, "BK must be a multiple of the MFMA K step");
    static_assert(CPR == 4 || CPR == 8 || CPR == 16 || CPR == 32, "BK must be 64..512");
    static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "stages are whole 1 KiB blocks");
    static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS is 160 KiB per workgroup");
    // Workgroups per CU the persistent grid is sized for: as many as fit in
    // the 160 KiB of LDS, up to three (small tiles: one workgroup's output
    // stores then overlap another's loads).
    static constexpr int OCCUPANCY = LDS_BYTES * 3 <= 160 * 1024   ? 3
                                     : LDS_BYTES * 2 <= 160 * 1024 ? 2
                                                                   : 1;
    static_assert(STAGES >= 2, "at least double buffering");
    static_assert(BN % 8 == 0 && BM * (BN * 2 + 16) <= MAIN_BYTES,
                  "the output tile (with its padded rows) fits the stage buffers");
    static_assert(LOADS * (STAGES - 1) <= 63, "vmcnt counts up to 63");
};

// Issue the direct-to-LDS loads of one K slice (k0) for this wave.
template <class C>
__device__ __forceinline__ void load_stage(uint8_t* lds_stage, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, int ld, int klim, int k0,
                                           int wave, int lane) {
    constexpr int RPB = 1024 / (C::CPR * 16);    // LDS rows per 1 KiB block
    // The lane-dependent offsets are cheap to recompute; keeping them live
    // across the K loop would only cost registers the MFMA pipeline needs.
    int l = lane;
    asm volatile("" : "+v"(l));
    const int rr = l / C::CPR;
    const int pos = l % C::CPR;
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
        const int blk = min(wave + i * C::WAVES, C::A_BLOCKS - 1);
        const int r = blk * RPB + rr;
        const int c = pos ^ chunk_swizzle<C::CPR>(r);
        const int k = k0 + c * 16;
        const uint32_t off = k < klim ? (uint32_t)(r * ld + k) : kOutOfRange;
        dma16(ra, lds_stage + blk * 1024, off, 0);
    }
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
        const int blk = min(wave + i * C::WAVES, C::B_BLOCKS - 1);
        const int r = blk * RPB + rr;
        const int c = pos ^ chunk_swizzle<C::CPR>(r);
        const int k = k0 + c * 16;
        const uint32_t off = k < klim ? (uint32_t)(r * ld + k) : kOutOfRange;
        dma16<C::STREAM_B>(rb, lds_stage + C::A_BYTES + blk * 1024, off, 0);
    }
}

// Load number `idx` (0 <= idx < LOADS) of this wave for one K slice: the
// first A_LOADS go to the A tile, the rest to the B tile.  With live == false
// every lane reads out of range (zeros land in a buffer nobody reads again);
// this keeps the number of loads per stage fixed, which the vmcnt waits use.
template <class C, int idx>
__device__ __forceinline__ void load_one(uint8_t* lds_stage, __amdgpu_buffer_rsrc_t ra,
                                         __amdgpu_buffer_rsrc_t rb, int ld, int klim, int k0,
                                         int wave, int l, bool live) {
    constexpr int RPB = 1024 / (C::CPR * 16);
    constexpr bool IS_A = idx < C::A_LOADS;
    constexpr int i = IS_A ? idx : idx - C::A_LOADS;
    const int blk = min(wave + i * C::WAVES, (IS_A ? C::A_BLOCKS : C::B_BLOCKS) - 1);
    const int rr = l / C::CPR;
    const int pos = l % C::CPR;
    const int r = blk * RPB + rr;
    const int c = pos ^ chunk_swizzle<C::CPR>(r);
    const int k = k0 + c * 16;
    const uint32_t off = (live && k < klim) ? (uint32_t)(r * ld + k) : kOutOfRange;
    if constexpr (IS_A)
        dma16(ra, lds_stage + blk * 1024, off, 0);
    else
        dma16<C::STREAM_B>(rb, lds_stage + C::A_BYTES + blk * 1024, off, 0);
}

template <class C, int LO, int HI>
__device__ __forceinline__ void load_range(uint8_t* lds_stage, __amdgpu_buffer_rsrc_t ra,
                                           __amdgpu_buffer_rsrc_t rb, int ld, int klim, int k0,
                                           int wave, int l, bool live) {
    if constexpr (LO < HI) {
        load_one<C, LO>(lds_stage, ra, rb, ld, klim, k0, wave, l, live);
        load_range<C, LO + 1, HI>(lds_stage, ra, rb, ld, klim, k0, wave, l, live);
    }
}

template <class C, int Q>
__device__ __forceinline__ void mfma_with_loads(typename Mfma<C::MI_>::acc_t (&acc)[C::FN][C::FM],
                                                const v8i (&fa)[C::FM], const v8i (&fb)[C::FN],
                                                uint8_t* lds_stage, __amdgpu_buffer_rsrc_t ra,
                                                __amdgpu_buffer_rsrc_t rb, int ld, int klim, int k0,
                                                int wave, int l, bool live) {
    constexpr int NQ = C::FN * C::FM;
    if constexpr (Q < NQ) {
        constexpr int i = Q / C::FM, j = Q % C::FM;
        acc[i][j] = Mfma<C::MI_>::template run<C::FMT>(fb[i], fa[j], acc[i][j]);
        // the share of loads issued after MFMA Q of NQ
        load_range<C, Q * C::LOADS / NQ, (Q + 1) * C::LOADS / NQ>(lds_stage, ra, rb, ld, klim, k0,
                                                                  wave, l, live);
        __builtin_amdgcn_sched_barrier(0);
        mfma_with_loads<C, Q + 1>(acc, fa, fb, lds_stage, ra, rb, ld, klim, k0, wave, l, live);
    }
}

// 32 operand bytes for one MFMA: row base + l of an LDS operand tile
// (base a multiple of 16, so the swizzle depends on l only), logical chunks c0
// and c0+1.
template <int CPR>
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int base, int l, int c0) {
    const int sw = chunk_swizzle<CPR>(l);
    const uint8_t* row = tile + (base + l) * (CPR * 16);
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

// Operand fragments of K step `ks` of one stage for this wave: FM row blocks
// of A and FN row blocks of B.  Lanes 0..MI-1 take rows, the lane group
// (lane / MI) takes chunk pair 2*(lane/MI) of the step (for MI=32 lanes
// 32..63 take chunks 2,3; for MI=16 four lane groups take pairs 0..3).  A and
// B use the same lane -> k assignment, which is all the MFMA contraction needs.
template <class C>
__device__ __forceinline__ void read_frags(v8i (&fa)[C::FM], v8i (&fb)[C::FN], const uint8_t* st,
                                           int ks, int wm, int wn, int lane) {
    constexpr int MI = C::MI_;
    const int c0 = ks * (C::KSTEP / 16) + (lane / MI) * 2;
    const int l = lane % MI;
#pragma unroll
    for (int j = 0; j < C::FM; ++j)
        fa[j] = read_frag<C::CPR>(st, wm * C::WTM + j * MI, l, c0);
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
        fb[i] = read_frag<C::CPR>(st + C::A_BYTES, wn * C::WTN + i * MI, l, c0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt encoding on gfx9: vmcnt low bits [3:0], high bits [15:14];
    // expcnt [6:4] and lgkmcnt [11:8] left at their maxima (no wait).
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Split-K partial tiles travel between workgroups, possibly on different XCDs
// whose L2s are not coherent with each other, as 16-byte buffer stores and
// loads with the sc1 cache policy (written through the L2, read past it).
// They are compiler builtins, so the compiler counts them and batches the
// loads (an atomic load per float would be waited for one by one).
typedef unsigned v4u __attribute__((ext_vector_type(4)));
constexpr int kPolicyCoherent = 16;   // cache-policy bit sc1

// acc (FN x FM blocks of NACC fp32 per lane) as 16-byte chunks: chunk c holds
// elements 4g .. 4g+3 of block (i, j), c = (i * FM + j) * (NACC / 4) + g.
template <int FN, int FM, class A>
__device__ __forceinline__ v4f acc_chunk(const A (&acc)[FN][FM], int c) {
    constexpr int G = sizeof(A) / 16;
    const int i = c / (FM * G), j = (c / G) % FM, g = c % G;
    return v4f{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
}

template <int FN, int FM, class A>
__device__ __forceinline__ void acc_chunk_add(A (&acc)[FN][FM], int c, v4f x) {
    constexpr int G = sizeof(A) / 16;
    const int i = c / (FM * G), j = (c / G) % FM, g = c % G;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][j][4 * g + e] += x[e];
}

// This thread's share of a partial tile of `bytes` bytes at base: chunk c at
// byte (c * stride + idx) * 16 (each wave writes and reads 1 KiB runs).
template <int FN, int FM, class A>
__device__ __forceinline__ void partial_publish(const A (&acc)[FN][FM], float* base, int stride,
                                                int idx, uint32_t bytes) {
    constexpr int NC = FN * FM * (int)(sizeof(A) / 16);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, bytes);
#pragma unroll
    for (int c = 0; c < NC; ++c)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, acc_chunk<FN, FM>(acc, c)), r,
                                               (c * stride + idx) * 16, 0, kPolicyCoherent);
}

// acc += this thread's share of a partial tile (same layout).  Loads go out
// in batches of up to 16 chunks, all issued before the first add (the
// scheduling barrier keeps the compiler from trading that for registers by
// waiting on one load at a time).
template <int FN, int FM, class A>
__device__ __forceinline__ void partial_accumulate(A (&acc)[FN][FM], const float* base, int stride,
                                                   int idx, uint32_t bytes) {
    constexpr int NC = FN * FM * (int)(sizeof(A) / 16);
    constexpr int B = NC < 16 ? NC : 16;
    static_assert(NC % B == 0, "whole batches");
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, bytes);
#pragma unroll
    for (int b = 0; b < NC; b += B) {
        v4u x[B];
#pragma unroll
        for (int k = 0; k < B; ++k)
            x[k] = __builtin_amdgcn_raw_buffer_load_b128(r, ((b + k) * stride + idx) * 16, 0,
                                                         kPolicyCoherent);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < B; ++k) acc_chunk_add<FN, FM>(acc, b + k, __builtin_bit_cast(v4f, x[k]));
    }
}

template <int FN, int FM, class A>
__device__ __forceinline__ void acc_add(A (&acc)[FN][FM], const A (&x)[FN][FM]) {
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int e = 0; e < (int)(sizeof(A) / 4); ++e) acc[i][j][e] += x[i][j][e];
}

// acc += the partial tiles 0 .. splits-1 of one tile (stored one after the
// other, tile_floats apart, each in the layout above), added in split order,
// for partials of at most 8 chunks per thread (small tiles): the loads of
// several partials go out together, up to 16 chunks per batch, so the fix-up
// costs one memory latency per batch instead of one per partial.
template <int FN, int FM, class A>
__device__ __forceinline__ void partial_accumulate_all(A (&acc)[FN][FM], const float* tile_parts,
                                                       int splits, int tile_floats, int stride,
                                                       int idx) {
    constexpr int NC = FN * FM * (int)(sizeof(A) / 16);
    static_assert(NC <= 8, "several partials per batch");
    {
        constexpr int QB = 16 / NC;    // partials per batch
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(tile_parts, (uint32_t)splits * (uint32_t)tile_floats * 4);
        for (int q0 = 0; q0 < splits; q0 += QB) {
            v4u x[QB][NC];
#pragma unroll
            for (int k = 0; k < QB; ++k)
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    x[k][c] = q0 + k < splits
                                  ? __builtin_amdgcn_raw_buffer_load_b128(
                                        r, (q0 + k) * tile_floats * 4 + (c * stride + idx) * 16, 0,
                                        kPolicyCoherent)
                                  : v4u{0u, 0u, 0u, 0u};
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < QB; ++k)
                if (q0 + k < splits)
#pragma unroll
                    for (int c = 0; c < NC; ++c)
                        acc_chunk_add<FN, FM>(acc, c, __builtin_bit_cast(v4f, x[k][c]));
        }
    }
}

// acc = the sum of the partial tiles 0 .. splits-1 of one tile, added in split
// order into zeroed accumulators; partial own_q is `own` (this unit's, still
// in registers), the others are read from memory (stored one after the
// other, tile_floats apart, each in the layout above).  For partials of more
// than 8 chunks per thread, which go out one partial per batch: not reading
// its own back saves one memory latency.
template <int FN, int FM, class A>
__device__ __forceinline__ void partial_sum_in_order(A (&acc)[FN][FM], const A (&own)[FN][FM],
                                                     int own_q, const float* tile_parts, int splits,
                                                     int tile_floats, int stride, int idx) {
    static_assert(FN * FM * (int)(sizeof(A) / 16) > 8, "one partial per batch");
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = A{};
    for (int q = 0; q < splits; ++q) {
        if (q == own_q)
            acc_add<FN, FM>(acc, own);
        else
            partial_accumulate<FN, FM>(acc, tile_parts + (size_t)q * tile_floats, stride, idx,
                                       (uint32_t)tile_floats * 4);
    }
}

// Two fp32 -> bf16 conversions, round to nearest even, packed low | high << 16
// (one v_cvt_pk_bf16_f32; fp32 denormals are kept, so the bf16 denormal range
// rounds like the rest).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{lo, hi}, bf2));
}

// Epilogue of one wave's FM x FN blocks of MI x MI outputs, whose top-left
// corner is (row0 + mbase, col0 + nbase).  The MFMA was fed B as its first
// operand, so lane l holds output row m = l % MI of each block and runs of 4
// consecutive columns n.  Row-wise scales and bias come from the LDS copies of
// the tile's parameters (indexed from the tile's corner).  y = acc * s, or
// fma(acc, s, bias) with a bias, with s = sa * sb formed in fp32; then RNE.
// RW, BIAS and FULL (the wave's block lies inside the output and 8-byte stores
// are allowed) are compile-time, so the block has no branches; all parameters
// are read from LDS before the first use.
template <int MI, int FM, int FN, bool RW, bool BIAS, bool FULL>
__device__ __forceinline__ void store_tile_impl(const typename Mfma<MI>::acc_t (&acc)[FN][FM],
                                                const Params& p, int row0, int col0, int mbase,
                                                int nbase, const float* epi_sa,
                                                const float* epi_sb, const uint16_t* epi_bias,
                                                float s_pt, int lane) {
    constexpr int G = Mfma<MI>::NACC / 4;   // runs of 4 columns per block and lane
    auto col = [&](int i, int g) {
        return nbase + i * MI + (MI == 32 ? 8 * g + 4 * (lane / 32) : 4 * (lane / 16));
    };
    float sa_r[FM];
    v4f sb_r[FN][G];
    uint2 b_r[FN][G];
#pragma unroll
    for (int j = 0; j < FM; ++j) sa_r[j] = RW ? epi_sa[mbase + j * MI + lane % MI] : s_pt;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if constexpr (RW) sb_r[i][g] = *reinterpret_cast<const v4f*>(epi_sb + col(i, g));
            if constexpr (BIAS) b_r[i][g] = *reinterpret_cast<const uint2*>(epi_bias + col(i, g));
        }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int ml = mbase + j * MI + lane % MI;
        const int m = row0 + ml;
        if (!FULL && m >= p.M) continue;
        uint16_t* orow = p.out + (size_t)m * p.N + col0;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int nl = col(i, g);
                if (!FULL && col0 + nl >= p.N) continue;
                float y[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float sc = RW ? sa_r[j] * sb_r[i][g][c] : s_pt;
                    const float v = acc[i][j][4 * g + c];
                    if constexpr (BIAS) {
                        const uint32_t bw = c < 2 ? b_r[i][g].x : b_r[i][g].y;
                        const float bv = __uint_as_float(c % 2 == 0 ? bw << 16 : bw & 0xffff0000u);
                        y[c] = __builtin_fmaf(v, sc, bv);
                    } else {
                        y[c] = v * sc;
                    }
                }
                const uint32_t lo = pack_bf16x2(y[0], y[1]);
                const uint32_t hi = pack_bf16x2(y[2], y[3]);
                if (FULL || (p.vec_store && col0 + nl + 3 < p.N)) {
                    uint2 w;
                    w.x = lo;
                    w.y = hi;
                    *reinterpret_cast<uint2*>(orow + nl) = w;
                } else {
                    const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi,
                                           (uint16_t)(hi >> 16)};
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (col0 + nl + c < p.N) orow[nl + c] = h[c];
                }
            }
    }
}

template <int MI, int FM, int FN>
__device__ __forceinline__ void store_tile(const typename Mfma<MI>::acc_t (&acc)[FN][FM],
                                           const Params& p, int row0, int col0, int mbase,
                                           int nbase, const float* epi_sa, const float* epi_sb,
                                           const uint16_t* epi_bias, float s_pt, bool has_bias,
                                           int lane) {
    // Derive every epilogue address from an opaque copy of the lane id, so the
    // compiler cannot hoist them out of the tile loop and keep them live (in
    // registers the K loop needs) across it.
    asm volatile("" : "+v"(lane));
    const bool full = p.vec_store && row0 + mbase + FM * MI <= p.M &&
                      col0 + nbase + FN * MI <= p.N;   // wave-uniform
#define FP8MM_EPI(RW, BIAS, FULL)                                                               \
    store_tile_impl<MI, FM, FN, RW, BIAS, FULL>(acc, p, row0, col0, mbase, nbase, epi_sa, epi_sb, \
                                                epi_bias, s_pt, lane)
    if (full) {
        if (p.rowwise) {
            if (has_bias) FP8MM_EPI(true, true, true); else FP8MM_EPI(true, false, true);
        } else {
            if (has_bias) FP8MM_EPI(false, true, true); else FP8MM_EPI(false, false, true);
        }
    } else {
        if (p.rowwise) {
            if (has_bias) FP8MM_EPI(true, true, false); else FP8MM_EPI(true, false, false);
        } else {
            if (has_bias) FP8MM_EPI(false, true, false); else FP8MM_EPI(false, false, false);
        }
    }
#undef FP8MM_EPI
}

// Staged epilogue of the generic kernel, first half: each wave converts its
// FM x FN blocks (y = acc * s, or fma(acc, s, bias); RNE to bf16) and writes
// them into a row-major copy of the whole BM x BN tile in LDS.  Row r of that
// copy has STG_CHUNKS 16-byte chunks; chunk c sits at position (c + r) mod
// STG_CHUNKS, so the lanes of one MFMA block, which hold one column run each
// of consecutive rows, write to different banks.  PAD instead: rows are
// STG_CHUNKS + 1 chunks apart and not rotated (the odd number of chunks per
// row spreads consecutive rows over the banks), so that any 16 bytes of a
// row, at any even offset, are contiguous.  Rows and columns outside the
// output are converted too (from zero accumulators) and never stored.
template <class C, bool RW, bool BIAS, bool PAD>
__device__ __forceinline__ void stage_tile_impl(
    const typename Mfma<C::MI_>::acc_t (&acc)[C::FN][C::FM], uint8_t* stg, int mbase, int nbase,
    const float* epi_sa, const float* epi_sb, const uint16_t* epi_bias, float s_pt, int lane) {
    constexpr int MI = C::MI_;
    constexpr int G = Mfma<MI>::NACC / 4;
    constexpr int NCH = C::STG_CHUNKS;
    float sa_r[C::FM];
#pragma unroll
    for (int j = 0; j < C::FM; ++j) sa_r[j] = RW ? epi_sa[mbase + j * MI + lane % MI] : s_pt;
    // Column runs outermost: each run's scales and bias are read once and
    // stay live only while its FM row blocks are written.
#pragma unroll
    for (int i = 0; i < C::FN; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int nl = nbase + i * MI + (MI == 32 ? 8 * g + 4 * (lane / 32) : 4 * (lane / 16));
            v4f sb_r;
            uint2 b_r;
            if constexpr (RW) sb_r = *reinterpret_cast<const v4f*>(epi_sb + nl);
            if constexpr (BIAS) b_r = *reinterpret_cast<const uint2*>(epi_bias + nl);
            const int byte = nl * 2;   // a multiple of 8: one half of a chunk
#pragma unroll
            for (int j = 0; j < C::FM; ++j) {
                const int ml = mbase + j * MI + lane % MI;
                float y[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float sc = RW ? sa_r[j] * sb_r[c] : s_pt;
                    const float v = acc[i][j][4 * g + c];
                    if constexpr (BIAS) {
                        const uint32_t bw = c < 2 ? b_r.x : b_r.y;
                        const float bv = __uint_as_float(c % 2 == 0 ? bw << 16 : bw & 0xffff0000u);
                        y[c] = __builtin_fmaf(v, sc, bv);
                    } else {
                        y[c] = v * sc;
                    }
                }
                uint2 w;
                w.x = pack_bf16x2(y[0], y[1]);
                w.y = pack_bf16x2(y[2], y[3]);
                if constexpr (PAD)
                    *reinterpret_cast<uint2*>(stg + ml * ((NCH + 1) * 16) + byte) = w;
                else
                    *reinterpret_cast<uint2*>(stg + ml * (NCH * 16) + (((byte >> 4) + ml) % NCH) * 16 +
                                              (byte & 15)) = w;
            }
        }
}

// Second half: the workgroup stores the staged tile row by row, consecutive
// lanes on consecutive 16-byte pieces of a row, so each store instruction
// writes whole runs of a row instead of a few bytes of many rows.  Rows whose
// start is 16-byte aligned (N % 8 == 0 and out 16-byte aligned) are all
// pieces; only rows and columns inside the output are written.
template <class C>
__device__ __forceinline__ void store_staged(const uint8_t* stg, const Params& p, int row0, int col0,
                                             int tid) {
    constexpr int NCH = C::STG_CHUNKS;
    constexpr int TOTAL = C::BM_ * NCH;
    constexpr int ITERS = (TOTAL + C::THREADS - 1) / C::THREADS;
    const int rows = min(C::BM_, p.M - row0);
    const int pieces = min(NCH, (p.N - col0) / 8);   // N % 8 == 0 here
#pragma unroll 4
    for (int it = 0; it < ITERS; ++it) {
        const int q = tid + it * C::THREADS;
        const int r = q / NCH;
        const int cw = q - r * NCH;
        if (q >= TOTAL || r >= rows || cw >= pieces) continue;
        const uint8_t* src = stg + r * (NCH * 16) + ((cw + r) % NCH) * 16;
        uint16_t* dst = p.out + (size_t)(row0 + r) * p.N + col0 + cw * 8;
        *reinterpret_cast<v4i*>(dst) = *reinterpret_cast<const v4i*>(src);
    }
}

// The same for rows whose start is not 16-byte aligned (odd N, or an output
// only 2- or 4-byte aligned), from the padded copy.  Row r of the tile is a
// head of h < 8 values up to the first 16-byte boundary of its output row, a
// body of 16-byte pieces and a tail of fewer than 8 values.  Two passes, each
// with consecutive lanes on consecutive work items and no loop inside a lane:
// the body pieces (each one 16-byte LDS read at the piece's even offset, 2h
// bytes into a staged chunk: gfx950's LDS reads unaligned vectors whole, so
// no shifts or selects), then one value per lane for the heads and tails.
template <class C>
__device__ __forceinline__ void store_staged_unaligned(const uint8_t* stg, const Params& p, int row0,
                                                       int col0, int tid) {
    constexpr int NCH = C::STG_CHUNKS;
    constexpr int PITCH = (NCH + 1) * 16;
    const int rows = min(C::BM_, p.M - row0);
    const int ncols = min(C::BN_, p.N - col0);
    auto head_of = [&](int r) {
        const uint16_t* orow = p.out + (size_t)(row0 + r) * p.N + col0;
        return min((8 - (int)(((uintptr_t)orow >> 1) & 7)) & 7, ncols);
    };
    {   // body pieces: NCH per row at most
        constexpr int TOTAL = C::BM_ * NCH;
        constexpr int ITERS = (TOTAL + C::THREADS - 1) / C::THREADS;
#pragma unroll 2
        for (int it = 0; it < ITERS; ++it) {
            const int q = tid + it * C::THREADS;
            const int r = q / NCH;
            const int b = q - r * NCH;
            if (q >= TOTAL || r >= rows) continue;
            const int head = head_of(r);
            if (b >= (ncols - head) / 8) continue;
            const v4i v = *reinterpret_cast<const v4i_a2*>(stg + r * PITCH + head * 2 + b * 16);
            uint16_t* orow = p.out + (size_t)(row0 + r) * p.N + col0;
            *reinterpret_cast<v4i*>(orow + head + b * 8) = v;
        }
    }
    {   // heads (items 0..7 of a row) and tails (items 8..15), one value each
        constexpr int TOTAL = C::BM_ * 16;
        constexpr int ITERS = (TOTAL + C::THREADS - 1) / C::THREADS;
#pragma unroll 2
        for (int it = 0; it < ITERS; ++it) {
            const int q = tid + it * C::THREADS;
            const int r = q / 16;
            const int item = q - r * 16;
            if (q >= TOTAL || r >= rows) continue;
            const int head = head_of(r);
            const int e = item < 8 ? item : head + (ncols - head) / 8 * 8 + (item - 8);
            if (item < 8 ? e >= head : e >= ncols) continue;
            p.out[(size_t)(row0 + r) * p.N + col0 + e] =
                *reinterpret_cast<const uint16_t*>(stg + r * PITCH + e * 2);
        }
    }
}

template <class C>
__device__ __forceinline__ void stage_and_store(
    const typename Mfma<C::MI_>::acc_t (&acc)[C::FN][C::FM], uint8_t* stg, const Params& p,
    int row0, int col0, int mbase, int nbase, const float* epi_sa, const float* epi_sb,
    const uint16_t* epi_bias, float s_pt, bool has_bias, int lane, int tid) {
    // As in store_tile: opaque lane id, so the addresses are not kept live
    // across the K loop.
    asm volatile("" : "+v"(lane));
    auto stage = [&](auto pad) {
        constexpr bool PAD = decltype(pad)::value;
        if (p.rowwise) {
            if (has_bias)
                stage_tile_impl<C, true, true, PAD>(acc, stg, mbase, nbase, epi_sa, epi_sb, epi_bias, s_pt, lane);
            else
                stage_tile_impl<C, true, false, PAD>(acc, stg, mbase, nbase, epi_sa, epi_sb, epi_bias, s_pt, lane);
        } else {
            if (has_bias)
                stage_tile_impl<C, false, true, PAD>(acc, stg, mbase, nbase, epi_sa, epi_sb, epi_bias, s_pt, lane);
            else
                stage_tile_impl<C, false, false, PAD>(acc, stg, mbase, nbase, epi_sa, epi_sb, epi_bias, s_pt, lane);
        }
        barrier_lds();
    };
    if (p.vec16) {
        stage(std::false_type{});
        store_staged<C>(stg, p, row0, col0, tid);
    } else {
        stage(std::true_type{});
        store_staged_unaligned<C>(stg, p, row0, col0, tid);
    }
}

// One K stage (BK bytes of K) of the software pipeline.  The fragments of
// the stage's first K step are already in buffer CUR0.  Each step first
// issues the LDS reads of the next step into the other buffer, then the MFMAs
// of this step.  At the last step, if another stage follows (HAS_NEXT), the
// wave waits for its own loads of that stage, joins the barrier (after which
// every wave's reads of this stage are done and every wave's loads of the next
// stage have landed), refills this stage's buffer with the slice STAGES ahead,
// and reads the next stage's first fragments.
// K offset of logical slice s of a unit that walks its k_iters slices from
// slice rot on (and wraps).  Past the end (s >= k_iters: dead loads, which
// read out of range anyway) the value is only kept in range of an int.
__device__ __forceinline__ int slice_k0(int s, int rot, int k_iters, int bk) {
    const int x = s + rot;
    return (x >= k_iters ? x - k_iters : x) * bk;
}

template <class C, int CUR0, bool HAS_NEXT>
__device__ __forceinline__ void run_stage(typename Mfma<C::MI_>::acc_t (&acc)[C::FN][C::FM],
                                          v8i (&fa)[2][C::FM], v8i (&fb)[2][C::FN], uint8_t* smem,
                                          int kt, int k_iters, __amdgpu_buffer_rsrc_t ra,
                                          __amdgpu_buffer_rsrc_t rb, int ld, int klim, int wave,
                                          int wm, int wn, int lane, int rot) {
    using F = Mfma<C::MI_>;
    constexpr int S = C::STAGES_;
    const uint8_t* st = smem + (kt % S) * C::STAGE_BYTES;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
        const int cur = (CUR0 + ks) & 1;
        if (ks + 1 < C::NKS) {
            read_frags<C>(fa[cur ^ 1], fb[cur ^ 1], st, ks + 1, wm, wn, lane);
        } else if (HAS_NEXT) {
            if constexpr (C::INTERLEAVE) {
                // Every earlier stage issued exactly LOADS loads per wave (dead
                // ones read out of range), so slice kt+1 has landed once the
                // S-2 newest slices' loads remain.
                wait_vmcnt<C::LOADS * (S - 2)>();
                barrier_lds();
                // The buffer just released is refilled with slice kt+S.
                // MFMA-bound tiles: the loads are spread between this step's
                // MFMAs; issued as one burst they stall the wave in the memory
                // pipeline's queue while the MFMA unit idles.
                read_frags<C>(fa[cur ^ 1], fb[cur ^ 1], smem + ((kt + 1) % S) * C::STAGE_BYTES, 0,
                              wm, wn, lane);
                __builtin_amdgcn_sched_barrier(0);
                int l = lane;
                asm volatile("" : "+v"(l));
                mfma_with_loads<C, 0>(acc, fa[cur], fb[cur], smem + (kt % S) * C::STAGE_BYTES, ra,
                                      rb, ld, klim, slice_k0(kt + S, rot, k_iters, C::BK_), wave, l,
                                      kt + S < k_iters);
                continue;
            } else {
                // Memory-bound tiles: the loads go out first, as early as
                // possible, and only for slices that exist.  Loads issued so
                // far cover slices up to min(kt+S-1, k_iters-1) (the prologue
                // may add dead ones past the end); slice kt+1 has landed once
                // the S-2 newest slices remain, near the end once none do.
                if (kt + S - 1 < k_iters) wait_vmcnt<C::LOADS * (S - 2)>();
                else wait_vmcnt<0>();
                barrier_lds();
                if (kt + S < k_iters)
                    load_stage<C>(smem + (kt % S) * C::STAGE_BYTES, ra, rb, ld, klim,
                                  slice_k0(kt + S, rot, k_iters, C::BK_), wave, lane);
                read_frags<C>(fa[cur ^ 1], fb[cur ^ 1], smem + ((kt + 1) % S) * C::STAGE_BYTES, 0,
                              wm, wn, lane);
            }
        }
        // Keep the compiler from sinking the LDS reads below the MFMAs: they
        // must be in flight while the MFMAs of this step run.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
            for (int j = 0; j < C::FM; ++j)
                acc[i][j] = F::template run<C::FMT>(fb[cur][i], fa[cur][j], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int MI, int GROUP_M,
          bool NT_B, int FMT, bool SK = false>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * kWave,
                                  (Cfg<BM, BN, BK, WAVES_M, WAVES_N, STAGES, MI, GROUP_M>::OCCUPANCY))
fp8_gemm_kernel(Params p) {
    using C = Cfg<BM, BN, BK, WAVES_M, WAVES_N, STAGES, MI, GROUP_M, NT_B, FMT>;
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
    float* epi_sa = reinterpret_cast<float*>(smem + C::MAIN_BYTES);
    float* epi_sb = epi_sa + BM;
    uint16_t* epi_bias = reinterpret_cast<uint16_t*>(epi_sb + BN);
    const bool has_bias = p.bias != nullptr;

    __shared__ unsigned arrival;
    // One work unit: K slices [kb, kb + k_iters) of tile t, part `part` of the
    // tile's `nparts` (nparts > 1: its partial goes to slot t * splits + part,
    // and the last of them to arrive finishes the tile).
    auto unit = [&](const int t, const int kb, const int k_iters, const int part, const int nparts) {
        int pm, pn;
        tile_coords(t, p.tiles_m, p.tiles_n, GROUP_M, pm, pn);
        const int row0 = pm * BM;
        const int col0 = pn * BN;
        // The buffer resources start at the unit's first K byte, so the stage
        // code sees a K range beginning at 0.
        const int kskip = kb * BK;
        const int klim = p.K - kskip;
        // With a single row of tiles (the skinny shapes) every workgroup reads
        // the same A rows while streaming its own B rows: each workgroup
        // starts at its own K slice (and wraps), so the workgroups of an XCD
        // do not all ask its L2 for the same lines of A at the same moment.
        const int rot = (C::STREAM_B && k_iters > 1) ? (int)(((int64_t)wg * k_iters) / G) % k_iters
                                                      : 0;
        const uint32_t rows_a = (uint32_t)min(BM, p.M - row0);
        const uint32_t rows_b = (uint32_t)min(BN, p.N - col0);
        const __amdgpu_buffer_rsrc_t ra =
            make_rsrc(p.A + (size_t)row0 * p.K + kskip, rows_a * (uint32_t)p.K - (uint32_t)kskip);
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(p.B + (size_t)col0 * p.K + kskip, rows_b * (uint32_t)p.K - (uint32_t)kskip);

        // Every wave must be done with the LDS of the previous tile before
        // this tile's loads start.  The previous tile's output stores may
        // still be in flight: vector memory operations are counted together,
        // and loads return in order among themselves, so a wait for "at most
        // n outstanding" still covers every load older than the last n; the
        // stores only make the first wait of the tile longer.
        barrier_lds();

        // This tile's scales and bias, fetched now into registers and moved to
        // LDS after the K loop (their latency hides under the loop).
        float sa_v[C::NSA], sb_v[C::NSB];
        uint16_t bias_v[C::NSB];
#pragma unroll
        for (int i = 0; i < C::NSA; ++i) {
            const int r = tid + i * C::THREADS;
            sa_v[i] = (p.rowwise && r < BM && row0 + r < p.M) ? p.scale_a[row0 + r] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < C::NSB; ++i) {
            const int c = tid + i * C::THREADS;
            const bool ok = c < BN && col0 + c < p.N;
            sb_v[i] = (p.rowwise && ok) ? p.scale_b[col0 + c] : 0.f;
            bias_v[i] = (has_bias && ok) ? p.bias[col0 + c] : (uint16_t)0;
        }

        typename F::acc_t acc[C::FN][C::FM];
#pragma unroll
        for (int i = 0; i < C::FN; ++i)
#pragma unroll
            for (int j = 0; j < C::FM; ++j)
#pragma unroll
                for (int v = 0; v < F::NACC; ++v) acc[i][j][v] = 0.f;

        // Fill every stage buffer; the buffer of stage kt is refilled with
        // slice kt + STAGES once stage kt has been read.
#pragma unroll
        for (int s = 0; s < STAGES; ++s)
            load_stage<C>(smem + s * C::STAGE_BYTES, ra, rb, p.K, s < k_iters ? klim : 0,
                          slice_k0(s, rot, k_iters, BK),
                          wave, lane);

        // Software pipeline over K steps: the operand fragments of step q+1 are
        // read from LDS while the MFMAs of step q run.  At the last step of a
        // stage the wave first makes the next stage visible (own loads landed,
        // barrier), recycles the stage it has just finished reading for the
        // loads STAGES slices ahead, and reads the next stage's first fragments;
        // the barrier therefore sits under the tail of the previous MFMAs.
        v8i fa[2][C::FM], fb[2][C::FN];
        wait_vmcnt<C::LOADS * (STAGES - 1)>();   // stage 0 landed (S-1 newer slices may not)
        barrier_lds();
        if (k_iters > 0) read_frags<C>(fa[0], fb[0], smem, 0, wm, wn, lane);

        // Every stage but the last hands over to the next one; the fragment
        // parity of each stage is a compile-time constant.
        int kt = 0;
        if (k_iters > 0) {
            if constexpr (C::NKS % 2 == 0) {
                for (; kt + 1 < k_iters; ++kt)
                    run_stage<C, 0, true>(acc, fa, fb, smem, kt, k_iters, ra, rb, p.K, klim, wave, wm,
                                          wn, lane, rot);
                run_stage<C, 0, false>(acc, fa, fb, smem, kt, k_iters, ra, rb, p.K, klim, wave, wm, wn,
                                       lane, rot);
            } else {
                for (; kt + 2 < k_iters; kt += 2) {
                    run_stage<C, 0, true>(acc, fa, fb, smem, kt, k_iters, ra, rb, p.K, klim, wave, wm,
                                          wn, lane, rot);
                    run_stage<C, 1, true>(acc, fa, fb, smem, kt + 1, k_iters, ra, rb, p.K, klim, wave,
                                          wm, wn, lane, rot);
                }
                if (kt + 1 < k_iters) {
                    run_stage<C, 0, true>(acc, fa, fb, smem, kt, k_iters, ra, rb, p.K, klim, wave, wm,
                                          wn, lane, rot);
                    run_stage<C, 1, false>(acc, fa, fb, smem, kt + 1, k_iters, ra, rb, p.K, klim, wave,
                                           wm, wn, lane, rot);
                } else {
                    run_stage<C, 0, false>(acc, fa, fb, smem, kt, k_iters, ra, rb, p.K, klim, wave, wm,
                                           wn, lane, rot);
                }
            }
        }

        if constexpr (C::SPLIT_OK) if (nparts > 1) {
            // Publish this unit's partial tile and count the arrival; the
            // stores have completed (vmcnt 0) before the arrival is counted.
            float* parts = p.partials + (size_t)t * p.splits * (BM * BN);
            partial_publish<C::FN, C::FM>(acc, parts + (size_t)part * (BM * BN), C::THREADS, tid,
                                          BM * BN * 4);
            wait_vmcnt<0>();
            __syncthreads();
            if (tid == 0)
                arrival = __hip_atomic_fetch_add(&p.counters[t], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            // Only the last of the tile's units goes on; it adds the partials in
            // split order (deterministic whatever the arrival order), its own
            // from registers where the partials are large.
            if (arrival != (unsigned)(nparts - 1)) return;
            if (tid == 0)
                __hip_atomic_store(&p.counters[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if constexpr (C::FN * C::FM * (F::NACC / 4) <= 8) {
                // Small partials: all of them go out in one batch, so reading
                // this unit's own back costs no extra latency.
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
#pragma unroll
                    for (int j = 0; j < C::FM; ++j) acc[i][j] = typename F::acc_t{};
                partial_accumulate_all<C::FN, C::FM>(acc, parts, nparts, BM * BN, C::THREADS, tid);
            } else if (nparts == 2) {
                // P0 + P1 in place: fp32 addition commutes, so the sum is the
                // same whichever unit is last.
                partial_accumulate<C::FN, C::FM>(acc, parts + (size_t)(1 - part) * (BM * BN), C::THREADS,
                                                 tid, BM * BN * 4);
            } else {
                const typename F::acc_t(&own)[C::FN][C::FM] = acc;
                typename F::acc_t sum[C::FN][C::FM];
                partial_sum_in_order<C::FN, C::FM>(sum, own, part, parts, nparts, BM * BN, C::THREADS,
                                                   tid);
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
#pragma unroll
                    for (int j = 0; j < C::FM; ++j) acc[i][j] = sum[i][j];
            }
        }

        // Epilogue parameters into LDS (beside the stage buffers).
        if (p.rowwise || has_bias) {
#pragma unroll
            for (int i = 0; i < C::NSA; ++i) {
                const int r = tid + i * C::THREADS;
                if (r < BM) epi_sa[r] = sa_v[i];
            }
#pragma unroll
            for (int i = 0; i < C::NSB; ++i) {
                const int c = tid + i * C::THREADS;
                if (c < BN) {
                    epi_sb[c] = sb_v[i];
                    epi_bias[c] = bias_v[i];
                }
            }
        }
        // The output tile is staged in the stage buffers: every wave must be
        // done reading the last stage, and every load (including the trailing
        // ones of slices past the end) must have landed.
        wait_vmcnt<0>();
        barrier_lds();
        stage_and_store<C>(acc, smem, p, row0, col0, wm * C::WTM, wn * C::WTN, epi_sa, epi_sb,
                           epi_bias, s_pt, has_bias, lane, tid);
    };

    if constexpr (SK) {
        // This workgroup's equal share of the tile-major (tile, K slice)
        // iterations; each tile it meets is one unit, whose part is its rank
        // among the workgroups meeting that tile.
        const int64_t total = (int64_t)p.num_tiles * p.k_iters;
        auto start_of = [&](int64_t w) { return w * total / G; };
        auto wg_of = [&](int64_t i) {   // the workgroup whose range holds iteration i
            int64_t w = i * G / total;
            while (w + 1 < G && start_of(w + 1) <= i) ++w;
            return w;
        };
        const int64_t end = start_of(wg + 1);
        for (int64_t it = start_of(wg); it < end;) {
            const int t = (int)(it / p.k_iters);
            const int kb = (int)(it - (int64_t)t * p.k_iters);
            const int kn = (int)min((int64_t)(p.k_iters - kb), end - it);
            const int64_t first = wg_of((int64_t)t * p.k_iters);
            const int64_t last = wg_of((int64_t)(t + 1) * p.k_iters - 1);
            unit(t, kb, kn, (int)(wg - first), (int)(last - first + 1));
            it += kn;
        }
    } else {
        const int num_units = p.num_tiles * p.splits;
        for (int u = wg; u < num_units; u += G) {
            const int t = u / p.splits;             // the splits of a tile are neighbours
            const int split = u - t * p.splits;
            const int kb = split * p.k_chunk;
            unit(t, kb, max(0, min(p.k_chunk, p.k_iters - kb)), split, p.splits);
        }
    }
}

// ------------------------------------------------------ ping-pong kernel ---
//
// 256 x 256 output tiles, K slices of 128 bytes, 8 waves in two groups of four
// with one wave of each group on every SIMD (waves w and w+4 share SIMD w).
// Group 1 runs one phase behind group 0, so on every SIMD one wave issues the
// 32 MFMAs (16 x 16 x 128) of a K slice from registers while the other reads
// its fragments of that slice from LDS and issues global -> LDS loads; at the
// end of each phase a workgroup barrier swaps the roles.  Wave (g, q) computes
// rows g*128 .. +128 and columns q*64 .. +64 of the tile with fp32 accumulators
// in registers.  The 16 x 16 x 128 form does the same work per wave as the
// 32 x 32 x 64 one (same fragment bytes, same 128 accumulators per lane) but
// draws less power per operation with random operands, so the power-limited
// shader clock settles higher.
//
// Two LDS stage buffers, slice s in buffer s % 2, each holding the slice's A
// rows 0-127 ("A-top", read only by group 0), A rows 128-255 ("A-bottom", read
// only by group 1) and B (read by both).  Group 0 reads slice s in phase 2s,
// group 1 in phase 2s+1.  The loads are issued in memory phases only, 8 per wave
// per phase:
//   phase 2s   (group 0): B of slice s+1        (its buffer was last read in 2s-1)
//   phase 2s+1 (group 1): A-bottom of slice s+1 (last read in 2s-1) and A-top of
//                         slice s+2             (last read in 2s)
// and each wave waits for its own loads (vmcnt 0) at the end of its next
// compute phase, before the barrier after which the data is first read.
// Between tiles, group 0 writes its outputs while group 1 runs its last
// compute phase; then group 1 writes its outputs while group 0 issues the next
// tile's first slices and epilogue parameters and waits for them.  (Issued
// before group 0's own stores, those loads made the stores wait behind them in
// the CU's memory queue; issued after them, their latency overlaps group 1's
// epilogue: 8192^3 340.5 -> 337.0 us, 16384^2 x 8192 1444 -> 1423 us on one
// MI355X.)
namespace pp {
constexpr int BM = 256, BN = 256, BK = 128;
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * kWave;
constexpr int CPR = BK / 16;                        // 16-byte chunks per LDS row
constexpr int A_BYTES = BM * BK;                    // 32 KiB
constexpr int HALF_A = A_BYTES / 2;                 // A-top / A-bottom, 16 KiB
constexpr int STAGE_BYTES = (BM + BN) * BK;         // 64 KiB
constexpr int MAIN_BYTES = 2 * STAGE_BYTES;
constexpr int MI = 16;                              // 16 x 16 x 128 MFMAs
using acc_t = Mfma<MI>::acc_t;
constexpr int FM = 128 / MI, FN = 64 / MI;          // MFMA blocks per wave
constexpr int KSTEPS = BK / Mfma<MI>::KSTEP;        // MFMA K steps per slice
constexpr int NOFF = 8;                             // load row groups per wave
constexpr int EPI_BYTES = BM * 4 + BN * 4 + BN * 2; // row scales, column scales, bias
// Output staging: group 0's waves use 4 KiB each after the parameters; group 1's
// waves use the A-bottom part of stage buffer 1, which is idle while they write
// their outputs (the next tile's first loads fill buffer 0 and buffer 1's A-top).
constexpr int STG_BYTES = 4096;
constexpr int STG0 = MAIN_BYTES + 2 * EPI_BYTES;
constexpr int STG1 = STAGE_BYTES + HALF_A;
constexpr int LDS_BYTES = STG0 + 4 * STG_BYTES;
static_assert(LDS_BYTES <= 160 * 1024, "gfx950 LDS is 160 KiB per workgroup");
static_assert(4 * STG_BYTES <= HALF_A, "group 1 staging fits in the A-bottom half");
}  // namespace pp

// Per-lane load offsets of wave q (0..3 within its group): offset i covers LDS
// block q + 4i (rows 8*(q + 4i) .. +8 of a 256-row panel, 1 KiB); lane l fills
// position l % 8 of row 8*(q + 4i) + l / 8 with logical chunk (l % 8) ^
// swizzle(row).  Row bits 0..3 are the same for every i, so is the chunk.
struct PpLoads {
    uint32_t off[pp::NOFF];   // row * K + chunk * 16
    uint32_t cbyte;           // chunk * 16
    uint32_t bot;             // 128 * K: A-bottom rows relative to A-top rows
};

__device__ __forceinline__ void pp_dma(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t off,
                                       uint32_t k0, bool inside) {
    dma16(r, dst, inside ? off : kOutOfRange, k0);
}

// Loads of slice s (K bytes s*BK ..) into stage buffer buf.  In the K-tail
// slice, lanes whose chunk lies at or past K read zeros (offset beyond the
// record limit).
__device__ __forceinline__ void pp_load_b(uint8_t* smem, int buf, int q, int s,
                                          __amdgpu_buffer_rsrc_t rb, const PpLoads& L, int K) {
    const uint32_t k0 = (uint32_t)s * pp::BK;
    const bool inside = k0 + L.cbyte < (uint32_t)K;
    uint8_t* st = smem + buf * pp::STAGE_BYTES + pp::A_BYTES;
#pragma unroll
    for (int i = 0; i < pp::NOFF; ++i) pp_dma(rb, st + (q + 4 * i) * 1024, L.off[i], k0, inside);
}

template <bool BOTTOM>
__device__ __forceinline__ void pp_load_a_half(uint8_t* smem, int buf, int q, int s,
                                               __amdgpu_buffer_rsrc_t ra, const PpLoads& L, int K) {
    const uint32_t k0 = (uint32_t)s * pp::BK;
    const bool inside = k0 + L.cbyte < (uint32_t)K;
    uint8_t* st = smem + buf * pp::STAGE_BYTES + (BOTTOM ? pp::HALF_A : 0);
#pragma unroll
    for (int i = 0; i < pp::NOFF / 2; ++i)
        pp_dma(ra, st + (q + 4 * i) * 1024, L.off[i] + (BOTTOM ? L.bot : 0u), k0, inside);
}

// Fragments of one slice for wave (grp, q): A rows grp*128 + j*MI + l, B rows
// q*64 + i*MI + l with l = lane % MI; lane group lane / MI takes the 32 K bytes
// 32 * (lane / MI) .. of each K step.
__device__ __forceinline__ void pp_read(v8i (&fa)[pp::KSTEPS][pp::FM],
                                        v8i (&fb)[pp::KSTEPS][pp::FN], const uint8_t* st, int grp,
                                        int q, int lane) {
    // Addresses are recomputed here from an opaque copy of the lane id: kept
    // live across the loop they would cost registers the fragments need.
    int l = lane % pp::MI;
    int lh = lane / pp::MI;
    asm volatile("" : "+v"(l), "+v"(lh));
#pragma unroll
    for (int ks = 0; ks < pp::KSTEPS; ++ks) {
        const int c0 = ks * (Mfma<pp::MI>::KSTEP / 16) + lh * 2;
#pragma unroll
        for (int j = 0; j < pp::FM; ++j)
            fa[ks][j] = read_frag<pp::CPR>(st, grp * 128 + j * pp::MI, l, c0);
#pragma unroll
        for (int i = 0; i < pp::FN; ++i)
            fb[ks][i] = read_frag<pp::CPR>(st + pp::A_BYTES, q * 64 + i * pp::MI, l, c0);
    }
}

// The MFMAs of one slice (128 x 64 x 128 per wave), from registers only.
template <int FMT>
__device__ __forceinline__ void pp_compute(pp::acc_t (&acc)[pp::FN][pp::FM],
                                           const v8i (&fa)[pp::KSTEPS][pp::FM],
                                           const v8i (&fb)[pp::KSTEPS][pp::FN]) {
#pragma unroll
    for (int ks = 0; ks < pp::KSTEPS; ++ks)
#pragma unroll
        for (int i = 0; i < pp::FN; ++i)
#pragma unroll
            for (int j = 0; j < pp::FM; ++j)
                acc[i][j] = Mfma<pp::MI>::template run<FMT>(fb[ks][i], fa[ks][j], acc[i][j]);
}

// One work unit: output tile t and its K slices kb .. kb + n - 1 (the whole
// K range without split-K; one of `splits` consecutive ranges with it).  The
// unit walks its slices starting at kb + rot and wraps (see the kernel head).
// This lane's id, recomputed (two VALU instructions) wherever the ping-pong
// kernel needs it: volatile, so the compiler neither merges the calls nor
// keeps the value live across the K loop (register pressure there made it
// spill lane-derived values, and each reload of a spill waited for every
// outstanding load, next tile's slices included).
__device__ __forceinline__ int pp_lane() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

struct PpTile {
    int row0, col0;
    int t, kb, n, rot;
    __amdgpu_buffer_rsrc_t ra, rb;
};

__device__ __forceinline__ int pp_slice(const PpTile& T, int step) {
    const int s = step + T.rot;
    return T.kb + (s < T.n ? s : s - T.n);
}

__device__ __forceinline__ PpTile pp_tile(const Params& p, int u, int group_m, int xcd) {
    PpTile T;
    T.t = u / p.splits;
    T.kb = (u - T.t * p.splits) * p.k_chunk;
    T.n = min(p.k_chunk, p.k_iters - T.kb);   // >= 1: the host leaves no empty unit
    T.rot = xcd * T.n / kXcds;
    int pm, pn;
    tile_coords(T.t, p.tiles_m, p.tiles_n, group_m, pm, pn);
    T.row0 = pm * pp::BM;
    T.col0 = pn * pp::BN;
    const uint32_t rows_a = (uint32_t)min(pp::BM, p.M - T.row0);
    const uint32_t rows_b = (uint32_t)min(pp::BN, p.N - T.col0);
    T.ra = make_rsrc(p.A + (size_t)T.row0 * p.K, rows_a * (uint32_t)p.K);
    T.rb = make_rsrc(p.B + (size_t)T.col0 * p.K, rows_b * (uint32_t)p.K);
    return T;
}

// A unit's epilogue parameters (256 row scales, 256 column scales, 256 bias
// values), one of each per thread of group 0 (tid 0..255): loaded into
// registers with the unit's first slices and written to the LDS parameter
// area once those loads have been waited for.  Entries past the last row or
// column are 0 (the epilogue never uses them).  Element loads, not 16-byte
// LDS-direct ones: the bias is only 2-byte aligned, and a 16-byte load whose
// record limit ends inside a dword reads that whole dword as zero (with an
// odd number of columns left, the last bias value would be lost).
struct PpParams {
    float sa, sb;
    uint16_t bias;
};

__device__ __forceinline__ PpParams pp_params_load(const Params& p, const PpTile& T, int t,
                                                   bool has_bias) {
    PpParams v;
    const bool row_ok = T.row0 + t < p.M, col_ok = T.col0 + t < p.N;
    v.sa = (p.rowwise && row_ok) ? p.scale_a[T.row0 + t] : 0.f;
    v.sb = (p.rowwise && col_ok) ? p.scale_b[T.col0 + t] : 0.f;
    v.bias = (has_bias && col_ok) ? p.bias[T.col0 + t] : (uint16_t)0;
    return v;
}

__device__ __forceinline__ void pp_params_store(const PpParams& v, int t, float* epi_sa,
                                                float* epi_sb, uint16_t* epi_bias) {
    epi_sa[t] = v.sa;
    epi_sb[t] = v.sb;
    epi_bias[t] = v.bias;
}

// A unit's first loads, all from group 0 (wave q): its first K slice whole
// and A-top of its second.
__device__ __forceinline__ void pp_tile_start(uint8_t* smem, const Params& p, const PpTile& T,
                                              const PpLoads& L, int q) {
    const int s0 = pp_slice(T, 0);
    pp_load_b(smem, 0, q, s0, T.rb, L, p.K);
    pp_load_a_half<false>(smem, 0, q, s0, T.ra, L, p.K);
    pp_load_a_half<true>(smem, 0, q, s0, T.ra, L, p.K);
    if (T.n > 1) pp_load_a_half<false>(smem, 1, q, pp_slice(T, 1), T.ra, L, p.K);
}

// Epilogue of wave (g, q) of the ping-pong kernel through a private 4 KiB LDS
// area: each band of 32 x 64 outputs is written to LDS in the MFMA layout (a
// lane holds runs of 4 consecutive columns of one row) and read back as 8 rows
// x 128 bytes per instruction, so every global store writes 8 whole 128-byte
// lines (instead of 32 pieces of 16 bytes).  LDS operations of one wave
// complete in order, so no barrier is needed.  In the LDS area, 16-byte chunk c
// of row r sits at c ^ ((r >> 1) & 7) (at most 2-way bank conflicts on the
// writes).  Falls back to store_tile where the block is not wholly inside the
// output or 16-byte stores are not allowed.
template <bool RW, bool BIAS>
__device__ __forceinline__ void pp_store_staged(const pp::acc_t (&acc)[pp::FN][pp::FM],
                                                const Params& p, int row0, int col0, int mbase,
                                                int nbase, const float* epi_sa,
                                                const float* epi_sb, const uint16_t* epi_bias,
                                                float s_pt, int lane, uint8_t* stg) {
    constexpr int MI = pp::MI, FM = pp::FM, FN = pp::FN;
    constexpr int G = Mfma<MI>::NACC / 4;   // runs of 4 columns per block and lane
    constexpr int JB = 32 / MI;             // MFMA row blocks per 32-row band
    // Column, within the wave's 64, of run g of block i for this lane.
    auto col = [&](int i, int g) {
        return i * MI + (MI == 32 ? 8 * g + 4 * (lane / 32) : 4 * (lane / 16));
    };
    float sa_r[FM];
    v4f sb_r[FN][G];
    uint2 b_r[FN][G];
#pragma unroll
    for (int j = 0; j < FM; ++j) sa_r[j] = RW ? epi_sa[mbase + j * MI + lane % MI] : s_pt;
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int nl = nbase + col(i, g);
            if constexpr (RW) sb_r[i][g] = *reinterpret_cast<const v4f*>(epi_sb + nl);
            if constexpr (BIAS) b_r[i][g] = *reinterpret_cast<const uint2*>(epi_bias + nl);
        }
#pragma unroll
    for (int band = 0; band < FM / JB; ++band) {
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
            const int j = band * JB + jj;
            const int r = jj * MI + lane % MI;
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float y[4];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float sc = RW ? sa_r[j] * sb_r[i][g][c] : s_pt;
                        const float v = acc[i][j][4 * g + c];
                        if constexpr (BIAS) {
                            const uint32_t bw = c < 2 ? b_r[i][g].x : b_r[i][g].y;
                            const float bv =
                                __uint_as_float(c % 2 == 0 ? bw << 16 : bw & 0xffff0000u);
                            y[c] = __builtin_fmaf(v, sc, bv);
                        } else {
                            y[c] = v * sc;
                        }
                    }
                    uint2 w;
                    w.x = pack_bf16x2(y[0], y[1]);
                    w.y = pack_bf16x2(y[2], y[3]);
                    const int cl = col(i, g);
                    const int cpos = (cl / 8) ^ ((r >> 1) & 7);
                    *reinterpret_cast<uint2*>(stg + r * 128 + cpos * 16 + (cl % 8) * 2) = w;
                }
        }
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int rr = pass * 8 + lane / 8;
            const int cc = lane % 8;
            const v4i v = *reinterpret_cast<const v4i*>(stg + rr * 128 + ((cc ^ ((rr >> 1) & 7)) * 16));
            uint16_t* dst = p.out + (size_t)(row0 + mbase + band * 32 + rr) * p.N + col0 + nbase + cc * 8;
            *reinterpret_cast<v4i*>(dst) = v;
        }
    }
}

// One wave's 128 x 64 outputs: staged through LDS where the block lies wholly
// inside the output and rows allow 16-byte stores, else store_tile.
__device__ __forceinline__ void pp_store(const pp::acc_t (&acc)[pp::FN][pp::FM], const Params& p,
                                         int row0, int col0, int mbase, int nbase,
                                         const float* epi_sa, const float* epi_sb,
                                         const uint16_t* epi_bias, float s_pt, bool has_bias,
                                         int lane, uint8_t* stg) {
    asm volatile("" : "+v"(lane));
    const bool full = p.vec16 && row0 + mbase + 128 <= p.M &&
                      col0 + nbase + 64 <= p.N;   // wave-uniform
    if (!full) {
        store_tile<pp::MI, pp::FM, pp::FN>(acc, p, row0, col0, mbase, nbase, epi_sa, epi_sb, epi_bias,
                                       s_pt, has_bias, lane);
        return;
    }
    if (p.rowwise) {
        if (has_bias)
            pp_store_staged<true, true>(acc, p, row0, col0, mbase, nbase, epi_sa, epi_sb, epi_bias,
                                        s_pt, lane, stg);
        else
            pp_store_staged<true, false>(acc, p, row0, col0, mbase, nbase, epi_sa, epi_sb, epi_bias,
                                         s_pt, lane, stg);
    } else {
        if (has_bias)
            pp_store_staged<false, true>(acc, p, row0, col0, mbase, nbase, epi_sa, epi_sb, epi_bias,
                                         s_pt, lane, stg);
        else
            pp_store_staged<false, false>(acc, p, row0, col0, mbase, nbase, epi_sa, epi_sb,
                                          epi_bias, s_pt, lane, stg);
    }
}

// Split-K for one wave of the ping-pong kernel.  The wave publishes its fp32
// partial of unit u (each store is a 1 KiB run) and counts
// its arrival on the counter of (tile, wave); the wave that arrives last sums
// the partials of all the tile's units in split order into acc (the same sum
// whatever the arrival order) and returns true: it runs the epilogue.  The
// other waves return false.  Partials travel with agent-coherent stores and
// loads (through the XCD's L2 to memory and back), and the stores have
// completed (vmcnt 0) before the arrival is counted.  The last wave leaves
// the counter at zero for the next launch.  Each wave works alone: no
// workgroup barrier is involved.
__device__ __forceinline__ bool pp_split_fixup(pp::acc_t (&acc)[pp::FN][pp::FM], const Params& p,
                                               int u, int t, int wave, int lane) {
    constexpr int PER_WAVE = 128 * 64;   // floats: the wave's 128 x 64 outputs
    partial_publish<pp::FN, pp::FM>(acc, p.partials + ((size_t)u * pp::WAVES + wave) * PER_WAVE,
                                    kWave, lane, PER_WAVE * 4);
    wait_vmcnt<0>();
    unsigned* counter = p.counters + (size_t)t * pp::WAVES + wave;
    unsigned old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (unsigned)(p.splits - 1)) return false;
    if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int i = 0; i < pp::FN; ++i)
#pragma unroll
        for (int j = 0; j < pp::FM; ++j) acc[i][j] = pp::acc_t{};
    for (int q = 0; q < p.splits; ++q)
        partial_accumulate<pp::FN, pp::FM>(
            acc, p.partials + ((size_t)(t * p.splits + q) * pp::WAVES + wave) * PER_WAVE, kWave, lane,
            PER_WAVE * 4);
    return true;
}

template <int GROUP_M, int FMT>
__global__ void __launch_bounds__(pp::THREADS) fp8_gemm_pp_kernel(Params p) {
    using namespace pp;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid % kWave;
    const int grp = wave / 4;
    const int q = wave % 4;

    const int G = gridDim.x;
    int wg = blockIdx.x;
    if (G % kXcds == 0) wg = (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds;
    const int num_units = p.num_tiles * p.splits;
    if (wg >= num_units) return;   // whole workgroup
    // The workgroups of XCD x walk a unit's K slices starting x/8 of the way
    // in (and wrap): the XCDs finish their tiles at different times, so the
    // output stores of the whole GPU do not all arrive at once.  The 32
    // workgroups of one XCD stay in step and keep sharing the slices in its L2.
    const int xcd = G % kXcds == 0 ? (int)(blockIdx.x % kXcds) : 0;
    const bool split = p.splits > 1;

    PpLoads L;
    L.cbyte = (uint32_t)(((lane % 8) ^ chunk_swizzle<CPR>((q & 1) * 8 + lane / 8)) * 16);
#pragma unroll
    for (int i = 0; i < NOFF; ++i)
        L.off[i] = (uint32_t)((8 * (q + 4 * i) + lane / 8) * p.K) + L.cbyte;
    L.bot = 128u * (uint32_t)p.K;

    const float s_pt = p.rowwise ? 0.f : p.scale_a[0] * p.scale_b[0];
    const bool has_bias = p.bias != nullptr;
    const bool need_epi = p.rowwise || has_bias;
    auto epi_area = [&](int parity, float*& sa, float*& sb, uint16_t*& bias) {
        sa = reinterpret_cast<float*>(smem + MAIN_BYTES + parity * EPI_BYTES);
        sb = sa + BM;
        bias = reinterpret_cast<uint16_t*>(sb + BN);
    };

    int parity = 0;
    PpTile T = pp_tile(p, wg, GROUP_M, xcd);
    if (grp == 0) {
        PpParams pv;
        if (need_epi) pv = pp_params_load(p, T, tid, has_bias);
        pp_tile_start(smem, p, T, L, q);
        wait_vmcnt<0>();
        if (need_epi) {
            float *sa, *sb;
            uint16_t* bias;
            epi_area(0, sa, sb, bias);
            pp_params_store(pv, tid, sa, sb, bias);
        }
    }
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);

    for (int u = wg; u < num_units; u += G, parity ^= 1) {
        acc_t acc[FN][FM];
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = acc_t{};
        v8i fa[KSTEPS][FM], fb[KSTEPS][FN];
        float *epi_sa, *epi_sb;
        uint16_t* epi_bias;
        epi_area(parity, epi_sa, epi_sb, epi_bias);

        if (grp == 0) {
            for (int s = 0; s < T.n; ++s) {
                // memory phase 2s: fragments of slice s, B of slice s+1
                pp_read(fa, fb, smem + (s & 1) * STAGE_BYTES, 0, q, pp_lane());
                if (s + 1 < T.n) pp_load_b(smem, (s + 1) & 1, q, pp_slice(T, s + 1), T.rb, L, p.K);
                barrier_lds();
                __builtin_amdgcn_sched_barrier(0);
                // compute phase 2s+1
                pp_compute<FMT>(acc, fa, fb);
                __builtin_amdgcn_sched_barrier(0);
                wait_vmcnt<0>();
                barrier_lds();
                __builtin_amdgcn_sched_barrier(0);
            }
            // Between units: this unit's outputs first (with split-K, only
            // from the tile's last arriving unit), while group 1 runs its last
            // compute phase; then, after the barrier that ends it, group 1
            // writes its outputs while this group issues the next unit's
            // parameters and first slices (behind its own stores, ahead of
            // group 1's) and waits for them.  Every stage buffer those loads
            // fill is free by then (group 1's last reads ended before the
            // barrier, and its staging area, A-bottom of buffer 1, is not
            // loaded).  The next barrier ends group 1's epilogue and follows
            // this group's wait, so the next unit's first reads, which take
            // rows all four waves of this group loaded, find them landed.
            const int un = u + G;
            if (!split || pp_split_fixup(acc, p, u, T.t, wave, pp_lane()))
                pp_store(acc, p, T.row0, T.col0, 0, q * 64, epi_sa, epi_sb, epi_bias, s_pt,
                         has_bias, pp_lane(), smem + STG0 + q * STG_BYTES);
            barrier_lds();   // pairs with group 1's last barrier of the tile
            __builtin_amdgcn_sched_barrier(0);
            if (un < num_units) {
                T = pp_tile(p, un, GROUP_M, xcd);
                PpParams pv;
                if (need_epi) pv = pp_params_load(p, T, tid, has_bias);
                pp_tile_start(smem, p, T, L, q);
                wait_vmcnt<0>();
                if (need_epi) {
                    float *sa, *sb;
                    uint16_t* bias;
                    epi_area(parity ^ 1, sa, sb, bias);
                    pp_params_store(pv, tid, sa, sb, bias);
                }
            }
            barrier_lds();   // group 1's outputs issued; this group's first slices landed
            __builtin_amdgcn_sched_barrier(0);
        } else {
            __builtin_amdgcn_s_barrier();   // one phase behind group 0
            __builtin_amdgcn_sched_barrier(0);
            for (int s = 0; s < T.n; ++s) {
                // memory phase 2s+1: fragments of slice s, A-bottom of s+1, A-top of s+2
                pp_read(fa, fb, smem + (s & 1) * STAGE_BYTES, 1, q, pp_lane());
                if (s + 1 < T.n)
                    pp_load_a_half<true>(smem, (s + 1) & 1, q, pp_slice(T, s + 1), T.ra, L, p.K);
                if (s + 2 < T.n)
                    pp_load_a_half<false>(smem, s & 1, q, pp_slice(T, s + 2), T.ra, L, p.K);
                barrier_lds();
                __builtin_amdgcn_sched_barrier(0);
                // compute phase 2s+2
                pp_compute<FMT>(acc, fa, fb);
                __builtin_amdgcn_sched_barrier(0);
                wait_vmcnt<0>();
                barrier_lds();
                __builtin_amdgcn_sched_barrier(0);
            }
            if (!split || pp_split_fixup(acc, p, u, T.t, wave, pp_lane()))
                pp_store(acc, p, T.row0, T.col0, 128, q * 64, epi_sa, epi_sb, epi_bias, s_pt,
                         has_bias, pp_lane(), smem + STG1 + q * STG_BYTES);
            __builtin_amdgcn_s_barrier();   // group 0's first slices of the next unit have landed
            __builtin_amdgcn_sched_barrier(0);
            if (u + G < num_units) T = pp_tile(p, u + G, GROUP_M, xcd);
        }
    }
}

template <int GROUP_M, int FMT>
void launch_pp(const Params& p, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((fp8_gemm_pp_kernel<GROUP_M, FMT>), grid, dim3(pp::THREADS), 0, stream, p);
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int MI, int GROUP_M,
          bool NT_B, int FMT, bool SK = false>
void launch_cfg(const Params& p, dim3 grid, hipStream_t stream) {
    using C = Cfg<BM, BN, BK, WAVES_M, WAVES_N, STAGES, MI, GROUP_M, NT_B, FMT>;
    hipLaunchKernelGGL((fp8_gemm_kernel<BM, BN, BK, WAVES_M, WAVES_N, STAGES, MI, GROUP_M, NT_B, FMT, SK>),
                       grid, dim3(C::THREADS), 0, stream, p);
}

// The stream-K launch of a configuration, or null where none is compiled.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int MI, int GROUP_M, int FMT>
constexpr Launch stream_k_launch() {
    if constexpr (Cfg<BM, BN, BK, WAVES_M, WAVES_N, STAGES, MI, GROUP_M>::STREAM_K_OK)
        return &launch_cfg<BM, BN, BK, WAVES_M, WAVES_N, STAGES, MI, GROUP_M, false, FMT, true>;
    else
        return nullptr;
}

}  // namespace

#define FP8MM_LAUNCH_PAIR(FMT, name, BM, BN, BK, WMW, WNW, ST, MI, GM)                        \
    LaunchPair{&launch_cfg<BM, BN, BK, WMW, WNW, ST, MI, GM, false, FMT>,                    \
               &launch_cfg<BM, BN, BK, WMW, WNW, ST, MI, GM, true, FMT>,                     \
               stream_k_launch<BM, BN, BK, WMW, WNW, ST, MI, GM, FMT>()},
#define FP8MM_PAIR_F(FMT) FP8MM_PAIR_F_##FMT
#define FP8MM_PAIR_F_0(...) FP8MM_LAUNCH_PAIR(0, __VA_ARGS__)
#define FP8MM_PAIR_F_1(...) FP8MM_LAUNCH_PAIR(1, __VA_ARGS__)
#define FP8MM_PAIR_F_2(...) FP8MM_LAUNCH_PAIR(2, __VA_ARGS__)
#define FP8MM_PAIR_F_3(...) FP8MM_LAUNCH_PAIR(3, __VA_ARGS__)

// Defines fp8mm::NAME: the launch wrappers of every configuration for the
// operand formats FMT (instantiating their kernels).
#define FP8MM_DEFINE_LAUNCH_TABLE(NAME, FMT)                                        \
    namespace fp8mm {                                                             \
    LaunchPair NAME[kNumConfigs] = {                                              \
        FP8MM_GENERIC_CONFIGS(FP8MM_PAIR_F(FMT))                                  \
        LaunchPair{&launch_pp<8, FMT>, nullptr, nullptr}};                        \
    }
