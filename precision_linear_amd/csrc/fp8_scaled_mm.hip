// FP8 (e4m3fn / e5m2) scaled matrix multiply for gfx950 (MI355X, CDNA4): host logic and C ABI.
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
//     then the bf16 tile goes through LDS so that the stores to the output
//     write whole runs of its rows (16, 4 or 2 bytes per lane, as wide as the
//     row alignment allows).
//
// The kernels and their launch wrappers are in fp8_gemm_kernels.h; each
// operand format pair's instances come from fp8_gemm_f<k>.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

#include "../../include/fp8_scaled_mm.h"
#include "fp8_gemm_kernels.h"

namespace {

// ------------------------------------------------------------------ host ---

struct ConfigInfo {
    const char* name;
    int bm, bn, bk;
    bool split_ok;
    int threads;
    int lds_bytes;
    int occupancy;   // workgroups per CU the persistent grid assumes
};

#define FP8MM_CFG_INFO(name, BM, BN, BK, WMW, WNW, ST, MI, GM)                               \
    ConfigInfo{name, BM, BN, BK, Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::SPLIT_OK,             \
               Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::THREADS,                                \
               Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::LDS_BYTES,                              \
               Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::OCCUPANCY},

// Ids are the positions in this table (the C ABI's config_id).
const ConfigInfo kConfigs[kNumConfigs] = {
    FP8MM_GENERIC_CONFIGS(FP8MM_CFG_INFO)
    ConfigInfo{"pp_bm256_bn256_bk128_w8_mfma16", pp::BM, pp::BN, pp::BK, true, pp::THREADS,
               pp::LDS_BYTES, 1},
    FP8MM_GENERIC_CONFIGS_2(FP8MM_CFG_INFO)
};
#undef FP8MM_CFG_INFO

// Launch wrappers by operand formats, then configuration.
LaunchPair* const kLaunch[kFormats] = {kLaunchF0, kLaunchF1, kLaunchF2, kLaunchF3};
constexpr int kMidConfig = 8;         // "bm128_bn128_bk128_w2x4_s4_mfma32"
constexpr int kSkinny16x64 = 1;       // "bm16_bn64_bk256_w1x4_s4_mfma16"
constexpr int kSkinny16x112 = 2;      // "bm16_bn112_bk256_w1x7_s4_mfma16"
constexpr int kSkinny64x112 = 5;      // "bm64_bn112_bk256_w1x7_s3_mfma16"
constexpr int kSkinny64x64 = 6;       // "bm64_bn64_bk256_w1x4_s4_mfma16"
constexpr int kSkinny128x128 = 8;     // "bm128_bn128_bk128_w2x4_s4_mfma32"
constexpr int kNarrow16x32 = 3;       // "bm16_bn32_bk512_w1x2_s6_mfma16"
constexpr int kNarrow128x32 = 17;     // "bm128_bn32_bk256_w4x2_s3_mfma16"
constexpr int kNarrow64x32 = 18;      // "bm64_bn32_bk256_w4x2_s4_mfma16"
constexpr int kNarrow128x64 = 19;     // "bm128_bn64_bk256_w4x2_s3_mfma16"
constexpr int kPingPongConfig = kPingPongId;   // "pp_bm256_bn256_bk128_w8_mfma16"
constexpr int kTwoPerCuConfig = 16;   // "bm128_bn128_bk128_w2x2_s2_mfma32", two workgroups per CU

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int choose_splits(int cfg, int64_t M, int64_t N, int64_t K);

int choose_config(int64_t M, int64_t N, int64_t K, int mode, int has_bias) {
    (void)mode; (void)has_bias;
    // Skinny problems (M <= 128) are HBM-bound on B: tiles as tall as M and
    // 112 columns wide when that gives about one tile per CU (N = 28672 is
    // 256 x 112), else narrower tiles whose K reduction is split until the
    // work units fill the CUs (choose_splits).  Chosen from measurements on
    // MI355X of the six skinny inference shapes.
    // Few columns as well (under 2048, or under 8192 for 128 rows: the
    // column shards of those shapes over 8 GPUs) take narrower tiles, split
    // over K: the last unit of a tile sums every partial of it, and with
    // s splits of a BM x BN tile that fix-up reads s * BM * BN * 4 bytes, so
    // narrower tiles with more of them make it cheaper (MI355X: M=128,
    // K=28672, N=1024: 128 x 128 with 16 splits 30.0 us, 128 x 32 with 8
    // splits 21.8 us).
    const bool wide = cdiv(N, 112) >= 224;
    if (M <= 16) return wide ? kSkinny16x112 : (N < 2048 ? kNarrow16x32 : kSkinny16x64);
    if (M <= 64) return wide ? kSkinny64x112 : (N < 2048 ? kNarrow64x32 : kSkinny64x64);
    if (M <= 128) {
        if (N < 2048) return kNarrow128x32;
        if (N < 8192) return kNarrow128x64;
        return kSkinny128x128;
    }
    // Large grids: 256 x 256 tiles on the ping-pong kernel (needs N % 8 == 0
    // for its 16-byte output rows), also from about 96 tiles on when K is
    // long enough for it to split K.  Other grids of at least 384 tiles of
    // 128 x 128: those tiles with two workgroups per CU, so one's stores
    // overlap the other's loads.  Then the ping-pong kernel down to about 96
    // tiles (it beats 128 x 128 tiles down to there even with CUs idle), else
    // 128 x 128 tiles on 8 waves with split-K when they leave CUs idle.  All
    // from same-box A/B sweeps on MI355X (e.g. 512 x 12288 x 3072: 28.6 us
    // two-per-CU vs 34.2 us ping-pong; 8191 x 1000 x 4160: 44.5 vs 47.5 us;
    // 4095 x 4097 x 96: 26.7 vs 29.0 us on 8 waves).
    const int64_t big_tiles = cdiv(M, 256) * cdiv(N, 256);
    const int64_t tiles128 = cdiv(M, 128) * cdiv(N, 128);
    const bool pp_ok = N % 8 == 0;
    if (pp_ok && big_tiles >= 192) return kPingPongConfig;
    if (pp_ok && big_tiles >= 96 && choose_splits(kPingPongConfig, M, N, K) > 1)
        return kPingPongConfig;
    if (tiles128 >= 384) return kTwoPerCuConfig;
    if (pp_ok && big_tiles >= 96) return kPingPongConfig;
    // Fewer tiles with a long K: two workgroups per CU, split over K until
    // the units fill those slots (512 x 12288 x 3072: 39.2 -> 35.9 us with 5
    // splits; 1152 x 12288 x 3072: 66.3 -> 60.2 us with 2).
    if (tiles128 < 256 && cdiv(K, 128) >= 48) return kTwoPerCuConfig;
    return kMidConfig;
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

// Split-K factor for a configuration: only when the tile grid leaves most of
// the workgroup slots (256 CUs times the configuration's workgroups per CU)
// idle, and never below 8 K slices per split.  The ping-pong
// kernel's 256 x 256 fp32 partials (256 KiB per unit, written and read back
// through memory) cost about as much as 20-30 of its K slices, so it splits
// at most 3 ways and only into units of at least 40 slices (measured on
// MI355X: 2304 x 3072 x 12288 goes from 112 to 88 us with 2 units of 48
// slices, while 8191 x 1000 x 4160 gets slower with 2 units of 17).
int choose_splits(int cfg, int64_t M, int64_t N, int64_t K) {
    const ConfigInfo& c = kConfigs[cfg];
    if (!c.split_ok) return 1;
    const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
    const int64_t k_iters = cdiv(K, c.bk);
    const int64_t slots = 256 * c.occupancy;   // workgroups the GPU runs at once
    if (tiles * 256 >= 160 * slots) return 1;
    int64_t s = slots / tiles;
    const bool pp = cfg == kPingPongConfig;
    const int64_t min_slices = pp ? 40 : 8;
    if (s > k_iters / min_slices) s = k_iters / min_slices;
    if (s > (pp ? 3 : 16)) s = pp ? 3 : 16;
    return s < 1 ? 1 : (int)s;
}

int64_t grid_for(int cfg, int64_t M, int64_t N, int splits, int cus) {
    const ConfigInfo& c = kConfigs[cfg];
    const int64_t units = cdiv(M, c.bm) * cdiv(N, c.bn) * splits;
    const int64_t slots = (int64_t)cus * c.occupancy;
    return units < slots ? units : slots;
}

// Workspace layout of a split plan: a fixed block of arrival counters (one per
// tile in the generic kernel, one per tile and wave in the ping-pong kernel,
// room for kMaxCounters) followed by one fp32 partial tile per work unit.
// The counter block sits at the same place for every plan, so a workspace
// reused by plans of different shapes never finds stale partials where it
// expects zero counters.
constexpr int64_t kMaxCounters = 65536;
constexpr int64_t kCounterBytes = kMaxCounters * 4;

int counters_per_tile(int cfg) { return cfg == kPingPongConfig ? pp::WAVES : 1; }

// The split count a plan uses: `requested` (> 0) or the automatic choice,
// at most the number of K slices, then the smallest count with the same
// units of ceil(k_iters / splits) slices (so no unit is empty); 1 where the
// configuration cannot split or its counters would not fit.
int plan_splits(int cfg, int64_t M, int64_t N, int64_t K, int requested) {
    const ConfigInfo& c = kConfigs[cfg];
    const int64_t k_iters = cdiv(K, c.bk);
    int64_t sp = requested > 0 ? requested : choose_splits(cfg, M, N, K);
    if (sp > k_iters) sp = k_iters;
    const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
    if (!c.split_ok || tiles * counters_per_tile(cfg) > kMaxCounters) sp = 1;
    if (sp > 1) sp = cdiv(k_iters, cdiv(k_iters, sp));
    return (int)sp;
}

int64_t workspace_bytes(int cfg, int64_t M, int64_t N, int splits) {
    if (splits <= 1) return 0;
    const ConfigInfo& c = kConfigs[cfg];
    const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
    return kCounterBytes + tiles * splits * (int64_t)c.bm * c.bn * 4;
}

// Library-owned split-K workspaces, one per (device, stream): calls on one
// stream are ordered, so a stream's workspace is never used by two launches at
// once.  Created on the first split call (zero-filled), grown when needed,
// kept until the process ends.
struct OwnedWorkspace {
    void* ptr = nullptr;
    int64_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, OwnedWorkspace> g_ws;

int owned_workspace(int dev, hipStream_t stream, int64_t bytes, void** out) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    OwnedWorkspace& w = g_ws[std::make_pair(dev, stream)];
    if (w.bytes < bytes) {
        if (w.ptr) {
            if (hipStreamSynchronize(stream) != hipSuccess) return FP8MM_ERR_LAUNCH;
            (void)hipFree(w.ptr);
            w.ptr = nullptr;
            w.bytes = 0;
        }
        void* p = nullptr;
        if (hipMalloc(&p, (size_t)bytes) != hipSuccess) return FP8MM_ERR_DEVICE;
        // Counters must start at zero; every launch leaves them at zero.
        if (hipMemset(p, 0, (size_t)bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
            (void)hipFree(p);
            return FP8MM_ERR_DEVICE;
        }
        w.ptr = p;
        w.bytes = bytes;
    }
    *out = w.ptr;
    return FP8MM_OK;
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
    return grid_for(id, M, N, 1, num_cus);
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
        case FP8MM_ERR_CONFIG: return "unknown tile configuration or split count";
        case FP8MM_ERR_WORKSPACE: return "workspace smaller than fp8_scaled_mm_workspace_size()";
        case FP8MM_ERR_FORMAT: return "unknown operand format (FP8MM_E4M3FN or FP8MM_E5M2)";
        default: return "unknown status";
    }
}

int fp8_scaled_mm_typed(const void* A, int a_format, const void* B, int b_format,
                        const float* scale_a, const float* scale_b, const void* bias, void* out,
                        int64_t M, int64_t N, int64_t K, int mode, struct ihipStream_t* stream,
                        int config_id, int splits, void* workspace, int64_t workspace_size) {
    if ((a_format != FP8MM_E4M3FN && a_format != FP8MM_E5M2) ||
        (b_format != FP8MM_E4M3FN && b_format != FP8MM_E5M2))
        return FP8MM_ERR_FORMAT;
    const int fmt = (a_format == FP8MM_E5M2 ? 1 : 0) | (b_format == FP8MM_E5M2 ? 2 : 0);
    int st = validate(A, B, scale_a, scale_b, bias, out, M, N, K, mode);
    if (st != FP8MM_OK) return st;
    if (config_id >= kNumConfigs) return FP8MM_ERR_CONFIG;
    if (splits < 0 || splits > 64) return FP8MM_ERR_CONFIG;
    if (M == 0 || N == 0) return FP8MM_OK;
    const int cfg = config_id >= 0 ? config_id : choose_config(M, N, K, mode, bias != nullptr);
    const ConfigInfo& c = kConfigs[cfg];
    const int64_t k_iters = cdiv(K, c.bk);
    const int sp = plan_splits(cfg, M, N, K, splits);
    const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
    if (tiles * sp > INT32_MAX) return FP8MM_ERR_SHAPE;
    const int64_t ws_need = workspace_bytes(cfg, M, N, sp);
    if (workspace && workspace_size < ws_need) return FP8MM_ERR_WORKSPACE;
    if (workspace && ((uintptr_t)workspace & 255)) return FP8MM_ERR_ALIGN;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FP8MM_ERR_DEVICE;
    const int cus = device_cus(dev);
    if (cus <= 0) return FP8MM_ERR_DEVICE;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);

    void* ws = workspace;
    if (ws_need > 0 && !ws) {
        st = owned_workspace(dev, hs, ws_need, &ws);
        if (st != FP8MM_OK) return st;
    }

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
    p.tiles_m = (int)cdiv(M, c.bm);
    p.tiles_n = (int)cdiv(N, c.bn);
    p.num_tiles = (int)tiles;
    p.k_iters = (int)k_iters;
    p.rowwise = mode == FP8MM_ROWWISE;
    p.vec_store = (N % 4 == 0) && aligned(out, 8);
    p.vec16 = (N % 8 == 0) && aligned(out, 16);
    p.vec4 = (N % 2 == 0) && aligned(out, 4);
    p.splits = sp;
    p.k_chunk = (int)cdiv(k_iters, sp);
    p.counters = nullptr;
    p.partials = nullptr;
    if (sp > 1) {
        p.counters = static_cast<unsigned*>(ws);
        p.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
    }

    const dim3 grid((unsigned)grid_for(cfg, M, N, sp, cus));
    (void)hipGetLastError();  // clear a stale error from earlier, unrelated calls
    const LaunchPair& l = kLaunch[fmt][cfg];
    if (p.tiles_m == 1 && l.stream) l.stream(p, grid, hs);
    else l.plain(p, grid, hs);
    if (hipGetLastError() != hipSuccess) return FP8MM_ERR_LAUNCH;
    return FP8MM_OK;
}

int fp8_scaled_mm_with_plan(const void* A, const void* B, const float* scale_a,
                            const float* scale_b, const void* bias, void* out, int64_t M, int64_t N,
                            int64_t K, int mode, struct ihipStream_t* stream, int config_id,
                            int splits, void* workspace, int64_t workspace_size) {
    return fp8_scaled_mm_typed(A, FP8MM_E4M3FN, B, FP8MM_E4M3FN, scale_a, scale_b, bias, out, M, N,
                               K, mode, stream, config_id, splits, workspace, workspace_size);
}

int fp8_scaled_mm_with_config(const void* A, const void* B, const float* scale_a,
                              const float* scale_b, const void* bias, void* out, int64_t M,
                              int64_t N, int64_t K, int mode, struct ihipStream_t* stream,
                              int config_id) {
    return fp8_scaled_mm_with_plan(A, B, scale_a, scale_b, bias, out, M, N, K, mode, stream,
                                   config_id, 0, nullptr, 0);
}

int fp8_scaled_mm(const void* A, const void* B, const float* scale_a, const float* scale_b,
                  const void* bias, void* out, int64_t M, int64_t N, int64_t K, int mode,
                  struct ihipStream_t* stream) {
    return fp8_scaled_mm_with_plan(A, B, scale_a, scale_b, bias, out, M, N, K, mode, stream, -1, 0,
                                   nullptr, 0);
}

int fp8_scaled_mm_select_splits(int64_t M, int64_t N, int64_t K, int mode, int has_bias,
                                int config_id) {
    if (mode != FP8MM_PER_TENSOR && mode != FP8MM_ROWWISE) return -1;
    if (M <= 0 || N <= 0 || K < 16 || K % 16 != 0 || config_id >= kNumConfigs) return -1;
    const int cfg = config_id >= 0 ? config_id : choose_config(M, N, K, mode, has_bias);
    return plan_splits(cfg, M, N, K, 0);
}

int64_t fp8_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K, int mode, int has_bias,
                                     int config_id, int splits) {
    if (mode != FP8MM_PER_TENSOR && mode != FP8MM_ROWWISE) return -1;
    if (M <= 0 || N <= 0 || K < 16 || K % 16 != 0 || config_id >= kNumConfigs) return 0;
    const int cfg = config_id >= 0 ? config_id : choose_config(M, N, K, mode, has_bias);
    return workspace_bytes(cfg, M, N, plan_splits(cfg, M, N, K, splits));
}

}  // extern "C"
