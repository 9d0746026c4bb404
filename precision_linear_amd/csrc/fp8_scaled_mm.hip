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

#include <string.h>

#include <mutex>

#include "../../include/fp8_scaled_mm.h"
#include "fp8_gemm_kernels.h"
#include "plan_cost_table.h"

namespace {

// ------------------------------------------------------------------ host ---

struct ConfigInfo {
    const char* name;
    int bm, bn, bk;
    bool split_ok;
    int threads;
    int lds_bytes;
    int occupancy;   // workgroups per CU the persistent grid assumes
    bool stream_k_ok;
};

#define FP8MM_CFG_INFO(name, BM, BN, BK, WMW, WNW, ST, MI, GM)                               \
    ConfigInfo{name, BM, BN, BK, Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::SPLIT_OK,             \
               Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::THREADS,                                \
               Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::LDS_BYTES,                              \
               Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::OCCUPANCY,                              \
               Cfg<BM, BN, BK, WMW, WNW, ST, MI, GM>::STREAM_K_OK},

// Ids are the positions in this table (the C ABI's config_id).
const ConfigInfo kConfigs[kNumConfigs] = {
    FP8MM_GENERIC_CONFIGS(FP8MM_CFG_INFO)
    ConfigInfo{"pp_bm256_bn256_bk128_w8_mfma16", pp::BM, pp::BN, pp::BK, true, pp::THREADS,
               pp::LDS_BYTES, 1, false},
};
#undef FP8MM_CFG_INFO

// Launch wrappers by operand formats, then configuration.
LaunchPair* const kLaunch[kFormats] = {kLaunchF0, kLaunchF1, kLaunchF2, kLaunchF3};
constexpr int kNarrow16x32 = 0;       // "bm16_bn32_bk512_w1x2_s6_mfma16"
constexpr int kSkinny16x64 = 1;       // "bm16_bn64_bk256_w1x4_s4_mfma16"
constexpr int kSkinny16x112 = 2;      // "bm16_bn112_bk256_w1x7_s4_mfma16"
constexpr int kNarrow64x32 = 3;       // "bm64_bn32_bk256_w4x2_s4_mfma16"
constexpr int kSkinny64x64 = 4;       // "bm64_bn64_bk256_w1x4_s4_mfma16"
constexpr int kSkinny64x112 = 5;      // "bm64_bn112_bk256_w1x7_s3_mfma16"
constexpr int kNarrow128x32 = 6;      // "bm128_bn32_bk256_w4x2_s3_mfma16"
constexpr int kNarrow128x64 = 7;      // "bm128_bn64_bk256_w4x2_s3_mfma16"
constexpr int kMidConfig = 8;         // "bm128_bn128_bk128_w2x4_s4_mfma32"
constexpr int kSkinny128x128 = kMidConfig;
constexpr int kTwoPerCuConfig = 9;    // "bm128_bn128_bk128_w2x2_s2_mfma32", two workgroups per CU
constexpr int kThreePerCuConfig = 10; // "bm64_bn128_bk128_w2x2_s2_mfma32", three workgroups per CU
constexpr int kPingPongConfig = kPingPongId;   // "pp_bm256_bn256_bk128_w8_mfma16"

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int fixed_rule_splits(int cfg, int64_t M, int64_t N, int64_t K);

// A grid of at least 384 tiles of 128 x 128 whose K is one slice (the output
// write is the bound) and whose rows are not 16-byte aligned (N % 8 != 0):
// 64 x 128 tiles three per CU keep more output stores overlapping other
// workgroups' loads (MI355X: 4095 x 4097 x 96 18.3 us against 20.2 us with
// 128 x 128 tiles two per CU; 16.9 against 18.4 us back to back).  With
// aligned rows the 256 x 256 or two-per-CU tiles are faster.
bool write_bound_unaligned(int64_t M, int64_t N, int64_t K) {
    return N % 8 != 0 && K <= 128 && cdiv(M, 128) * cdiv(N, 128) >= 384;
}

// The tile configuration for a call that may split K.
int choose_config_split(int64_t M, int64_t N, int64_t K) {
    // Skinny problems (M <= 128) are HBM-bound on B: tiles as tall as M and
    // 112 columns wide when that gives about one tile per CU (N = 28672 is
    // 256 x 112), else narrower tiles whose K reduction is split until the
    // work units fill the CUs (fixed_rule_splits).  Chosen from measurements on
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
    // 4095 x 4097 x 96: 19.3 vs 23.2 us on 8 waves).
    const int64_t big_tiles = cdiv(M, 256) * cdiv(N, 256);
    const int64_t tiles128 = cdiv(M, 128) * cdiv(N, 128);
    const bool pp_ok = N % 8 == 0;
    if (pp_ok && big_tiles >= 192) return kPingPongConfig;
    if (pp_ok && big_tiles >= 96 && fixed_rule_splits(kPingPongConfig, M, N, K) > 1)
        return kPingPongConfig;
    if (write_bound_unaligned(M, N, K)) return kThreePerCuConfig;
    if (tiles128 >= 384) return kTwoPerCuConfig;
    if (pp_ok && big_tiles >= 96) return kPingPongConfig;
    // Fewer tiles with a long K: two workgroups per CU, split over K until
    // the units fill those slots (512 x 12288 x 3072: 39.2 -> 35.9 us with 5
    // splits; 1152 x 12288 x 3072: 66.3 -> 60.2 us with 2).
    if (tiles128 < 256 && cdiv(K, 128) >= 48) return kTwoPerCuConfig;
    return kMidConfig;
}

// The tile configuration for a call that cannot split K, where the plan
// above would: the tallest tile (of at most M rows) whose grid has at least
// 200 tiles, else the smallest tile; for larger M, 128 x 128 tiles two per
// CU or on 8 waves, or 128 x 64.  From a sweep of every configuration
// without split-K on MI355X: M=128, K=28672, N=1024: 16 x 32 tiles (256 of
// them) 40 us against 73 us with 128 x 32; M=64, K=8192, N=3584: 16 x 64
// tiles 18 us; 512 x 3072 x 12288: 128 x 64 tiles 44 us against 76 us with
// 128 x 128 two per CU.
int choose_config_nosplit(int64_t M, int64_t N, int64_t K) {
    auto tiles = [&](int cfg) { return cdiv(M, kConfigs[cfg].bm) * cdiv(N, kConfigs[cfg].bn); };
    if (M <= 128) {
        const int order[] = {kNarrow128x32, kNarrow64x32, kSkinny16x64, kNarrow16x32};
        for (int cfg : order)
            if (kConfigs[cfg].bm <= (M <= 16 ? 16 : M <= 64 ? 64 : 128) && tiles(cfg) >= 200)
                return cfg;
        return kNarrow16x32;
    }
    const int64_t tiles128 = cdiv(M, 128) * cdiv(N, 128);
    if (write_bound_unaligned(M, N, K)) return kThreePerCuConfig;
    if (tiles128 >= 384) return kTwoPerCuConfig;
    if (tiles128 >= 160) return kMidConfig;
    return tiles(kNarrow128x64) > tiles128 ? kNarrow128x64 : kMidConfig;
}

// ---------------------------------------------------------- plan model ---

static_assert(sizeof(kPlanCost_streamed) / sizeof(PlanCostRow) == kNumConfigs &&
                  sizeof(kPlanCost_resident) / sizeof(PlanCostRow) == kNumConfigs,
              "plan cost tables need one row per configuration (re-run plan_fit.py)");

// Grids that the 256 x 256 tiles fill (at least 192 of them, N % 8 == 0) or
// that have more than 1536 tiles of 128 x 128 take the fixed rules above.
// So do grids whose K is one slice and whose rows are not 16-byte aligned
// (write_bound_unaligned: the measurements behind the model have aligned
// rows).  Every other grid takes the plan -- tile configuration and split
// count -- of least predicted time under a cost model fitted to
// measurements on MI355X of every plan on a few hundred shapes (M from 16 to
// 8192, N from 256 to 28672, K from 128 to 28672; plan_sweep.py,
// plan_fit.py): a linear function, per configuration, of the features below.
// Two coefficient tables: M <= 128 (fitted on launches whose operands come
// from HBM, as a decode step's weights do) and M > 128 (operands left in the
// caches).  On held-out shapes the chosen plan ran within 1.2-1.4% of the
// fastest measured one (geometric mean), where the fixed rules alone were
// 14-17% off.
bool plan_modelled(int64_t M, int64_t N, int64_t K) {
    const bool pp_fills = N % 8 == 0 && cdiv(M, 256) * cdiv(N, 256) >= 192;
    return !pp_fills && cdiv(M, 128) * cdiv(N, 128) <= 1536 && !write_bound_unaligned(M, N, K);
}

// The split count a plan with `s` requested runs: at most the K slices, then
// the smallest count with the same slices per unit (as plan_splits).
int64_t normalised_splits(int64_t s, int64_t k_iters) {
    if (s > k_iters) s = k_iters;
    return s > 1 ? cdiv(k_iters, cdiv(k_iters, s)) : 1;
}

// Predicted time (us) of configuration cfg with s splits: T tiles, U = T * s
// units, S = 256 * occupancy workgroup slots, R = ceil(U / S) rounds of
// units per slot, Lc = ceil(U / 256) units per CU, kk K slices per unit, act
// = min(U, S) / S the busy fraction of the slots, a = BM * BN / 16384, and
// Lc - U / 256 the busiest CUs' extra load.
double plan_cost(const PlanCostRow& row, const ConfigInfo& c, int64_t M, int64_t N, int64_t K,
                 int64_t s) {
    const int64_t S = 256 * (int64_t)c.occupancy;
    const int64_t T = cdiv(M, c.bm) * cdiv(N, c.bn);
    const int64_t U = T * s;
    const int64_t R = cdiv(U, S);
    const int64_t kk = cdiv(cdiv(K, c.bk), s);
    const double act = (double)(U < S ? U : S) / (double)S;
    const int64_t Lc = cdiv(U, 256);
    const double sp = s > 1 ? 1.0 : 0.0;
    const double a = (double)(c.bm * c.bn) / 16384.0;
    const double f[kPlanFeatures] = {
        1.0, (double)(R * kk), (double)(R * kk) * act, (double)R, sp, sp * (double)s * a,
        sp * (double)R * a, sp * (double)T * (double)s * (double)c.bm * (double)c.bn / 1e6,
        (double)((M + N) * K) / 1e6, sp * (double)s * (double)R * a, (double)(Lc * kk), (double)Lc,
        (double)(Lc * kk) * act, ((double)Lc - (double)U / 256.0) * (double)kk};
    double t = 0.0;
    for (int i = 0; i < kPlanFeatures; ++i) t += row.c[i] * f[i];
    return t;
}

struct Plan {
    int cfg;       // -1: no configuration is modelled here
    int splits;
};

constexpr int kSplitCandidates[] = {2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 24, 32};

// The modelled plan of least predicted time, over every configuration or
// only `only_cfg` (>= 0).  Candidates: configurations fitted for this M, the
// ping-pong kernel only with N % 8 == 0, tile grids of at most 6 rounds of
// slots; split counts (with can_split) leaving at least 2 K slices per unit
// and at most 3 rounds of units, the ping-pong kernel at most 3 ways and
// only into units of at least 40 slices.  Ties keep the earlier candidate.
Plan model_plan(int64_t M, int64_t N, int64_t K, bool can_split, int only_cfg) {
    const PlanCostRow* table = M <= 128 ? kPlanCost_streamed : kPlanCost_resident;
    Plan best{-1, 1};
    double best_t = 0.0;
    auto consider = [&](int cfg, int64_t s) {
        const double t = plan_cost(table[cfg], kConfigs[cfg], M, N, K, s);
        if (best.cfg < 0 || t < best_t) {
            best = Plan{cfg, (int)s};
            best_t = t;
        }
    };
    for (int cfg = 0; cfg < kNumConfigs; ++cfg) {
        if (only_cfg >= 0 && cfg != only_cfg) continue;
        const ConfigInfo& c = kConfigs[cfg];
        if (!table[cfg].usable) continue;
        const bool pp = cfg == kPingPongConfig;
        if (pp && N % 8 != 0) continue;
        const int64_t S = 256 * (int64_t)c.occupancy;
        const int64_t T = cdiv(M, c.bm) * cdiv(N, c.bn);
        if (T > 6 * S) continue;
        consider(cfg, 1);
        if (!can_split || !c.split_ok || !table[cfg].split_usable) continue;
        const int64_t k_iters = cdiv(K, c.bk);
        for (int s : kSplitCandidates) {
            if (2 * s > k_iters || T * s > 3 * S) continue;
            if (pp && (s > 3 || k_iters / s < 40)) continue;
            consider(cfg, normalised_splits(s, k_iters));
        }
    }
    return best;
}

// model_plan's results, per thread and direct-mapped (64 entries): weighing
// every candidate plan takes a few microseconds of host time, and a caller
// usually repeats a few shapes (a network's layers), each then planned once.
// `key` is 1 + 2 * (only_cfg + 1) + can_split, so a zeroed entry matches no
// query.
struct PlanMemo {
    int64_t M, N, K;
    int key;
    Plan plan;
};
thread_local PlanMemo t_plan_memo[64];

Plan model_plan_memo(int64_t M, int64_t N, int64_t K, bool can_split, int only_cfg) {
    const int key = 1 + 2 * (only_cfg + 1) + (can_split ? 1 : 0);
    const uint64_t h = (uint64_t)M * 0x9E3779B97F4A7C15ull ^ (uint64_t)N * 0xC2B2AE3D27D4EB4Full ^
                       (uint64_t)K * 0x165667B19E3779F9ull ^ (uint64_t)key * 0xD6E8FEB86659FD93ull;
    PlanMemo& e = t_plan_memo[h >> 58];
    if (e.key == key && e.M == M && e.N == N && e.K == K) return e.plan;
    const Plan p = model_plan(M, N, K, can_split, only_cfg);
    e = PlanMemo{M, N, K, key, p};
    return p;
}

// The automatic tile configuration.  can_split: the call has a workspace for
// split-K partials; without one, K is never split, and where the plan with a
// workspace would split, narrower tiles take its place.
int choose_config(int64_t M, int64_t N, int64_t K, int mode, int has_bias, bool can_split) {
    (void)mode; (void)has_bias;
    if (plan_modelled(M, N, K)) {
        const Plan p = model_plan_memo(M, N, K, can_split, -1);
        if (p.cfg >= 0) return p.cfg;
    }
    const int cfg = choose_config_split(M, N, K);
    if (can_split || fixed_rule_splits(cfg, M, N, K) <= 1) return cfg;
    return choose_config_nosplit(M, N, K);
}

// The automatic split count of a configuration: the modelled plan's for
// that configuration, else the fixed rule.
int choose_splits(int cfg, int64_t M, int64_t N, int64_t K) {
    if (plan_modelled(M, N, K)) {
        const Plan p = model_plan_memo(M, N, K, true, cfg);
        if (p.cfg >= 0) return p.splits;
    }
    return fixed_rule_splits(cfg, M, N, K);
}

// Per-device facts, read once per device: the compute-unit count and whether
// the device is a gfx950 (the kernels are built for it only).  0 = not read
// yet; a lost race only reads them twice.
constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices];
int g_arch_ok[kMaxDevices];   // 1: gfx950, 2: another architecture

int device_cus(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return 0;
    if (__atomic_load_n(&g_arch_ok[dev], __ATOMIC_ACQUIRE) == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
        const bool gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                            (prop.gcnArchName[6] == 0 || prop.gcnArchName[6] == ':');
        __atomic_store_n(&g_cus[dev], prop.multiProcessorCount, __ATOMIC_RELAXED);
        __atomic_store_n(&g_arch_ok[dev], gfx950 ? 1 : 2, __ATOMIC_RELEASE);
    }
    if (__atomic_load_n(&g_arch_ok[dev], __ATOMIC_ACQUIRE) != 1) return 0;
    return __atomic_load_n(&g_cus[dev], __ATOMIC_RELAXED);
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

// Split-K factor of the fixed rules (grids the plan model leaves out, see
// plan_modelled): only when the tile grid leaves most of
// the workgroup slots (256 CUs times the configuration's workgroups per CU)
// idle, and never below 8 K slices per split.  The ping-pong
// kernel's 256 x 256 fp32 partials (256 KiB per unit, written and read back
// through memory) cost about as much as 20-30 of its K slices, so it splits
// at most 3 ways and only into units of at least 40 slices (measured on
// MI355X: 2304 x 3072 x 12288 goes from 112 to 88 us with 2 units of 48
// slices, while 8191 x 1000 x 4160 gets slower with 2 units of 17).
int fixed_rule_splits(int cfg, int64_t M, int64_t N, int64_t K) {
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

// Stream-K: the grid's g workgroups share the tiles * k_iters (tile, K slice)
// iterations, workgroup w from floor(w * total / g) on, so the range starts
// inside one tile (k_iters long) number at most ceil(g / tiles), and the
// workgroups meeting a tile at most ceil(g / tiles) + 1 (checked by brute force
// over random tile counts, K lengths and grids): the room for partial tiles
// per tile.  Workspace sizes use the largest grid a device can have
// (kMaxSlots workgroups); the bound grows with g, so it covers every smaller
// grid.
constexpr int64_t kMaxSlots = 1024;

int64_t sk_segments(int64_t tiles, int64_t k_iters, int64_t g) {
    const int64_t total = tiles * k_iters;
    if (g > total) g = total;
    const int64_t m = cdiv(g, tiles) + 1;
    return m < g ? m : g;
}

// Device scratch for fp8_scaled_mm_noalloc: its split-K counters and partial
// tiles, for callers that cannot allocate.  Each GPU the library runs on
// holds one copy from module load until the process ends; every call on that
// GPU shares it.  In host code `scratch` names a host-side stand-in, not the
// device memory: kernels and copies get the device address that
// hipGetSymbolAddress returns, resolved once per device.
constexpr int64_t kScratchBytes = int64_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on device `dev` (the current device), or
// null if the runtime cannot give it.
void* scratch_on(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

// Zeroes n arrival counters (a kernel, not a memset, so that it can be
// captured into a graph like the multiply that follows it).
__global__ void __launch_bounds__(256) clear_counters_kernel(unsigned* c, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) c[i] = 0u;
}

// Where a call's split-K workspace comes from.
enum class WsSource { kNone, kCaller, kScratch };

Params base_params(const void* A, const void* B, const float* scale_a, const float* scale_b,
                   const void* bias, void* out, int64_t M, int64_t N, int64_t K, int mode,
                   const ConfigInfo& c) {
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
    p.num_tiles = p.tiles_m * p.tiles_n;
    p.k_iters = (int)cdiv(K, c.bk);
    p.rowwise = mode == FP8MM_ROWWISE;
    p.vec_store = (N % 4 == 0) && aligned(out, 8);
    p.vec16 = (N % 8 == 0) && aligned(out, 16);
    p.splits = 1;
    p.k_chunk = p.k_iters;
    p.counters = nullptr;
    p.partials = nullptr;
    return p;
}

// A stream-K plan (splits == FP8MM_SPLITS_STREAM_K): every workgroup slot of
// the GPU takes an equal share of the (tile, K slice) iterations; the tiles
// that several workgroups share are finished through partials and counters
// as in split-K.  Configurations with a stream-K kernel only (the 128 x 128
// tiles); validated arguments.
int run_stream_k(const void* A, int fmt, const void* B, const float* scale_a, const float* scale_b,
                 const void* bias, void* out, int64_t M, int64_t N, int64_t K, int mode,
                 struct ihipStream_t* stream, int config_id, void* workspace, int64_t workspace_size,
                 WsSource src) {
    const bool can_split = src != WsSource::kNone;
    if (!can_split) return FP8MM_ERR_WORKSPACE;
    const int cfg = config_id >= 0 ? config_id : choose_config(M, N, K, mode, bias != nullptr, true);
    const ConfigInfo& c = kConfigs[cfg];
    if (!c.stream_k_ok) return FP8MM_ERR_CONFIG;
    const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
    const int64_t k_iters = cdiv(K, c.bk);
    if (tiles > kMaxCounters || tiles * k_iters > INT32_MAX) return FP8MM_ERR_SHAPE;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FP8MM_ERR_DEVICE;
    const int cus = device_cus(dev);
    if (cus <= 0) return FP8MM_ERR_DEVICE;
    int64_t g = (int64_t)cus * c.occupancy;
    if (g > kMaxSlots) g = kMaxSlots;
    if (g > tiles * k_iters) g = tiles * k_iters;
    const int64_t segs = sk_segments(tiles, k_iters, g);
    const int64_t ws_need = kCounterBytes + tiles * segs * (int64_t)c.bm * c.bn * 4;
    if (src == WsSource::kCaller) {
        if (workspace_size < ws_need) return FP8MM_ERR_WORKSPACE;
        if ((uintptr_t)workspace & 255) return FP8MM_ERR_ALIGN;
    } else if (ws_need > kScratchBytes) {
        return FP8MM_ERR_SCRATCH;
    }
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    void* ws = workspace;
    (void)hipGetLastError();
    if (src == WsSource::kScratch) {
        ws = scratch_on(dev);
        if (!ws) return FP8MM_ERR_DEVICE;
        const int n = (int)tiles;
        const int blocks = (n + 255) / 256 < 256 ? (n + 255) / 256 : 256;
        hipLaunchKernelGGL(clear_counters_kernel, dim3(blocks), dim3(256), 0, hs,
                           static_cast<unsigned*>(ws), n);
    }
    Params p = base_params(A, B, scale_a, scale_b, bias, out, M, N, K, mode, c);
    p.splits = (int)segs;
    p.counters = static_cast<unsigned*>(ws);
    p.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
    kLaunch[fmt][cfg].stream_k(p, dim3((unsigned)g), hs);
    if (hipGetLastError() != hipSuccess) return FP8MM_ERR_LAUNCH;
    return FP8MM_OK;
}

int run_mm(const void* A, int a_format, const void* B, int b_format, const float* scale_a,
           const float* scale_b, const void* bias, void* out, int64_t M, int64_t N, int64_t K,
           int mode, struct ihipStream_t* stream, int config_id, int splits, void* workspace,
           int64_t workspace_size, WsSource src) {
    if ((a_format != FP8MM_E4M3FN && a_format != FP8MM_E5M2) ||
        (b_format != FP8MM_E4M3FN && b_format != FP8MM_E5M2))
        return FP8MM_ERR_FORMAT;
    const int fmt = (a_format == FP8MM_E5M2 ? 1 : 0) | (b_format == FP8MM_E5M2 ? 2 : 0);
    int st = validate(A, B, scale_a, scale_b, bias, out, M, N, K, mode);
    if (st != FP8MM_OK) return st;
    if (config_id >= kNumConfigs) return FP8MM_ERR_CONFIG;
    if (splits < FP8MM_SPLITS_STREAM_K || splits > 64) return FP8MM_ERR_CONFIG;
    if (M == 0 || N == 0) return FP8MM_OK;
    if (splits == FP8MM_SPLITS_STREAM_K)
        return run_stream_k(A, fmt, B, scale_a, scale_b, bias, out, M, N, K, mode, stream, config_id,
                            workspace, workspace_size, src);
    // K is split only where the partial tiles have somewhere to go: without a
    // workspace the automatic plan does not split, and an explicit split
    // count that still splits after clamping to the K slices is refused.
    const bool can_split = src != WsSource::kNone;
    const int cfg = config_id >= 0 ? config_id : choose_config(M, N, K, mode, bias != nullptr, can_split);
    const ConfigInfo& c = kConfigs[cfg];
    const int64_t k_iters = cdiv(K, c.bk);
    int sp = plan_splits(cfg, M, N, K, can_split || splits > 1 ? splits : 1);
    if (!can_split && sp > 1) return FP8MM_ERR_WORKSPACE;
    if (src == WsSource::kScratch && workspace_bytes(cfg, M, N, sp) > kScratchBytes) {
        if (splits > 1) return FP8MM_ERR_SCRATCH;       // asked for a plan that does not fit
        while (sp > 1 && workspace_bytes(cfg, M, N, sp) > kScratchBytes)
            sp = plan_splits(cfg, M, N, K, sp - 1);
    }
    const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
    if (tiles * sp > INT32_MAX) return FP8MM_ERR_SHAPE;
    const int64_t ws_need = workspace_bytes(cfg, M, N, sp);
    if (src == WsSource::kCaller) {
        if (workspace_size < ws_need) return FP8MM_ERR_WORKSPACE;
        if ((uintptr_t)workspace & 255) return FP8MM_ERR_ALIGN;
    }

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FP8MM_ERR_DEVICE;
    const int cus = device_cus(dev);
    if (cus <= 0) return FP8MM_ERR_DEVICE;
    const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);

    void* ws = src == WsSource::kCaller ? workspace : nullptr;
    (void)hipGetLastError();  // clear a stale error from earlier, unrelated calls
    if (src == WsSource::kScratch && sp > 1) {
        ws = scratch_on(dev);
        if (!ws) return FP8MM_ERR_DEVICE;
        // The scratch keeps whatever the last call on this GPU left in it:
        // the counters this plan uses start from zero.
        const int n = (int)(tiles * counters_per_tile(cfg));
        const int blocks = (n + 255) / 256 < 256 ? (n + 255) / 256 : 256;
        hipLaunchKernelGGL(clear_counters_kernel, dim3(blocks), dim3(256), 0, hs,
                           static_cast<unsigned*>(ws), n);
    }

    Params p = base_params(A, B, scale_a, scale_b, bias, out, M, N, K, mode, c);
    p.splits = sp;
    p.k_chunk = (int)cdiv(k_iters, sp);
    if (sp > 1) {
        p.counters = static_cast<unsigned*>(ws);
        p.partials = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
    }

    const dim3 grid((unsigned)grid_for(cfg, M, N, sp, cus));
    const LaunchPair& l = kLaunch[fmt][cfg];
    if (p.tiles_m == 1 && l.stream) l.stream(p, grid, hs);
    else l.plain(p, grid, hs);
    if (hipGetLastError() != hipSuccess) return FP8MM_ERR_LAUNCH;
    return FP8MM_OK;
}

}  // namespace

extern "C" {

int fp8_scaled_mm_num_configs(void) { return kNumConfigs; }

const char* fp8_scaled_mm_config_name(int id) {
    return (id >= 0 && id < kNumConfigs) ? kConfigs[id].name : "";
}

int fp8_scaled_mm_select_config(int64_t M, int64_t N, int64_t K, int mode, int has_bias,
                                int with_workspace) {
    if (mode != FP8MM_PER_TENSOR && mode != FP8MM_ROWWISE) return -1;
    if (M < 0 || N < 0 || K < 16 || K % 16 != 0) return -1;
    return choose_config(M, N, K, mode, has_bias, with_workspace != 0);
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
        case FP8MM_ERR_ALIGN: return "misaligned pointer (A,B: 16 B; scales: 4 B; bias,out: 2 B; workspace: 256 B)";
        case FP8MM_ERR_MODE: return "unknown scaling mode";
        case FP8MM_ERR_DEVICE: return "no usable gfx950 device";
        case FP8MM_ERR_LAUNCH: return "kernel launch failed";
        case FP8MM_ERR_CONFIG: return "unknown tile configuration or split count";
        case FP8MM_ERR_WORKSPACE:
            return "split-K needs a workspace of at least fp8_scaled_mm_workspace_size() bytes";
        case FP8MM_ERR_FORMAT: return "unknown operand format (FP8MM_E4M3FN or FP8MM_E5M2)";
        case FP8MM_ERR_SCRATCH:
            return "the requested split-K plan needs more than the 64 MiB device scratch of "
                   "fp8_scaled_mm_noalloc";
        default: return "unknown status";
    }
}

const char* fp8mm_status_string(int s) { return fp8_scaled_mm_status_string(s); }

int fp8_scaled_mm_typed(const void* A, int a_format, const void* B, int b_format,
                        const float* scale_a, const float* scale_b, const void* bias, void* out,
                        int64_t M, int64_t N, int64_t K, int mode, struct ihipStream_t* stream,
                        int config_id, int splits, void* workspace, int64_t workspace_size) {
    return run_mm(A, a_format, B, b_format, scale_a, scale_b, bias, out, M, N, K, mode, stream,
                  config_id, splits, workspace, workspace_size,
                  workspace ? WsSource::kCaller : WsSource::kNone);
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

int fp8_scaled_mm_noalloc(const void* A, const void* B, const float* scale_a,
                          const float* scale_b, const void* bias, void* out, int64_t M, int64_t N,
                          int64_t K, int mode, struct ihipStream_t* stream, int config_id,
                          int splits) {
    return run_mm(A, FP8MM_E4M3FN, B, FP8MM_E4M3FN, scale_a, scale_b, bias, out, M, N, K, mode,
                  stream, config_id, splits, nullptr, 0, WsSource::kScratch);
}

int fp8_scaled_mm_select_splits(int64_t M, int64_t N, int64_t K, int mode, int has_bias,
                                int config_id) {
    if (mode != FP8MM_PER_TENSOR && mode != FP8MM_ROWWISE) return -1;
    if (M <= 0 || N <= 0 || K < 16 || K % 16 != 0 || config_id >= kNumConfigs) return -1;
    const int cfg = config_id >= 0 ? config_id : choose_config(M, N, K, mode, has_bias, true);
    return plan_splits(cfg, M, N, K, 0);
}

int64_t fp8_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K, int mode, int has_bias,
                                     int config_id, int splits) {
    if (mode != FP8MM_PER_TENSOR && mode != FP8MM_ROWWISE) return -1;
    if (M <= 0 || N <= 0 || K < 16 || K % 16 != 0 || config_id >= kNumConfigs) return 0;
    if (splits < FP8MM_SPLITS_STREAM_K || splits > 64) return 0;
    const int cfg = config_id >= 0 ? config_id : choose_config(M, N, K, mode, has_bias, true);
    if (splits == FP8MM_SPLITS_STREAM_K) {
        const ConfigInfo& c = kConfigs[cfg];
        if (!c.stream_k_ok) return 0;
        const int64_t tiles = cdiv(M, c.bm) * cdiv(N, c.bn);
        const int64_t k_iters = cdiv(K, c.bk);
        return kCounterBytes + tiles * sk_segments(tiles, k_iters, kMaxSlots) * (int64_t)c.bm * c.bn * 4;
    }
    return workspace_bytes(cfg, M, N, plan_splits(cfg, M, N, K, splits));
}

}  // extern "C"
