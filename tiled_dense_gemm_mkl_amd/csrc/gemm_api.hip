// gemm_api.hip -- the C ABI (include/gemm_mkl.h): argument checks, the
// configuration choice, the split-K workspace and the kernel launches.
//
// The boundary takes plain device pointers, sizes, a dtype, an epilogue and a
// stream, as the GEMM entry of "深入解析 CUTLASS CuTe DSL 的 JIT 函数参数生成机制"
// (section 2.3) takes tensors, a stream and a compile-time epilogue.  Bad
// arguments are rejected before any HIP call, with a code that names the
// problem (the type-check errors of section 3.1 there); a negative prefetch
// depth is rejected as the loop-attribute diagnostic of section 3 of
// "CUTLASS CuTe DSL 控制流编程指南" does.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/gemm_mkl.h"
#include "configs.hpp"

using namespace gmk;

// ---------------------------------------------------------------- the allocation-free variant

// Device scratch of gemm_mkl_noalloc: its split-K partial sums and repacked
// operands live here instead of in memory the library allocates.  One copy
// per device, allocated with the code object when the library is loaded on
// that device and held until the process ends.  In host code `scratch` only
// names the symbol; its device address comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = GEMM_MKL_NOALLOC_SCRATCH_BYTES;
// Its last MiB holds the split-K fix-up's per-tile counter words: zero when
// the library is loaded, nothing else writes there, and every completed call
// leaves them zero.  Partial sums and repacked operands use the rest.
constexpr size_t kScratchCounterBytes = (size_t)1 << 20;
constexpr size_t kScratchDataBytes = kScratchBytes - kScratchCounterBytes;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kNumCUs = 256;          // MI355X compute units (8 XCDs x 32)
constexpr double kMallBytes = 256.0 * (1 << 20);   // memory-side (Infinity) cache
constexpr int64_t kMaxSplit = 16;
constexpr int64_t kMaxGroups = 65536;   // grouped GEMM: groups per call
constexpr int64_t kMaxFixupTiles = 8192;   // fix-up counter lines (the no-alloc scratch keeps 1 MiB of them)

struct Registry {
    std::vector<ConfigEntry> table;
    DtypeKernels k[3];
    Registry()
    {
        register_f32(table, k[GEMM_MKL_F32]);
        register_f16(table, k[GEMM_MKL_F16]);
        register_bf16(table, k[GEMM_MKL_BF16]);
    }
};

Registry &registry()
{
    static Registry r;
    return r;
}

thread_local hipError_t t_last_hip = hipSuccess;
thread_local char t_hip_msg[192];

int elem_bytes(int dtype) { return dtype == GEMM_MKL_F32 ? 4 : 2; }

int env_int(const char *name, int dflt)
{
    const char *v = std::getenv(name);
    if (!v || !*v) return dflt;
    return std::atoi(v);
}

// The environment overrides, read once, at the first call that needs them.
struct EnvSettings {
    int force_config, stages, split_k, streamk, group_m, grouped_group_m, log, persistent, fixup;
    bool has_ws_limit;
    size_t ws_limit;
    EnvSettings()
        : force_config(env_int("GEMM_MKL_FORCE_CONFIG", -1)), stages(env_int("GEMM_MKL_STAGES", -1)),
          split_k(env_int("GEMM_MKL_SPLIT_K", 0)), streamk(env_int("GEMM_MKL_STREAMK", 0)),
          group_m(env_int("GEMM_MKL_GROUP_M", 4)),
          // the grouped kernel's raster height inside a group: on 4096 rows in
          // 8 groups x 5632 x 2048 bf16 (256 x 256 tiles) heights 1, 2, 3, 4,
          // 6, 8 and 16 read FETCH_SIZE 217, 169, 144, 145, 140, 148 and 142
          // thousand KiB per call, at 104-110 us per call
          grouped_group_m(env_int("GEMM_MKL_GROUP_M", 6)), log(env_int("GEMM_MKL_LOG", 0)),
          persistent(env_int("GEMM_MKL_PERSISTENT", 0)), fixup(env_int("GEMM_MKL_FIXUP", -1)), has_ws_limit(false),
          ws_limit(0)
    {
        const char *lim = std::getenv("GEMM_MKL_WORKSPACE_LIMIT");
        if (lim && *lim) {
            has_ws_limit = true;
            ws_limit = (size_t)std::strtoull(lim, nullptr, 10);
        }
    }
};

const EnvSettings &env()
{
    static const EnvSettings e;
    return e;
}

bool mul_ok(int64_t a, int64_t b, int64_t *out)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *out = a * b;
    return true;
}

// True when the byte ranges [p, p + pn) and [q, q + qn) share a byte (no end
// address is formed, so ranges near the top of the address space compare
// correctly).
bool overlaps(const void *p, uint64_t pn, const void *q, uint64_t qn)
{
    if (pn == 0 || qn == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a <= b ? b - a < pn : a - b < qn;
}

struct Plan {
    int config_id = -1;
    int P = 0;
    int S = 1;
    bool general = false;
    bool streamk = false;
    bool persistent = false;       // persistent grid with one ring across each workgroup's tiles
    bool fixup = false;            // split-K summed inside the GEMM kernel (no reduction launch)
    int32_t fix_per = 0;           // fix-up: tiles per XCD
    size_t fix_counter_bytes = 0;  // fix-up: per-tile counter words, 256-byte padded
    int64_t sk_units = 0;          // stream-K: tiles (all batches) * chunks per tile
    size_t sk_counter_bytes = 0;   // stream-K: per-tile counters (one 128-byte line each), 256-byte padded
    int64_t grid = 0;
    int32_t tiles_m = 0, tiles_n = 0, group_m = 1;
    int32_t total_chunks = 0, chunks_per_split = 0;
    size_t ws_bytes = 0;
    // operands repacked into zero-padded, 16-byte aligned rows of Kp elements
    // in the workspace (after the split-K partials) before the tile kernel
    bool packed = false, pack_a = false, pack_b = false;
    int64_t Kp = 0;
    size_t off_a = 0, off_b = 0;
};

// Alignment of a call's operands, as the planner sees it.
enum : int {
    kAlignA = 1,     // A 16-byte aligned
    kAlignB = 2,     // B 16-byte aligned
    kAlignC = 4,     // C aligned to 4 elements
    kAlignAll = 7,
};

int check_args(int64_t M, int64_t N, int64_t K, int64_t L, int dtype, int epilogue, const gemm_mkl_opts *o)
{
    if (dtype != GEMM_MKL_F32 && dtype != GEMM_MKL_F16 && dtype != GEMM_MKL_BF16)
        return GEMM_MKL_STATUS_UNSUPPORTED_DTYPE;
    if (epilogue != GEMM_MKL_EPI_IDENTITY && epilogue != GEMM_MKL_EPI_RELU && epilogue != GEMM_MKL_EPI_SILU)
        return GEMM_MKL_STATUS_UNSUPPORTED_EPILOGUE;
    if (M < 0 || N < 0 || K < 0 || L < 0) return GEMM_MKL_STATUS_INVALID_VALUE;
    // every operand's byte size must fit in int64
    const int64_t es = elem_bytes(dtype);
    int64_t t;
    if (!mul_ok(M, K, &t) || !mul_ok(t, L, &t) || !mul_ok(t, es, &t)) return GEMM_MKL_STATUS_INVALID_VALUE;
    if (!mul_ok(N, K, &t) || !mul_ok(t, L, &t) || !mul_ok(t, es, &t)) return GEMM_MKL_STATUS_INVALID_VALUE;
    if (!mul_ok(M, N, &t) || !mul_ok(t, L, &t) || !mul_ok(t, 4 * kMaxSplit, &t))
        return GEMM_MKL_STATUS_INVALID_VALUE;
    if (o) {
        if (o->prefetch_stages < -1) return GEMM_MKL_STATUS_INVALID_VALUE;
        if (o->split_k < 0) return GEMM_MKL_STATUS_INVALID_VALUE;
        if (o->config_id < -1) return GEMM_MKL_STATUS_INVALID_VALUE;
        const int32_t known = GEMM_MKL_OPT_FORCE_GENERAL | GEMM_MKL_OPT_STREAMK | GEMM_MKL_OPT_NO_STREAMK |
                              GEMM_MKL_OPT_PERSISTENT | GEMM_MKL_OPT_NO_PERSISTENT | GEMM_MKL_OPT_FIXUP |
                              GEMM_MKL_OPT_NO_FIXUP | GEMM_MKL_OPT_FIXUP_RECOMPUTE;
        if (o->flags & ~known) return GEMM_MKL_STATUS_INVALID_VALUE;
        if ((o->flags & GEMM_MKL_OPT_STREAMK) && (o->flags & GEMM_MKL_OPT_NO_STREAMK))
            return GEMM_MKL_STATUS_INVALID_VALUE;
        if ((o->flags & GEMM_MKL_OPT_PERSISTENT) && (o->flags & GEMM_MKL_OPT_NO_PERSISTENT))
            return GEMM_MKL_STATUS_INVALID_VALUE;
        if ((o->flags & GEMM_MKL_OPT_FIXUP) && (o->flags & GEMM_MKL_OPT_NO_FIXUP)) return GEMM_MKL_STATUS_INVALID_VALUE;
        if (o->workspace == nullptr && o->workspace_bytes != 0) return GEMM_MKL_STATUS_INVALID_VALUE;
        if (o->workspace && (reinterpret_cast<uintptr_t>(o->workspace) & 255)) return GEMM_MKL_STATUS_INVALID_VALUE;
    }
    return GEMM_MKL_STATUS_OK;
}

// Modelled time of one configuration at prefetch depth p, in cycles of one
// CU, for the heuristic (p < 0: no workgroups sharing a CU).
double model_cycles(const ConfigEntry &c, int dtype, int64_t M, int64_t N, int64_t K, int64_t L, int S, int p,
                    bool fixup = false)
{
    const int total_chunks = (int)((K * elem_bytes(dtype) + c.rb - 1) / c.rb);
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * L;
    const int64_t units = tiles * S;
    // Two workgroups share a CU when two prefetch rings fit in its 160 KB of
    // LDS.  A round of w co-resident workgroups is taken to last f w times
    // one workgroup's time (one alone leaves memory latency exposed that the
    // other fills).  f = 0.8 for 16-bit types, fitted on 48 bf16 shapes
    // (M 256..4096, N 1024..8192, K 512..8192, two boxes), where it chose
    // 64 x 64 tiles for 257..512 tiles of short K (e.g. 256 x 5632 x 512: 5.6
    // against 6.7 us on 128 x 128 tiles).  f = 0.95 for fp32, fitted on 36
    // shapes (M 128..1024, N 1024..4096, K 512..4096), where it chose two
    // workgroups per CU through a split for K = 4096 (1024 x 1024 x 4096: 72.7
    // against 78.4 us); below 0.9 it would pick 8 splits for 128 x 2048 x 2048,
    // measured slower than 4.
    // 16-bit tiles with producer waves gain nothing from a second workgroup
    // on the CU: bf16 64 x 64 with four producers ran 3-5% slower than without
    // them at 352..512 tiles (two per CU: 256 x 5632 x 512 5.89 against 5.70
    // us, 256 x 8192 x 512 6.25 against 5.95) but 6-8% faster at 176..256
    // tiles (128 x 5632 x 2048 9.28 against 9.84, 512 x 2048 x 2048 9.85
    // against 10.69).  fp32's producer tile did gain (1024 x 1024 x 4096 two
    // splits, two per CU, 67.6 us, within 1% of its best).
    const bool can_share = !(c.producers > 0 && dtype != GEMM_MKL_F32);
    int64_t w = 1;
    if (can_share && p >= 0 && 2 * (int64_t)(c.bm + c.bn) * c.rb * (p + 1) <= 160 * 1024)
        w = std::min<int64_t>(2, (units + kNumCUs - 1) / kNumCUs);
    const int64_t rounds = (units + kNumCUs * w - 1) / (kNumCUs * w);
    const double share = w > 1 ? (dtype == GEMM_MKL_F32 ? 0.95 : 0.8) * (double)w : 1.0;
    const int chunks = (total_chunks + S - 1) / S;
    const double bk = (double)c.rb / elem_bytes(dtype);
    const double peak = dtype == GEMM_MKL_F32 ? 256.0 : 4096.0;  // flop / clk / CU
    double eff = c.eff;
    // Operands far larger than the 256 MB memory-side cache stream from HBM,
    // whose latency a ring with a single chunk in flight does not cover.
    // Measured: on the batched 512x3584x18944 bf16 shape (1.2 GB of
    // operands) depth 1 with 64-wide chunks ran 4% slower than depth 4 with
    // 32-wide chunks; on operands that fit the cache it ran 4% faster.
    const double operand_bytes = (double)L * (double)(M + N) * (double)K * elem_bytes(dtype);
    if (c.default_p <= 1 && operand_bytes > 2.0 * kMallBytes) eff *= 0.9;
    const double per_chunk = 2.0 * c.bm * c.bn * bk / (peak * eff) + 60.0;
    double cyc = (double)rounds * (chunks * per_chunk * share + 1500.0);
    if (S > 1 && fixup) {
        // every piece stores its fp32 partial tile, the last one reads the
        // other S - 1 back through the L2 (about 45 B/clk per CU) after one
        // device-scope atomic; in the model's units (about 1.8 x cycles)
        const double tile_bytes = 4.0 * c.bm * c.bn;
        cyc += (double)rounds * 1.8 * (tile_bytes * S / 45.0 + 1000.0);
    } else if (S > 1) {
        const double out = (double)L * M * N;
        const double bytes = out * 4.0 * S * 2.0 + out * elem_bytes(dtype);
        cyc += bytes / 2000.0 + 5000.0;  // ~4.8 TB/s and one more launch
    }
    return cyc;
}

bool fast_path_ok(const ConfigEntry &c, int dtype, int64_t K)
{
    const int64_t es = elem_bytes(dtype);
    if ((K * es) % 16 != 0) return false;
    // offsets inside one tile's buffer resource (which starts kRsrcBias bytes
    // before the tile) must stay below 2^31
    if (((int64_t)c.bm + 1) * K * es + 2 * kRsrcBias + 256 >= (int64_t)kOutOfRange) return false;
    if (((int64_t)c.bn + 1) * K * es + 2 * kRsrcBias + 256 >= (int64_t)kOutOfRange) return false;
    return true;
}

// Largest number of ranges (pieces) one tile's chunks fall into when U units
// are cut into G ranges of floor/ceil(U/G) units.
int64_t max_pieces(int64_t U, int64_t G, int64_t C)
{
    const int64_t minr = U / G;
    if (minr < 1) return INT64_MAX;
    return (C + minr - 1) / minr + 1;
}

constexpr int kMaxPieces = 8;   // pieces per tile the stream-K kernel can combine

// Stream-K grid: one workgroup per CU, fewer when needed so that every range
// holds at least ceil(C / (kMaxPieces - 1)) units (at most kMaxPieces pieces per tile).
int64_t streamk_grid(int64_t U, int64_t C)
{
    const int64_t need = (C + kMaxPieces - 2) / (kMaxPieces - 1);
    int64_t G = std::min<int64_t>(kNumCUs, U / std::max<int64_t>(need, 1));
    return std::max<int64_t>(G, 1);
}

// Modelled stream-K time: every CU runs ceil(U / G) chunks, plus the fix-up of
// split tiles (save and read back an fp32 tile, fences, counters).
double model_streamk_cycles(const ConfigEntry &c, int dtype, int64_t M, int64_t N, int64_t K, int64_t L)
{
    const int64_t C = (K * elem_bytes(dtype) + c.rb - 1) / c.rb;
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * L;
    const int64_t U = tiles * C;
    const int64_t G = streamk_grid(U, C);
    const double one_round = model_cycles(c, dtype, M, N, K, L, 1, -1);
    const int64_t rounds = (tiles + kNumCUs - 1) / kNumCUs;
    const double per_chunk = (one_round / (double)rounds - 1500.0) / (double)C;
    const int64_t per_wg = (U + G - 1) / G;
    double cyc = per_wg * per_chunk + 1500.0;
    if (U % G != 0 || per_wg % C != 0) cyc += 2.0 * c.bm * c.bn * 4.0 / 64.0 + 2000.0;
    return cyc;
}

// ws_cap > 0: the workspace the call can have (gemm_mkl_noalloc's scratch).
// The automatic choice then skips splits whose partial sums would not fit;
// a plan that still needs more (forced options, repacked operands) is
// GEMM_MKL_STATUS_WORKSPACE.
int make_plan(int64_t M, int64_t N, int64_t K, int64_t L, int dtype, const gemm_mkl_opts *o, int align,
              Plan *plan, size_t ws_cap = 0)
{
    Registry &R = registry();
    const int64_t es = elem_bytes(dtype);
    int forced_cfg = o ? o->config_id : -1;
    if (forced_cfg < 0) forced_cfg = env().force_config;
    int forced_p = o ? o->prefetch_stages : -1;
    if (forced_p < 0) forced_p = env().stages;
    int forced_s = o ? o->split_k : 0;
    if (forced_s <= 0) forced_s = env().split_k;
    const bool force_general = o && (o->flags & GEMM_MKL_OPT_FORCE_GENERAL);
    // stream-K: -1 automatic, 0 never, 1 always (where a configuration has it)
    // (automatic choice is off until the stream-K fix-up beats the data-parallel grid)
    int sk_mode = env().streamk;
    if (o && (o->flags & GEMM_MKL_OPT_STREAMK)) sk_mode = 1;
    if (o && (o->flags & GEMM_MKL_OPT_NO_STREAMK)) sk_mode = 0;
    // an explicit split_k selects the split-K grid (1: no split of K at all);
    // stream-K then only runs when forced, and never together with a split
    if (forced_s > 1 && sk_mode == 1) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    if (forced_s >= 1 && sk_mode != 1) sk_mode = 0;
    // persistent grid: -1 whenever there are more tiles than compute units, 0 never
    // (the default: it measured no faster than the data-parallel grid), 1 always
    int pers_mode = env().persistent;
    if (o && (o->flags & GEMM_MKL_OPT_PERSISTENT)) pers_mode = 1;
    if (o && (o->flags & GEMM_MKL_OPT_NO_PERSISTENT)) pers_mode = 0;
    if (pers_mode == 1) {   // a forced persistent grid never splits K
        if (forced_s > 1 || sk_mode == 1) return GEMM_MKL_STATUS_NOT_AVAILABLE;
        forced_s = 1;
        sk_mode = 0;
    }
    // split-K summed inside the kernel: 0 never, 1 for every split plan, -1 by the model
    int fix_mode = env().fixup;
    if (o && (o->flags & GEMM_MKL_OPT_FIXUP)) fix_mode = 1;
    if (o && (o->flags & GEMM_MKL_OPT_NO_FIXUP)) fix_mode = 0;
    if (fix_mode == 1 && sk_mode == 1) {
        if (o && (o->flags & GEMM_MKL_OPT_FIXUP) && (o->flags & GEMM_MKL_OPT_STREAMK))
            return GEMM_MKL_STATUS_NOT_AVAILABLE;
        fix_mode = 0;
    }

    if (forced_cfg >= (int)R.table.size()) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    if (forced_cfg >= 0 && R.table[forced_cfg].dtype != dtype) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    if (forced_p > kMaxPrefetch) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    if (forced_s > kMaxSplit) return GEMM_MKL_STATUS_NOT_AVAILABLE;

    if ((K * es + 63) / 64 > INT32_MAX) return GEMM_MKL_STATUS_NOT_AVAILABLE;

    // Operands whose rows (K elements) or base pointers are not 16-byte
    // aligned are first copied into zero-padded, aligned rows in the
    // workspace, and the call is then planned like an aligned one at the
    // padded K (the zeros add nothing to any sum).  C is stored as it is.
    const bool rows_ok = (K * es) % 16 == 0;
    if (!force_general && (align & kAlignC) && K > 0 &&
        (!rows_ok || !(align & kAlignA) || !(align & kAlignB))) {
        if (sk_mode == 1 || pers_mode == 1) return GEMM_MKL_STATUS_NOT_AVAILABLE;
        const int64_t vec = 16 / es;
        const int64_t Kp = rows_ok ? K : (K + vec - 1) / vec * vec;
        gemm_mkl_opts inner;
        if (o)
            inner = *o;
        else
            gemm_mkl_opts_init(&inner);
        inner.flags = (inner.flags & ~(GEMM_MKL_OPT_STREAMK | GEMM_MKL_OPT_PERSISTENT)) | GEMM_MKL_OPT_NO_STREAMK |
                      GEMM_MKL_OPT_NO_PERSISTENT;
        const int64_t pack_bytes = (!rows_ok || !(align & kAlignA) ? (L * M * Kp * es + 255) / 256 * 256 : 0) +
                                   (!rows_ok || !(align & kAlignB) ? (L * N * Kp * es + 255) / 256 * 256 : 0);
        if (ws_cap > 0 && (size_t)pack_bytes + 256 > ws_cap) return GEMM_MKL_STATUS_WORKSPACE;
        Plan fast;
        const size_t inner_cap = ws_cap > 0 ? std::max<size_t>(ws_cap - (size_t)pack_bytes - 256, 1) : 0;
        const int st = make_plan(M, N, Kp, L, dtype, &inner, kAlignAll, &fast, inner_cap);
        if (st != GEMM_MKL_STATUS_OK) return st;
        if (!fast.general) {
            *plan = fast;
            plan->packed = true;
            plan->Kp = Kp;
            plan->pack_a = !rows_ok || !(align & kAlignA);
            plan->pack_b = !rows_ok || !(align & kAlignB);
            // repacked operands follow the partial sums (the data part; a
            // fix-up plan's counters, when in the workspace, come first)
            size_t off = (plan->ws_bytes - plan->fix_counter_bytes + 255) / 256 * 256;
            if (plan->pack_a) {
                plan->off_a = off;
                off += ((size_t)(L * M * Kp * es) + 255) / 256 * 256;
            }
            if (plan->pack_b) {
                plan->off_b = off;
                off += ((size_t)(L * N * Kp * es) + 255) / 256 * 256;
            }
            plan->ws_bytes = plan->fix_counter_bytes + off;
            if (ws_cap > 0 && off > ws_cap) return GEMM_MKL_STATUS_WORKSPACE;
            return GEMM_MKL_STATUS_OK;
        }
        // (a K too long for every tile configuration: the general kernel below)
    }

    bool general = force_general || align != kAlignAll;
    if (!general) {
        if (forced_cfg >= 0) {
            if (!fast_path_ok(R.table[forced_cfg], dtype, K)) general = true;
        } else {
            bool any = false;
            for (const ConfigEntry &c : R.table)
                if (c.dtype == dtype && fast_path_ok(c, dtype, K)) any = true;
            general = !any;
        }
    }
    if (general) {
        if (forced_cfg >= 0 || forced_p >= 0 || forced_s > 1 || sk_mode == 1) return GEMM_MKL_STATUS_NOT_AVAILABLE;
        plan->general = true;
        plan->config_id = -1;
        plan->P = 0;
        plan->S = 1;
        plan->tiles_m = (int32_t)((M + 63) / 64);
        plan->tiles_n = (int32_t)((N + 63) / 64);
        plan->grid = (int64_t)plan->tiles_m * plan->tiles_n * L;
        if (plan->grid > INT32_MAX) return GEMM_MKL_STATUS_NOT_AVAILABLE;
        plan->ws_bytes = 0;
        return GEMM_MKL_STATUS_OK;
    }

    // candidate (config, split) pairs and stream-K configurations
    double best = 1e300;
    int best_c = -1, best_s = 1;
    bool best_sk = false, best_fix = false;
    for (int id = 0; id < (int)R.table.size(); ++id) {
        const ConfigEntry &c = R.table[id];
        if (c.dtype != dtype) continue;
        if (forced_cfg >= 0 && id != forced_cfg) continue;
        if (!fast_path_ok(c, dtype, K)) continue;
        const int p = forced_p >= 0 ? forced_p : c.default_p;
        const int total_chunks = (int)((K * es + c.rb - 1) / c.rb);
        if (sk_mode != 0 && c.sk[p][0] != nullptr && total_chunks > 0) {
            const int64_t tiles_all = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * L;
            const int64_t U = tiles_all * total_chunks;
            const int64_t G = streamk_grid(U, total_chunks);
            if (max_pieces(U, G, total_chunks) <= kMaxPieces && tiles_all <= INT32_MAX) {
                const double cyc = model_streamk_cycles(c, dtype, M, N, K, L);
                if (cyc < best) {
                    best = cyc;
                    best_c = id;
                    best_s = 1;
                    best_sk = true;
                }
            }
        }
        if (sk_mode == 1) continue;
        if (c.fn[p][0] == nullptr) continue;
        for (int S = 1; S <= kMaxSplit; ++S) {
            if (forced_s > 0 && S != forced_s) continue;
            if (forced_s <= 0 && S > 1 && (total_chunks + S - 1) / S < 4) break;
            if (forced_s <= 0 && S != 1 && S != 2 && S != 3 && S != 4 && S != 6 && S != 8 && S != 12 && S != 16)
                continue;
            if (ws_cap > 0 && S > 1 && forced_s <= 0 && (double)S * (double)(L * M * N) * 4.0 > (double)ws_cap)
                continue;
            if (S == 1 || fix_mode != 1) {
                const double cyc = model_cycles(c, dtype, M, N, K, L, S, p);
                if (cyc < best) {
                    best = cyc;
                    best_c = id;
                    best_s = S;
                    best_sk = false;
                    best_fix = false;
                }
            }
            const int64_t tiles_all = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn) * L;
            // 16-bit plans take the fix-up only when it or the split is
            // forced: no 16-bit shape measured faster with it than with the
            // best plan without it, and the model ranked it first where it
            // lost (bf16, graph replay: 256 x 8192 x 2048 two pieces 20.0 us
            // against 15.3 on 128 x 128 unsplit; 1024 x 8192 x 8192 two pieces
            // of 256 x 256 131.7 against 111.1 on 128 x 256 unsplit;
            // 1024 x 1024 x 4096 four pieces 22.7 against 17.6 on 64 x 64;
            // the K-heavy L=8 shape two pieces 585 against 547 unsplit).  fp32
            // takes it by the model (128 x 2048 x 2048: 13.4 us, four pieces).
            const bool fix_s_ok = fix_mode == 1 || forced_s > 0 || dtype == GEMM_MKL_F32;
            const bool fix_ok = S > 1 && fix_mode != 0 && c.fixup[0] != nullptr && S <= kMaxFixupSplit &&
                                fix_s_ok && p == c.default_p && tiles_all <= kMaxFixupTiles &&
                                (ws_cap == 0 || (double)tiles_all * S * c.bm * c.bn * 4.0 <= (double)ws_cap);
            if (fix_ok) {
                const double cyc = model_cycles(c, dtype, M, N, K, L, S, p, true);
                if (cyc < best) {
                    best = cyc;
                    best_c = id;
                    best_s = S;
                    best_sk = false;
                    best_fix = true;
                }
            }
        }
    }
    if (best_c < 0) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    const ConfigEntry &c = R.table[best_c];
    const int total_chunks = (int)((K * es + c.rb - 1) / c.rb);
    plan->general = false;
    plan->config_id = best_c;
    plan->P = forced_p >= 0 ? forced_p : c.default_p;
    plan->S = best_s;
    plan->tiles_m = (int32_t)((M + c.bm - 1) / c.bm);
    plan->tiles_n = (int32_t)((N + c.bn - 1) / c.bn);
    plan->total_chunks = total_chunks;
    plan->chunks_per_split = (total_chunks + best_s - 1) / best_s;
    if (plan->chunks_per_split == 0) plan->chunks_per_split = 1;
    // splits whose chunk range would be empty are dropped (the grid shrinks)
    if (best_s > 1) {
        int used = (total_chunks + plan->chunks_per_split - 1) / plan->chunks_per_split;
        if (used < 1) used = 1;
        plan->S = used;
    }
    // raster groups of up to 4 tile rows: the 32 workgroups an XCD runs at
    // once then share few A row-blocks and B column-blocks in its L2
    plan->group_m = std::min<int32_t>(plan->tiles_m, (int32_t)env().group_m);
    if (plan->group_m < 1) plan->group_m = 1;
    plan->grid = (int64_t)plan->tiles_m * plan->tiles_n * plan->S * L;
    if (plan->grid > INT32_MAX) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    plan->ws_bytes = plan->S > 1 ? (size_t)plan->S * (size_t)(L * M * N) * 4 : 0;
    if (best_fix && plan->S > 1) {
        // S pieces of every tile on one XCD: ceil(tiles / 8) tiles per XCD
        const int64_t tiles_all = (int64_t)plan->tiles_m * plan->tiles_n * L;
        plan->fixup = true;
        plan->fix_per = (int32_t)((tiles_all + 7) / 8);
        plan->grid = (int64_t)plan->fix_per * 8 * plan->S;
        plan->fix_counter_bytes = ((size_t)tiles_all * kCounterStride * 4 + 255) / 256 * 256;
        // [counters][partial tiles: S per tile]
        plan->ws_bytes = plan->fix_counter_bytes + (size_t)tiles_all * plan->S * c.bm * c.bn * 4;
    }
    plan->streamk = best_sk;
    if (best_sk) {
        const int64_t tiles_all = (int64_t)plan->tiles_m * plan->tiles_n * L;
        plan->sk_units = tiles_all * total_chunks;
        plan->grid = streamk_grid(plan->sk_units, total_chunks);
        plan->sk_counter_bytes = ((size_t)tiles_all * kCounterStride * 4 + 255) / 256 * 256;
        // [counters][2 partial tiles per workgroup]
        plan->ws_bytes = plan->sk_counter_bytes + (size_t)2 * plan->grid * c.bm * c.bn * 4;
    }
    // The persistent grid: one workgroup per compute unit, each running one
    // ring across its tiles, so that a tile's first loads overlap the end of
    // the tile before it.  It can only pay off with more tiles than compute
    // units (a single round has no next tile to overlap); measured on MI355X
    // it was no faster than the data-parallel grid at depth 4 (the staging
    // area leaves room for depth 3 only), so it runs only when asked for.
    const int64_t tiles_all = (int64_t)plan->tiles_m * plan->tiles_n * L;
    const bool pers_ok = c.persist[0] != nullptr && plan->S == 1 && !best_sk && total_chunks > 0 &&
                         (forced_p < 0 || forced_p == c.persist_p) && tiles_all <= INT32_MAX;
    if (pers_mode == 1 && !pers_ok) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    if (pers_ok && (pers_mode == 1 || (pers_mode == -1 && tiles_all > kNumCUs))) {
        plan->persistent = true;
        plan->P = c.persist_p;
        plan->grid = std::min<int64_t>(tiles_all, kNumCUs);
    }
    if (ws_cap > 0 && plan->ws_bytes - plan->fix_counter_bytes > ws_cap) return GEMM_MKL_STATUS_WORKSPACE;
    return GEMM_MKL_STATUS_OK;
}

// Plans depend only on the sizes, the dtype, pointer alignment and the
// options, so each distinct request is planned once and then looked up.
struct PlanKey {
    int64_t M, N, K, L;
    int64_t ws_cap;
    int32_t dtype, aligned, config_id, prefetch, split, flags;
    bool operator<(const PlanKey &o) const
    {
        return std::memcmp(this, &o, sizeof(PlanKey)) < 0;
    }
};
static_assert(sizeof(PlanKey) == 64, "PlanKey must have no padding (compared bytewise)");

std::mutex g_plan_mutex;
std::map<PlanKey, std::pair<int, Plan>> g_plans;
constexpr size_t kMaxCachedPlans = 4096;

int cached_plan(int64_t M, int64_t N, int64_t K, int64_t L, int dtype, const gemm_mkl_opts *o, int align,
                Plan *plan, size_t ws_cap = 0)
{
    PlanKey key;
    std::memset(&key, 0, sizeof key);
    key.M = M;
    key.N = N;
    key.K = K;
    key.L = L;
    key.ws_cap = (int64_t)ws_cap;
    key.dtype = dtype;
    key.aligned = align;
    key.config_id = o ? o->config_id : -1;
    key.prefetch = o ? o->prefetch_stages : -1;
    key.split = o ? o->split_k : 0;
    key.flags = o ? o->flags : 0;
    {
        std::lock_guard<std::mutex> g(g_plan_mutex);
        auto it = g_plans.find(key);
        if (it != g_plans.end()) {
            *plan = it->second.second;
            return it->second.first;
        }
    }
    Plan fresh;
    const int st = make_plan(M, N, K, L, dtype, o, align, &fresh, ws_cap);
    std::lock_guard<std::mutex> g(g_plan_mutex);
    if (g_plans.size() >= kMaxCachedPlans) g_plans.clear();
    g_plans.emplace(key, std::make_pair(st, fresh));
    *plan = fresh;
    return st;
}

// ---------------------------------------------------------------- internal workspace

struct Workspace {
    std::mutex mu;              // held while this entry grows (and while a call reads it)
    void *ptr = nullptr;        // split-K / stream-K partial sums
    size_t bytes = 0;
    void *counters = nullptr;   // stream-K per-tile counters: zero between calls
    size_t counter_bytes = 0;
};

// One entry per (device, stream).  g_ws_mutex guards only the map itself:
// growing one stream's workspace synchronises that stream while holding that
// entry's own mutex, so calls on other streams (other entries) never wait for
// it.  Entries are never erased while the library is in use (only
// gemm_mkl_release_workspace frees their buffers), so a reference taken under
// g_ws_mutex stays valid after it is released.
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, std::unique_ptr<Workspace>> g_ws;

Workspace *ws_entry(hipStream_t stream, int *status)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        t_last_hip = e;
        *status = GEMM_MKL_STATUS_HIP_ERROR;
        return nullptr;
    }
    std::lock_guard<std::mutex> g(g_ws_mutex);
    std::unique_ptr<Workspace> &w = g_ws[std::make_pair(dev, stream)];
    if (!w) w.reset(new Workspace);
    *status = GEMM_MKL_STATUS_OK;
    return w.get();
}

// Grows *ptr / *bytes to hold `need` bytes (at least `floor`); the caller
// holds the entry's mutex.  The old buffer may still be read by work queued
// on `stream`, so it is freed only after that stream has drained.
int grow(hipStream_t stream, void **ptr, size_t *bytes, size_t need, size_t floor, bool zero)
{
    if (*bytes >= need) return GEMM_MKL_STATUS_OK;
    hipError_t e;
    if (*ptr) {
        e = hipStreamSynchronize(stream);
        if (e == hipSuccess) e = hipFree(*ptr);
        *ptr = nullptr;
        *bytes = 0;
        if (e != hipSuccess) {
            t_last_hip = e;
            return GEMM_MKL_STATUS_HIP_ERROR;
        }
    }
    const size_t sz = need < floor ? floor : need;
    e = hipMalloc(ptr, sz);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        *ptr = nullptr;
        return GEMM_MKL_STATUS_WORKSPACE;
    }
    if (zero) {
        e = hipMemsetAsync(*ptr, 0, sz, stream);
        if (e != hipSuccess) {
            t_last_hip = e;
            return GEMM_MKL_STATUS_HIP_ERROR;
        }
    }
    *bytes = sz;
    return GEMM_MKL_STATUS_OK;
}

// The entry of (device, stream) locked into `lk` (kept locked until the
// caller has enqueued the work that uses its buffers, so that a second thread
// on the same stream cannot free them in between); `lk` may already hold it.
Workspace *locked_entry(hipStream_t stream, std::unique_lock<std::mutex> &lk, int *status)
{
    Workspace *w = ws_entry(stream, status);
    if (!w) return nullptr;
    if (!lk.owns_lock()) lk = std::unique_lock<std::mutex>(w->mu);
    return w;
}

// Per-tile stream-K counters of (device, stream): zeroed when allocated, and
// every completed stream-K call leaves them zero again.
int get_counters(hipStream_t stream, size_t need, void **out, std::unique_lock<std::mutex> &lk)
{
    int st;
    Workspace *w = locked_entry(stream, lk, &st);
    if (!w) return st;
    st = grow(stream, &w->counters, &w->counter_bytes, need, (size_t)65536, true);
    if (st != GEMM_MKL_STATUS_OK) return st;
    *out = w->counters;
    return GEMM_MKL_STATUS_OK;
}

int get_workspace(hipStream_t stream, size_t need, void **out, std::unique_lock<std::mutex> &lk)
{
    if (env().has_ws_limit && need > env().ws_limit) return GEMM_MKL_STATUS_WORKSPACE;
    int st;
    Workspace *w = locked_entry(stream, lk, &st);
    if (!w) return st;
    st = grow(stream, &w->ptr, &w->bytes, need, (size_t)1 << 20, false);
    if (st != GEMM_MKL_STATUS_OK) return st;
    *out = w->ptr;
    return GEMM_MKL_STATUS_OK;
}

std::mutex g_scratch_mutex;
std::map<int, void *> g_scratch_ptr;   // device -> address of that device's `scratch`

// The address of the current device's scratch, looked up once per device
// (with that device current) and kept.
int scratch_address(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        t_last_hip = e;
        return GEMM_MKL_STATUS_HIP_ERROR;
    }
    std::lock_guard<std::mutex> g(g_scratch_mutex);
    auto it = g_scratch_ptr.find(dev);
    if (it == g_scratch_ptr.end()) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            t_last_hip = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return GEMM_MKL_STATUS_HIP_ERROR;
        }
        it = g_scratch_ptr.emplace(dev, ptr).first;
    }
    *out = it->second;
    return GEMM_MKL_STATUS_OK;
}

int run(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int64_t L, int dtype, int epilogue,
        void *stream_v, const gemm_mkl_opts *o, size_t ws_cap = 0)
{
    int st = check_args(M, N, K, L, dtype, epilogue, o);
    if (st != GEMM_MKL_STATUS_OK) return st;
    if (M == 0 || N == 0 || L == 0) return GEMM_MKL_STATUS_OK;
    if (C == nullptr) return GEMM_MKL_STATUS_INVALID_VALUE;
    if (K > 0 && (A == nullptr || B == nullptr)) return GEMM_MKL_STATUS_INVALID_VALUE;
    const int es = elem_bytes(dtype);
    auto al = [](const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
    if (!al(A, es) || !al(B, es) || !al(C, es)) return GEMM_MKL_STATUS_INVALID_VALUE;
    // C is written while A and B are read, and a caller workspace takes
    // partial sums or repacked operands while all three are in use: ranges
    // that share a byte would feed results back into the sums.  (The sizes
    // were checked for overflow above.)
    {
        const uint64_t a_bytes = K > 0 ? uint64_t(L * M * K * es) : 0, b_bytes = K > 0 ? uint64_t(L * N * K * es) : 0;
        const uint64_t c_bytes = uint64_t(L * M * N * es);
        if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes)) return GEMM_MKL_STATUS_INVALID_VALUE;
        if (o && o->workspace) {
            const uint64_t w = o->workspace_bytes;
            if (overlaps(o->workspace, w, A, a_bytes) || overlaps(o->workspace, w, B, b_bytes) ||
                overlaps(o->workspace, w, C, c_bytes))
                return GEMM_MKL_STATUS_INVALID_VALUE;
        }
    }
    const int align = (al(A, 16) ? kAlignA : 0) | (al(B, 16) ? kAlignB : 0) | (al(C, 4 * es) ? kAlignC : 0);

    Plan plan;
    st = cached_plan(M, N, K, L, dtype, o, align, &plan, ws_cap);
    if (st != GEMM_MKL_STATUS_OK) return st;
    // gemm_mkl_noalloc: every check is done; the scratch is the workspace
    void *scratch_ws = nullptr;
    if (ws_cap > 0) {
        st = scratch_address(&scratch_ws);
        if (st != GEMM_MKL_STATUS_OK) return st;
    }

    Registry &R = registry();
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    if (env().log)
        std::fprintf(stderr, "gemm_mkl: M=%lld N=%lld K=%lld L=%lld dtype=%d epi=%d -> %s P=%d S=%d%s%s grid=%lld\n",
                     (long long)M, (long long)N, (long long)K, (long long)L, dtype, epilogue,
                     plan.general ? "general" : R.table[plan.config_id].name, plan.P, plan.S,
                     plan.streamk ? " stream-K" : (plan.persistent ? " persistent" : (plan.fixup ? " fix-up" : "")),
                     plan.packed ? " packed" : "", (long long)plan.grid);

    hipError_t e;
    if (plan.general) {
        e = R.k[dtype].general[epilogue](A, B, C, M, N, K, L, stream);
    } else {
        const ConfigEntry &c = R.table[plan.config_id];
        TileParams p;
        p.A = A;
        p.B = B;
        p.M = M;
        p.N = N;
        p.K = K;
        p.L = L;
        p.tiles_m = plan.tiles_m;
        p.tiles_n = plan.tiles_n;
        p.group_m = plan.group_m;
        p.split = plan.S;
        p.chunks_per_split = plan.chunks_per_split;
        p.total_chunks = plan.total_chunks;
        p.map = make_tile_map(plan.tiles_m, plan.tiles_n, (int)L, plan.S, plan.group_m, (int)plan.grid);
        // the workspace of split-K partials (from offset 0) and repacked
        // operands; a fix-up plan's counter words come first in a caller's
        // workspace, and from a buffer of their own otherwise
        void *ws = nullptr, *fix_cnt = nullptr;
        std::unique_lock<std::mutex> ws_lock;   // the internal workspace stays ours until launched
        if (!plan.streamk && plan.ws_bytes > 0) {
            if (o && o->workspace) {
                if (o->workspace_bytes < plan.ws_bytes) return GEMM_MKL_STATUS_WORKSPACE;
                fix_cnt = o->workspace;
                ws = static_cast<char *>(o->workspace) + plan.fix_counter_bytes;
            } else if (scratch_ws) {
                ws = scratch_ws;   // the plan fits it (ws_cap)
                fix_cnt = static_cast<char *>(scratch_ws) + kScratchDataBytes;
            } else {
                st = get_workspace(stream, plan.ws_bytes - plan.fix_counter_bytes, &ws, ws_lock);
                if (st != GEMM_MKL_STATUS_OK) return st;
                if (plan.fixup) {
                    st = get_counters(stream, plan.fix_counter_bytes, &fix_cnt, ws_lock);
                    if (st != GEMM_MKL_STATUS_OK) return st;
                }
            }
        }
        if (plan.packed) {
            char *w = static_cast<char *>(ws);
            e = hipSuccess;
            if (plan.pack_a) {
                e = R.k[dtype].pack(A, w + plan.off_a, L * M, K, plan.Kp, stream);
                p.A = w + plan.off_a;
            }
            if (e == hipSuccess && plan.pack_b) {
                e = R.k[dtype].pack(B, w + plan.off_b, L * N, K, plan.Kp, stream);
                p.B = w + plan.off_b;
            }
            if (e != hipSuccess) {
                t_last_hip = e;
                return GEMM_MKL_STATUS_HIP_ERROR;
            }
            p.K = plan.Kp;
        }
        if (plan.streamk) {
            p.C = C;
            void *ws = nullptr, *cnt = nullptr;
            if (o && o->workspace) {
                if (o->workspace_bytes < plan.ws_bytes) return GEMM_MKL_STATUS_WORKSPACE;
                cnt = o->workspace;
                ws = static_cast<char *>(o->workspace) + plan.sk_counter_bytes;
            } else {
                st = get_workspace(stream, plan.ws_bytes - plan.sk_counter_bytes, &ws, ws_lock);
                if (st != GEMM_MKL_STATUS_OK) return st;
                st = get_counters(stream, plan.sk_counter_bytes, &cnt, ws_lock);
                if (st != GEMM_MKL_STATUS_OK) return st;
            }
            StreamKParams sp;
            sp.t = p;
            sp.ws = reinterpret_cast<float *>(ws);
            sp.counters = reinterpret_cast<int *>(cnt);
            sp.units = plan.sk_units;
            e = c.sk[plan.P][epilogue](sp, (int)plan.grid, stream);
        } else if (plan.persistent) {
            p.C = C;
            e = c.persist[epilogue](p, (int)plan.grid, stream);
        } else if (plan.fixup) {
            p.C = C;
            FixupParams fp;
            fp.t = p;
            fp.ws = reinterpret_cast<float *>(ws);
            fp.counters = reinterpret_cast<uint32_t *>(fix_cnt);
            fp.per = plan.fix_per;
            fp.force_remote = (o && (o->flags & GEMM_MKL_OPT_FIXUP_RECOMPUTE)) ? 1 : 0;
            e = c.fixup[epilogue](fp, (int)plan.grid, stream);
        } else if (plan.S == 1) {
            p.C = C;
            e = c.fn[plan.P][epilogue](p, (int)plan.grid, stream);
        } else {
            p.C = ws;
            e = c.fn[plan.P][MODE_PARTIAL](p, (int)plan.grid, stream);
            if (e == hipSuccess)
                e = R.k[dtype].reduce[epilogue](reinterpret_cast<const float *>(ws), C, L * M * N, plan.S, stream);
        }
    }
    if (e != hipSuccess) {
        t_last_hip = e;
        return GEMM_MKL_STATUS_HIP_ERROR;
    }
    return GEMM_MKL_STATUS_OK;
}

// The configuration a grouped call uses (-1: none fits).  Sizes and options
// are assumed checked.
int grouped_config(int64_t G, int64_t total_m, int64_t N, int64_t K, int dtype, int epilogue,
                   const gemm_mkl_opts *o)
{
    Registry &R = registry();
    const int forced = o ? o->config_id : -1;
    int best = -1;
    double best_cyc = 1e300;
    for (int id = 0; id < (int)R.table.size(); ++id) {
        const ConfigEntry &c = R.table[id];
        if (c.dtype != dtype || c.grouped[epilogue] == nullptr) continue;
        if (forced >= 0 && id != forced) continue;
        if (o && o->prefetch_stages >= 0 && o->prefetch_stages != c.grouped_p) continue;
        if (!fast_path_ok(c, dtype, K)) continue;
        // with several groups every group ends in a partly filled row tile,
        // about half a tile on average; the kernel skips the MFMAs of its
        // empty row blocks, but the tile still takes a workgroup for one
        // round.  Measured on 4096 rows in 8 groups x 5632 x 2048 bf16 (MFMAs
        // skipped): 256 x 256 tiles with 8 waves 105 us, with 4 waves 115 us,
        // 128 x 128 + 4 producers 132 us, 64 x 64 180 us; the model ranks them
        // in that order.  A single group is a plain GEMM.
        const int64_t m_eff = G > 1 ? total_m + G * c.bm / 2 : total_m;
        const double cyc = model_cycles(c, dtype, m_eff, N, K, 1, 1, -1);
        if (cyc < best_cyc) {
            best_cyc = cyc;
            best = id;
        }
    }
    return best;
}

// Grouped GEMM: checks, the configuration choice and the launch.
int run_grouped(const void *A, const void *B, void *C, const int32_t *offs, int64_t G, int64_t total_m, int64_t N,
                int64_t K, int dtype, int epilogue, void *stream_v, const gemm_mkl_opts *o)
{
    if (dtype != GEMM_MKL_F32 && dtype != GEMM_MKL_F16 && dtype != GEMM_MKL_BF16)
        return GEMM_MKL_STATUS_UNSUPPORTED_DTYPE;
    if (epilogue != GEMM_MKL_EPI_IDENTITY && epilogue != GEMM_MKL_EPI_RELU && epilogue != GEMM_MKL_EPI_SILU)
        return GEMM_MKL_STATUS_UNSUPPORTED_EPILOGUE;
    if (G < 0 || total_m < 0 || N < 0 || K < 0) return GEMM_MKL_STATUS_INVALID_VALUE;
    if (G > kMaxGroups || total_m > INT32_MAX) return GEMM_MKL_STATUS_INVALID_VALUE;
    const int64_t es = elem_bytes(dtype);
    int64_t t;
    if (!mul_ok(total_m, K, &t) || !mul_ok(t, es, &t)) return GEMM_MKL_STATUS_INVALID_VALUE;
    if (!mul_ok(G, N, &t) || !mul_ok(t, K, &t) || !mul_ok(t, es, &t)) return GEMM_MKL_STATUS_INVALID_VALUE;
    if (!mul_ok(total_m, N, &t) || !mul_ok(t, es, &t)) return GEMM_MKL_STATUS_INVALID_VALUE;
    if (o) {
        if (o->prefetch_stages < -1 || o->split_k < 0 || o->config_id < -1) return GEMM_MKL_STATUS_INVALID_VALUE;
        if (o->flags != 0 || o->split_k > 1) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    }
    if (G == 0 || total_m == 0 || N == 0) return GEMM_MKL_STATUS_OK;
    if (C == nullptr || offs == nullptr) return GEMM_MKL_STATUS_INVALID_VALUE;
    if (K > 0 && (A == nullptr || B == nullptr)) return GEMM_MKL_STATUS_INVALID_VALUE;
    auto al = [](const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
    if (!al(A, es) || !al(B, es) || !al(C, es) || !al(offs, 4)) return GEMM_MKL_STATUS_INVALID_VALUE;
    // C is written while A, B and the offsets are read (and a caller
    // workspace takes the repacked operands): no two may share a byte.
    {
        const uint64_t a_bytes = K > 0 ? uint64_t(total_m * K * es) : 0, b_bytes = K > 0 ? uint64_t(G * N * K * es) : 0;
        const uint64_t c_bytes = uint64_t(total_m * N * es), o_bytes = uint64_t(G) * 4;
        if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes) || overlaps(C, c_bytes, offs, o_bytes))
            return GEMM_MKL_STATUS_INVALID_VALUE;
        if (o && o->workspace) {
            const uint64_t w = o->workspace_bytes;
            if (overlaps(o->workspace, w, A, a_bytes) || overlaps(o->workspace, w, B, b_bytes) ||
                overlaps(o->workspace, w, C, c_bytes) || overlaps(o->workspace, w, offs, o_bytes))
                return GEMM_MKL_STATUS_INVALID_VALUE;
        }
    }
    // The tiled kernels read 16-byte pieces: rows of K elements that are not
    // a multiple of 16 bytes, or an A or B off a 16-byte boundary, are first
    // copied into zero-padded rows of Kp elements in the workspace (the zeros
    // add nothing to any sum).
    const bool rows_ok = (K * es) % 16 == 0;
    const bool pack_a = K > 0 && (!rows_ok || !al(A, 16));
    const bool pack_b = K > 0 && (!rows_ok || !al(B, 16));
    const int64_t vec = 16 / es;
    const int64_t Kp = rows_ok ? K : (K + vec - 1) / vec * vec;

    const int best = grouped_config(G, total_m, N, Kp, dtype, epilogue, o);
    if (best < 0) return best == -1 ? GEMM_MKL_STATUS_NOT_AVAILABLE : best;
    Registry &R = registry();
    const ConfigEntry &c = R.table[best];
    GroupedParams gp;
    gp.A = A;
    gp.B = B;
    gp.C = C;
    gp.offs = offs;
    gp.G = (int32_t)G;
    gp.total_m = (int32_t)total_m;
    gp.N = N;
    gp.K = Kp;
    const int64_t tiles_n = (N + c.bn - 1) / c.bn;
    const int64_t row_tiles = (total_m + c.bm - 1) / c.bm + G;   // each group adds at most one partial tile
    const int64_t grid = row_tiles * tiles_n;
    if (tiles_n > INT32_MAX || row_tiles > INT32_MAX || grid > INT32_MAX) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    gp.tiles_n = (int32_t)tiles_n;
    gp.row_tiles = (int32_t)row_tiles;
    gp.total_chunks = (int32_t)((Kp * es + c.rb - 1) / c.rb);
    gp.group_m = std::max<int32_t>(1, (int32_t)env().grouped_group_m);
    if (env().log)
        std::fprintf(stderr, "gemm_mkl_grouped: G=%lld rows=%lld N=%lld K=%lld dtype=%d epi=%d -> %s P=%d grid=%lld\n",
                     (long long)G, (long long)total_m, (long long)N, (long long)K, dtype, epilogue, c.name,
                     c.grouped_p, (long long)grid);
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    std::unique_lock<std::mutex> ws_lock;   // the internal workspace stays ours until launched
    if (pack_a || pack_b) {
        const size_t bytes_a = pack_a ? ((size_t)(total_m * Kp * es) + 255) / 256 * 256 : 0;
        const size_t need = bytes_a + (pack_b ? ((size_t)(G * N * Kp * es) + 255) / 256 * 256 : 0);
        void *ws = nullptr;
        if (o && o->workspace) {
            if (o->workspace_bytes < need) return GEMM_MKL_STATUS_WORKSPACE;
            ws = o->workspace;
        } else {
            const int st = get_workspace(stream, need, &ws, ws_lock);
            if (st != GEMM_MKL_STATUS_OK) return st;
        }
        char *w = static_cast<char *>(ws);
        hipError_t e = hipSuccess;
        if (pack_a) {
            e = R.k[dtype].pack(A, w, total_m, K, Kp, stream);
            gp.A = w;
        }
        if (e == hipSuccess && pack_b) {
            e = R.k[dtype].pack(B, w + bytes_a, G * N, K, Kp, stream);
            gp.B = w + bytes_a;
        }
        if (e != hipSuccess) {
            t_last_hip = e;
            return GEMM_MKL_STATUS_HIP_ERROR;
        }
    }
    hipError_t e = c.grouped[epilogue](gp, (int)grid, stream);
    if (e != hipSuccess) {
        t_last_hip = e;
        return GEMM_MKL_STATUS_HIP_ERROR;
    }
    return GEMM_MKL_STATUS_OK;
}

}  // namespace

namespace gmk {
// Records a HIP error of another unit's launch for gemm_mkl_status_string.
void note_hip_error(hipError_t e) { t_last_hip = e; }
}  // namespace gmk

extern "C" {

void gemm_mkl_opts_init(gemm_mkl_opts *o)
{
    if (!o) return;
    std::memset(o, 0, sizeof(*o));
    o->prefetch_stages = -1;
    o->split_k = 0;
    o->config_id = -1;
}

int gemm_mkl(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int64_t L, int dtype,
             int epilogue, void *stream)
{
    return run(A, B, C, M, N, K, L, dtype, epilogue, stream, nullptr);
}

int gemm_mkl_ex(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int64_t L, int dtype,
                int epilogue, void *stream, const gemm_mkl_opts *opts)
{
    return run(A, B, C, M, N, K, L, dtype, epilogue, stream, opts);
}

int gemm_mkl_noalloc(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int64_t L, int dtype,
                     int epilogue, void *stream, const gemm_mkl_opts *opts)
{
    if (opts && (opts->workspace != nullptr || opts->workspace_bytes != 0)) return GEMM_MKL_STATUS_INVALID_VALUE;
    gemm_mkl_opts o;
    if (opts)
        o = *opts;
    else
        gemm_mkl_opts_init(&o);
    const int st = check_args(M, N, K, L, dtype, epilogue, &o);
    if (st != GEMM_MKL_STATUS_OK) return st;
    // stream-K needs counters that start at zero: not offered here
    if (o.flags & GEMM_MKL_OPT_STREAMK) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    o.flags |= GEMM_MKL_OPT_NO_STREAMK;
    // run() makes every check of gemm_mkl_ex, plans within the scratch and
    // only then looks up the scratch: a rejected call touches no device state
    return run(A, B, C, M, N, K, L, dtype, epilogue, stream, &o, kScratchDataBytes);
}

int gemm_mkl_grouped(const void *A, const void *B, void *C, const int32_t *offs, int64_t G, int64_t total_m,
                     int64_t N, int64_t K, int dtype, int epilogue, void *stream, const gemm_mkl_opts *opts)
{
    return run_grouped(A, B, C, offs, G, total_m, N, K, dtype, epilogue, stream, opts);
}

int gemm_mkl_grouped_config(int64_t G, int64_t total_m, int64_t N, int64_t K, int dtype, int epilogue,
                            const gemm_mkl_opts *opts)
{
    // the checks of gemm_mkl_grouped that need no pointers
    if (dtype != GEMM_MKL_F32 && dtype != GEMM_MKL_F16 && dtype != GEMM_MKL_BF16)
        return GEMM_MKL_STATUS_UNSUPPORTED_DTYPE;
    if (epilogue != GEMM_MKL_EPI_IDENTITY && epilogue != GEMM_MKL_EPI_RELU && epilogue != GEMM_MKL_EPI_SILU)
        return GEMM_MKL_STATUS_UNSUPPORTED_EPILOGUE;
    if (G < 0 || total_m < 0 || N < 0 || K < 0 || G > kMaxGroups || total_m > INT32_MAX)
        return GEMM_MKL_STATUS_INVALID_VALUE;
    if (opts) {
        if (opts->prefetch_stages < -1 || opts->split_k < 0 || opts->config_id < -1) return GEMM_MKL_STATUS_INVALID_VALUE;
        if (opts->flags != 0 || opts->split_k > 1) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    }
    const int64_t vec = 16 / elem_bytes(dtype);
    const int64_t Kp = (K + vec - 1) / vec * vec;   // rows are repacked to a 16-byte multiple
    const int id = grouped_config(G, total_m, N, Kp, dtype, epilogue, opts);
    return id >= 0 ? id : GEMM_MKL_STATUS_NOT_AVAILABLE;
}

int gemm_mkl_get_plan(int64_t M, int64_t N, int64_t K, int64_t L, int dtype, int epilogue,
                      const gemm_mkl_opts *opts, gemm_mkl_plan *out)
{
    int st = check_args(M, N, K, L, dtype, epilogue, opts);
    if (st != GEMM_MKL_STATUS_OK) return st;
    if (!out) return GEMM_MKL_STATUS_INVALID_VALUE;
    std::memset(out, 0, sizeof(*out));
    if (M == 0 || N == 0 || L == 0) {
        out->config_id = -1;
        out->split_k = 1;
        return GEMM_MKL_STATUS_OK;
    }
    Plan plan;
    st = cached_plan(M, N, K, L, dtype, opts, kAlignAll, &plan);
    if (st != GEMM_MKL_STATUS_OK) return st;
    out->config_id = plan.config_id;
    out->prefetch_stages = plan.P;
    out->split_k = plan.S;
    out->general = plan.general ? 1 : 0;
    out->grid = plan.grid;
    if (plan.general) {
        out->block_m = 64;
        out->block_n = 64;
        out->block_k = 16;
        out->threads = 256;
    } else {
        const ConfigEntry &c = registry().table[plan.config_id];
        out->block_m = c.bm;
        out->block_n = c.bn;
        out->block_k = c.rb / elem_bytes(dtype);
        out->threads = (c.waves_m * c.waves_n * c.waves_k + c.producers) * 64;
    }
    out->workspace_bytes = plan.ws_bytes;
    out->streamk = plan.streamk ? 1 : 0;
    out->counter_bytes = (int32_t)(plan.streamk ? plan.sk_counter_bytes : plan.fix_counter_bytes);
    out->fixup = plan.fixup ? 1 : 0;
    out->persistent = plan.persistent ? 1 : 0;
    out->packed = plan.packed ? 1 : 0;
    return GEMM_MKL_STATUS_OK;
}

int gemm_mkl_tile_order(int64_t M, int64_t N, int64_t K, int64_t L, int dtype, int epilogue,
                        const gemm_mkl_opts *opts, int32_t *out, int64_t capacity)
{
    int st = check_args(M, N, K, L, dtype, epilogue, opts);
    if (st != GEMM_MKL_STATUS_OK) return st;
    if (M == 0 || N == 0 || L == 0) return GEMM_MKL_STATUS_OK;
    Plan plan;
    st = cached_plan(M, N, K, L, dtype, opts, kAlignAll, &plan);
    if (st != GEMM_MKL_STATUS_OK) return st;
    if (plan.general || plan.streamk || plan.persistent) return GEMM_MKL_STATUS_NOT_AVAILABLE;
    if (!out || capacity < 4 * plan.grid) return GEMM_MKL_STATUS_INVALID_VALUE;
    const TileMap m = make_tile_map(plan.tiles_m, plan.tiles_n, (int)L, plan.S, plan.group_m, (int)plan.grid);
    for (int64_t b = 0; b < plan.grid; ++b) {
        int l, s, tm, tn;
        if (plan.fixup) {
            (void)fixup_map(m, plan.fix_per, (uint32_t)b, l, s, tm, tn);
            if (l >= L) l = s = tm = tn = -1;   // past the last tile of its XCD's run
        } else {
            map_workgroup(m, (uint32_t)b, l, s, tm, tn);
        }
        out[4 * b] = l;
        out[4 * b + 1] = s;
        out[4 * b + 2] = tm;
        out[4 * b + 3] = tn;
    }
    return GEMM_MKL_STATUS_OK;
}

size_t gemm_mkl_workspace_size(int64_t M, int64_t N, int64_t K, int64_t L, int dtype, int split_k)
{
    gemm_mkl_opts o;
    gemm_mkl_opts_init(&o);
    o.split_k = split_k;
    gemm_mkl_plan p;
    if (gemm_mkl_get_plan(M, N, K, L, dtype, GEMM_MKL_EPI_IDENTITY, &o, &p) != GEMM_MKL_STATUS_OK) return 0;
    return p.workspace_bytes;
}

int gemm_mkl_release_workspace(void)
{
    std::lock_guard<std::mutex> g(g_ws_mutex);
    int st = GEMM_MKL_STATUS_OK;
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto &kv : g_ws) {
        Workspace &w = *kv.second;
        std::lock_guard<std::mutex> gw(w.mu);
        for (void **ptr : {&w.ptr, &w.counters}) {
            if (!*ptr) continue;
            hipError_t e = hipSetDevice(kv.first.first);
            if (e == hipSuccess) e = hipFree(*ptr);
            if (e != hipSuccess) {
                t_last_hip = e;
                st = GEMM_MKL_STATUS_HIP_ERROR;
            }
            *ptr = nullptr;
        }
        w.bytes = 0;
        w.counter_bytes = 0;
    }
    (void)hipSetDevice(cur);
    return st;
}

const char *gemm_mkl_status_string(int status)
{
    switch (status) {
    case GEMM_MKL_STATUS_OK: return "success";
    case GEMM_MKL_STATUS_INVALID_VALUE:
        return "invalid value: null pointer for a non-empty problem, negative or overflowing size, "
               "misaligned pointer, or an invalid option (prefetch_stages must be -1 (auto) or >= 0)";
    case GEMM_MKL_STATUS_UNSUPPORTED_DTYPE: return "unsupported dtype: expected GEMM_MKL_F32, GEMM_MKL_F16 or GEMM_MKL_BF16";
    case GEMM_MKL_STATUS_UNSUPPORTED_EPILOGUE:
        return "unsupported epilogue: expected GEMM_MKL_EPI_IDENTITY, GEMM_MKL_EPI_RELU or GEMM_MKL_EPI_SILU";
    case GEMM_MKL_STATUS_WORKSPACE: return "split-K workspace too small or could not be allocated";
    case GEMM_MKL_STATUS_HIP_ERROR:
        std::snprintf(t_hip_msg, sizeof t_hip_msg, "HIP error: %s", hipGetErrorString(t_last_hip));
        return t_hip_msg;
    case GEMM_MKL_STATUS_NOT_AVAILABLE:
        return "not available: the forced configuration, prefetch depth or split does not exist or does not fit";
    default: return "unknown status";
    }
}

int gemm_mkl_num_configs(void) { return (int)registry().table.size(); }

const char *gemm_mkl_config_name(int id)
{
    Registry &R = registry();
    if (id < 0 || id >= (int)R.table.size()) return nullptr;
    return R.table[id].name;
}

int gemm_mkl_version(void) { return 100; }

}  // extern "C"
