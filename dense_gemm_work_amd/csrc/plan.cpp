// plan.cpp -- host-side planning of a GEMM call: tile and wave arithmetic, the
// decomposition rule, Stream-K unit ranges and workspace sizing.  Integer code
// only; no GPU is touched.
//
// Sources (Split-K/Stream-K book chapter, "Split-K and Stream-K: The Last Wave
// of a GEMM"):
//  * Case 1: tiles = ceil(M/BM) ceil(N/BN), waves = ceil(tiles/SMs), tail wave.
//  * Stream-K paragraph after the glossary: unit u owns a contiguous slice of
//    the flattened (tile, k-iteration) space; Case 2 gives the first
//    (total mod units) units one extra iteration.
//  * The toy figure's caption, Case 2's discussion and Case 4's knob table
//    (decomposition rule): data-parallel when there is no partial wave or a
//    tile has at most 8 k-iterations; data-parallel when the tail wave is at
//    least half full; otherwise Stream-K over the last two waves with at least
//    8 iterations per unit, and Split-K when the units divide evenly over the
//    split tiles.
// docc StreamK page, "MMA fragment accumulators (aligned split)": Split-K with
// S dividing the panel count -- also a condition of the rule's Split-K choice.
#include "plan.h"

#include <algorithm>
#include <cstring>

namespace dgw {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

int64_t unit_begin(int64_t unit, int64_t q, int64_t big) {
    // units below `big` are one iteration longer
    return unit * q + std::min(unit, big);
}

constexpr uint32_t kTileBits = GEMM_TILE_256x128 | GEMM_TILE_64x128;

// GEMM_TILE_AUTO (CUTLASS guide, "Tile Size Selection": the tile follows the
// problem's shape).  Measured on MI355X, each against the 128 x 128 default:
// 64 x 128 tiles win wherever the 128 x 128 grid has too few tiles to fill half
// the CUs (256x512x2048 10.7 vs 12.1 us, 96x512x2048 9.5 vs 11.2 us,
// 128x4096x4096 14.2 vs 18.1 us); 256 x 128 Stream-K tiles halve the L2 -> LDS
// bytes per flop and win where a unit still runs many iterations
// (1536^2x16384: 72 per unit, 86.6 vs 91.7 us; 4096x4224x4096: 132 per unit,
// 130.0 vs 143.1 us) but lose where the fixed cost of a unit's segments
// dominates (2048x2176x4096: 34 per unit, 47.5 vs 42.4 us).
uint32_t choose_tile(int64_t M, int64_t N, int64_t K, int64_t batch, uint32_t layout, uint32_t mode, int32_t splits,
                     int32_t num_cus) {
    if ((mode & kTileBits) != GEMM_TILE_AUTO) return mode;
    const uint32_t base = mode & ~kTileBits;   // 128 x 128
    const char *why = nullptr;
    gemm_plan_t p128, p;
    if (make_plan(M, N, K, batch, layout, base, splits, num_cus, &p128, &why) != GEMM_OK) return base;
    if (2 * p128.tiles <= num_cus) {
        const uint32_t skinny = base | GEMM_TILE_64x128;
        return make_plan(M, N, K, batch, layout, skinny, splits, num_cus, &p, &why) == GEMM_OK ? skinny : base;
    }
    const uint32_t decomp = base & 0xFu;
    if (p128.decision == GEMM_STREAMK && !(base & GEMM_TWO_PASS) &&
        (decomp == GEMM_HEURISTIC || decomp == GEMM_STREAMK)) {
        const uint32_t tall = (base & ~0xFu) | GEMM_STREAMK | GEMM_TILE_256x128;
        if (make_plan(M, N, K, batch, layout, tall, splits, num_cus, &p, &why) == GEMM_OK && p.q >= 64) return tall;
    }
    return base;
}

int make_plan(int64_t M, int64_t N, int64_t K, int64_t batch, uint32_t layout, uint32_t mode, int32_t splits,
              int32_t num_cus, gemm_plan_t *out, const char **why) {
    static const char *none = "";
    *why = none;
    if (!out) { *why = "plan output pointer is null"; return GEMM_ERR_INVALID; }
    if ((mode & kTileBits) == GEMM_TILE_AUTO && num_cus >= 1)
        mode = choose_tile(M, N, K, batch, layout, mode, splits, num_cus);
    std::memset(out, 0, sizeof *out);
    if (M < 0 || N < 0 || K < 0) { *why = "M, N and K must be >= 0"; return GEMM_ERR_INVALID; }
    if (num_cus < 1) { *why = "num_cus must be >= 1"; return GEMM_ERR_INVALID; }
    if (batch < 1) { *why = "batch must be >= 1"; return GEMM_ERR_INVALID; }
    const uint32_t b_layout = layout & 0xFu, dtype = layout & 0xF0u;
    if ((layout & ~0xFFu) || (b_layout != GEMM_B_KN && b_layout != GEMM_B_NK) ||
        (dtype != GEMM_BF16 && dtype != GEMM_FP16)) {
        *why = "layout word has unknown bits";
        return GEMM_ERR_INVALID;
    }
    const uint32_t decomp = mode & 0xFu;
    const bool atomic = (mode & GEMM_ATOMIC) != 0;
    const bool two_pass = (mode & GEMM_TWO_PASS) != 0;
    const uint32_t tile = mode & (GEMM_TILE_256x128 | GEMM_TILE_64x128);
    const bool tall = tile == GEMM_TILE_256x128;
    if ((mode & ~(0xFu | GEMM_ATOMIC | GEMM_TWO_PASS | GEMM_TILE_256x128 | GEMM_TILE_64x128)) ||
        decomp > GEMM_STREAMK || tile == (GEMM_TILE_256x128 | GEMM_TILE_64x128)) {
        *why = "mode word has unknown bits";
        return GEMM_ERR_INVALID;
    }
    if (tall && (decomp != GEMM_STREAMK || two_pass)) {
        *why = "GEMM_TILE_256x128 applies to GEMM_STREAMK with the turnstile or atomic merge only";
        return GEMM_ERR_UNSUPPORTED;
    }
    if (atomic && decomp == GEMM_DP) {
        *why = "GEMM_ATOMIC applies to Stream-K and Split-K only";
        return GEMM_ERR_INVALID;
    }
    if (two_pass && (atomic || decomp == GEMM_DP)) {
        *why = "GEMM_TWO_PASS applies to deterministic Split-K and Stream-K only";
        return GEMM_ERR_INVALID;
    }
    if ((decomp == GEMM_DP || decomp == GEMM_HEURISTIC) && splits != 0) {
        *why = "splits must be 0 for GEMM_DP and GEMM_HEURISTIC";
        return GEMM_ERR_INVALID;
    }
    if (splits < 0) { *why = "splits must be >= 0"; return GEMM_ERR_INVALID; }
    if (K % 8 != 0) { *why = "K must be a multiple of 8 (128-bit row loads)"; return GEMM_ERR_UNSUPPORTED; }
    if (b_layout == GEMM_B_KN && N % 8 != 0) {
        *why = "N must be a multiple of 8 when B is stored [K,N] (128-bit row loads)";
        return GEMM_ERR_UNSUPPORTED;
    }
    // keep every flattened index and every per-tile buffer range (32-bit byte
    // offsets of a 128-row panel) within the kernels' arithmetic
    if (M > (int64_t(1) << 31) || N > (int64_t(1) << 22) || K > (int64_t(1) << 22)) {
        *why = "M must be at most 2^31, N and K at most 2^22";
        return GEMM_ERR_UNSUPPORTED;
    }

    gemm_plan_t &p = *out;
    p.atomic = 0;
    p.bm = tall ? 2 * GEMM_BM : (tile == GEMM_TILE_64x128 ? GEMM_BM / 2 : GEMM_BM);
    p.bn = GEMM_BN; p.bk = GEMM_BK;
    p.num_cus = num_cus;
    p.batch = batch;
    p.tiles_m = ceil_div(M, p.bm);
    p.tiles_n = ceil_div(N, GEMM_BN);
    // a batched call is one problem of batch x tiles_m x tiles_n tiles, numbered
    // batch after batch; the rule and the Stream-K flattening see that count
    p.tiles = batch * p.tiles_m * p.tiles_n;
    p.ipt = ceil_div(K, GEMM_BK);
    p.full_waves = p.tiles / num_cus;
    p.total_waves = ceil_div(p.tiles, num_cus);
    p.tail = p.tiles - (p.total_waves > 0 ? (p.total_waves - 1) * num_cus : 0);
    p.splits = 1;
    if (p.tiles * std::max<int64_t>(p.ipt, 1) >= (int64_t(1) << 31)) {
        *why = "tiles x k-iterations must stay below 2^31";
        return GEMM_ERR_UNSUPPORTED;
    }

    uint32_t chosen = decomp;
    int64_t units = 0, sk_tiles = 0;
    int32_t S = 1;
    if (decomp == GEMM_HEURISTIC) {
        // the tail wave is the only thing the rule balances: a whole number of
        // waves, a short K loop (at most 8 iterations) or a tail at least half
        // the CUs stays data-parallel
        const int64_t min_iters = 8;
        const bool ragged = p.tail > 0 && p.tail < num_cus;
        if (!ragged || p.ipt <= min_iters || 2 * p.tail >= num_cus) {
            chosen = GEMM_DP;
        } else {
            // Stream-K over the tail wave and the full wave before it (if any);
            // one unit per CU, but no fewer than 8 iterations per unit on average
            const int64_t kept_waves = std::max<int64_t>(p.total_waves - 2, 0);
            sk_tiles = p.tiles - kept_waves * num_cus;
            units = std::min<int64_t>(num_cus, (p.ipt * sk_tiles) / min_iters);
            // whole splits of every tile: plain Split-K, when S divides the tile's
            // iterations (the aligned split); otherwise Stream-K with those units
            const int64_t per_tile = units / sk_tiles;
            if (units % sk_tiles == 0 && per_tile > 1 && p.ipt % per_tile == 0) {
                chosen = GEMM_SPLITK;
                S = int32_t(per_tile);
            } else {
                chosen = GEMM_STREAMK;
            }
        }
        // GEMM_ATOMIC / GEMM_TWO_PASS apply to whichever of Stream-K and Split-K
        // the rule picks; data-parallel ignores them
    } else if (decomp == GEMM_SPLITK) {
        if (splits < 1) { *why = "GEMM_SPLITK needs splits >= 1"; return GEMM_ERR_INVALID; }
        if (p.ipt == 0 || p.ipt % splits != 0) {
            *why = "GEMM_SPLITK needs splits to divide ceil(K/64)";
            return GEMM_ERR_INVALID;
        }
        S = splits;
    } else if (decomp == GEMM_STREAMK) {
        units = splits > 0 ? splits : num_cus;
        sk_tiles = p.tiles;
    }

    p.decision = int32_t(chosen);
    switch (chosen) {
    case GEMM_DP:
        p.dp_tiles = p.tiles;
        p.workers = p.tiles;
        p.max_segments = 1;
        p.max_fold = 1;
        p.workspace_bytes = 0;
        break;
    case GEMM_SPLITK: {
        p.splits = S;
        p.atomic = atomic && S > 1 ? 1 : 0;
        // Deterministic: the partials are added in split order, by a second
        // kernel, or in the launch -- by all S splits of a tile, each adding up
        // its own row bands, when the whole grid is resident at once (the
        // library checks residency), else by the last arriver at the tile's
        // counter.  Same bits.  Measured on grids that fit the CUs: the row
        // bands win from S = 8 on small grids (96x512x2048 S = 8: 11.2 us
        // against 12.0 us with the second kernel; 64 and 128 workgroups within
        // 10 %), the second kernel below S = 8 (S = 2 and 4: 13.7 vs 15.0 us,
        // 11.5 vs 12.0 us), where a tile's fold is spread over too few
        // workgroups, and on grids of more than half the CUs, where every
        // split waits for the slowest (128x4096x4096 S = 8, 256 workgroups:
        // 18.1 us against 21.7 us in the launch); grids larger than the CUs
        // keep the last arriver, which folds partials still warm in L2
        // (2048x2176x4096 S = 2: 71.6 us in the launch, 75.9 us with the
        // second kernel).
        const bool fits = p.tiles * S <= num_cus;
        const bool bands = S >= 8 && 2 * p.tiles * S <= num_cus;
        p.two_pass = !p.atomic && S > 1 && (two_pass || (fits && !bands)) ? 1 : 0;
        p.workers = p.tiles * S;
        p.max_segments = 1;
        p.max_fold = S;
        // fp32 partials [batch, S, M, N] (none with atomics) and an arrival
        // counter per tile
        p.workspace_bytes = S > 1 && !p.atomic ? batch * int64_t(S) * M * N * 4 : 0;
        break;
    }
    case GEMM_STREAMK: {
        p.atomic = atomic ? 1 : 0;
        p.sk_units = units;
        p.sk_tiles = sk_tiles;
        p.dp_tiles = p.tiles - sk_tiles;
        const int64_t total = sk_tiles * p.ipt;
        p.q = units > 0 ? total / units : 0;
        p.big = units > 0 ? total % units : 0;
        p.workers = units + p.dp_tiles;
        const int64_t longest = p.q + (p.big > 0 ? 1 : 0);
        const int64_t ipt1 = std::max<int64_t>(p.ipt, 1);
        p.max_segments = int32_t(std::min<int64_t>(std::max<int64_t>(sk_tiles, 1),
                                                   ceil_div(longest, ipt1) + 1));
        p.max_fold = int32_t(std::min<int64_t>(units, ceil_div(ipt1, std::max<int64_t>(p.q, 1)) + 1));
        p.max_fold = std::max(p.max_fold, 1);
        // Deterministic: the owner of a split tile adds its peers' partials in k
        // order in the launch (turnstile), or every split segment publishes and a
        // second kernel adds them in the same order (same bits).  The turnstile's
        // owner takes its peers one after another, so with three or more peers per
        // tile (short units: max_fold >= 4) the second kernel is faster (measured:
        // 32 units of 8 iterations on 8 tiles 13.6 -> 11.9 us); with one or two
        // peers the turnstile is (2048x2176x4096: 45.7 vs 49.3 us; 1536^2 x 16384
        // fp16: 86.1 vs 88.9 us).
        p.two_pass = !atomic && !tall && (two_pass || p.max_fold >= 4) ? 1 : 0;
        // fp32 partial slots: one per unit for the turnstile (a unit publishes at
        // most its first segment); two per unit with the second kernel (its first
        // segment as a contributor, its last as an owner)
        p.workspace_bytes = atomic ? 0 : (p.two_pass ? 2 : 1) * units * int64_t(p.bm) * p.bn * 4;
        break;
    }
    default:
        *why = "internal: no decision";
        return GEMM_ERR_INVALID;
    }
    // control words: status (64 B), Stream-K flags, Split-K counters, each 256-B aligned
    p.workspace_bytes += control_bytes(p);
    p.trace_ints = 8 + p.workers * (1 + 4 * int64_t(p.max_segments)) +
                   p.tiles * (1 + int64_t(p.max_fold)) + p.tiles * p.ipt;
    return GEMM_OK;
}

int64_t group_table_bytes(int32_t count) { return (int64_t(count) * 48 + 255) / 256 * 256; }

int make_plan_grouped(const gemm_group_t *groups, int32_t count, int64_t K, uint32_t layout, uint32_t mode,
                      int32_t splits, int32_t num_cus, gemm_plan_t *out, const char **why) {
    static const char *none = "";
    *why = none;
    if (!out) { *why = "plan output pointer is null"; return GEMM_ERR_INVALID; }
    if (!groups || count < 1 || count > GEMM_MAX_GROUPS) {
        *why = "a grouped call takes 1..GEMM_MAX_GROUPS problems";
        return GEMM_ERR_INVALID;
    }
    if ((mode & kTileBits) == GEMM_TILE_AUTO && num_cus >= 1)
        mode = choose_tile_grouped(groups, count, K, layout, mode, splits, num_cus);
    const uint32_t tile = mode & kTileBits;
    if (tile == GEMM_TILE_256x128) {
        *why = "grouped calls run 128- and 64-row tiles (GEMM_TILE_256x128 is not offered)";
        return GEMM_ERR_UNSUPPORTED;
    }
    const int64_t bm = tile == GEMM_TILE_64x128 ? GEMM_BM / 2 : GEMM_BM;
    int64_t tiles = 0, mn = 0;
    for (int32_t g = 0; g < count; ++g) {
        const int64_t M = groups[g].M, N = groups[g].N;
        if (M < 0 || N < 0) { *why = "every problem's M and N must be >= 0"; return GEMM_ERR_INVALID; }
        if (M > (int64_t(1) << 31) || N > (int64_t(1) << 22)) {
            *why = "every problem's M must be at most 2^31 and N at most 2^22";
            return GEMM_ERR_UNSUPPORTED;
        }
        if ((layout & 0xFu) == GEMM_B_KN && N % 8 != 0) {
            *why = "every N must be a multiple of 8 when B is stored [K,N] (128-bit row loads)";
            return GEMM_ERR_UNSUPPORTED;
        }
        tiles += ceil_div(M, bm) * ceil_div(N, GEMM_BN);
        mn += M * N;
    }
    // tiles are numbered problem after problem: the schedule is that of one
    // problem of the same tile count (a column of `tiles` tiles)
    const int rc = make_plan(tiles * bm, GEMM_BN, K, 1, layout, mode, splits, num_cus, out, why);
    if (rc != GEMM_OK) return rc;
    if (out->decision == GEMM_SPLITK && !out->atomic && out->splits > 1)
        out->workspace_bytes = control_bytes(*out) + int64_t(out->splits) * mn * 4;
    out->workspace_bytes = (out->workspace_bytes + 255) / 256 * 256 + group_table_bytes(count);
    return GEMM_OK;
}

// GEMM_TILE_AUTO for a grouped call (no epilogue, no 256-row tiles): 64 x 128
// tiles when the problems' 128 x 128 tiles cannot fill half the CUs.
uint32_t choose_tile_grouped(const gemm_group_t *groups, int32_t count, int64_t K, uint32_t layout, uint32_t mode,
                             int32_t splits, int32_t num_cus) {
    if ((mode & kTileBits) != GEMM_TILE_AUTO) return mode;
    const uint32_t base = mode & ~kTileBits;
    const char *why = nullptr;
    gemm_plan_t p128, p;
    if (make_plan_grouped(groups, count, K, layout, base, splits, num_cus, &p128, &why) != GEMM_OK) return base;
    const uint32_t skinny = base | GEMM_TILE_64x128;
    if (2 * p128.tiles <= num_cus &&
        make_plan_grouped(groups, count, K, layout, skinny, splits, num_cus, &p, &why) == GEMM_OK)
        return skinny;
    return base;
}

int64_t control_bytes(const gemm_plan_t &p) {
    auto round = [](int64_t b) { return (b + 255) / 256 * 256; };
    return 256 + round(std::max<int64_t>(p.sk_units, 1) * 4) + round(std::max<int64_t>(p.tiles, 1) * 4);
}

}  // namespace dgw

extern "C" int gemm_plan_grouped(const gemm_group_t *groups, int32_t count, int64_t K, uint32_t layout, uint32_t mode,
                                 int32_t splits, int32_t num_cus, gemm_plan_t *out) {
    const char *why = "";
    return dgw::make_plan_grouped(groups, count, K, layout, mode, splits, num_cus, out, &why);
}

extern "C" int gemm_unit_range(const gemm_plan_t *plan, int64_t unit, int64_t *begin, int64_t *end) {
    if (!plan || !begin || !end) return GEMM_ERR_INVALID;
    if (plan->decision != GEMM_STREAMK || unit < 0 || unit >= plan->sk_units) return GEMM_ERR_INVALID;
    *begin = dgw::unit_begin(unit, plan->q, plan->big);
    *end = *begin + plan->q + (unit < plan->big ? 1 : 0);
    return GEMM_OK;
}
