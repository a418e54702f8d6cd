// kernels.h -- launch interface of the gfx950 GEMM kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fastdiv.h"

namespace dgw {

// Which epilogue/fixup a launch performs.
enum KernelMode : int {
    K_DP = 0,         // whole-K tiles, plain store
    K_SPLITK = 1,     // split s of tile t; fp32 partial [S,M,N] folded in split order (see KParams::merge)
    K_SK = 2,         // Stream-K, deterministic turnstile through per-unit partial slots
    K_SK_ATOMIC = 3,  // Stream-K, split tiles merged by fp32 atomic adds into zeroed C
    K_DP_GROUP = 4,   // whole-K tiles, one 2x2 group of tiles (256x256) per workgroup
};

// How Split-K merges its partials: folded in the same launch by the last
// arriver at the tile's counter, folded by a second kernel, added atomically
// into a zero-filled C, or (MERGE_BANDS, grids whose workgroups are all
// resident at once) folded in the same launch by all S splits of a tile, each
// adding up its own row bands once every split has arrived.  Every
// deterministic form adds the partials in split order: the same bits.
enum : int { MERGE_IN_LAUNCH = 0, MERGE_TWO_PASS = 1, MERGE_ATOMIC = 2, MERGE_BANDS = 3 };

// How final values reach C (the fused epilogue of the CUTLASS optimisation
// guide, "Epilogue Optimization": D = act(alpha acc + beta C + bias)).
enum : int {
    EPI_PLAIN = 0,   // C = acc
    EPI_FULL = 1,    // C = act(alpha acc + beta C_in + bias[col]), C_in read only when beta != 0
    EPI_ACCUM = 2,   // atomic merges: C already holds beta C_in + bias; whole tiles store
                     // fma(alpha, acc, C), split parts add alpha acc atomically (activation: a later pass)
};
enum : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2 };

// Stages of the elementwise epilogue pass over C.
enum : int {
    EPASS_PRE = 0,    // C = beta C + bias (before atomic merges)
    EPASS_POST = 1,   // C = act(C) (after atomic merges)
    EPASS_ONLY = 2,   // C = act(beta C + bias) (K == 0: the product is zero)
};

// Error bits of the device status word.
enum : uint32_t { STATUS_TIMEOUT = 1u };

// One problem of a grouped call (device table, nonempty problems only, in
// call order): its operands, sizes, first global tile id and the offset of
// its Split-K partials [S][M][N] in KParams::part.
struct GroupDesc {
    const uint16_t *A;
    const uint16_t *B;
    float *C;
    long long part;        // floats from KParams::part
    int M, N;
    int tile0;             // global id of the problem's first tile
    int pad;
};
static_assert(sizeof(GroupDesc) == 48, "device table entry");
// Problems per grouped call: one wave's lanes find a tile's problem at once.
constexpr int MAX_GROUPS = 64;

struct KParams {
    const uint16_t *A;     // [M,K] row-major 16-bit operands
    const uint16_t *B;     // [K,N] or [N,K] row-major
    float *C;              // [M,N] row-major fp32
    int M, N, K;
    int tm;                // tile rows: 128, 256 (tall Stream-K tile) or 64 (skinny tile); tiles are tm x 128
    int tiles_m, tiles_n;  // output tiles along M and N (of one batch entry)
    int group_m;           // tile ids run column by column in groups of group_m tile rows (0: row-major)
    int xcd_spread;        // 1: give each XCD a contiguous range of workers
    int ipt;               // k-iterations per tile
    int tile_base;         // first tile id of this launch (hybrid: Stream-K part starts at dp_tiles)
    int dp_tiles;          // Stream-K launch of a hybrid: whole-K tiles [0, dp_tiles) the units run first
    int ntiles;            // tiles of a DP / Split-K launch
    int units, q, big;     // Stream-K unit ranges: unit u starts at u*q + min(u, big)
    int splits;            // Split-K factor S
    int merge;             // MERGE_IN_LAUNCH, MERGE_TWO_PASS or (Split-K) MERGE_ATOMIC
    int worker_base;       // trace id of this launch's worker 0
    float *part;           // Stream-K slots [units][tm*BN] ([2][units][tm*BN] two-pass) or Split-K [S][M][N]
    uint32_t *flags;       // Stream-K: flag per unit (epoch-valued)
    uint32_t *counters;    // Split-K: arrival counter per tile (reset by the last arriver)
    uint32_t *status;      // device error word
    uint32_t epoch;        // value a publishing unit writes into its flag
    uint32_t spin_limit;   // polls before a wait gives up
    uint32_t debug;        // GEMM_DEBUG_* bits
    int batch;             // matrices of a batched call (tiles numbered batch after batch)
    const GroupDesc *groups;  // grouped call: the problems' table (tiles numbered problem after problem)
    int ngroups;           // entries of `groups` (0: not a grouped call)
    long long sA, sB, sC;  // element strides between batch entries of A, B (0: one shared matrix) and C
    long long sP;          // Split-K: element stride between batch entries' partials ([batch][S][M][N])
    int epi, act;          // EPI_* and ACT_*: the fused epilogue of the final stores
    float alpha, beta;     // epilogue scalars (EPI_FULL; EPI_ACCUM uses alpha)
    const float *bias;     // optional fp32 [N] added per column (EPI_FULL)
    const int *perm;       // optional workgroup -> worker map
    int *trace;            // optional debug trace (see gemm.h)
    long long *timing;     // optional per-workgroup {start, end, HW_ID | XCC_ID << 32, cycles, marks}
    int timing_base;       // entry of this launch's workgroup 0
    int trace_maxseg, trace_maxfold, trace_workers, trace_tiles;
    // launch constants for the kernels' index arithmetic (set by the launch
    // functions below from the fields above and the grid)
    FastDiv d_band;        // tiles of a full raster band: group_m (or tiles_m) x tiles_n
    FastDiv d_rows;        // tile rows of a full band
    FastDiv d_rows_last;   // tile rows of the last band
    FastDiv d_entry;       // tiles of one batch entry: tiles_m x tiles_n
    FastDiv d_ipt;         // k-iterations per tile
    FastDiv d_q, d_q1;     // Stream-K unit lengths max(q, 1) and q + 1
    FastDiv d_splits;      // Split-K factor
    int spread_a, spread_r;  // workers of the launch: per XCD (n / 8) and the remainder (n % 8)
};

// Launch `grid` workgroups of the kernel for (dtype, B layout, mode) on `stream`.
// dtype: 0 bf16, 1 fp16; blayout: 0 = B [K,N], 1 = B [N,K].  p.tm = 256 selects
// the 256 x 128 tile build (Stream-K kinds only, no fused epilogue); p.tm = 64
// the 64 x 128 tile builds (data-parallel, Split-K, Stream-K; no fused epilogue
// in Stream-K, no 2x2 tile groups).
hipError_t launch_gemm(int dtype, int blayout, int kmode, int grid, const KParams &p,
                       hipStream_t stream);

// Second pass of two-pass Split-K: C = ((P[0] + P[1]) + ...) + P[S-1] over the
// partials [S,M,N] of `p` (p.part, p.splits, p.M, p.N, the tile grid and raster).
hipError_t launch_splitk_reduce(const KParams &p, hipStream_t stream);

// Second pass of two-pass Stream-K: every split tile of the launch's Stream-K
// part (sk_tiles tiles from p.tile_base) gets its owner's and peers' partials
// added in k order.
hipError_t launch_streamk_reduce(const KParams &p, int64_t sk_tiles, hipStream_t stream);

// Elementwise epilogue pass over C[M,N] of every batch entry (stage EPASS_*;
// p.C, p.M, p.N, p.batch, p.sC, p.beta, p.bias, p.act).
hipError_t launch_epilogue_pass(const KParams &p, int stage, hipStream_t stream);

// Write a grouped call's problem table (at most MAX_GROUPS entries) to `dst`.
struct GroupTable {
    GroupDesc g[MAX_GROUPS];
};
hipError_t launch_put_groups(GroupDesc *dst, const GroupTable &t, int n, hipStream_t stream);

// Fill n 32-bit words with zero (used instead of hipMemsetAsync so the call can
// be captured in a HIP graph).
hipError_t launch_zero(void *ptr, int64_t n_words, hipStream_t stream);

// Resident workgroups per CU for the kernel of (dtype, blayout, kmode, tile rows
// tm), the grouped build when grp.
hipError_t blocks_per_cu(int dtype, int blayout, int kmode, int tm, bool grp, int *out);

}  // namespace dgw
