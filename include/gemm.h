/*
 * gemm.h -- C ABI of the MI355X (gfx950) data-parallel / Split-K / Stream-K GEMM.
 *
 * Operation (every entry point computes the same thing):
 *
 *     C[M,N] = A[M,K] . B          (B stored [K,N], row-major)        layout GEMM_B_KN
 *     C[M,N] = A[M,K] . B^T        (B stored [N,K], row-major)        layout GEMM_B_NK
 *
 * for one product or (gemm_ex, gemm_args_t.batch) a batch of products of one
 * shape with strided operands.
 *
 * A and B hold bf16 or fp16 values; products are accumulated in fp32 and C is
 * written in fp32: overwritten with the product, or (gemm_ex with an epilogue
 * word) C = act(alpha A.B + beta C + bias), see GEMM_EPI_* below.  The work decomposition is the
 * subject of the Split-K/Stream-K book chapter ("Split-K and Stream-K: The Last
 * Wave of a GEMM", kanthi.in): output tiles of 128x128 elements, one
 * "MAC-loop iteration" per 64-wide step of K (glossary table), and three ways
 * to hand iterations to workgroups:
 *
 *   GEMM_DP       one workgroup per output tile, whole K loop (glossary, "Data-parallel").
 *   GEMM_SPLITK   S workgroups per tile; tile t, split s covers k-iterations
 *                 [s P/S, (s+1) P/S) of the tile's P iterations, stores an fp32
 *                 partial into a [S,M,N] workspace, and C receives the S
 *                 partials added in split order (docc StreamK page, "MMA
 *                 fragment accumulators (aligned split)"): by a second kernel
 *                 ("serial" Split-K; chosen when all tiles x S workgroups fit on
 *                 the CUs at once, unless S >= 8 and they fill at most half of
 *                 them, or asked for with GEMM_TWO_PASS; plan.two_pass says
 *                 which), else in the same launch -- by all S splits of each
 *                 tile, each adding up its own row bands (an eighth of the tile
 *                 each) once every split has arrived, when the grid is resident
 *                 at once, or by the last arriver at the tile's counter.  All
 *                 give the same bits.  GEMM_ATOMIC adds
 *                 every split into a zero-filled C instead ("parallel" Split-K;
 *                 CUTLASS optimisation guide, "Parallelized Reductions (Split-K)").
 *   GEMM_STREAMK  one persistent workgroup per unit; unit u owns a contiguous,
 *                 equal slice of the flattened (tile x k-iteration) space, the
 *                 first (total mod units) units taking one extra iteration
 *                 (book chapter, Stream-K paragraph after the glossary, and Case 2).
 *                 A unit that starts a tile mid-K publishes an fp32 partial and
 *                 a flag; the unit holding the tile's k = 0 iteration waits for
 *                 its peers in k order, adds their partials and writes C
 *                 (deterministic "turnstile", Case 4's reduction modes).  When a
 *                 tile can have three or more peers (plan.max_fold >= 4), or with
 *                 GEMM_TWO_PASS, every split segment publishes instead and a
 *                 second kernel adds each tile's partials in the same k order
 *                 (Case 3's separate fixup kernel; same bits; plan.two_pass).  With
 *                 GEMM_ATOMIC, split tiles are instead merged by fp32 atomic
 *                 adds into C, which the library zero-fills first
 *                 (nondeterministic mode; docc StreamK page, "Rewrite it produces").
 *   GEMM_HEURISTIC  the decomposition rule of Case 2 / Case 4 with SMs = CUs:
 *                 DP if there is no partial wave or P <= 8; DP if the tail wave
 *                 is at least half full; otherwise Stream-K over the last two
 *                 waves with at least 8 iterations per unit (the earlier waves
 *                 stay DP: the persistent units run those whole-K tiles first,
 *                 in the same launch), or Split-K when those units divide
 *                 evenly over the Stream-K tiles.
 *
 * Threading and streams: every call is asynchronous on a HIP stream (the one
 * given to gemm_ex, else the calling thread's stream from gemm_set_stream,
 * else the null stream).  The library-owned workspace is one per device;
 * calls that use it must be ordered on the device (one stream, or streams
 * synchronised by the caller).  Calls that overlap on one device race.
 *
 * Graph capture: a call enqueues kernels only (no memset or copy), so it can be
 * captured in a HIP graph once an eager call with the same plan (any eager call
 * on the device, with a caller workspace) has sized the library workspace;
 * replays must not overlap.  A call that would have to grow the library
 * workspace while its stream is being captured returns GEMM_ERR_WORKSPACE and
 * launches nothing.  The library workspace only grows: an outgrown block is
 * retired but stays allocated until gemm_release(), so a graph captured before
 * a larger eager call still replays into valid memory (gemm_release() ends
 * that: do not replay graphs of library-workspace calls after it).  Stream-K
 * flags clear themselves after use, so the replays' fixed epoch works.
 *
 * Errors: a negative status is returned and nothing is launched (C untouched)
 * for every condition the host can detect; gemm_last_error() then describes it.
 */
#ifndef DGW_GEMM_H
#define DGW_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------------- */
#define GEMM_OK               0
#define GEMM_ERR_INVALID     (-1)   /* bad argument (null pointer, bad size, bad mode bits, ...) */
#define GEMM_ERR_UNSUPPORTED (-2)   /* legal but outside what the kernels handle (alignment, capacity) */
#define GEMM_ERR_WORKSPACE   (-3)   /* workspace too small or could not be allocated */
#define GEMM_ERR_HIP         (-4)   /* a HIP runtime call or a launch failed */
#define GEMM_ERR_TIMEOUT     (-5)   /* a Stream-K/Split-K wait hit its spin limit (gemm_sync_status) */

/* ---- layout word ------------------------------------------------------------- */
/* bits 0-3: how B is stored (A is always [M,K] row-major, C always fp32 [M,N] row-major) */
#define GEMM_B_KN   0x00u   /* B is [K,N] row-major: C = A.B                      */
#define GEMM_B_NK   0x01u   /* B is [N,K] row-major: C = A.B^T (weights as [N,K]) */
/* bits 4-7: operand type of A and B */
#define GEMM_BF16   0x00u
#define GEMM_FP16   0x10u

/* ---- mode word ----------------------------------------------------------------- */
/* bits 0-3: decomposition */
#define GEMM_HEURISTIC 0x0u
#define GEMM_DP        0x1u
#define GEMM_SPLITK    0x2u
#define GEMM_STREAMK   0x3u
/* bits 8-9: how split tiles are merged (Stream-K and Split-K) */
#define GEMM_DETERMINISTIC 0x000u  /* k-ordered: Stream-K turnstile / Split-K fold in the same launch */
#define GEMM_ATOMIC        0x100u  /* fp32 atomic adds into a zero-filled C (Stream-K, Split-K) */
#define GEMM_TWO_PASS      0x200u  /* always add split tiles' partials in k order by a second
                                      kernel (Split-K and Stream-K; same bits as in the launch) */
/* bits 12-13: output tile shape */
#define GEMM_TILE_128x128  0x0000u /* 128 x 128 tiles (every decomposition)                     */
#define GEMM_TILE_256x128  0x1000u /* 256 x 128 tiles: GEMM_STREAMK only (turnstile or
                                      GEMM_ATOMIC merge; no GEMM_TWO_PASS).
                                      The tile the book chapter's Case 4 names for CUTLASS's
                                      Stream-K example (MmaTileShape 256 x 128 x 64); a unit's
                                      64-wide k-iteration is then twice the work, the partial
                                      slot 128 KiB.                                            */
#define GEMM_TILE_64x128   0x2000u /* 64 x 128 tiles: the skinny shape for small M (the CUTLASS
                                      guide's "Tile Size Selection", tall/skinny tab: 64-row
                                      tiles when N is much larger than M; the book chapter's
                                      skinny-problem paragraph: a decode batch of M = 128 has
                                      too few 128-row tiles to fill the GPU).  Every
                                      decomposition, merge and fused epilogue; no 2x2
                                      tile groups for data-parallel launches.  Twice the tile
                                      rows of 128 x 128 tiles (M = 128 gives two), half the
                                      partial bytes per split (32 KiB slots).                 */
#define GEMM_TILE_AUTO     0x3000u /* the library picks one of the three per call (the CUTLASS
                                      guide's "Tile Size Selection": the tile follows the
                                      problem's shape).  The choice is fixed per shape, CU
                                      count and mode, and is taken before planning; gemm_plan
                                      reports it in bm.  With T = tiles of the 128 x 128 plan
                                      and C the CUs: 64 x 128 when 2 T <= C (too few tiles to
                                      fill half the GPU; every decomposition); else
                                      256 x 128 Stream-K when the 128 x 128 plan is Stream-K
                                      (GEMM_HEURISTIC or GEMM_STREAMK; not GEMM_TWO_PASS)
                                      and each unit of the 256 x 128 plan runs
                                      at least 64 k-iterations, so its fixed cost stays small
                                      beside its loop; else 128 x 128.  Grouped calls choose
                                      between 128 x 128 and 64 x 128 only.                    */

/* ---- debug bits for gemm_args_t.debug -------------------------------------------- */
#define GEMM_DEBUG_NO_PUBLISH 0x1u /* Stream-K contributors store partials but never
                                      raise their flags: every wait ends at its spin
                                      limit and gemm_sync_status() reports
                                      GEMM_ERR_TIMEOUT.  Exercises the failure path;
                                      C is not valid.                               */
#define GEMM_DEBUG_IN_LAUNCH 0x4u /* deterministic merges stay in the launch (Split-K:
                                    the last arriver at each tile's counter; Stream-K:
                                    the turnstile) even where the plan chose a second
                                    kernel.  Same result bits; exercises that path. */
#define GEMM_DEBUG_TILE_DP 0x8u /* data-parallel launches run one 128x128 tile per
                                   workgroup even where 2x2 tile groups apply.     */
#define GEMM_DEBUG_HYBRID_SPLIT 0x10u /* a hybrid's data-parallel tiles run as a second
                                         launch after the Stream-K one instead of by
                                         the persistent units first.  Same values.  */
#define GEMM_DEBUG_SPLITK_BANDS 0x40u /* deterministic Split-K on a grid whose workgroups
                                         are all resident: add the partials in the launch,
                                         each split adding up its own row bands, even where
                                         the plan chose a second kernel.  Same bits.      */
#define GEMM_DEBUG_ZERO_PARTIAL 0x20u /* numerical control: every partial a split tile
                                         hands to another workgroup is written as zeros
                                         (Stream-K slots, Split-K partials of both merge
                                         forms, atomic adds into C).  Every call with a
                                         split tile then returns a wrong C; a parity
                                         check that still passes has no teeth (Metal
                                         split-K note, "Contract and numerical
                                         coverage": the zero-partial control).       */

/* ---- epilogue word for gemm_args_t.epilogue ------------------------------------------ */
/*
 * Fused epilogue (CUTLASS optimisation guide, "Epilogue Optimization": the
 * epilogue forms alpha.AB + beta.C; "Fused Epilogue Operations": bias addition
 * and a ReLU or GELU activation in the same pass).  With a non-zero word the
 * call writes, for every element,
 *
 *     C[i][j] = act(alpha * (A.B)[i][j] + beta * C_in[i][j] + bias[j])
 *
 * where C_in is C's content before the call (read only when beta != 0, so a
 * NaN there is ignored with beta == 0) and bias is one fp32 value per column.
 * Arithmetic (fp32, each step rounded, no contraction): t = beta * C_in
 * (0 when beta == 0), y = fma(alpha, acc, t), y = y + bias[j], then ReLU
 * max(y, 0) or GELU (y / 2) * (1 + erf(y / sqrt 2)), erf from the rational
 * approximation of Abramowitz and Stegun 7.1.26 (absolute error below
 * 1.5e-7; relative error of GELU below 4e-7 of |y|).  Deterministic merges
 * keep their guarantee: the same call gives the same bits on every run, and a
 * two-pass merge the same bits as the in-launch one.  With GEMM_ATOMIC, C is
 * first set to beta * C_in + bias, tiles and split segments add alpha * acc,
 * and an activation runs as a final elementwise pass (tolerance only).  With
 * K == 0 the product is zero: C = act(beta * C_in + bias).
 */
#define GEMM_EPI_ALPHA_BETA 0x01u  /* use alpha and beta (else alpha = 1, beta = 0)      */
#define GEMM_EPI_BIAS       0x02u  /* add bias[j]: device fp32 [N], 16-byte aligned     */
#define GEMM_EPI_RELU       0x10u  /* act = max(y, 0)                                   */
#define GEMM_EPI_GELU       0x20u  /* act = y Phi(y), Phi the standard normal CDF       */

/* Tile shape used by every decomposition. */
#define GEMM_BM 128
#define GEMM_BN 128
#define GEMM_BK 64

/*
 * Result of planning one call (host arithmetic only; never touches a GPU).
 * Tile counts follow the wave arithmetic of the book chapter, Case 1:
 * tiles = ceil(M/BM) ceil(N/BN), waves = ceil(tiles/CUs).
 */
typedef struct gemm_plan_t {
    int32_t decision;     /* GEMM_DP, GEMM_SPLITK or GEMM_STREAMK                          */
    int32_t atomic;       /* 1 when split tiles (Stream-K or Split-K) merge by atomics      */
    int32_t bm, bn, bk;   /* tile shape                                                     */
    int32_t num_cus;      /* compute units the plan was made for                            */
    int64_t tiles_m, tiles_n, tiles;
    int64_t ipt;          /* k-iterations per tile, P = ceil(K / bk)                        */
    int64_t full_waves;   /* floor(tiles / CUs)                                             */
    int64_t total_waves;  /* ceil(tiles / CUs)                                              */
    int64_t tail;         /* tiles in the last wave                                         */
    int64_t sk_tiles;     /* Stream-K: tiles in the stream part (the LAST sk_tiles tiles)   */
    int64_t sk_units;     /* Stream-K: units (persistent workgroups)                        */
    int64_t dp_tiles;     /* tiles run as whole-K data-parallel tiles (tiles 0..dp_tiles-1) */
    int64_t q;            /* Stream-K: floor(sk_tiles * ipt / units)                        */
    int64_t big;          /* Stream-K: (sk_tiles * ipt) mod units = units with q+1 iters    */
    int32_t splits;       /* Split-K factor S (1 for the other decompositions)              */
    int32_t max_segments; /* most tile segments one worker can touch                        */
    int32_t max_fold;     /* most workers contributing to one tile                          */
    int32_t two_pass;     /* 1 when split tiles' partials are added by a second kernel (the
                             plan picks it for Split-K grids that fit on the CUs at once,
                             except S >= 8 on at most half of them, and for Stream-K
                             tiles with three or more peers)                              */
    int64_t workers;      /* traced workers: units + dp_tiles, tiles * S, or tiles          */
    int64_t workspace_bytes; /* device workspace the call needs                             */
    int64_t trace_ints;   /* int32 elements of a debug trace buffer for this call           */
    int64_t batch;        /* products in the call; tiles = batch * tiles_m * tiles_n,
                             numbered batch entry after batch entry                        */
} gemm_plan_t;

/*
 * Extended arguments.  Zero-initialise, then fill what you need.
 *   A, B, C, M, N, K, layout, mode, splits: as for gemm().
 *   stream:   hipStream_t to enqueue on; NULL = the thread's gemm_set_stream value.
 *   workspace, workspace_bytes: caller-owned device memory of at least
 *             plan.workspace_bytes, zero-filled before its first use and used by
 *             one stream at a time; NULL = the library's per-device workspace.
 *   num_cus:  plan for this many CUs instead of the device's count (>= 1).  The
 *             Stream-K grid must still fit on the device (all units co-resident).
 *   unit_perm: optional device int32[grid]: workgroup b runs unit unit_perm[b]
 *             (Stream-K) or worker unit_perm[b] (DP / Split-K).  Must be a
 *             permutation of 0..grid-1.  The schedule does not change, only which
 *             workgroup runs it (stresses arrival order).
 *   trace, trace_ints: optional device int32 buffer of at least plan.trace_ints
 *             elements; the kernels record what they did (layout in
 *             gemm_trace_layout below).  The library zero-fills it first.
 *   spin_limit: bound on every inter-workgroup wait, in polls (0 = default).
 *   debug:    GEMM_DEBUG_* bits (0 in normal use).
 *   timing:   optional device int64 buffer of at least 8 * plan.workers elements:
 *             workgroup g of the call (launch order: the main grid, then, with
 *             GEMM_DEBUG_HYBRID_SPLIT, the DP tiles of a hybrid) writes
 *             {start, end, HW_ID | XCC_ID << 32, cycles,
 *             m0, m1, m2, m3}: times in ticks of the 100 MHz s_memrealtime clock,
 *             HW_ID and XCC_ID as read from the hardware registers (CU, SE and XCD
 *             placement), cycles = shader-clock ticks (s_memtime) from start to end,
 *             so cycles / (end - start) * 100 MHz is the workgroup's mean clock.
 *             Marks: DP m0 = mainloop done; Split-K m0 = mainloop done, m1 =
 *             partial stored, m2 = fold done (last arriver, or a split's bands),
 *             m3 = every split of the tile arrived (row-band merge); Stream-K m0/m1 =
 *             first segment's mainloop / fixup-and-store done, m2/m3 = the same
 *             for the unit's last segment.  Unset marks stay as the caller left them.
 *   epilogue: GEMM_EPI_* bits (0: C is overwritten with A.B).  RELU and GELU
 *             exclude each other; GEMM_EPI_BIAS is set exactly when bias != NULL.
 *   alpha, beta: epilogue scalars, used with GEMM_EPI_ALPHA_BETA.
 *   bias:     device fp32 [N] (16-byte aligned, not overlapping C), or NULL; one
 *             bias serves every batch entry.
 *   batch:    number of independent products C_b = A_b . B_b of one shape
 *             (0 or 1: a single product).  Entry b starts stride_a / stride_b /
 *             stride_c ELEMENTS after entry b - 1 (A and B: >= 0, a 0 stride
 *             shares one matrix among all entries; C: >= M*N, entries must not
 *             overlap; A and B strides multiples of 8, C's of 4, keeping 16-byte
 *             alignment).  The decomposition sees batch * tiles_m * tiles_n tiles,
 *             numbered entry after entry, so Stream-K units and Split-K work
 *             spread over all entries (docc StreamK page, generality: batched
 *             GEMM).  Strides are ignored when batch <= 1.
 * Tuning overrides read once from the environment (defaults in brackets):
 *   DGW_GROUP_M    tile rows per raster group [8]; tile ids run column by column
 *                  within a group of rows (0 = plain row-major)
 *   DGW_XCD_SPREAD 1: consecutive workers on the same XCD [1]; 0: workgroup order
 */
typedef struct gemm_args_t {
    const void *A;
    const void *B;
    float *C;
    int64_t M, N, K;
    uint32_t layout;
    uint32_t mode;
    int32_t splits;
    int32_t num_cus;
    void *stream;
    void *workspace;
    size_t workspace_bytes;
    const int32_t *unit_perm;
    int32_t *trace;
    int64_t trace_ints;
    uint32_t spin_limit;
    uint32_t debug;
    int64_t *timing;
    uint32_t epilogue;
    float alpha;
    float beta;
    const float *bias;
    int64_t batch;
    int64_t stride_a;
    int64_t stride_b;
    int64_t stride_c;
} gemm_args_t;

/*
 * Debug trace layout (int32 elements), written only when gemm_args_t.trace is set:
 *   [0..7]   header: 0x4B525453 ("STRK"), decision, workers, tiles, ipt,
 *            max_segments, max_fold, splits
 *   then, per worker w (0..workers-1): 1 + 4*max_segments ints:
 *            count, then count records (tile, k0, k1, role) in execution order,
 *            role 0 = whole tile, 1 = k = 0 holder that waits and folds,
 *            2 = starts mid-tile and publishes a partial
 *   then, per tile t: 1 + max_fold ints: count, then the workers whose partials
 *            were summed into the tile, in summation order (a whole tile lists
 *            its one worker; under GEMM_ATOMIC a split tile's count stays 0)
 *   then, per tile t: ipt ints: how many times each (tile, k-iteration) was run.
 * Worker ids: Stream-K unit u -> u; hybrid DP tile t -> units + t;
 * Split-K tile t split s -> t*S + s; DP tile t -> t.
 */

/*
 * gemm -- the core call.
 *   A: device pointer, [M,K] row-major bf16/fp16.
 *   B: device pointer, [K,N] (GEMM_B_KN) or [N,K] (GEMM_B_NK) row-major, same type as A.
 *   C: device pointer, [M,N] row-major fp32; overwritten.  Must not overlap A or B.
 *   M, N, K >= 0.  M == 0 or N == 0: nothing to do.  K == 0: C is zero-filled.
 *   layout: GEMM_B_KN|GEMM_B_NK combined with GEMM_BF16|GEMM_FP16.
 *   mode: GEMM_HEURISTIC|GEMM_DP|GEMM_SPLITK|GEMM_STREAMK, optionally | GEMM_ATOMIC
 *         or | GEMM_TWO_PASS (Stream-K and Split-K; not both).
 *   splits: GEMM_SPLITK: S >= 1 dividing ceil(K/64).  GEMM_STREAMK: unit count
 *           (0 = one per CU).  GEMM_DP / GEMM_HEURISTIC: must be 0.
 * Requirements (else GEMM_ERR_UNSUPPORTED): A, B, C 16-byte aligned; K a
 * multiple of 8; N a multiple of 8 for GEMM_B_KN (128-bit row loads).
 * Ownership: the caller owns A, B, C and the stream; nothing is retained.
 * Returns GEMM_OK once the work is enqueued (asynchronous).
 */
int gemm(const void *A, const void *B, float *C, int64_t M, int64_t N, int64_t K,
         uint32_t layout, uint32_t mode, int32_t splits);

/* gemm_ex -- gemm() with the extended arguments above. */
int gemm_ex(const gemm_args_t *args);

/*
 * gemm_ex_noalloc -- gemm_ex() that allocates no device memory, for callers
 * that cannot: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, same kernels and the same result bits
 * as gemm_ex() with the library workspace, except:
 *   - args->workspace must be NULL (else GEMM_ERR_INVALID): the workspace is a
 *     fixed array of GEMM_NOALLOC_MAX_BYTES inside the library, one copy per
 *     GPU, set up by the first call on that GPU and held until the process
 *     ends.
 *   - A call whose plan needs more (plan.workspace_bytes, e.g. Split-K
 *     partials [S,M,N] beyond it) returns GEMM_ERR_WORKSPACE and launches
 *     nothing.  Every decomposition of a 128x128-tile problem with at most 256
 *     Stream-K units fits (two-pass Stream-K: 32 MiB of slots).
 *   - Every call on a GPU shares that GPU's array and leaves its contents
 *     behind; each call clears the flags and counters it uses (a kernel, no
 *     memset).  Calls that overlap on one GPU race: order them on one stream
 *     (or synchronise), as for the library workspace.
 *   - gemm_sync_status() also reports the array's status word.
 * Calls no hipMalloc, hipFree or other allocating routine.
 */
#define GEMM_NOALLOC_MAX_BYTES (32u * 1024u * 1024u + 256u * 1024u)
int gemm_ex_noalloc(const gemm_args_t *args);

/*
 * Grouped calls: several problems C_g = A_g . B_g (or A_g . B_g^T) of one K,
 * layout and dtype but their own M_g and N_g (e.g. the experts of a mixture
 * layer), decomposed as one call (docc StreamK page, generality: grouped
 * GEMM).  Their tiles are numbered problem after problem, so the rule, the
 * Stream-K flattening and Split-K see every problem's tiles at once and one
 * persistent launch balances them; the plan is the plan of one problem with
 * the same tile count.  Up to GEMM_MAX_GROUPS problems; M_g = 0 or N_g = 0
 * skips a problem.
 */
typedef struct gemm_group_t {
    const void *A;   /* device, [M,K] row-major, 16-byte aligned (may be NULL when M*N == 0) */
    const void *B;   /* device, [K,N] or [N,K] row-major, 16-byte aligned                   */
    float *C;        /* device, [M,N] row-major fp32, overwritten; must not overlap A or B  */
    int64_t M, N;    /* >= 0; N a multiple of 8 for GEMM_B_KN                               */
} gemm_group_t;
#define GEMM_MAX_GROUPS 64

/*
 * gemm_grouped -- run `count` (1..GEMM_MAX_GROUPS) problems as one call.
 * `common` carries what the problems share and the call's options, as for
 * gemm_ex(): K, layout, mode, splits, stream, workspace / workspace_bytes,
 * num_cus, unit_perm, trace / trace_ints, spin_limit, debug, timing.  Its A, B,
 * C, M, N, bias and batch must be zero / NULL (GEMM_ERR_INVALID otherwise), and
 * the fused epilogue is not offered (epilogue != 0: GEMM_ERR_UNSUPPORTED).
 * Tiles: 128x128 or GEMM_TILE_64x128 (GEMM_TILE_256x128: GEMM_ERR_UNSUPPORTED).
 * Data-parallel launches run one tile per workgroup (no 2x2 tile groups).
 * The problem table is copied into the workspace by a kernel (no memset, no
 * host-to-device copy), so the call can be captured in a graph; `groups` is
 * read on the host before the call returns.  Asynchronous; returns a status.
 */
int gemm_grouped(const gemm_args_t *common, const gemm_group_t *groups, int32_t count);

/*
 * gemm_plan_grouped -- gemm_plan for a grouped call (only M and N of each group
 * are read).  tiles is the problems' total; tiles_m = tiles and tiles_n = 1
 * (the stacked problem whose schedule the call runs); workspace_bytes includes
 * the Split-K partials of every problem ([S][M_g][N_g] each) and the table.
 */
int gemm_plan_grouped(const gemm_group_t *groups, int32_t count, int64_t K, uint32_t layout, uint32_t mode,
                      int32_t splits, int32_t num_cus, gemm_plan_t *out);

/*
 * gemm_plan -- decide the decomposition for a call without running it.
 * num_cus >= 1 (no device is queried).  Fills *out; returns a status.  With
 * GEMM_TILE_AUTO, bm reports the tile the call runs.
 */
int gemm_plan(int64_t M, int64_t N, int64_t K, uint32_t layout, uint32_t mode,
              int32_t splits, int32_t num_cus, gemm_plan_t *out);

/* gemm_plan_batched -- gemm_plan for a call of `batch` (>= 1) products. */
int gemm_plan_batched(int64_t M, int64_t N, int64_t K, int64_t batch, uint32_t layout,
                      uint32_t mode, int32_t splits, int32_t num_cus, gemm_plan_t *out);

/*
 * gemm_workspace_size -- device workspace bytes a call with these arguments
 * needs (plan.workspace_bytes), for a caller that passes its own
 * gemm_args_t.workspace.  What it holds follows the pages' merge designs: the
 * docc StreamK page's aligned split ("MMA fragment accumulators") keeps one fp32
 * slot per split and an arrival counter per tile (here Split-K partials
 * [batch][S][M][N] and a counter per tile); the book chapter's Stream-K paragraph
 * has a unit that starts mid-tile store an fp32 partial and signal (here one
 * 64 KiB slot and one flag per unit; two slots per unit when a second kernel
 * adds the partials, Case 3's fixup kernel).  Plus a 256-byte status block.
 * Layout: [status 256 B | flags, 256-B aligned | counters, 256-B aligned | data].
 * batch >= 1; num_cus >= 1 (no device is queried).  Returns the byte count
 * (>= 0) or a negative status for arguments gemm_plan_batched rejects.
 * Ownership: the caller allocates, zero-fills once and frees it.
 */
int64_t gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t batch, uint32_t layout,
                            uint32_t mode, int32_t splits, int32_t num_cus);

/*
 * gemm_unit_range -- [begin, end) of Stream-K unit u in the flattened
 * (tile x k-iteration) space of the plan's Stream-K tiles: the book chapter's
 * Stream-K paragraph gives every unit an equal contiguous slice of that space,
 * and its Case 2 gives the first (total mod units) units one iteration more, so
 * begin = u q + min(u, big) and end = begin + q + (u < big).  Iteration g of the
 * space is k-iteration g mod ipt of Stream-K tile g / ipt (tile dp_tiles + g / ipt
 * of the call).  Host arithmetic only.  Returns GEMM_OK, or GEMM_ERR_INVALID
 * for a null pointer, a plan that is not Stream-K, or u outside [0, sk_units).
 */
int gemm_unit_range(const gemm_plan_t *plan, int64_t unit, int64_t *begin, int64_t *end);

/* gemm_set_stream -- the calling thread's default stream (hipStream_t, may be NULL). */
int gemm_set_stream(void *stream);

/*
 * gemm_sync_status -- wait for the calling thread's stream (or `stream` if not
 * NULL), then report and clear the device-side error word of the current
 * device's library workspace: GEMM_OK, or GEMM_ERR_TIMEOUT if a bounded wait
 * gave up since the last call.
 */
int gemm_sync_status(void *stream);

/* gemm_release -- free the library-owned workspace of every device, retired
 * blocks included (synchronises every device first).  Graphs captured from
 * calls on the library workspace must not be replayed afterwards. */
void gemm_release(void);

/* gemm_last_error -- text for the calling thread's last failing call ("" if none). */
const char *gemm_last_error(void);

/* gemm_num_cus -- compute units of the current device (0 if there is none). */
int32_t gemm_num_cus(void);

/* gemm_version -- ABI version of this header (2: gemm_args_t gained the epilogue fields). */
int32_t gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DGW_GEMM_H */
