// gemm_kernels.hip -- gfx950 (MI355X) kernels of the DP / Split-K / Stream-K GEMM.
//
// One mainloop serves every decomposition.  A workgroup of 256 threads (four
// 64-wide waves in a 2x2 arrangement) computes one 128x128 fp32 output tile;
// one "MAC-loop iteration" (Split-K/Stream-K book chapter, glossary) is a
// 64-wide step of K: the A slab [128 x 64] and the B slab [64 x 128] are staged
// in LDS and each wave issues 16 v_mfma_f32_32x32x16_{bf16,f16} on its 64x64
// quarter.  Slabs are double-buffered in LDS: the 128-bit global loads of
// iteration i+1 are in flight while iteration i runs on the matrix cores
// (CUTLASS optimisation guide, "Software Pipelining").
//
// LDS layout: both operands are stored "k-contiguous", one 128-byte row of 64
// values per M row (A) or N column (B), with the 16-byte chunks of row r
// XOR-swizzled by (r ^ r>>3) & 7 so that the MFMA operand reads (eight rows,
// same logical chunk, per 128 bytes) hit distinct banks.  A [M,K] and B [N,K]
// rows are copied as they are; B [K,N] is transposed in registers on its way
// to LDS (four k-rows of eight n-values per thread become eight 4-value
// k-runs), so the matrix cores always read 8 consecutive k per lane.
//
// Epilogues (book chapter, Stream-K paragraph after the glossary; Case 4's
// reduction modes; docc StreamK page):
//   K_DP         store the tile.
//   K_SPLITK     store the fp32 partial into P[s] of [S,M,N], arrive at the
//                tile's counter; the last arriver sums P[0..S-1] in split order
//                (its own split from registers) and stores C.
//   K_SK         a segment that covers the whole tile is stored; one that starts
//                mid-tile (always the unit's first) publishes its accumulator to
//                the unit's slot and raises the unit's flag; the unit holding the
//                tile's k = 0 iteration (its last segment) waits for the next
//                units in ascending k, adds each partial to its accumulator, and
//                stores the tile.
//   K_SK_ATOMIC  whole tiles are stored; every other segment atomically adds its
//                accumulator into C (zero-filled by the host first).
//
// Every wait is bounded by spin_limit polls; on expiry the status word records
// STATUS_TIMEOUT and the kernel goes on, so every wave always exits.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gemm.h"
#include "kernels.h"

namespace dgw {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = GEMM_BM, BN = GEMM_BN, BK = GEMM_BK;
constexpr int NT = 256;                       // threads per workgroup
constexpr int SLAB = BM * BK;                 // 16-bit values per operand slab (A and B alike)
constexpr int STAGE = 2 * SLAB;               // A slab then B slab
static_assert(BM == BN, "the LDS addressing below assumes square tiles");

struct Acc {
    f32x16 v[2][2];   // [i: 32-row block][j: 32-column block] of the wave's 64x64 quarter
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ u32x4 load16(const uint16_t *p, bool ok) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (ok) v = *reinterpret_cast<const u32x4 *>(p);
    return v;
}

template <int DT>
__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (DT == 0)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Global -> register staging of one k-iteration
// ---------------------------------------------------------------------------
// k-contiguous operand (A [M,K], or B [N,K]): thread t moves the 16-byte chunk
// (t & 7) of rows (t >> 3) + 32 i, i = 0..3.
struct RowStage {
    u32x4 r[4];
};

__device__ __forceinline__ void fetch_rows(RowStage &s, const uint16_t *X, int rows, int ld,
                                           int r0, int kb) {
    const int t = threadIdx.x;
    const int ch = t & 7;
    const int kc = kb + ch * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = r0 + (t >> 3) + 32 * i;
        const bool ok = row < rows && kc < ld;
        s.r[i] = load16(X + (size_t)row * ld + kc, ok);
    }
}

__device__ __forceinline__ void put_rows(const RowStage &s, uint16_t *slab) {
    const int t = threadIdx.x;
    const int ch = t & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = (t >> 3) + 32 * i;
        *reinterpret_cast<u32x4 *>(slab + row * BK + ((ch ^ swz(row)) << 3)) = s.r[i];
    }
}

// n-contiguous B [K,N]: thread t loads k-rows 4g..4g+3 (g = 2 (t>>5) + (t&1)) of
// the eight n-values of chunk c = (t>>1) & 15, and writes them transposed.
struct ColStage {
    u32x4 r[4];
};

__device__ __forceinline__ void fetch_cols(ColStage &s, const uint16_t *B, int K, int N, int n0,
                                           int kb) {
    const int t = threadIdx.x;
    const int g = ((t >> 5) << 1) | (t & 1);
    const int c = (t >> 1) & 15;
    const int n = n0 + c * 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int k = kb + 4 * g + r;
        s.r[r] = load16(B + (size_t)k * N + n, k < K && n < N);
    }
}

__device__ __forceinline__ void put_cols(const ColStage &s, uint16_t *slab) {
    const int t = threadIdx.x;
    const int gh = t >> 5;          // 8-value k chunk within the row
    const int h = t & 1;            // which 4-value half of that chunk
    const int c = (t >> 1) & 15;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int d = j >> 1;
        uint32_t lo, hi;
        if (j & 1) {
            lo = (s.r[0][d] >> 16) | (s.r[1][d] & 0xffff0000u);
            hi = (s.r[2][d] >> 16) | (s.r[3][d] & 0xffff0000u);
        } else {
            lo = (s.r[0][d] & 0xffffu) | (s.r[1][d] << 16);
            hi = (s.r[2][d] & 0xffffu) | (s.r[3][d] << 16);
        }
        const int n = c * 8 + j;
        u32x2 v = {lo, hi};
        *reinterpret_cast<u32x2 *>(slab + n * BK + ((gh ^ swz(n)) << 3) + h * 4) = v;
    }
}

// ---------------------------------------------------------------------------
// Matrix-core work on one staged slab pair
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void mma_stage(const uint16_t *stage, Acc &acc) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const uint16_t *As = stage;
    const uint16_t *Bs = stage + SLAB;
    const int ra0 = wm * 64 + (lane & 31), ra1 = ra0 + 32;
    const int rb0 = wn * 64 + (lane & 31), rb1 = rb0 + 32;
    const int hk = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
        const int ch = kk * 2 + hk;
        const u32x4 a0 = *reinterpret_cast<const u32x4 *>(As + ra0 * BK + ((ch ^ swz(ra0)) << 3));
        const u32x4 a1 = *reinterpret_cast<const u32x4 *>(As + ra1 * BK + ((ch ^ swz(ra1)) << 3));
        const u32x4 b0 = *reinterpret_cast<const u32x4 *>(Bs + rb0 * BK + ((ch ^ swz(rb0)) << 3));
        const u32x4 b1 = *reinterpret_cast<const u32x4 *>(Bs + rb1 * BK + ((ch ^ swz(rb1)) << 3));
        acc.v[0][0] = mfma<DT>(a0, b0, acc.v[0][0]);
        acc.v[0][1] = mfma<DT>(a0, b1, acc.v[0][1]);
        acc.v[1][0] = mfma<DT>(a1, b0, acc.v[1][0]);
        acc.v[1][1] = mfma<DT>(a1, b1, acc.v[1][1]);
    }
}

// acc += A[m0:m0+128, k0*64:k1*64] . B[k0*64:k1*64, n0:n0+128], k-iterations k0..k1-1.
// Ends with a barrier, so the LDS is free again on return.
template <int DT, int BL>
__device__ __forceinline__ void mac_loop(const KParams &p, uint16_t *lds, int m0, int n0, int k0,
                                         int k1, Acc &acc, int *cov) {
    RowStage sa;
    RowStage sb_rows;
    ColStage sb_cols;
    auto fetch = [&](int it) {
        const int kb = it * BK;
        fetch_rows(sa, p.A, p.M, p.K, m0, kb);
        if constexpr (BL == 1)
            fetch_rows(sb_rows, p.B, p.N, p.K, n0, kb);
        else
            fetch_cols(sb_cols, p.B, p.K, p.N, n0, kb);
    };
    auto put = [&](uint16_t *stage) {
        put_rows(sa, stage);
        if constexpr (BL == 1)
            put_rows(sb_rows, stage + SLAB);
        else
            put_cols(sb_cols, stage + SLAB);
    };
    fetch(k0);
    put(lds);
    __syncthreads();
    for (int it = k0; it < k1; ++it) {
        uint16_t *cur = lds + ((it - k0) & 1) * STAGE;
        uint16_t *nxt = lds + (((it - k0) & 1) ^ 1) * STAGE;
        const bool more = it + 1 < k1;
        if (more) fetch(it + 1);
        mma_stage<DT>(cur, acc);
        if (cov && threadIdx.x == 0) atomicAdd(cov + it, 1);
        if (more) put(nxt);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Epilogue helpers.  Accumulator element e of block (i, j) in lane l sits at
// row 32 i + 8 (e / 4) + 4 (l / 32) + e % 4 and column 32 j + l % 32 of the
// wave's quarter (output layout of the 32x32 MFMA).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void zero_acc(Acc &acc) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc.v[i][j][e] = 0.0f;
}

template <class F>
__device__ __forceinline__ void for_each_element(int m0, int n0, int M, int N, F &&f) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + wn * 64 + j * 32 + (lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                if (row < M && col < N) f(i, j, e, (size_t)row * N + col);
            }
        }
}

__device__ __forceinline__ void store_c(float *C, int m0, int n0, int M, int N, const Acc &acc) {
    for_each_element(m0, n0, M, N, [&](int i, int j, int e, size_t off) { C[off] = acc.v[i][j][e]; });
}

__device__ __forceinline__ void atomic_add_c(float *C, int m0, int n0, int M, int N, const Acc &acc) {
    for_each_element(m0, n0, M, N,
                     [&](int i, int j, int e, size_t off) { unsafeAtomicAdd(C + off, acc.v[i][j][e]); });
}

// Stream-K partial slot: register-native order, one float4 per lane per store,
// so every store/load instruction moves 1 KiB of contiguous memory.
__device__ __forceinline__ void put_slot(float *slot, const Acc &acc) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    f32x4 *s = reinterpret_cast<f32x4 *>(slot);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const f32x16 &v = acc.v[b >> 1][b & 1];
            f32x4 x = {v[4 * e4], v[4 * e4 + 1], v[4 * e4 + 2], v[4 * e4 + 3]};
            s[((wave * 4 + b) * 4 + e4) * 64 + lane] = x;
        }
}

__device__ __forceinline__ void add_slot(const float *slot, Acc &acc) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const f32x4 *s = reinterpret_cast<const f32x4 *>(slot);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const f32x4 x = s[((wave * 4 + b) * 4 + e4) * 64 + lane];
            f32x16 &v = acc.v[b >> 1][b & 1];
            v[4 * e4] += x[0];
            v[4 * e4 + 1] += x[1];
            v[4 * e4 + 2] += x[2];
            v[4 * e4 + 3] += x[3];
        }
}

// Poll `flag` until it holds `epoch` (one thread).  Gives up after `limit`
// polls, recording STATUS_TIMEOUT.
__device__ __forceinline__ void wait_flag(const uint32_t *flag, uint32_t epoch, uint32_t limit,
                                          uint32_t *status) {
    uint32_t polls = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
        if (++polls >= limit) {
            __hip_atomic_fetch_or(status, STATUS_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// Trace helpers (thread 0 only; active only when p.trace is set).
__device__ __forceinline__ int *trace_worker(const KParams &p, int w) {
    return p.trace + 8 + (size_t)w * (1 + 4 * p.trace_maxseg);
}
__device__ __forceinline__ int *trace_fold(const KParams &p, int tile) {
    return p.trace + 8 + (size_t)p.trace_workers * (1 + 4 * p.trace_maxseg) +
           (size_t)tile * (1 + p.trace_maxfold);
}
__device__ __forceinline__ int *trace_cov(const KParams &p, int tile) {
    return p.trace + 8 + (size_t)p.trace_workers * (1 + 4 * p.trace_maxseg) +
           (size_t)p.trace_tiles * (1 + p.trace_maxfold) + (size_t)tile * p.ipt;
}
__device__ __forceinline__ void trace_segment(const KParams &p, int w, int nseg, int tile, int k0,
                                              int k1, int role) {
    if (!p.trace || threadIdx.x != 0 || nseg >= p.trace_maxseg) return;
    int *rec = trace_worker(p, w);
    rec[1 + 4 * nseg + 0] = tile;
    rec[1 + 4 * nseg + 1] = k0;
    rec[1 + 4 * nseg + 2] = k1;
    rec[1 + 4 * nseg + 3] = role;
    rec[0] = nseg + 1;
}
__device__ __forceinline__ void trace_folded(const KParams &p, int tile, int pos, int w) {
    if (!p.trace || threadIdx.x != 0 || pos >= p.trace_maxfold) return;
    int *rec = trace_fold(p, tile);
    rec[1 + pos] = w;
    rec[0] = pos + 1;
}

// ---------------------------------------------------------------------------
// Data-parallel: one workgroup per tile of [tile_base, tile_base + ntiles).
// ---------------------------------------------------------------------------
template <int DT, int BL>
__global__ __launch_bounds__(NT, 2) void gemm_dp(KParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];
    const int w = p.perm ? p.perm[blockIdx.x] : (int)blockIdx.x;
    const int tile = p.tile_base + w;
    const int m0 = (tile / p.tiles_n) * BM, n0 = (tile % p.tiles_n) * BN;
    Acc acc;
    zero_acc(acc);
    mac_loop<DT, BL>(p, lds, m0, n0, 0, p.ipt, acc, p.trace ? trace_cov(p, tile) : nullptr);
    store_c(p.C, m0, n0, p.M, p.N, acc);
    trace_segment(p, p.worker_base + w, 0, tile, 0, p.ipt, 0);
    trace_folded(p, tile, 0, p.worker_base + w);
}

// ---------------------------------------------------------------------------
// Split-K: worker w = tile * S + s covers k-iterations [s P / S, (s+1) P / S).
// ---------------------------------------------------------------------------
template <int DT, int BL>
__global__ __launch_bounds__(NT, 2) void gemm_splitk(KParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];
    const int w = p.perm ? p.perm[blockIdx.x] : (int)blockIdx.x;
    const int S = p.splits;
    const int tile = w / S, s = w % S;
    const int k0 = (int)((int64_t)s * p.ipt / S), k1 = (int)((int64_t)(s + 1) * p.ipt / S);
    const int m0 = (tile / p.tiles_n) * BM, n0 = (tile % p.tiles_n) * BN;
    Acc acc;
    zero_acc(acc);
    mac_loop<DT, BL>(p, lds, m0, n0, k0, k1, acc, p.trace ? trace_cov(p, tile) : nullptr);
    trace_segment(p, w, 0, tile, k0, k1, S == 1 ? 0 : (s == 0 ? 1 : 2));
    if (S == 1) {
        store_c(p.C, m0, n0, p.M, p.N, acc);
        trace_folded(p, tile, 0, w);
        return;
    }
    const size_t mn = (size_t)p.M * p.N;
    store_c(p.part + (size_t)s * mn, m0, n0, p.M, p.N, acc);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    int *last = reinterpret_cast<int *>(lds);
    if (threadIdx.x == 0) {
        const uint32_t before =
            __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        const bool is_last = before == (uint32_t)(S - 1);
        if (is_last)
            __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *last = is_last ? 1 : 0;
    }
    __syncthreads();
    if (!*last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // Fold the S partials in split order: ((P0 + P1) + P2) + ...
    Acc sum;
    zero_acc(sum);
    for (int t = 0; t < S; ++t) {
        const float *P = p.part + (size_t)t * mn;
        for_each_element(m0, n0, p.M, p.N, [&](int i, int j, int e, size_t off) {
            const float x = (t == s) ? acc.v[i][j][e] : P[off];
            sum.v[i][j][e] = (t == 0) ? x : sum.v[i][j][e] + x;
        });
        trace_folded(p, tile, t, tile * S + t);
    }
    store_c(p.C, m0, n0, p.M, p.N, sum);
}

// ---------------------------------------------------------------------------
// Stream-K: persistent; workgroup b runs unit perm[b] (default b).
// ---------------------------------------------------------------------------
template <int DT, int BL, bool ATOMIC>
__global__ __launch_bounds__(NT, 1) void gemm_streamk(KParams p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];
    const int u = p.perm ? p.perm[blockIdx.x] : (int)blockIdx.x;
    const int ipt = p.ipt;
    const int begin = u * p.q + min(u, p.big);
    const int end = begin + p.q + (u < p.big ? 1 : 0);
    int nseg = 0;
    for (int pos = begin; pos < end;) {
        const int t = pos / ipt;                 // tile index within the Stream-K part
        const int tb = t * ipt;
        const int k0 = pos - tb;
        const int k1 = min(end - tb, ipt);
        const int tile = p.tile_base + t;
        const int m0 = (tile / p.tiles_n) * BM, n0 = (tile % p.tiles_n) * BN;
        const int role = k0 > 0 ? 2 : (k1 == ipt ? 0 : 1);
        Acc acc;
        zero_acc(acc);
        mac_loop<DT, BL>(p, lds, m0, n0, k0, k1, acc, p.trace ? trace_cov(p, tile) : nullptr);
        trace_segment(p, u, nseg++, tile, k0, k1, role);
        if (role == 0) {
            store_c(p.C, m0, n0, p.M, p.N, acc);
            trace_folded(p, tile, 0, u);
        } else if constexpr (ATOMIC) {
            atomic_add_c(p.C, m0, n0, p.M, p.N, acc);
        } else if (role == 2) {
            // starts mid-tile: publish the partial, then the flag
            put_slot(p.part + (size_t)u * (BM * BN), acc);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            __syncthreads();
            if (threadIdx.x == 0 && !(p.debug & GEMM_DEBUG_NO_PUBLISH))
                __hip_atomic_store(p.flags + u, p.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            // holds k = 0 of a split tile: fold the next units' partials in k order
            trace_folded(p, tile, 0, u);
            const int tile_end = tb + ipt;
            int pos_fold = 1;
            for (int v = u + 1; v < p.units; ++v) {
                if (v * p.q + min(v, p.big) >= tile_end) break;
                if (threadIdx.x == 0) wait_flag(p.flags + v, p.epoch, p.spin_limit, p.status);
                __syncthreads();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                add_slot(p.part + (size_t)v * (BM * BN), acc);
                trace_folded(p, tile, pos_fold++, v);
            }
            store_c(p.C, m0, n0, p.M, p.N, acc);
        }
        pos = tb + k1;
    }
}

// ---------------------------------------------------------------------------
// Zero fill (n 32-bit words), 16-byte stores where possible.
// ---------------------------------------------------------------------------
__global__ void zero_words(uint32_t *p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // words before the first 16-byte boundary
    const int64_t mis = (int64_t)((reinterpret_cast<uintptr_t>(p) & 15) / 4);
    int64_t head = mis ? 4 - mis : 0;
    if (head > n) head = n;
    for (int64_t i = tid; i < head; i += stride) p[i] = 0u;
    u32x4 *q = reinterpret_cast<u32x4 *>(p + head);
    const int64_t nv = (n - head) / 4;
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = tid; i < nv; i += stride) q[i] = z;
    for (int64_t i = head + nv * 4 + tid; i < n; i += stride) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
namespace {

typedef void (*KernelFn)(KParams);

template <int DT, int BL>
KernelFn pick(int kmode) {
    switch (kmode) {
    case K_DP: return gemm_dp<DT, BL>;
    case K_SPLITK: return gemm_splitk<DT, BL>;
    case K_SK: return gemm_streamk<DT, BL, false>;
    case K_SK_ATOMIC: return gemm_streamk<DT, BL, true>;
    default: return nullptr;
    }
}

KernelFn kernel_for(int dtype, int blayout, int kmode) {
    if (dtype == 0) return blayout == 0 ? pick<0, 0>(kmode) : pick<0, 1>(kmode);
    if (dtype == 1) return blayout == 0 ? pick<1, 0>(kmode) : pick<1, 1>(kmode);
    return nullptr;
}

}  // namespace

hipError_t launch_gemm(int dtype, int blayout, int kmode, int grid, const KParams &p,
                       hipStream_t stream) {
    KernelFn fn = kernel_for(dtype, blayout, kmode);
    if (!fn || grid <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_zero(void *ptr, int64_t n_words, hipStream_t stream) {
    if (n_words <= 0) return hipSuccess;
    int64_t blocks = (n_words / 4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(zero_words, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t *>(ptr), n_words);
    return hipGetLastError();
}

hipError_t blocks_per_cu(int dtype, int blayout, int kmode, int *out) {
    KernelFn fn = kernel_for(dtype, blayout, kmode);
    if (!fn) return hipErrorInvalidValue;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(out, reinterpret_cast<const void *>(fn), NT, 0);
}

}  // namespace dgw
