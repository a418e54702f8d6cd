// gemm_kernels.hip -- gfx950 (MI355X) kernels of the DP / Split-K / Stream-K GEMM.
//
// One mainloop serves every decomposition (large data-parallel launches use a
// second one for 2x2 tile groups, further down).  A workgroup computes one
// 128x128 fp32 output tile at a time; one "MAC-loop iteration" (Split-K/Stream-K book
// chapter, glossary) is a 64-wide step of K: the A slab [128 x 64] and the
// B slab [64 x 128] are staged in LDS and the workgroup issues 64
// v_mfma_f32_32x32x16_{bf16,f16} on them.  Every kernel runs eight waves (two
// per SIMD): waves w and w + 4 own the same 64x64 quarter of the tile and
// split each iteration's four 16-wide k-steps between them; after a segment
// they swap halves through LDS so that each holds the complete sums of one
// 32-row block of the quarter.
//
// Operands move global -> LDS with buffer_load ... lds (16 bytes per lane, no
// register round trip) into four LDS stages (A slabs of all stages first, then
// the B slabs, so every fragment read is a base register plus an immediate
// offset).  Iteration i waits for the loads of iteration i + 1, synchronises
// the workgroup once, issues the loads of iteration i + 4 into the stage just
// consumed, reads all fragments of iteration i + 1 into a second register set
// and issues the MFMAs of iteration i, which therefore never wait for LDS
// (CUTLASS optimisation guide, "Software Pipelining": multistage shared-memory
// pipeline plus register double buffering).  A [M,K] and B [N,K] rows are
// stored k-contiguous (128 bytes per row), 16-byte chunks XOR-swizzled by
// (r & 7) ^ ((r >> 3) & 3); B [K,N] is stored as k-rows of 128 n-values, chunk
// c of k-row r at c ^ nswz(r), and read with ds_read_b64_tr_b16, which hands
// every MFMA lane four consecutive k of one column.

// Epilogues (book chapter, Stream-K paragraph after the glossary; Case 4's
// reduction modes; docc StreamK page):
//   K_DP         store the tile.
//   K_DP_GROUP   store the four tiles of the group.
//   K_SPLITK     store the fp32 partial into P[s] of [batch][S,M,N]; then either arrive
//                at the tile's counter, the last arriver summing P[0..S-1] in
//                split order (its own split from LDS) and storing C, or leave
//                the sum to splitk_reduce (two-pass), or (atomic) add the
//                accumulator into a zero-filled C instead of storing a partial.
//   K_SK         a segment that covers the whole tile is stored; one that starts
//                mid-tile (always the unit's first) publishes its accumulator to
//                the unit's slot and raises the unit's flag; the unit holding the
//                tile's k = 0 iteration (its last segment) waits for the next
//                units in ascending k, adds each partial to its accumulator, and
//                stores the tile.  Two-pass: both kinds of split segment publish
//                (two slots per unit) and streamk_reduce adds them in k order.
//   K_SK_ATOMIC  whole tiles are stored; every other segment atomically adds its
//                accumulator into C (zero-filled by the host first).
// In a hybrid plan the Stream-K units first run the data-parallel tiles, whole
// K, before their Stream-K ranges.  Every final store can apply the fused
// epilogue act(alpha acc + beta C + bias) (CUTLASS optimisation guide,
// "Epilogue Optimization"); batched calls number their tiles entry after
// entry and each tile's kernel code addresses its entry's operands.
//
// Every wait is bounded by spin_limit polls; on expiry the status word records
// STATUS_TIMEOUT and the kernel goes on, so every wave always exits.
#include <hip/hip_runtime.h>

#include <algorithm>
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
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr int BM = GEMM_BM, BN = GEMM_BN, BK = GEMM_BK;

// Accumulators of one wave: its (TM / 2) x 64 part of a TM x 128 tile, as
// [i: 32-row block][j: 32-column block].
template <int TM>
struct AccT {
    f32x16 v[TM / 64][2];
};
using Acc = AccT<128>;

// Wave roles in a workgroup of NW waves.
template <int NW>
struct Role {
    static constexpr int NT = 64 * NW;              // threads
    int lane, wave, quad, wm, wn, kh;
    __device__ __forceinline__ Role() {
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        quad = wave & 3;
        wm = quad >> 1;
        wn = quad & 1;
        kh = wave >> 2;                             // which half of the k-steps (8 waves only)
    }
};

// A [M,K] and B [N,K] slabs in LDS: row r (64 values = 128 bytes = 8 chunks of
// 16 bytes) at r * 128, logical chunk c at physical chunk c ^ kswz(r).  Any 8
// consecutive rows read at one logical chunk then cover 8 distinct chunk
// positions, and 16 consecutive rows all 64 banks, so the 32-row fragment reads
// are conflict free; rows 32 apart share the swizzle, so a second 32-row block
// is a constant 4 KiB further.
__device__ __forceinline__ int kswz(int r) { return (r & 7) ^ ((r >> 3) & 3); }

// B [K,N] slabs: k-row r (128 n-values = 256 bytes = 16 chunks) at r * 256,
// chunk c at c ^ nswz(r).  The four k-rows read together by a 16-lane transpose
// read then fall on distinct banks; the swizzle depends on r % 4 only, so other
// k-steps and the second k-half of a fragment are constant offsets.
__device__ __forceinline__ int nswz(int r) { return ((r & 1) << 2) ^ ((r & 2) * 5); }

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
// Operand staging: buffer loads straight into LDS
// ---------------------------------------------------------------------------
// Each buffer_load ... lds instruction moves 16 bytes per lane into LDS at
// (wave-uniform base) + 16 * lane, i.e. 1 KiB of contiguous LDS per wave; the
// swizzle is applied by choosing which global 16-byte chunk each lane fetches.
// Loads whose address falls outside the buffer's range return zero, which
// masks ragged M/N edges; a ragged K tail is masked by pointing the lane at an
// offset beyond the range.
constexpr uint32_t OOB = 0x7ffffff0u;        // an offset outside every buffer range used here
constexpr uint32_t RSRC_DW3 = 0x00020000u;    // raw buffer, 32-bit data format
// Cache policy of the final C stores: non-temporal.  C is written once and not
// read again by the call, so it should not displace the A and B panels that
// neighbouring tiles still read from L2 (measured: 8192^3 2.8 %, the
// 2048x2176x4096 Stream-K call 1.5 % faster).
constexpr int CPOL_NT = 2;

__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = (int)RSRC_DW3;
    return r;
}

// Issued as inline assembly so that the compiler does not wait for it before
// unrelated LDS reads; completion is awaited explicitly (wait_vm_lgkm).
// `lds_addr` is the wave-uniform LDS byte address of the 1 KiB destination.
// The s_nop is the one wait state a GFX9 LDS DMA needs after an SALU write of
// M0 (the compiler cannot insert it inside the asm block).
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc)
                 : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding
// and all of its LDS reads have returned.
// s_waitcnt on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
template <int N>
__device__ __forceinline__ void wait_vm_lgkm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// The same with N known only at run time (0 <= n <= 3 stages' worth).
template <int DPI>
__device__ __forceinline__ void wait_vm_lgkm_stages(int stages) {
    switch (stages) {
    case 3: wait_vm_lgkm<3 * DPI>(); break;
    case 2: wait_vm_lgkm<2 * DPI>(); break;
    case 1: wait_vm_lgkm<1 * DPI>(); break;
    default: wait_vm_lgkm<0>(); break;
    }
}
__device__ __forceinline__ void wait_stage0() {
    wait_vm_lgkm<0>();
    __builtin_amdgcn_s_barrier();
}

// A device-scope (sc1) load of a 32-bit flag that the compiler does not track
// (it is awaited by an explicit vmcnt wait; measured cheaper to poll with than
// an atomic load).  flag_value() must only be applied after such a wait has
// covered the load.
__device__ __forceinline__ uint32_t load_flag_async(const uint32_t *flag) {
    uint32_t v;
    asm volatile("global_load_dword %0, %1, off sc1" : "=v"(v) : "v"(flag) : "memory");
    return v;
}
__device__ __forceinline__ uint32_t flag_value(uint32_t v) {
    asm volatile("" : "+v"(v));   // keeps every use of v after the preceding wait
    return v;
}

template <int OFF>
__device__ __forceinline__ u32x4 lds_b128(uint32_t addr) {
    return *reinterpret_cast<const lds_u32x4 *>(static_cast<uintptr_t>(addr + OFF));
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_tr16(uint32_t addr) {
    return __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4i16 *>(static_cast<uintptr_t>(addr + OFF))));
}

// ---------------------------------------------------------------------------
// The mainloop.  One "MAC-loop iteration" is a 64-wide step of K: the A slab
// [128 x 64] and B slab [64 x 128] of the iteration are in LDS stage i % NS
// (A slabs of all stages in [0, NS * 16 KiB), B slabs after them, so every
// fragment read is a base register plus an immediate), and each wave issues
// 4 * KSW MFMAs on them: its 64x64 quarter over KSW of the iteration's four
// 16-wide k-steps.
//
// Iteration i, per wave: wait until its own loads of iteration i + 1 landed and
// its fragment reads of iteration i returned; barrier (every wave's loads of
// i + 1 landed, every wave finished reading stage i); issue the loads of
// iteration i + NS into stage i; read all fragments of iteration i + 1 into the
// other register buffer; issue the MFMAs of iteration i.  The MFMAs never wait
// for LDS, and the fragment reads have a whole iteration to return.
// ---------------------------------------------------------------------------
constexpr int SLAB_BYTES = BM * BK * 2;   // 16 KiB: a B slab, or the A slab of a 128-row tile

// Tile of TM x 128 (TM = 128; 256 for the tall Stream-K tile; 64 for the
// skinny tile, with 4 waves): the A slab is TM x 64, the B slab 64 x 128; each
// wave owns (TM / 2) x 64, i.e. RB 32-row blocks by two 32-column blocks.
template <int TM>
constexpr int aslab_bytes() { return TM * BK * 2; }
template <int TM>
constexpr int lds_bytes(int ns) { return ns * (aslab_bytes<TM>() + SLAB_BYTES); }

template <int DT, int BL, int NS, int NW, int TM = 128>
struct MainLoop {
    static constexpr int KSW = 16 / NW;          // k-steps per wave and iteration
    static constexpr int RB = TM / 64;           // 32-row blocks per wave
    static constexpr int ASLAB = aslab_bytes<TM>();
    static constexpr int DPWA = TM / 8 / NW;     // loads per wave of the A slab (1 KiB each)
    static constexpr int DPWB = 16 / NW;         // loads per wave of the B slab
    static constexpr int DPI = DPWA + DPWB;      // loads per wave and iteration
    static constexpr int BREG = NS * ASLAB;      // start of the B slabs
    static_assert(TM == 64 || TM == 128 || TM == 256, "64-, 128- or 256-row tiles");
    static_assert(TM != 64 || NW == 4, "the 64-row tile runs four waves (no k-halves to merge)");
    static_assert(NS >= 3 && NS <= 4, "three or four stages");
    static_assert(NW == 4 || NW == 8, "four or eight waves");

    const KParams &p;
    uint32_t lds0;
    int lane, wave, kh;
    // fragment read addresses (stage 0): A block 0 per k-step of the wave;
    // B [N,K]: block 0 per k-step; B [K,N]: column block jb at the wave's first k-step
    uint32_t aoff[KSW], boff[KSW > 2 ? KSW : 2];
    // per-lane global byte offsets of the wave's loads at k-slab 0
    uint32_t adma[DPWA], bdma[DPWB];
    int a_kc[DPWA], b_kc[DPWB];   // first k of the lane's chunk / B [K,N]: k-row of the lane
    const char *a_base, *b_base;
    uint32_t a_rows_bytes, b_rows_bytes;

    __device__ __forceinline__ MainLoop(const KParams &p_, char *lds, int m0, int n0) : p(p_) {
        lds0 = (uint32_t)reinterpret_cast<uintptr_t>((const lds_void *)lds);
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        const int quad = wave & 3, wm = quad >> 1, wn = quad & 1;
        kh = wave >> 2;
        const int K = p.K, N = p.N;
        const int r32 = lane & 31, hk = lane >> 5;
#pragma unroll
        for (int j = 0; j < KSW; ++j) {
            const int kk = kh * KSW + j;
            const uint32_t rowpart = (uint32_t)(r32 * 128 + ((((2 * kk + hk) ^ kswz(r32)) & 7) << 4));
            aoff[j] = lds0 + wm * (TM / 2) * 128 + rowpart;
            if constexpr (BL == 1) boff[j] = lds0 + BREG + wn * 8192 + rowpart;
        }
        if constexpr (BL == 0) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const int n = wn * 64 + jb * 32 + ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
                const int r = kh * KSW * 16 + 8 * hk + ((lane & 15) >> 2);
                boff[jb] = lds0 + BREG + r * 256 + ((((n >> 3) ^ nswz(r)) & 15) << 4) + ((n & 7) << 1);
            }
        }
        a_base = reinterpret_cast<const char *>(p.A) + (size_t)m0 * K * 2;
        a_rows_bytes = (uint32_t)(min(TM, p.M - m0) * K * 2);
#pragma unroll
        for (int x = 0; x < DPWA; ++x) {
            const int r = 8 * (wave * DPWA + x) + (lane >> 3);
            const int c = (lane & 7) ^ kswz(r);
            adma[x] = (uint32_t)(r * K + 8 * c) * 2;
            a_kc[x] = 8 * c;
        }
#pragma unroll
        for (int x = 0; x < DPWB; ++x) {
            if constexpr (BL == 1) {
                const int r = 8 * (wave * DPWB + x) + (lane >> 3);
                const int c = (lane & 7) ^ kswz(r);
                bdma[x] = (uint32_t)(r * K + 8 * c) * 2;
                b_kc[x] = 8 * c;
            } else {
                const int rb = 4 * (wave * DPWB + x) + (lane >> 4);
                const int cb = (lane & 15) ^ nswz(rb);
                // chunks beyond N (last tile column only) always read zeros
                bdma[x] = n0 + 8 * cb >= N ? OOB : (uint32_t)(rb * N + 8 * cb) * 2;
                b_kc[x] = rb;
            }
        }
        if constexpr (BL == 1) {
            b_base = reinterpret_cast<const char *>(p.B) + (size_t)n0 * K * 2;
            b_rows_bytes = (uint32_t)(min(BN, N - n0) * K * 2);
        } else {
            b_base = reinterpret_cast<const char *>(p.B) + (size_t)n0 * 2;
            b_rows_bytes = 0;
        }
    }

    // Loads of physical K-slab `slab` into stage `st`.  RAGGED (K not a multiple
    // of 64): lanes whose chunk starts at or beyond K read zeros.
    template <bool RAGGED>
    __device__ __forceinline__ void issue(int slab, int st) const {
        const int kb = slab * BK;
        const i32x4 ra = make_rsrc(a_base + (size_t)kb * 2, a_rows_bytes - kb * 2);
        i32x4 rb;
        int krows = BK;
        if constexpr (BL == 1) {
            rb = make_rsrc(b_base + (size_t)kb * 2, b_rows_bytes - kb * 2);
        } else {
            krows = min(BK, p.K - kb);   // k-rows beyond K fall outside the range
            rb = make_rsrc(b_base + (size_t)kb * p.N * 2, (uint32_t)(krows * p.N * 2));
        }
        const uint32_t a_dst = lds0 + st * ASLAB + wave * DPWA * 1024;
        const uint32_t b_dst = lds0 + BREG + st * SLAB_BYTES + wave * DPWB * 1024;
#pragma unroll
        for (int x = 0; x < DPWA; ++x) dma16(ra, a_dst + x * 1024, !RAGGED || kb + a_kc[x] < p.K ? adma[x] : OOB);
#pragma unroll
        for (int x = 0; x < DPWB; ++x) {
            uint32_t off = bdma[x];
            if constexpr (RAGGED && BL == 1) off = kb + b_kc[x] < p.K ? off : OOB;
            dma16(rb, b_dst + x * 1024, off);
        }
    }

    struct Frags {
        u32x4 a[KSW][RB];  // [k-step][32-row block]
        u32x4 b[KSW][2];   // [k-step][32-column block]
    };

    template <int ST>
    __device__ __forceinline__ void read(Frags &f) const {
        // A fragment offsets are immediates of at most 64 KiB: a stage that lies
        // beyond moves 48 KiB of its offset into the base address
        constexpr int AO = ST * ASLAB;
        constexpr int AHI = AO + (RB - 1) * 4096 >= 65536 ? 49152 : 0;
#pragma unroll
        for (int j = 0; j < KSW; ++j) {
            const uint32_t abase = aoff[j] + AHI;
            auto row_block = [&](auto RBC) {
                constexpr int rb = decltype(RBC)::value;
                f.a[j][rb] = lds_b128<AO - AHI + rb * 4096>(abase);
            };
            row_block(std::integral_constant<int, 0>());
            if constexpr (RB > 1) row_block(std::integral_constant<int, 1>());
            if constexpr (RB > 2) {
                row_block(std::integral_constant<int, 2>());
                row_block(std::integral_constant<int, 3>());
            }
            if constexpr (BL == 1) {
                f.b[j][0] = lds_b128<ST * SLAB_BYTES>(boff[j]);
                f.b[j][1] = lds_b128<ST * SLAB_BYTES + 4096>(boff[j]);
            }
        }
        if constexpr (BL == 0) {
#pragma unroll
            for (int j = 0; j < KSW; ++j)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const u32x2 h0 = lds_tr16<ST * SLAB_BYTES>(boff[jb] + j * 4096);
                    const u32x2 h1 = lds_tr16<ST * SLAB_BYTES + 1024>(boff[jb] + j * 4096);
                    f.b[j][jb] = u32x4{h0[0], h0[1], h1[0], h1[1]};
                }
        }
    }

    // One k-step's fragments (the tall tile's loop double-buffers per k-step:
    // a whole iteration's fragments next to its 128 accumulator registers would
    // not fit two waves per SIMD).
    struct StepFrags {
        u32x4 a[RB];
        u32x4 b[2];
    };

    // Fragments of the wave's k-step J (0 .. KSW - 1) of stage ST.
    template <int ST, int J>
    __device__ __forceinline__ void read_step(StepFrags &f) const {
        constexpr int AO = ST * ASLAB;
        constexpr int AHI = AO + (RB - 1) * 4096 >= 65536 ? 49152 : 0;
        const uint32_t abase = aoff[J] + AHI;
        auto row_block = [&](auto RBC) {
            constexpr int rb = decltype(RBC)::value;
            f.a[rb] = lds_b128<AO - AHI + rb * 4096>(abase);
        };
        row_block(std::integral_constant<int, 0>());
        if constexpr (RB > 1) row_block(std::integral_constant<int, 1>());
        if constexpr (RB > 2) {
            row_block(std::integral_constant<int, 2>());
            row_block(std::integral_constant<int, 3>());
        }
        if constexpr (BL == 1) {
            f.b[0] = lds_b128<ST * SLAB_BYTES>(boff[J]);
            f.b[1] = lds_b128<ST * SLAB_BYTES + 4096>(boff[J]);
        } else {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const u32x2 h0 = lds_tr16<ST * SLAB_BYTES + J * 4096>(boff[jb]);
                const u32x2 h1 = lds_tr16<ST * SLAB_BYTES + J * 4096 + 1024>(boff[jb]);
                f.b[jb] = u32x4{h0[0], h0[1], h1[0], h1[1]};
            }
        }
    }

    static __device__ __forceinline__ void mma_step(const StepFrags &f, AccT<TM> &acc) {
#pragma unroll
        for (int a = 0; a < RB; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc.v[a][b] = mfma<DT>(f.a[a], f.b[b], acc.v[a][b]);
    }

    static __device__ __forceinline__ void mma(const Frags &f, AccT<TM> &acc) {
#pragma unroll
        for (int j = 0; j < KSW; ++j)
#pragma unroll
            for (int a = 0; a < RB; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc.v[a][b] = mfma<DT>(f.a[j][a], f.b[j][b], acc.v[a][b]);
    }
};

// acc += A[m0:m0+128, K-slabs] . B[K-slabs, n0:n0+128] over the tile's MAC
// iterations k0..k1-1, iteration k reading the 64-wide K-slab (k + rot) mod ipt
// (rot = 0 maps iteration k to slab k; the caller uses one rot per tile, so the
// iterations of all of a tile's segments still cover every slab exactly once).
// With 8 waves each wave covers half of every slab's k-steps and holds a
// partial sum of its quarter (see merge_k_halves).  Ends with a barrier, so the
// LDS is free again on return.  `probe` (optional): a flag every lane loads
// once the first iteration's operands have landed, into `probe_val` (complete
// on return; unchanged when the segment is empty).
template <int DT, int BL, int NS, int NW, int TM, bool RAGGED>
__device__ __forceinline__ void mac_loop_impl(const KParams &p, char *lds, int m0, int n0, int k0, int k1,
                                              int rot, AccT<TM> &acc, int *cov, uint32_t *raise,
                                              const uint32_t *probe = nullptr, uint32_t *probe_val = nullptr) {
    using ML = MainLoop<DT, BL, NS, NW, TM>;
    constexpr int DPI = ML::DPI;
    const int n = k1 - k0;
    if (n <= 0) return;
    const ML ml(p, lds, m0, n0);
    const int ipt = p.ipt;
    int phys = k0 + rot;                       // physical slab of the next load
    phys = phys >= ipt ? phys - ipt : phys;
    phys = phys >= ipt ? phys - ipt : phys;
    auto issue_next = [&](int st) {
        ml.template issue<RAGGED>(phys, st);
        phys = phys + 1 == ipt ? 0 : phys + 1;
    };
    typename ML::Frags f[2];
    issue_next(0);
    if (n > 1) issue_next(1);
    if (n > 2) issue_next(2);
    if (NS > 3 && n > 3) issue_next(3);
    wait_vm_lgkm_stages<DPI>(min(NS, n) - 1);   // this wave's loads of iteration 0 landed
    __builtin_amdgcn_s_barrier();
    // A partial published just before this loop: its stores were issued before
    // the loads waited for above, and completion is reported in issue order, so
    // in every wave they are complete (the barrier covers all waves) and the
    // flag may rise.
    if (raise && threadIdx.x == 0) __hip_atomic_store(raise, p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // issued after the prologue's loads, so no wait of the loop waits for it
    // before those (completion is reported in issue order)
    if (probe) *probe_val = load_flag_async(probe);
    ml.template read<0>(f[0]);
    int done = 0;                              // iterations issued to the matrix cores
    // One iteration i: its stage U = i % NS, its register buffer P = i % 2.
    auto body = [&](int i, auto U, auto P, auto STEADY) {
        constexpr int u = decltype(U)::value;
        constexpr int par = decltype(P)::value;
        constexpr bool steady = decltype(STEADY)::value;
        if constexpr (steady) wait_vm_lgkm<(NS - 2) * DPI>();
        else wait_vm_lgkm_stages<DPI>(max(0, min(NS - 2, n - i - 2)));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (steady || i + NS < n) issue_next(u);
        if (steady || i + 1 < n) ml.template read<(u + 1) % NS>(f[par ^ 1]);
        ML::mma(f[par], acc);
        __builtin_amdgcn_sched_barrier(0);
        ++done;
    };
    // the loop body is unrolled over L = lcm(NS, 2) iterations, so that both the
    // stage and the register buffer of every iteration are compile-time constants
    constexpr int L = NS % 2 == 0 ? NS : 2 * NS;
    using T = std::true_type;
    using F = std::false_type;
    auto group = [&](int i0, auto STEADY) {
        using ST = decltype(STEADY);
        body(i0 + 0, std::integral_constant<int, 0 % NS>(), std::integral_constant<int, 0>(), ST());
        if (ST::value || i0 + 1 < n) body(i0 + 1, std::integral_constant<int, 1 % NS>(), std::integral_constant<int, 1>(), ST());
        if (ST::value || i0 + 2 < n) body(i0 + 2, std::integral_constant<int, 2 % NS>(), std::integral_constant<int, 0>(), ST());
        if (ST::value || i0 + 3 < n) body(i0 + 3, std::integral_constant<int, 3 % NS>(), std::integral_constant<int, 1>(), ST());
        if constexpr (L == 6) {
            if (ST::value || i0 + 4 < n) body(i0 + 4, std::integral_constant<int, 4 % NS>(), std::integral_constant<int, 0>(), ST());
            if (ST::value || i0 + 5 < n) body(i0 + 5, std::integral_constant<int, 5 % NS>(), std::integral_constant<int, 1>(), ST());
        }
    };
    int i0 = 0;
    for (; i0 + L + NS <= n; i0 += L) group(i0, T());
    for (; i0 < n; i0 += L) group(i0, F());
    wait_stage0();
    // debug coverage: one count per logical iteration the loop above executed
    if (cov && threadIdx.x == 0)
        for (int k = 0; k < done; ++k) atomicAdd(cov + k0 + k, 1);
}

// The same iterations for the 256 x 128 tile, fragments double-buffered per
// k-step.  Iteration i on stage U = i % NS, the wave's k-step 0 already in F0:
// read k-step 1 into F1 and multiply F0; then (unless i is the last) wait for
// this wave's loads of i + 1 and its reads of F1, barrier (every wave's loads
// of i + 1 landed, every wave done reading stage U), read k-step 0 of i + 1
// into F0 and issue the loads of i + NS into stage U; multiply F1.
template <int DT, int BL, int NS, int NW, bool RAGGED>
__device__ __forceinline__ void mac_loop_tall_impl(const KParams &p, char *lds, int m0, int n0, int k0, int k1,
                                                   int rot, AccT<256> &acc, int *cov, uint32_t *raise) {
    using ML = MainLoop<DT, BL, NS, NW, 256>;
    static_assert(ML::KSW == 2, "two k-steps per wave and iteration");
    constexpr int DPI = ML::DPI;
    const int n = k1 - k0;
    if (n <= 0) return;
    const ML ml(p, lds, m0, n0);
    const int ipt = p.ipt;
    int phys = k0 + rot;                       // physical slab of the next load
    phys = phys >= ipt ? phys - ipt : phys;
    phys = phys >= ipt ? phys - ipt : phys;
    auto issue_next = [&](int st) {
        ml.template issue<RAGGED>(phys, st);
        phys = phys + 1 == ipt ? 0 : phys + 1;
    };
    typename ML::StepFrags f0, f1;
    issue_next(0);
    if (n > 1) issue_next(1);
    if (n > 2) issue_next(2);
    if (NS > 3 && n > 3) issue_next(3);
    wait_vm_lgkm_stages<DPI>(min(NS, n) - 1);   // this wave's loads of iteration 0 landed
    __builtin_amdgcn_s_barrier();
    // a partial published just before this loop: see mac_loop_impl
    if (raise && threadIdx.x == 0) __hip_atomic_store(raise, p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ml.template read_step<0, 0>(f0);
    int done = 0;
    auto iter = [&](int i, auto U, auto STEADY) {
        constexpr int u = decltype(U)::value;
        constexpr bool steady = decltype(STEADY)::value;
        __builtin_amdgcn_sched_barrier(0);
        ml.template read_step<u, 1>(f1);
        ML::mma_step(f0, acc);
        __builtin_amdgcn_sched_barrier(0);
        if (steady || i + 1 < n) {
            if constexpr (steady) wait_vm_lgkm<(NS - 2) * DPI>();
            else wait_vm_lgkm_stages<DPI>(max(0, min(NS - 2, n - i - 2)));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            ml.template read_step<(u + 1) % NS, 0>(f0);
            if (steady || i + NS < n) issue_next(u);
        }
        ML::mma_step(f1, acc);
        __builtin_amdgcn_sched_barrier(0);
        ++done;
    };
    auto group = [&](int i0, auto STEADY) {
        using ST = decltype(STEADY);
        iter(i0 + 0, std::integral_constant<int, 0>(), ST());
        if (ST::value || i0 + 1 < n) iter(i0 + 1, std::integral_constant<int, 1 % NS>(), ST());
        if (ST::value || i0 + 2 < n) iter(i0 + 2, std::integral_constant<int, 2 % NS>(), ST());
        if constexpr (NS == 4)
            if (ST::value || i0 + 3 < n) iter(i0 + 3, std::integral_constant<int, 3>(), ST());
    };
    int i0 = 0;
    for (; i0 + 2 * NS <= n; i0 += NS) group(i0, std::true_type());
    for (; i0 < n; i0 += NS) group(i0, std::false_type());
    wait_stage0();
    if (cov && threadIdx.x == 0)
        for (int k = 0; k < done; ++k) atomicAdd(cov + k0 + k, 1);
}

// `raise` (optional): a flag to set to p.epoch once this workgroup's earlier
// global stores are complete (the loop's first wait establishes that).
// `probe` / `probe_val` (64- and 128-row tiles only): see mac_loop_impl.
template <int DT, int BL, int NS, int NW, int TM = 128>
__device__ __forceinline__ void mac_loop(const KParams &p, char *lds, int m0, int n0, int k0, int k1,
                                         int rot, AccT<TM> &acc, int *cov, uint32_t *raise = nullptr,
                                         const uint32_t *probe = nullptr, uint32_t *probe_val = nullptr) {
    if constexpr (TM == 256) {
        if (p.K % BK == 0) mac_loop_tall_impl<DT, BL, NS, NW, false>(p, lds, m0, n0, k0, k1, rot, acc, cov, raise);
        else mac_loop_tall_impl<DT, BL, NS, NW, true>(p, lds, m0, n0, k0, k1, rot, acc, cov, raise);
    } else {
        if (p.K % BK == 0)
            mac_loop_impl<DT, BL, NS, NW, TM, false>(p, lds, m0, n0, k0, k1, rot, acc, cov, raise, probe, probe_val);
        else
            mac_loop_impl<DT, BL, NS, NW, TM, true>(p, lds, m0, n0, k0, k1, rot, acc, cov, raise, probe, probe_val);
    }
}

// With 8 waves the two waves of a quadrant (k-halves 0 and 1) each hold a
// partial sum of the whole (TM / 2) x 64 part of the tile.  They swap halves
// through LDS: of its RB 32-row blocks, wave (quad, kh) keeps blocks
// kh R .. kh R + R - 1 (R = RB / 2), sends the others to its partner and adds
// the partner's copies of the kept ones, so afterwards it holds the complete
// sums of R block rows (fp32 addition is commutative, so both waves' blocks
// are exactly acc(kh 0) + acc(kh 1)).  With 4 waves every wave already holds
// all its block rows.  The result names its block rows at run time but keeps
// the values in fixed registers (the accumulator is only ever indexed by
// constants, so it stays in registers).  `lds` must be free (TM / 2 KiB per
// wave); it is free on return.
template <int NW, int TM = 128>
struct Tile {
    static constexpr int RB = TM / 64;              // 32-row blocks of a wave's part
    static constexpr int R = NW == 8 ? RB / 2 : RB; // block rows a wave holds
    f32x16 v[R][2];                                 // [held row][32-column block]
    int i[R];                                       // which 32-row block of the wave's part
};

// The block row merge_k_halves leaves in slot r of a wave's Tile.
template <int NW, int TM>
__device__ __forceinline__ int held_row(int r) {
    return NW == 8 ? Role<NW>().kh * Tile<NW, TM>::R + r : r;
}

template <int NW, int TM = 128>
__device__ __forceinline__ Tile<NW, TM> merge_k_halves(const AccT<TM> &acc, char *lds) {
    Tile<NW, TM> t;
    constexpr int R = Tile<NW, TM>::R;
    if constexpr (NW == 8) {
        const Role<NW> w;
        const bool hi = w.kh != 0;
        f32x4 *buf = reinterpret_cast<f32x4 *>(lds);
        // wave (quad, kh) writes R x 2 blocks of 16 floats per lane at slot
        // ((quad * 2 + kh) * R * 8 + (r * 2 + j) * 4 + e4) * 64 + lane
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const f32x16 give = hi ? acc.v[r][j] : acc.v[R + r][j];
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4)
                    buf[((w.quad * 2 + w.kh) * R * 8 + (r * 2 + j) * 4 + e4) * 64 + w.lane] =
                        f32x4{give[4 * e4], give[4 * e4 + 1], give[4 * e4 + 2], give[4 * e4 + 3]};
            }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x16 keep = hi ? acc.v[R + r][j] : acc.v[r][j];
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const f32x4 x = buf[((w.quad * 2 + (1 - w.kh)) * R * 8 + (r * 2 + j) * 4 + e4) * 64 + w.lane];
                    keep[4 * e4] += x[0];
                    keep[4 * e4 + 1] += x[1];
                    keep[4 * e4 + 2] += x[2];
                    keep[4 * e4 + 3] += x[3];
                }
                t.v[r][j] = keep;
            }
            t.i[r] = held_row<NW, TM>(r);
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            t.v[r][0] = acc.v[r][0];
            t.v[r][1] = acc.v[r][1];
            t.i[r] = held_row<NW, TM>(r);
        }
    }
    return t;
}

// ---------------------------------------------------------------------------
// Work placement.  Workgroup b runs on XCD b % 8; `spread` gives every XCD a
// contiguous range of workers so that neighbouring tiles share an L2.  Tiles
// are numbered in groups of `group_m` tile rows, column by column inside a
// group, so a contiguous range of tile ids is a compact 2-D block.
// ---------------------------------------------------------------------------
// floor(n / d) for 0 <= n < 2^31 (FastDiv in fastdiv.h).
__device__ __forceinline__ int fdiv(int n, FastDiv d) {
    return (int)((__umulhi((uint32_t)n, d.m) + (uint32_t)n) >> d.s);
}

// First flattened iteration of Stream-K unit u (the first `big` units own q + 1).
__device__ __forceinline__ int unit_start(int u, int q, int big) { return u * q + min(u, big); }

// The unit whose range contains flattened iteration g (q >= 1, or g < big).
__device__ __forceinline__ int unit_of(const KParams &p, int g) {
    const int long_part = p.big * (p.q + 1);
    return g < long_part ? fdiv(g, p.d_q1) : p.big + fdiv(g - long_part, p.d_q);
}

// The worker workgroup b runs: unit_perm's entry, or with XCD spreading the
// b / 8-th worker of XCD b % 8's contiguous range (XCD x holds n / 8 workers,
// one more for x < n % 8, after those of the XCDs before it), or b.  The same
// value in every lane.
__device__ __forceinline__ int worker_of(const KParams &p) {
    const int b = (int)blockIdx.x;
    if (p.perm) return __builtin_amdgcn_readfirstlane(p.perm[b]);
    if (!p.xcd_spread) return b;
    const int x = b & 7;
    return x * p.spread_a + min(x, p.spread_r) + (b >> 3);
}

// Origin of tile `tile` of one batch entry's tile grid, by the launch's
// division constants.
__device__ __forceinline__ void tile_origin_fast(const KParams &p, int tile, int &m0, int &n0) {
    const int gm_full = p.group_m > 0 ? p.group_m : p.tiles_m;
    const int g = fdiv(tile, p.d_band);
    const int first = g * gm_full;
    const bool last = p.tiles_m - first < gm_full;
    const int gm = last ? p.tiles_m - first : gm_full;
    const int w = tile - g * gm_full * p.tiles_n;
    const int col = fdiv(w, last ? p.d_rows_last : p.d_rows);
    m0 = (first + w - col * gm) * p.tm;
    n0 = col * BN;
}

// The same for any tile grid (a grouped call's problems have grids of their own).
__device__ __forceinline__ void tile_origin(const KParams &p, int tile, int &m0, int &n0) {
    const int gm_full = p.group_m > 0 ? p.group_m : p.tiles_m;
    const int per_group = gm_full * p.tiles_n;
    const int g = tile / per_group;
    const int first = g * gm_full;
    const int gm = min(gm_full, p.tiles_m - first);
    const int w = tile - g * per_group;
    m0 = (first + w % gm) * p.tm;
    n0 = (w / gm) * BN;
}

// A copy of p whose A, B, C (and Split-K partials) point at batch entry b.
__device__ __forceinline__ KParams batch_entry(const KParams &p, int b) {
    KParams q = p;
    q.A += (size_t)b * p.sA;
    q.B += (size_t)b * p.sB;
    q.C += (size_t)b * p.sC;
    q.part += (size_t)b * p.sP;
    return q;
}

// Grouped call: the problem holding global tile `tile` (the nonempty problems'
// first tile ids ascend; lane l compares problem l's, so one vector load and a
// ballot find it), and the view of it.
__device__ __forceinline__ KParams group_view(const KParams &p, int tile, int &m0, int &n0) {
    const int lane = threadIdx.x & 63;
    const int t0 = lane < p.ngroups ? p.groups[lane].tile0 : 0x7fffffff;
    const uint64_t below = __ballot(t0 <= tile);
    const int g = __builtin_amdgcn_readfirstlane(63 - __builtin_clzll(below));
    const GroupDesc &d = p.groups[g];
    KParams q = p;
    q.A = d.A;
    q.B = d.B;
    q.C = d.C;
    q.part = p.part ? p.part + d.part : nullptr;
    q.M = d.M;
    q.N = d.N;
    q.tiles_m = (d.M + p.tm - 1) / p.tm;
    q.tiles_n = (d.N + BN - 1) / BN;
    tile_origin(q, tile - d.tile0, m0, n0);
    return q;
}

// Tiles are numbered batch after batch (or problem after problem in a grouped
// call, the GRP builds): the view of global tile `tile`'s batch entry and the
// tile's origin in it.
template <bool GRP = false>
__device__ __forceinline__ KParams tile_view(const KParams &p, int tile, int &m0, int &n0) {
    if constexpr (GRP) return group_view(p, tile, m0, n0);
    if (p.batch <= 1) {
        tile_origin_fast(p, tile, m0, n0);
        return p;
    }
    const int b = fdiv(tile, p.d_entry);
    tile_origin_fast(p, tile - b * p.tiles_m * p.tiles_n, m0, n0);
    return batch_entry(p, b);
}

// ---------------------------------------------------------------------------
// Epilogue helpers.  Accumulator element e of block (i, j) in lane l sits at
// row 32 i + 8 (e / 4) + 4 (l / 32) + e % 4 and column 32 j + l % 32 of the
// wave's quarter (output layout of the 32x32 MFMA).  After merge_k_halves each
// wave touches only the block rows it owns.
// ---------------------------------------------------------------------------
template <int TM>
__device__ __forceinline__ void zero_acc(AccT<TM> &acc) {
#pragma unroll
    for (int i = 0; i < TM / 64; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc.v[i][j][e] = 0.0f;
}

template <int NW, int TM, class F>
__device__ __forceinline__ void for_each_element(const Tile<NW, TM> &t, int m0, int n0, int M, int N, F &&f) {
    const Role<NW> w;
#pragma unroll
    for (int r = 0; r < Tile<NW, TM>::R; ++r)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = n0 + w.wn * 64 + j * 32 + (w.lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + w.wm * (TM / 2) + t.i[r] * 32 + 8 * (e >> 2) + 4 * (w.lane >> 5) + (e & 3);
                if (row < M && col < N) f(t.v[r][j][e], (size_t)row * N + col);
            }
        }
}

// Row-major staging of the fp32 tile in LDS (TM / 2 KiB), then coalesced float4
// traffic: thread t owns quads t + NT q, quad f covering columns 4 (f % 32) .. +3
// of tile row f / 32.  Column c of row r is stored at c ^ epi_swz(r): the two
// rows written by one MFMA result register (4 apart) then fall on different
// banks, and every aligned quad stays contiguous.
constexpr int EPI_LD = BN;
__device__ __forceinline__ int epi_swz(int r) { return ((r >> 2) & 1) << 5; }

template <int NW, int TM>
__device__ __forceinline__ void acc_to_lds(float *tile, const Tile<NW, TM> &t) {
    const Role<NW> w;
#pragma unroll
    for (int r = 0; r < Tile<NW, TM>::R; ++r)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = w.wn * 64 + j * 32 + (w.lane & 31);
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = w.wm * (TM / 2) + t.i[r] * 32 + 8 * (e >> 2) + 4 * (w.lane >> 5) + (e & 3);
                tile[row * EPI_LD + (col ^ epi_swz(row))] = t.v[r][j][e];
            }
        }
}

__device__ __forceinline__ f32x4 staged_quad(const float *tile, int r, int c) {
    return *reinterpret_cast<const f32x4 *>(tile + r * EPI_LD + (c ^ epi_swz(r)));
}

// Calls f(q, row, col, global offset, valid columns in the quad (1..4)) for the
// thread's quads; rows beyond M and quads wholly beyond N are skipped.
template <int NW, int TM, class F>
__device__ __forceinline__ void for_each_quad(int m0, int n0, int M, int N, F &&f) {
    constexpr int NT = Role<NW>::NT, QPT = TM * BN / 4 / NT;
#pragma unroll
    for (int q = 0; q < QPT; ++q) {
        const int fq = threadIdx.x + NT * q;
        const int r = fq >> 5, c = (fq & 31) * 4;
        const int row = m0 + r, col = n0 + c;
        if (row < M && col < N) f(q, r, c, (size_t)row * N + col, min(4, N - col));
    }
}

__device__ __forceinline__ void put_quad(float *dst, f32x4 v, int nvalid, bool vec) {
    if (vec && nvalid == 4) {
        *reinterpret_cast<f32x4 *>(dst) = v;
    } else {
        for (int x = 0; x < nvalid; ++x) dst[x] = v[x];
    }
}

// Write the held rows to C straight from registers: each store instruction
// writes two 128-byte row segments (lanes 0-31 and 32-63), non-temporal.
template <int NW, int TM>
__device__ __forceinline__ void store_tile(float *X, int m0, int n0, int M, int N, const Tile<NW, TM> &t) {
    for_each_element<NW>(t, m0, n0, M, N, [&](float v, size_t off) { __builtin_nontemporal_store(v, X + off); });
}

// ---------------------------------------------------------------------------
// Fused epilogue (CUTLASS optimisation guide, "Epilogue Optimization" and
// "Fused Epilogue Operations"): y = alpha acc + beta c + bias[col], then ReLU
// or GELU.  Every kernel evaluates it with this one sequence of fp32
// operations, contraction off: y = fma(alpha, acc, beta c) + b, where c = 0
// when beta == 0 (C is then not read) and b = 0 without a bias, then the
// activation (GELU: (y / 2) (1 + erf(y / sqrt 2)), each step rounded).  A
// deterministic merge therefore gives the same bits whichever kernel stores
// the tile.  Stores of many elements run the activation's branch once for all
// of them (`finish`), so the unrolled code runs straight through: with the
// branch inside every element the code for 32 elements spans tens of KiB and
// misses in the instruction cache on every tile.
// ---------------------------------------------------------------------------
// GELU(y) = (y / 2) (1 + erf(z)), z = y / sqrt 2.  1 + erf(z) is formed from
// q = erfc(|z|) as 2 - q (y >= 0) or q (y < 0), so the negative side keeps its
// relative accuracy, with q from the rational approximation of Abramowitz and
// Stegun, Handbook of Mathematical Functions, 7.1.26:
//   erfc(x) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2) + e(x),
//   t = 1 / (1 + p x), |e(x)| <= 1.5e-7 for x >= 0,
// evaluated with explicit fma, the hardware reciprocal and exp2, branch free.
__device__ __forceinline__ float gelu_value(float y) {
#pragma clang fp contract(off)
    constexpr float P = 0.3275911f, A1 = 0.254829592f, A2 = -0.284496736f, A3 = 1.421413741f,
                    A4 = -1.453152027f, A5 = 1.061405429f;
    constexpr float RSQRT2 = 0.70710678118654752f, NEG_HALF_LOG2E = -0.72134752044448170f;
    const float x = fabsf(y) * RSQRT2;
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(P, x, 1.0f));
    float poly = __builtin_fmaf(A5, t, A4);
    poly = __builtin_fmaf(poly, t, A3);
    poly = __builtin_fmaf(poly, t, A2);
    poly = __builtin_fmaf(poly, t, A1);
    const float q = (poly * t) * __builtin_amdgcn_exp2f((y * y) * NEG_HALF_LOG2E);   // exp(-x^2) = 2^(-y^2 log2(e) / 2)
    const float one_plus_erf = y >= 0.0f ? 2.0f - q : q;
    return (0.5f * y) * one_plus_erf;
}

__device__ __forceinline__ float act_apply(int act, float y) {
    if (act == ACT_RELU) return y > 0.0f ? y : 0.0f;
    if (act == ACT_GELU) return gelu_value(y);
    return y;
}

__device__ __forceinline__ float lin_value(float alpha, float beta, float acc, float c, float b) {
#pragma clang fp contract(off)
    return __builtin_fmaf(alpha, acc, beta * c) + b;
}

__device__ __forceinline__ float epi_value(const KParams &p, float acc, float c, float b) {
    return act_apply(p.act, lin_value(p.alpha, p.beta, acc, c, b));
}

__device__ __forceinline__ bool reads_c(const KParams &p) { return p.epi == EPI_ACCUM || p.beta != 0.0f; }

// Numerical control (GEMM_DEBUG_ZERO_PARTIAL): every partial handed to another
// workgroup is written as zeros, so every split tile must come out wrong.
__device__ __forceinline__ bool zero_partials(const KParams &p) { return (p.debug & GEMM_DEBUG_ZERO_PARTIAL) != 0; }

// Final values of n elements, in place: v holds the sums, c the prior C values
// (0 where not read), b the bias values (0 without a bias).  EPI_ACCUM:
// v = fma(alpha, v, c) with no activation (a later pass applies it).
template <int N>
__device__ __forceinline__ void finish(const KParams &p, float (&v)[N], const float (&c)[N], const float (&b)[N]) {
    const float alpha = p.alpha, beta = p.beta;
    if (p.epi == EPI_ACCUM) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = __builtin_fmaf(alpha, v[i], c[i]);
        return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = lin_value(alpha, beta, v[i], c[i], b[i]);
    if (p.act == ACT_RELU) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = v[i] > 0.0f ? v[i] : 0.0f;
    } else if (p.act == ACT_GELU) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = gelu_value(v[i]);
    }
}

// One element, loads included (element-by-element paths only).
__device__ __forceinline__ float final_scalar(const KParams &p, float acc, size_t off, int col) {
    if (p.epi == EPI_PLAIN) return acc;
    float v[1] = {acc};
    const float c[1] = {reads_c(p) ? p.C[off] : 0.0f};
    const float b[1] = {p.bias ? p.bias[col] : 0.0f};
    finish<1>(p, v, c, b);
    return v[0];
}

// One wave's 32-row block of C for the epilogue: element (e, j) of lane l is at
// row R0 + 8 (e / 4) + 4 (l / 32) + e % 4, column C0 + 32 j + l % 32 (the
// 32x32 MFMA result layout).  Accesses go through a buffer range that ends at
// the block's last element inside C, so rows beyond M fall outside it, and a
// lane whose column is beyond N gets an offset outside every range: masked
// elements need no branches (their loads return 0, their stores are dropped).
// The row offsets are wave-uniform (scalar) multiples of the row pitch.
template <int NB>
struct CBlock {
    __amdgpu_buffer_rsrc_t r;
    uint32_t lane_off[NB];
    uint32_t pitch;
    __device__ __forceinline__ CBlock(const KParams &p, int R0, int C0) {
        R0 = __builtin_amdgcn_readfirstlane(R0);
        C0 = __builtin_amdgcn_readfirstlane(C0);
        const int lane = threadIdx.x & 63;
        const int vr = min(32, p.M - R0);
        const uint32_t bytes =
            (vr > 0 && C0 < p.N) ? ((uint32_t)(vr - 1) * (uint32_t)p.N + (uint32_t)(p.N - C0)) * 4u : 0u;
        r = __builtin_amdgcn_make_buffer_rsrc(p.C + (size_t)R0 * p.N + C0, (short)0, (int)bytes, (int)RSRC_DW3);
        pitch = (uint32_t)p.N * 4u;
#pragma unroll
        for (int j = 0; j < NB; ++j)
            lane_off[j] = C0 + 32 * j + (lane & 31) < p.N
                              ? ((uint32_t)(4 * (lane >> 5)) * (uint32_t)p.N + 32 * j + (lane & 31)) * 4u
                              : OOB;
    }
    __device__ __forceinline__ uint32_t off(int e, int j) const {
        return lane_off[j] + (uint32_t)(8 * (e >> 2) + (e & 3)) * pitch;
    }
    __device__ __forceinline__ float load(int e, int j) const {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off(e, j), 0, 0));
    }
    __device__ __forceinline__ void store(int e, int j, float v) const {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off(e, j), 0, CPOL_NT);
    }
};

// The bias values of a lane's NB 32-column blocks from column C0 (0 outside N
// or without a bias).
template <int NB>
__device__ __forceinline__ void lane_bias(const KParams &p, int C0, float (&bj)[NB]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int col = C0 + 32 * j + (lane & 31);
        bj[j] = (p.bias && col < p.N) ? p.bias[col] : 0.0f;
    }
}

// The epilogue inputs of the one 32-row block an 8-wave tile's wave holds after
// merge_k_halves (block row kh of its quarter): prior C values and the
// column's bias.  Loaded early (before the k-half merge and any fixup), they
// arrive while the tile is still being completed.
__device__ __forceinline__ void epi_prefetch(const KParams &p, int m0, int n0, float (&cin)[32], float (&bj)[2]) {
    const Role<8> w;
    const int C0 = n0 + w.wn * 64;
    lane_bias<2>(p, C0, bj);
    const CBlock<2> cb(p, m0 + w.wm * 64 + w.kh * 32, C0);
    const bool rc = reads_c(p);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) cin[j * 16 + e] = rc ? cb.load(e, j) : 0.0f;
}

// The epilogue and the stores of one held 32-row block (row r of the tile),
// its prior C values and bias values given.
template <int NW, int TM>
__device__ __forceinline__ void finish_block(const KParams &p, int m0, int n0, const Tile<NW, TM> &t, int r,
                                             const float (&cin)[32], const float (&bj)[2]) {
    const Role<NW> w;
    const CBlock<2> cb(p, m0 + w.wm * (TM / 2) + t.i[r] * 32, n0 + w.wn * 64);
    float v[32], c[32], bv[32];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            v[j * 16 + e] = t.v[r][j][e];
            c[j * 16 + e] = cin[j * 16 + e];
            bv[j * 16 + e] = bj[j];
        }
    finish<32>(p, v, c, bv);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) cb.store(e, j, v[j * 16 + e]);
}

// store_tile with the epilogue: the prior C values of the held rows are loaded
// before the first store.
template <int NW, bool EPI = true, int TM = 128>
__device__ __forceinline__ void store_final(const KParams &p, int m0, int n0, const Tile<NW, TM> &t) {
    if constexpr (!EPI) {
        store_tile<NW>(p.C, m0, n0, p.M, p.N, t);
    } else {
        if (p.epi == EPI_PLAIN) {
            store_tile<NW>(p.C, m0, n0, p.M, p.N, t);
            return;
        }
        const Role<NW> w;
        const bool rc = reads_c(p);
        const int C0 = n0 + w.wn * 64;
        float bj[2];
        lane_bias<2>(p, C0, bj);
#pragma unroll
        for (int r = 0; r < Tile<NW, TM>::R; ++r) {
            const CBlock<2> cb(p, m0 + w.wm * (TM / 2) + t.i[r] * 32, C0);
            float cin[32];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) cin[j * 16 + e] = rc ? cb.load(e, j) : 0.0f;
            finish_block<NW, TM>(p, m0, n0, t, r, cin, bj);
        }
    }
}

// Split parts of atomic merges: C += acc (EPI_ACCUM: C += alpha acc).
template <int NW, bool EPI = true, int TM = 128>
__device__ __forceinline__ void atomic_add_c(const KParams &p, int m0, int n0, const Tile<NW, TM> &t) {
    if (zero_partials(p)) {
        for_each_element<NW>(t, m0, n0, p.M, p.N, [&](float, size_t off) { unsafeAtomicAdd(p.C + off, 0.0f); });
    } else if (EPI && p.epi == EPI_ACCUM) {
        const float a = p.alpha;
        for_each_element<NW>(t, m0, n0, p.M, p.N, [&](float v, size_t off) { unsafeAtomicAdd(p.C + off, a * v); });
    } else {
        for_each_element<NW>(t, m0, n0, p.M, p.N, [&](float v, size_t off) { unsafeAtomicAdd(p.C + off, v); });
    }
}

// Store the thread's quads res[g] (quad g = threadIdx.x + NT g of the tile, N a
// multiple of 4) with the epilogue; loads of prior C and bias quads come first.
template <int NW, int QPT>
__device__ __forceinline__ void store_quads_final(const KParams &p, int m0, int n0, const f32x4 (&res)[QPT]) {
    constexpr int NT = Role<NW>::NT;
    if (p.epi == EPI_PLAIN) {
#pragma unroll
        for (int g = 0; g < QPT; ++g) {
            const int fq = threadIdx.x + NT * g, r = fq >> 5, c = (fq & 31) * 4;
            if (m0 + r < p.M && n0 + c < p.N)
                __builtin_nontemporal_store(res[g], reinterpret_cast<f32x4 *>(p.C + (size_t)(m0 + r) * p.N + n0 + c));
        }
        return;
    }
    const bool rc = reads_c(p);
    float v[4 * QPT], cin[4 * QPT], bv[4 * QPT];
#pragma unroll
    for (int g = 0; g < QPT; ++g) {
        const int fq = threadIdx.x + NT * g, r = fq >> 5, c = (fq & 31) * 4;
        const bool in = m0 + r < p.M && n0 + c < p.N;
        f32x4 cq = {0.f, 0.f, 0.f, 0.f}, bq = {0.f, 0.f, 0.f, 0.f};
        if (in && rc) cq = *reinterpret_cast<const f32x4 *>(p.C + (size_t)(m0 + r) * p.N + n0 + c);
        if (in && p.bias) bq = *reinterpret_cast<const f32x4 *>(p.bias + n0 + c);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            v[4 * g + x] = res[g][x];
            cin[4 * g + x] = cq[x];
            bv[4 * g + x] = bq[x];
        }
    }
    finish<4 * QPT>(p, v, cin, bv);
#pragma unroll
    for (int g = 0; g < QPT; ++g) {
        const int fq = threadIdx.x + NT * g, r = fq >> 5, c = (fq & 31) * 4;
        if (m0 + r < p.M && n0 + c < p.N)
            __builtin_nontemporal_store(f32x4{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]},
                                        reinterpret_cast<f32x4 *>(p.C + (size_t)(m0 + r) * p.N + n0 + c));
    }
}

// One 16-byte quad (quad q of the thread, N a multiple of 4) of final values with
// the epilogue, or nothing when it lies outside C.
template <int NW>
__device__ __forceinline__ void store_quad_final(const KParams &p, int m0, int n0, int q, f32x4 v) {
    constexpr int NT = Role<NW>::NT;
    const int fq = threadIdx.x + NT * q, r = fq >> 5, c = (fq & 31) * 4;
    if (m0 + r >= p.M || n0 + c >= p.N) return;
    f32x4 *dst = reinterpret_cast<f32x4 *>(p.C + (size_t)(m0 + r) * p.N + n0 + c);
    if (p.epi != EPI_PLAIN) {
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 cq = reads_c(p) ? *dst : zero;
        const f32x4 bq = p.bias ? *reinterpret_cast<const f32x4 *>(p.bias + n0 + c) : zero;
        float w[4] = {v[0], v[1], v[2], v[3]};
        const float cin[4] = {cq[0], cq[1], cq[2], cq[3]}, bv[4] = {bq[0], bq[1], bq[2], bq[3]};
        finish<4>(p, w, cin, bv);
        v = f32x4{w[0], w[1], w[2], w[3]};
    }
    __builtin_nontemporal_store(v, dst);
}

// ---------------------------------------------------------------------------
// Partial exchange between workgroups ("store the partial, signal, the owner
// waits and reads it": book chapter, "Mental model").  It rests on two
// properties of the GFX942 memory model that gfx950 follows (LLVM AMDGPU
// backend documentation, "Memory Model GFX942"):
//  1. sc1 loads and stores are how the backend implements agent-scope relaxed
//     atomic loads and stores, so they are coherent across the XCDs' separate
//     L2 caches.  Every partial is written and read with sc1 buffer accesses,
//     every flag and counter with agent-scope atomics.
//  2. A wave's vector memory operations report completion (vmcnt) in the order
//     they were issued, stores included; flat instructions that reach LDS are
//     the documented exception and none is used here.
// The writer waits until its partial stores are complete (a vmcnt wait in every
// wave, then a barrier) before the flag or counter changes; the reader issues
// its partial loads only after the flag's value has come back.  That is the
// model's release/acquire pair without the L2 write-back and invalidate, which
// serve non-sc1 accesses only -- and the invalidate would throw away the A and
// B panels the other CUs of the XCD are streaming.
// ---------------------------------------------------------------------------
constexpr int CPOL_DEVICE = 16;   // cache-policy bits: sc1 (device scope)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, (int)RSRC_DW3);
}
__device__ __forceinline__ void put4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, CPOL_DEVICE);
}
__device__ __forceinline__ f32x4 get4_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CPOL_DEVICE));
}
__device__ __forceinline__ void put_coherent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float get_coherent(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every vector-memory operation of this wave has completed.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }

// Stream-K partial slot (TM x 128 fp32: 64 or 128 KiB) in register-native
// order: for accumulator block b = 2 i + j of a wave's part and element quad
// e4, the 64 lanes of a wave move 1 KiB of contiguous memory.
template <int TM = 128>
__device__ __forceinline__ uint32_t slot_off(int quad, int b, int e4, int lane) {
    return (uint32_t)((((quad * 2 * (TM / 64) + b) * 4 + e4) * 64 + lane) * 16);
}

template <int NW, int TM>
__device__ __forceinline__ void put_slot(float *slot, const Tile<NW, TM> &t, bool zero) {
    const Role<NW> w;
    const __amdgpu_buffer_rsrc_t r = span(slot, TM * BN * 4);
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};   // the zero-partial control
#pragma unroll
    for (int h = 0; h < Tile<NW, TM>::R; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const f32x16 &v = t.v[h][j];
                put4_coherent(r, slot_off<TM>(w.quad, 2 * t.i[h] + j, e4, w.lane),
                              zero ? zero4 : f32x4{v[4 * e4], v[4 * e4 + 1], v[4 * e4 + 2], v[4 * e4 + 3]});
            }
}

// A wave's share of a partial slot: the values of its held block rows.
template <int NW, int TM>
struct SlotPart {
    f32x4 x[Tile<NW, TM>::R][2][4];
};

// Loads of the wave's share of `slot` for the block rows held_row(0 .. R - 1),
// all issued at once (the wave later waits for them once).
template <int NW, int TM>
__device__ __forceinline__ void load_slot(const float *slot, SlotPart<NW, TM> &s) {
    const Role<NW> w;
    const __amdgpu_buffer_rsrc_t r = span(slot, TM * BN * 4);
#pragma unroll
    for (int h = 0; h < Tile<NW, TM>::R; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
                s.x[h][j][e4] = get4_coherent(r, slot_off<TM>(w.quad, 2 * held_row<NW, TM>(h) + j, e4, w.lane));
}

template <int NW, int TM>
__device__ __forceinline__ void add_part(Tile<NW, TM> &t, const SlotPart<NW, TM> &s) {
#pragma unroll
    for (int h = 0; h < Tile<NW, TM>::R; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
                for (int y = 0; y < 4; ++y) t.v[h][j][4 * e4 + y] += s.x[h][j][e4][y];
}

// t += slot over the held rows.
template <int NW, int TM>
__device__ __forceinline__ void add_slot(const float *slot, Tile<NW, TM> &t) {
    SlotPart<NW, TM> s;
    load_slot<NW, TM>(slot, s);
    add_part(t, s);
}

// Poll `flag` (one thread) until it holds `epoch`, one untracked load per poll.
// Gives up after `limit` polls, recording STATUS_TIMEOUT.
__device__ __forceinline__ void wait_flag(const uint32_t *flag, uint32_t epoch, uint32_t limit, uint32_t *status) {
    for (uint32_t polls = 1;; ++polls) {
        uint32_t v = load_flag_async(flag);
        wait_vm_all();
        if (flag_value(v) == epoch) return;
        if (polls >= limit) {
            __hip_atomic_fetch_or(status, STATUS_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Poll a counter (one thread) until it reaches at least `target`; bounded like
// wait_flag.
__device__ __forceinline__ void wait_count(const uint32_t *ctr, uint32_t target, uint32_t limit, uint32_t *status) {
    for (uint32_t polls = 1;; ++polls) {
        uint32_t v = load_flag_async(ctr);
        wait_vm_all();
        if (flag_value(v) >= target) return;
        if (polls >= limit) {
            __hip_atomic_fetch_or(status, STATUS_TIMEOUT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// wait_flag whose first poll was issued earlier (v0 from load_flag_async), so
// its latency overlapped other work.
__device__ __forceinline__ void wait_flag_issued(const uint32_t *flag, uint32_t v0, uint32_t epoch, uint32_t limit,
                                                 uint32_t *status) {
    wait_vm_all();
    if (flag_value(v0) == epoch) return;
    wait_flag(flag, epoch, limit, status);
}

// ---------------------------------------------------------------------------
// Debug trace (thread 0 only; active only when p.trace is set)
// ---------------------------------------------------------------------------
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
    rec[0] = max(rec[0], nseg + 1);
}
__device__ __forceinline__ void trace_folded(const KParams &p, int tile, int pos, int w) {
    if (!p.trace || threadIdx.x != 0 || pos >= p.trace_maxfold) return;
    int *rec = trace_fold(p, tile);
    rec[1 + pos] = w;
    rec[0] = pos + 1;
}

// Per-workgroup placement and busy time (only when p.timing is set): 8 int64 per
// workgroup, {start, end, HW_ID | XCC_ID << 32, shader cycles, mark0..mark3},
// times in 100 MHz ticks.
struct WgClock {
    unsigned long long t0, c0;   // start: 100 MHz real time, shader clock cycles
    __device__ __forceinline__ explicit WgClock(const KParams &p) : t0(0), c0(0) {
        if (p.timing) {
            t0 = __builtin_amdgcn_s_memrealtime();
            c0 = __builtin_amdgcn_s_memtime();
        }
    }
    __device__ __forceinline__ long long *entry(const KParams &p) const {
        return p.timing + 8 * ((size_t)p.timing_base + blockIdx.x);
    }
    __device__ __forceinline__ void mark(const KParams &p, int k) const {
        if (p.timing && threadIdx.x == 0 && k < 4) entry(p)[4 + k] = (long long)__builtin_amdgcn_s_memrealtime();
    }
    __device__ __forceinline__ void done(const KParams &p) const {
        if (!p.timing || threadIdx.x != 0) return;
        long long *e = entry(p);
        const unsigned long long c1 = __builtin_amdgcn_s_memtime();
        e[0] = (long long)t0;
        e[1] = (long long)__builtin_amdgcn_s_memrealtime();
        const uint32_t hw = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));    // HW_REG_HW_ID
        const uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11));  // HW_REG_XCC_ID
        e[2] = (long long)(((unsigned long long)xcc << 32) | hw);
        e[3] = (long long)(c1 - c0);
    }
};

// ---------------------------------------------------------------------------
// Data-parallel: one workgroup per tile of [tile_base, tile_base + ntiles).
// ---------------------------------------------------------------------------
template <int DT, int BL, int NS, int NW, int TM = 128, bool GRP = false>
__global__ __launch_bounds__(64 * NW) void gemm_dp(KParams p) {
    __shared__ __attribute__((aligned(16))) char lds[lds_bytes<TM>(NS)];
    const WgClock clk(p);
    const int w = worker_of(p);
    const int tile = p.tile_base + w;
    int m0, n0;
    const KParams q = tile_view<GRP>(p, tile, m0, n0);
    AccT<TM> acc;
    zero_acc(acc);
    mac_loop<DT, BL, NS, NW, TM>(q, lds, m0, n0, 0, p.ipt, 0, acc, p.trace ? trace_cov(p, tile) : nullptr);
    const Tile<NW, TM> t = merge_k_halves<NW, TM>(acc, lds);
    clk.mark(p, 0);
    store_final<NW>(q, m0, n0, t);
    trace_segment(p, p.worker_base + w, 0, tile, 0, p.ipt, 0);
    trace_folded(p, tile, 0, p.worker_base + w);
    clk.done(p);
}

// ---------------------------------------------------------------------------
// Data-parallel tile groups: one workgroup computes a 2x2 group of 128x128
// tiles (a 256x256 block of C) over the whole K, for launches with enough
// tiles to fill the chip four times over.  Each tile is still computed whole
// by one workgroup with no fixup (the data-parallel schedule is unchanged);
// what changes is the operand traffic per flop.  A 256x256x64 step moves
// 64 KiB global -> LDS (half of what four 128x128 steps move) and, with eight
// waves of 128x64, 192 KiB LDS -> registers (three quarters).  On MI355X the
// clock under a dense MFMA load is set by that traffic, so the group runs
// closer to the matrix-core bound (CUTLASS optimisation guide: larger
// threadblock tiles raise arithmetic intensity).
//
// Waves: wave w owns rows 128 (w & 1) .. +128 and columns 64 (w >> 1) .. +64 of
// the group, 4 x 2 blocks of 32 x 32 (eight accumulators), and issues all four
// 16-wide k-steps of each iteration (no k-split, no merge).  Two LDS stages of
// (A slab [256 x 64] | B slab [64 x 256]) = 64 KiB each; iteration i + 2 is
// loaded into the stage iteration i used, after the barrier that ends
// iteration i, one load between each pair of k-step-3 MFMAs; within an
// iteration the fragments of k-step j + 1 are read while the MFMAs of k-step j
// run.
// ---------------------------------------------------------------------------
constexpr int GB = 2 * BM;                     // group edge: 256
constexpr int G_SLAB = GB * BK * 2;            // bytes of one operand slab of one stage: 32 KiB
constexpr int G_NS = 2;                        // stages
constexpr int G_BREG = G_NS * G_SLAB;          // B slabs start at 64 KiB
// Waves per group: 8 of 128x64 (two per SIMD).  GroupLoop also builds with 4
// waves of 128x128 (one per SIMD, accumulators in AGPRs, a third less LDS read
// traffic); measured on the 8192^3 launch the eight-wave form is 2-4 % faster.
constexpr int G_NW = 8;

template <int NW>
struct GAcc {
    static constexpr int JB = NW == 4 ? 4 : 2; // 32-column blocks of a wave
    f32x16 v[4][JB];                           // [32-row block][32-column block]
};

template <int DT, int BL, int NW>
struct GroupLoop {
    static constexpr int WCOLS = NW == 4 ? 128 : 64;   // columns of a wave
    static constexpr int JB = WCOLS / 32;              // 32-column blocks of a wave
    static constexpr int DPW = 32 / NW;                // DMA instructions per wave and operand slab
    static constexpr int DPI = 2 * DPW;                // per iteration
    static_assert(NW == 4 || NW == 8, "four or eight waves");

    const KParams &p;
    uint32_t lds0;
    int lane, wave;
    uint32_t aoff[4];                          // A fragment read address per k-step (stage 0, row block 0)
    uint32_t boff[4];                          // B [N,K]: per k-step (column block 0); B [K,N]: per column block
    uint32_t adma[DPW], bdma[DPW];             // per-lane global byte offsets of the wave's loads at k = 0
    int a_kc[DPW], b_kc[DPW];                  // first k of the lane's chunk (B [K,N]: the lane's k-row)
    const char *a_base, *b_base;
    uint32_t a_rows_bytes, b_rows_bytes;

    __device__ __forceinline__ GroupLoop(const KParams &p_, char *lds, int m0, int n0) : p(p_) {
        lds0 = (uint32_t)reinterpret_cast<uintptr_t>((const lds_void *)lds);
        lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
        const int wm = wave & 1, wn = wave >> 1;
        const int K = p.K, N = p.N;
        const int r32 = lane & 31, hk = lane >> 5;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const uint32_t rowpart = (uint32_t)(r32 * 128 + ((((2 * kk + hk) ^ kswz(r32)) & 7) << 4));
            aoff[kk] = lds0 + wm * 128 * 128 + rowpart;
            if constexpr (BL == 1) boff[kk] = lds0 + G_BREG + wn * WCOLS * 128 + rowpart;
        }
        if constexpr (BL == 0) {
            // 256-column k-rows of 512 bytes (32 chunks), chunk c of k-row r at c ^ nswz(r)
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                const int n = wn * WCOLS + jb * 32 + ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
                const int r = 8 * hk + ((lane & 15) >> 2);
                boff[jb] = lds0 + G_BREG + r * 512 + ((((n >> 3) ^ nswz(r)) & 31) << 4) + ((n & 7) << 1);
            }
        }
        const int first = wave * DPW;
        a_base = reinterpret_cast<const char *>(p.A) + (size_t)m0 * K * 2;
        a_rows_bytes = (uint32_t)(min(GB, p.M - m0) * K * 2);
#pragma unroll
        for (int x = 0; x < DPW; ++x) {
            const int r = 8 * (first + x) + (lane >> 3);          // 0..255
            const int c = (lane & 7) ^ kswz(r);
            adma[x] = (uint32_t)(r * K + 8 * c) * 2;
            a_kc[x] = 8 * c;
            if constexpr (BL == 1) {
                bdma[x] = adma[x];
                b_kc[x] = 8 * c;
            } else {
                const int rb = 2 * (first + x) + (lane >> 5);      // k-row 0..63
                const int cb = (lane & 31) ^ nswz(rb);
                bdma[x] = n0 + 8 * cb >= N ? OOB : (uint32_t)(rb * N + 8 * cb) * 2;
                b_kc[x] = rb;
            }
        }
        if constexpr (BL == 1) {
            b_base = reinterpret_cast<const char *>(p.B) + (size_t)n0 * K * 2;
            b_rows_bytes = (uint32_t)(min(GB, N - n0) * K * 2);
        } else {
            b_base = reinterpret_cast<const char *>(p.B) + (size_t)n0 * 2;
            b_rows_bytes = 0;
        }
    }

    // Buffer resources and LDS destinations of the loads of K-slab `slab` into stage `st`.
    struct Issue {
        i32x4 ra, rb;
        uint32_t a_dst, b_dst;
        int kb;
    };
    __device__ __forceinline__ Issue prepare(int slab, int st) const {
        Issue q;
        q.kb = slab * BK;
        q.ra = make_rsrc(a_base + (size_t)q.kb * 2, a_rows_bytes - q.kb * 2);
        if constexpr (BL == 1) {
            q.rb = make_rsrc(b_base + (size_t)q.kb * 2, b_rows_bytes - q.kb * 2);
        } else {
            const int krows = min(BK, p.K - q.kb);
            q.rb = make_rsrc(b_base + (size_t)q.kb * p.N * 2, (uint32_t)(krows * p.N * 2));
        }
        q.a_dst = lds0 + st * G_SLAB + wave * DPW * 1024;
        q.b_dst = lds0 + G_BREG + st * G_SLAB + wave * DPW * 1024;
        return q;
    }
    // Load number x of the iteration (A slab loads first, then B); RAGGED: chunks
    // at or beyond K read zeros.
    template <bool RAGGED>
    __device__ __forceinline__ void issue_one(const Issue &q, int x) const {
        if (x < DPW) {
            dma16(q.ra, q.a_dst + x * 1024, !RAGGED || q.kb + a_kc[x] < p.K ? adma[x] : OOB);
        } else {
            const int y = x - DPW;
            uint32_t off = bdma[y];
            if constexpr (RAGGED && BL == 1) off = q.kb + b_kc[y] < p.K ? off : OOB;
            dma16(q.rb, q.b_dst + y * 1024, off);
        }
    }
    template <bool RAGGED>
    __device__ __forceinline__ void issue(int slab, int st) const {
        const Issue q = prepare(slab, st);
#pragma unroll
        for (int x = 0; x < DPI; ++x) issue_one<RAGGED>(q, x);
    }

    struct Frags {
        u32x4 a[4];   // [32-row block]
        u32x4 b[JB];  // [32-column block]
    };

    // Fragments of k-step KK of stage ST.
    template <int ST, int KK>
    __device__ __forceinline__ void read(Frags &f) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) f.a[i] = lds_b128<ST * G_SLAB>(aoff[KK] + i * 4096);
        if constexpr (BL == 1) {
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) f.b[jb] = lds_b128<ST * G_SLAB>(boff[KK] + jb * 4096);
        } else {
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                const u32x2 h0 = lds_tr16<ST * G_SLAB + KK * 16 * 512>(boff[jb]);
                const u32x2 h1 = lds_tr16<ST * G_SLAB + KK * 16 * 512 + 4 * 512>(boff[jb]);
                f.b[jb] = u32x4{h0[0], h0[1], h1[0], h1[1]};
            }
        }
    }

    static __device__ __forceinline__ void mma(const Frags &f, GAcc<NW> &acc) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) acc.v[i][jb] = mfma<DT>(f.a[i], f.b[jb], acc.v[i][jb]);
    }
    // The MFMAs of f, with the DPI loads of `q` (when `load`) issued between
    // them so that the matrix pipe keeps running while they go out.
    template <bool RAGGED>
    __device__ __forceinline__ void mma_issue(const Frags &f, GAcc<NW> &acc, bool load, const Issue &q) const {
        static_assert(4 * JB == DPI, "one load per MFMA");
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jb = 0; jb < JB; ++jb) {
                acc.v[i][jb] = mfma<DT>(f.a[i], f.b[jb], acc.v[i][jb]);
                __builtin_amdgcn_sched_barrier(0);
                if (load) issue_one<RAGGED>(q, i * JB + jb);
                __builtin_amdgcn_sched_barrier(0);
            }
    }
};

// acc += the group's A rows . B columns over all ipt iterations.  Ends with a
// barrier (LDS free on return).
template <int DT, int BL, int NW, bool RAGGED>
__device__ __forceinline__ void group_loop(const KParams &p, char *lds, int m0, int n0, GAcc<NW> &acc) {
    using GL = GroupLoop<DT, BL, NW>;
    const int n = p.ipt;
    if (n <= 0) return;
    const GL gl(p, lds, m0, n0);
    typename GL::Frags f[2];
    gl.template issue<RAGGED>(0, 0);
    if (n > 1) {
        gl.template issue<RAGGED>(1, 1);
        wait_vm_lgkm<GL::DPI>();
    } else {
        wait_vm_lgkm<0>();
    }
    __builtin_amdgcn_s_barrier();
    gl.template read<0, 0>(f[0]);
    // One iteration on stage ST: k-steps 0..2 read the next k-step's fragments
    // and multiply the current ones; k-step 3 first hands the stage over: wait
    // for this wave's loads of i + 1 and reads of (i, 3), barrier (every wave's
    // loads of i + 1 landed and every wave is done reading stage ST), read
    // (i + 1, 0), then multiply k-step 3 while loading iteration i + 2 into
    // stage ST.
    auto iter = [&](int i, auto ST) {
        constexpr int st = decltype(ST)::value;
        __builtin_amdgcn_sched_barrier(0);
        gl.template read<st, 1>(f[1]);
        GL::mma(f[0], acc);
        __builtin_amdgcn_sched_barrier(0);
        gl.template read<st, 2>(f[0]);
        GL::mma(f[1], acc);
        __builtin_amdgcn_sched_barrier(0);
        gl.template read<st, 3>(f[1]);
        GL::mma(f[0], acc);
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < n) {
            wait_vm_lgkm<0>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            gl.template read<st ^ 1, 0>(f[0]);
        }
        gl.template mma_issue<RAGGED>(f[1], acc, i + 2 < n, gl.prepare(i + 2, st));
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int i = 0; i < n; i += 2) {
        iter(i, std::integral_constant<int, 0>());
        if (i + 1 < n) iter(i + 1, std::integral_constant<int, 1>());
    }
    wait_stage0();
}

// The 128x128 tile with tile-grid coordinates (tm, tn): the inverse of tile_origin.
__device__ __forceinline__ int tile_id(const KParams &p, int tm, int tn) {
    const int gm_full = p.group_m > 0 ? p.group_m : p.tiles_m;
    const int g = tm / gm_full;
    const int first = g * gm_full;
    const int gm = min(gm_full, p.tiles_m - first);
    return g * gm_full * p.tiles_n + tn * gm + (tm - first);
}

// Group g of the ceil(tiles_m / 2) x ceil(tiles_n / 2) group grid, numbered like
// tile_origin numbers tiles (bands of group_m / 2 group rows, column by column).
// With an odd tile count along M or N the last groups hang over the edge; their
// loads beyond M / N read zeros and their stores are masked.
__device__ __forceinline__ void group_origin(const KParams &p, int g, int &m0, int &n0) {
    const int gms = (p.tiles_m + 1) / 2, gns = (p.tiles_n + 1) / 2;
    const int gm_full = p.group_m > 1 ? p.group_m / 2 : gms;
    const int per_band = gm_full * gns;
    const int band = g / per_band;
    const int first = band * gm_full;
    const int gm = min(gm_full, gms - first);
    const int w = g - band * per_band;
    m0 = (first + w % gm) * GB;
    n0 = (w / gm) * GB;
}

// Launch: one workgroup per group (ntiles = the group count), tile_base 0.
template <int DT, int BL>
__global__ __launch_bounds__(64 * G_NW) void gemm_dp_group(KParams p) {
    __shared__ __attribute__((aligned(16))) char lds[G_NS * 2 * G_SLAB];
    constexpr int JB = GAcc<G_NW>::JB;
    const WgClock clk(p);
    const int g = worker_of(p);
    // groups are numbered batch after batch, gpb per batch entry
    const int gpb = ((p.tiles_m + 1) / 2) * ((p.tiles_n + 1) / 2);
    const int b = p.batch > 1 ? g / gpb : 0;
    const KParams q = p.batch > 1 ? batch_entry(p, b) : p;
    int m0, n0;
    group_origin(p, g - b * gpb, m0, n0);
    GAcc<G_NW> acc;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc.v[i][j][e] = 0.0f;
    if (p.K % BK == 0) group_loop<DT, BL, G_NW, false>(q, lds, m0, n0, acc);
    else group_loop<DT, BL, G_NW, true>(q, lds, m0, n0, acc);
    clk.mark(p, 0);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    if (p.epi == EPI_PLAIN) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                const int col = n0 + wn * JB * 32 + j * 32 + (lane & 31);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = m0 + wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    if (row < p.M && col < p.N) __builtin_nontemporal_store(acc.v[i][j][e], q.C + (size_t)row * p.N + col);
                }
            }
    } else {
        // epilogue, one 32-row block at a time; the prior C values of block
        // i + 1 are loaded before block i is stored, so no wait for loaded
        // values ever waits for stores as well (one counter covers both)
        const bool rc = reads_c(p);
        const int C0 = n0 + wn * JB * 32;
        float bj[JB];
        lane_bias<JB>(p, C0, bj);
        auto block = [&](int i) { return CBlock<JB>(q, m0 + wm * 128 + i * 32, C0); };
        float cbuf[2][JB * 16];
        auto load_block = [&](int i, float (&cin)[JB * 16]) {
            const CBlock<JB> cb = block(i);
#pragma unroll
            for (int j = 0; j < JB; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) cin[j * 16 + e] = rc ? cb.load(e, j) : 0.0f;
        };
        load_block(0, cbuf[0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i + 1 < 4) load_block(i + 1, cbuf[(i + 1) & 1]);
            const CBlock<JB> cb = block(i);
            // 16 values at a time, fenced from the scheduler, so the epilogue
            // arithmetic of many values is not interleaved into more live
            // registers than the accumulators leave free
#pragma unroll
            for (int j = 0; j < JB; ++j) {
                float v[16], cin[16], bv[16];
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    bv[e] = bj[j];
                    v[e] = acc.v[i][j][e];
                    cin[e] = cbuf[i & 1][j * 16 + e];
                }
                finish<16>(p, v, cin, bv);
#pragma unroll
                for (int e = 0; e < 16; ++e) cb.store(e, j, v[e]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (p.trace && threadIdx.x == 0) {
        // the four tiles of the group, each a whole-K data-parallel tile
        for (int x = 0; x < 4; ++x) {
            const int tm = m0 / BM + (x & 1), tn = n0 / BN + (x >> 1);
            if (tm >= p.tiles_m || tn >= p.tiles_n) continue;   // over the edge of the tile grid
            const int tile = b * p.tiles_m * p.tiles_n + tile_id(p, tm, tn);
            trace_segment(p, p.worker_base + tile, 0, tile, 0, p.ipt, 0);
            trace_folded(p, tile, 0, p.worker_base + tile);
            int *cov = trace_cov(p, tile);
            for (int k = 0; k < p.ipt; ++k) atomicAdd(cov + k, 1);
        }
    }
    clk.done(p);
}

// ---------------------------------------------------------------------------
// Split-K: worker w = tile * S + s covers k-iterations [s P / S, (s+1) P / S).
// ---------------------------------------------------------------------------
template <int DT, int BL, int NS, int NW, int TM = 128, bool GRP = false>
__global__ __launch_bounds__(64 * NW) void gemm_splitk(KParams p0) {
    constexpr int NT = Role<NW>::NT, QPT = TM * BN / 4 / NT;
    // the stages, reused to stage the fp32 tile (TM x 128) after the loop
    static_assert(lds_bytes<TM>(NS) >= TM * BN * 4, "the staged tile fits the stages");
    __shared__ __attribute__((aligned(16))) char lds[lds_bytes<TM>(NS)];
    __shared__ int last_arriver;
    const WgClock clk(p0);
    const int S = p0.splits;
    const int w = worker_of(p0);
    const int tile = fdiv(w, p0.d_splits), s = w - tile * S;
    // S divides the iterations in every plan (aligned split); the general
    // bounds [s P / S, (s + 1) P / S) otherwise
    const int chunk = fdiv(p0.ipt, p0.d_splits);
    const bool aligned = chunk * S == p0.ipt;
    const int k0 = aligned ? s * chunk : (int)((int64_t)s * p0.ipt / S);
    const int k1 = aligned ? k0 + chunk : (int)((int64_t)(s + 1) * p0.ipt / S);
    int m0, n0;
    const KParams p = tile_view<GRP>(p0, tile, m0, n0);   // the tile's batch entry
    AccT<TM> acc;
    zero_acc(acc);
    mac_loop<DT, BL, NS, NW, TM>(p, lds, m0, n0, k0, k1, 0, acc, p.trace ? trace_cov(p, tile) : nullptr);
    const Tile<NW, TM> t = merge_k_halves<NW, TM>(acc, lds);
    clk.mark(p, 0);
    trace_segment(p, w, 0, tile, k0, k1, S == 1 ? 0 : (s == 0 ? 1 : 2));
    if (S == 1) {
        store_final<NW>(p, m0, n0, t);
        trace_folded(p, tile, 0, w);
        clk.done(p);
        return;
    }
    if (p.merge == MERGE_ATOMIC) {   // "parallel" Split-K: add into the zero-filled C
        atomic_add_c<NW>(p, m0, n0, t);
        clk.done(p);
        return;
    }
    // stage the accumulator in LDS; write this split's partial P[s] as row quads
    // with device-scope stores (LDS keeps the copy this workgroup may fold itself)
    const size_t mn = (size_t)p.M * p.N;
    float *stg = reinterpret_cast<float *>(lds);
    acc_to_lds<NW, TM>(stg, t);
    __syncthreads();
    const size_t org = (size_t)m0 * p.N + n0;                 // tile origin within [M,N]
    const uint32_t span_bytes = (uint32_t)(((size_t)(min(TM, p.M - m0) - 1) * p.N + min(BN, p.N - n0)) * 4);
    auto quad_off = [&](int r, int c) { return (uint32_t)(((size_t)r * p.N + c) * 4); };
    // MERGE_BANDS: row band q (rows TM q / 8 .. TM (q + 1) / 8 - 1 of the tile,
    // the threads' quad q) is added up by split q mod S, which takes its own part of the band
    // from LDS and so does not store it
    const bool bands = p.merge == MERGE_BANDS;
    {
        const __amdgpu_buffer_rsrc_t rp = span(p.part + (size_t)s * mn + org, span_bytes);
        float *Ps = p.part + (size_t)s * mn;
        const bool zero = zero_partials(p);   // the zero-partial control
        for_each_quad<NW, TM>(m0, n0, p.M, p.N, [&](int q, int r, int c, size_t off, int nv) {
            if (bands && q % S == s) return;
            const f32x4 v = zero ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : staged_quad(stg, r, c);
            if (nv == 4) {
                put4_coherent(rp, quad_off(r, c), v);
            } else {
                for (int x = 0; x < nv; ++x) put_coherent(Ps + off + x, v[x]);
            }
        });
    }
    wait_vm_all();                 // this wave's partial stores are complete
    __syncthreads();               // ... and every other wave's
    clk.mark(p, 1);
    if (p.merge == MERGE_TWO_PASS) {   // the second kernel folds the partials
        clk.done(p);
        return;
    }
    auto quad_rc = [&](int g, int &r, int &c) {
        const int fq = threadIdx.x + NT * g;
        r = fq >> 5;
        c = (fq & 31) * 4;
    };
    auto in_c = [&](int r, int c) { return m0 + r < p.M && n0 + c < p.N; };
    auto get4 = [&](int t, int r, int c) {
        return get4_coherent(span(p.part + (size_t)t * mn + org, span_bytes), quad_off(r, c));
    };
    if (bands) {
        // every split arrives at the tile's counter and waits until all S have (the
        // whole grid is resident, so the wait ends); then it adds up its own bands
        // q = s, s + S, ... (at most 4 of the QPT = 8), the partials in split
        // order with its own from LDS; then it departs, and the last of the 2 S
        // arrivals and departures resets the counter for the next call
        if (threadIdx.x == 0) {
            __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wait_count(p.counters + tile, (uint32_t)S, p.spin_limit, p.status);
        }
        __syncthreads();
        clk.mark(p, 3);
        static_assert(QPT == 8, "eight row bands of 16 rows");
        // every load of the split's bands in one round, then the adds: G band
        // slots (q = s + g S) by the T splits other than s (the j-th other split
        // is j, or j + 1 from s on)
        auto fold = [&](auto GC, auto TC) {
            constexpr int G = decltype(GC)::value, T = decltype(TC)::value;
            f32x4 x[G][T];
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int j = 0; j < T; ++j) {
                    const int q = s + g * S, t = j < s ? j : j + 1;
                    int r, c;
                    quad_rc(q, r, c);
                    x[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (q < QPT && j < S - 1 && in_c(r, c)) x[g][j] = get4(t, r, c);
                }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int q = s + g * S;
                if (q >= QPT) continue;
                int r, c;
                quad_rc(q, r, c);
                const f32x4 own = staged_quad(stg, r, c);
                f32x4 sum = own;
#pragma unroll
                for (int t = 0; t <= T; ++t) {   // partial t in split order
                    if (t >= S) break;
                    // indices clamped into range; the loop is unrolled, so they are constants
                    const f32x4 below = x[g][t < T ? t : T - 1], above = x[g][t >= 1 ? t - 1 : 0];
                    const f32x4 v = t < s ? below : (t > s ? above : own);
                    sum = t == 0 ? v : sum + v;
                }
                store_quad_final<NW>(p, m0, n0, q, sum);
            }
        };
        if (S <= 4) {
            fold(std::integral_constant<int, 4>(), std::integral_constant<int, 3>());
        } else if (S <= 8) {
            fold(std::integral_constant<int, 2>(), std::integral_constant<int, 7>());
        } else if (s < QPT) {
            // one band, its S partials in rounds of 8 loads
            int r, c;
            quad_rc(s, r, c);
            f32x4 sum = staged_quad(stg, r, c);
            for (int t0 = 0; t0 < S; t0 += 8) {
                f32x4 x[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int t = t0 + k;
                    x[k] = t == s || t >= S || !in_c(r, c) ? staged_quad(stg, r, c) : get4(t, r, c);
                }
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    if (t0 + k < S) sum = t0 + k == 0 ? x[k] : sum + x[k];
            }
            store_quad_final<NW>(p, m0, n0, s, sum);
        }
        if (threadIdx.x == 0) {
            const uint32_t before =
                __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (before == (uint32_t)(2 * S - 1))
                __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (s == 0)
            for (int t = 0; t < S; ++t) trace_folded(p, tile, t, tile * S + t);
        clk.mark(p, 2);
        clk.done(p);
        return;
    }
    if (threadIdx.x == 0) {
        const uint32_t before =
            __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool is_last = before == (uint32_t)(S - 1);
        if (is_last)   // every split has arrived: reset for the next call
            __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_arriver = is_last ? 1 : 0;
    }
    __syncthreads();
    if (!last_arriver) {
        clk.done(p);
        return;
    }
    // Fold the S partials in split order, ((P0 + P1) + P2) + ..., taking this
    // workgroup's own split from LDS.  With N % 4 == 0 every quad of the tile is
    // whole or wholly outside C, and the fold moves 16-byte quads: for S <= 4 all
    // QPT quads of the thread with the S - 1 other partials in one round of
    // loads, for larger S rounds of 4 quads with up to 4 partials each.  Any
    // other N folds element by element.
    if ((p.N & 3) != 0) {
        for (int g = 0; g < QPT; ++g) {
            int r, c;
            quad_rc(g, r, c);
            const f32x4 own = staged_quad(stg, r, c);
            for (int x = 0; x < 4; ++x) {
                if (!in_c(r, c + x)) continue;
                const size_t off = (size_t)(m0 + r) * p.N + n0 + c + x;
                float sum = 0.f;
                for (int t = 0; t < S; ++t) {
                    const float v = t == s ? own[x] : get_coherent(p.part + (size_t)t * mn + off);
                    sum = t == 0 ? v : sum + v;
                }
                p.C[off] = final_scalar(p, sum, off, n0 + c + x);
            }
        }
    } else {
      f32x4 res[QPT];
      if (S <= 4) {
        f32x4 buf[3][QPT];   // buf[j]: the j-th partial other than this split's
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int t = j < s ? j : j + 1;
#pragma unroll
            for (int g = 0; g < QPT; ++g) {
                int r, c;
                quad_rc(g, r, c);
                buf[j][g] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (j < S - 1 && in_c(r, c)) buf[j][g] = get4(t, r, c);
            }
        }
#pragma unroll
        for (int g = 0; g < QPT; ++g) {
            int r, c;
            quad_rc(g, r, c);
            // partial t in split order: this split's from LDS, else buf[t] (t < s)
            // or buf[t - 1] (t > s)
            const f32x4 own = staged_quad(stg, r, c);
            f32x4 sum = s == 0 ? own : buf[0][g];
            if (S > 1) sum += s == 1 ? own : (s > 1 ? buf[1][g] : buf[0][g]);
            if (S > 2) sum += s == 2 ? own : (s > 2 ? buf[2][g] : buf[1][g]);
            if (S > 3) sum += s == 3 ? own : buf[2][g];
            res[g] = sum;
        }
      } else {
#pragma unroll
        for (int q0 = 0; q0 < QPT; q0 += 4) {
            f32x4 sum[4];
            for (int t0 = 0; t0 < S; t0 += 4) {
                f32x4 buf[4][4];
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int t = t0 + tt;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        int r, c;
                        quad_rc(q0 + g, r, c);
                        buf[tt][g] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (t < S && t != s && in_c(r, c)) buf[tt][g] = get4(t, r, c);
                    }
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    const int t = t0 + tt;
                    if (t >= S) break;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        int r, c;
                        quad_rc(q0 + g, r, c);
                        const f32x4 x = (t == s) ? staged_quad(stg, r, c) : buf[tt][g];
                        sum[g] = (t == 0) ? x : sum[g] + x;
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) res[q0 + g] = sum[g];
        }
      }
      store_quads_final<NW, QPT>(p, m0, n0, res);
    }
    for (int t = 0; t < S; ++t) trace_folded(p, tile, t, tile * S + t);
    clk.mark(p, 2);
    clk.done(p);
}

// ---------------------------------------------------------------------------
// Two-pass Split-K, second pass ("serial" Split-K: a separate reduction over the
// partials; CUTLASS optimisation guide, "Parallelized Reductions (Split-K)").
// One thread per 16-byte quad of C, 16 workgroups of 256 threads per tile; the
// partials are added in split order, ((P0 + P1) + P2) + ..., the loads of up to
// 8 partials in flight before their adds -- the same order, hence the same
// bits, as the in-launch fold.
// ---------------------------------------------------------------------------
constexpr int RED_THREADS = 256;
// workgroups per tile of tm rows: 16 for 128-row tiles
__host__ __device__ constexpr int red_blocks_per_tile(int tm) { return tm * BN / 4 / RED_THREADS; }

template <bool EPI, bool GRP = false>
__global__ __launch_bounds__(RED_THREADS) void splitk_reduce(KParams p0) {
    const int bpt = red_blocks_per_tile(p0.tm);
    const int tile = blockIdx.x / bpt;
    const int q = (blockIdx.x % bpt) * RED_THREADS + threadIdx.x;   // quad within the tile
    int m0, n0;
    const KParams p = tile_view<GRP>(p0, tile, m0, n0);   // the tile's batch entry
    const int r = q >> 5, c = (q & 31) * 4;
    const int S = p.splits;
    if (threadIdx.x == 0 && blockIdx.x % bpt == 0)
        for (int t = 0; t < S; ++t) trace_folded(p, tile, t, tile * S + t);
    if (m0 + r >= p.M || n0 + c >= p.N) return;
    const size_t mn = (size_t)p.M * p.N;
    const size_t off = (size_t)(m0 + r) * p.N + n0 + c;
    if ((p.N & 3) == 0) {
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
        for (int t0 = 0; t0 < S; t0 += 8) {
            f32x4 x[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (t0 + j < S) x[j] = *reinterpret_cast<const f32x4 *>(p.part + (size_t)(t0 + j) * mn + off);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (t0 + j < S) sum = t0 + j == 0 ? x[j] : sum + x[j];
        }
        if (EPI) {
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const f32x4 cq = reads_c(p) ? *reinterpret_cast<const f32x4 *>(p.C + off) : zero;
            const f32x4 bq = p.bias ? *reinterpret_cast<const f32x4 *>(p.bias + n0 + c) : zero;
            float v[4] = {sum[0], sum[1], sum[2], sum[3]};
            const float cin[4] = {cq[0], cq[1], cq[2], cq[3]}, bv[4] = {bq[0], bq[1], bq[2], bq[3]};
            finish<4>(p, v, cin, bv);
            sum = f32x4{v[0], v[1], v[2], v[3]};
        }
        __builtin_nontemporal_store(sum, reinterpret_cast<f32x4 *>(p.C + off));
    } else {
        for (int e = 0; e < 4 && n0 + c + e < p.N; ++e) {
            float sum = 0.f;
            for (int t = 0; t < S; ++t) {
                const float v = p.part[(size_t)t * mn + off + e];
                sum = t == 0 ? v : sum + v;
            }
            p.C[off + e] = EPI ? final_scalar(p, sum, off + e, n0 + c + e) : sum;
        }
    }
}

// ---------------------------------------------------------------------------
// Two-pass Stream-K, second pass (the book chapter's Case 3 design: a separate
// fixup kernel that sums each split tile's partials in k order).  The owner of
// tile T (the unit holding its k = 0 iteration) published its segment into the
// second slot bank, the next units their first segments into the first bank;
// C = ((owner + peer 1) + peer 2) + ..., the turnstile's order, so the bits are
// the turnstile's.  Slots are in register-native order: 16-byte element f =
// ((quad * BPQ + b) * 4 + e4) * 64 + lane (BPQ = tm / 32 blocks of 32 x 32 per
// wave quadrant) holds rows r..r+3 of one column.  One thread per such element,
// tm / 8 workgroups of 256 threads per Stream-K tile; tiles that one unit
// computed whole were stored by it and are skipped.
// ---------------------------------------------------------------------------
template <bool EPI, bool GRP = false>
__global__ __launch_bounds__(RED_THREADS) void streamk_reduce(KParams p) {
    const int bpt = red_blocks_per_tile(p.tm);
    const int slot = p.tm * BN;                 // floats of one partial slot
    const int ts = blockIdx.x / bpt;
    const int f = (blockIdx.x % bpt) * RED_THREADS + threadIdx.x;
    const int tb = ts * p.ipt, tile_end = tb + p.ipt;
    const int owner = unit_of(p, tb);
    if (unit_start(owner, p.q, p.big) + p.q + (owner < p.big ? 1 : 0) >= tile_end) return;   // whole tile
    int vend = owner + 1;
    while (vend < p.units && unit_start(vend, p.q, p.big) < tile_end) ++vend;
    const int tile = p.tile_base + ts;
    if (f == 0) {
        trace_folded(p, tile, 0, owner);
        for (int v = owner + 1; v < vend; ++v) trace_folded(p, tile, v - owner, v);
    }
    const f32x4 *own = reinterpret_cast<const f32x4 *>(p.part + ((size_t)p.units + owner) * slot);
    const f32x4 *first = reinterpret_cast<const f32x4 *>(p.part);
    f32x4 sum = own[f];
    for (int v0 = owner + 1; v0 < vend; v0 += 4) {
        f32x4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (v0 + j < vend) x[j] = first[(size_t)(v0 + j) * (slot / 4) + f];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (v0 + j < vend) sum += x[j];
    }
    int m0, n0;
    const KParams pv = tile_view<GRP>(p, tile, m0, n0);   // the tile's batch entry
    const int bpq = p.tm / 32;                  // 32 x 32 blocks per wave quadrant
    const int lane = f & 63, e4 = (f >> 6) & 3, b = (f >> 8) % bpq, quad = (f >> 8) / bpq;
    const int row = m0 + (quad >> 1) * (p.tm / 2) + (b >> 1) * 32 + 8 * e4 + 4 * (lane >> 5);
    const int col = n0 + (quad & 1) * 64 + (b & 1) * 32 + (lane & 31);
    if (col >= pv.N) return;
    if (EPI) {
        const bool rc = reads_c(p);
        const float b = p.bias ? p.bias[col] : 0.0f;
        float v[4], cin[4];
        const float bv[4] = {b, b, b, b};
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            cin[y] = (rc && row + y < pv.M) ? pv.C[(size_t)(row + y) * pv.N + col] : 0.0f;
            v[y] = sum[y];
        }
        finish<4>(p, v, cin, bv);
#pragma unroll
        for (int y = 0; y < 4; ++y) sum[y] = v[y];
    }
#pragma unroll
    for (int y = 0; y < 4; ++y)
        if (row + y < pv.M) __builtin_nontemporal_store(sum[y], pv.C + (size_t)(row + y) * pv.N + col);
}

// ---------------------------------------------------------------------------
// Stream-K: persistent; workgroup b runs unit worker_of(b).
//
// A unit's range [begin, end) of the flattened (tile, k) space falls into
// segments at tile edges (book chapter, Stream-K paragraph): a first segment
// that may start mid-tile (a contributor: it publishes its partial), whole
// tiles (stored directly) and a last segment that may hold k = 0 of a tile and
// end mid-tile (its owner: it adds the next units' partials in k order and
// stores the tile).  Segments run in range order; every unit publishes before
// it waits, so all waits end.
//
// MAC iteration k of tile T reads K-slab (k + rot_T) mod ipt, where rot_T is
// the number of iterations T's owner (the unit holding k = 0) computes before
// reaching T.  This is a bijection on each tile's slabs, so every tile still
// sums all of K exactly once, in the fixed fold order.  Its effect: an owner
// or a whole tile reads slab (step mod ipt) at each step of its unit, and a
// first segment that starts mid-tile reads slab ((step + q) mod ipt), so all
// units stream the same few K-slabs at any moment and the A and B panels
// shared by neighbouring tiles are reused from the XCD's L2.
// ---------------------------------------------------------------------------
template <int DT, int BL, int NS, int NW, bool ATOMIC, bool EPI, int TM = 128, bool GRP = false>
__global__ __launch_bounds__(64 * NW) void gemm_streamk(KParams p) {
    constexpr int SLOT = TM * BN;              // floats of one partial slot
    // turnstile owners load their first peer's partial before the k-half merge
    // (not in the epilogue build, whose C prefetch holds those registers, nor for
    // 256-row tiles, whose accumulators fill them)
    constexpr bool EARLY = !EPI && !ATOMIC && TM <= 128;
    __shared__ __attribute__((aligned(16))) char lds[lds_bytes<TM>(NS)];
    const WgClock clk(p);
    const int u = worker_of(p);
    const int ipt = p.ipt;
    const int begin = unit_start(u, p.q, p.big);
    const int end = begin + p.q + (u < p.big ? 1 : 0);
    // Hybrid: the units first run the data-parallel tiles [0, dp_tiles), unit u
    // the tiles u, u + units, ... (whole K, stored directly; traced as the DP
    // workers units + tile), then their Stream-K ranges over the last tiles.
    for (int tile = u; tile < p.dp_tiles; tile += p.units) {
        int m0, n0;
        const KParams pv = tile_view<GRP>(p, tile, m0, n0);
        AccT<TM> acc;
        zero_acc(acc);
        mac_loop<DT, BL, NS, NW, TM>(pv, lds, m0, n0, 0, ipt, 0, acc, p.trace ? trace_cov(p, tile) : nullptr);
        const Tile<NW, TM> t = merge_k_halves<NW, TM>(acc, lds);
        trace_segment(p, p.units + tile, 0, tile, 0, ipt, 0);
        store_final<NW, EPI>(pv, m0, n0, t);
        trace_folded(p, tile, 0, p.units + tile);
    }
    int nseg = 0;
    uint32_t *pending = nullptr;   // a published partial whose flag rises in the next segment's loop
    for (int pos = begin; pos < end;) {
        const int ts = fdiv(pos, p.d_ipt);       // tile index within the Stream-K part
        const int tb = ts * ipt;
        const int k0 = pos - tb;
        const int k1 = min(end - tb, ipt);
        const int tile = p.tile_base + ts;
        int m0, n0;
        const KParams pv = tile_view<GRP>(p, tile, m0, n0);   // the tile's batch entry
        const int role = k0 > 0 ? 2 : (k1 == ipt ? 0 : 1);
        const int owner = unit_of(p, tb);
        const int since = tb - unit_start(owner, p.q, p.big);   // the owner's iterations before this tile
        const int rot = since - fdiv(since, p.d_ipt) * ipt;
        // a turnstile owner's first peer is always unit u + 1, which published
        // its partial at the end of its first segment, usually long before this
        // owner's segment ends
        const bool turnstile_owner = role == 1 && !ATOMIC && p.merge != MERGE_TWO_PASS;
        uint32_t first_flag = 0;
        AccT<TM> acc;
        zero_acc(acc);
        // EARLY: every wave reads that flag during the mainloop; if it is already
        // up there, the wave's loads of the peer's partial go out right after the
        // loop and land during the k-half merge
        mac_loop<DT, BL, NS, NW, TM>(pv, lds, m0, n0, k0, k1, rot, acc, p.trace ? trace_cov(p, tile) : nullptr,
                                     pending, EARLY && turnstile_owner ? p.flags + u + 1 : nullptr, &first_flag);
        pending = nullptr;
        // a segment that stores C: with the epilogue, its inputs are loaded now,
        // while the k-halves merge and any peers are waited for and added
        const bool stores_c = role == 0 || (role == 1 && !ATOMIC && p.merge != MERGE_TWO_PASS);
        // otherwise thread 0 reads the flag now, its latency hidden behind the
        // k-half merge
        if (!EARLY && turnstile_owner && threadIdx.x == 0) first_flag = load_flag_async(p.flags + u + 1);
        SlotPart<NW, TM> early_part;
        bool early = false;
        if constexpr (EARLY) {
            if (turnstile_owner) {
                // the loop's last wait covered the flag's load; the same value in
                // every lane of the wave
                early = __builtin_amdgcn_readfirstlane(flag_value(first_flag)) == p.epoch;
                if (early) load_slot<NW, TM>(p.part + (size_t)(u + 1) * SLOT, early_part);
            }
        }
        // (128-row tiles; 64- and 256-row tiles load them when they store)
        float pre_c[32], pre_b[2];
        if constexpr (EPI && TM == 128) {
            static_assert(NW == 8, "the prefetch assumes one 32-row block per wave");
            if (stores_c && p.epi != EPI_PLAIN) epi_prefetch(pv, m0, n0, pre_c, pre_b);
        }
        Tile<NW, TM> t = merge_k_halves<NW, TM>(acc, lds);
        clk.mark(p, 2 * min(nseg, 1));
        trace_segment(p, u, nseg++, tile, k0, k1, role);
        if (role == 0) {
            if constexpr (!EPI) store_final<NW, false>(pv, m0, n0, t);
            trace_folded(p, tile, 0, u);
        } else if constexpr (ATOMIC) {
            atomic_add_c<NW, EPI>(pv, m0, n0, t);
        } else if (p.merge == MERGE_TWO_PASS) {
            // streamk_reduce adds the tile's partials: contributors publish into
            // the first slot bank, owners into the second
            put_slot<NW>(p.part + ((size_t)(role == 1 ? p.units : 0) + u) * SLOT, t, zero_partials(p));
        } else if (role == 2) {
            // starts mid-tile: publish the partial, then the flag -- at once if
            // this is the unit's last segment, else from the next segment's loop
            // as soon as the stores are known complete (the loop has to wait for
            // its first loads anyway)
            put_slot<NW>(p.part + (size_t)u * SLOT, t, zero_partials(p));
            uint32_t *flag = (p.debug & GEMM_DEBUG_NO_PUBLISH) ? nullptr : p.flags + u;
            if (tb + k1 < end) {
                pending = flag;
            } else {
                wait_vm_all();             // this wave's partial stores are complete
                __syncthreads();           // ... and every other wave's
                if (flag && threadIdx.x == 0)
                    __hip_atomic_store(flag, p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            // holds k = 0 of a split tile: fold the next units' partials in k order
            trace_folded(p, tile, 0, u);
            const int tile_end = tb + ipt;
            int pos_fold = 1;
            for (int v = u + 1; v < p.units; ++v) {
                if (unit_start(v, p.q, p.big) >= tile_end) break;
                if (threadIdx.x == 0) {
                    if (v == u + 1) wait_flag_issued(p.flags + v, first_flag, p.epoch, p.spin_limit, p.status);
                    else wait_flag(p.flags + v, p.epoch, p.spin_limit, p.status);
                    // each flag has this one reader: clear it once seen, so every
                    // call starts with the flags at zero, also the replays of a
                    // captured graph, whose epoch is fixed at capture
                    __hip_atomic_store(p.flags + v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                __syncthreads();
                if (EARLY && v == u + 1 && early) add_part(t, early_part);
                else add_slot<NW>(p.part + (size_t)v * SLOT, t);
                trace_folded(p, tile, pos_fold++, v);
            }
            if constexpr (!EPI) store_final<NW, false>(pv, m0, n0, t);
        }
        // the epilogue build stores whole tiles and folded tiles from one call
        // site (one inlined copy of the epilogue code)
        if constexpr (EPI) {
            if (stores_c) {
                if constexpr (TM == 128) {
                    if (p.epi == EPI_PLAIN) store_tile<NW>(pv.C, m0, n0, pv.M, pv.N, t);
                    else finish_block<NW>(pv, m0, n0, t, 0, pre_c, pre_b);
                } else {
                    store_final<NW, true, TM>(pv, m0, n0, t);
                }
            }
        }
        clk.mark(p, 2 * min(nseg - 1, 1) + 1);
        pos = tb + k1;
    }
    clk.done(p);
}

// ---------------------------------------------------------------------------
// Elementwise epilogue pass over C, every batch entry (atomic merges and the
// empty sum):
// EPASS_PRE  C = beta C + bias (C not read when beta == 0),
// EPASS_POST C = act(C),
// EPASS_ONLY C = act(beta C + bias), i.e. the epilogue of a zero product.
// Rows are spread over blockIdx.y, columns over the x grid.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void epilogue_pass(KParams p, int stage) {
#pragma clang fp contract(off)
    const bool rc = p.beta != 0.0f;
    for (int z = blockIdx.z; z < p.batch; z += gridDim.z)
    for (int row = blockIdx.y; row < p.M; row += gridDim.y)
        for (int col = blockIdx.x * blockDim.x + threadIdx.x; col < p.N; col += gridDim.x * blockDim.x) {
            float *c = p.C + (size_t)z * p.sC + (size_t)row * p.N + col;
            const float b = p.bias ? p.bias[col] : 0.0f;
            if (stage == EPASS_POST) {
                *c = act_apply(p.act, *c);
            } else if (stage == EPASS_ONLY) {
                *c = epi_value(p, 0.0f, rc ? *c : 0.0f, b);
            } else {
                const float t = rc ? p.beta * *c : 0.0f;
                *c = p.bias ? t + b : t;
            }
        }
}

// ---------------------------------------------------------------------------
// Zero fill (n 32-bit words), 16-byte stores where possible.
// ---------------------------------------------------------------------------
__global__ void put_groups(GroupDesc *dst, GroupTable t, int n) {
    const int i = threadIdx.x;
    if (i < n) dst[i] = t.g[i];
}

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
// Host-side dispatch.  The 128x128 tile kernels run 8 waves on 128 KiB of LDS
// (one workgroup per CU): 4 stages of 128x128 tiles, or 2 stages of 2x2 tile
// groups; the 256x128 tile 8 waves on 3 stages (144 KiB); the 64x128 tile 4
// waves on 3 stages (72 KiB, two workgroups per CU).
// Split-K and Stream-K share the per-segment accumulation order, so the two
// agree bit for bit whenever their segments coincide.
// ---------------------------------------------------------------------------
namespace {

typedef void (*KernelFn)(KParams);

struct Shape {
    int ns, nw;
};

// Grouped calls (problem table, no epilogue, 128- and 64-row tiles) run builds
// of their own, so the plain builds carry no table lookup.
template <int DT, int BL>
KernelFn pick_grouped(int kmode, bool epi, int tm, Shape &shape) {
    if (epi) return nullptr;
    if (tm == 64) {
        shape = {3, 4};
        switch (kmode) {
        case K_DP: return gemm_dp<DT, BL, 3, 4, 64, true>;
        case K_SPLITK: return gemm_splitk<DT, BL, 3, 4, 64, true>;
        case K_SK: return gemm_streamk<DT, BL, 3, 4, false, false, 64, true>;
        case K_SK_ATOMIC: return gemm_streamk<DT, BL, 3, 4, true, false, 64, true>;
        default: return nullptr;
        }
    }
    if (tm != 128) return nullptr;
    shape = {4, 8};
    switch (kmode) {
    case K_DP: return gemm_dp<DT, BL, 4, 8, 128, true>;
    case K_SPLITK: return gemm_splitk<DT, BL, 4, 8, 128, true>;
    case K_SK: return gemm_streamk<DT, BL, 4, 8, false, false, 128, true>;
    case K_SK_ATOMIC: return gemm_streamk<DT, BL, 4, 8, true, false, 128, true>;
    default: return nullptr;
    }
}

template <int DT, int BL>
KernelFn pick(int kmode, bool epi, int tm, Shape &shape) {
    if (tm == 256) {
        // the 256 x 128 tile: three stages of (32 KiB A + 16 KiB B), Stream-K
        // only, a separate build with the epilogue
        shape = {3, 8};
        if (kmode == K_SK)
            return epi ? gemm_streamk<DT, BL, 3, 8, false, true, 256> : gemm_streamk<DT, BL, 3, 8, false, false, 256>;
        if (kmode == K_SK_ATOMIC)
            return epi ? gemm_streamk<DT, BL, 3, 8, true, true, 256> : gemm_streamk<DT, BL, 3, 8, true, false, 256>;
        return nullptr;
    }
    if (tm == 64) {
        // the skinny 64 x 128 tile: four waves of 32 x 64 over every k-step, three
        // stages of (8 KiB A + 16 KiB B), so two workgroups share a CU; Stream-K
        // has a separate build with the epilogue, like the 128-row tile
        shape = {3, 4};
        switch (kmode) {
        case K_DP: return gemm_dp<DT, BL, 3, 4, 64>;
        case K_SPLITK: return gemm_splitk<DT, BL, 3, 4, 64>;
        case K_SK: return epi ? gemm_streamk<DT, BL, 3, 4, false, true, 64> : gemm_streamk<DT, BL, 3, 4, false, false, 64>;
        case K_SK_ATOMIC:
            return epi ? gemm_streamk<DT, BL, 3, 4, true, true, 64> : gemm_streamk<DT, BL, 3, 4, true, false, 64>;
        default: return nullptr;
        }
    }
    if (tm != 128) return nullptr;
    // Stream-K has a separate build with the epilogue: its plain build keeps
    // the register allocation of a kernel without one
    switch (kmode) {
    case K_DP: shape = {4, 8}; return gemm_dp<DT, BL, 4, 8>;
    case K_SPLITK: shape = {4, 8}; return gemm_splitk<DT, BL, 4, 8>;
    case K_SK:
        shape = {4, 8};
        return epi ? gemm_streamk<DT, BL, 4, 8, false, true> : gemm_streamk<DT, BL, 4, 8, false, false>;
    case K_SK_ATOMIC:
        shape = {4, 8};
        return epi ? gemm_streamk<DT, BL, 4, 8, true, true> : gemm_streamk<DT, BL, 4, 8, true, false>;
    case K_DP_GROUP: shape = {G_NS, G_NW}; return gemm_dp_group<DT, BL>;
    default: return nullptr;
    }
}

KernelFn kernel_for(int dtype, int blayout, int kmode, bool epi, int tm, bool grp, Shape &shape) {
    if (grp) {
        if (dtype == 0)
            return blayout == 0 ? pick_grouped<0, 0>(kmode, epi, tm, shape) : pick_grouped<0, 1>(kmode, epi, tm, shape);
        if (dtype == 1)
            return blayout == 0 ? pick_grouped<1, 0>(kmode, epi, tm, shape) : pick_grouped<1, 1>(kmode, epi, tm, shape);
        return nullptr;
    }
    if (dtype == 0) return blayout == 0 ? pick<0, 0>(kmode, epi, tm, shape) : pick<0, 1>(kmode, epi, tm, shape);
    if (dtype == 1) return blayout == 0 ? pick<1, 0>(kmode, epi, tm, shape) : pick<1, 1>(kmode, epi, tm, shape);
    return nullptr;
}

// The launch constants of the index arithmetic, for a launch of `grid` workers.
KParams with_divisors(const KParams &p, int grid) {
    KParams q = p;
    const int gm_full = p.group_m > 0 ? p.group_m : p.tiles_m;
    const int bands = gm_full > 0 ? (p.tiles_m + gm_full - 1) / gm_full : 1;
    q.d_band = fast_div(int64_t(gm_full) * p.tiles_n);
    q.d_rows = fast_div(gm_full);
    q.d_rows_last = fast_div(p.tiles_m - (bands - 1) * gm_full);
    q.d_entry = fast_div(int64_t(p.tiles_m) * p.tiles_n);
    q.d_ipt = fast_div(p.ipt);
    q.d_q = fast_div(std::max(p.q, 1));
    q.d_q1 = fast_div(int64_t(p.q) + 1);
    q.d_splits = fast_div(p.splits);
    q.spread_a = grid / 8;
    q.spread_r = grid % 8;
    return q;
}

}  // namespace

hipError_t launch_gemm(int dtype, int blayout, int kmode, int grid, const KParams &p,
                       hipStream_t stream) {
    Shape shape{0, 0};
    KernelFn fn = kernel_for(dtype, blayout, kmode, p.epi != EPI_PLAIN, p.tm, p.ngroups > 0, shape);
    if (!fn || grid <= 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * shape.nw), 0, stream, with_divisors(p, grid));
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const KParams &p, hipStream_t stream) {
    const int64_t tiles = (int64_t)std::max(p.batch, 1) * p.tiles_m * p.tiles_n;   // every batch entry's tiles
    if (tiles <= 0) return hipSuccess;
    // a separate build with the epilogue keeps the plain one's code unchanged
    const KParams q = with_divisors(p, 0);
    if (p.ngroups > 0)
        hipLaunchKernelGGL((splitk_reduce<false, true>), dim3((unsigned)(tiles * red_blocks_per_tile(p.tm))),
                           dim3(RED_THREADS), 0, stream, q);
    else if (p.epi != EPI_PLAIN)
        hipLaunchKernelGGL(splitk_reduce<true>, dim3((unsigned)(tiles * red_blocks_per_tile(p.tm))), dim3(RED_THREADS), 0,
                           stream, q);
    else
        hipLaunchKernelGGL(splitk_reduce<false>, dim3((unsigned)(tiles * red_blocks_per_tile(p.tm))), dim3(RED_THREADS), 0,
                           stream, q);
    return hipGetLastError();
}

hipError_t launch_streamk_reduce(const KParams &p, int64_t sk_tiles, hipStream_t stream) {
    if (sk_tiles <= 0) return hipSuccess;
    const KParams q = with_divisors(p, 0);
    if (p.ngroups > 0)
        hipLaunchKernelGGL((streamk_reduce<false, true>), dim3((unsigned)(sk_tiles * red_blocks_per_tile(p.tm))),
                           dim3(RED_THREADS), 0, stream, q);
    else if (p.epi != EPI_PLAIN)
        hipLaunchKernelGGL(streamk_reduce<true>, dim3((unsigned)(sk_tiles * red_blocks_per_tile(p.tm))), dim3(RED_THREADS),
                           0, stream, q);
    else
        hipLaunchKernelGGL(streamk_reduce<false>, dim3((unsigned)(sk_tiles * red_blocks_per_tile(p.tm))), dim3(RED_THREADS),
                           0, stream, q);
    return hipGetLastError();
}

hipError_t launch_epilogue_pass(const KParams &p, int stage, hipStream_t stream) {
    const int gx = (int)std::min<int64_t>((p.N + 255) / 256, 16);
    const int gy = (int)std::min<int64_t>(p.M, 4096);
    const int gz = std::max(1, std::min(p.batch, 64));
    hipLaunchKernelGGL(epilogue_pass, dim3(gx, gy, gz), dim3(256), 0, stream, p, stage);
    return hipGetLastError();
}

hipError_t launch_put_groups(GroupDesc *dst, const GroupTable &t, int n, hipStream_t stream) {
    if (n <= 0 || n > MAX_GROUPS) return hipErrorInvalidValue;
    hipLaunchKernelGGL(put_groups, dim3(1), dim3(64), 0, stream, dst, t, n);
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

hipError_t blocks_per_cu(int dtype, int blayout, int kmode, int tm, bool grp, int *out) {
    // the smaller of the builds with and without the epilogue (the grouped
    // builds have no epilogue build; for the data-parallel and Split-K kernels
    // both lookups give the one build that serves both)
    int best = 1 << 30;
    for (int epi = 0; epi < (grp ? 1 : 2); ++epi) {
        Shape shape{0, 0};
        KernelFn fn = kernel_for(dtype, blayout, kmode, epi != 0, tm, grp, shape);
        if (!fn) return hipErrorInvalidValue;
        int n = 0;
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void *>(fn),
                                                                    64 * shape.nw, 0);
        if (e != hipSuccess) return e;
        best = std::min(best, n);
    }
    *out = best;
    return hipSuccess;
}

}  // namespace dgw
