// gemm_api.hip -- the C ABI declared in include/gemm.h: argument checks,
// planning, workspace management and kernel launches.
//
// Workspace (per device, owned by the library unless the caller passes one):
//   control: a status word (64 words reserved), one flag per Stream-K unit and
//            one arrival counter per Split-K tile.  It is zero-filled when it is
//            (re)allocated and never again: flags hold the epoch of the launch
//            that last raised them (a fresh epoch per Stream-K launch, so stale
//            flags never match), and the last arriver of a tile resets its
//            counter to zero.
//   data:    Stream-K partial slots [units][128*128] fp32, or Split-K partials
//            [S][M][N] fp32.
// Both blocks only grow.  A block that is outgrown is retired, not freed: a
// graph captured earlier keeps the addresses it was captured with, so retired
// blocks stay allocated until gemm_release().  Growth needs hipMalloc and a
// synchronous fill, so it is refused on a stream that is being captured.
// A caller workspace holds [flags | counters | data] for the call's own plan
// and has its control part zero-filled by the library on every call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gemm.h"
#include "kernels.h"
#include "plan.h"

namespace {

using dgw::KParams;

thread_local std::string g_err;
thread_local hipStream_t g_stream = nullptr;

constexpr uint32_t kDefaultSpin = 1u << 22;
constexpr int64_t kStatusWords = 64;
constexpr int kGroupM = 8;   // tile rows per raster group (DGW_GROUP_M overrides)

// Tuning overrides from the environment, read once.
struct Tuning {
    int group_m = kGroupM;
    int xcd_spread = 1;
    Tuning() {
        if (const char *v = std::getenv("DGW_GROUP_M")) group_m = std::max(0, std::atoi(v));
        if (const char *v = std::getenv("DGW_XCD_SPREAD")) xcd_spread = std::atoi(v) ? 1 : 0;
    }
};
const Tuning &tuning() {
    static const Tuning t;
    return t;
}

int fail(int code, const std::string &msg) {
    g_err = msg;
    return code;
}

int fail_hip(hipError_t e, const char *what) {
    g_err = std::string(what) + ": " + hipGetErrorString(e);
    return GEMM_ERR_HIP;
}

// Workspace of gemm_ex_noalloc: one fixed array per device, laid out like a
// caller workspace ([status 256 B | flags | counters | data]).  Host code never
// names it directly: its device address comes from hipGetSymbolAddress, once
// per device (DeviceState::scratch).
static __device__ __align__(256) unsigned char scratch[GEMM_NOALLOC_MAX_BYTES];

struct DeviceState {
    bool ready = false;
    unsigned char *scratch = nullptr;   // this device's copy of `scratch` (its device address)
    int num_cus = 0;
    uint32_t *control = nullptr;   // status words, then flags[cap_units], then counters[cap_tiles]
    int64_t cap_units = 0, cap_tiles = 0;
    void *data = nullptr;
    int64_t cap_data = 0;
    std::vector<void *> retired;   // outgrown data blocks, freed by gemm_release()
    std::vector<uint32_t *> retired_control;   // outgrown control blocks (status word first)
    int bpc[2][2][5][3][2] = {};   // resident workgroups per CU [dtype][B layout][kind][tile shape][grouped], 0 = not queried
};

std::mutex g_mu;
std::vector<DeviceState> g_dev;
std::atomic<uint32_t> g_epoch{0};

uint32_t next_epoch() {
    uint32_t e;
    do {
        e = g_epoch.fetch_add(1) + 1;
    } while (e == 0);
    return e;
}

// Returns the state of `dev`, creating it (and its status word) on first use.
int device_state(int dev, DeviceState **out) {
    if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
    DeviceState &d = g_dev[dev];
    if (!d.ready) {
        int n = 0;
        hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute(multiProcessorCount)");
        d.num_cus = n;
        d.ready = true;
    }
    *out = &d;
    return GEMM_OK;
}

// GEMM_OK when `stream` is not being captured into a graph, else a
// GEMM_ERR_WORKSPACE refusal naming `what`.
int refuse_if_capturing(hipStream_t stream, const char *what) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) return fail_hip(e, "hipStreamIsCapturing");
    if (cs != hipStreamCaptureStatusNone)
        return fail(GEMM_ERR_WORKSPACE, std::string("the library workspace must grow (") + what +
                                            ") while the stream is being captured; make one eager call "
                                            "with the same plan first, or pass a caller workspace");
    return GEMM_OK;
}

// Make sure the library control block covers `units` flags and `tiles` counters.
// An outgrown block is retired (still allocated), never freed here.
int ensure_control(DeviceState &d, int64_t units, int64_t tiles, hipStream_t stream) {
    if (d.control && units <= d.cap_units && tiles <= d.cap_tiles) return GEMM_OK;
    int rc = refuse_if_capturing(stream, "control block");
    if (rc != GEMM_OK) return rc;
    const int64_t cu = std::max<int64_t>({units, d.cap_units, 1024});
    const int64_t ct = std::max<int64_t>({tiles, d.cap_tiles, 4096});
    const size_t bytes = (size_t)(kStatusWords + cu + ct) * 4;
    uint32_t *fresh = nullptr;
    hipError_t e;
    if ((e = hipMalloc(&fresh, bytes)) != hipSuccess)
        return fail(GEMM_ERR_WORKSPACE, std::string("hipMalloc(control): ") + hipGetErrorString(e));
    if ((e = hipMemset(fresh, 0, bytes)) != hipSuccess) {
        (void)hipFree(fresh);
        return fail_hip(e, "hipMemset(control)");
    }
    // a retired block keeps its status word, which gemm_sync_status still reads
    if (d.control) d.retired_control.push_back(d.control);
    d.control = fresh;
    d.cap_units = cu;
    d.cap_tiles = ct;
    return GEMM_OK;
}

int ensure_data(DeviceState &d, int64_t bytes, hipStream_t stream) {
    if (bytes <= d.cap_data) return GEMM_OK;
    int rc = refuse_if_capturing(stream, "data block");
    if (rc != GEMM_OK) return rc;
    void *fresh = nullptr;
    hipError_t e;
    if ((e = hipMalloc(&fresh, (size_t)bytes)) != hipSuccess)
        return fail(GEMM_ERR_WORKSPACE, std::string("hipMalloc(workspace): ") + hipGetErrorString(e));
    if (d.data) d.retired.push_back(d.data);
    d.data = fresh;
    d.cap_data = bytes;
    return GEMM_OK;
}

// The device address of this device's `scratch` array, looked up the first time
// gemm_ex_noalloc runs on the device (the device is current); its status words
// are cleared then, on the call's stream (a kernel, so a captured first call
// records no memset).
int scratch_setup(DeviceState &d, hipStream_t stream) {
    if (d.scratch) return GEMM_OK;
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail_hip(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(GEMM_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
    if ((e = dgw::launch_zero(ptr, kStatusWords, stream)) != hipSuccess) return fail_hip(e, "zero scratch status");
    d.scratch = static_cast<unsigned char *>(ptr);
    return GEMM_OK;
}

int scratch_too_small(const gemm_plan_t &p) {
    return fail(GEMM_ERR_WORKSPACE, "the call needs " + std::to_string(p.workspace_bytes) +
                                        " workspace bytes; gemm_ex_noalloc holds at most " +
                                        std::to_string((int64_t)GEMM_NOALLOC_MAX_BYTES));
}

bool overlaps(const void *a, int64_t abytes, const void *b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

// Host-detectable problems with the operands (no HIP call).
int check_operands(const gemm_args_t &a) {
    // with K == 0 the operands are empty and never read, so they may be null
    if (!a.C || (a.K > 0 && (!a.A || !a.B)))
        return fail(GEMM_ERR_INVALID, "A, B and C must be non-null");
    const uintptr_t mis = (reinterpret_cast<uintptr_t>(a.A) | reinterpret_cast<uintptr_t>(a.B) |
                           reinterpret_cast<uintptr_t>(a.C)) & 15;
    if (mis) return fail(GEMM_ERR_UNSUPPORTED, "A, B and C must be 16-byte aligned");
    const int64_t batch = a.batch > 1 ? a.batch : 1;
    if (batch > 1) {
        if (a.stride_a < 0 || a.stride_b < 0 || a.stride_c < a.M * a.N)
            return fail(GEMM_ERR_INVALID, "batch strides: stride_a, stride_b >= 0 and stride_c >= M*N");
        if ((a.stride_a & 7) || (a.stride_b & 7) || (a.stride_c & 3))
            return fail(GEMM_ERR_UNSUPPORTED, "batch strides must keep 16-byte alignment "
                                              "(stride_a, stride_b multiples of 8, stride_c of 4)");
    }
    // byte extents of all batch entries (a zero stride shares one matrix)
    const int64_t sa = batch > 1 ? a.stride_a : 0, sb = batch > 1 ? a.stride_b : 0, sc = batch > 1 ? a.stride_c : 0;
    const int64_t cb = ((batch - 1) * sc + a.M * a.N) * 4, ab = ((batch - 1) * sa + a.M * a.K) * 2,
                  bb = ((batch - 1) * sb + a.K * a.N) * 2;
    if (overlaps(a.C, cb, a.A, ab) || overlaps(a.C, cb, a.B, bb))
        return fail(GEMM_ERR_INVALID, "C must not overlap A or B");
    if (a.trace && a.trace_ints <= 0) return fail(GEMM_ERR_INVALID, "trace_ints must be > 0");
    if (a.epilogue & GEMM_EPI_BIAS) {
        if (reinterpret_cast<uintptr_t>(a.bias) & 15) return fail(GEMM_ERR_UNSUPPORTED, "bias must be 16-byte aligned");
        if (overlaps(a.C, cb, a.bias, a.N * 4)) return fail(GEMM_ERR_INVALID, "bias must not overlap C");
    }
    if (a.workspace && reinterpret_cast<uintptr_t>(a.workspace) & 255)
        return fail(GEMM_ERR_INVALID, "a caller workspace must be 256-byte aligned");
    return GEMM_OK;
}

// Epilogue word and its operands (no HIP call).
int check_epilogue(const gemm_args_t &a) {
    const uint32_t known = GEMM_EPI_ALPHA_BETA | GEMM_EPI_BIAS | GEMM_EPI_RELU | GEMM_EPI_GELU;
    if (a.epilogue & ~known) return fail(GEMM_ERR_INVALID, "epilogue word has unknown bits");
    if ((a.epilogue & GEMM_EPI_RELU) && (a.epilogue & GEMM_EPI_GELU))
        return fail(GEMM_ERR_INVALID, "GEMM_EPI_RELU and GEMM_EPI_GELU exclude each other");
    if (((a.epilogue & GEMM_EPI_BIAS) != 0) != (a.bias != nullptr))
        return fail(GEMM_ERR_INVALID, "bias must be given exactly when GEMM_EPI_BIAS is set");
    return GEMM_OK;
}

// Fill the epilogue fields of `kp` for the final stores of a deterministic
// launch (EPI_FULL) or of the launches around atomic merges (EPI_ACCUM).
void set_epilogue(const gemm_args_t &a, bool accum, KParams &kp) {
    const bool ab = (a.epilogue & GEMM_EPI_ALPHA_BETA) != 0;
    kp.alpha = ab ? a.alpha : 1.0f;
    kp.beta = ab ? a.beta : 0.0f;
    kp.bias = (a.epilogue & GEMM_EPI_BIAS) ? a.bias : nullptr;
    kp.act = (a.epilogue & GEMM_EPI_RELU) ? dgw::ACT_RELU : (a.epilogue & GEMM_EPI_GELU) ? dgw::ACT_GELU : dgw::ACT_NONE;
    kp.epi = a.epilogue == 0 ? dgw::EPI_PLAIN : accum ? dgw::EPI_ACCUM : dgw::EPI_FULL;
}

// C := 0 in every batch entry (what lies between entries is not touched).
hipError_t zero_c(const gemm_args_t &a, int64_t batch, hipStream_t stream) {
    if (batch == 1 || a.stride_c == a.M * a.N) return dgw::launch_zero(a.C, batch * a.M * a.N, stream);
    KParams z;
    std::memset(&z, 0, sizeof z);
    z.C = a.C;
    z.M = (int)a.M;
    z.N = (int)a.N;
    z.batch = (int)batch;
    z.sC = a.stride_c;
    z.alpha = 1.0f;   // EPASS_PRE with beta = 0 and no bias writes zeros
    return dgw::launch_epilogue_pass(z, dgw::EPASS_PRE, stream);
}

struct TraceHeader {
    int v[8];
};

__global__ void put_trace_header(int *t, TraceHeader h) {
    if (threadIdx.x < 8) t[threadIdx.x] = h.v[threadIdx.x];
}

// The problems of a grouped call (no HIP call): the common arguments carry no
// problem of their own, every problem's operands are aligned and C does not
// overlap its A or B.
int check_groups(const gemm_args_t &a, const gemm_group_t *groups, int32_t count) {
    if (a.A || a.B || a.C || a.M || a.N || a.bias || a.batch > 1)
        return fail(GEMM_ERR_INVALID, "a grouped call's common arguments must leave A, B, C, M, N, bias and batch unset");
    if (a.epilogue) return fail(GEMM_ERR_UNSUPPORTED, "grouped calls have no fused epilogue");
    for (int32_t g = 0; g < count; ++g) {
        const gemm_group_t &x = groups[g];
        if (x.M == 0 || x.N == 0) continue;
        if (!x.C || (a.K > 0 && (!x.A || !x.B)))
            return fail(GEMM_ERR_INVALID, "problem " + std::to_string(g) + ": A, B and C must be non-null");
        if ((reinterpret_cast<uintptr_t>(x.A) | reinterpret_cast<uintptr_t>(x.B) | reinterpret_cast<uintptr_t>(x.C)) & 15)
            return fail(GEMM_ERR_UNSUPPORTED, "problem " + std::to_string(g) + ": A, B and C must be 16-byte aligned");
        if (overlaps(x.C, x.M * x.N * 4, x.A, x.M * a.K * 2) || overlaps(x.C, x.M * x.N * 4, x.B, a.K * x.N * 2))
            return fail(GEMM_ERR_INVALID, "problem " + std::to_string(g) + ": C must not overlap A or B");
    }
    if (a.trace && a.trace_ints <= 0) return fail(GEMM_ERR_INVALID, "trace_ints must be > 0");
    if (a.workspace && reinterpret_cast<uintptr_t>(a.workspace) & 255)
        return fail(GEMM_ERR_INVALID, "a caller workspace must be 256-byte aligned");
    return GEMM_OK;
}

// One call.  noalloc: the workspace is this device's `scratch` array and no
// device memory is allocated (gemm_ex_noalloc).  groups / ngroups: a grouped
// call (gemm_grouped), whose problems replace a's A, B, C, M and N.
int run(const gemm_args_t &a, bool noalloc = false, const gemm_group_t *groups = nullptr, int32_t ngroups = 0) {
    g_err.clear();
    gemm_plan_t p;
    const char *why = "";
    // plan first with a placeholder CU count so argument errors surface before any HIP call
    const int64_t batch = a.batch > 1 ? a.batch : 1;
    auto plan_for = [&](int32_t cus) {
        return groups ? dgw::make_plan_grouped(groups, ngroups, a.K, a.layout, a.mode, a.splits, cus, &p, &why)
                      : dgw::make_plan(a.M, a.N, a.K, batch, a.layout, a.mode, a.splits, cus, &p, &why);
    };
    int rc = plan_for(a.num_cus > 0 ? a.num_cus : 256);
    if (rc != GEMM_OK) return fail(rc, why);
    if (a.num_cus < 0) return fail(GEMM_ERR_INVALID, "num_cus must be >= 0");
    if ((a.debug & ~(GEMM_DEBUG_NO_PUBLISH | GEMM_DEBUG_IN_LAUNCH | GEMM_DEBUG_TILE_DP | GEMM_DEBUG_HYBRID_SPLIT |
                    GEMM_DEBUG_ZERO_PARTIAL | GEMM_DEBUG_SPLITK_BANDS)) != 0)
        return fail(GEMM_ERR_INVALID, "unknown debug bits");
    if ((rc = check_epilogue(a)) != GEMM_OK) return rc;
    if (groups) {
        if ((rc = check_groups(a, groups, ngroups)) != GEMM_OK) return rc;
        if (p.tiles == 0) return GEMM_OK;
    } else {
        if (a.M == 0 || a.N == 0) return GEMM_OK;
        if ((rc = check_operands(a)) != GEMM_OK) return rc;
    }
    if (noalloc) {
        if (a.workspace) return fail(GEMM_ERR_INVALID, "gemm_ex_noalloc uses its own scratch: workspace must be NULL");
        // with an explicit CU count this plan is final: refuse before any HIP call
        if (a.num_cus > 0 && p.workspace_bytes > (int64_t)GEMM_NOALLOC_MAX_BYTES) return scratch_too_small(p);
    }

    hipStream_t stream = a.stream ? reinterpret_cast<hipStream_t>(a.stream) : g_stream;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");

    std::lock_guard<std::mutex> lock(g_mu);
    DeviceState *ds = nullptr;
    if ((rc = device_state(dev, &ds)) != GEMM_OK) return rc;
    const int ncu = a.num_cus > 0 ? a.num_cus : ds->num_cus;
    if ((rc = plan_for(ncu)) != GEMM_OK) return fail(rc, why);
    if (noalloc && p.workspace_bytes > (int64_t)GEMM_NOALLOC_MAX_BYTES) return scratch_too_small(p);

    const int dtype = (a.layout & 0xF0u) == GEMM_FP16 ? 1 : 0;
    const int blayout = (a.layout & 0xFu) == GEMM_B_NK ? 1 : 0;
    // tile shape: 0 = 128 x 128, 1 = 256 x 128, 2 = 64 x 128
    const int shape = p.bm == GEMM_BM ? 0 : (p.bm > GEMM_BM ? 1 : 2);

    if (a.K == 0 && groups) {   // the empty sums: every problem's C := 0
        for (int32_t g = 0; g < ngroups; ++g)
            if (groups[g].M > 0 && groups[g].N > 0 &&
                (e = dgw::launch_zero(groups[g].C, groups[g].M * groups[g].N, stream)) != hipSuccess)
                return fail_hip(e, "zero C");
        return GEMM_OK;
    }
    if (a.K == 0) {  // the empty sum
        if (a.epilogue == 0) {
            if ((e = zero_c(a, batch, stream)) != hipSuccess) return fail_hip(e, "zero C");
        } else {
            KParams ep;
            std::memset(&ep, 0, sizeof ep);
            ep.C = a.C;
            ep.M = (int)a.M;
            ep.N = (int)a.N;
            ep.batch = (int)batch;
            ep.sC = batch > 1 ? a.stride_c : 0;
            set_epilogue(a, false, ep);
            if ((e = dgw::launch_epilogue_pass(ep, dgw::EPASS_ONLY, stream)) != hipSuccess)
                return fail_hip(e, "epilogue of an empty sum");
        }
        return GEMM_OK;
    }

    const int kmode = p.decision == GEMM_DP       ? dgw::K_DP
                      : p.decision == GEMM_SPLITK ? dgw::K_SPLITK
                      : p.atomic                  ? dgw::K_SK_ATOMIC
                                                  : dgw::K_SK;
    if (p.decision == GEMM_STREAMK) {
        // every unit must be resident at once: owners wait for higher units
        int &bpc = ds->bpc[dtype][blayout][kmode][shape][ngroups > 0];
        if (bpc == 0) {
            if ((e = dgw::blocks_per_cu(dtype, blayout, kmode, p.bm, ngroups > 0, &bpc)) != hipSuccess)
                return fail_hip(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
        }
        if (p.sk_units > (int64_t)bpc * ds->num_cus)
            return fail(GEMM_ERR_UNSUPPORTED, "Stream-K units exceed the resident workgroup capacity (" +
                                                  std::to_string((int64_t)bpc * ds->num_cus) + ")");
    }

    // the status word lives in the library's control block (the scratch array's
    // first words for gemm_ex_noalloc); its flags and counters are used only
    // without a caller workspace
    if (noalloc) {
        if ((rc = scratch_setup(*ds, stream)) != GEMM_OK) return rc;
    } else if ((rc = a.workspace ? ensure_control(*ds, 1, 1, stream)
                                 : ensure_control(*ds, std::max<int64_t>(p.sk_units, 1), p.tiles, stream)) !=
               GEMM_OK) {
        return rc;
    }

    // flags, counters and the data region
    uint32_t *flags = nullptr, *counters = nullptr;
    float *part = nullptr;
    const int64_t data_bytes = p.workspace_bytes - dgw::control_bytes(p);
    if (a.workspace || noalloc) {
        if (a.workspace && (int64_t)a.workspace_bytes < p.workspace_bytes)
            return fail(GEMM_ERR_WORKSPACE, "caller workspace is smaller than plan.workspace_bytes (" +
                                                std::to_string(p.workspace_bytes) + ")");
        const int64_t cb = dgw::control_bytes(p);
        char *base = noalloc ? reinterpret_cast<char *>(ds->scratch) : static_cast<char *>(a.workspace);
        flags = reinterpret_cast<uint32_t *>(base + 256);
        counters = reinterpret_cast<uint32_t *>(base + 256 + (std::max<int64_t>(p.sk_units, 1) * 4 + 255) / 256 * 256);
        part = reinterpret_cast<float *>(base + cb);
        // flags and counters start every call at zero (the scratch array keeps the
        // last call's contents); the scratch status words stay until
        // gemm_sync_status reads and clears them
        const int64_t skip = noalloc ? 256 : 0;
        if ((e = dgw::launch_zero(base + skip, (cb - skip) / 4, stream)) != hipSuccess)
            return fail_hip(e, "zero control");
    } else {
        if ((rc = ensure_data(*ds, data_bytes, stream)) != GEMM_OK) return rc;
        flags = ds->control + kStatusWords;
        counters = flags + ds->cap_units;
        part = static_cast<float *>(ds->data);
    }

    // a grouped call's problem table, at the end of the data region: nonempty
    // problems in call order, their first tile ids and the offsets of their
    // Split-K partials [S][M_g][N_g]
    dgw::GroupDesc *table = nullptr;
    int32_t nonempty = 0;
    bool all_n4 = (a.N & 3) == 0;
    if (groups) {
        static_assert(sizeof(dgw::GroupTable) <= 3200, "the table travels as kernel arguments");
        dgw::GroupTable t;
        std::memset(&t, 0, sizeof t);
        const int64_t bm = p.bm, splits_kept = p.decision == GEMM_SPLITK && !p.atomic ? p.splits : 0;
        int64_t tile0 = 0, part_off = 0;
        for (int32_t g = 0; g < ngroups; ++g) {
            const gemm_group_t &x = groups[g];
            if (x.M == 0 || x.N == 0) continue;
            dgw::GroupDesc &d = t.g[nonempty++];
            d.A = static_cast<const uint16_t *>(x.A);
            d.B = static_cast<const uint16_t *>(x.B);
            d.C = x.C;
            d.part = part_off;
            d.M = (int)x.M;
            d.N = (int)x.N;
            d.tile0 = (int)tile0;
            tile0 += (x.M + bm - 1) / bm * ((x.N + GEMM_BN - 1) / GEMM_BN);
            part_off += splits_kept * x.M * x.N;
            all_n4 = all_n4 && (x.N & 3) == 0;
        }
        table = reinterpret_cast<dgw::GroupDesc *>(reinterpret_cast<char *>(part) + data_bytes -
                                                   dgw::group_table_bytes(ngroups));
        if ((e = dgw::launch_put_groups(table, t, nonempty, stream)) != hipSuccess)
            return fail_hip(e, "write the problem table");
    }

    KParams kp;
    std::memset(&kp, 0, sizeof kp);
    kp.A = static_cast<const uint16_t *>(a.A);
    kp.B = static_cast<const uint16_t *>(a.B);
    kp.C = a.C;
    kp.M = (int)a.M;
    kp.N = (int)a.N;
    kp.K = (int)a.K;
    kp.groups = table;
    kp.ngroups = nonempty;
    kp.tm = p.bm;
    kp.tiles_m = (int)p.tiles_m;
    kp.tiles_n = (int)p.tiles_n;
    // raster bands of group_m 128-row tile rows: the same height in rows for
    // 256- and 64-row tiles
    kp.group_m = tuning().group_m > 0 ? std::max(1, tuning().group_m * GEMM_BM / p.bm) : 0;
    kp.xcd_spread = a.unit_perm ? 0 : tuning().xcd_spread;
    kp.timing = reinterpret_cast<long long *>(a.timing);
    kp.ipt = (int)p.ipt;
    kp.splits = p.splits;
    kp.part = part;
    kp.flags = flags;
    kp.counters = counters;
    kp.status = noalloc ? reinterpret_cast<uint32_t *>(ds->scratch) : ds->control;
    kp.spin_limit = a.spin_limit ? a.spin_limit : kDefaultSpin;
    kp.debug = a.debug;
    kp.perm = a.unit_perm;
    kp.batch = (int)batch;
    kp.sA = batch > 1 ? a.stride_a : 0;
    kp.sB = batch > 1 ? a.stride_b : 0;
    kp.sC = batch > 1 ? a.stride_c : 0;
    // Split-K partials [batch][S][M][N]
    kp.sP = p.decision == GEMM_SPLITK && !p.atomic ? (long long)p.splits * a.M * a.N : 0;
    // atomic merges add into C: with an epilogue, C first becomes beta C + bias,
    // the merges add alpha acc, and the activation is a last elementwise pass
    const bool atomic_merge = p.atomic && p.decision != GEMM_DP;
    set_epilogue(a, atomic_merge, kp);
    auto prepare_atomic_c = [&]() -> int {
        if (groups) {   // no epilogue in a grouped call: every problem's C := 0
            for (int32_t g = 0; g < ngroups; ++g)
                if (groups[g].M > 0 && groups[g].N > 0 &&
                    (e = dgw::launch_zero(groups[g].C, groups[g].M * groups[g].N, stream)) != hipSuccess)
                    return fail_hip(e, "zero C");
            return GEMM_OK;
        }
        if (kp.epi == dgw::EPI_PLAIN) {
            if ((e = zero_c(a, batch, stream)) != hipSuccess) return fail_hip(e, "zero C");
        } else if ((e = dgw::launch_epilogue_pass(kp, dgw::EPASS_PRE, stream)) != hipSuccess) {
            return fail_hip(e, "epilogue pre-pass");
        }
        return GEMM_OK;
    };

    if (a.trace) {
        if (a.trace_ints < p.trace_ints)
            return fail(GEMM_ERR_INVALID, "trace buffer smaller than plan.trace_ints (" +
                                              std::to_string(p.trace_ints) + ")");
        if ((e = dgw::launch_zero(a.trace, p.trace_ints, stream)) != hipSuccess) return fail_hip(e, "zero trace");
        TraceHeader h = {{0x4B525453, p.decision, (int)p.workers, (int)p.tiles, (int)p.ipt,
                          p.max_segments, p.max_fold, p.splits}};
        hipLaunchKernelGGL(put_trace_header, dim3(1), dim3(64), 0, stream, a.trace, h);
        if ((e = hipGetLastError()) != hipSuccess) return fail_hip(e, "trace header");
        kp.trace = a.trace;
        kp.trace_maxseg = p.max_segments;
        kp.trace_maxfold = p.max_fold;
        kp.trace_workers = (int)p.workers;
        kp.trace_tiles = (int)p.tiles;
    }

    if (p.decision == GEMM_DP) {
        kp.ntiles = (int)p.tiles;
        // 2x2 tile groups when their waves finish sooner than the tiles' waves:
        // a group takes about 4 / 1.4 tile times (measured on 8192^3: 1207 us
        // with one tile per workgroup, 840 us with groups), so with G groups and
        // T tiles on C CUs groups win when ceil(G / C) * 4 < ceil(T / C) * 1.4
        const int64_t quads = batch * ((p.tiles_m + 1) / 2) * ((p.tiles_n + 1) / 2);
        const int64_t gwaves = (quads + ncu - 1) / ncu, twaves = (p.tiles + ncu - 1) / ncu;
        const bool tile_groups = shape == 0 && !groups && gwaves * 40 < twaves * 14 && !(a.debug & GEMM_DEBUG_TILE_DP);
        if (tile_groups) {
            kp.ntiles = (int)quads;
            if ((e = dgw::launch_gemm(dtype, blayout, dgw::K_DP_GROUP, (int)quads, kp, stream)) != hipSuccess)
                return fail_hip(e, "launch DP tile-group kernel");
        } else if ((e = dgw::launch_gemm(dtype, blayout, dgw::K_DP, (int)p.tiles, kp, stream)) != hipSuccess) {
            return fail_hip(e, "launch DP kernel");
        }
    } else if (p.decision == GEMM_SPLITK) {
        kp.ntiles = (int)p.tiles;
        const bool in_launch = (a.debug & (GEMM_DEBUG_IN_LAUNCH | GEMM_DEBUG_SPLITK_BANDS)) != 0;
        kp.merge = p.atomic                      ? dgw::MERGE_ATOMIC
                   : p.two_pass && !in_launch ? dgw::MERGE_TWO_PASS
                                              : dgw::MERGE_IN_LAUNCH;
        // in the launch: when every workgroup of the grid is resident at once, all
        // S splits of a tile add up its row bands (the waits end); otherwise the
        // last arriver at the tile's counter adds up the whole tile.
        // GEMM_DEBUG_IN_LAUNCH keeps the last arriver.
        if (kp.merge == dgw::MERGE_IN_LAUNCH && p.splits > 1 && all_n4 && !(a.debug & GEMM_DEBUG_IN_LAUNCH)) {
            int &bpc = ds->bpc[dtype][blayout][dgw::K_SPLITK][shape][ngroups > 0];
            if (bpc == 0 &&
                (e = dgw::blocks_per_cu(dtype, blayout, dgw::K_SPLITK, p.bm, ngroups > 0, &bpc)) != hipSuccess)
                return fail_hip(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
            if (p.tiles * p.splits <= (int64_t)bpc * ds->num_cus) kp.merge = dgw::MERGE_BANDS;
        }
        if (p.atomic && (rc = prepare_atomic_c()) != GEMM_OK) return rc;
        if ((e = dgw::launch_gemm(dtype, blayout, dgw::K_SPLITK, (int)(p.tiles * p.splits), kp, stream)) !=
            hipSuccess)
            return fail_hip(e, "launch Split-K kernel");
        if (kp.merge == dgw::MERGE_TWO_PASS) {
            KParams rp = kp;
            rp.timing = nullptr;   // timing records cover the Split-K launch's workgroups
            if ((e = dgw::launch_splitk_reduce(rp, stream)) != hipSuccess) return fail_hip(e, "launch Split-K reduction");
        }
    } else {
        if (p.atomic) {
            if ((rc = prepare_atomic_c()) != GEMM_OK) return rc;
        } else {
            kp.epoch = next_epoch();
        }
        kp.units = (int)p.sk_units;
        kp.q = (int)p.q;
        kp.big = (int)p.big;
        kp.tile_base = (int)p.dp_tiles;
        // hybrid: the persistent units run the data-parallel tiles first, in the
        // same launch (GEMM_DEBUG_HYBRID_SPLIT: a second launch after it)
        const bool split_hybrid = (a.debug & GEMM_DEBUG_HYBRID_SPLIT) != 0;
        kp.dp_tiles = split_hybrid ? 0 : (int)p.dp_tiles;
        const bool two_pass = p.two_pass && !(a.debug & GEMM_DEBUG_IN_LAUNCH);
        kp.merge = two_pass ? dgw::MERGE_TWO_PASS : dgw::MERGE_IN_LAUNCH;
        if ((e = dgw::launch_gemm(dtype, blayout, kmode, (int)p.sk_units, kp, stream)) != hipSuccess)
            return fail_hip(e, "launch Stream-K kernel");
        if (two_pass) {
            KParams rp = kp;
            rp.timing = nullptr;   // timing records cover the Stream-K launch's workgroups
            if ((e = dgw::launch_streamk_reduce(rp, p.sk_tiles, stream)) != hipSuccess)
                return fail_hip(e, "launch Stream-K reduction");
        }
        if (p.dp_tiles > 0 && split_hybrid) {
            // hybrid, second launch: the first dp_tiles tiles run as whole-K tiles
            KParams dp = kp;
            dp.tile_base = 0;
            dp.ntiles = (int)p.dp_tiles;
            dp.worker_base = (int)p.sk_units;
            dp.timing_base = (int)p.sk_units;
            dp.perm = nullptr;
            if ((e = dgw::launch_gemm(dtype, blayout, dgw::K_DP, (int)p.dp_tiles, dp, stream)) != hipSuccess)
                return fail_hip(e, "launch DP kernel (hybrid part)");
        }
    }
    if (atomic_merge && kp.act != dgw::ACT_NONE) {
        if ((e = dgw::launch_epilogue_pass(kp, dgw::EPASS_POST, stream)) != hipSuccess)
            return fail_hip(e, "epilogue activation pass");
    }
    return GEMM_OK;
}

}  // namespace

extern "C" {

int gemm(const void *A, const void *B, float *C, int64_t M, int64_t N, int64_t K, uint32_t layout,
         uint32_t mode, int32_t splits) {
    gemm_args_t a;
    std::memset(&a, 0, sizeof a);
    a.A = A;
    a.B = B;
    a.C = C;
    a.M = M;
    a.N = N;
    a.K = K;
    a.layout = layout;
    a.mode = mode;
    a.splits = splits;
    return run(a);
}

int gemm_ex(const gemm_args_t *args) {
    if (!args) return fail(GEMM_ERR_INVALID, "args is null");
    return run(*args);
}

int gemm_grouped(const gemm_args_t *common, const gemm_group_t *groups, int32_t count) {
    if (!common || !groups) return fail(GEMM_ERR_INVALID, "common arguments and groups must be non-null");
    return run(*common, false, groups, count);
}

int gemm_ex_noalloc(const gemm_args_t *args) {
    if (!args) return fail(GEMM_ERR_INVALID, "args is null");
    return run(*args, true);
}

int gemm_plan(int64_t M, int64_t N, int64_t K, uint32_t layout, uint32_t mode, int32_t splits,
              int32_t num_cus, gemm_plan_t *out) {
    return gemm_plan_batched(M, N, K, 1, layout, mode, splits, num_cus, out);
}

int gemm_plan_batched(int64_t M, int64_t N, int64_t K, int64_t batch, uint32_t layout, uint32_t mode,
                      int32_t splits, int32_t num_cus, gemm_plan_t *out) {
    const char *why = "";
    int rc = dgw::make_plan(M, N, K, batch, layout, mode, splits, num_cus, out, &why);
    if (rc != GEMM_OK) return fail(rc, why);
    g_err.clear();
    return GEMM_OK;
}

int64_t gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t batch, uint32_t layout, uint32_t mode,
                            int32_t splits, int32_t num_cus) {
    gemm_plan_t p;
    const char *why = "";
    int rc = dgw::make_plan(M, N, K, batch, layout, mode, splits, num_cus, &p, &why);
    if (rc != GEMM_OK) return fail(rc, why);
    g_err.clear();
    return p.workspace_bytes;
}

int gemm_set_stream(void *stream) {
    g_stream = reinterpret_cast<hipStream_t>(stream);
    return GEMM_OK;
}

int gemm_sync_status(void *stream) {
    hipStream_t s = stream ? reinterpret_cast<hipStream_t>(stream) : g_stream;
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail_hip(e, "hipStreamSynchronize");
    int dev = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return fail_hip(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_mu);
    if ((int)g_dev.size() <= dev || (!g_dev[dev].control && !g_dev[dev].scratch)) return GEMM_OK;
    // the current control block, the retired ones that captured graphs may still
    // use, and the no-allocation scratch array's status words
    std::vector<uint32_t *> blocks = g_dev[dev].retired_control;
    if (g_dev[dev].control) blocks.push_back(g_dev[dev].control);
    if (g_dev[dev].scratch) blocks.push_back(reinterpret_cast<uint32_t *>(g_dev[dev].scratch));
    uint32_t status = 0;
    for (uint32_t *blk : blocks) {
        uint32_t st = 0;
        if ((e = hipMemcpy(&st, blk, 4, hipMemcpyDeviceToHost)) != hipSuccess) return fail_hip(e, "read status");
        if (st == 0) continue;
        status |= st;
        const uint32_t zero = 0;
        if ((e = hipMemcpy(blk, &zero, 4, hipMemcpyHostToDevice)) != hipSuccess) return fail_hip(e, "clear status");
    }
    if (status == 0) return GEMM_OK;
    return fail(GEMM_ERR_TIMEOUT, "a bounded inter-workgroup wait gave up (status word " +
                                      std::to_string(status) + ")");
}

void gemm_release(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) cur = 0;
    for (size_t dev = 0; dev < g_dev.size(); ++dev) {
        DeviceState &d = g_dev[dev];
        if (!d.control && !d.data && d.retired.empty() && d.retired_control.empty()) continue;
        if (hipSetDevice((int)dev) != hipSuccess) continue;
        (void)hipDeviceSynchronize();
        if (d.control) (void)hipFree(d.control);
        if (d.data) (void)hipFree(d.data);
        for (void *r : d.retired) (void)hipFree(r);
        for (uint32_t *r : d.retired_control) (void)hipFree(r);
        d.retired.clear();
        d.retired_control.clear();
        d.control = nullptr;
        d.data = nullptr;
        d.cap_units = d.cap_tiles = d.cap_data = 0;
    }
    (void)hipSetDevice(cur);
}

const char *gemm_last_error(void) { return g_err.c_str(); }

int32_t gemm_num_cus(void) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return n;
}

int32_t gemm_version(void) { return 2; }

}  // extern "C"
