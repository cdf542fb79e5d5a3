// api.hip — the C ABI of moe_ffn.h: validation, workspace layout, launches.
//
// Host side of the operator.  The two-phase shape of the interface (query the
// workspace size, then execute) follows the HyperMegaMoE issue page, section
// 2.3 (workspace query + execute entry points for forward and backward);
// checking shapes, dtypes, layout and buffer sizes at the host boundary
// before any kernel runs follows section 4.2, and the host-computed workspace
// size follows section 5.3.  The library keeps no per-call state: every
// buffer belongs to the caller (the issue page of the FSDP + EP composition
// shows why per-call context must not live in the operator).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kernels.h"
#include "moe_ffn.h"

static_assert(moe::MOE_DEV_BAD_ID == MOE_FFN_DEV_BAD_ID, "status bits");
static_assert(moe::MOE_DEV_TIMEOUT == MOE_FFN_DEV_TIMEOUT, "status bits");
static_assert(moe::MOE_DEV_BAD_SAVED == MOE_FFN_DEV_BAD_SAVED, "status bits");
static_assert(moe::MOE_DEV_BAD_WS == MOE_FFN_DEV_BAD_WS, "status bits");

namespace {

thread_local char g_err[512];
// epoch stamped into every saved context (distinct per forward that saves one)
std::atomic<uint64_t> g_epoch{1};

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int hip_fail(hipError_t err, const char *what)
{
    return fail(MOE_FFN_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

#define HIP_TRY(expr, what)                                                                        \
    do {                                                                                           \
        hipError_t e_ = (expr);                                                                    \
        if (e_ != hipSuccess)                                                                      \
            return hip_fail(e_, what);                                                             \
    } while (0)

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t elem_size(int dtype) { return dtype == MOE_FFN_BF16 ? 2 : 4; }

int validate_problem(const moe_ffn_problem *p)
{
    if (!p)
        return fail(MOE_FFN_ERR_NULL, "problem is NULL");
    if (p->dtype != MOE_FFN_F32 && p->dtype != MOE_FFN_BF16)
        return fail(MOE_FFN_ERR_DTYPE, "dtype must be F32 or BF16 (got %d)", p->dtype);
    if (p->ids_dtype != MOE_FFN_I32 && p->ids_dtype != MOE_FFN_I64)
        return fail(MOE_FFN_ERR_DTYPE, "ids_dtype must be I32 or I64 (got %d)", p->ids_dtype);
    if (p->T < 0)
        return fail(MOE_FFN_ERR_SHAPE, "T must be >= 0 (got %lld)", (long long)p->T);
    if (p->K < 1 || p->K > 32)
        return fail(MOE_FFN_ERR_SHAPE, "K must be in [1, 32] (got %lld)", (long long)p->K);
    if (p->E < 1 || p->E > 1024)
        return fail(MOE_FFN_ERR_SHAPE, "E must be in [1, 1024] (got %lld)", (long long)p->E);
    if (p->H < 8 || p->H % 8)
        return fail(MOE_FFN_ERR_SHAPE, "H must be a positive multiple of 8 (got %lld)",
                    (long long)p->H);
    if (p->I < 8 || p->I % 8)
        return fail(MOE_FFN_ERR_SHAPE, "I must be a positive multiple of 8 (got %lld)",
                    (long long)p->I);
    if (p->T * p->K >= (int64_t(1) << 31))
        return fail(MOE_FFN_ERR_SHAPE, "T*K must be < 2^31");
    if (p->H * 2 * p->I >= (int64_t(1) << 31))
        return fail(MOE_FFN_ERR_SHAPE, "H*2I must be < 2^31");
    if (p->Is < 0 || p->Is % p->I)
        return fail(MOE_FFN_ERR_SHAPE, "Is must be a non-negative multiple of I (got %lld)",
                    (long long)p->Is);
    if (p->E + p->Is / p->I > 1024)
        return fail(MOE_FFN_ERR_SHAPE, "E + Is / I must be <= 1024");
    if (p->T * (p->K + p->Is / p->I) >= (int64_t(1) << 31) || p->H * 2 * p->Is >= (int64_t(1) << 31))
        return fail(MOE_FFN_ERR_SHAPE, "T*(K + Is/I) and H*2Is must be < 2^31");
    return MOE_FFN_OK;
}

// Shared-expert chunks S = Is / I; the plan covers E + S experts and
// T*K + S*T permuted rows (the shared rows after the routed ones).
int nshared(const moe_ffn_problem &p) { return (int)(p.Is / p.I); }

bool aligned16(const void *ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

int check_ptr(const void *ptr, const char *name, size_t align = 16)
{
    if (!ptr)
        return fail(MOE_FFN_ERR_NULL, "%s is NULL", name);
    if (reinterpret_cast<uintptr_t>(ptr) % align)
        return fail(MOE_FFN_ERR_ALIGN, "%s is not %zu-byte aligned", name, align);
    return MOE_FFN_OK;
}

// The current device must be a gfx950 GPU.  Cached per device ordinal, with
// its compute-unit count (the persistent kernels size their grids by it).
int g_num_cus[64] = {0};
int g_clock_khz[64] = {0}; // rate of the device's constant wall clock (s_memrealtime)

int check_device(int *num_cus = nullptr, int *clock_khz = nullptr)
{
    static std::mutex mu;
    static signed char known[64] = {0}; // 0 unknown, 1 ok, -1 not gfx950
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return hip_fail(err, "hipGetDevice");
    if (dev < 0 || dev >= 64)
        return fail(MOE_FFN_ERR_DEVICE, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (known[dev] == 0) {
        hipDeviceProp_t prop;
        err = hipGetDeviceProperties(&prop, dev);
        if (err != hipSuccess)
            return hip_fail(err, "hipGetDeviceProperties");
        int khz = 0;
        err = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
        if (err != hipSuccess)
            return hip_fail(err, "hipDeviceGetAttribute(WallClockRate)");
        known[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
        g_num_cus[dev] = prop.multiProcessorCount;
        g_clock_khz[dev] = khz > 0 ? khz : 100000;
    }
    if (known[dev] < 0)
        return fail(MOE_FFN_ERR_DEVICE, "device %d is not gfx950", dev);
    if (num_cus)
        *num_cus = g_num_cus[dev];
    if (clock_khz)
        *clock_khz = g_clock_khz[dev];
    return MOE_FFN_OK;
}

// Tile height of the forward's M-tiles from the mean rows per expert.  bf16
// with whole tiles (the fast path): 64 for small segments (decode, bound by
// weight streaming) and 128 (two workgroups per CU) up to 512 rows per expert
// (gemm_mfma.hip); longer segments take 256-row tiles of the 256 x 256 tile
// kernel (gemm_big.hip; measured: prefill's 384 rows per expert 345 vs 388 us
// on GEMM1, forward+backward's 1024 rows 466 vs 446 us, the skewed shape's
// 2048 rows 3.63 vs 3.35 ms).  The pipelined forward (one launch,
// gemm_mfma.hip) keeps 128 up to 1024 rows, 256 above.  Other bf16 shapes
// (the engine) use 64 or 128, fp32 64.  All fast-path kernels give the same
// bits whatever the tile height.
moe::FwdTiles pick_tiles(const moe_ffn_problem &p, uint32_t flags)
{
    moe::FwdTiles t;
    t.num_cus = 0;
    t.big = false;
    t.big2 = false;
    if (p.dtype == MOE_FFN_F32) {
        t.BM = 64;
        return t;
    }
    const double avg_rows = (double)(p.T * p.K) / (double)p.E;
    const bool fast = moe::fast_gemm_supported(p.dtype, p.H, p.I);
    const bool pipe = (flags & MOE_FFN_PIPELINE) && p.Is == 0;
    // the 256 x 256 kernel addresses token rows by 32-bit byte offsets
    const int64_t TKp = p.T * (p.K + p.Is / p.I);
    const bool offsets32 = p.T * p.H * 2 < (int64_t(1) << 32) && TKp * p.I * 2 < (int64_t(1) << 32);
    if (avg_rows <= 64.0) {
        t.BM = 64;
    } else if (fast && !pipe && offsets32 && avg_rows > 512.0) {
        t.BM = 256;
        t.big = true;
    } else {
        t.BM = (avg_rows <= 1024.0 || !fast) ? 128 : 256;
        // from 256 rows per expert on, GEMM2 alone runs on 256 x 256 tiles:
        // measured on 384 rows per expert (H = 2048, I = 1408, E = 64) it is
        // 9 % faster there than on 128-row tiles in spite of a third of padded
        // rows, while GEMM1 is 15 % slower (the 11 N-tiles of I = 1408 leave
        // the last of six rounds of tiles half empty)
        t.big2 = fast && !pipe && offsets32 && t.BM == 128 && avg_rows > 256.0;
    }
    return t;
}

// Whether a forward of this problem runs GEMM1 and GEMM2 as the one pipelined
// launch: on request, and by default for problems on 64-row tiles (HBM-bound
// weight streaming, where it measured faster than the two launches); never
// with a shared expert or off the bf16 tile path.
bool use_pipeline(const moe_ffn_problem &p, uint32_t flags)
{
    if (p.Is != 0 || p.dtype != MOE_FFN_BF16 || !moe::fast_gemm_supported(p.dtype, p.H, p.I) ||
        (flags & MOE_FFN_BULK))
        return false;
    return (flags & MOE_FFN_PIPELINE) || pick_tiles(p, 0).BM == 64;
}

// the smallest tile height any call mode of this problem may use (sizes the
// M-tile tables of the workspace, which serves every mode)
int min_tile_rows(const moe_ffn_problem &p)
{
    const int a = pick_tiles(p, 0).BM, b = pick_tiles(p, MOE_FFN_PIPELINE).BM;
    return a < b ? a : b;
}

// ticket counters of the pipelined launch, after its release counters
constexpr int kTickets = 16;

// Region offsets inside the forward workspace (and the saved context).
struct FwdLayout {
    moe::FwdTiles tiles;
    moe::RoutePlan rp;
    int64_t max_mtiles;
    int64_t max_mtiles2; // M-tiles of 256 rows (GEMM2 on the 256 x 256 kernel), or 0
    // ws
    size_t status, hist, bad, counts, offsets, mtile_off, mtile_expert, sorted_slot, slot_pos;
    size_t mtile2_off, mtile2_expert;
    size_t ctr, act, o, ws_total;
    // saved
    size_t s_hdr, s_counts, s_offsets, s_sorted, s_slotpos, s_h, saved_total;
};

FwdLayout fwd_layout(const moe_ffn_problem &p, uint32_t flags = 0)
{
    FwdLayout L;
    const int64_t TK = p.T * p.K;
    const int E = (int)p.E;
    const int Ep = E + nshared(p);                  // experts of the plan
    const int64_t TKp = TK + (int64_t)nshared(p) * p.T; // permuted rows
    const size_t es = elem_size(p.dtype);
    L.tiles = pick_tiles(p, flags);
    L.rp = moe::make_route_plan(TK, E);
    L.max_mtiles = moe::max_mtiles_bound(TKp, Ep, min_tile_rows(p));
    // the 256-row tables exist whenever the bulk forward of this problem runs
    // its GEMM2 on 256 x 256 tiles, whatever the flags (one size serves all)
    L.max_mtiles2 = pick_tiles(p, 0).big2 ? moe::max_mtiles_bound(TKp, Ep, 256) : 0;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + (bytes ? bytes : 1));
        return at;
    };
    L.status = take(sizeof(int32_t));
    L.hist = take(sizeof(int32_t) * (size_t)E * (size_t)L.rp.NB);
    L.bad = take(sizeof(int32_t) * (size_t)L.rp.NB);
    L.counts = take(sizeof(int32_t) * (size_t)Ep);
    L.offsets = take(sizeof(int32_t) * (size_t)(Ep + 1));
    L.mtile_off = take(sizeof(int32_t) * (size_t)(Ep + 1));
    L.mtile_expert = take(sizeof(int32_t) * (size_t)L.max_mtiles);
    L.mtile2_off = take(L.max_mtiles2 ? sizeof(int32_t) * (size_t)(Ep + 1) : 0);
    L.mtile2_expert = take(sizeof(int32_t) * (size_t)L.max_mtiles2);
    // sorted_slot (here and in the saved context) has 256 entries of padding:
    // the GEMMs read their gather indices in whole blocks (up to a tile's rows
    // or a K step's past the end)
    L.sorted_slot = take(sizeof(int32_t) * ((size_t)TKp + 256));
    L.slot_pos = take(sizeof(int32_t) * (size_t)TK);
    L.ctr = take(sizeof(int32_t) * ((size_t)L.max_mtiles + kTickets));
    L.act = take(es * (size_t)TKp * (size_t)p.I);
    L.o = take(es * (size_t)TKp * (size_t)p.H);
    L.ws_total = off;
    off = 0;
    L.s_hdr = take(sizeof(moe::SavedHeader));
    L.s_counts = take(sizeof(int32_t) * (size_t)Ep);
    L.s_offsets = take(sizeof(int32_t) * (size_t)(Ep + 1));
    L.s_sorted = take(sizeof(int32_t) * ((size_t)TKp + 256));
    L.s_slotpos = take(sizeof(int32_t) * (size_t)TK);
    L.s_h = take(es * (size_t)TKp * (size_t)(2 * p.I));
    L.saved_total = off;
    return L;
}

// Workspace of the routing step alone.
struct RouteLayout {
    moe::RoutePlan rp;
    int BM;
    size_t status, hist, bad, mtile_off, mtile_expert, total;
};

RouteLayout route_layout(const moe_ffn_problem &p)
{
    RouteLayout R;
    const int64_t TK = p.T * p.K;
    const int E = (int)p.E;
    R.rp = moe::make_route_plan(TK, E);
    R.BM = pick_tiles(p, 0).BM;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + (bytes ? bytes : 1));
        return at;
    };
    R.status = take(sizeof(int32_t));
    R.hist = take(sizeof(int32_t) * (size_t)E * (size_t)R.rp.NB);
    R.bad = take(sizeof(int32_t) * (size_t)R.rp.NB);
    R.mtile_off = take(sizeof(int32_t) * (size_t)(E + 1));
    R.mtile_expert = take(sizeof(int32_t) * (size_t)moe::max_mtiles_bound(TK, E, R.BM));
    R.total = off;
    return R;
}

// Region offsets inside the backward workspace.
struct BwdLayout {
    int BM;
    int64_t max_mtiles;
    int dgp_width;
    size_t status, whdr, counts, offsets, mtile_off, mtile_expert, xcd_bounds, dh, act_g, dgp, dxp,
        total;
};

BwdLayout bwd_layout(const moe_ffn_problem &p)
{
    BwdLayout B;
    const int64_t TK = p.T * p.K + (int64_t)nshared(p) * p.T; // permuted rows
    const int E = (int)p.E + nshared(p);                     // experts of the plan
    B.BM = 128;
    B.max_mtiles = moe::max_mtiles_bound(TK, E, B.BM);
    B.dgp_width = moe::engine_dgp_width((int)p.I);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + (bytes ? bytes : 1));
        return at;
    };
    B.status = take(sizeof(int32_t));
    B.whdr = take(sizeof(moe::SavedHeader));
    B.counts = take(sizeof(int32_t) * (size_t)E);
    B.offsets = take(sizeof(int32_t) * (size_t)(E + 1));
    B.mtile_off = take(sizeof(int32_t) * (size_t)(E + 1));
    B.mtile_expert = take(sizeof(int32_t) * (size_t)B.max_mtiles);
    B.xcd_bounds = take(sizeof(int32_t) * 2 * 9);
    B.dh = take(2 * (size_t)TK * (size_t)(2 * p.I));
    B.act_g = take(2 * (size_t)TK * (size_t)p.I);
    B.dgp = take(sizeof(float) * (size_t)TK * (size_t)B.dgp_width);
    B.dxp = take(2 * (size_t)TK * (size_t)p.H);
    B.total = off;
    return B;
}

// FNV-1a over the problem's sizes and dtypes: the identity a saved context
// carries from the forward to the backward
uint64_t problem_hash(const moe_ffn_problem &p)
{
    const int64_t v[8] = {p.T, p.H, p.I, p.E, p.K, p.dtype, p.ids_dtype, p.Is};
    uint64_t h = 1469598103934665603ull;
    for (int64_t x : v)
        for (int b = 0; b < 8; ++b) {
            h ^= (uint64_t)((x >> (8 * b)) & 0xff);
            h *= 1099511628211ull;
        }
    return h;
}

// Scratch of moe_ffn_fwd_noalloc: device memory that the library owns, one
// copy per GPU, held until the process ends.  Host code never uses the
// array's name as an address; noalloc_scratch() resolves, once per device
// (with that device current), the device address of this GPU's copy.
static __device__ __align__(256) unsigned char scratch[MOE_FFN_NOALLOC_WS_BYTES];
std::mutex g_scratch_mu;
void *g_scratch_ptr[64] = {};

int noalloc_scratch(void **ptr)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return hip_fail(err, "hipGetDevice");
    if (dev < 0 || dev >= 64)
        return fail(MOE_FFN_ERR_DEVICE, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p)
            return hip_fail(err, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MOE_FFN_OK;
}

// The backward's second stream (default priority, like every stream here):
// the weight-gradient branch runs on it beside input_grad and the dx combine.
// Created once per device, with its two events, on the first whole backward
// (normally an eager call, before any graph capture).
// The events are shared by the calls on one device, so a call holds the
// device's enqueue lock from its first record to its last wait.
struct SideStream {
    hipStream_t s;
    hipEvent_t ready; // the main stream reached the branch point
    hipEvent_t done;  // the side stream finished its branch
};
std::mutex g_side_mu;
std::mutex g_side_enqueue[64];
SideStream g_side[64];
bool g_side_ok[64] = {};

int side_stream(SideStream *out, std::unique_lock<std::mutex> *enqueue_lock)
{
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess)
        return hip_fail(err, "hipGetDevice");
    if (dev < 0 || dev >= 64)
        return fail(MOE_FFN_ERR_DEVICE, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_side_mu);
    if (!g_side_ok[dev]) {
        SideStream ss{};
        if ((err = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking)) != hipSuccess)
            return hip_fail(err, "hipStreamCreateWithFlags");
        if ((err = hipEventCreateWithFlags(&ss.ready, hipEventDisableTiming)) != hipSuccess ||
            (err = hipEventCreateWithFlags(&ss.done, hipEventDisableTiming)) != hipSuccess)
            return hip_fail(err, "hipEventCreateWithFlags");
        g_side[dev] = ss;
        g_side_ok[dev] = true;
    }
    *out = g_side[dev];
    *enqueue_lock = std::unique_lock<std::mutex>(g_side_enqueue[dev]);
    return MOE_FFN_OK;
}

template <typename P> P *at(void *base, size_t off)
{
    return reinterpret_cast<P *>(static_cast<char *>(base) + off);
}

void record(const moe_ffn_stage_events *ev, int stage, bool begin, hipStream_t s)
{
    if (!ev)
        return;
    void *e = begin ? ev->begin[stage] : ev->end[stage];
    if (e)
        (void)hipEventRecord(static_cast<hipEvent_t>(e), s);
}

} // namespace

extern "C" {

int moe_ffn_fwd_workspace_size(const moe_ffn_problem *p, uint32_t flags, size_t *ws_bytes,
                               size_t *saved_bytes)
{
    (void)flags;
    g_err[0] = 0;
    int rc = validate_problem(p);
    if (rc)
        return rc;
    if (!ws_bytes)
        return fail(MOE_FFN_ERR_NULL, "ws_bytes is NULL");
    const FwdLayout L = fwd_layout(*p);
    *ws_bytes = L.ws_total;
    if (saved_bytes)
        *saved_bytes = L.saved_total;
    return MOE_FFN_OK;
}

int moe_ffn_fwd_stages(const moe_ffn_problem *p, uint32_t flags, moe_ffn_fwd_stage_layout *layout)
{
    g_err[0] = 0;
    int rc = validate_problem(p);
    if (rc)
        return rc;
    if (!layout)
        return fail(MOE_FFN_ERR_NULL, "layout is NULL");
    const FwdLayout L = fwd_layout(*p, flags);
    layout->counts = L.counts;
    layout->offsets = L.offsets;
    layout->sorted_slot = L.sorted_slot;
    layout->slot_pos = L.slot_pos;
    layout->act = L.act;
    layout->o = L.o;
    layout->tile_rows = L.tiles.BM;
    const bool fast = moe::fast_gemm_supported(p->dtype, p->H, p->I);
    layout->kernel = p->dtype == MOE_FFN_F32 ? MOE_FFN_KERNEL_GENERIC
                     : !fast                 ? MOE_FFN_KERNEL_ENGINE
                     : use_pipeline(*p, flags) ? MOE_FFN_KERNEL_PIPELINED
                     : L.tiles.big           ? MOE_FFN_KERNEL_BIG_TILES
                     : L.tiles.big2          ? MOE_FFN_KERNEL_TILES_BIG_GEMM2
                                             : MOE_FFN_KERNEL_TILES;
    return MOE_FFN_OK;
}

// The forward, with or without a shared expert (sh: its weights; p->Is > 0).
static int fwd_run(const moe_ffn_problem *p, const void *x, const void *topk_ids,
                   const float *topk_weights, const void *up_proj_weight,
                   const void *down_proj_weight, const moe_ffn_shared_weights *sh, void *y,
                   void *saved, void *ws, size_t ws_bytes, uint32_t flags, void *stream,
                   const moe_ffn_stage_events *ev)
{
    g_err[0] = 0;
    int rc = validate_problem(p);
    if (rc)
        return rc;
    if ((flags & MOE_FFN_PIPELINE) && (flags & MOE_FFN_BULK))
        return fail(MOE_FFN_ERR_SHAPE, "flags: MOE_FFN_PIPELINE and MOE_FFN_BULK exclude each other");
    const int S = nshared(*p);
    if (S > 0 && !sh)
        return fail(MOE_FFN_ERR_NULL, "a problem with Is > 0 needs the shared-expert weights");
    const FwdLayout L = fwd_layout(*p, flags);
    if (p->T == 0)
        return MOE_FFN_OK;
    if (S > 0 && ((rc = check_ptr(sh->up_proj_weight, "shared up_proj_weight")) ||
                  (rc = check_ptr(sh->down_proj_weight, "shared down_proj_weight"))))
        return rc;
    const size_t id_align = p->ids_dtype == MOE_FFN_I64 ? 8 : 4;
    if ((rc = check_ptr(x, "x")) || (rc = check_ptr(topk_ids, "topk_ids", id_align)) ||
        (rc = check_ptr(topk_weights, "topk_weights", 4)) ||
        (rc = check_ptr(up_proj_weight, "up_proj_weight")) ||
        (rc = check_ptr(down_proj_weight, "down_proj_weight")) || (rc = check_ptr(y, "y")) ||
        (rc = check_ptr(ws, "ws")))
        return rc;
    if (saved && !aligned16(saved))
        return fail(MOE_FFN_ERR_ALIGN, "saved is not 16-byte aligned");
    if (ws_bytes < L.ws_total)
        return fail(MOE_FFN_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, L.ws_total);
    int num_cus = 0, clock_khz = 0;
    if ((rc = check_device(&num_cus, &clock_khz)))
        return rc;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t TK = p->T * p->K;
    const int E = (int)p->E;
    moe::RouteBufs rb;
    rb.hist = at<int32_t>(ws, L.hist);
    rb.bad = at<int32_t>(ws, L.bad);
    rb.mtile_off = at<int32_t>(ws, L.mtile_off);
    rb.mtile_expert = at<int32_t>(ws, L.mtile_expert);
    rb.status = at<int32_t>(ws, L.status);
    rb.ctr = at<int32_t>(ws, L.ctr);
    rb.nctr = (int)(L.max_mtiles + kTickets);
    // GEMM2 on 256 x 256 tiles (not in the pipelined launch, which runs both
    // GEMMs on GEMM1's tiles): routing also builds the 256-row M-tile tables
    const bool big2 = L.tiles.big2 && !use_pipeline(*p, flags);
    if (big2) {
        rb.mtile2_off = at<int32_t>(ws, L.mtile2_off);
        rb.mtile2_expert = at<int32_t>(ws, L.mtile2_expert);
        rb.BM2 = 256;
    }
    rb.saved_hdr = saved ? at<moe::SavedHeader>(saved, L.s_hdr) : nullptr;
    rb.problem_hash = problem_hash(*p);
    rb.epoch = saved ? g_epoch.fetch_add(1) : 0;
    rb.nshared = S;
    rb.T = p->T;
    const int Ep = E + S; // experts of the plan: routed, then the shared chunks
    const int64_t Is = p->Is;
    if (saved) {
        rb.counts = at<int32_t>(saved, L.s_counts);
        rb.offsets = at<int32_t>(saved, L.s_offsets);
        rb.sorted_slot = at<int32_t>(saved, L.s_sorted);
        rb.slot_pos = at<int32_t>(saved, L.s_slotpos);
    } else {
        rb.counts = at<int32_t>(ws, L.counts);
        rb.offsets = at<int32_t>(ws, L.offsets);
        rb.sorted_slot = at<int32_t>(ws, L.sorted_slot);
        rb.slot_pos = at<int32_t>(ws, L.slot_pos);
    }

    record(ev, MOE_FFN_STAGE_ROUTE, true, s);
    HIP_TRY(moe::launch_route(topk_ids, p->ids_dtype == MOE_FFN_I64, TK, E, L.tiles.BM, L.rp, rb,
                              s),
            "route launch");
    record(ev, MOE_FFN_STAGE_ROUTE, false, s);

    if (flags & MOE_FFN_CHECK_IDS) {
        int32_t st = 0;
        HIP_TRY(hipMemcpyAsync(&st, rb.status, sizeof st, hipMemcpyDeviceToHost, s),
                "status copy");
        HIP_TRY(hipStreamSynchronize(s), "stream sync");
        if (st)
            return fail(MOE_FFN_ERR_EXPERT_ID, "topk_ids holds a value outside [0, %d)", E);
    }

    const bool fast = moe::fast_gemm_supported(p->dtype, p->H, p->I);
    if (p->dtype == MOE_FFN_BF16 && !fast) {
        // bf16, ragged H or I: the persistent engine (gemm_engine.hip)
        moe::EngineArgs g1{};
        g1.A = static_cast<const moe::bf16_t *>(x);
        g1.B = static_cast<const moe::bf16_t *>(up_proj_weight);
        g1.C = at<moe::bf16_t>(ws, L.act);
        g1.C2 = saved ? at<moe::bf16_t>(saved, L.s_h) : nullptr;
        g1.sorted_slot = rb.sorted_slot;
        g1.offsets = rb.offsets;
        g1.mtile_off = rb.mtile_off;
        g1.mtile_expert = rb.mtile_expert;
        g1.topk = (int)p->K;
        g1.E = Ep;
        g1.N = (int)p->I;
        g1.Kd = (int)p->H;
        g1.lda = (int)p->H;
        g1.ldb = (int)(2 * p->I);
        g1.ldc = (int)p->I;
        g1.b_estride = p->H * 2 * p->I;
        g1.Er = E;
        if (S > 0) {
            g1.Bs = static_cast<const moe::bf16_t *>(sh->up_proj_weight);
            g1.bs_cstride = p->I;
            g1.bs_ldb = (int)(2 * Is);
            g1.bs_panel = (int)Is;
        }
        record(ev, MOE_FFN_STAGE_GEMM1, true, s);
        HIP_TRY(moe::launch_engine(moe::ENG_F1, L.tiles.BM, g1, num_cus, s), "gemm1 launch");
        record(ev, MOE_FFN_STAGE_GEMM1, false, s);

        moe::EngineArgs g2 = g1;
        g2.A = at<moe::bf16_t>(ws, L.act);
        g2.B = static_cast<const moe::bf16_t *>(down_proj_weight);
        g2.C = at<moe::bf16_t>(ws, L.o);
        g2.C2 = nullptr;
        g2.N = (int)p->H;
        g2.Kd = (int)p->I;
        g2.lda = (int)p->I;
        g2.ldb = (int)p->H;
        g2.ldc = (int)p->H;
        g2.b_estride = p->I * p->H;
        if (S > 0) {
            g2.Bs = static_cast<const moe::bf16_t *>(sh->down_proj_weight);
            g2.bs_cstride = p->I * p->H;
            g2.bs_ldb = (int)p->H;
            g2.bs_panel = 0;
        }
        record(ev, MOE_FFN_STAGE_GEMM2, true, s);
        HIP_TRY(moe::launch_engine(moe::ENG_F2, L.tiles.BM, g2, num_cus, s), "gemm2 launch");
        record(ev, MOE_FFN_STAGE_GEMM2, false, s);
    } else if (fast) {
        // bf16 with whole tiles: the tile engine of gemm_mfma.hip, as separate
        // launches or, on request, pipelined (one launch, tile-granular release)
        moe::FastFwdArgs a{};
        a.x = x;
        a.w1 = up_proj_weight;
        a.w2 = down_proj_weight;
        a.act = at<void>(ws, L.act);
        a.hsave = saved ? at<void>(saved, L.s_h) : nullptr;
        a.o = at<void>(ws, L.o);
        a.sorted_slot = rb.sorted_slot;
        a.offsets = rb.offsets;
        a.mtile_off = rb.mtile_off;
        a.mtile_expert = rb.mtile_expert;
        a.ctr = rb.ctr;
        a.tickets = rb.ctr + L.max_mtiles;
        a.status = rb.status;
        const int64_t watchdog_ms = (flags & MOE_FFN_TEST_DROP_RELEASE) ? 20 : 2000;
        a.timeout_ticks = watchdog_ms * (int64_t)clock_khz;
        a.T = (int)p->T;
        a.H = (int)p->H;
        a.I = (int)p->I;
        a.E = Ep;
        a.K = (int)p->K;
        a.sh.Er = E;
        a.sh.S = S;
        a.sh.Is = (int)Is;
        a.sh.w1 = S > 0 ? sh->up_proj_weight : nullptr;
        a.sh.w2 = S > 0 ? sh->down_proj_weight : nullptr;
        a.max_mtiles = (int)L.max_mtiles;
        a.grid = (flags & MOE_FFN_TEST_SMALL_GRID) ? 16 : 0;
        a.drop_mt = (flags & MOE_FFN_TEST_DROP_RELEASE) ? 0 : -1;
        const int BM = L.tiles.BM;
        // the pipelined launch serves routed experts only; with a shared expert
        // the bulk launches run
        if (use_pipeline(*p, flags)) {
            // GEMM1 and GEMM2 in one launch; the combine follows as its own
            // launch (no token block's combine could start before the last
            // experts' GEMM2 tiles anyway)
            if (flags & MOE_FFN_TEST_ONE_WORKGROUP)
                a.grid = 1;
            record(ev, MOE_FFN_STAGE_PIPELINE, true, s);
            HIP_TRY(moe::launch_fast_fwd(moe::FAST_PIPE, BM, a, num_cus, s), "pipeline launch");
            record(ev, MOE_FFN_STAGE_PIPELINE, false, s);
        } else {
            const int g1mode = a.hsave ? moe::FAST_G1H : moe::FAST_G1;
            record(ev, MOE_FFN_STAGE_GEMM1, true, s);
            HIP_TRY(L.tiles.big ? moe::launch_fast_fwd_big(g1mode, a, num_cus, s)
                                : moe::launch_fast_fwd(g1mode, BM, a, num_cus, s),
                    "gemm1 launch");
            record(ev, MOE_FFN_STAGE_GEMM1, false, s);
            moe::FastFwdArgs a2 = a;
            if (big2) {
                a2.mtile_off = rb.mtile2_off;
                a2.mtile_expert = rb.mtile2_expert;
                a2.max_mtiles = (int)L.max_mtiles2;
            }
            record(ev, MOE_FFN_STAGE_GEMM2, true, s);
            // GEMM2 on 256-row tiles over GEMM1's 128: one M-tile in two is
            // short (prefill: 79-175 of 256 rows), so its padding is not copied
            HIP_TRY(L.tiles.big || big2 ? moe::launch_fast_fwd_big(moe::FAST_G2, a2, num_cus, s, big2)
                                        : moe::launch_fast_fwd(moe::FAST_G2, BM, a, num_cus, s),
                    "gemm2 launch");
            record(ev, MOE_FFN_STAGE_GEMM2, false, s);
        }
    } else {
        // fp32: the generic kernels (gemm.hip)
        moe::GroupedGemmArgs g1{};
        g1.A = x;
        g1.B = up_proj_weight;
        g1.C = at<void>(ws, L.act);
        g1.Hsave = saved ? at<void>(saved, L.s_h) : nullptr;
        g1.sorted_slot = rb.sorted_slot;
        g1.offsets = rb.offsets;
        g1.mtile_off = rb.mtile_off;
        g1.mtile_expert = rb.mtile_expert;
        g1.Kdim = (int)p->H;
        g1.Nout = (int)p->I;
        g1.ldb = (int)(2 * p->I);
        g1.topk = (int)p->K;
        g1.E = Ep;
        g1.max_mtiles = (int)L.max_mtiles;
        g1.Er = E;
        if (S > 0) {
            g1.Bs = sh->up_proj_weight;
            g1.bs_cstride = p->I;
            g1.bs_ldb = (int)(2 * Is);
            g1.bs_panel = (int)Is;
        }
        record(ev, MOE_FFN_STAGE_GEMM1, true, s);
        HIP_TRY(moe::launch_gemm1_swiglu(p->dtype, L.tiles, g1, s), "gemm1 launch");
        record(ev, MOE_FFN_STAGE_GEMM1, false, s);

        moe::GroupedGemmArgs g2 = g1;
        g2.A = at<void>(ws, L.act);
        g2.B = down_proj_weight;
        g2.C = at<void>(ws, L.o);
        g2.Hsave = nullptr;
        g2.sorted_slot = nullptr;
        g2.Kdim = (int)p->I;
        g2.Nout = (int)p->H;
        g2.ldb = (int)p->H;
        if (S > 0) {
            g2.Bs = sh->down_proj_weight;
            g2.bs_cstride = p->I * p->H;
            g2.bs_ldb = (int)p->H;
            g2.bs_panel = 0;
        }
        record(ev, MOE_FFN_STAGE_GEMM2, true, s);
        HIP_TRY(moe::launch_gemm2(p->dtype, L.tiles, g2, s), "gemm2 launch");
        record(ev, MOE_FFN_STAGE_GEMM2, false, s);
    }

    record(ev, MOE_FFN_STAGE_COMBINE, true, s);
    HIP_TRY(moe::launch_combine(p->dtype, at<void>(ws, L.o), rb.slot_pos, topk_weights, y, p->T,
                                (int)p->H, (int)p->K, rb.offsets, E, S, s),
            "combine launch");
    record(ev, MOE_FFN_STAGE_COMBINE, false, s);
    if (flags & MOE_FFN_CHECK_STATUS) {
        int32_t st = 0;
        HIP_TRY(hipMemcpyAsync(&st, rb.status, sizeof st, hipMemcpyDeviceToHost, s),
                "status copy");
        HIP_TRY(hipStreamSynchronize(s), "stream sync");
        if (st & moe::MOE_DEV_TIMEOUT)
            return fail(MOE_FFN_ERR_TIMEOUT, "a wait of the pipelined forward hit its watchdog; "
                                             "y is unreliable");
        if (st & moe::MOE_DEV_BAD_ID)
            return fail(MOE_FFN_ERR_EXPERT_ID, "topk_ids holds a value outside [0, %d)", E);
    }
    return MOE_FFN_OK;
}

int moe_ffn_fwd_ex(const moe_ffn_problem *p, const void *x, const void *topk_ids,
                   const float *topk_weights, const void *up_proj_weight,
                   const void *down_proj_weight, void *y, void *saved, void *ws, size_t ws_bytes,
                   uint32_t flags, void *stream, const moe_ffn_stage_events *ev)
{
    if (p && p->Is != 0)
        return fail(MOE_FFN_ERR_SHAPE, "Is != 0: use moe_ffn_fwd_shared");
    return fwd_run(p, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, nullptr, y,
                   saved, ws, ws_bytes, flags, stream, ev);
}

int moe_ffn_fwd_shared(const moe_ffn_problem *p, const void *x, const void *topk_ids,
                       const float *topk_weights, const void *up_proj_weight,
                       const void *down_proj_weight, const moe_ffn_shared_weights *shared,
                       void *y, void *saved, void *ws, size_t ws_bytes, uint32_t flags,
                       void *stream, const moe_ffn_stage_events *ev)
{
    return fwd_run(p, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, shared, y,
                   saved, ws, ws_bytes, flags, stream, ev);
}

int moe_ffn_fwd(const moe_ffn_problem *p, const void *x, const void *topk_ids,
                const float *topk_weights, const void *up_proj_weight,
                const void *down_proj_weight, void *y, void *saved, void *ws, size_t ws_bytes,
                uint32_t flags, void *stream)
{
    return moe_ffn_fwd_ex(p, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, y,
                          saved, ws, ws_bytes, flags, stream, nullptr);
}

int moe_ffn_fwd_noalloc(const moe_ffn_problem *p, const void *x, const void *topk_ids,
                        const float *topk_weights, const void *up_proj_weight,
                        const void *down_proj_weight, void *y, uint32_t flags, void *stream)
{
    g_err[0] = 0;
    int rc = validate_problem(p);
    if (rc)
        return rc;
    if (p->Is != 0)
        return fail(MOE_FFN_ERR_SHAPE, "moe_ffn_fwd_noalloc: Is != 0 is not supported");
    if (flags & (MOE_FFN_CHECK_IDS | MOE_FFN_CHECK_STATUS))
        return fail(MOE_FFN_ERR_SHAPE, "moe_ffn_fwd_noalloc: MOE_FFN_CHECK_IDS and "
                                       "MOE_FFN_CHECK_STATUS are not supported (they copy to the host)");
    const FwdLayout L = fwd_layout(*p, flags);
    if (L.ws_total > MOE_FFN_NOALLOC_WS_BYTES)
        return fail(MOE_FFN_ERR_WORKSPACE,
                    "moe_ffn_fwd_noalloc: this problem needs %zu bytes of scratch, more than the "
                    "%zu the library holds per GPU; call moe_ffn_fwd with a workspace",
                    L.ws_total, (size_t)MOE_FFN_NOALLOC_WS_BYTES);
    if (p->T == 0)
        return MOE_FFN_OK;
    if ((rc = check_device()))
        return rc;
    void *ws = nullptr;
    if ((rc = noalloc_scratch(&ws)))
        return rc;
    return fwd_run(p, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight, nullptr, y,
                   nullptr, ws, MOE_FFN_NOALLOC_WS_BYTES, flags, stream, nullptr);
}

int moe_ffn_route_workspace_size(const moe_ffn_problem *p, size_t *ws_bytes)
{
    g_err[0] = 0;
    int rc = validate_problem(p);
    if (rc)
        return rc;
    if (!ws_bytes)
        return fail(MOE_FFN_ERR_NULL, "ws_bytes is NULL");
    *ws_bytes = route_layout(*p).total;
    return MOE_FFN_OK;
}

int moe_ffn_route(const moe_ffn_problem *p, const void *topk_ids, int32_t *counts,
                  int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos, void *ws,
                  size_t ws_bytes, void *stream)
{
    g_err[0] = 0;
    int rc = validate_problem(p);
    if (rc)
        return rc;
    const RouteLayout R = route_layout(*p);
    const size_t need = R.total;
    const int64_t TK = p->T * p->K;
    const size_t id_align = p->ids_dtype == MOE_FFN_I64 ? 8 : 4;
    if ((rc = check_ptr(counts, "counts", 4)) || (rc = check_ptr(offsets, "offsets", 4)) ||
        (rc = check_ptr(ws, "ws")))
        return rc;
    if (TK > 0 && ((rc = check_ptr(topk_ids, "topk_ids", id_align)) ||
                   (rc = check_ptr(sorted_slot, "sorted_slot", 4)) ||
                   (rc = check_ptr(slot_pos, "slot_pos", 4))))
        return rc;
    if (ws_bytes < need)
        return fail(MOE_FFN_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, need);
    if ((rc = check_device()))
        return rc;
    moe::RouteBufs rb;
    rb.status = at<int32_t>(ws, R.status);
    rb.ctr = nullptr;
    rb.nctr = 0;
    rb.saved_hdr = nullptr;
    rb.problem_hash = 0;
    rb.epoch = 0;
    rb.nshared = 0;
    rb.T = p->T;
    rb.hist = at<int32_t>(ws, R.hist);
    rb.bad = at<int32_t>(ws, R.bad);
    rb.mtile_off = at<int32_t>(ws, R.mtile_off);
    rb.mtile_expert = at<int32_t>(ws, R.mtile_expert);
    rb.counts = counts;
    rb.offsets = offsets;
    rb.sorted_slot = sorted_slot;
    rb.slot_pos = slot_pos;
    HIP_TRY(moe::launch_route(topk_ids, p->ids_dtype == MOE_FFN_I64, TK, (int)p->E, R.BM, R.rp,
                              rb, static_cast<hipStream_t>(stream)),
            "route launch");
    return MOE_FFN_OK;
}

int moe_ffn_bwd_workspace_size(const moe_ffn_problem *p, uint32_t flags, size_t *ws_bytes)
{
    (void)flags;
    g_err[0] = 0;
    int rc = validate_problem(p);
    if (rc)
        return rc;
    if (!ws_bytes)
        return fail(MOE_FFN_ERR_NULL, "ws_bytes is NULL");
    if (p->dtype != MOE_FFN_BF16)
        return fail(MOE_FFN_ERR_DTYPE, "the backward supports bf16 problems only");
    *ws_bytes = bwd_layout(*p).total;
    return MOE_FFN_OK;
}

// The backward, whole (BWD_STAGE_ALL) or one of its two stages: D computes
// act_grad, input_grad and the dx / d_topk combine and leaves dh and act_g in
// the workspace; W computes the weight gradients from them.
static int bwd_run(const moe_ffn_problem *p, int stage, const void *dy, const void *x,
                   const float *topk_weights, const void *up_proj_weight,
                   const void *down_proj_weight, const moe_ffn_shared_weights *sh,
                   const void *saved, void *dx, void *d_up_proj_weight,
                   void *d_down_proj_weight, float *d_topk_weights,
                   const moe_ffn_shared_grads *sg, void *ws, size_t ws_bytes, uint32_t flags,
                   void *stream, const moe_ffn_stage_events *ev)
{
    g_err[0] = 0;
    int rc = validate_problem(p);
    if (rc)
        return rc;
    if (p->dtype != MOE_FFN_BF16)
        return fail(MOE_FFN_ERR_DTYPE, "the backward supports bf16 problems only");
    const int S = nshared(*p);
    if (S > 0 && stage != moe::BWD_STAGE_ALL)
        return fail(MOE_FFN_ERR_SHAPE, "the split backward serves problems without a shared expert");
    if (S > 0 && (!sh || !sg))
        return fail(MOE_FFN_ERR_NULL, "a problem with Is > 0 needs the shared weights and gradients");
    if (S > 0 && ((rc = check_ptr(sg->d_up_proj_weight, "d_shared_up_proj_weight")) ||
                  (rc = check_ptr(sg->d_down_proj_weight, "d_shared_down_proj_weight"))))
        return rc;
    if (S > 0 && p->T > 0 &&
        ((rc = check_ptr(sh->up_proj_weight, "shared up_proj_weight")) ||
         (rc = check_ptr(sh->down_proj_weight, "shared down_proj_weight"))))
        return rc;
    const bool do_d = stage != moe::BWD_STAGE_W, do_w = stage != moe::BWD_STAGE_D;
    const BwdLayout B = bwd_layout(*p);
    const FwdLayout L = fwd_layout(*p);
    if (do_w && ((rc = check_ptr(d_up_proj_weight, "d_up_proj_weight")) ||
                 (rc = check_ptr(d_down_proj_weight, "d_down_proj_weight"))))
        return rc;
    if (p->T > 0 &&
        ((rc = check_ptr(dy, "dy")) || (rc = check_ptr(saved, "saved")) ||
         (rc = check_ptr(ws, "ws")) ||
         (do_d && ((rc = check_ptr(topk_weights, "topk_weights", 4)) ||
                   (rc = check_ptr(up_proj_weight, "up_proj_weight")) ||
                   (rc = check_ptr(down_proj_weight, "down_proj_weight")) ||
                   (rc = check_ptr(dx, "dx")) ||
                   (rc = check_ptr(d_topk_weights, "d_topk_weights", 4)))) ||
         (do_w && (rc = check_ptr(x, "x")))))
        return rc;
    if (p->T > 0 && ws_bytes < B.total)
        return fail(MOE_FFN_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, B.total);
    int num_cus = 0;
    if ((rc = check_device(&num_cus)))
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t dw_bytes = 2 * (size_t)p->E * (size_t)p->H * (size_t)p->I;
    if (p->T == 0) {
        // no slot reached any expert: the weight gradients are exactly zero
        if (do_w) {
            HIP_TRY(moe::launch_zero_fill(d_up_proj_weight, 2 * dw_bytes, s), "zero fill");
            HIP_TRY(moe::launch_zero_fill(d_down_proj_weight, dw_bytes, s), "zero fill");
        }
        if (S > 0) {
            const size_t sw_bytes = 2 * (size_t)p->Is * (size_t)p->H;
            HIP_TRY(moe::launch_zero_fill(sg->d_up_proj_weight, 2 * sw_bytes, s), "zero fill");
            HIP_TRY(moe::launch_zero_fill(sg->d_down_proj_weight, sw_bytes, s), "zero fill");
        }
        return MOE_FFN_OK;
    }
    const int E = (int)p->E, I = (int)p->I, H = (int)p->H;
    void *sv = const_cast<void *>(saved);
    const moe::SavedHeader *hdr = at<moe::SavedHeader>(sv, L.s_hdr);
    moe::SavedHeader *whdr = at<moe::SavedHeader>(ws, B.whdr);
    const uint64_t phash = problem_hash(*p);
    if (flags & MOE_FFN_CHECK_SAVED) {
        moe::SavedHeader h_host{}, w_host{};
        HIP_TRY(hipMemcpyAsync(&h_host, hdr, sizeof h_host, hipMemcpyDeviceToHost, s),
                "saved header copy");
        if (stage == moe::BWD_STAGE_W)
            HIP_TRY(hipMemcpyAsync(&w_host, whdr, sizeof w_host, hipMemcpyDeviceToHost, s),
                    "workspace header copy");
        HIP_TRY(hipStreamSynchronize(s), "stream sync");
        if (h_host.magic != moe::kSavedMagic || h_host.version != moe::kSavedVersion ||
            h_host.problem != phash)
            return fail(MOE_FFN_ERR_SAVED, "saved context was not written by a forward of this problem");
        if (stage == moe::BWD_STAGE_W &&
            (w_host.magic != h_host.magic || w_host.version != h_host.version ||
             w_host.problem != h_host.problem || w_host.epoch != h_host.epoch))
            return fail(MOE_FFN_ERR_SAVED,
                        "workspace does not hold the data-gradient stage of this saved context");
    }
    const int32_t *saved_counts = at<int32_t>(sv, L.s_counts);
    const int32_t *saved_offsets = at<int32_t>(sv, L.s_offsets);
    int32_t *counts = at<int32_t>(ws, B.counts);
    int32_t *offsets = at<int32_t>(ws, B.offsets);
    int32_t *bstatus = at<int32_t>(ws, B.status);
    const int32_t *sorted_slot = at<int32_t>(sv, L.s_sorted);
    const int32_t *slot_pos = at<int32_t>(sv, L.s_slotpos);
    const moe::bf16_t *h = at<moe::bf16_t>(sv, L.s_h);
    int32_t *mtile_off = at<int32_t>(ws, B.mtile_off);
    int32_t *mtile_expert = at<int32_t>(ws, B.mtile_expert);
    moe::bf16_t *dh = at<moe::bf16_t>(ws, B.dh);
    moe::bf16_t *act_g = at<moe::bf16_t>(ws, B.act_g);
    float *dgp = at<float>(ws, B.dgp);
    moe::bf16_t *dxp = at<moe::bf16_t>(ws, B.dxp);

    const int Ep = E + S; // experts of the plan: routed, then the shared chunks
    const int64_t Is = p->Is;
    // XCD bounds of the two weight-gradient launches (W2Grad, W1Grad)
    moe::XcdSplits splits{};
    splits.n = 2;
    splits.bounds = at<int32_t>(ws, B.xcd_bounds);
    moe::engine_feature_tiling(moe::ENG_B5, I, H, num_cus, &splits.F[0], &splits.wgx[0]);
    moe::engine_feature_tiling(moe::ENG_B7, H, 2 * I, num_cus, &splits.F[1], &splits.wgx[1]);
    HIP_TRY(moe::launch_bwd_setup(hdr, phash, saved_counts, saved_offsets, Ep,
                                  p->T * p->K + (int64_t)S * p->T, B.BM, counts, offsets,
                                  mtile_off, mtile_expert, bstatus, whdr, stage, splits, s),
            "backward set-up launch");
    (void)counts;

    moe::EngineArgs base{};
    base.sorted_slot = sorted_slot;
    base.offsets = offsets;
    base.mtile_off = mtile_off;
    base.mtile_expert = mtile_expert;
    base.topk = (int)p->K;
    base.E = Ep;
    base.Er = E;

    // The whole backward overlaps its two branches (issue page, section 2.2:
    // W2Grad beside the activation-gradient branch, W1Grad beside the dx
    // combine): after act_grad, the weight gradients (which need only act_g,
    // dh, dY and x) run on a second stream of the same priority while
    // input_grad and the dx combine run on the caller's stream, joined by
    // events.  The split entry points keep one stream (their caller schedules).
    const bool overlap = do_d && do_w;
    SideStream side{};
    std::unique_lock<std::mutex> enqueue_lock;
    if (overlap && (rc = side_stream(&side, &enqueue_lock)))
        return rc;
    hipStream_t sw = overlap ? side.s : s; // stream of the weight-gradient branch
    if (do_d) {
        // act_grad with the SwiGLU backward in its epilogue: dh, act_g, d_g partials
        moe::EngineArgs a2 = base;
        a2.A = static_cast<const moe::bf16_t *>(dy);
        a2.B = static_cast<const moe::bf16_t *>(down_proj_weight);
        a2.C = dh;
        a2.C2 = act_g;
        a2.Hs = h;
        a2.gates = topk_weights;
        a2.dgp = dgp;
        a2.dgp_stride = B.dgp_width;
        a2.N = I;
        a2.Kd = H;
        a2.lda = H;
        a2.ldb = H;
        a2.b_estride = (int64_t)I * H;
        if (S > 0) { // shared chunk c: rows [cI, cI + I) of the shared down_proj
            a2.Bs = static_cast<const moe::bf16_t *>(sh->down_proj_weight);
            a2.bs_cstride = (int64_t)I * H;
            a2.bs_ldb = H;
        }
        record(ev, MOE_FFN_STAGE_BWD_ACT_GRAD, true, s);
        HIP_TRY(moe::launch_engine(moe::ENG_B2, B.BM, a2, num_cus, s), "act_grad launch");
        record(ev, MOE_FFN_STAGE_BWD_ACT_GRAD, false, s);

        if (overlap) {
            HIP_TRY(hipEventRecord(side.ready, s), "event record");
            HIP_TRY(hipStreamWaitEvent(sw, side.ready, 0), "stream wait");
        }
    }
    if (do_d) {
        // input_grad: dx_perm = dh W1[e]^T
        moe::EngineArgs a4 = base;
        a4.A = dh;
        a4.B = static_cast<const moe::bf16_t *>(up_proj_weight);
        a4.C = dxp;
        a4.N = H;
        a4.Kd = 2 * I;
        a4.lda = 2 * I;
        a4.ldb = 2 * I;
        a4.ldc = H;
        a4.b_estride = (int64_t)H * 2 * I;
        if (S > 0) { // shared chunk c: gate columns cI.., up columns Is + cI.. of its rows
            a4.Bs = static_cast<const moe::bf16_t *>(sh->up_proj_weight);
            a4.bs_cstride = I;
            a4.bs_ldb = (int)(2 * Is);
            a4.bs_kjump = (int)(Is - I);
        }
        record(ev, MOE_FFN_STAGE_BWD_INPUT_GRAD, true, s);
        HIP_TRY(moe::launch_engine(moe::ENG_B4, B.BM, a4, num_cus, s), "input_grad launch");
        record(ev, MOE_FFN_STAGE_BWD_INPUT_GRAD, false, s);

        record(ev, MOE_FFN_STAGE_BWD_COMBINE, true, s);
        HIP_TRY(moe::launch_combine_bwd(dxp, dgp, B.dgp_width, slot_pos, bstatus, dx,
                                        d_topk_weights, p->T, H, (int)p->K, offsets, E, S, s),
                "dx combine launch");
        record(ev, MOE_FFN_STAGE_BWD_COMBINE, false, s);
    }
    if (do_w) {
        // W2Grad: dW2[e] = act_g^T dY_perm
        moe::EngineArgs a5 = base;
        a5.A = act_g;
        a5.B = static_cast<const moe::bf16_t *>(dy);
        a5.C = static_cast<moe::bf16_t *>(d_down_proj_weight);
        a5.M = I;
        a5.N = H;
        a5.lda = I;
        a5.ldb = H;
        a5.xcd_bounds = splits.bounds;
        if (S > 0) { // shared chunk c: rows [cI, cI + I) of the shared down_proj gradient
            a5.Cs = static_cast<moe::bf16_t *>(sg->d_down_proj_weight);
            a5.cs_cstride = (int64_t)I * H;
            a5.cs_ldc = H;
        }
        record(ev, MOE_FFN_STAGE_BWD_W2_GRAD, true, sw);
        HIP_TRY(moe::launch_engine(moe::ENG_B5, B.BM, a5, num_cus, sw), "W2Grad launch");
        record(ev, MOE_FFN_STAGE_BWD_W2_GRAD, false, sw);

        // W1Grad: dW1[e] = x_perm^T dh
        moe::EngineArgs a7 = base;
        a7.A = static_cast<const moe::bf16_t *>(x);
        a7.B = dh;
        a7.C = static_cast<moe::bf16_t *>(d_up_proj_weight);
        a7.M = H;
        a7.N = 2 * I;
        a7.lda = H;
        a7.ldb = 2 * I;
        a7.xcd_bounds = splits.bounds + 9;
        if (S > 0) { // shared chunk c: its gate and up column chunks of the shared gradient
            a7.Cs = static_cast<moe::bf16_t *>(sg->d_up_proj_weight);
            a7.cs_cstride = I;
            a7.cs_ldc = (int)(2 * Is);
            a7.cs_cjump = (int)(Is - I);
        }
        record(ev, MOE_FFN_STAGE_BWD_W1_GRAD, true, sw);
        HIP_TRY(moe::launch_engine(moe::ENG_B7, B.BM, a7, num_cus, sw), "W1Grad launch");
        record(ev, MOE_FFN_STAGE_BWD_W1_GRAD, false, sw);
    }
    if (overlap)
        HIP_TRY(hipEventRecord(side.done, sw), "event record");
    if (overlap)
        HIP_TRY(hipStreamWaitEvent(s, side.done, 0), "stream wait");
    return MOE_FFN_OK;
}

int moe_ffn_bwd_ex(const moe_ffn_problem *p, const void *dy, const void *x, const void *topk_ids,
                   const float *topk_weights, const void *up_proj_weight,
                   const void *down_proj_weight, const void *saved, void *dx,
                   void *d_up_proj_weight, void *d_down_proj_weight, float *d_topk_weights,
                   void *ws, size_t ws_bytes, uint32_t flags, void *stream,
                   const moe_ffn_stage_events *ev)
{
    // topk_ids is part of the signature the pages give the operator; the
    // backward reads the routing the forward saved instead
    const size_t id_align = p && p->ids_dtype == MOE_FFN_I64 ? 8 : 4;
    if (p && p->T > 0) {
        int rc = check_ptr(topk_ids, "topk_ids", id_align);
        if (rc)
            return rc;
    }
    if (p && p->Is != 0)
        return fail(MOE_FFN_ERR_SHAPE, "Is != 0: use moe_ffn_bwd_shared");
    return bwd_run(p, moe::BWD_STAGE_ALL, dy, x, topk_weights, up_proj_weight, down_proj_weight,
                   nullptr, saved, dx, d_up_proj_weight, d_down_proj_weight, d_topk_weights,
                   nullptr, ws, ws_bytes, flags, stream, ev);
}

int moe_ffn_bwd(const moe_ffn_problem *p, const void *dy, const void *x, const void *topk_ids,
                const float *topk_weights, const void *up_proj_weight,
                const void *down_proj_weight, const void *saved, void *dx,
                void *d_up_proj_weight, void *d_down_proj_weight, float *d_topk_weights,
                void *ws, size_t ws_bytes, uint32_t flags, void *stream)
{
    return moe_ffn_bwd_ex(p, dy, x, topk_ids, topk_weights, up_proj_weight, down_proj_weight,
                          saved, dx, d_up_proj_weight, d_down_proj_weight, d_topk_weights, ws,
                          ws_bytes, flags, stream, nullptr);
}

int moe_ffn_bwd_d(const moe_ffn_problem *p, const void *dy, const float *topk_weights,
                  const void *up_proj_weight, const void *down_proj_weight, const void *saved,
                  void *dx, float *d_topk_weights, void *ws, size_t ws_bytes, uint32_t flags,
                  void *stream)
{
    return bwd_run(p, moe::BWD_STAGE_D, dy, nullptr, topk_weights, up_proj_weight,
                   down_proj_weight, nullptr, saved, dx, nullptr, nullptr, d_topk_weights,
                   nullptr, ws, ws_bytes, flags, stream, nullptr);
}

int moe_ffn_bwd_w(const moe_ffn_problem *p, const void *dy, const void *x, const void *saved,
                  void *d_up_proj_weight, void *d_down_proj_weight, void *ws, size_t ws_bytes,
                  uint32_t flags, void *stream)
{
    return bwd_run(p, moe::BWD_STAGE_W, dy, x, nullptr, nullptr, nullptr, nullptr, saved,
                   nullptr, d_up_proj_weight, d_down_proj_weight, nullptr, nullptr, ws, ws_bytes,
                   flags, stream, nullptr);
}

int moe_ffn_bwd_shared(const moe_ffn_problem *p, const void *dy, const void *x,
                       const void *topk_ids, const float *topk_weights,
                       const void *up_proj_weight, const void *down_proj_weight,
                       const moe_ffn_shared_weights *shared, const void *saved, void *dx,
                       void *d_up_proj_weight, void *d_down_proj_weight, float *d_topk_weights,
                       const moe_ffn_shared_grads *d_shared, void *ws, size_t ws_bytes,
                       uint32_t flags, void *stream, const moe_ffn_stage_events *ev)
{
    const size_t id_align = p && p->ids_dtype == MOE_FFN_I64 ? 8 : 4;
    if (p && p->T > 0) {
        int rc = check_ptr(topk_ids, "topk_ids", id_align);
        if (rc)
            return rc;
    }
    return bwd_run(p, moe::BWD_STAGE_ALL, dy, x, topk_weights, up_proj_weight, down_proj_weight,
                   shared, saved, dx, d_up_proj_weight, d_down_proj_weight, d_topk_weights,
                   d_shared, ws, ws_bytes, flags, stream, ev);
}

int moe_ffn_read_status(const void *ws, void *stream, int32_t *device_status)
{
    g_err[0] = 0;
    if (!ws || !device_status)
        return fail(MOE_FFN_ERR_NULL, "ws or device_status is NULL");
    hipStream_t s = static_cast<hipStream_t>(stream);
    HIP_TRY(hipStreamSynchronize(s), "stream sync");
    HIP_TRY(hipMemcpy(device_status, ws, sizeof(int32_t), hipMemcpyDeviceToHost), "status copy");
    return MOE_FFN_OK;
}

const char *moe_ffn_status_string(int status)
{
    switch (status) {
    case MOE_FFN_OK: return "ok";
    case MOE_FFN_ERR_NULL: return "a required pointer is NULL";
    case MOE_FFN_ERR_SHAPE: return "a size is out of the supported range";
    case MOE_FFN_ERR_DTYPE: return "unsupported dtype";
    case MOE_FFN_ERR_ALIGN: return "a pointer is not suitably aligned";
    case MOE_FFN_ERR_WORKSPACE: return "workspace or saved buffer too small";
    case MOE_FFN_ERR_EXPERT_ID: return "an expert id is outside [0, E)";
    case MOE_FFN_ERR_SAVED: return "saved context does not match the problem";
    case MOE_FFN_ERR_HIP: return "HIP runtime error";
    case MOE_FFN_ERR_DEVICE: return "current device is not gfx950";
    case MOE_FFN_ERR_TIMEOUT: return "a pipelined wait hit its watchdog";
    default: return "unknown status";
    }
}

const char *moe_ffn_last_error(void) { return g_err; }

int moe_ffn_event_create(void **event)
{
    if (!event)
        return fail(MOE_FFN_ERR_NULL, "event is NULL");
    hipEvent_t e;
    HIP_TRY(hipEventCreate(&e), "hipEventCreate");
    *event = e;
    return MOE_FFN_OK;
}

int moe_ffn_event_destroy(void *event)
{
    if (event)
        HIP_TRY(hipEventDestroy(static_cast<hipEvent_t>(event)), "hipEventDestroy");
    return MOE_FFN_OK;
}

int moe_ffn_event_elapsed_ms(void *begin, void *end, float *ms)
{
    if (!begin || !end || !ms)
        return fail(MOE_FFN_ERR_NULL, "event or ms is NULL");
    // an event that was never recorded (a stage the call's path does not run)
    // fails here; the runtime's sticky error is cleared so that it is not
    // reported by the next, unrelated launch
    hipError_t err = hipEventSynchronize(static_cast<hipEvent_t>(end));
    if (err == hipSuccess)
        err = hipEventElapsedTime(ms, static_cast<hipEvent_t>(begin), static_cast<hipEvent_t>(end));
    if (err != hipSuccess) {
        (void)hipGetLastError();
        return hip_fail(err, "event elapsed time");
    }
    return MOE_FFN_OK;
}

const char *moe_ffn_version(void) { return "0.1.0"; }

} // extern "C"
