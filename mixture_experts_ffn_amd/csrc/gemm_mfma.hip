// gemm_mfma.hip — the forward bf16 grouped GEMMs of the MoE expert FFN for
// gfx950, and the pipelined forward that chains them with tile-granular
// release.  Fast path for H a multiple of 256 and I of 128 (whole K steps and
// whole output tiles); other bf16 shapes and the backward use the engine of
// gemm_engine.hip, fp32 uses gemm.hip.
//
// The two operations (HyperMegaMoE issue page, section 2.1: GMM1/up_proj with
// the SwiGLU epilogue, GMM2/down_proj):
//   GEMM1: act[p, j] = silu(x[t_p] · W1[e][:, j]) · (x[t_p] · W1[e][:, I + j])
//   GEMM2: o[p, :]   = act[p, :] · W2[e]
//
// One tile engine serves both, in three modes:
//   FAST_G1, FAST_G2  one grouped GEMM per launch (the bulk forward: route,
//                     GEMM1, GEMM2 and combine as separate launches);
//   FAST_G1H          FAST_G1 that also saves the pre-activation h for the
//                     backward;
//   FAST_PIPE         one launch runs every GEMM1 tile, then every GEMM2 tile,
//                     then the combine, with device counters in place of the
//                     launch boundaries (the overlap explainer page, sections
//                     5-6, and the issue page's tile-level pipelining: a
//                     consumer starts as soon as the tiles it reads are done).
//
// Tile engine, organised for the CDNA4 memory pipeline:
//  * Global -> LDS copies go straight into LDS (16 bytes per lane, no
//    register staging), NSTAGE stages deep, NSTAGE - 1 K steps ahead of the
//    matrix cores; each wave waits only for its own copies of the stage it is
//    about to use, then one barrier per K step publishes the stage, and a
//    step's copies are issued after its MFMAs.
//  * A (token rows, K-contiguous) lands as [BM][BK] with the 16-byte piece
//    index XOR-ed by a function of the row, so the 16 lanes of one 128-bit
//    LDS read hit 16 different bank groups.  The dispatch gather x[sorted_slot / K] is
//    just the per-lane source address of those copies.
//  * B (weights, N-contiguous [k][n]) lands untransposed as two panels of
//    [BK][128] with the 32-byte unit index XOR-ed by a 3-bit hash of k; the
//    MFMA fragments are read with the transposing 64-bit LDS read.  GEMM1's
//    panels are 128 gate and the matching 128 up columns, so SwiGLU pairs two
//    accumulators of one lane; GEMM2's panels are 256 adjacent output columns.
//  * The matrix-core step computes C^T = W^T · X^T (weights as the first
//    operand), so each lane owns 4 consecutive output columns of one row; the
//    epilogue passes the tile through LDS and stores it as whole rows.
//  * Block tile BM rows x 256 weight columns, two waves per SIMD (one wave's
//    MFMAs cover the other's LDS waits):
//      BM = 64:  one workgroup of 8 waves per CU, each wave all 64 rows and 16
//                columns of each panel (BK = 64, 3 stages);
//      BM = 128: TWO workgroups of 4 waves per CU, each wave all 128 rows and
//                32 columns of each panel (BK = 32, 3 stages, 72 KB each).
//                The per-K-step barrier then holds only one of the two waves
//                on a SIMD, so the two drift apart and one's MFMAs fill the
//                other's read and barrier waits; each wave also reads 40 %
//                fewer LDS bytes per MFMA than with 8 waves of 16 columns;
//      BM = 256: one workgroup of 8 waves per CU as 2 x 4, each wave 128 rows
//                and 32 columns of each panel (BK = 32, 4 stages).
//    A wave whose 128 rows lie past an expert's count skips its MFMAs, so
//    tall tiles waste no more matrix-core time than short ones.
//  * Persistent: the workgroups resident on the CUs walk XCD-local slices of
//    the tile order (the hardware hands workgroup b to XCD b % 8), so tiles
//    in flight on one XCD share weight panels and token rows in its L2; a
//    slice's partial last round goes by tickets to the workgroups that finish
//    first; the next tile's first copies overlap the current tile's last
//    steps and its epilogue.
#include "common.h"
#include "kernels.h"
#include "tile_common.h"

namespace moe {
namespace fast {
using namespace tile;

// waves per workgroup for a block tile of BM rows: 128-row tiles run as two
// 4-wave workgroups per CU, the others as one 8-wave workgroup
constexpr int waves_for(int BM) { return BM == 128 ? 4 : 8; }

// Block tile BM x (2 x 128): BM = 64 with 8 waves, BK = 64 and a 3-stage ring;
// BM = 128 with 4 waves, BK = 32 and a 3-stage ring (two workgroups share a
// CU); waves side by side along N.  BM = 256 with 8 waves as 2 (M) x 4 (N),
// BK = 32 and a 4-stage ring, so each wave owns 128 rows x 32 columns per
// panel and needs a third fewer LDS reads and copied bytes per flop.
template <int BM_, int NW_ = 8> struct Cfg {
    static constexpr int BM = BM_;
    static constexpr int NW = NW_;                   // waves per workgroup
    static constexpr int BK = BM == 256 || NW == 4 ? 32 : 64; // K per step
    static constexpr int NSTAGE = BM == 256 ? 4 : 3; // LDS ring depth
    static constexpr int WM = BM == 256 && NW == 8 ? 2 : 1; // waves along M
    static constexpr int WN = NW / WM;               // waves along N
    static constexpr int WTM = BM / WM;              // rows per wave
    static constexpr int WTN = PW / WN;              // columns per wave per panel
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int KH = BK / 32;               // 32-deep MFMA steps per K step
    static constexpr int PIECES = BK / 8;            // 16-byte pieces per A row
    static constexpr int RPC = 1024 / (BK * 2);      // A rows per 1 KB copy chunk
    static constexpr int CPP = BK / 4;               // 1 KB B chunks per panel (4 k-rows each)
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BK * 2 * PW * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_LOADS = A_BYTES / 1024 / NW; // per wave per stage
    static constexpr int B_LOADS = B_BYTES / 1024 / NW;
    static constexpr int NL = A_LOADS + B_LOADS;
    static_assert(A_LOADS >= 1 && A_LOADS * NW * 1024 == A_BYTES, "stage split");
    static_assert(B_LOADS >= 1 && B_LOADS * NW * 1024 == B_BYTES, "stage split");
    static_assert(NSTAGE * STAGE_BYTES <= 160 * 1024, "LDS");
    static_assert(FN >= 1 && KH >= 1, "wave tile");
};

// ---- release / acquire of the pipelined forward -------------------------------
// Everything one workgroup of the pipelined launch hands to another (act rows
// from GEMM1 to GEMM2, o rows from GEMM2 to the combine) is written with
// device-coherent stores and read with device-coherent loads (the sc1 scope
// bit; the encoding of device-scope relaxed atomics), so no cache holds a
// stale or a dirty private copy of it and no whole-cache write-back or
// invalidate is needed.  Each producer wave waits until its own stores of a
// tile are acknowledged (vmcnt) and its lane 0 bumps the tile's counter, so a
// tile is complete at NW bumps per N-tile; a consumer polls the counter with
// device-coherent loads, bounded by the watchdog, and issues its loads only
// after the poll has returned.
__device__ __forceinline__ void store_coherent(void *p, u32x2 v)
{
    __hip_atomic_store(static_cast<uint64_t *>(p), __builtin_bit_cast(uint64_t, v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ u32x4 load_coherent16(const void *p)
{
    const uint64_t *q = static_cast<const uint64_t *>(p);
    const uint64_t lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    u32x4 v;
    v[0] = (uint32_t)lo;
    v[1] = (uint32_t)(lo >> 32);
    v[2] = (uint32_t)hi;
    v[3] = (uint32_t)(hi >> 32);
    return v;
}
__device__ __forceinline__ int poll(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// one increment per wave (lane 0 only)
__device__ __forceinline__ void bump(int32_t *p)
{
    if (__lane_id() == 0)
        __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-wide wait until every lane's counter (p != nullptr) reaches `need`.
// On timeout the status word gets MOE_DEV_TIMEOUT and the wave goes on, so
// every wave ends.
__device__ __forceinline__ void wait_counters(const int32_t *p, int need, const FastFwdArgs &a)
{
    auto pending = [&]() { return __ballot(p != nullptr && poll(p) < need) != 0ull; };
    if (!pending())
        return;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (pending()) {
        if ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) > a.timeout_ticks) {
            if (__lane_id() == 0)
                __hip_atomic_fetch_or(a.status, MOE_DEV_TIMEOUT, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    asm volatile("" ::: "memory"); // the consumer's loads stay after the poll
}

// Position of a workgroup in one phase (the tiles of one grouped GEMM): each
// XCD owns a contiguous eighth of the tile order; its workgroups take every
// (gridDim.x / 8)-th tile of it (separate launches), or claim its tiles from
// the XCD's ticket counter (the pipelined launch; `tried` counts the XCD
// slices this workgroup has found exhausted in the current phase).  In the
// separate launches the tiles of each slice from `tail` on (its last, partial
// round) also go by tickets, to the workgroups that finish first.
struct Cursor {
    int kind, L, hi, step, tried;
    int tail;   // offset in each slice of the ticketed tiles (-1: none)
    int send;   // end of the strided part of this workgroup's slice
    bool tick;  // the walk has reached the ticketed tiles
};

template <int BM, int MODE, int NWAVES>
__global__ __launch_bounds__(64 * NWAVES, 8 / NWAVES) void moe_fwd_bf16(FastFwdArgs args)
{
    using C = Cfg<BM, NWAVES>;
    constexpr int NW = C::NW;
    constexpr int BK = C::BK, NSTAGE = C::NSTAGE;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * C::STAGE_BYTES];

    constexpr bool PIPE = MODE == FAST_PIPE;
    constexpr bool G1ONLY = MODE == FAST_G1 || MODE == FAST_G1H;
    const int H = args.H, I = args.I;
    const int ntn1 = I / TILE_N1, ntn2 = H / TILE_N2;
    const int mtiles = uni(ldc(args.mtile_off, args.E));
    const int per_xcd_wg = gridDim.x >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = uni(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN; // this wave's block of the tile
    int32_t *const ctr1 = args.ctr; // GEMM1 N-tiles done per M-tile

    auto kind_of = [&](int k) {
        return G1ONLY ? (int)KIND_G1 : MODE == FAST_G2 ? (int)KIND_G2 : k;
    };
    // Tickets.  The pipelined launch hands out its tiles by tickets, so that
    // any tile a GEMM2 tile waits for has been claimed by a running workgroup:
    // per-XCD counters over the same XCD slices (tiles in flight on one XCD
    // still share panels in its L2); a workgroup whose slice is exhausted
    // claims from the other XCDs' counters in turn, and GEMM2 tickets are only
    // drawn once every GEMM1 slice is exhausted.  GEMM1 tiles wait for
    // nothing, so every claimed tile completes whether or not the other
    // workgroups of the launch are resident.  The separate launches draw the
    // tickets of their slices' last rounds the same way (one GEMM each, so
    // they stop after the eighth slice).  Wave 0 draws the ticket and passes
    // it to the other waves through LDS.
    __shared__ int tick_bcast[2];
    int tick_par = 0;
    auto claim = [&](Cursor &c) {
        while (true) {
            const int total = mtiles * (c.kind == KIND_G1 ? ntn1 : ntn2);
            const int range = (total + 7) >> 3;
            const int x = (xcd + c.tried) & 7;
            const int hi = min((x + 1) * range, total);
            const int lo = min(x * range + c.tail, hi);
            if (wave == 0 && lane == 0)
                tick_bcast[tick_par] =
                    lo < hi ? __hip_atomic_fetch_add(args.tickets + (c.kind == KIND_G1 ? 0 : 8) + x,
                                                     1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : 0x7fffffff;
            __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): the ticket is in LDS
            lds_barrier();
            const int t = uni(tick_bcast[tick_par]);
            tick_par ^= 1;
            if (t < hi - lo) {
                c.L = lo + t;
                return true;
            }
            // The slice is exhausted.  Rather than trying the others one
            // atomic at a time, wave 0 reads all eight counters at once (a
            // load per lane; a counter only grows, so a slice seen exhausted
            // stays so) and picks the next slice in ring order from this XCD
            // that still has tiles; should its atomic find it exhausted after
            // all, this repeats.
            if (wave == 0) {
                bool left = false;
                if (lane < 8) {
                    const int hx = min((lane + 1) * range, total);
                    const int lx = min(lane * range + c.tail, hx);
                    const int32_t *ctr = args.tickets + (c.kind == KIND_G1 ? 0 : 8) + lane;
                    left = lx < hx && __hip_atomic_load(ctr, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT) < hx - lx;
                }
                const uint64_t m = __ballot(left); // bit x: slice x has tiles left
                int nd = 8;
                for (int d = c.tried + 1; d < 8; ++d)
                    if ((m >> ((xcd + d) & 7)) & 1) {
                        nd = d;
                        break;
                    }
                if (lane == 0)
                    tick_bcast[tick_par] = nd;
            }
            __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): the choice is in LDS
            lds_barrier();
            c.tried = uni(tick_bcast[tick_par]);
            tick_par ^= 1;
            if (c.tried < 8)
                continue;
            if (!PIPE || c.kind == KIND_G2)
                return false;
            c.kind = KIND_G2;
            c.tried = 0;
        }
    };
    auto phase_begin = [&](int kind, Cursor &c) {
        const int total = mtiles * (kind == KIND_G1 ? ntn1 : ntn2);
        const int range = (total + 7) >> 3;
        c.kind = kind;
        // 64-row tiles stream weights (HBM-bound): as many workgroups as make
        // every round of the XCD's range full, so no round runs half-empty
        int wg = per_xcd_wg;
        if (BM == 64) {
            const int rounds = (range + per_xcd_wg - 1) / per_xcd_wg;
            wg = rounds > 0 ? (range + rounds - 1) / rounds : per_xcd_wg;
        }
        c.step = wg;
        c.L = xcd * range + slot;
        c.hi = min((xcd + 1) * range, total);
        c.tried = 0;
        // A partial last round after two full ones or more goes by tickets:
        // with the strided walk alone, the workgroups that hold one tile more
        // than the others (and those on slower compute units) set the end of
        // the launch while the rest idle.  (64-row tiles make every round
        // full instead, above.)
        const int rounds = (range + wg - 1) / wg;
        const bool ticketed = BM != 64 && rounds >= 3 && range % wg != 0;
        c.tail = ticketed ? (rounds - 1) * wg : -1;
        c.send = ticketed ? min(c.hi, xcd * range + c.tail) : c.hi;
        c.tick = false;
        if (slot >= wg)
            return false;
        if (c.L < c.send)
            return true;
        if (!ticketed)
            return false;
        c.tick = true;
        return claim(c);
    };
    auto advance = [&](Cursor &c) {
        if (!PIPE && !c.tick) {
            c.L += c.step;
            if (c.L < c.send)
                return true;
            if (c.tail < 0)
                return false;
            c.tick = true;
        }
        return claim(c);
    };
    auto decode = [&](const Cursor &c) {
        const int kind = kind_of(c.kind);
        return decode_tile(args, kind, c.L, kind == KIND_G1 ? ntn1 : ntn2, BM);
    };

    // per-lane copy sources of one tile
    struct Src {
        const bf16 *a[C::A_LOADS];
        const bf16 *b[C::B_LOADS];
        int ldb;
        bool coherent_a; // A rows written by this launch (pipelined GEMM2)
    };
    auto make_src = [&](const Tile &t, Src &sr) {
        const bool g1 = kind_of(t.kind) == KIND_G1;
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i) {
            // chunk c covers rows RPC*c .. RPC*c + RPC-1; this lane fills 16-byte
            // unit `lane` of it
            const int c = wave * C::A_LOADS + i;
            const int r = c * C::RPC + lane / C::PIECES;
            const int piece = aswz<C::PIECES>(r, lane % C::PIECES);
            if (g1) {
                // the chunk's row indices are wave-uniform and consecutive: one
                // wide scalar load (sorted_slot is padded past its end by more
                // than a tile); rows past the expert's count copy row 0
                const __attribute__((address_space(4))) int32_t *ix =
                    (const __attribute__((address_space(4))) int32_t *)args.sorted_slot +
                    uni(t.row0 + c * C::RPC);
                const int idx0 = ldc(args.sorted_slot, t.row0);
                int v = 0;
#pragma unroll
                for (int j = 0; j < C::RPC; ++j) {
                    const int idx = c * C::RPC + j < t.rows ? ix[j] : idx0;
                    v = lane / C::PIECES == j ? idx : v;
                }
                const int64_t grow = v / args.K;
                sr.a[i] = static_cast<const bf16 *>(args.x) + grow * H + piece * 8;
            } else {
                const int64_t grow = t.row0 + (r < t.rows ? r : 0);
                sr.a[i] = static_cast<const bf16 *>(args.act) + grow * I + piece * 8;
            }
        }
        // a shared-expert chunk c = e - Er reads its column chunk of the shared
        // up_proj (rows of 2Is, up panel Is columns in) or its row chunk of the
        // shared down_proj
        const bool shd = args.sh.S > 0 && t.e >= args.sh.Er;
        const int64_t sc = t.e - args.sh.Er;
        const bf16 *W =
            g1 ? (shd ? static_cast<const bf16 *>(args.sh.w1) + sc * I
                      : static_cast<const bf16 *>(args.w1) + (int64_t)t.e * H * (2 * I))
               : (shd ? static_cast<const bf16 *>(args.sh.w2) + sc * I * H
                      : static_cast<const bf16 *>(args.w2) + (int64_t)t.e * I * H);
        sr.ldb = g1 ? 2 * (shd ? args.sh.Is : I) : H;
        sr.coherent_a = PIPE && !g1;
        const int pstride = g1 ? (shd ? args.sh.Is : I) : PW; // column offset of the second panel
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
            // chunk c covers 1024 bytes = 4 k-rows of one 128-column panel
            const int c = wave * C::B_LOADS + i;
            const int panel = c / C::CPP;
            const int kr = (c % C::CPP) * 4 + (lane >> 4);
            const int pp = lane & 15;
            const int u = (pp >> 1) ^ bswz(kr);
            const int col = t.n0 + panel * pstride + (2 * u + (pp & 1)) * 8;
            sr.b[i] = W + (int64_t)kr * sr.ldb + col;
        }
    };
    auto issue = [&](const Src &sr, int kb, unsigned char *sbase) {
        const int k0 = kb * BK;
        if (PIPE && sr.coherent_a) {
#pragma unroll
            for (int i = 0; i < C::A_LOADS; ++i)
                g2l16_coherent(sr.a[i] + k0, (lds_void *)(sbase + (wave * C::A_LOADS + i) * 1024));
        } else {
#pragma unroll
            for (int i = 0; i < C::A_LOADS; ++i)
                g2l16(sr.a[i] + k0, (lds_void *)(sbase + (wave * C::A_LOADS + i) * 1024));
        }
        // 64-row tiles (at most 64 rows per expert on average): each weight
        // panel is streamed once, so it is copied with the non-temporal hint
        // (decode: the launch 496 -> 455 us)
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
            if constexpr (BM == 64)
                g2l16_nt(sr.b[i] + (int64_t)k0 * sr.ldb,
                         (lds_void *)(sbase + C::A_BYTES + (wave * C::B_LOADS + i) * 1024));
            else
                g2l16(sr.b[i] + (int64_t)k0 * sr.ldb,
                      (lds_void *)(sbase + C::A_BYTES + (wave * C::B_LOADS + i) * 1024));
        }
    };

    f32x4 acc[2][C::FM][C::FN];
    const int fr = lane & 15;                      // A: row within a 16-row block
    const int fk = lane >> 4;                      // A: piece in a 32-k step; B: 8-k group
    const int tq = lane & 3, tr = (lane >> 2) & 3; // B transposing read: column part / row

    // One K step of this wave's WTM x (2 x WTN) block: 2*FN*FM MFMAs per 32 k,
    // fed by FM 128-bit A reads and 4*FN transposing 64-bit B reads.  The LDS
    // pipe and the matrix cores are close to balanced, so the order is pinned:
    // the first MFMA group's operands, then one read per MFMA until all reads
    // are out, then the remaining MFMAs.
    //
    // FMA (a compile-time count, fma_c's value) is the number of this wave's
    // 16-row blocks the step computes: a tile whose rows end early (the last
    // M-tile of an expert) reads and multiplies only the blocks that hold
    // rows, rounded up to an even count; the others keep their zeros and are
    // never stored.
    auto compute = [&](auto fma_c, const unsigned char *sA) {
        constexpr int FMA = decltype(fma_c)::value;
        static_assert(FMA >= 1 && FMA <= C::FM, "active row blocks");
        const unsigned char *sB = sA + C::A_BYTES;
        bf16x8 af[C::KH][FMA];
        bf16x8 bfr[C::KH][2][C::FN]; // [k half][panel][16-column block]
#pragma unroll
        for (int h2 = 0; h2 < C::KH; ++h2) {
            const int kk = h2 * 32;
#pragma unroll
            for (int fm = 0; fm < FMA; ++fm) {
                const int r = wm * C::WTM + fm * 16 + fr;
                const int piece = aswz<C::PIECES>(r, (kk >> 3) + fk);
                af[h2][fm] = *reinterpret_cast<const bf16x8 *>(sA + r * (BK * 2) + piece * 16);
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const unsigned char *sP = sB + p * (BK * PW * 2);
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn) {
                    const int nb = wn * C::WTN + fn * 16 + 4 * tq; // column this lane reads
                    v4i16 half[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int kr = kk + 8 * fk + 4 * h + tr;
                        const int u = (nb >> 4) ^ bswz(kr);
                        const unsigned char *addr = sP + kr * (PW * 2) + u * 32 + (nb & 15) * 2;
                        half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(addr));
                    }
                    bfr[h2][p][fn] = __builtin_bit_cast(
                        bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
                }
            }
        }
#pragma unroll
        for (int h2 = 0; h2 < C::KH; ++h2)
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
                    for (int fm = 0; fm < FMA; ++fm)
                        acc[p][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            bfr[h2][p][fn], af[h2][fm], acc[p][fm][fn], 0, 0, 0);
        constexpr int NDS = C::KH * (FMA + 4 * C::FN), NMF = C::KH * 2 * C::FN * FMA;
        constexpr int FIRST = FMA + 2, PAIRS = NDS - FIRST;
        static_assert(PAIRS <= NMF, "read schedule");
        __builtin_amdgcn_sched_group_barrier(0x100, FIRST, 0);
#pragma unroll
        for (int i = 0; i < PAIRS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NMF - PAIRS, 0);
    };

    // The output tiles, written through LDS: in the MFMA layout a lane holds
    // 4 columns of one row, so direct stores write 32-byte pieces of 16 rows
    // per instruction, and those stores measured a fifth of GEMM2's time and a
    // fourteenth of GEMM1's.  Instead the tile passes
    // through the LDS stage the last K step used (no copy of the next tile
    // targets it before the next tile's first barrier) PR rows at a time and
    // is stored as whole rows, 16 bytes per lane: GEMM2's 256 output columns,
    // GEMM1's 128 act columns and, when GEMM1 saves the pre-activation for the
    // backward, in a second sweep its gate and up panels (`hpart`) into the
    // two halves of h.  Same values, same rounding.  The pipelined launch
    // stores device-coherently (other workgroups of the launch read the rows).
    auto epilogue_staged = [&](const Tile &t, unsigned char *stg, bool hpart) {
        const bool g1 = kind_of(t.kind) == KIND_G1 && !hpart;
        constexpr int PR = 32;                                 // rows per pass
        const int ncol = g1 ? TILE_N1 : TILE_N2;                // output columns of the tile
        const int rs = ncol * 2 + 16;                           // bytes per staged row (padded)
        const int cpr = ncol * 2 / 16;                          // 16-byte chunks per row
        const int rd = PR * cpr / (NW * 64);                    // chunks each lane stores per pass
        static_assert(PR * (TILE_N2 * 2 + 16) <= C::STAGE_BYTES && BM % PR == 0 && PR % 16 == 0,
                      "staging");
        static_assert(PR * (TILE_N1 * 2 / 16) % (NW * 64) == 0, "staging reads");
        bf16 *__restrict__ Cout = static_cast<bf16 *>(hpart ? args.hsave : g1 ? args.act : args.o);
        const int ldo = hpart ? 2 * I : g1 ? I : H;
        lds_barrier(); // every wave is done with the last K step's stage
#pragma unroll 1
        for (int q = 0; q < BM / PR; ++q) {
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm) {
                const int rt = wm * C::WTM + fm * 16; // first tile row of the 16-row block
                if (rt < q * PR || rt >= (q + 1) * PR)
                    continue;
                const int rl = rt - q * PR + (lane & 15);
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn) {
                    const int cw = wn * C::WTN + fn * 16 + 4 * (lane >> 4);
                    if (g1) {
                        u32x2 outv;
                        bf16 *o = reinterpret_cast<bf16 *>(&outv);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            o[i] = static_cast<bf16>(silu_f(acc[0][fm][fn][i]) * acc[1][fm][fn][i]);
                        *reinterpret_cast<u32x2 *>(stg + rl * rs + cw * 2) = outv;
                    } else {
#pragma unroll
                        for (int pn = 0; pn < 2; ++pn) {
                            u32x2 outv;
                            bf16 *o = reinterpret_cast<bf16 *>(&outv);
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                o[i] = static_cast<bf16>(acc[pn][fm][fn][i]);
                            *reinterpret_cast<u32x2 *>(stg + rl * rs + (pn * PW + cw) * 2) = outv;
                        }
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): this wave's rows are in LDS
            lds_barrier();
            if (PIPE && g1) {
                // act rows, which GEMM2 tiles of this launch read: device-
                // coherent stores, which are 8 bytes wide, so each lane takes
                // an 8-byte piece and one store instruction covers whole rows
                const int cpr8 = 2 * cpr, rd8 = 2 * rd;
#pragma unroll 1
                for (int j = 0; j < rd8; ++j) {
                    const int ch = (j * NW + wave) * 64 + lane;
                    const int rl = ch / cpr8, c8 = ch - rl * cpr8;
                    const int r = q * PR + rl;
                    const u32x2 v = *reinterpret_cast<const u32x2 *>(stg + rl * rs + c8 * 8);
                    const int dc = hpart && c8 * 4 >= PW ? I - PW : 0;
                    if (r < t.rows)
                        store_coherent(Cout + (int64_t)(t.row0 + r) * ldo + t.n0 + dc + c8 * 4, v);
                }
            } else {
                for (int j = 0; j < rd; ++j) {
                    const int ch = (j * NW + wave) * 64 + lane;
                    const int rl = ch / cpr, cc = ch - rl * cpr;
                    const int r = q * PR + rl;
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + rl * rs + cc * 16);
                    // h: the tile's up panel (staged columns PW..2PW) goes to the second half
                    const int dc = hpart && cc * 8 >= PW ? I - PW : 0;
                    if (r < t.rows)
                        *reinterpret_cast<u32x4 *>(Cout + (int64_t)(t.row0 + r) * ldo + t.n0 + dc + cc * 8) = v;
                }
            }
            lds_barrier(); // the stage is read before the next pass (or the next tile's copies) writes it
        }
    };

    // Counter that a finished tile releases (-1: none).  Every wave bumps it
    // once its own stores of the tile are acknowledged, so a tile is complete
    // at NW bumps per N-tile; the test hook drops one wave's bump.
    auto release_index = [&](const Tile &t) {
        if (!PIPE || t.kind != KIND_G1)
            return -1;
        return (t.mt == args.drop_mt && t.nt == 0 && wave == 0) ? -1 : t.mt;
    };
    // a GEMM2 tile reads the act rows of its M-tile: every GEMM1 N-tile of it
    auto wait_ready = [&](const Tile &t) {
        if (!PIPE || t.kind != KIND_G2)
            return;
        wait_counters(ctr1 + t.mt, NW * ntn1, args);
    };
    Cursor cc;
    cc.tried = 0;
    bool have = false;
    if (PIPE) {
        cc.kind = KIND_G1;
        cc.tail = 0;
        have = claim(cc);
    } else {
        if (MODE != FAST_G2)
            have = phase_begin(KIND_G1, cc);
        if (!have && !G1ONLY)
            have = phase_begin(KIND_G2, cc);
    }

    if (have) {
        Tile cur = decode(cc);
        Tile nxt = cur;
        Src scur, snext;
        make_src(cur, scur);
        // first NSTAGE-1 steps (every tile has at least that many K steps),
        // in flight while the next tile is found and decoded
        wait_ready(cur);
#pragma unroll
        for (int st = 0; st < NSTAGE - 1; ++st)
            issue(scur, st, smem + st * C::STAGE_BYTES);
        Cursor nc = cc;
        bool has_next = advance(nc);
        if (has_next) {
            nxt = decode(nc);
            make_src(nxt, snext);
        }
        // copies run ahead into the next tile only within one GEMM: a GEMM2
        // tile may read this very tile's output
        bool chain = has_next && nxt.kind == cur.kind;
        int s_cur = 0; // stage of the current step (global step index % NSTAGE)
        int owed = -1; // release of the previous tile, made once its stores are done
        while (true) {
            const int nk = (kind_of(cur.kind) == KIND_G1 ? H : I) / BK;
            // a wave whose rows all lie past the expert's count skips the MFMAs;
            // fmv = its 16-row blocks that hold rows
            const bool active = wm * C::WTM < cur.rows;
            const int fmv = min(C::FM, (cur.rows - wm * C::WTM + 15) >> 4);
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < C::FN; ++fn)
                        acc[p][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
            // the K loop of the tile, instantiated once per count of active row
            // blocks (a wave-uniform choice made per tile, outside the loop)
            auto kloop = [&](auto fma_c) {
            for (int kb = 0; kb < nk; ++kb) {
                // wait for this wave's copies of the current step (copy groups
                // issued after it may stay in flight), publish the stage, run
                // the step's MFMAs, then start the copies of step
                // kb + NSTAGE - 1 into the stage the previous step used (after
                // the MFMAs are issued, so they start right at the barrier:
                // prefill GEMM1 on 128-row tiles 335 -> 323 us against issuing
                // the copies first)
                const int ahead = min(NSTAGE - 2, nk - 1 - kb + (chain ? NSTAGE - 1 : 0));
                if (ahead >= 2)
                    wait_vm<2 * C::NL>();
                else if (ahead == 1)
                    wait_vm<C::NL>();
                else
                    wait_vm<0>();
                // by step NSTAGE - 2 of a tile every copy group still allowed in
                // flight was issued after the previous tile's epilogue stores,
                // so those are acknowledged: release that tile
                if (PIPE && kb == NSTAGE - 2 && owed >= 0) {
                    bump(args.ctr + owed);
                    owed = -1;
                }
                lds_barrier();
                const int s_next = s_cur == 0 ? NSTAGE - 1 : s_cur - 1; // (step + NSTAGE - 1) % NSTAGE
                const int step = kb + NSTAGE - 1;
                if (active)
                    compute(fma_c, smem + s_cur * C::STAGE_BYTES);
                if (step < nk) {
                    issue(scur, step, smem + s_next * C::STAGE_BYTES);
                } else if (chain) {
                    if (step == nk)
                        wait_ready(nxt);
                    issue(snext, step - nk, smem + s_next * C::STAGE_BYTES);
                }
                s_cur = s_cur == NSTAGE - 1 ? 0 : s_cur + 1;
            }
            };
            if constexpr (C::FM == 8) {
                if (fmv > 6)
                    kloop(IC<8>{});
                else if (fmv > 4)
                    kloop(IC<6>{});
                else if (fmv > 2)
                    kloop(IC<4>{});
                else
                    kloop(IC<2>{});
            } else if constexpr (C::FM == 4) {
                if (fmv > 2)
                    kloop(IC<4>{});
                else
                    kloop(IC<2>{});
            } else {
                kloop(IC<C::FM>{});
            }
            {
                unsigned char *stg = smem + ((s_cur + NSTAGE - 1) % NSTAGE) * C::STAGE_BYTES;
                epilogue_staged(cur, stg, false);
                if (MODE == FAST_G1H || (PIPE && args.hsave && kind_of(cur.kind) == KIND_G1))
                    epilogue_staged(cur, stg, true);
            }
            const int done = release_index(cur);
            if (!has_next) {
                if (done >= 0) {
                    wait_vm<0>();
                    bump(args.ctr + done);
                }
                break;
            }
            const bool chained = chain;
            cur = nxt;
            scur = snext;
            has_next = advance(nc);
            if (has_next) {
                nxt = decode(nc);
                make_src(nxt, snext);
            }
            chain = has_next && nxt.kind == cur.kind;
            if (chained) {
                owed = done;
            } else {
                // A new GEMM: release the finished tile, then refill the
                // pipeline.  Every stage but the last step's was left behind by
                // all waves at the last barrier: s_cur, s_cur + 1, ... (mod
                // NSTAGE).  Each wave releases before it waits for the new
                // tile's inputs, so no wait depends on a release behind it.
                if (done >= 0) {
                    wait_vm<0>();
                    bump(args.ctr + done);
                }
                wait_ready(cur);
#pragma unroll
                for (int st = 0; st < NSTAGE - 1; ++st)
                    issue(scur, st, smem + ((s_cur + st) % NSTAGE) * C::STAGE_BYTES);
            }
        }
    }

    if (PIPE)
        wait_vm<0>(); // no copy into this workgroup's LDS outlives it
}

template <int BM, int MODE, int NWAVES = waves_for(BM)>
static hipError_t launch(const FastFwdArgs &a, int num_cus, hipStream_t stream)
{
    // 8 / NWAVES workgroups per CU (8 waves per CU), whole XCDs
    const int grid = a.grid > 0 ? a.grid : (num_cus + 7) / 8 * 8 * (8 / NWAVES);
    hipLaunchKernelGGL((moe_fwd_bf16<BM, MODE, NWAVES>), dim3((unsigned)grid), dim3(64 * NWAVES),
                       0, stream, a);
    return hipGetLastError();
}

} // namespace fast

bool fast_gemm_supported(int dtype, int64_t H, int64_t I)
{
    return dtype == 1 && H % fast::TILE_N2 == 0 && I % fast::TILE_N1 == 0;
}

template <int MODE>
static hipError_t launch_bm(int BM, const FastFwdArgs &a, int num_cus, hipStream_t stream)
{
    if (BM == 64)
        return fast::launch<64, MODE>(a, num_cus, stream);
    if (BM == 128)
        return fast::launch<128, MODE>(a, num_cus, stream);
    return fast::launch<256, MODE>(a, num_cus, stream);
}

hipError_t launch_fast_fwd(int mode, int BM, const FastFwdArgs &a, int num_cus, hipStream_t stream)
{
    if (a.T <= 0)
        return hipSuccess;
    if (BM != 64 && BM != 128 && BM != 256)
        return hipErrorInvalidValue;
    switch (mode) {
    case FAST_G1: return launch_bm<FAST_G1>(BM, a, num_cus, stream);
    case FAST_G1H: return launch_bm<FAST_G1H>(BM, a, num_cus, stream);
    case FAST_G2: return launch_bm<FAST_G2>(BM, a, num_cus, stream);
    default: return launch_bm<FAST_PIPE>(BM, a, num_cus, stream);
    }
}

} // namespace moe
