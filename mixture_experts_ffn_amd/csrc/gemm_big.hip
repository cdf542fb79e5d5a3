// gemm_big.hip — the forward bf16 grouped GEMMs (GEMM1 + SwiGLU, GEMM2) of the
// MoE expert FFN on 256 x 256 block tiles, one 4-wave workgroup per CU.
//
// The operations (HyperMegaMoE issue page, section 2.1: GMM1/up_proj with the
// SwiGLU epilogue, GMM2/down_proj):
//   GEMM1: act[p, j] = silu(x[t_p] · W1[e][:, j]) · (x[t_p] · W1[e][:, I + j])
//   GEMM2: o[p, :]   = act[p, :] · W2[e]
//
// Tile engine for long expert segments, laid out for the CDNA4 compute unit:
//  * one workgroup of 4 waves per CU; each wave owns a 128 x 128 block of the
//    256-row x 256-column tile (2 x 2 waves: rows wm*128.., columns wn*64..
//    of each of the two 128-column weight panels) in 256 accumulator
//    registers.  Per flop this moves a third fewer bytes from L2 into LDS and
//    from LDS into registers than two workgroups of 128 x 256 tiles, the
//    layout of gemm_mfma.hip, which serves shorter segments;
//  * the matrix-core step is the 16 x 16 x 32 bf16 one, one per 32-deep K step
//    and output block, in ascending k, as in gemm_mfma.hip: every element is
//    the same chain of fp32 MFMA accumulations whichever kernel or tile
//    height computes it, so the outputs agree bit for bit;
//  * one wave per SIMD: nothing else covers a stall, so each step is
//    hand-scheduled as fenced groups of one MFMA plus at most one fragment
//    read or copy, and the fragments are software-pipelined across the
//    per-step barrier: the MFMAs of the first weight panel run while the
//    second panel's fragments are read, those of the second panel while the
//    next step's token rows and first panel are read (each token-row block
//    right after its last MFMA, into the same registers);
//  * global -> LDS copies land directly in a 4-stage ring (32 KB per 32-deep
//    K step), each step's issued NSTAGE - 1 steps ahead into the stage whose
//    reads ended at the previous barrier;
//  * token rows (K-contiguous, gathered through sorted_slot) and weight panels
//    (N-contiguous) are swizzled as in gemm_mfma.hip: conflict-free 128-bit
//    row-fragment reads and transposing 64-bit weight reads;
//  * the output tile passes through the last step's LDS stage 64 rows at a
//    time and is stored as whole rows (GEMM1: act, and h when saving it for
//    the backward; GEMM2: o);
//  * persistent: each XCD walks a contiguous eighth of the tile order (expert
//    major, groups of M-tiles with N outer), its workgroups strided through
//    it (the last two rounds, from six on, by tickets), so tiles in flight on
//    one XCD share weight panels and token rows in its L2; a tile's last
//    steps already copy the next tile's first steps.
// A tile's rows are split between the two wave rows in 32-row steps (a tile
// of r rows gives the first ceil(r / 64) * 32 of them to wave row 0 and the
// rest to wave row 1), and each wave multiplies only the 16-row blocks that
// hold rows (rounded up to an even count).
#include "common.h"
#include "kernels.h"
#include "tile_common.h"

namespace moe {
namespace big {
using namespace tile;

constexpr int BM = 256;                       // rows per tile
constexpr int BK = 32;                        // K per step (one MFMA deep)
#ifndef MOE_BIG_NSTAGE
#define MOE_BIG_NSTAGE 4
#endif
constexpr int NSTAGE = MOE_BIG_NSTAGE;        // LDS ring depth
constexpr int NW = 4;                         // waves per workgroup
constexpr int A_BYTES = BM * BK * 2;          // token rows of one step (16 KB)
constexpr int B_BYTES = BK * 2 * PW * 2;      // two weight panels of one step (16 KB)
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int A_LOADS = A_BYTES / 1024 / NW;  // 1 KB copy chunks per wave per step
constexpr int B_LOADS = B_BYTES / 1024 / NW;
constexpr int NL = A_LOADS + B_LOADS;         // copy instructions per wave per step
constexpr int A_ROWS = A_LOADS * (1024 / (BK * 2)); // token rows one wave copies
constexpr int PIECES = BK / 8;                // 16-byte pieces per token row
constexpr int RPC = 1024 / (BK * 2);          // token rows per 1 KB chunk
constexpr int CPP = BK / 4;                   // 1 KB chunks per weight panel (4 k-rows each)
constexpr int WTM = 128, WTN = 64;            // rows, columns per panel of one wave
constexpr int FM = WTM / 16, FN = WTN / 16;   // 16 x 16 blocks per wave and panel
constexpr int HALF = FM * FN;                 // MFMAs of one panel per step
static_assert(NSTAGE * STAGE_BYTES <= 160 * 1024, "LDS");
static_assert(A_LOADS * NW * 1024 == A_BYTES && B_LOADS * NW * 1024 == B_BYTES, "copy split");
static_assert(HALF == 4 * NL && HALF == 4 * 2 * FN && FN == 4, "one read and one copy per 4 MFMAs");
static_assert(NSTAGE == 4 && A_ROWS * NW == BM, "two copy groups stay in flight; waves' rows tile the tile");

// fragments of one step: token rows (MFMA B operand), and one panel's weight
// columns (MFMA A operand, two transposing reads of 4 k values each)
struct XFrag {
    bf16x8 x[FM];
};
struct WFrag {
    v4i16 h[FN][2];
};

// Position of a workgroup in its XCD's slice [lo, hi) of the tile order:
// round j of the walk takes tile lo + j*step + slot, or + (step - 1 - slot) in
// odd rounds, so that where full and partial M-tiles alternate in the order
// no workgroup gets only the expensive ones.  With six rounds or more, the
// last two rounds of every slice (from offset `tail` on) go by tickets
// instead, to the workgroups that finish first: with the strided walk alone
// the launch ends with the workgroups that hold one tile more or whose tiles
// ran slower (weight panels fetched from memory rather than a cache), while
// the others idle.
struct Cursor {
    int lo, hi, step, j;
    int send;  // end of the strided rounds of this slice
    int tail;  // offset in each slice of the ticketed tiles (-1: none)
    int L;     // the claimed tile, once the walk takes tickets
    int tried; // slices found exhausted
    bool tick; // the walk takes tickets
};

// Reads an accumulator element (an AGPR) into a VGPR exactly here: volatile
// asm keeps the compiler from hoisting all 256 accumulator reads of the
// epilogue to the end of the K loop, which would need 256 more VGPRs.
__device__ __forceinline__ float acc_rd(float a)
{
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

// SKIP: waves leave out the copies of token rows that lie past a tile's rows
// (for launches where many tiles are short: a per-step choice of wait that
// costs launches of full tiles about 8 %, so it is compiled only where used)
template <int MODE, bool SKIP>
__global__ __launch_bounds__(64 * NW, 1) void moe_fwd_bf16_big(FastFwdArgs args)
{
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * STAGE_BYTES];
    constexpr bool G1 = MODE == FAST_G1 || MODE == FAST_G1H;
    constexpr int KIND = G1 ? KIND_G1 : KIND_G2;
    const int H = args.H, I = args.I;
    const int ntn = G1 ? I / TILE_N1 : H / TILE_N2;
    const int nk = (G1 ? H : I) / BK;
    const int mtiles = uni(ldc(args.mtile_off, args.E));
    const int per_xcd_wg = gridDim.x >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int lane = threadIdx.x & 63;
    const int wave = uni(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // this XCD's eighth of the tile order, walked by its workgroups
    const int total = mtiles * ntn;
    const int range = (total + 7) >> 3;
    Cursor cc;
    {
        cc.step = per_xcd_wg;
        cc.lo = xcd * range;
        cc.hi = min((xcd + 1) * range, total);
        cc.j = 0;
        const int rounds = (range + cc.step - 1) / cc.step;
        cc.tail = rounds >= 6 ? (rounds - 2) * cc.step : -1;
        cc.send = cc.tail >= 0 ? min(cc.hi, cc.lo + cc.tail) : cc.hi;
        cc.L = 0;
        cc.tried = 0;
        cc.tick = false;
    }
    auto pos = [&](const Cursor &c) __attribute__((always_inline)) {
        return c.tick ? c.L : c.lo + c.j * c.step + ((c.j & 1) ? c.step - 1 - slot : slot);
    };
    // A ticket of the slices' ticketed tiles, this XCD's slice first: wave 0
    // draws it from the slice's counter (zeroed by the routing kernel; this
    // GEMM's eight of them) and passes it to the other waves through LDS.
    __shared__ int tick_bcast[2];
    int tick_par = 0;
    auto claim = [&](Cursor &c) {
        for (; c.tried < 8; ++c.tried) {
            const int x = (xcd + c.tried) & 7;
            const int hi = min((x + 1) * range, total);
            const int lo = min(x * range + c.tail, hi);
            if (wave == 0 && lane == 0)
                tick_bcast[tick_par] =
                    lo < hi ? __hip_atomic_fetch_add(args.tickets + (G1 ? 0 : 8) + x, 1,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : 0x7fffffff;
            __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): the ticket is in LDS
            lds_barrier();
            const int t = tick_bcast[tick_par];
            tick_par ^= 1;
            if (t < hi - lo) {
                c.L = lo + t;
                return true;
            }
        }
        return false;
    };
    // the walk's next tile; false when none is left
    auto advance = [&](Cursor &c) {
        if (!c.tick) {
            c.j += 1;
            if (pos(c) < c.send)
                return true;
            if (c.tail < 0)
                return false;
            c.tick = true;
        }
        return claim(c);
    };
    if (pos(cc) >= cc.send) {
        if (cc.tail < 0)
            return;
        cc.tick = true;
        if (!claim(cc))
            return;
    }

    // Copy sources of one tile: a wave-uniform base per operand and a 32-bit
    // byte offset per lane and copy (the host takes this kernel only when the
    // token-row tensors stay below 4 GiB)
    struct Src {
        uint32_t a[A_LOADS];
        uint32_t b[B_LOADS];
        const unsigned char *wbase; // weight matrix of the tile's expert
        int ldb;                    // its row stride (elements)
        bool skip_a;                // this wave's token rows all lie past the tile's
    };
    const unsigned char *abase =
        static_cast<const unsigned char *>(G1 ? args.x : args.act); // token rows
    const int lda = G1 ? H : I;
    auto make_src = [&](const Tile &t, Src &sr) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            // chunk c covers token rows RPC*c .. RPC*c + RPC-1 of the tile
            const int c = wave * A_LOADS + i;
            const int r = c * RPC + lane / PIECES;
            const int piece = aswz<PIECES>(r, lane % PIECES);
            uint32_t grow;
            if (G1) {
                // the chunk's gather indices are wave-uniform and consecutive:
                // one wide scalar load (sorted_slot is padded past its end by
                // more than a tile); rows past the expert's count copy row 0
                const __attribute__((address_space(4))) int32_t *ix =
                    (const __attribute__((address_space(4))) int32_t *)args.sorted_slot +
                    uni(t.row0 + c * RPC);
                const int idx0 = ldc(args.sorted_slot, t.row0);
                int v = 0;
#pragma unroll
                for (int j = 0; j < RPC; ++j) {
                    const int idx = c * RPC + j < t.rows ? ix[j] : idx0;
                    v = lane / PIECES == j ? idx : v;
                }
                grow = (uint32_t)(v / args.K);
            } else {
                grow = (uint32_t)(t.row0 + (r < t.rows ? r : 0));
            }
            sr.a[i] = grow * (uint32_t)(lda * 2) + (uint32_t)(piece * 16);
        }
        // a shared-expert chunk c = e - Er reads its column chunk of the shared
        // up_proj (rows of 2Is, up panel Is columns in) or its row chunk of the
        // shared down_proj
        const bool shd = args.sh.S > 0 && t.e >= args.sh.Er;
        const int64_t sc = t.e - args.sh.Er;
        const bf16 *W =
            G1 ? (shd ? static_cast<const bf16 *>(args.sh.w1) + sc * I
                      : static_cast<const bf16 *>(args.w1) + (int64_t)t.e * H * (2 * I))
               : (shd ? static_cast<const bf16 *>(args.sh.w2) + sc * I * H
                      : static_cast<const bf16 *>(args.w2) + (int64_t)t.e * I * H);
        sr.wbase = reinterpret_cast<const unsigned char *>(W);
        sr.ldb = G1 ? 2 * (shd ? args.sh.Is : I) : H;
        // This wave copies token rows A_ROWS * wave .. + A_ROWS - 1.  When they
        // all lie past the tile's rows no wave reads them (the row split
        // below never reaches a 32-row step past the last row), so the wave
        // leaves them out: a third of prefill's GEMM2 rows are such padding.
        sr.skip_a = SKIP && wave * A_ROWS >= t.rows;
        const int pstride = G1 ? (shd ? args.sh.Is : I) : PW; // column offset of the second panel
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            // chunk c covers 1024 bytes = 4 k-rows of one 128-column panel
            const int c = wave * B_LOADS + i;
            const int panel = c / CPP;
            const int kr = (c % CPP) * 4 + (lane >> 4);
            const int pp = lane & 15;
            const int u = (pp >> 1) ^ bswz(kr);
            const int col = t.n0 + panel * pstride + (2 * u + (pp & 1)) * 8;
            sr.b[i] = (uint32_t)(kr * sr.ldb + col) * 2u;
        }
    };
    // copy i (0 .. NL-1: the A chunks, then the B chunks) of step kb of a
    // tile into a stage
    auto copy_one = [&](const Src &sr, int kb, int stage, int i) __attribute__((always_inline)) {
        unsigned char *sbase = smem + stage * STAGE_BYTES;
        const int k0 = kb * BK;
        if (i < A_LOADS) {
            if (!(SKIP && sr.skip_a))
                g2l16s(abase + (size_t)k0 * 2, sr.a[i],
                       (lds_void *)(sbase + (wave * A_LOADS + i) * 1024));
        } else
            g2l16s(sr.wbase + (size_t)k0 * sr.ldb * 2, sr.b[i - A_LOADS],
                   (lds_void *)(sbase + A_BYTES + (wave * B_LOADS + i - A_LOADS) * 1024));
    };
    auto issue = [&](const Src &sr, int kb, int stage) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NL; ++i)
            copy_one(sr, kb, stage, i);
    };
    // copies in one group (one step) of a tile's sources
    auto group_size = [&](const Src &sr) { return SKIP && sr.skip_a ? B_LOADS : NL; };
    // Wait until the oldest of this wave's three copy groups in flight has
    // landed, the two younger ones (n copies together) may stay in flight.
    // (Stores issued between them only make the wait stricter.)
    auto wait_groups = [&](int n) __attribute__((always_inline)) {
        if (!SKIP || n >= 2 * NL)
            wait_vm<2 * NL>();
        else if (n >= NL + B_LOADS)
            wait_vm<NL + B_LOADS>();
        else
            wait_vm<2 * B_LOADS>();
    };

    // Fragment reads of one step from a stage.  Token-row block fm: lane l
    // reads row l % 16 of the 16-row block, the 8 k values 8 (l / 16) .. (one
    // 128-bit read).  Weight block fn of panel p, half h: the transposing
    // read serves 16 lanes with a 4 (k) x 16 (column) block, lane group
    // g = l / 16 at k 8 g + 4 h .., lane l % 16 receiving column l % 16.
    const int fr = lane & 15, fk = lane >> 4;
    const int tq = lane & 3, tr = (lane >> 2) & 3;
    // The tile's rows are split between the two row halves at 32-row
    // granularity: half 0 takes ceil(rows / 64) * 32 rows, half 1 the rest
    // (split = 128 for a full tile), so a short tile costs its waves about
    // proportionally less and only half 1's last 32-row group is padded.
    int split = WTM;
    auto read_x = [&](XFrag &X, int stage, int fm) __attribute__((always_inline)) {
        const unsigned char *sA = smem + stage * STAGE_BYTES;
        const int r = wm * split + fm * 16 + fr;
        const int piece = aswz<PIECES>(r, fk);
        X.x[fm] = *reinterpret_cast<const bf16x8 *>(sA + r * (BK * 2) + piece * 16);
    };
    auto read_w = [&](WFrag &W, int stage, int p, int q) __attribute__((always_inline)) {
        const int fn = q >> 1, h = q & 1;
        const unsigned char *sP = smem + stage * STAGE_BYTES + A_BYTES + p * (BK * PW * 2);
        const int nb = wn * WTN + fn * 16 + 4 * tq;
        const int kr = 8 * fk + 4 * h + tr;
        const int u = (nb >> 4) ^ bswz(kr);
        W.h[fn][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16 *)(sP + kr * (PW * 2) + u * 32 + (nb & 15) * 2));
    };

    f32x4 acc[2][FM][FN];
    // MFMA (fm, fn) of panel p
    auto mma_one = [&](const XFrag &X, const WFrag &W, int p, int fm, int fn) __attribute__((always_inline)) {
        const bf16x8 w = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(W.h[fn][0], W.h[fn][1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[p][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, X.x[fm], acc[p][fm][fn], 0, 0, 0);
    };

    // The output tile through LDS, 64 rows per pass: in pass q every wave
    // stages its 16-row blocks 2q and 2q + 1 (staging rows wm*32 ..), then the
    // four waves store the 64 rows (tile rows wm*128 + 32 q ..) as whole rows.
    // A staged row's 16-byte units are XOR-swizzled by the row, so 64 rows of
    // 256 columns fill exactly one 32 KB stage and the 8-byte writes of 16
    // rows spread over the banks.  In the 16 x 16 result layout lane l holds
    // row l % 16 and columns 4 (l / 16) + [0, 4) of a 16-column block.  The
    // passes are unrolled, so each accumulator has one use per pass kind:
    // the act (GEMM1) or o (GEMM2) pass, and for the training GEMM1 the h
    // pass of the same rows right after it.
    auto stage_store = [&](const Tile &t, unsigned char *stg, int q, int kind)
        __attribute__((always_inline)) {
        // kind 0: act (128 columns), 1: o (256), 2: h (gate | up panels, 256)
        const int rsb = kind == 0 ? TILE_N1 * 2 : TILE_N2 * 2; // bytes per staged row
        const int cpr = rsb / 16;                               // 16-byte units per row
        const int umask = cpr - 1;
#pragma unroll
        for (int f2 = 0; f2 < 2; ++f2) {
            const int fm = 2 * q + f2;
            const int sr = wm * 32 + f2 * 16 + fr; // this lane's staging row
            unsigned char *srow = stg + sr * rsb;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int u = wn * 8 + fn * 2 + (fk >> 1); // 16-byte unit of columns 4 fk ..
                const int hb = 8 * (fk & 1);               // its 8-byte half
                if (kind == 0) {
                    u32x2 outv;
                    bf16 *o = reinterpret_cast<bf16 *>(&outv);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        o[i] = static_cast<bf16>(silu_f(acc_rd(acc[0][fm][fn][i])) *
                                                 acc_rd(acc[1][fm][fn][i]));
                    *reinterpret_cast<u32x2 *>(srow + ((u ^ (sr & umask)) << 4) + hb) = outv;
                } else {
#pragma unroll
                    for (int pn = 0; pn < 2; ++pn) {
                        u32x2 outv;
                        bf16 *o = reinterpret_cast<bf16 *>(&outv);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            o[i] = static_cast<bf16>(acc_rd(acc[pn][fm][fn][i]));
                        const int up = pn * 16 + u;
                        *reinterpret_cast<u32x2 *>(srow + ((up ^ (sr & umask)) << 4) + hb) = outv;
                    }
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): this wave's rows are in LDS
        lds_barrier();
        bf16 *__restrict__ Cout = static_cast<bf16 *>(kind == 2 ? args.hsave : kind == 0 ? args.act : args.o);
        const int ldo = kind == 2 ? 2 * I : kind == 0 ? I : H;
        const int rd = 64 * cpr / (NW * 64); // units each lane stores
        for (int j = 0; j < rd; ++j) {
            const int ch = (j * NW + wave) * 64 + lane;
            const int rl = ch / cpr, cu = ch - rl * cpr;
            const int hr = rl >> 5, local = q * 32 + (rl & 31); // row half, row within it
            const int hrows = hr == 0 ? min(split, t.rows) : t.rows - split;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + rl * rsb + ((cu ^ (rl & umask)) << 4));
            // h: the tile's up panel (staged columns PW..2PW) goes to the second half
            const int dc = kind == 2 && cu * 8 >= PW ? I - PW : 0;
            if (local < hrows)
                *reinterpret_cast<u32x4 *>(Cout + (int64_t)(t.row0 + hr * split + local) * ldo + t.n0 +
                                           dc + cu * 8) = v;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f); // staged rows read before the next pass writes
        lds_barrier();
    };
    auto epilogue = [&](const Tile &t, unsigned char *stg) __attribute__((always_inline)) {
        static_assert(64 * TILE_N2 * 2 <= STAGE_BYTES, "staging");
#pragma unroll
        for (int q = 0; q < FM / 2; ++q) {
            if (q * 32 >= min(split, t.rows)) // no row of either half in this pass (uniform)
                break;
            stage_store(t, stg, q, G1 ? 0 : 1);
            if (MODE == FAST_G1H)
                stage_store(t, stg, q, 2);
        }
    };

    Tile cur = decode_tile(args, KIND, pos(cc), ntn, BM);
    Tile nxt = cur;
    Src scur, snext;
    make_src(cur, scur);
    // Ring schedule (stage of a step = its global step index % NSTAGE): a
    // step's copies are issued NSTAGE - 1 steps ahead, during the first half
    // of an earlier step, into the stage whose reads all ended at that step's
    // previous barrier.  The next tile's steps continue the same sequence, so
    // a tile's last steps already copy the next tile's first ones; the
    // epilogue stages through the stage of the tile's last step, which the
    // next tile's first step refills after the epilogue.  Every step issues
    // one copy group: past the last tile it re-copies that tile's last step
    // into a stage nobody reads again, so every wait counts the same.
    // prologue: steps 0 .. NSTAGE-2 of the first tile, in flight while the
    // next tile is found and decoded
#pragma unroll
    for (int st = 0; st < NSTAGE - 1; ++st)
        issue(scur, st, st);
    Cursor nc = cc;
    bool has_next = advance(nc);
    if (has_next) {
        nxt = decode_tile(args, KIND, pos(nc), ntn, BM);
        make_src(nxt, snext);
    }
    int sg = 0; // stage of the current step
    XFrag XA;
    WFrag W0, W1;
    split = ((cur.rows + 63) >> 6) << 5;
    // size of the copy group issued last (the prologue's, of the first tile)
    int gprev = group_size(scur);
    wait_groups(2 * gprev);
    lds_barrier();
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
        read_x(XA, 0, fm);
#pragma unroll
    for (int q = 0; q < 2 * FN; ++q)
        read_w(W0, 0, 0, q);

    while (true) {
        // this wave's 16-row blocks that hold rows, rounded up to even
        const int wrows = wm == 0 ? min(split, cur.rows) : cur.rows - split;
        const int fmv = wrows <= 0 ? 0 : min(FM, ((wrows + 31) >> 5) * 2);
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[p][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
        // One step on the token rows in X (panel-0 fragments in W0), which
        // its second half replaces with the next step's.  Hand-scheduled as
        // fenced groups of one MFMA and at most one read or copy, row block
        // by row block (fm outer): first half, the panel-0 MFMAs with the
        // panel-1 reads and this step's copy group (one each per 4 MFMAs);
        // then the wait and the barrier that publish the next step's stage;
        // second half, the panel-1 MFMAs, each row block's token rows for
        // the next step read right after its last MFMA (so they reuse its
        // registers), with the next step's panel-0 reads.  MFMAs of row
        // blocks past this wave's rows are left out.
        auto step = [&](auto fma_c, XFrag &X, int kb) __attribute__((always_inline)) {
            constexpr int FMA = decltype(fma_c)::value;
            const int sprev = sg == 0 ? NSTAGE - 1 : sg - 1; // stage of the previous step
            const int snxt = sg == NSTAGE - 1 ? 0 : sg + 1;  // stage of the next step
            const int ahead = kb + NSTAGE - 1;
            const bool own = ahead < nk;
            const bool use_next = !own && has_next;
            Src cs;
#pragma unroll
            for (int i = 0; i < A_LOADS; ++i)
                cs.a[i] = use_next ? snext.a[i] : scur.a[i];
#pragma unroll
            for (int i = 0; i < B_LOADS; ++i)
                cs.b[i] = use_next ? snext.b[i] : scur.b[i];
            cs.wbase = use_next ? snext.wbase : scur.wbase;
            cs.ldb = use_next ? snext.ldb : scur.ldb;
            cs.skip_a = use_next ? snext.skip_a : scur.skip_a;
            const int gsz = group_size(cs);
            const int ckb = own ? ahead : has_next ? ahead - nk : nk - 1;
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
                const int fm = j / FN, fn = j % FN;
                if (fm < FMA)
                    mma_one(X, W0, 0, fm, fn);
                if ((j & 3) == 0)
                    read_w(W1, sg, 1, j >> 2);
                if ((j & 3) == 2)
                    copy_one(cs, ckb, sprev, j >> 2);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the next step (this tile's kb + 1 or, chained, the next tile's
            // step 0) must have landed; the NSTAGE - 2 copy groups issued
            // after it (the previous step's and this one's) may stay in flight
            wait_groups(gprev + gsz);
            gprev = gsz;
            __builtin_amdgcn_s_waitcnt(0xc07f); // this wave's reads of the stage are done
            lds_barrier();
            // (after a tile's last step these reads are repeated after the
            // epilogue, so that no fragment stays live across it)
#pragma unroll
            for (int j = 0; j < HALF; ++j) {
                const int fm = j / FN, fn = j % FN;
                if (fm < FMA)
                    mma_one(X, W1, 1, fm, fn);
                if (fn == FN - 1)
                    read_x(X, snxt, fm);
                if (fn == 1)
                    read_w(W0, snxt, 0, fm);
                __builtin_amdgcn_sched_barrier(0);
            }
            sg = snxt;
        };
        auto kloop = [&](auto fma_c) __attribute__((always_inline)) {
            for (int kb = 0; kb < nk; ++kb)
                step(fma_c, XA, kb);
        };
        if (fmv >= 8)
            kloop(IC<8>{});
        else if (fmv == 6)
            kloop(IC<6>{});
        else if (fmv == 4)
            kloop(IC<4>{});
        else if (fmv == 2)
            kloop(IC<2>{});
        else
            kloop(IC<0>{});

        // stage of the tile's last step: all its reads ended before the last
        // barrier, and the next copy into it is the next tile's first step's
        unsigned char *stg = smem + (sg == 0 ? NSTAGE - 1 : sg - 1) * STAGE_BYTES;
        epilogue(cur, stg);
        if (!has_next) {
            wait_vm<0>(); // no copy into this workgroup's LDS outlives it
            break;
        }
        // the next tile's step 0 (landed, published by the last barrier),
        // with the next tile's row split
        cur = nxt;
        split = ((cur.rows + 63) >> 6) << 5;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            read_x(XA, sg, fm);
#pragma unroll
        for (int q = 0; q < 2 * FN; ++q)
            read_w(W0, sg, 0, q);
        scur = snext;
        has_next = advance(nc);
        if (has_next) {
            nxt = decode_tile(args, KIND, pos(nc), ntn, BM);
            make_src(nxt, snext);
        }
    }
}

template <int MODE, bool SKIP>
static hipError_t launch(const FastFwdArgs &a, int num_cus, hipStream_t stream)
{
    // one workgroup per CU, whole XCDs
    const int grid = a.grid > 0 ? a.grid : (num_cus + 7) / 8 * 8;
    hipLaunchKernelGGL((moe_fwd_bf16_big<MODE, SKIP>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                       a);
    return hipGetLastError();
}

} // namespace big

hipError_t launch_fast_fwd_big(int mode, const FastFwdArgs &a, int num_cus, hipStream_t stream,
                              bool skip_padding)
{
    if (a.T <= 0)
        return hipSuccess;
    switch (mode) {
    case FAST_G1: return big::launch<FAST_G1, false>(a, num_cus, stream);
    case FAST_G1H: return big::launch<FAST_G1H, false>(a, num_cus, stream);
    case FAST_G2:
        return skip_padding ? big::launch<FAST_G2, true>(a, num_cus, stream)
                            : big::launch<FAST_G2, false>(a, num_cus, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace moe
