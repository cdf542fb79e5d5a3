// gemm_engine.hip — the bf16 grouped-GEMM engine of the MoE expert FFN on
// gfx950 matrix cores: all six contractions of the layer, forward and
// backward, as instances of one persistent, LDS-pipelined kernel.
//
// The contractions (HyperMegaMoE issue page, section 2.1 "forward fusion" and
// section 2.2 "backward fusion"); p is a permuted (expert-contiguous) row,
// t_p its token, g_p its gate, e its expert:
//
//   F1  act = SwiGLU(x[t_p] · W1[e])        M = rows of e, N = I, K = H
//   F2  o   = act[p] · W2[e]                M = rows of e, N = H, K = I
//   B2  u   = dY[t_p] · W2[e]^T, epilogue:  M = rows of e, N = I, K = H
//       dact = g_p u, dh = [dact ⊙ b ⊙ σ(a)(1 + a(1-σ(a))), dact ⊙ silu(a)],
//       act_g = g_p silu(a) ⊙ b and per-row partials of Σ_i u·act (= d_g)
//   B4  dx_p = dh[p] · W1[e]^T              M = rows of e, N = H, K = 2I
//   B5  dW2[e] = Σ_p act_g[p]^T dY[t_p]     M = I, N = H, K = rows of e
//   B7  dW1[e] = Σ_p x[t_p]^T dh[p]         M = H, N = 2I, K = rows of e
//
// Operand layouts in memory decide the LDS layout and the fragment read:
//  * KROW: the operand's M (or N) rows are contiguous along K (x, act, dY,
//    dh rows; W2 rows for B2; W1 rows for B4).  LDS tile [R][BK] with the
//    16-byte piece index XOR-ed by (row / 2) % 8 (BK = 64); fragments are one
//    128-bit LDS read.
//  * KCOL: memory rows are K indices, contiguous along M (or N) (W1/W2 in
//    the forward; act_g, dY, x, dh rows in the weight gradients).  LDS tile
//    [BK][R] untransposed with the 32-byte unit index XOR-ed by a 3-bit hash
//    of k; fragments are two transposing 64-bit LDS reads.
//  Both swizzles were measured conflict-free.  Copies go global -> LDS
//  directly (16 bytes per lane); pieces outside the problem (K or N edges,
//  rows past an expert's count in the weight gradients) copy from a zero
//  page, so no tile needs a special path.
//
// Pipeline: 8 waves per CU, 3-stage LDS ring, copies two K steps ahead; one
// 8-wave workgroup with BK = 64 (144 KB), or for the weight gradients two
// 4-wave workgroups with BK = 32 (72 KB each), whose per-step barriers hold
// only one of the two waves on a SIMD.  A producer cursor walks the workgroup's tile sequence two
// steps ahead of the consumer, across tile boundaries and over tiles without
// K steps (empty experts), so the next tile's first copies overlap the
// current tile's tail and epilogue.  Each wave waits only for its own copies
// of the stage it consumes (vmcnt), then one barrier publishes the stage; a
// step's copies are issued after its MFMAs.
//
// Matrix-core step: v_mfma_f32_16x16x32_bf16 with the B fragment as the first
// operand, so the accumulator block is C^T and each lane holds row
// (lane % 16) and columns 4 (lane / 16) + [0, 4) of a 16x16 block.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace eng {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int NSTAGE = 3; // LDS ring depth

// Swizzled 16-byte piece of KROW row r (rows of PIECES pieces): 128-byte rows
// XOR by (r / 2) % 8, 64-byte rows by (r / 4) % 4, so the 16 rows one 128-bit
// fragment read touches fall in 16 different bank groups.
template <int PIECES> __device__ __forceinline__ int krow_piece(int r, int q)
{
    static_assert(PIECES == 8 || PIECES == 4, "KROW row length");
    return PIECES == 8 ? q ^ ((r >> 1) & 7) : q ^ ((r >> 2) & 3);
}

// A page of zeros that out-of-problem pieces copy from.
__device__ __attribute__((aligned(256))) const uint32_t kZeroPage[64] = {0};

enum Kind { F1 = 0, F2 = 1, B2 = 2, B4 = 3, B5 = 4, B7 = 5 };
enum Lay { KROW = 0, KCOL = 1 };

template <int KIND> struct KindTraits;
// token-tiled kinds: M = permuted rows of one expert
template <> struct KindTraits<F1> {
    static constexpr bool TOKEN_M = true, A_GATHER = true, B_GATHER = false, PAIRED = true;
    static constexpr int ALAY = KROW, BLAY = KCOL;
};
template <> struct KindTraits<F2> {
    static constexpr bool TOKEN_M = true, A_GATHER = false, B_GATHER = false, PAIRED = false;
    static constexpr int ALAY = KROW, BLAY = KCOL;
};
template <> struct KindTraits<B2> {
    static constexpr bool TOKEN_M = true, A_GATHER = true, B_GATHER = false, PAIRED = false;
    static constexpr int ALAY = KROW, BLAY = KROW;
};
template <> struct KindTraits<B4> {
    static constexpr bool TOKEN_M = true, A_GATHER = false, B_GATHER = false, PAIRED = false;
    static constexpr int ALAY = KROW, BLAY = KROW;
};
// feature-tiled kinds: K = permuted rows of one expert
template <> struct KindTraits<B5> {
    static constexpr bool TOKEN_M = false, A_GATHER = false, B_GATHER = true, PAIRED = false;
    static constexpr int ALAY = KCOL, BLAY = KCOL;
};
template <> struct KindTraits<B7> {
    static constexpr bool TOKEN_M = false, A_GATHER = true, B_GATHER = false, PAIRED = false;
    static constexpr int ALAY = KCOL, BLAY = KCOL;
};

// Workgroup shape per kind.  The weight gradients (KCOL A: k-rows of 256
// bytes or more in every copy) run as two 4-wave workgroups per CU with
// BK = 32, so each SIMD holds one wave of each and one workgroup's per-step
// barrier holds only its own wave.  The kinds with KROW operands keep one
// 8-wave workgroup with BK = 64: their copies fetch BK * 2 bytes per row, and
// 64-byte row pieces (half a cache line) measured slower than the gain.
template <int KIND> struct Shape {
    static constexpr bool SPLIT = KindTraits<KIND>::ALAY == KCOL;
    static constexpr int NW = SPLIT ? 4 : 8;   // waves per workgroup
    static constexpr int BK = SPLIT ? 32 : 64; // K per step
    static constexpr int WGPC = SPLIT ? 2 : 1; // workgroups per CU
};

template <int KIND, int BM_, int WM_> struct Cfg {
    using KT = KindTraits<KIND>;
    static constexpr int NW = Shape<KIND>::NW;
    static constexpr int BK = Shape<KIND>::BK;
    static constexpr int WGPC = Shape<KIND>::WGPC;
    static constexpr int KPIECES = BK / 8;         // KROW: 16-byte pieces per row
    static constexpr int KRPC = 1024 / (BK * 2);   // KROW: rows per 1 KB copy chunk
    static constexpr int KCPP = BK / 4;            // paired KCOL: chunks per 128-column panel
    static constexpr int BM = BM_;
    static constexpr int BNT = 256;                      // B columns staged per tile
    static constexpr int PW = KT::PAIRED ? 128 : 256;    // columns per panel
    static constexpr int NPANEL = KT::PAIRED ? 2 : 1;
    static constexpr int OUT_N = KT::PAIRED ? 128 : 256; // output columns per tile
    static constexpr int WAVES_M = WM_;
    static constexpr int WAVES_N = NW / WAVES_M;
    static constexpr int WTM = BM / WAVES_M;
    static constexpr int WTN = PW / WAVES_N; // per panel
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BK * BNT * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int A_LOADS = A_BYTES / 1024 / NW;
    static constexpr int B_LOADS = B_BYTES / 1024 / NW;
    static constexpr int NL = A_LOADS + B_LOADS;
    static_assert(A_LOADS * NW * 1024 == A_BYTES && B_LOADS * NW * 1024 == B_BYTES, "split");
    static_assert(FM >= 1 && FN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
    static_assert(NSTAGE * STAGE_BYTES <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int bswz(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

// 16-byte global -> LDS copy per lane into [l, l + 1024) (lane i at l + 16 i),
// issued as inline assembly so that the compiler does not track these LDS
// writes: completion is established per stage with wait_vm, instead of the
// compiler waiting for every copy in flight before each LDS read.  `l` must
// be wave-uniform.  M0 is not used by any compiler-generated code here.
__device__ __forceinline__ void g2l16(const void *g, lds_void *l)
{
    const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_addr), "v"(g)
                 : "memory", "m0");
}

// wait until at most N vector-memory operations of this wave are in flight
template <int N> __device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Barrier of the K loop.  Inside the loop LDS is written only by the
// global->LDS copies, whose completion each wave establishes itself before
// arriving, and read only into registers that the matrix cores consume
// before the wave can arrive again; so no memory fence is needed, only a
// compiler-level ordering of LDS accesses around the barrier.  (A fence would
// also wait for the copies of later stages still in flight.)
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct TileInfo {
    int e;     // expert
    int m0;    // token-tiled: first permuted row; feature-tiled: first feature row
    int rows;  // valid M rows of the tile
    int n0;    // first output column
    int seg0;  // feature-tiled: first permuted row of the expert (K origin)
    int klen;  // contraction length of the tile (Kd, or the expert's row count)
    int nk;    // K steps
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Load of routing metadata (offsets, M-tile tables, sorted_slot) that earlier
// launches wrote and this kernel only reads: through the constant address
// space, so a wave-uniform address becomes a scalar load.
__device__ __forceinline__ int ldc(const int32_t *p, int i)
{
    return ((const __attribute__((address_space(4))) int32_t *)p)[uni(i)];
}

// All fields are wave-uniform; readfirstlane keeps the decode on the scalar
// unit (scalar loads, tracked by lgkmcnt) so it never waits for the copies in
// flight on the vector-memory counter.
template <int KIND, int BM, int WM>
__device__ __forceinline__ TileInfo decode_tile(const EngineArgs &a, int L)
{
    using C = Cfg<KIND, BM, WM>;
    TileInfo t;
    L = uni(L);
    if constexpr (C::KT::TOKEN_M) {
        const int ntn = (a.N + C::OUT_N - 1) / C::OUT_N;
        t.e = ldc(a.mtile_expert, L / ntn);
        const int mt0 = ldc(a.mtile_off, t.e);
        const int mt_e = ldc(a.mtile_off, t.e + 1) - mt0;
        const int local = L - mt0 * ntn;
        constexpr int GM = 8;
        const int grp = local / (GM * ntn);
        const int first_m = grp * GM;
        const int gm = min(mt_e - first_m, GM);
        const int rr = local - grp * GM * ntn;
        const int n_t = rr / gm;
        const int m_t = first_m + rr % gm;
        t.m0 = ldc(a.offsets, t.e) + m_t * BM;
        t.rows = min(BM, ldc(a.offsets, t.e + 1) - t.m0);
        t.n0 = n_t * C::OUT_N;
        t.seg0 = 0;
        t.klen = a.Kd;
    } else {
        const int mtm = (a.M + BM - 1) / BM, ntn = (a.N + C::OUT_N - 1) / C::OUT_N;
        t.e = L / (mtm * ntn);
        const int local = L - t.e * mtm * ntn;
        // groups of GM feature tiles, N outer: the 32 tiles in flight on one
        // XCD then span 8 M-tiles x 4 N-tiles of one expert (their operand
        // blocks fit its L2) instead of 32 M-tiles of one N-tile
        constexpr int GM = 8;
        const int grp = local / (GM * ntn);
        const int first_m = grp * GM;
        const int gm = min(mtm - first_m, GM);
        const int rr = local - grp * GM * ntn;
        const int n_t = rr / gm, m_t = first_m + rr % gm;
        t.m0 = m_t * BM;
        t.rows = min(BM, a.M - t.m0);
        t.n0 = n_t * C::OUT_N;
        t.seg0 = ldc(a.offsets, t.e);
        t.klen = ldc(a.offsets, t.e + 1) - t.seg0;
    }
    t.e = uni(t.e);
    t.m0 = uni(t.m0);
    t.rows = uni(t.rows);
    t.n0 = uni(t.n0);
    t.seg0 = uni(t.seg0);
    t.klen = uni(t.klen);
    t.nk = (t.klen + C::BK - 1) / C::BK;
    return t;
}

template <int KIND, int BM, int WM>
__device__ __forceinline__ int total_tiles(const EngineArgs &a)
{
    using C = Cfg<KIND, BM, WM>;
    const int ntn = (a.N + C::OUT_N - 1) / C::OUT_N;
    if constexpr (C::KT::TOKEN_M)
        return ldc(a.mtile_off, a.E) * ntn;
    else
        return a.E * ((a.M + BM - 1) / BM) * ntn;
}

// The contiguous tile range [lo, hi) of XCD x: an eighth of the tile count, or,
// for the feature-tiled kinds when the backward set-up has computed them, the
// cost-balanced bounds in a.xcd_bounds (a weight-gradient tile's K loop runs
// over its expert's rows, so its cost follows the routing).
template <int KIND, int BM, int WM>
__device__ __forceinline__ void xcd_range(const EngineArgs &a, int x, int &lo, int &hi)
{
    using C = Cfg<KIND, BM, WM>;
    if constexpr (!C::KT::TOKEN_M) {
        if (a.xcd_bounds) {
            lo = ldc(a.xcd_bounds, x);
            hi = ldc(a.xcd_bounds, x + 1);
            return;
        }
    }
    const int total = uni(total_tiles<KIND, BM, WM>(a));
    const int range = (total + 7) >> 3;
    lo = min(x * range, total);
    hi = min((x + 1) * range, total);
}

// Per-lane copy state of one tile.  KROW operands and weight operands are
// affine in k, so one pointer per chunk suffices; token-row KCOL operands
// (the weight gradients) look their rows up per K step.
template <int KIND, int BM, int WM> struct Src {
    using C = Cfg<KIND, BM, WM>;
    const bf16 *a[C::A_LOADS];
    const bf16 *b[C::B_LOADS];
    int a_k[C::A_LOADS];       // KROW: k offset of the lane's piece
    int b_k[C::B_LOADS];
    bool a_col_ok[C::A_LOADS]; // KCOL: column inside the problem
    bool b_col_ok[C::B_LOADS];
    int64_t ldb; // row stride of the tile's weight operand
    int kjump;   // KROW weights: extra offset of k >= Kd / 2 (shared up_proj chunk in B4)
};

// Row indices of the gathered token-row KCOL operand of a weight gradient
// (B7: x rows, B5: dY rows) for one K step: the sorted_slot entries of the
// k-rows this wave copies, read with scalar loads (wave-uniform addresses,
// lgkmcnt) one producer step before the copies that use them, so their
// latency hides behind a K step instead of stalling the copy issue.
template <int KIND, int BM, int WM> struct GatherIdx {
    using C = Cfg<KIND, BM, WM>;
    using KT = typename C::KT;
    static constexpr bool ON_A = KT::A_GATHER && KT::ALAY == KCOL;
    static constexpr bool ON_B = KT::B_GATHER && KT::BLAY == KCOL && !KT::TOKEN_M;
    static constexpr int NCH = ON_A ? C::A_LOADS : ON_B ? C::B_LOADS : 1; // chunks per wave
    static constexpr int RB = ON_A ? BM * 2 : C::PW * 2;                   // bytes per k-row
    static constexpr int KPC = 1024 / RB;                                  // k-rows per chunk
    // index (i, q) at element i * KPC + q; a vector value, so it stays in registers
    typedef int vec __attribute__((ext_vector_type(NCH * KPC)));
    vec v;
};

template <int KIND, int BM, int WM>
__device__ __forceinline__ void fetch_gather(const EngineArgs &a, const TileInfo &t, int kb,
                                             int wave, GatherIdx<KIND, BM, WM> &g)
{
    using G = GatherIdx<KIND, BM, WM>;
    if constexpr (G::ON_A || G::ON_B) {
        // the wave's NCH x KPC k-rows are consecutive, so their indices are one
        // block of sorted_slot, read as one wide scalar load; the block may run
        // past the expert's rows (and up to a K step past the array, which is
        // padded for this): those rows copy zeros whatever their index
        const int base = uni(t.seg0 + kb * Cfg<KIND, BM, WM>::BK + wave * G::NCH * G::KPC);
        const __attribute__((address_space(4))) int32_t *src =
            (const __attribute__((address_space(4))) int32_t *)a.sorted_slot + base;
#pragma unroll
        for (int j = 0; j < G::NCH * G::KPC; ++j)
            g.v[j] = src[j];
    }
}

// Memory row of the lane's k-row for a token-row KCOL operand (weight
// gradients): k-rows kbase .. kbase + KPC - 1 of the chunk are permuted rows
// seg0 + k; a gathered operand maps them through the prefetched indices.
// slot / topk for 0 <= slot < 2^31 by multiply and shift: with l = ceil(log2 d)
// and m = floor(2^(31+l) / d) + 1 (set by launch_engine), floor(v m / 2^(31+l))
// equals floor(v / d) for every v below 2^31 (Granlund and Montgomery,
// "Division by invariant integers using multiplication", section 4).
__device__ __forceinline__ int div_topk(int v, const EngineArgs &a)
{
    return a.topk_l == 0 ? v : (int)(__umulhi((uint32_t)v, a.topk_m) >> (a.topk_l - 1));
}

template <int RB, typename G>
__device__ __forceinline__ int64_t kcol_gather_row(const EngineArgs &a, int lane, const G &g, int i)
{
    constexpr int KPC = 1024 / RB;
    static_assert(KPC == G::KPC, "chunk geometry");
    const int j = lane / (RB / 16);
    int v = g.v[i * KPC];
#pragma unroll
    for (int q = 1; q < KPC; ++q)
        v = j == q ? g.v[i * KPC + q] : v;
    return (int64_t)div_topk(v, a);
}

// k-row of lane within chunk c for a KCOL operand with `RB`-byte k-rows
template <int RB> __device__ __forceinline__ int kcol_krow(int c, int lane)
{
    return c * (1024 / RB) + lane / (RB / 16);
}

template <int KIND, int BM, int WM>
__device__ __forceinline__ void make_src(const EngineArgs &a, const TileInfo &t, int wave, int lane,
                                         Src<KIND, BM, WM> &s)
{
    using C = Cfg<KIND, BM, WM>;
    using KT = typename C::KT;
    // ---- A
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
        const int c = wave * C::A_LOADS + i;
        if constexpr (KT::ALAY == KROW) {
            // chunk c: rows KRPC c .. KRPC c + KRPC-1 of the tile, 16-byte unit `lane`
            constexpr int KRPC = C::KRPC, KPIECES = C::KPIECES;
            const int r = c * KRPC + lane / KPIECES;
            const int piece = krow_piece<KPIECES>(r, lane % KPIECES);
            int64_t mrow;
            if constexpr (KT::A_GATHER) {
                // the chunk's KRPC row indices are wave-uniform: scalar loads
                int idx[KRPC];
#pragma unroll
                for (int j = 0; j < KRPC; ++j) {
                    const int rj = c * KRPC + j < t.rows ? c * KRPC + j : 0; // tail rows repeat row 0
                    idx[j] = ldc(a.sorted_slot, t.m0 + rj);
                }
                int v = idx[0];
#pragma unroll
                for (int j = 1; j < KRPC; ++j)
                    v = lane / KPIECES == j ? idx[j] : v;
                mrow = div_topk(v, a);
            } else {
                mrow = t.m0 + (r < t.rows ? r : 0);
            }
            s.a[i] = a.A + mrow * a.lda + piece * 8;
            s.a_k[i] = piece * 8;
            s.a_col_ok[i] = true;
        } else {
            // KCOL A (feature tiles): chunk c covers 1024 / (2 BM) k-rows of BM columns
            constexpr int RB = BM * 2;       // bytes per k-row
            constexpr int KPC = 1024 / RB;   // k-rows per chunk
            const int pp = lane % (RB / 16); // 16-byte piece within the k-row
            const int u = (pp >> 1) ^ bswz(c * KPC + lane / (RB / 16));
            const int col = t.m0 + (2 * u + (pp & 1)) * 8;
            s.a_col_ok[i] = col < a.M;
            s.a[i] = a.A + (s.a_col_ok[i] ? col : 0); // gathered: row part added per step
            if constexpr (!GatherIdx<KIND, BM, WM>::ON_A) // token rows seg0 + k: k0 rows added per step
                s.a[i] += ((int64_t)t.seg0 + kcol_krow<RB>(c, lane)) * a.lda;
            s.a_k[i] = 0;
        }
    }
    // ---- B
    // weight operand of the tile's expert: a shared-expert chunk (e >= Er) reads
    // its chunk of the shared weights with their own strides
    const bool shd = KT::TOKEN_M && a.Bs && t.e >= a.Er;
    const bf16_t *wbase = shd ? a.Bs + (int64_t)(t.e - a.Er) * a.bs_cstride
                              : a.B + (int64_t)t.e * a.b_estride;
    s.ldb = shd ? a.bs_ldb : a.ldb;
    s.kjump = shd ? a.bs_kjump : 0;
    const int upanel = shd ? a.bs_panel : a.N; // F1: column offset of the up panel
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
        const int c = wave * C::B_LOADS + i;
        if constexpr (KT::BLAY == KROW) {
            // weight rows n of expert e (B2: W2[e][n][:], B4: W1[e][n][:])
            const int r = c * C::KRPC + lane / C::KPIECES;
            const int piece = krow_piece<C::KPIECES>(r, lane % C::KPIECES);
            const int n = t.n0 + r;
            const int nc = n < a.N ? n : 0; // tail columns repeat column 0; never stored
            s.b[i] = wbase + (int64_t)nc * s.ldb + piece * 8;
            s.b_k[i] = piece * 8;
            s.b_col_ok[i] = true;
        } else {
            int panel, kr, pp;
            if constexpr (KT::PAIRED) { // two 128-column panels: 256-byte k-rows
                panel = c / C::KCPP;
                kr = (c % C::KCPP) * 4 + (lane >> 4);
                pp = lane & 15;
            } else { // one 256-column panel: 512-byte k-rows
                panel = 0;
                kr = c * 2 + (lane >> 5);
                pp = lane & 31;
            }
            const int u = (pp >> 1) ^ bswz(kr);
            const int colp = t.n0 + (2 * u + (pp & 1)) * 8; // column within the panel
            s.b_col_ok[i] = colp < a.N;
            s.b_k[i] = 0;
            if constexpr (KT::TOKEN_M) // weight operand: memory rows are k
                s.b[i] = wbase + (int64_t)kr * s.ldb + (s.b_col_ok[i] ? colp : 0) + panel * upanel;
            else if constexpr (GatherIdx<KIND, BM, WM>::ON_B) // gathered token operand: row per step
                s.b[i] = a.B + (s.b_col_ok[i] ? colp : 0) + panel * a.N;
            else // token rows seg0 + k: k0 rows added per step
                s.b[i] = a.B + (s.b_col_ok[i] ? colp : 0) + panel * a.N +
                         ((int64_t)t.seg0 + kcol_krow<C::PW * 2>(c, lane)) * a.ldb;
        }
    }
}

template <int KIND, int BM, int WM>
__device__ __forceinline__ void issue(const EngineArgs &a, const TileInfo &t,
                                      const Src<KIND, BM, WM> &s, int kb, lds_u8 *sbase,
                                      int wave, int lane, const GatherIdx<KIND, BM, WM> &g)
{
    using C = Cfg<KIND, BM, WM>;
    using KT = typename C::KT;
    using G = GatherIdx<KIND, BM, WM>;
    const int k0 = kb * C::BK;
    // ---- A
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
        lds_void *dst = (lds_void *)(sbase + (wave * C::A_LOADS + i) * 1024);
        const void *src;
        if constexpr (KT::ALAY == KROW) {
            src = (k0 + s.a_k[i] < t.klen) ? (const void *)(s.a[i] + k0) : (const void *)kZeroPage;
        } else {
            constexpr int RB = BM * 2;
            const int kr = kcol_krow<RB>(wave * C::A_LOADS + i, lane);
            const int kk = k0 + kr;
            const bf16_t *p;
            if constexpr (G::ON_A)
                p = s.a[i] + kcol_gather_row<RB>(a, lane, g, i) * a.lda;
            else
                p = s.a[i] + (int64_t)k0 * a.lda;
            src = (s.a_col_ok[i] && kk < t.klen) ? (const void *)p : (const void *)kZeroPage;
        }
        g2l16(src, dst);
    }
    // ---- B
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
        lds_void *dst = (lds_void *)(sbase + C::A_BYTES + (wave * C::B_LOADS + i) * 1024);
        const void *src;
        if constexpr (KT::BLAY == KROW) {
            const int kk = k0 + s.b_k[i];
            const bf16_t *p = s.b[i] + k0;
            if constexpr (KIND == B4) // a shared up_proj chunk: the up half starts Is - I further on
                p += kk >= (a.Kd >> 1) ? s.kjump : 0;
            src = kk < t.klen ? (const void *)p : (const void *)kZeroPage;
        } else if constexpr (KT::TOKEN_M) {
            constexpr int RB = C::PW * 2;
            const int c = wave * C::B_LOADS + i;
            const int kr = KT::PAIRED ? (c % C::KCPP) * 4 + (lane >> 4) : kcol_krow<RB>(c, lane);
            src = (s.b_col_ok[i] && k0 + kr < t.klen) ? (const void *)(s.b[i] + (int64_t)k0 * s.ldb)
                                                       : (const void *)kZeroPage;
        } else {
            constexpr int RB = C::PW * 2;
            const int kr = kcol_krow<RB>(wave * C::B_LOADS + i, lane);
            const int kk = k0 + kr;
            const bf16_t *p;
            if constexpr (G::ON_B)
                p = s.b[i] + kcol_gather_row<RB>(a, lane, g, i) * a.ldb;
            else
                p = s.b[i] + (int64_t)k0 * a.ldb;
            src = (s.b_col_ok[i] && kk < t.klen) ? (const void *)p : (const void *)kZeroPage;
        }
        g2l16(src, dst);
    }
}

// fragment reads ------------------------------------------------------------
// KROW tile [R][BK]: row r, 8 k values starting at logical piece q
template <int BK>
__device__ __forceinline__ bf16x8 frag_krow(const unsigned char *tile, int r, int q)
{
    return *reinterpret_cast<const bf16x8 *>(tile + r * (BK * 2) + krow_piece<BK / 8>(r, q) * 16);
}
// KCOL tile [BK][R] (R*2-byte k-rows): lane's column block nb (multiple of 16),
// 8 k values starting at k8 (multiple of 8); two transposing reads
template <int RB>
__device__ __forceinline__ bf16x8 frag_kcol(const unsigned char *tile, int nb, int k8, int lane)
{
    const int col = nb + 4 * (lane & 3);
    const int tr = (lane >> 2) & 3;
    v4i16 half[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int kr = k8 + 4 * h + tr;
        const int u = (col >> 4) ^ bswz(kr);
        half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16 *)(tile + kr * RB + u * 32 + (col & 15) * 2));
    }
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// epilogues ------------------------------------------------------------------
// lane (fm, fn) element i: row wm*WTM + fm*16 + (lane % 16) of the tile,
// column wn*WTN + fn*16 + 4 (lane / 16) + i of panel p.
// Epilogue of F1 (the ragged-shape GEMM1): act = silu(gate) * up from the two
// panels' accumulators, and with a saved-h buffer the raw gate and up halves,
// stored directly (8 bytes per lane: row lane & 15, columns 4 * (lane >> 4)).
template <int KIND, int BM, int WM>
__device__ __forceinline__ void epilogue_f1(const EngineArgs &a, const TileInfo &t,
                                            f32x4 (&acc)[Cfg<KIND, BM, WM>::NPANEL][Cfg<KIND, BM, WM>::FM]
                                                        [Cfg<KIND, BM, WM>::FN],
                                            int wm, int wn, int lane)
{
    using C = Cfg<KIND, BM, WM>;
    static_assert(KIND == F1 && C::NPANEL == 2, "F1 only");
    auto pack4 = [](float v0, float v1, float v2, float v3) {
        u32x2 r;
        bf16 *o = reinterpret_cast<bf16 *>(&r);
        o[0] = static_cast<bf16>(v0);
        o[1] = static_cast<bf16>(v1);
        o[2] = static_cast<bf16>(v2);
        o[3] = static_cast<bf16>(v3);
        return r;
    };
    const int cl = 4 * (lane >> 4);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
        const int r = wm * C::WTM + fm * 16 + (lane & 15);
        if (r >= t.rows)
            continue;
        const int64_t p = t.m0 + r;
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) {
            const int c = t.n0 + wn * C::WTN + fn * 16 + cl;
            if (c >= a.N)
                continue;
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = silu_f(acc[0][fm][fn][i]) * acc[1][fm][fn][i];
            *reinterpret_cast<u32x2 *>(a.C + p * a.ldc + c) = pack4(o[0], o[1], o[2], o[3]);
            if (a.C2) {
                *reinterpret_cast<u32x2 *>(a.C2 + p * 2 * a.N + c) =
                    pack4(acc[0][fm][fn][0], acc[0][fm][fn][1], acc[0][fm][fn][2], acc[0][fm][fn][3]);
                *reinterpret_cast<u32x2 *>(a.C2 + p * 2 * a.N + a.N + c) =
                    pack4(acc[1][fm][fn][0], acc[1][fm][fn][1], acc[1][fm][fn][2], acc[1][fm][fn][3]);
            }
        }
    }
}

// Epilogue of the kinds with one bf16 output array (the input gradient, the
// shared expert's second GEMM, both weight gradients).  In the MFMA layout a
// lane holds 4 columns of one row, so direct stores write 8-byte pieces of 16
// rows per instruction.  Instead the tile passes through the LDS stage that
// the last K step consumed (the copies in flight target the other two stages,
// and the next tile's first barrier precedes the next copy into this one),
// PR rows per pass, and is stored as whole rows, 16 bytes per lane.  Same
// values, same rounding as the direct stores.
template <int KIND, int BM, int WM>
__device__ __forceinline__ void epilogue_staged(const EngineArgs &a, const TileInfo &t,
                                                f32x4 (&acc)[Cfg<KIND, BM, WM>::NPANEL]
                                                            [Cfg<KIND, BM, WM>::FM][Cfg<KIND, BM, WM>::FN],
                                                int wm, int wn, int wave, int lane, unsigned char *stg)
{
    using C = Cfg<KIND, BM, WM>;
    constexpr int PR = 32;                     // rows per pass
    constexpr int RS = C::OUT_N * 2 + 16;      // bytes per staged row (padded)
    constexpr int CPR = C::OUT_N * 2 / 16;     // 16-byte chunks per row
    constexpr int RD = PR * CPR / (C::NW * 64); // chunks each lane stores per pass
    static_assert(C::NPANEL == 1 && PR * RS <= C::STAGE_BYTES && BM % PR == 0 && PR % 16 == 0 &&
                      RD * C::NW * 64 == PR * CPR,
                  "staging");
    bf16 *out = a.C;
    int64_t ld = a.ldc;
    int cjump = 0;
    if constexpr (KIND == B5 || KIND == B7) {
        // dW[e] [M, N]; a shared-expert chunk writes its rows (B5) or its gate
        // and up column chunks (B7) of the shared gradient
        const bool shd = a.Cs && t.e >= a.Er;
        out = shd ? a.Cs + (int64_t)(t.e - a.Er) * a.cs_cstride : a.C + (int64_t)t.e * a.M * a.N;
        ld = shd ? a.cs_ldc : a.N;
        cjump = shd ? a.cs_cjump : 0;
    }
    const int cl = 4 * (lane >> 4);
    lds_barrier(); // every wave is done reading the last K step's stage
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
                u32x2 v;
                bf16 *o = reinterpret_cast<bf16 *>(&v);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    o[i] = static_cast<bf16>(acc[0][fm][fn][i]);
                *reinterpret_cast<u32x2 *>(stg + rl * RS + (wn * C::WTN + fn * 16 + cl) * 2) = v;
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): this wave's rows are in LDS
        lds_barrier();
#pragma unroll
        for (int j = 0; j < RD; ++j) {
            const int ch = (j * C::NW + wave) * 64 + lane;
            const int rl = ch / CPR, cc = ch - rl * CPR;
            const int r = q * PR + rl, c = t.n0 + cc * 8; // N is a multiple of 8
            const u32x4 v = *reinterpret_cast<const u32x4 *>(stg + rl * RS + cc * 16);
            if (r < t.rows && c < a.N) {
                u32x4 *dst = reinterpret_cast<u32x4 *>(out + (int64_t)(t.m0 + r) * ld + c +
                                                       (c >= (a.N >> 1) ? cjump : 0));
                // the weight gradients are written once and not read again
                // by the layer: stored with the non-temporal hint, they do not
                // displace cached operands (forward + backward step -1 %, the
                // following step's GEMM1 454 -> 438 us)
                if constexpr (KIND == B5 || KIND == B7)
                    __builtin_nontemporal_store(v, dst);
                else
                    *dst = v;
            }
        }
        lds_barrier(); // read before the next pass (or the next tile's copies) writes the stage
    }
}

// Act-gradient epilogue through LDS.  The fp32 tile of u = dy W2^T passes
// through the last K step's stage PR rows at a time; each lane then finishes
// 8 consecutive columns of one row, so the saved pre-activation is read and
// the three outputs (both halves of dh, act_g) are written 16 bytes per lane
// as whole rows.  The row partial of Σ u act keeps its layout, one value per
// 64 columns, now summed over 8 lanes of 8 columns each.  Every gate, slot and
// pre-activation load of the tile is issued before the first pass (rows and
// columns outside the tile read row 0 / the first column instead).
template <int BM, int WM>
__device__ __forceinline__ void epilogue_b2_staged(const EngineArgs &a, const TileInfo &t,
                                                   f32x4 (&acc)[1][Cfg<B2, BM, WM>::FM][Cfg<B2, BM, WM>::FN],
                                                   int wm, int wn, int wave, int lane, unsigned char *stg)
{
    using C = Cfg<B2, BM, WM>;
    constexpr int PR = 32;                      // rows per pass
    constexpr int NP = BM / PR;                 // passes
    constexpr int RS = C::OUT_N * 4 + 16;       // bytes per staged fp32 row (padded)
    constexpr int CPR = C::OUT_N / 8;           // 8-column chunks per row
    constexpr int RPW = 64 / CPR;               // rows a wave finishes per read step
    constexpr int RD = PR / (C::NW * RPW);      // read steps per pass
    static_assert(PR * RS <= C::STAGE_BYTES && BM % PR == 0 && PR % 16 == 0 && CPR == 32 &&
                      RD * C::NW * RPW == PR && C::WTN == 64 && C::OUT_N == C::WAVES_N * 64,
                  "staging");
    const int I = a.N;
    const int cc = lane % CPR;                  // this lane's chunk of every row it finishes
    const int c = t.n0 + cc * 8;
    const bool cok = c < I;                     // I is a multiple of 8
    const int cs = cok ? c : t.n0;
    auto row_of = [&](int q, int j) { return q * PR + (j * C::NW + wave) * RPW + lane / CPR; };
    float gv[NP][RD];
    u32x4 hav[NP][RD], hbv[NP][RD];
    {
        int slot[NP][RD];
#pragma unroll
        for (int q = 0; q < NP; ++q)
#pragma unroll
            for (int j = 0; j < RD; ++j) {
                const int r = row_of(q, j);
                const int64_t p = t.m0 + (r < t.rows ? r : 0);
                slot[q][j] = a.sorted_slot[p];
                hav[q][j] = *reinterpret_cast<const u32x4 *>(a.Hs + p * 2 * I + cs);
                hbv[q][j] = *reinterpret_cast<const u32x4 *>(a.Hs + p * 2 * I + I + cs);
            }
        // rows of the shared expert's chunks (from offsets[Er] on) have gate 1
        const int64_t shared_row0 = a.Bs && a.Er < a.E ? (int64_t)ldc(a.offsets, a.Er) : INT64_MAX;
#pragma unroll
        for (int q = 0; q < NP; ++q)
#pragma unroll
            for (int j = 0; j < RD; ++j)
                gv[q][j] = t.m0 + row_of(q, j) >= shared_row0 ? 1.0f : a.gates[slot[q][j]];
    }
    const int cl = 4 * (lane >> 4);
    lds_barrier(); // every wave is done reading the last K step's stage
#pragma unroll
    for (int q = 0; q < NP; ++q) {
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            const int rt = wm * C::WTM + fm * 16;
            if (rt < q * PR || rt >= (q + 1) * PR)
                continue;
            const int rl = rt - q * PR + (lane & 15);
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn)
                *reinterpret_cast<f32x4 *>(stg + rl * RS + (wn * C::WTN + fn * 16 + cl) * 4) = acc[0][fm][fn];
        }
        __builtin_amdgcn_s_waitcnt(0xc07f); // lgkmcnt(0): this wave's rows are in LDS
        lds_barrier();
        // Every load of the epilogue has landed before the first store.  The
        // stores are conditional, so a wait placed by the compiler after one
        // cannot count it and would drain every store issued so far.
        if (q == 0)
            wait_vm<0>();
#pragma unroll
        for (int j = 0; j < RD; ++j) {
            const int r = row_of(q, j);
            const bool ok = r < t.rows && cok;
            const int64_t p = t.m0 + (r < t.rows ? r : 0);
            const f32x4 u0 = *reinterpret_cast<const f32x4 *>(stg + (r - q * PR) * RS + cc * 32);
            const f32x4 u1 = *reinterpret_cast<const f32x4 *>(stg + (r - q * PR) * RS + cc * 32 + 16);
            const bf16 *ha = reinterpret_cast<const bf16 *>(&hav[q][j]);
            const bf16 *hb = reinterpret_cast<const bf16 *>(&hbv[q][j]);
            const float g = gv[q][j];
            u32x4 oa, ob, og;
            bf16 *pa = reinterpret_cast<bf16 *>(&oa), *pb = reinterpret_cast<bf16 *>(&ob),
                 *pg = reinterpret_cast<bf16 *>(&og);
            float dg = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                // dact = g u; dh = [dact b σ(a)(1 + a(1-σ(a))), dact silu(a)]; act_g = g silu(a) b
                const float u = i < 4 ? u0[i] : u1[i - 4];
                const float av = static_cast<float>(ha[i]), bv = static_cast<float>(hb[i]);
                const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-av));
                const float sl = av * sg;
                const float act = sl * bv;
                const float dact = g * u;
                pa[i] = static_cast<bf16>(dact * bv * sg * (1.0f + av * (1.0f - sg)));
                pb[i] = static_cast<bf16>(dact * sl);
                pg[i] = static_cast<bf16>(g * act);
                dg += u * act;
            }
            if (ok) {
                *reinterpret_cast<u32x4 *>(a.C + p * 2 * I + c) = oa;
                *reinterpret_cast<u32x4 *>(a.C + p * 2 * I + I + c) = ob;
                *reinterpret_cast<u32x4 *>(a.C2 + p * I + c) = og;
            }
            // per-row partial over the 64 columns of 8 neighbouring lanes
            dg = ok ? dg : 0.f;
            dg += __shfl_xor(dg, 1, 64);
            dg += __shfl_xor(dg, 2, 64);
            dg += __shfl_xor(dg, 4, 64);
            if (r < t.rows && (lane & 7) == 0)
                a.dgp[p * a.dgp_stride + (t.n0 / C::OUT_N) * C::WAVES_N + cc / 8] = dg;
        }
        lds_barrier(); // read before the next pass (or the next tile's copies) writes the stage
    }
}

template <int KIND, int BM, int WM>
__global__ __launch_bounds__(64 * Shape<KIND>::NW, Shape<KIND>::WGPC) void engine_kernel(EngineArgs a)
{
    using C = Cfg<KIND, BM, WM>;
    using KT = typename C::KT;
    constexpr int BK = C::BK;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * C::STAGE_BYTES];

    const int per_xcd_wg = gridDim.x >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    int lo, hi;
    xcd_range<KIND, BM, WM>(a, xcd, lo, hi);
    lo = uni(lo);
    hi = uni(hi);
    const int L0 = lo + slot;
    if (L0 >= hi)
        return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

    // producer cursor: the next K step to copy
    int pL = L0, pkb = 0;
    TileInfo pt = decode_tile<KIND, BM, WM>(a, pL);
    Src<KIND, BM, WM> ps;
    make_src<KIND, BM, WM>(a, pt, wave, lane, ps);
    bool pvalid = true;
    auto p_skip_empty = [&]() {
        while (pvalid && pkb >= pt.nk) {
            pL += per_xcd_wg;
            pkb = 0;
            pvalid = pL < hi;
            if (pvalid) {
                pt = decode_tile<KIND, BM, WM>(a, pL);
                make_src<KIND, BM, WM>(a, pt, wave, lane, ps);
            }
        }
    };
    p_skip_empty();
    // row indices of the producer's next step (gathered weight-gradient operands);
    // in the K loop they are fetched after the step's MFMAs, so the barrier
    // wait covers their latency before the next step's first LDS wait
    GatherIdx<KIND, BM, WM> pg;
    auto fetch = [&]() {
        if (pvalid)
            fetch_gather<KIND, BM, WM>(a, pt, pkb, wave, pg);
    };
    int gstage_issue = 0; // stage the producer writes next
    int inflight = 0;     // steps copied but not yet consumed
    auto produce = [&]() {
        // the stage as an LDS pointer formed here, beside the shared array:
        // each copy's M0 is then one scalar add, not a null-checked
        // conversion of a generic pointer
        issue<KIND, BM, WM>(a, pt, ps, pkb, (lds_u8 *)(smem + gstage_issue * C::STAGE_BYTES), wave,
                            lane, pg);
        gstage_issue = gstage_issue == NSTAGE - 1 ? 0 : gstage_issue + 1;
        ++inflight;
        ++pkb;
        p_skip_empty();
    };
    fetch();
    if (pvalid)
        produce();
    fetch();
    if (pvalid)
        produce();
    fetch();

    f32x4 acc[C::NPANEL][C::FM][C::FN];
    int cstage = 0;

    for (int L = L0; L < hi; L += per_xcd_wg) {
        const TileInfo t = decode_tile<KIND, BM, WM>(a, L);
#pragma unroll
        for (int p = 0; p < C::NPANEL; ++p)
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn)
                    acc[p][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int kb = 0; kb < t.nk; ++kb) {
            // this step's copies are the oldest in flight; the next step's may stay
            if (inflight > 1)
                wait_vm<C::NL>();
            else
                wait_vm<0>();
            lds_barrier();
            --inflight;
            const unsigned char *sA = smem + cstage * C::STAGE_BYTES;
            const unsigned char *sB = sA + C::A_BYTES;
            cstage = cstage == NSTAGE - 1 ? 0 : cstage + 1;
            // all fragments of the K step first, then the MFMAs; the LDS pipe
            // and the matrix cores are close to balanced, so the interleave is
            // pinned: the first MFMA group's operands, then one read per MFMA
            constexpr int KH = BK / 32;
            bf16x8 af[KH][C::FM];
            bf16x8 bf[KH][C::NPANEL][C::FN];
#pragma unroll
            for (int h2 = 0; h2 < KH; ++h2) {
                const int kk = h2 * 32;
#pragma unroll
                for (int fm = 0; fm < C::FM; ++fm) {
                    if constexpr (KT::ALAY == KROW)
                        af[h2][fm] = frag_krow<BK>(sA, wm * C::WTM + fm * 16 + (lane & 15),
                                               (kk >> 3) + (lane >> 4));
                    else
                        af[h2][fm] = frag_kcol<BM * 2>(sA, wm * C::WTM + fm * 16,
                                                       kk + 8 * (lane >> 4), lane);
                }
#pragma unroll
                for (int p = 0; p < C::NPANEL; ++p) {
#pragma unroll
                    for (int fn = 0; fn < C::FN; ++fn) {
                        const int nb = p * C::PW + wn * C::WTN + fn * 16;
                        if constexpr (KT::BLAY == KROW)
                            bf[h2][p][fn] = frag_krow<BK>(sB, nb + (lane & 15), (kk >> 3) + (lane >> 4));
                        else if constexpr (KT::PAIRED)
                            bf[h2][p][fn] = frag_kcol<C::PW * 2>(sB + p * (BK * C::PW * 2),
                                                                 wn * C::WTN + fn * 16,
                                                                 kk + 8 * (lane >> 4), lane);
                        else
                            bf[h2][p][fn] = frag_kcol<C::PW * 2>(sB, nb, kk + 8 * (lane >> 4), lane);
                    }
                }
            }
#pragma unroll
            for (int h2 = 0; h2 < KH; ++h2)
#pragma unroll
                for (int p = 0; p < C::NPANEL; ++p)
#pragma unroll
                    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
                        for (int fm = 0; fm < C::FM; ++fm)
                            acc[p][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                bf[h2][p][fn], af[h2][fm], acc[p][fm][fn], 0, 0, 0);
            {
                constexpr int RA = KT::ALAY == KROW ? 1 : 2, RB = KT::BLAY == KROW ? 1 : 2;
                constexpr int NDS = KH * (C::FM * RA + C::NPANEL * C::FN * RB);
                constexpr int NMF = KH * C::NPANEL * C::FN * C::FM;
                constexpr int FIRST = C::FM * RA + RB;
                constexpr int PAIRS = NDS - FIRST < NMF ? NDS - FIRST : NMF;
                __builtin_amdgcn_sched_group_barrier(0x100, FIRST, 0);
#pragma unroll
                for (int i = 0; i < PAIRS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, NMF - PAIRS, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, NDS - FIRST - PAIRS, 0);
            }
            // the step's copies after its MFMAs, so that these start right at
            // the barrier (act-grad 310 -> 299 us, input-grad -1 %, against
            // issuing the copies first)
            __builtin_amdgcn_sched_barrier(0);
            if (pvalid)
                produce();
            if constexpr (GatherIdx<KIND, BM, WM>::ON_A || GatherIdx<KIND, BM, WM>::ON_B) {
                __builtin_amdgcn_sched_barrier(0);
                fetch();
            }
        }
        if constexpr (KIND == B2)
            epilogue_b2_staged<BM, WM>(a, t, acc, wm, wn, wave, lane,
                                       smem + (cstage == 0 ? NSTAGE - 1 : cstage - 1) * C::STAGE_BYTES);
        else if constexpr (KIND == F1)
            epilogue_f1<KIND, BM, WM>(a, t, acc, wm, wn, lane);
        else
            epilogue_staged<KIND, BM, WM>(a, t, acc, wm, wn, wave, lane,
                                          smem + (cstage == 0 ? NSTAGE - 1 : cstage - 1) * C::STAGE_BYTES);
    }
}

template <int KIND, int BM, int WM>
static hipError_t launch(const EngineArgs &a, int num_cus, hipStream_t stream)
{
    using S = Shape<KIND>;
    const int grid = (num_cus + 7) / 8 * 8 * S::WGPC; // whole XCDs
    hipLaunchKernelGGL((engine_kernel<KIND, BM, WM>), dim3((unsigned)grid), dim3(64 * S::NW), 0,
                       stream, a);
    return hipGetLastError();
}

} // namespace eng

void engine_feature_tiling(int kind, int M, int N, int num_cus, int *tiles_per_expert,
                           int *wg_per_xcd)
{
    using namespace eng;
    // the weight-gradient kinds launch with 128-row feature tiles (launch_engine)
    const int out_n = kind == ENG_B5 ? Cfg<B5, 128, 2>::OUT_N : Cfg<B7, 128, 2>::OUT_N;
    const int wgpc = kind == ENG_B5 ? Shape<B5>::WGPC : Shape<B7>::WGPC;
    *tiles_per_expert = ((M + 127) / 128) * ((N + out_n - 1) / out_n);
    *wg_per_xcd = (num_cus + 7) / 8 * wgpc;
}

int engine_dgp_width(int I) { return ((I + 255) / 256) * eng::Cfg<eng::B2, 128, 2>::WAVES_N; }

hipError_t launch_engine(int kind, int BM, const EngineArgs &args, int num_cus, hipStream_t stream)
{
    using namespace eng;
    // multiplier of the slot / topk divisions (div_topk)
    EngineArgs a = args;
    a.topk_l = 0;
    while ((1 << a.topk_l) < a.topk)
        ++a.topk_l;
    a.topk_m = a.topk_l == 0 ? 0u : (uint32_t)((1ull << (31 + a.topk_l)) / (uint64_t)a.topk + 1);
    switch (kind) {
    case F1: return BM == 64 ? launch<F1, 64, 1>(a, num_cus, stream) : launch<F1, 128, 1>(a, num_cus, stream);
    case F2: return BM == 64 ? launch<F2, 64, 1>(a, num_cus, stream) : launch<F2, 128, 1>(a, num_cus, stream);
    case B2: return launch<B2, 128, 2>(a, num_cus, stream);
    case B4: return launch<B4, 128, 2>(a, num_cus, stream);
    case B5: return launch<B5, 128, 2>(a, num_cus, stream);
    case B7: return launch<B7, 128, 2>(a, num_cus, stream);
    default: return hipErrorInvalidValue;
    }
}

} // namespace moe
