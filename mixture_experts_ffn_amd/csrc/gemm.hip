// gemm.hip — grouped GEMMs of the MoE expert FFN on gfx950 matrix cores.
//
// GEMM1 (up_proj, HyperMegaMoE issue page section 2.1 "GMM1") computes, for
// every expert e and every permuted row p of its segment,
//     h[p, :] = x[token(p), :] · W1[e]          W1 = up_proj_weight [E, H, 2I]
// and its epilogue applies SwiGLU (section 2.1 "SwiGLU"; section 4.2 fixes
// the activation) so that h never reaches memory:
//     act[p, j] = silu(h[p, j]) · h[p, I + j]
// One tile owns act columns [n0, n0 + BN) and therefore loads the gate panel
// W1[e][:, n0 : n0+BN] and the up panel W1[e][:, I+n0 : I+n0+BN] together.
// The dispatch gather x[sorted_slot[p] / K] is fused into the A-tile load.
//
// GEMM2 (down_proj, section 2.1 "GMM2"):
//     o[p, :] = act[p, :] · W2[e]               W2 = down_proj_weight [E, I, H]
//
// Tiles and layout:
//  * A tile [BM x BK] and B tile [NPANEL*BN x BK] are staged through LDS,
//    both K-contiguous, double-buffered with one barrier per K step; the next
//    K step's global loads are in flight while the matrix cores run.
//  * The weights are N-contiguous in memory ([k][n]); the B loader reads
//    16-byte row pieces of 4 consecutive k rows and transposes them in
//    registers so that LDS holds [n][k].
//  * Rows of the tail M-tile beyond the expert's real count and k beyond
//    Kdim are zero-filled; their outputs are not stored.
//  * Tile order: expert-major, then groups of up to 8 M-tiles, N-tiles
//    outer and M-tiles inner inside a group, so the tiles that share a
//    weight panel run back to back.  Workgroups are handed out round-robin
//    over the 8 XCDs, so block b takes logical tile (b % 8) * G/8 + b / 8:
//    each XCD walks one contiguous range of the order and its L2 sees the
//    reuse.
#include "common.h"
#include "kernels.h"

namespace moe {

template <typename T, int BM_, int BN_, int BK_, int WM_, int WN_, bool SWIGLU>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = kWave * WM * WN;
    static constexpr int NPANEL = SWIGLU ? 2 : 1;
    static constexpr int VEC = 16 / (int)sizeof(T);
    static constexpr int LDK = BK + VEC; // 16 bytes of padding per LDS row
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int KR = 4; // k rows per B load unit
    static constexpr int A_CHUNKS = BM * BK / VEC;
    static constexpr int A_CPT = A_CHUNKS / NT;
    static constexpr int NCH = NPANEL * BN / VEC; // 16-byte column pieces per k row of B
    static constexpr int B_UNITS = NCH * (BK / KR);
    static constexpr int B_UPT = B_UNITS / NT;
    static constexpr int A_ELEMS = BM * LDK;
    static constexpr int B_ELEMS = NPANEL * BN * LDK;
    static constexpr size_t LDS_BYTES = 2 * (size_t)(A_ELEMS + B_ELEMS) * sizeof(T);
    static_assert(A_CHUNKS % NT == 0 && A_CPT >= 1, "A tile must split evenly over threads");
    static_assert(B_UNITS % NT == 0 && B_UPT >= 1, "B tile must split evenly over threads");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole 16x16 blocks");
    static_assert(BK % Mfma<T>::KSTEP == 0 && BK % KR == 0, "BK must fit the MFMA step");
    static_assert(BN % VEC == 0, "BN must be whole 16-byte pieces");
};

// Transpose KR=4 loaded k-rows of VEC n-values into VEC LDS rows of 4 k-values.
__device__ inline void transpose_store(const u32x4 (&in)[4], bf16 *dst, int ldk)
{
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int w = n >> 1, sh = (n & 1) * 16;
        u32x2 v;
        v.x = ((in[0][w] >> sh) & 0xffffu) | (((in[1][w] >> sh) & 0xffffu) << 16);
        v.y = ((in[2][w] >> sh) & 0xffffu) | (((in[3][w] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2 *>(dst + n * ldk) = v;
    }
}

__device__ inline void transpose_store(const u32x4 (&in)[4], float *dst, int ldk)
{
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        u32x4 v;
        v.x = in[0][n];
        v.y = in[1][n];
        v.z = in[2][n];
        v.w = in[3][n];
        *reinterpret_cast<u32x4 *>(dst + n * ldk) = v;
    }
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool SWIGLU, bool GATHER>
__global__ __launch_bounds__(kWave *WM *WN, 2) void grouped_gemm_kernel(GroupedGemmArgs args)
{
    using Cfg = GemmCfg<T, BM, BN, BK, WM, WN, SWIGLU>;
    using MF = Mfma<T>;
    using Frag = typename MF::Frag;
    constexpr int LDK = Cfg::LDK, VEC = Cfg::VEC, KR = Cfg::KR;
    constexpr int NT = Cfg::NT;

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    T *As = reinterpret_cast<T *>(smem);
    T *Bs = As + 2 * Cfg::A_ELEMS;

    // ---- which tile: XCD-aware logical index, then (expert, m-tile, n-tile)
    const int ntn = (args.Nout + BN - 1) / BN;
    const int g8 = gridDim.x >> 3;
    const int L = (blockIdx.x & 7) * g8 + (blockIdx.x >> 3);
    const int total_mt = args.mtile_off[args.E];
    if (L >= total_mt * ntn)
        return;
    const int e = args.mtile_expert[L / ntn];
    const int mt0 = args.mtile_off[e];
    const int mt_e = args.mtile_off[e + 1] - mt0;
    const int local = L - mt0 * ntn;
    constexpr int GM = 8;
    const int grp = local / (GM * ntn);
    const int first_m = grp * GM;
    const int gm = min(mt_e - first_m, GM);
    const int rr = local - grp * GM * ntn;
    const int n_t = rr / gm;
    const int m_t = first_m + rr % gm;
    const int seg1 = args.offsets[e + 1];
    const int row0 = args.offsets[e] + m_t * BM;
    const int rows = min(BM, seg1 - row0);
    const int n0 = n_t * BN;
    // a shared-expert chunk (e >= Er) reads its chunk of the shared weights
    const bool shd = args.Bs && e >= args.Er;
    const int Kdim = args.Kdim, Nout = args.Nout, ldb = shd ? args.bs_ldb : args.ldb;
    const int upanel = shd ? args.bs_panel : Nout; // GEMM1: column offset of the up panel

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    const T *__restrict__ A = static_cast<const T *>(args.A);
    const T *__restrict__ Bw = shd ? static_cast<const T *>(args.Bs) + (int64_t)(e - args.Er) * args.bs_cstride
                                   : static_cast<const T *>(args.B) + (int64_t)e * Kdim * ldb;

    // ---- per-thread load assignments (fixed for the whole K loop)
    const T *a_src[Cfg::A_CPT];
    int a_k[Cfg::A_CPT], a_lds[Cfg::A_CPT];
    bool a_ok[Cfg::A_CPT];
#pragma unroll
    for (int i = 0; i < Cfg::A_CPT; ++i) {
        const int u = tid + i * NT;
        const int ar = u / (BK / VEC);
        const int ak = (u % (BK / VEC)) * VEC;
        a_ok[i] = ar < rows;
        int64_t grow = 0;
        if (a_ok[i])
            grow = GATHER ? (int64_t)(args.sorted_slot[row0 + ar] / args.topk) : (int64_t)(row0 + ar);
        a_src[i] = A + grow * Kdim + ak;
        a_k[i] = ak;
        a_lds[i] = ar * LDK + ak;
    }
    const T *b_src[Cfg::B_UPT];
    int b_k[Cfg::B_UPT], b_lds[Cfg::B_UPT];
    bool b_ok[Cfg::B_UPT];
#pragma unroll
    for (int i = 0; i < Cfg::B_UPT; ++i) {
        const int u = tid + i * NT;
        const int kg = u / Cfg::NCH;
        const int nc = u % Cfg::NCH;
        const int panel = nc / (BN / VEC);
        const int nn = (nc % (BN / VEC)) * VEC;
        const int col = n0 + nn;
        b_ok[i] = col < Nout;
        b_src[i] = Bw + (int64_t)(kg * KR) * ldb + panel * upanel + (b_ok[i] ? col : 0);
        b_k[i] = kg * KR;
        b_lds[i] = (panel * BN + nn) * LDK + kg * KR;
    }

    u32x4 ra[Cfg::A_CPT];
    u32x4 rb[Cfg::B_UPT][KR];
    const u32x4 zero = {0u, 0u, 0u, 0u};

    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < Cfg::A_CPT; ++i)
            ra[i] = (a_ok[i] && k0 + a_k[i] < Kdim)
                        ? *reinterpret_cast<const u32x4 *>(a_src[i] + k0)
                        : zero;
#pragma unroll
        for (int i = 0; i < Cfg::B_UPT; ++i)
#pragma unroll
            for (int kr = 0; kr < KR; ++kr)
                rb[i][kr] = (b_ok[i] && k0 + b_k[i] + kr < Kdim)
                                ? *reinterpret_cast<const u32x4 *>(b_src[i] + (int64_t)(k0 + kr) * ldb)
                                : zero;
    };
    auto lstore = [&](int buf) {
        T *as = As + buf * Cfg::A_ELEMS;
        T *bs = Bs + buf * Cfg::B_ELEMS;
#pragma unroll
        for (int i = 0; i < Cfg::A_CPT; ++i)
            *reinterpret_cast<u32x4 *>(as + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < Cfg::B_UPT; ++i)
            transpose_store(rb[i], bs + b_lds[i], LDK);
    };

    f32x4 acc[Cfg::NPANEL][Cfg::FM][Cfg::FN];
#pragma unroll
    for (int p = 0; p < Cfg::NPANEL; ++p)
#pragma unroll
        for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Cfg::FN; ++fn)
                acc[p][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (Kdim + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    const int frag_row = lane & 15, frag_k = (lane >> 4) * MF::KPL;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk)
            gload((kt + 1) * BK);
        const T *as = As + buf * Cfg::A_ELEMS + (wm * Cfg::WTM + frag_row) * LDK + frag_k;
        const T *bs = Bs + buf * Cfg::B_ELEMS + (wn * Cfg::WTN + frag_row) * LDK + frag_k;
#pragma unroll
        for (int kk = 0; kk < BK; kk += MF::KSTEP) {
            Frag a[Cfg::FM], b[Cfg::NPANEL][Cfg::FN];
#pragma unroll
            for (int fm = 0; fm < Cfg::FM; ++fm)
                a[fm] = *reinterpret_cast<const Frag *>(as + fm * 16 * LDK + kk);
#pragma unroll
            for (int p = 0; p < Cfg::NPANEL; ++p)
#pragma unroll
                for (int fn = 0; fn < Cfg::FN; ++fn)
                    b[p][fn] = *reinterpret_cast<const Frag *>(bs + (p * BN + fn * 16) * LDK + kk);
#pragma unroll
            for (int p = 0; p < Cfg::NPANEL; ++p)
#pragma unroll
                for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < Cfg::FN; ++fn)
                        acc[p][fm][fn] = MF::mma(a[fm], b[p][fn], acc[p][fm][fn]);
        }
        if (kt + 1 < nk)
            lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue
    T *__restrict__ Cout = static_cast<T *>(args.C);
    T *__restrict__ Hs = static_cast<T *>(args.Hsave);
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn) {
            const int c = n0 + wn * Cfg::WTN + fn * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * Cfg::WTM + fm * 16 + (lane >> 4) * 4 + i;
                if (r < rows && c < Nout) {
                    const int64_t p = row0 + r;
                    if constexpr (SWIGLU) {
                        const float gv = acc[0][fm][fn][i], uv = acc[1][fm][fn][i];
                        Cout[p * Nout + c] = from_f32<T>(silu_f(gv) * uv);
                        if (Hs) {
                            Hs[p * 2 * Nout + c] = from_f32<T>(gv);
                            Hs[p * 2 * Nout + Nout + c] = from_f32<T>(uv);
                        }
                    } else {
                        Cout[p * Nout + c] = from_f32<T>(acc[0][fm][fn][i]);
                    }
                }
            }
        }
    }
}

template <typename T, int BM, int BN, int BK, int WM, int WN, bool SWIGLU, bool GATHER>
static hipError_t launch_grouped(const GroupedGemmArgs &a, hipStream_t stream)
{
    using Cfg = GemmCfg<T, BM, BN, BK, WM, WN, SWIGLU>;
    auto kern = grouped_gemm_kernel<T, BM, BN, BK, WM, WN, SWIGLU, GATHER>;
    static bool attr_done = false; // benign race: the attribute is idempotent
    if (!attr_done) {
        hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)Cfg::LDS_BYTES);
        if (err != hipSuccess)
            return err;
        attr_done = true;
    }
    const int64_t ntn = (a.Nout + BN - 1) / BN;
    const int64_t tiles = (int64_t)a.max_mtiles * ntn;
    if (tiles <= 0)
        return hipSuccess;
    const int64_t grid = (tiles + 7) / 8 * 8;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::LDS_BYTES, stream, a);
    return hipGetLastError();
}

hipError_t launch_gemm1_swiglu(int dtype, const FwdTiles &t, const GroupedGemmArgs &a,
                               hipStream_t stream)
{
    if (dtype == 1) { // bf16
        if (t.BM == 64)
            return launch_grouped<bf16, 64, 64, 64, 2, 2, true, true>(a, stream);
        return launch_grouped<bf16, 128, 64, 64, 2, 2, true, true>(a, stream);
    }
    return launch_grouped<float, 64, 64, 32, 2, 2, true, true>(a, stream);
}

hipError_t launch_gemm2(int dtype, const FwdTiles &t, const GroupedGemmArgs &a,
                        hipStream_t stream)
{
    if (dtype == 1) {
        if (t.BM == 64)
            return launch_grouped<bf16, 64, 128, 64, 2, 2, false, false>(a, stream);
        return launch_grouped<bf16, 128, 128, 64, 2, 2, false, false>(a, stream);
    }
    // fp32: 64-column tiles (BK = 64 so the B tile still splits evenly over the
    // threads): twice the workgroups of 128-column tiles, which the small fp32
    // shapes need to fill the device
    return launch_grouped<float, 64, 64, 64, 2, 2, false, false>(a, stream);
}

} // namespace moe
