// gemm_mfma.hip — the forward bf16 grouped GEMMs of the MoE expert FFN,
// pipelined for gfx950: the fast path for shapes whose H is a multiple of 256
// and I of 128 (whole K steps and whole output tiles, so no edge handling).
// Other bf16 shapes and the backward use the engine of gemm_engine.hip,
// which adds zero-page edges and variable-K tiles; fp32 uses gemm.hip.
//
// Same two operations as gemm.hip (HyperMegaMoE issue page, section 2.1:
// GMM1/up_proj with the SwiGLU epilogue, GMM2/down_proj), organised for the
// CDNA4 memory pipeline:
//
//  * Global -> LDS copies go straight into LDS (16 bytes per lane, no
//    register staging), three stages deep, two K steps ahead of the matrix
//    cores; each wave waits only for its own copies of the stage it is about
//    to use, then one barrier per K step publishes the stage.
//  * A (token rows, K-contiguous) lands as [BM][64] with the 16-byte piece
//    index XOR-ed by (row / 2) % 8, so the 16 lanes of one 128-bit LDS read
//    hit 16 different bank groups.  The dispatch gather x[sorted_slot / K] is
//    just the per-lane source address of those copies.
//  * B (weights, N-contiguous [k][n]) lands untransposed as [64][PW] with the
//    32-byte unit index XOR-ed by a 3-bit hash of k; the MFMA fragments are
//    read with the transposing 64-bit LDS read, two per fragment.
//  * The matrix-core step computes C^T = W^T · X^T (weights as the first
//    operand), so each lane ends up owning 4 consecutive output columns of
//    one row and the epilogue writes 8 bytes per lane.
//  * Block tile 128 (or 64) rows x 256 weight columns, 4 waves; GEMM1's 256
//    columns are 128 gate + 128 up columns, so SwiGLU is elementwise in
//    registers.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace fast {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int BK = 64;
constexpr int NSTAGE = 3;
constexpr int kFastWaves = 8; // two waves per SIMD: one's MFMAs cover the other's LDS waits
constexpr int kWavesM128 = 1; // waves along M for 128-row tiles (each wave owns all rows)

template <int BM_, bool SWIGLU, int NW_, int WM_> struct Cfg {
    static constexpr int BM = BM_;
    static constexpr int NW = NW_; // waves per workgroup (4 or 8)
    static constexpr int NPANEL = SWIGLU ? 2 : 1;
    static constexpr int PW = SWIGLU ? 128 : 256; // weight columns per panel
    static constexpr int WAVES_M = WM_;           // waves along M
    static constexpr int WAVES_N = NW / WAVES_M;
    static constexpr int WTM = BM / WAVES_M;        // rows per wave
    static constexpr int WTN = PW / WAVES_N;        // columns per wave per panel
    static constexpr int FM = WTM / 16, FN = WTN / 16;
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BK * NPANEL * PW * 2; // 32 KB
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;
    static constexpr int A_LOADS = A_BYTES / 1024 / NW; // per wave per stage
    static constexpr int B_LOADS = B_BYTES / 1024 / NW;
    static_assert(A_LOADS >= 1 && B_LOADS * NW * 1024 == B_BYTES, "stage split");
    static_assert(A_LOADS * NW * 1024 == A_BYTES, "stage split");
    static_assert(FM >= 1 && FN >= 1, "wave tile");
};

__device__ __forceinline__ int bswz(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

// 16-byte global -> LDS copy per lane into [l, l + 1024) (lane i at l + 16 i).
// Issued as inline assembly so that the compiler does not track these LDS
// writes: their completion is established explicitly (wait_vm) per stage,
// instead of the compiler waiting for every copy in flight before each LDS
// read.  `l` must be wave-uniform.
__device__ __forceinline__ void g2l16(const void *g, lds_void *l)
{
    const uint32_t lds_addr = (uint32_t)(uintptr_t)l;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_addr), "v"(g)
                 : "memory", "m0");
}

// wait until at most n vector-memory operations of this wave are in flight
template <int N> __device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier for the K loop.  The main loop writes LDS only through
// global->LDS copies, whose completion each wave establishes itself (vmcnt)
// before arriving, and reads LDS only into registers that the matrix cores
// consume before the wave can arrive again; so the barrier needs no memory
// fence, only a compiler-level ordering of LDS accesses around it.  (A fence
// would also wait for the copies of later stages that are still in flight.)
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct TileInfo {
    int e, row0, rows, n0;
};

// Logical tile L -> (expert, first permuted row, real rows, first output
// column).  Order: expert-major; inside an expert, groups of up to 8 M-tiles
// with N-tiles outer and M-tiles inner, so consecutive tiles share a weight
// panel.  All operands are wave-uniform (scalar loads).
__device__ __forceinline__ TileInfo decode_tile(const GroupedGemmArgs &args, int L, int ntn,
                                                int BM, int out_tile)
{
    TileInfo t;
    t.e = args.mtile_expert[L / ntn];
    const int mt0 = args.mtile_off[t.e];
    const int mt_e = args.mtile_off[t.e + 1] - mt0;
    const int local = L - mt0 * ntn;
    constexpr int GM = 8;
    const int grp = local / (GM * ntn);
    const int first_m = grp * GM;
    const int gm = min(mt_e - first_m, GM);
    const int rr = local - grp * GM * ntn;
    const int n_t = rr / gm;
    const int m_t = first_m + rr % gm;
    t.row0 = args.offsets[t.e] + m_t * BM;
    t.rows = min(BM, args.offsets[t.e + 1] - t.row0);
    t.n0 = n_t * out_tile;
    return t;
}

// Persistent grouped GEMM: gridDim.x workgroups (a multiple of 8, one per CU)
// walk the logical tiles.  The hardware hands workgroups to the 8 XCDs round
// robin, so workgroup b sits on XCD b % 8; each XCD owns one contiguous eighth
// of the tile order and its workgroups take consecutive tiles of it, so the
// tiles in flight on one XCD share weight panels and token rows in its L2.
// The K loop runs continuously across a workgroup's tiles: the copies of the
// next tile's first two K steps are in flight while the current tile's last
// steps and its epilogue run.
template <int BM, bool SWIGLU, bool GATHER, int NW, int WM>
__global__ __launch_bounds__(64 * NW, 1) void moe_gemm_bf16(GroupedGemmArgs args)
{
    using C = Cfg<BM, SWIGLU, NW, WM>;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * C::STAGE_BYTES];

    const int out_tile = SWIGLU ? C::PW : C::NPANEL * C::PW; // output columns per tile
    const int ntn = args.Nout / out_tile;
    const int total = args.mtile_off[args.E] * ntn;
    const int per_xcd_wg = gridDim.x >> 3;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int range = (total + 7) >> 3;
    const int hi = min((xcd + 1) * range, total);
    int L = xcd * range + slot;
    if (L >= hi)
        return;

    const int Kdim = args.Kdim, Nout = args.Nout, ldb = args.ldb;
    const int nk = Kdim / BK;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
    const bf16 *__restrict__ A = static_cast<const bf16 *>(args.A);

    // per-lane copy sources of one tile
    struct Src {
        const bf16 *a[C::A_LOADS];
        const bf16 *b[C::B_LOADS];
    };
    auto make_src = [&](const TileInfo &t, Src &sr) {
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i) {
            // chunk c covers rows 8c .. 8c+7; this lane fills 16-byte unit `lane`
            const int c = wave * C::A_LOADS + i;
            const int r = c * 8 + (lane >> 3);
            const int piece = (lane & 7) ^ ((r >> 1) & 7);
            int64_t grow;
            if constexpr (GATHER) {
                // the 8 row indices of the chunk are wave-uniform: scalar loads
                int idx[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int rj = c * 8 + j < t.rows ? c * 8 + j : 0; // tail rows copy row 0
                    idx[j] = args.sorted_slot[t.row0 + rj];
                }
                int v = idx[0];
#pragma unroll
                for (int j = 1; j < 8; ++j)
                    v = (lane >> 3) == j ? idx[j] : v;
                grow = v / args.topk;
            } else {
                grow = t.row0 + (r < t.rows ? r : 0);
            }
            sr.a[i] = A + grow * Kdim + piece * 8;
        }
        const bf16 *W = static_cast<const bf16 *>(args.B) + (int64_t)t.e * Kdim * ldb;
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
            // chunk c covers 1024 bytes = 4 (SwiGLU panels) or 2 k-rows of one panel
            const int c = wave * C::B_LOADS + i;
            int panel, kr, pp;
            if constexpr (SWIGLU) {
                panel = c >> 4;
                kr = (c & 15) * 4 + (lane >> 4);
                pp = lane & 15;
            } else {
                panel = 0;
                kr = c * 2 + (lane >> 5);
                pp = lane & 31;
            }
            const int u = (pp >> 1) ^ bswz(kr);
            const int col = t.n0 + panel * Nout + (2 * u + (pp & 1)) * 8;
            sr.b[i] = W + (int64_t)kr * ldb + col;
        }
    };
    auto issue = [&](const Src &sr, int kb, unsigned char *sbase) {
        const int k0 = kb * BK;
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i)
            g2l16(sr.a[i] + k0, (lds_void *)(sbase + (wave * C::A_LOADS + i) * 1024));
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i)
            g2l16(sr.b[i] + (int64_t)k0 * ldb,
                  (lds_void *)(sbase + C::A_BYTES + (wave * C::B_LOADS + i) * 1024));
    };

    f32x4 acc[C::NPANEL][C::FM][C::FN];
    const int fr = lane & 15;                      // A: row within a 16-row block
    const int fk = lane >> 4;                      // A: piece in a 32-k step; B: 8-k group
    const int tq = lane & 3, tr = (lane >> 2) & 3; // B transposing read: column part / row

    auto compute = [&](const unsigned char *sA) {
        const unsigned char *sB = sA + C::A_BYTES;
#pragma unroll
        for (int kk = 0; kk < BK; kk += 32) {
            bf16x8 af[C::FM];
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm) {
                const int r = wm * C::WTM + fm * 16 + fr;
                const int piece = ((kk >> 3) + fk) ^ ((r >> 1) & 7);
                af[fm] = *reinterpret_cast<const bf16x8 *>(sA + r * 128 + piece * 16);
            }
#pragma unroll
            for (int p = 0; p < C::NPANEL; ++p) {
                const unsigned char *sP = sB + p * (BK * C::PW * 2);
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn) {
                    const int nb = wn * C::WTN + fn * 16 + 4 * tq; // column this lane reads
                    v4i16 half[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int kr = kk + 8 * fk + 4 * h + tr;
                        const int u = (nb >> 4) ^ bswz(kr);
                        const unsigned char *addr = sP + kr * (C::PW * 2) + u * 32 + (nb & 15) * 2;
                        half[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(addr));
                    }
                    const v8i16 both = __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5,
                                                               6, 7);
                    const bf16x8 bfrag = __builtin_bit_cast(bf16x8, both);
#pragma unroll
                    for (int fm = 0; fm < C::FM; ++fm)
                        acc[p][fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            bfrag, af[fm], acc[p][fm][fn], 0, 0, 0);
                }
            }
        }
    };

    // epilogue: lane owns row (lane & 15) and columns 4*(lane >> 4) + [0, 4)
    auto epilogue = [&](const TileInfo &t) {
        bf16 *__restrict__ Cout = static_cast<bf16 *>(args.C);
        bf16 *__restrict__ Hs = static_cast<bf16 *>(args.Hsave);
#pragma unroll
        for (int fm = 0; fm < C::FM; ++fm) {
            const int r = wm * C::WTM + fm * 16 + (lane & 15);
            if (r >= t.rows)
                continue;
            const int64_t p = t.row0 + r;
#pragma unroll
            for (int fn = 0; fn < C::FN; ++fn) {
                const int c = t.n0 + wn * C::WTN + fn * 16 + 4 * (lane >> 4);
                if constexpr (SWIGLU) {
                    u32x2 outv, gv, uv;
                    bf16 *o = reinterpret_cast<bf16 *>(&outv);
                    bf16 *go = reinterpret_cast<bf16 *>(&gv);
                    bf16 *uo = reinterpret_cast<bf16 *>(&uv);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float g = acc[0][fm][fn][i], u = acc[1][fm][fn][i];
                        o[i] = static_cast<bf16>(silu_f(g) * u);
                        go[i] = static_cast<bf16>(g);
                        uo[i] = static_cast<bf16>(u);
                    }
                    *reinterpret_cast<u32x2 *>(Cout + p * Nout + c) = outv;
                    if (Hs) {
                        *reinterpret_cast<u32x2 *>(Hs + p * 2 * Nout + c) = gv;
                        *reinterpret_cast<u32x2 *>(Hs + p * 2 * Nout + Nout + c) = uv;
                    }
                } else {
                    u32x2 outv;
                    bf16 *o = reinterpret_cast<bf16 *>(&outv);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        o[i] = static_cast<bf16>(acc[0][fm][fn][i]);
                    *reinterpret_cast<u32x2 *>(Cout + p * Nout + c) = outv;
                }
            }
        }
    };

    constexpr int NL = C::A_LOADS + C::B_LOADS;
    TileInfo cur = decode_tile(args, L, ntn, BM, out_tile);
    Src scur, snext;
    make_src(cur, scur);
    int Lnext = L + per_xcd_wg;
    bool has_next = Lnext < hi;
    TileInfo nxt = cur;
    if (has_next) {
        nxt = decode_tile(args, Lnext, ntn, BM, out_tile);
        make_src(nxt, snext);
    }
    // prologue: the first two K steps (nk >= 2 on this path)
    issue(scur, 0, smem);
    issue(scur, 1, smem + C::STAGE_BYTES);
    int s_cur = 0; // stage of the current step (global step index % 3)
    while (true) {
#pragma unroll
        for (int p = 0; p < C::NPANEL; ++p)
#pragma unroll
            for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < C::FN; ++fn)
                    acc[p][fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int kb = 0; kb < nk; ++kb) {
            // wait for this wave's copies of the current step (the next step's
            // may stay in flight), publish the stage, then start the copies of
            // the step after next into the stage the previous step used
            if (kb + 1 < nk || has_next)
                wait_vm<NL>();
            else
                wait_vm<0>();
            lds_barrier();
            const int s_next = s_cur == 0 ? 2 : s_cur - 1; // (step + 2) % 3
            if (kb + 2 < nk)
                issue(scur, kb + 2, smem + s_next * C::STAGE_BYTES);
            else if (has_next)
                issue(snext, kb + 2 - nk, smem + s_next * C::STAGE_BYTES);
            compute(smem + s_cur * C::STAGE_BYTES);
            s_cur = s_cur == 2 ? 0 : s_cur + 1;
        }
        epilogue(cur);
        if (!has_next)
            break;
        cur = nxt;
        scur = snext;
        Lnext += per_xcd_wg;
        has_next = Lnext < hi;
        if (has_next) {
            nxt = decode_tile(args, Lnext, ntn, BM, out_tile);
            make_src(nxt, snext);
        }
    }
}

template <int BM, bool SWIGLU, bool GATHER, int NW = kFastWaves,
          int WM = (BM == 128 ? kWavesM128 : 1)>
static hipError_t launch(const GroupedGemmArgs &a, int num_cus, hipStream_t stream)
{
    auto kern = moe_gemm_bf16<BM, SWIGLU, GATHER, NW, WM>;
    if (a.max_mtiles <= 0)
        return hipSuccess;
    const int grid = (num_cus + 7) / 8 * 8; // one workgroup per CU, whole XCDs
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NW), 0, stream, a);
    return hipGetLastError();
}

} // namespace fast

bool fast_gemm_supported(int dtype, int64_t H, int64_t I)
{
    return dtype == 1 && H % 256 == 0 && I % 128 == 0 && H % fast::BK == 0 &&
           I % fast::BK == 0;
}

hipError_t launch_fast_gemm1(const FwdTiles &t, const GroupedGemmArgs &a, hipStream_t stream)
{
    if (t.BM == 64)
        return fast::launch<64, true, true>(a, t.num_cus, stream);
    return fast::launch<128, true, true>(a, t.num_cus, stream);
}

hipError_t launch_fast_gemm2(const FwdTiles &t, const GroupedGemmArgs &a, hipStream_t stream)
{
    if (t.BM == 64)
        return fast::launch<64, false, false>(a, t.num_cus, stream);
    return fast::launch<128, false, false>(a, t.num_cus, stream);
}

} // namespace moe
