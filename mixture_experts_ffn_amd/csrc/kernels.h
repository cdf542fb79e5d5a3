// kernels.h — host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16_t;

// ---- routing -----------------------------------------------------------------
// Header at the front of the saved context: the forward's routing step writes
// it, the backward checks it before it trusts any of the saved arrays.
// The backward's data-gradient stage copies it into its workspace, and the
// weight-gradient stage, which reads that workspace, checks the copy against
// the saved context it is given.
struct SavedHeader {
    uint32_t magic;
    uint32_t version;
    uint64_t problem; // hash of (T, H, I, E, K, dtype, ids_dtype, Is)
    uint64_t epoch;   // distinct for every forward that saves a context
};
constexpr uint32_t kSavedMagic = 0x46454f4du; // "MOEF"
constexpr uint32_t kSavedVersion = 2u;

// The optional shared expert (issue page, section 6.1) of intermediate width
// Is = S * I, run as S extra experts Er .. Er + S - 1 that every token reaches
// with gate 1: expert Er + c uses gate columns [cI, cI + I) and up columns
// [Is + cI, Is + cI + I) of w1 [H, 2Is] and rows [cI, cI + I) of w2 [Is, H].
// Its rows follow the routed ones in permuted order: row offsets[Er] + cT + t
// is token t of chunk c.
struct SharedExperts {
    int Er = 0;              // routed experts; expert e >= Er is shared chunk e - Er
    int S = 0;               // chunks (0: no shared expert)
    int Is = 0;              // S * I
    const void *w1 = nullptr; // [H, 2Is]
    const void *w2 = nullptr; // [Is, H]
    void *dw1 = nullptr;      // backward: [H, 2Is]
    void *dw2 = nullptr;      // backward: [Is, H]
};

struct RoutePlan {
    int RC;    // slots per chunk (one wave per chunk)
    int NB;    // number of chunks
    int nbits; // bits needed for an expert id
};

struct RouteBufs {
    int32_t *hist;        // [E * NB]
    int32_t *bad;         // [NB]
    int32_t *counts;      // [E]
    int32_t *offsets;     // [E + 1]
    int32_t *mtile_off;   // [E + 1]
    int32_t *mtile_expert; // [max_mtiles]: expert owning each M-tile
    // optional second pair of M-tile tables for tiles of BM2 rows (a GEMM2 on
    // another tile height than GEMM1); BM2 = 0: none
    int32_t *mtile2_off = nullptr;    // [E + 1]
    int32_t *mtile2_expert = nullptr; // [max M-tiles of BM2 rows]
    int BM2 = 0;
    int32_t *status;      // [1]
    int32_t *sorted_slot; // [TK]
    int32_t *slot_pos;    // [TK]
    int32_t *ctr;         // optional: release counters of the pipelined forward, zeroed here
    int nctr;             // their number
    SavedHeader *saved_hdr; // optional: header of the saved context, written here
    uint64_t problem_hash;
    uint64_t epoch;
    int nshared = 0;        // shared-expert chunks S: experts E .. E+S-1 of T rows each
    int64_t T = 0;          // tokens (rows of every shared chunk)
};

// bits of the device status word
enum { MOE_DEV_BAD_ID = 1, MOE_DEV_TIMEOUT = 2, MOE_DEV_BAD_SAVED = 4, MOE_DEV_BAD_WS = 8 };


RoutePlan make_route_plan(int64_t TK, int E);
hipError_t launch_route(const void *ids, bool ids64, int64_t TK, int E, int BM,
                        const RoutePlan &rp, const RouteBufs &rb, hipStream_t stream);

// upper bound of sum_e ceil(counts[e] / BM) over any routing of TK slots
inline int64_t max_mtiles_bound(int64_t TK, int E, int BM)
{
    const int64_t ne = TK < E ? TK : E;
    return (TK + BM - 1) / BM + ne;
}

// ---- grouped GEMMs ---------------------------------------------------------------
// One launch covers every expert: M-tiles of BM rows walk each expert's
// segment [offsets[e], offsets[e+1]) of the permuted rows.
struct GroupedGemmArgs {
    const void *A;               // GEMM1: x [T, Kdim] (rows gathered); GEMM2: act [TK, Kdim]
    const void *B;               // weights [E, Kdim, ldb], N-contiguous
    void *C;                     // GEMM1: act [TK, Nout]; GEMM2: o [TK, Nout]
    void *Hsave;                 // GEMM1 only, optional: pre-activation h [TK, 2*Nout]
    const int32_t *sorted_slot;  // GEMM1: permuted row p -> slot s (token s / topk)
    const int32_t *offsets;      // [E + 1]
    const int32_t *mtile_off;    // [E + 1]
    const int32_t *mtile_expert; // [max_mtiles]
    int Kdim;                    // contraction length
    int Nout;                    // output columns
    int ldb;                     // row stride of B (2I for GEMM1, H for GEMM2)
    int topk;                    // K
    int E;
    int max_mtiles;              // upper bound of sum_e ceil(counts[e] / BM)
    // shared-expert chunks (experts e >= Er; E counts them too): weights
    // Bs + (e - Er) * bs_cstride, row stride bs_ldb, GEMM1's up panel bs_panel
    // columns in
    int Er;
    const void *Bs;
    int64_t bs_cstride;
    int bs_ldb, bs_panel;
};

// plan-level tile choice for the forward
struct FwdTiles {
    int BM;       // 64, 128 or 256
    bool big;     // bf16 fast path: the 256 x 256 tile kernel (BM = 256)
    bool big2;    // bf16 fast path, BM = 128: GEMM2 alone on the 256 x 256 kernel
    int num_cus;  // compute units of the device (persistent grids)
};

hipError_t launch_gemm1_swiglu(int dtype, const FwdTiles &t, const GroupedGemmArgs &a,
                               hipStream_t stream);
hipError_t launch_gemm2(int dtype, const FwdTiles &t, const GroupedGemmArgs &a,
                        hipStream_t stream);

// bf16 forward fast path (gemm_mfma.hip): H % 256 == 0, I % 128 == 0
bool fast_gemm_supported(int dtype, int64_t H, int64_t I);
struct FastFwdArgs {
    const void *x;               // [T, H]
    const void *w1;              // [E, H, 2I]
    const void *w2;              // [E, I, H]
    void *act;                   // [TK, I]
    void *hsave;                 // optional [TK, 2I]
    void *o;                     // [TK, H]
    const int32_t *sorted_slot;  // [TK]
    const int32_t *offsets;      // [E + 1]
    const int32_t *mtile_off;    // [E + 1]
    const int32_t *mtile_expert; // [max_mtiles]
    int32_t *ctr;                // pipelined: [max_mtiles] zeroed GEMM1 release counters
    int32_t *tickets;            // pipelined: [16] zeroed ticket counters (8 per GEMM, one per XCD)
    int grid;                    // workgroups of the launch (0: the persistent default)
    int32_t *status;             // device status word (MOE_DEV_* bits)
    int64_t timeout_ticks;       // watchdog of every wait, in s_memrealtime ticks
    int T, H, I, E, K;
    int max_mtiles;
    int drop_mt;                 // test hook: M-tile whose first GEMM1 release is dropped (-1)
    SharedExperts sh;            // E counts the shared chunks too (sh.Er routed)
};
enum { FAST_G1 = 0, FAST_G2 = 1, FAST_PIPE = 2, FAST_G1H = 3 }; // FAST_G1H: FAST_G1 saving h
hipError_t launch_fast_fwd(int mode, int BM, const FastFwdArgs &a, int num_cus,
                           hipStream_t stream);
// the same grouped GEMMs (FAST_G1, FAST_G1H, FAST_G2) on 256 x 256 tiles, one
// 4-wave workgroup per CU (gemm_big.hip); the M-tile tables must be built for
// 256-row tiles
// skip_padding (GEMM2 only): leave out the copies of token rows past a tile's
// rows, for launches where many tiles are short
hipError_t launch_fast_fwd_big(int mode, const FastFwdArgs &a, int num_cus, hipStream_t stream,
                               bool skip_padding = false);

// bf16 engine (gemm_engine.hip): forward F1/F2 and backward B2/B4/B5/B7
struct EngineArgs {
    const bf16_t *A;             // first operand (see the kind table in gemm_engine.hip)
    const bf16_t *B;             // second operand
    bf16_t *C;                   // main output
    bf16_t *C2;                  // F1: optional saved h [TK, 2I]; B2: act_g [TK, I]
    const bf16_t *Hs;            // B2: saved h [TK, 2I]
    const float *gates;          // B2: topk_weights by slot
    float *dgp;                  // B2: per-row partial dots [TK, dgp_stride]
    const int32_t *sorted_slot;  // permuted row -> slot
    const int32_t *offsets;      // [E + 1]
    const int32_t *mtile_off;    // [E + 1] (token-tiled kinds)
    const int32_t *mtile_expert; // [max M-tiles]
    int topk, E;
    uint32_t topk_m;             // set by launch_engine: slot / topk by multiply and shift
    int topk_l;
    int M, N, Kd;                // feature-tiled: M, N; token-tiled: N and Kd
    int lda, ldb, ldc;
    int64_t b_estride;           // expert stride of a weight operand (elements)
    int dgp_stride;
    // shared-expert chunks (experts e >= Er; E counts them too): their weight
    // operand is Bs + (e - Er) * bs_cstride with row stride bs_ldb; F1: its up
    // panel starts bs_panel columns in; B4: k >= Kd / 2 reads bs_kjump further
    // on; B5/B7: the gradient goes to Cs + (e - Er) * cs_cstride with row
    // stride cs_ldc, B7 columns >= N / 2 cs_cjump further on
    int Er;
    const bf16_t *Bs;
    int64_t bs_cstride;
    int bs_ldb, bs_panel, bs_kjump;
    bf16_t *Cs;
    int64_t cs_cstride;
    int cs_ldc, cs_cjump;
    // feature-tiled kinds, optional: [9] tile bounds of the eight XCDs (from
    // the backward set-up); null: an eighth of the tiles each
    const int32_t *xcd_bounds;
};
enum { ENG_F1 = 0, ENG_F2 = 1, ENG_B2 = 2, ENG_B4 = 3, ENG_B5 = 4, ENG_B7 = 5 };
hipError_t launch_engine(int kind, int BM, const EngineArgs &a, int num_cus, hipStream_t stream);
int engine_dgp_width(int I); // columns of the B2 partial-dot buffer
// a weight-gradient kind's (ENG_B5 / ENG_B7) feature tiles per expert for an
// M x N gradient, and its workgroups per XCD
void engine_feature_tiling(int kind, int M, int N, int num_cus, int *tiles_per_expert,
                           int *wg_per_xcd);

// ---- combine ---------------------------------------------------------------------
// y[t] = Σ_k g[t, k] o[slot_pos[tK+k]] + Σ_c o[offsets[Er] + cT + t] (the S
// shared-expert chunks, gate 1, after the routed terms; S = 0: none)
hipError_t launch_combine(int dtype, const void *o, const int32_t *slot_pos, const float *gates,
                          void *y, int64_t T, int H, int K, const int32_t *offsets, int Er, int S,
                          hipStream_t stream);
// backward combine: dx[t] = Σ_k dxp[slot_pos[tK+k]] + Σ_c dxp[offsets[Er] + cT + t] and
// d_topk[t, k] = Σ_j dgp[slot_pos[tK+k], j] (0 for a dropped slot)
// (all zeros when *status has MOE_DEV_BAD_SAVED or MOE_DEV_BAD_WS)
hipError_t launch_combine_bwd(const void *dxp, const float *dgp, int dgp_stride,
                              const int32_t *slot_pos, const int32_t *status, void *dx,
                              float *d_topk, int64_t T, int H, int K, const int32_t *offsets,
                              int Er, int S, hipStream_t stream);
// zero `bytes` (a multiple of 16) at a 16-byte aligned pointer
hipError_t launch_zero_fill(void *p, size_t bytes, hipStream_t stream);
// Backward set-up (one block): checks the saved context's header and the
// consistency of its counts/offsets; copies them into the workspace (all zero,
// and MOE_DEV_BAD_SAVED in *status, if the check fails) and builds the M-tile
// tables from the copies.  The stages of a split backward also pass the
// workspace's copy of the header, ws_hdr: the data-gradient stage
// (BWD_STAGE_D) writes it (zeros if the saved context failed its check); the
// weight-gradient stage (BWD_STAGE_W) requires it to equal the saved header,
// else the copies are zero and *status gets MOE_DEV_BAD_WS.
// It also writes, for each of `nsplit` (<= 2) weight-gradient launches with
// split_F[i] feature tiles per expert and split_wgx[i] workgroups per XCD, the
// nine tile bounds of a cost-balanced split over the eight XCDs into
// xcd_bounds[9 i .. 9 i + 8].
enum { BWD_STAGE_ALL = 0, BWD_STAGE_D = 1, BWD_STAGE_W = 2 };
struct XcdSplits {
    int n;          // launches (0..2)
    int F[2];       // feature tiles per expert
    int wgx[2];     // workgroups per XCD
    int32_t *bounds; // [n][9]
};
hipError_t launch_bwd_setup(const SavedHeader *hdr, uint64_t problem_hash, const int32_t *counts,
                            const int32_t *offsets, int E, int64_t TK, int BM, int32_t *counts_out,
                            int32_t *offsets_out, int32_t *mtile_off, int32_t *mtile_expert,
                            int32_t *status, SavedHeader *ws_hdr, int stage,
                            const XcdSplits &splits, hipStream_t stream);

} // namespace moe
