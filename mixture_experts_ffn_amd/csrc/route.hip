// route.hip — device-side routing of the T·K expert slots.
//
// The routing step of the HyperMegaMoE issue page (section 4.1: each token
// expands into K expert slots that are grouped by expert; section 6.2 lists
// the counts, the sort by expert and the unsort as part of the operator) and
// the device-side metadata of the overlap explainer page (section 5: counts,
// prefix sums, offsets and the token permutation live on the device).
//
// Output: counts[E], offsets[E+1], sorted_slot[p] = s (expert-major, stable in
// slot index s = t·K + k), slot_pos[s] = p (-1 for an out-of-range id) and
// mtile_off[E+1], the prefix sum of ceil(counts[e] / BM) M-tiles that the
// grouped GEMMs walk, with mtile_expert[j], the expert owning M-tile j (and,
// when a GEMM2 runs on taller tiles than GEMM1, the same pair of tables for
// those tiles).
//
// No global atomics and no memset.  The slots are cut into chunks of RC
// (512) and one wave routes one chunk; the work is
//   hist:    count each chunk's ids per expert (hist[E][NB]) and flag bad ids;
//   scan:    exclusive per-(expert, chunk) bases, counts and M-tile counts
//            scanned over experts, the status word, and the zeroed release
//            counters of the pipelined forward that follows;
//   scatter: each wave walks its chunk in order, 64 slots at a time; lanes
//            holding the same expert find each other with ballots over the id
//            bits, so the rank inside the round is a popcount and the order
//            stays stable.
// Launches: one 1024-thread block does all three when the slots fit 16
// chunks (decode-sized batches); up to 32768 slots, 1024-thread blocks of 16
// chunks that each count all the ids themselves, scan and scatter their own
// chunks; beyond that a hist launch first, whose table the blocks read
// instead of counting (also from 863 experts on, where the self-counting
// table of 19 x E words would not fit 64 KB of LDS).  With more than 910
// experts the per-block table would not fit either, and hist, scan and
// scatter run as three launches.
#include "common.h"
#include "kernels.h"

namespace moe {

// the optional second pair of M-tile tables, for tiles of BM rows (BM = 0: none)
struct MTileTable2 {
    int32_t *off;    // [E + 1]
    int32_t *expert; // [sum_e ceil(counts[e] / BM)]
    int BM;
};

// Ids of up to 8 rounds of 64 slots from r0 < s1 on (lane's slots
// r0 + 64 j + lane below s1; -1 past it).  The loads are unconditional (a
// slot past s1 re-reads slot s1 - 1), so all 8 are in flight together and a
// chunk costs one memory round trip per 512 slots instead of one per 64.
template <typename Id>
__device__ inline void load_ids8(const Id *__restrict__ ids, int64_t r0, int64_t s1, int64_t (&v)[8])
{
    const int lane = threadIdx.x & 63;
    Id raw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t s = r0 + 64 * j + lane;
        raw[j] = ids[s < s1 ? s : s1 - 1];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = r0 + 64 * j + lane < s1 ? (int64_t)raw[j] : -1;
}

template <typename Id>
__global__ __launch_bounds__(64) void route_hist_kernel(const Id *__restrict__ ids, int64_t TK,
                                                        int E, int RC, int NB,
                                                        int32_t *__restrict__ hist,
                                                        int32_t *__restrict__ bad)
{
    extern __shared__ int32_t lh[];
    for (int e = threadIdx.x; e < E; e += 64)
        lh[e] = 0;
    __syncthreads();
    const int b = blockIdx.x;
    const int64_t s0 = (int64_t)b * RC;
    const int64_t s1 = s0 + RC < TK ? s0 + RC : TK;
    int anybad = 0;
    for (int64_t r0 = s0; r0 < s1; r0 += 512) {
        int64_t v[8];
        load_ids8(ids, r0, s1, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t e = v[j];
            if (r0 + 64 * j + threadIdx.x >= s1)
                continue;
            if (e >= 0 && e < E)
                atomicAdd(&lh[e], 1);
            else
                anybad = 1;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 64)
        hist[(int64_t)e * NB + b] = lh[e];
    const uint64_t any = __ballot(anybad);
    if (threadIdx.x == 0)
        bad[b] = any != 0ull;
}

__device__ inline int32_t wave_incl_scan(int32_t v)
{
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int32_t u = __shfl_up(v, d, 64);
        if (lane >= d)
            v += u;
    }
    return v;
}

// Exclusive scan of one value per thread over a 1024-thread block; returns
// the exclusive prefix and writes the block total to *total.
__device__ inline int32_t block_excl_scan(int32_t v, int32_t *s_w, int32_t *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t incl = wave_incl_scan(v);
    __syncthreads();
    if (lane == 63)
        s_w[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        int32_t w = lane < 16 ? s_w[lane] : 0;
        const int32_t wi = wave_incl_scan(w);
        if (lane < 16)
            s_w[16 + lane] = wi - w; // exclusive wave base
        if (lane == 15)
            s_w[32] = wi;
    }
    __syncthreads();
    *total = s_w[32];
    return s_w[16 + wave] + incl - v;
}

// Exclusive scan of one value per expert, held by threads 0 .. n-1 of a
// 1024-thread block (the others hold 0).  With n <= 64 the values all sit in
// wave 0, which scans them with shuffles and no barrier: only wave 0's
// results (and *total) are defined then.  Otherwise the block scan, whose
// results every thread has.
__device__ inline int32_t expert_excl_scan(int32_t v, int n, int32_t *s_w, int32_t *total)
{
    if (n <= 64) {
        if (threadIdx.x >= 64)
            return 0;
        const int32_t incl = wave_incl_scan(v);
        *total = __shfl(incl, 63, 64);
        return incl - v;
    }
    return block_excl_scan(v, s_w, total);
}

// Start-of-forward bookkeeping done by the first routing block: the saved
// context's header and the zeroed release counters of the pipelined forward.
__device__ inline void write_header_and_counters(SavedHeader *hdr, uint64_t problem_hash,
                                                 uint64_t epoch, int32_t *ctr, int nctr)
{
    if (hdr && threadIdx.x == 0) {
        hdr->magic = kSavedMagic;
        hdr->version = kSavedVersion;
        hdr->problem = problem_hash;
        hdr->epoch = epoch;
    }
    for (int j = threadIdx.x; j < nctr; j += blockDim.x)
        ctr[j] = 0;
}

// The owner expert of M-tile j is the last e with s_moff[e] <= j (s_moff holds
// the exclusive prefix of the experts' M-tiles and the total at [E]).
__device__ inline void fill_mtile_owners(const int32_t *s_moff, int E, int32_t mtotal,
                                         int32_t *__restrict__ mtile_expert)
{
    for (int j = threadIdx.x; j < mtotal; j += 1024) {
        int lo = 0, hi = E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_moff[mid] <= j)
                lo = mid;
            else
                hi = mid;
        }
        mtile_expert[j] = lo;
    }
}

// counts, offsets, the M-tile tables and the status word, from expert e's
// count c and exclusive offset off held by thread e (all 1024 threads of one
// block call this; E counts the nsh shared-expert chunks, whose counts are T,
// and total = offsets[E]).  The rows of the shared chunks follow the routed
// ones: row offsets[E - nsh] + cT + t gets sorted_slot t·K, so the gather of a
// GEMM (slot / K) reads token t.
__device__ inline void publish_plan(int32_t c, int32_t off, int32_t total, bool anybad, int E,
                                    int BM, int32_t *__restrict__ counts,
                                    int32_t *__restrict__ offsets,
                                    int32_t *__restrict__ mtile_off,
                                    int32_t *__restrict__ mtile_expert, MTileTable2 t2,
                                    int32_t *__restrict__ status, int32_t *s_w, int32_t *s_moff,
                                    int nsh, int64_t T, int K, int32_t *__restrict__ sorted_slot)
{
    // off and total come from expert_excl_scan: with E <= 64 only wave 0
    // holds them, and wave 0 does all the per-expert work here.  s_moff holds
    // two prefix arrays of E + 1 entries: the M-tiles of BM rows, then those
    // of t2.BM rows.
    const int e = threadIdx.x;
    if (e < E) {
        counts[e] = c;
        offsets[e] = off;
    }
    int32_t *s_moff2 = s_moff + 1025;
    const int32_t mt = (c + BM - 1) / BM;
    int32_t mtotal = 0, mtotal2 = 0;
    const int32_t moff = expert_excl_scan(mt, E, s_w, &mtotal);
    // (t2.BM is uniform: either every thread scans or none)
    const int32_t moff2 =
        t2.BM > 0 ? expert_excl_scan((c + t2.BM - 1) / t2.BM, E, s_w, &mtotal2) : 0;
    if (e < E) {
        mtile_off[e] = moff;
        s_moff[e] = moff;
        if (t2.BM > 0) {
            t2.off[e] = moff2;
            s_moff2[e] = moff2;
        }
    }
    if (e == 0) {
        offsets[E] = total;
        mtile_off[E] = mtotal;
        s_moff[E] = mtotal;
        if (t2.BM > 0) {
            t2.off[E] = mtotal2;
            s_moff2[E] = mtotal2;
        }
        s_w[36] = total;
        s_w[37] = mtotal;
        s_w[38] = mtotal2;
        status[0] = anybad ? MOE_DEV_BAD_ID : 0;
    }
    __syncthreads();
    total = s_w[36];
    mtotal = s_w[37];
    fill_mtile_owners(s_moff, E, mtotal, mtile_expert);
    if (t2.BM > 0)
        fill_mtile_owners(s_moff2, E, s_w[38], t2.expert);
    const int64_t routed = total - (int64_t)nsh * T;
    for (int64_t i = threadIdx.x; i < (int64_t)nsh * T; i += 1024)
        sorted_slot[routed + i] = (int32_t)((i % T) * K);
}

__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t *__restrict__ hist,
                                                          const int32_t *__restrict__ bad, int E,
                                                          int NB, int BM,
                                                          int32_t *__restrict__ counts,
                                                          int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ mtile_off,
                                                          int32_t *__restrict__ mtile_expert,
                                                          MTileTable2 t2,
                                                          int32_t *__restrict__ status,
                                                          int32_t *__restrict__ ctr, int nctr,
                                                          SavedHeader *__restrict__ hdr,
                                                          uint64_t problem_hash, uint64_t epoch,
                                                          int nsh, int64_t T, int K,
                                                          int32_t *__restrict__ sorted_slot)
{
    write_header_and_counters(hdr, problem_hash, epoch, ctr, nctr);
    __shared__ int32_t s_cnt[1024];
    __shared__ int32_t s_moff[2 * 1025];
    __shared__ int32_t s_w[40];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int e = wave; e < E; e += 16) {
        int32_t running = 0;
        int32_t *row = hist + (int64_t)e * NB;
        for (int j0 = 0; j0 < NB; j0 += 64) {
            const int j = j0 + lane;
            const int32_t v = j < NB ? row[j] : 0;
            const int32_t incl = wave_incl_scan(v);
            if (j < NB)
                row[j] = running + incl - v;
            running += __shfl(incl, 63, 64);
        }
        if (lane == 0)
            s_cnt[e] = running;
    }
    int anybad = 0;
    for (int j = threadIdx.x; j < NB; j += 1024)
        anybad |= bad[j];
    anybad = __syncthreads_or(anybad);

    const int e = threadIdx.x;
    const int32_t c = e < E ? s_cnt[e] : e < E + nsh ? (int32_t)T : 0;
    int32_t total;
    const int32_t off = block_excl_scan(c, s_w, &total);
    publish_plan(c, off, total, anybad, E + nsh, BM, counts, offsets, mtile_off, mtile_expert,
                 t2, status, s_w, s_moff, nsh, T, K, sorted_slot);
}

// One wave routes the slots [r0, min(r0 + 512, s1)) in order, 64 at a time,
// from their ids in idv: lanes holding the same expert find each other with
// ballots over the id bits, so the rank inside the round is a popcount and the
// order stays stable.  base[e * bs] is expert e's next position for this chunk
// (LDS, advanced here).
__device__ inline void scatter_round(const int64_t (&idv)[8], int64_t r0, int64_t s1, int E,
                                     int nbits, int32_t *base, int bs,
                                     int32_t *__restrict__ sorted_slot,
                                     int32_t *__restrict__ slot_pos)
{
    const int lane = threadIdx.x & 63;
    const uint64_t lt = lanemask_lt();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t r = r0 + 64 * j;
        if (r >= s1)
            break;
        const int64_t s = r + lane;
        const bool in = s < s1;
        const int64_t eid = idv[j];
        const bool valid = in && eid >= 0 && eid < E;
        const int e = valid ? (int)eid : 0;
        uint64_t m = __ballot(valid);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool v = (e >> bit) & 1;
            const uint64_t bb = __ballot(v);
            m &= v ? bb : ~bb;
        }
        const int rank = __popcll(m & lt);
        int pos = 0;
        if (valid) {
            pos = base[e * bs] + rank;
            sorted_slot[pos] = (int32_t)s;
            slot_pos[s] = pos;
        } else if (in) {
            slot_pos[s] = -1;
        }
        // the lowest lane of each expert group advances that expert's base
        // after every lane of the round has read it (LDS operations of one
        // wave complete in program order)
        if (valid && rank == 0)
            base[e * bs] = pos + __popcll(m);
    }
}

// The same for the slots [s0, s1), a round of ids at a time.
template <typename Id>
__device__ inline void scatter_chunk(const Id *__restrict__ ids, int64_t s0, int64_t s1, int E,
                                     int nbits, int32_t *base, int bs,
                                     int32_t *__restrict__ sorted_slot,
                                     int32_t *__restrict__ slot_pos)
{
    for (int64_t r0 = s0; r0 < s1; r0 += 512) {
        int64_t idv[8];
        load_ids8(ids, r0, s1, idv);
        scatter_round(idv, r0, s1, E, nbits, base, bs, sorted_slot, slot_pos);
    }
}

template <typename Id>
__global__ __launch_bounds__(64) void route_scatter_kernel(
    const Id *__restrict__ ids, int64_t TK, int E, int nbits, int RC, int NB,
    const int32_t *__restrict__ hist, const int32_t *__restrict__ offsets,
    int32_t *__restrict__ sorted_slot, int32_t *__restrict__ slot_pos)
{
    extern __shared__ int32_t base[];
    const int b = blockIdx.x;
    for (int e = threadIdx.x; e < E; e += 64)
        base[e] = offsets[e] + hist[(int64_t)e * NB + b];
    __syncthreads();
    const int64_t s0 = (int64_t)b * RC;
    const int64_t s1 = s0 + RC < TK ? s0 + RC : TK;
    scatter_chunk(ids, s0, s1, E, nbits, base, 1, sorted_slot, slot_pos);
}

// Fused routing: a 1024-thread block owns the 16 consecutive chunks
// 16 b .. 16 b + 15, wave w the chunk 16 b + w.
//  ROUTE_ONE  (NB <= 16, one block): each wave first counts its chunk per
//             expert into the block's table, so routing is one launch.
//  ROUTE_SELF (up to kSelfCountSlots slots): every block counts ALL the ids
//             itself, per expert before its chunks, per (expert, chunk) in
//             them and after them, so routing is one launch and no block
//             waits on another's counts (the redundant reads are L2 hits).
//  ROUTE_HIST: the table comes from route_hist_kernel; every block reads
//             each expert's row of it (all loads issued at once) for the
//             total and the sum over chunks before its own, which replaces
//             the separate scan launch.
// Every block then scans the totals into offsets and turns its table into
// per-(expert, chunk) bases; block 0 also publishes counts, offsets, the
// M-tile tables and the status word.  LDS: tab[E][16], tot[E], bef[E] (and
// aft[E] in ROUTE_SELF).
enum { ROUTE_ONE = 0, ROUTE_SELF = 1, ROUTE_HIST = 2 };
constexpr int64_t kSelfCountSlots = 32768;

template <typename Id, int MODE>
__global__ __launch_bounds__(1024) void route_block_kernel(
    const Id *__restrict__ ids, int64_t TK, int E, int nbits, int RC, int NB, int BM,
    const int32_t *__restrict__ hist, const int32_t *__restrict__ bad,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ mtile_off,
    int32_t *__restrict__ mtile_expert, MTileTable2 t2, int32_t *__restrict__ status,
    int32_t *__restrict__ ctr, int nctr, SavedHeader *__restrict__ hdr, uint64_t problem_hash,
    uint64_t epoch, int nsh, int64_t T, int K, int32_t *__restrict__ sorted_slot,
    int32_t *__restrict__ slot_pos)
{
    extern __shared__ int32_t lds[];
    int32_t *tab = lds;         // [E][16]: chunk counts, then chunk bases
    int32_t *tot = tab + E * 16; // [E]: slots of expert e over all chunks
    int32_t *bef = tot + E;      // [E]: slots of expert e in chunks before this block's
    __shared__ int32_t s_w[40];
    __shared__ int32_t s_moff[2 * 1025];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int b0 = blockIdx.x * 16;
    const bool lead = blockIdx.x == 0;
    int64_t one_ids[8]; // ROUTE_ONE: this wave's ids, from the count to the scatter
    if (lead)
        write_header_and_counters(hdr, problem_hash, epoch, ctr, nctr);
    int anybad = 0;
    if constexpr (MODE == ROUTE_SELF) {
        int32_t *aft = bef + E; // [E]: slots of expert e after this block's chunks
        for (int i = threadIdx.x; i < E * 16; i += 1024)
            tab[i] = 0;
        for (int i = threadIdx.x; i < E; i += 1024)
            bef[i] = aft[i] = 0;
        __syncthreads();
        const int64_t lo = (int64_t)b0 * RC;
        const int64_t hi = lo + 16 * (int64_t)RC < TK ? lo + 16 * (int64_t)RC : TK;
        // thread t counts slots t, t + 1024, ...; 8 loads in flight per round
        for (int64_t s0 = threadIdx.x; s0 < TK; s0 += 8 * 1024) {
            Id raw[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t sl = s0 + 1024 * j;
                raw[j] = ids[sl < TK ? sl : TK - 1];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t sl = s0 + 1024 * j;
                const int64_t e = (int64_t)raw[j];
                if (sl >= TK)
                    continue;
                if (e < 0 || e >= E)
                    anybad = 1;
                else if (sl < lo)
                    atomicAdd(&bef[e], 1);
                else if (sl < hi)
                    atomicAdd(&tab[e * 16 + (int)((sl - lo) / RC)], 1);
                else
                    atomicAdd(&aft[e], 1);
            }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += 1024) {
            int32_t t = bef[e] + aft[e];
#pragma unroll
            for (int w = 0; w < 16; ++w)
                t += tab[e * 16 + w];
            tot[e] = t;
        }
    } else if constexpr (MODE == ROUTE_ONE) {
        for (int i = threadIdx.x; i < E * 16; i += 1024)
            tab[i] = 0;
        __syncthreads();
        // a chunk is one round of at most 512 slots here: its ids stay in
        // registers for the scatter
        const int64_t s0 = (int64_t)wave * RC;
        const int64_t s1 = s0 + RC < TK ? s0 + RC : TK;
        if (s0 < s1) {
            load_ids8(ids, s0, s1, one_ids);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t e = one_ids[j];
                if (s0 + 64 * j + lane >= s1)
                    continue;
                if (e >= 0 && e < E)
                    atomicAdd(&tab[e * 16 + wave], 1);
                else
                    anybad = 1;
            }
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += 1024) {
            int32_t t = 0;
#pragma unroll
            for (int w = 0; w < 16; ++w)
                t += tab[e * 16 + w];
            tot[e] = t;
            bef[e] = 0;
        }
    } else {
        // wave w reads the rows of experts w, w + 16, ...; RB rows x JB
        // 64-chunk segments of them are loaded before any is summed, so that
        // one memory round trip serves them (E = 64 and up to 256 chunks: all
        // of a wave's loads at once); the sums are wave reductions
        constexpr int RB = 4, JB = 4;
        for (int e0 = wave; e0 < E; e0 += 16 * RB) {
            int32_t t[RB], bs[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r)
                t[r] = bs[r] = 0;
            for (int j0 = 0; j0 < NB; j0 += 64 * JB) {
                int32_t v[RB][JB];
#pragma unroll
                for (int r = 0; r < RB; ++r)
#pragma unroll
                    for (int q = 0; q < JB; ++q) {
                        const int e = e0 + 16 * r, j = j0 + 64 * q + lane;
                        v[r][q] = e < E && j < NB ? hist[(int64_t)e * NB + j] : 0;
                    }
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const int e = e0 + 16 * r;
#pragma unroll
                    for (int q = 0; q < JB; ++q) {
                        const int j = j0 + 64 * q + lane;
                        t[r] += v[r][q];
                        bs[r] += j < b0 ? v[r][q] : 0;
                        if (e < E && j >= b0 && j < b0 + 16)
                            tab[e * 16 + (j - b0)] = v[r][q];
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int e = e0 + 16 * r;
                if (e >= E)
                    break;
                if (lane < 16 && b0 + lane >= NB)
                    tab[e * 16 + lane] = 0;
#pragma unroll
                for (int d = 32; d >= 1; d >>= 1) {
                    t[r] += __shfl_xor(t[r], d, 64);
                    bs[r] += __shfl_xor(bs[r], d, 64);
                }
                if (lane == 0) {
                    tot[e] = t[r];
                    bef[e] = bs[r];
                }
            }
        }
        if (lead)
            for (int j = threadIdx.x; j < NB; j += 1024)
                anybad |= bad[j];
    }
    anybad = __syncthreads_or(anybad);

    const int e = threadIdx.x; // E + nsh <= 1024
    const int32_t c = e < E ? tot[e] : e < E + nsh ? (int32_t)T : 0;
    int32_t total = 0;
    // with E + nsh <= 64 only wave 0 gets off and total; it is also the only
    // wave that uses them (publish_plan's per-expert work, the bases below)
    const int32_t off = expert_excl_scan(c, E + nsh, s_w, &total);
    if (lead)
        publish_plan(c, off, total, anybad, E + nsh, BM, counts, offsets, mtile_off,
                     mtile_expert, t2, status, s_w, s_moff, nsh, T, K, sorted_slot);
    if (e < E) {
        int32_t run = off + bef[e];
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int32_t v = tab[e * 16 + w];
            tab[e * 16 + w] = run;
            run += v;
        }
    }
    __syncthreads();
    const int b = b0 + wave;
    if (b < NB) {
        const int64_t s0 = (int64_t)b * RC;
        const int64_t s1 = s0 + RC < TK ? s0 + RC : TK;
        if constexpr (MODE == ROUTE_ONE)
            scatter_round(one_ids, s0, s1, E, nbits, tab + wave, 16, sorted_slot, slot_pos);
        else
            scatter_chunk(ids, s0, s1, E, nbits, tab + wave, 16, sorted_slot, slot_pos);
    }
}

// Backward set-up.  The saved context is trusted only if its header names
// this problem and its offsets are a consistent prefix sum of its counts
// within [0, TK]; then counts and offsets are copied into the workspace and
// the M-tile tables (prefix of ceil(counts[e] / BM) and the owner of every
// M-tile) are built from the copies.  Otherwise the copies are all zero (no
// kernel after this one reads a saved array beyond them) and the status word
// says so.  One 1024-thread block; E <= 1024.
__global__ __launch_bounds__(1024) void bwd_setup_kernel(
    const SavedHeader *__restrict__ hdr, uint64_t problem_hash, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int64_t TK, int BM,
    int32_t *__restrict__ counts_out, int32_t *__restrict__ offsets_out,
    int32_t *__restrict__ mtile_off, int32_t *__restrict__ mtile_expert,
    int32_t *__restrict__ status, SavedHeader *__restrict__ ws_hdr, int stage, XcdSplits splits)
{
    __shared__ int32_t s_moff[1025];
    __shared__ int32_t s_off[1025];
    __shared__ int32_t s_raw[2][8];
    __shared__ int32_t s_w[40];
    __shared__ int s_hdr_ok, s_ws_ok;
    if (threadIdx.x == 0) {
        const SavedHeader h = *hdr;
        s_hdr_ok = h.magic == kSavedMagic && h.version == kSavedVersion && h.problem == problem_hash;
        s_ws_ok = 1;
        if (stage == BWD_STAGE_W) {
            const SavedHeader w = *ws_hdr;
            s_ws_ok = w.magic == h.magic && w.version == h.version && w.problem == h.problem &&
                      w.epoch == h.epoch;
        }
    }
    __syncthreads();
    const int e = threadIdx.x;
    int32_t c = 0, off = 0;
    int bad = 0;
    if (s_hdr_ok && e < E) {
        c = counts[e];
        off = offsets[e];
        const int32_t next = offsets[e + 1];
        bad = c < 0 || off < 0 || next - off != c || (int64_t)next > TK || (e == 0 && off != 0);
    }
    bad = __syncthreads_or(bad);
    const bool ok = s_hdr_ok && !bad && s_ws_ok;
    if (!ok) {
        c = 0;
        off = 0;
    }
    if (e < E) {
        counts_out[e] = c;
        offsets_out[e] = off;
        s_off[e] = off;
    }
    if (e == 0) {
        offsets_out[E] = ok ? offsets[E] : 0;
        s_off[E] = ok ? offsets[E] : 0;
        status[0] = ok ? 0 : !(s_hdr_ok && !bad) ? MOE_DEV_BAD_SAVED : MOE_DEV_BAD_WS;
        if (stage == BWD_STAGE_D) {
            // the stamp the weight-gradient stage will check (zeros: nothing to trust)
            SavedHeader w{};
            if (ok)
                w = *hdr;
            *ws_hdr = w;
        }
    }
    const int32_t mt = e < E ? (c + BM - 1) / BM : 0;
    int32_t mtotal;
    const int32_t moff = block_excl_scan(mt, s_w, &mtotal);
    if (e < E) {
        mtile_off[e] = moff;
        s_moff[e] = moff;
    }
    if (e == 0) {
        mtile_off[E] = mtotal;
        s_moff[E] = mtotal;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < mtotal; j += 1024) {
        int lo = 0, hi = E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_moff[mid] <= j)
                lo = mid;
            else
                hi = mid;
        }
        mtile_expert[j] = lo;
    }

    // Cost-balanced XCD bounds of the weight-gradient launches.  A tile of
    // expert e contracts over its count[e] rows; its cost is modelled as
    // count[e] + TILE_EPS rows (TILE_EPS for the epilogue and tile switch), so
    // with F tiles per expert the cost before tile e F + j is
    // F (off[e] + e TILE_EPS) + j (count[e] + TILE_EPS).  XCD x starts at the
    // first tile whose cost prefix reaches x/8 of the total; that start is then
    // moved to a whole number of rounds of the XCD's workgroups (a multiple of
    // wgx tiles from the previous bound, when there are two rounds or more), so
    // that tiles of equal cost split evenly over the workgroups.
    constexpr int TILE_EPS = 64;
    if (splits.n > 0) {
        const int k = threadIdx.x >> 3, x = threadIdx.x & 7;
        if (k < splits.n && x > 0) {
            const int64_t F = k == 0 ? splits.F[0] : splits.F[1];
            auto prefix = [&](int ex) { return F * ((int64_t)s_off[ex] + (int64_t)ex * TILE_EPS); };
            const int64_t target = prefix(E) * x / 8;
            int lo = 0, hi = E; // largest ex in [0, E] with prefix(ex) <= target
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (prefix(mid) <= target)
                    lo = mid;
                else
                    hi = mid - 1;
            }
            int64_t L = (int64_t)E * F;
            if (lo < E) {
                const int64_t w = (int64_t)(s_off[lo + 1] - s_off[lo]) + TILE_EPS;
                const int64_t j = (target - prefix(lo) + w - 1) / w;
                L = lo * F + (j < F ? j : F);
            }
            s_raw[k][x] = (int32_t)L;
        }
        __syncthreads();
        if (threadIdx.x < splits.n) {
            const int kk = threadIdx.x;
            const int F = kk == 0 ? splits.F[0] : splits.F[1];
            const int wgx = kk == 0 ? splits.wgx[0] : splits.wgx[1];
            const int32_t total = E * F;
            int32_t b = 0;
            splits.bounds[9 * kk] = 0;
            for (int xx = 1; xx < 8; ++xx) {
                int32_t n = max(s_raw[kk][xx], b) - b;
                if (n >= 2 * wgx)
                    n = (n + wgx / 2) / wgx * wgx;
                b = min(b + n, total);
                splits.bounds[9 * kk + xx] = b;
            }
            splits.bounds[9 * kk + 8] = total;
        }
    }
}

hipError_t launch_bwd_setup(const SavedHeader *hdr, uint64_t problem_hash, const int32_t *counts,
                            const int32_t *offsets, int E, int64_t TK, int BM, int32_t *counts_out,
                            int32_t *offsets_out, int32_t *mtile_off, int32_t *mtile_expert,
                            int32_t *status, SavedHeader *ws_hdr, int stage,
                            const XcdSplits &splits, hipStream_t stream)
{
    hipLaunchKernelGGL(bwd_setup_kernel, dim3(1), dim3(1024), 0, stream, hdr, problem_hash, counts,
                       offsets, E, TK, BM, counts_out, offsets_out, mtile_off, mtile_expert, status,
                       ws_hdr, stage, splits);
    return hipGetLastError();
}

// Chunk size: a chunk is one wave's serial work (rounds of 64 slots, each a
// load, a few ballots and a dependent LDS update), so chunks are kept short
// enough that many waves share it: up to 8192 slots spread over the 16 waves
// of one block (at least 64 slots each), beyond that 128-slot chunks over
// several blocks, doubled while there would be more than 4096 chunks.
RoutePlan make_route_plan(int64_t TK, int E)
{
    RoutePlan rp;
    int64_t rc;
    if (TK <= 8192) {
        rc = ((TK + 15) / 16 + 63) / 64 * 64;
        if (rc < 64)
            rc = 64;
    } else {
        rc = 128;
        while ((TK + rc - 1) / rc > 4096)
            rc *= 2;
    }
    rp.RC = (int)rc;
    rp.NB = (int)((TK + rc - 1) / rc);
    if (rp.NB < 1)
        rp.NB = 1;
    int nbits = 0;
    while ((1 << nbits) < E)
        ++nbits;
    rp.nbits = nbits;
    return rp;
}

template <typename Id>
static void launch_route_t(const Id *ids, int64_t TK, int E, int BM, const RoutePlan &rp,
                           const RouteBufs &rb, hipStream_t stream)
{
    const size_t lds = sizeof(int32_t) * (size_t)E;
    const size_t lds_block = sizeof(int32_t) * (size_t)E * 18; // tab[E][16], tot[E], bef[E]
    const size_t lds_self = lds_block + sizeof(int32_t) * (size_t)E; // and aft[E]
    const int K = rb.T > 0 ? (int)(TK / rb.T) : 1;
    const int nctr = rb.ctr ? rb.nctr : 0;
    MTileTable2 t2{rb.mtile2_off, rb.mtile2_expert, rb.mtile2_off ? rb.BM2 : 0};
    if (TK > 0 && lds_block <= 65536) {
        const int nblk = (rp.NB + 15) / 16;
        // (one block means at most 8192 slots, so chunks of at most 512 slots:
        // one round of ids per wave, which ROUTE_ONE keeps in registers)
        const int mode = nblk == 1 && rp.RC <= 512 ? ROUTE_ONE
                         : TK <= kSelfCountSlots && lds_self <= 65536 ? ROUTE_SELF
                                                                     : ROUTE_HIST;
        if (mode == ROUTE_HIST)
            hipLaunchKernelGGL(route_hist_kernel<Id>, dim3(rp.NB), dim3(64), lds, stream, ids, TK, E,
                               rp.RC, rp.NB, rb.hist, rb.bad);
        auto kern = mode == ROUTE_ONE    ? route_block_kernel<Id, ROUTE_ONE>
                    : mode == ROUTE_SELF ? route_block_kernel<Id, ROUTE_SELF>
                                         : route_block_kernel<Id, ROUTE_HIST>;
        hipLaunchKernelGGL(kern, dim3(nblk), dim3(1024), mode == ROUTE_SELF ? lds_self : lds_block,
                           stream, ids, TK, E, rp.nbits, rp.RC, rp.NB, BM, rb.hist, rb.bad,
                           rb.counts, rb.offsets, rb.mtile_off, rb.mtile_expert, t2, rb.status,
                           rb.ctr,
                           nctr, rb.saved_hdr, rb.problem_hash, rb.epoch, rb.nshared, rb.T, K,
                           rb.sorted_slot, rb.slot_pos);
        return;
    }
    // many experts (the block table would not fit), or no slots: hist, scan, scatter
    if (TK > 0)
        hipLaunchKernelGGL(route_hist_kernel<Id>, dim3(rp.NB), dim3(64), lds, stream, ids, TK, E,
                           rp.RC, rp.NB, rb.hist, rb.bad);
    const int nb_scan = TK > 0 ? rp.NB : 0;
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, rb.hist, rb.bad, E,
                       nb_scan, BM, rb.counts, rb.offsets, rb.mtile_off, rb.mtile_expert, t2,
                       rb.status, rb.ctr, nctr, rb.saved_hdr, rb.problem_hash, rb.epoch,
                       rb.nshared, rb.T, K, rb.sorted_slot);
    if (TK > 0)
        hipLaunchKernelGGL(route_scatter_kernel<Id>, dim3(rp.NB), dim3(64), lds, stream, ids, TK, E,
                           rp.nbits, rp.RC, rp.NB, rb.hist, rb.offsets, rb.sorted_slot,
                           rb.slot_pos);
}

// One launch up to 32768 slots (16 chunks: one block; more: self-counting
// blocks), two (hist, block) beyond, three (hist, scan, scatter) when an
// expert table of 18 x E words would not fit 64 KB.
hipError_t launch_route(const void *ids, bool ids64, int64_t TK, int E, int BM,
                        const RoutePlan &rp, const RouteBufs &rb, hipStream_t stream)
{
    if (ids64)
        launch_route_t((const int64_t *)ids, TK, E, BM, rp, rb, stream);
    else
        launch_route_t((const int32_t *)ids, TK, E, BM, rp, rb, stream);
    return hipGetLastError();
}

} // namespace moe
