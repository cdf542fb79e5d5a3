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
// grouped GEMMs walk, with mtile_expert[j], the expert owning M-tile j.
//
// Three launches, no global atomics and no memset:
//   1. hist:    one wave per chunk of RC slots counts ids per expert in LDS
//               and writes its column of hist[E][NB] plus a bad-id flag.
//   2. scan:    one 1024-thread block turns hist into per-(expert, chunk)
//               exclusive bases, then scans counts and M-tile counts over
//               experts, writes the status word and zeroes the release
//               counters of the pipelined forward that follows.
//   3. scatter: one wave per chunk walks its slots in order, 64 at a time;
//               lanes holding the same expert find each other with ballots
//               over the id bits, so the rank inside the round is a popcount
//               and the order stays stable.
#include "common.h"
#include "kernels.h"

namespace moe {

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
    for (int64_t s = s0 + threadIdx.x; s < s1; s += 64) {
        const int64_t e = (int64_t)ids[s];
        if (e >= 0 && e < E)
            atomicAdd(&lh[e], 1);
        else
            anybad = 1;
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

__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t *__restrict__ hist,
                                                          const int32_t *__restrict__ bad, int E,
                                                          int NB, int BM,
                                                          int32_t *__restrict__ counts,
                                                          int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ mtile_off,
                                                          int32_t *__restrict__ mtile_expert,
                                                          int32_t *__restrict__ status,
                                                          int32_t *__restrict__ ctr, int nctr,
                                                          SavedHeader *__restrict__ hdr,
                                                          uint64_t problem_hash)
{
    if (hdr && threadIdx.x == 0) {
        hdr->magic = kSavedMagic;
        hdr->version = kSavedVersion;
        hdr->problem = problem_hash;
    }
    for (int j = threadIdx.x; j < nctr; j += 1024)
        ctr[j] = 0;
    __shared__ int32_t s_cnt[1024];
    __shared__ int32_t s_moff[1025];
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
    const int32_t c = e < E ? s_cnt[e] : 0;
    int32_t total;
    const int32_t off = block_excl_scan(c, s_w, &total);
    if (e < E) {
        counts[e] = c;
        offsets[e] = off;
    }
    const int32_t mt = (c + BM - 1) / BM;
    int32_t mtotal;
    const int32_t moff = block_excl_scan(mt, s_w, &mtotal);
    if (e < E) {
        mtile_off[e] = moff;
        s_moff[e] = moff;
    }
    if (e == 0) {
        offsets[E] = total;
        mtile_off[E] = mtotal;
        s_moff[E] = mtotal;
        status[0] = anybad ? MOE_DEV_BAD_ID : 0;
    }
    __syncthreads();
    // owner expert of every M-tile: the last e with s_moff[e] <= j
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
    const int lane = threadIdx.x;
    const uint64_t lt = lanemask_lt();
    const int64_t s0 = (int64_t)b * RC;
    const int64_t s1 = s0 + RC < TK ? s0 + RC : TK;
    for (int64_t r = s0; r < s1; r += 64) {
        const int64_t s = r + lane;
        const bool in = s < s1;
        const int64_t eid = in ? (int64_t)ids[s] : -1;
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
            pos = base[e] + rank;
            sorted_slot[pos] = (int32_t)s;
            slot_pos[s] = pos;
        } else if (in) {
            slot_pos[s] = -1;
        }
        // the lowest lane of each expert group advances that expert's base
        // after every lane of the round has read it (LDS operations of one
        // wave complete in program order)
        if (valid && rank == 0)
            base[e] = pos + __popcll(m);
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
    int32_t *__restrict__ status)
{
    __shared__ int32_t s_moff[1025];
    __shared__ int32_t s_w[40];
    __shared__ int s_hdr_ok;
    if (threadIdx.x == 0)
        s_hdr_ok = hdr->magic == kSavedMagic && hdr->version == kSavedVersion &&
                   hdr->problem == problem_hash;
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
    const bool ok = s_hdr_ok && !bad;
    if (!ok) {
        c = 0;
        off = 0;
    }
    if (e < E) {
        counts_out[e] = c;
        offsets_out[e] = off;
    }
    if (e == 0) {
        offsets_out[E] = ok ? offsets[E] : 0;
        status[0] = ok ? 0 : MOE_DEV_BAD_SAVED;
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
}

hipError_t launch_bwd_setup(const SavedHeader *hdr, uint64_t problem_hash, const int32_t *counts,
                            const int32_t *offsets, int E, int64_t TK, int BM, int32_t *counts_out,
                            int32_t *offsets_out, int32_t *mtile_off, int32_t *mtile_expert,
                            int32_t *status, hipStream_t stream)
{
    hipLaunchKernelGGL(bwd_setup_kernel, dim3(1), dim3(1024), 0, stream, hdr, problem_hash, counts,
                       offsets, E, TK, BM, counts_out, offsets_out, mtile_off, mtile_expert, status);
    return hipGetLastError();
}

RoutePlan make_route_plan(int64_t TK, int E)
{
    RoutePlan rp;
    int64_t rc = 512;
    while ((TK + rc - 1) / rc > 4096)
        rc *= 2;
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

hipError_t launch_route(const void *ids, bool ids64, int64_t TK, int E, int BM,
                        const RoutePlan &rp, const RouteBufs &rb, hipStream_t stream)
{
    const size_t lds = sizeof(int32_t) * (size_t)E;
    if (TK > 0) {
        if (ids64)
            hipLaunchKernelGGL(route_hist_kernel<int64_t>, dim3(rp.NB), dim3(64), lds, stream,
                               (const int64_t *)ids, TK, E, rp.RC, rp.NB, rb.hist, rb.bad);
        else
            hipLaunchKernelGGL(route_hist_kernel<int32_t>, dim3(rp.NB), dim3(64), lds, stream,
                               (const int32_t *)ids, TK, E, rp.RC, rp.NB, rb.hist, rb.bad);
    }
    const int nb_scan = TK > 0 ? rp.NB : 0;
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, stream, rb.hist, rb.bad, E,
                       nb_scan, BM, rb.counts, rb.offsets, rb.mtile_off, rb.mtile_expert,
                       rb.status, rb.ctr, rb.ctr ? rb.nctr : 0, rb.saved_hdr, rb.problem_hash);
    if (TK > 0) {
        if (ids64)
            hipLaunchKernelGGL(route_scatter_kernel<int64_t>, dim3(rp.NB), dim3(64), lds, stream,
                               (const int64_t *)ids, TK, E, rp.nbits, rp.RC, rp.NB, rb.hist,
                               rb.offsets, rb.sorted_slot, rb.slot_pos);
        else
            hipLaunchKernelGGL(route_scatter_kernel<int32_t>, dim3(rp.NB), dim3(64), lds, stream,
                               (const int32_t *)ids, TK, E, rp.nbits, rp.RC, rp.NB, rb.hist,
                               rb.offsets, rb.sorted_slot, rb.slot_pos);
    }
    return hipGetLastError();
}

} // namespace moe
