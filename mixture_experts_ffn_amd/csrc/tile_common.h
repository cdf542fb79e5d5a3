// tile_common.h — device helpers of the forward tile kernels (gemm_mfma.hip,
// gemm_big.hip): LDS swizzles, direct global -> LDS copies, explicit memory
// waits and the decoding of a grouped GEMM's logical tile index.  Internal.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {
namespace tile {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int PW = 128;         // weight columns per panel (two panels per tile)
constexpr int TILE_N1 = PW;     // GEMM1 output columns per tile
constexpr int TILE_N2 = 2 * PW; // GEMM2 output columns per tile

enum { KIND_G1 = 1, KIND_G2 = 2 };

__device__ __forceinline__ int bswz(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

template <int N> struct IC {
    static constexpr int value = N;
};

// swizzled 16-byte piece of A row r: rows of 8 pieces (128 B) XOR by
// (r / 2) % 8, rows of 4 pieces (64 B) by (r / 4) % 4, so the 16 rows that one
// 128-bit fragment read touches fall in 16 different bank groups
template <int PIECES> __device__ __forceinline__ int aswz(int r, int piece)
{
    return PIECES == 8 ? piece ^ ((r >> 1) & 7) : piece ^ ((r >> 2) & 3);
}
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Routing metadata that earlier launches wrote and this kernel only reads:
// loaded through the constant address space, so a wave-uniform index becomes
// a scalar load (lgkmcnt) that never waits for the copies on vmcnt.
__device__ __forceinline__ int ldc(const int32_t *p, int i)
{
    return ((const __attribute__((address_space(4))) int32_t *)p)[uni(i)];
}
__device__ __forceinline__ float ldcf(const float *p, int i)
{
    return ((const __attribute__((address_space(4))) float *)p)[uni(i)];
}

// 16-byte global -> LDS copy per lane into [l, l + 1024) (lane i at l + 16 i).
// Issued as inline assembly so that the compiler does not track these LDS
// writes: their completion is established explicitly (wait_vm) per stage,
// instead of the compiler waiting for every copy in flight before each LDS
// read.  `l` must be wave-uniform.
__device__ __forceinline__ void g2l16(const void *g, lds_void *l)
{
    const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_addr), "v"(g)
                 : "memory", "m0");
}

// The same copy addressed as a wave-uniform 64-bit base (scalar registers)
// plus a 32-bit unsigned per-lane byte offset: one VGPR per copy source
// instead of two, and the per-step advance is scalar arithmetic.
__device__ __forceinline__ void g2l16s(const void *base, uint32_t voff, lds_void *l)
{
    const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
    // the base is wave-uniform; readfirstlane pins it to scalar registers.
    // The builtin returns a signed int: each half is taken as uint32_t
    // before widening, so a low word with bit 31 set is not sign-extended
    // into the high word.
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t sb = (uint64_t)lo | ((uint64_t)hi << 32);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(sb)
                 : "memory", "m0");
}

// The same copy with the non-temporal hint: for weight panels a launch
// streams from HBM once, so that they do not displace the token rows the
// tiles of the same expert re-read from L2.
__device__ __forceinline__ void g2l16_nt(const void *g, lds_void *l)
{
    const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                 :
                 : "s"(lds_addr), "v"(g)
                 : "memory", "m0");
}

// The same copy as a device-coherent load (sc1: served at the device's
// coherence point, never from a stale cache line), for data that another
// workgroup of the same launch wrote with device-coherent stores.
__device__ __forceinline__ void g2l16_coherent(const void *g, lds_void *l)
{
    const uint32_t lds_addr = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off sc1"
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

struct Tile {
    int kind, e, row0, rows, n0, nt, mt;
};

// Logical tile L of one grouped GEMM -> (expert, first permuted row, real
// rows, first output column, N-tile, global M-tile).  Order: expert-major;
// inside an expert, groups of up to 8 M-tiles with N-tiles outer and M-tiles
// inner, so consecutive tiles share a weight panel.  Wave-uniform.
__device__ __forceinline__ Tile decode_tile(const FastFwdArgs &a, int kind, int L, int ntn,
                                            int BM)
{
    Tile t;
    t.kind = kind;
    L = uni(L);
    t.e = ldc(a.mtile_expert, L / ntn);
    const int mt0 = ldc(a.mtile_off, t.e);
    const int mt_e = ldc(a.mtile_off, t.e + 1) - mt0;
    const int local = L - mt0 * ntn;
    constexpr int GM = 8;
    const int grp = local / (GM * ntn);
    const int first_m = grp * GM;
    const int gm = min(mt_e - first_m, GM);
    const int rr = local - grp * GM * ntn;
    t.nt = uni(rr / gm);
    const int m_t = first_m + rr % gm;
    t.mt = uni(mt0 + m_t);
    t.row0 = uni(ldc(a.offsets, t.e) + m_t * BM);
    t.rows = uni(min(BM, ldc(a.offsets, t.e + 1) - t.row0));
    t.n0 = uni(t.nt * (kind == KIND_G1 ? TILE_N1 : TILE_N2));
    t.e = uni(t.e);
    return t;
}

} // namespace tile
} // namespace moe
