// combine.hip — unpermute and top-k gate-weighted combine.
//
// y[t, :] = Σ_{k = 0..K-1} g[t, k] · o[slot_pos[t·K + k], :]
//           + Σ_{c = 0..S-1} o[offsets[Er] + c·T + t, :]   (shared expert, if any)
//
// (HyperMegaMoE issue page, section 2.1 "Combine" and section 4.1: expert
// outputs go back to their token and are summed with the routing weights.)
// The overlap explainer page (section 6) asks that every one of a token's K
// branches is merged exactly once with its own gate, and weighs float atomics
// (rounding-order nondeterminism) against a segmented reduction whose
// segments match the route.  This kernel is that segmented reduction: one
// workgroup owns whole tokens, reads the K rows in k order, accumulates in
// fp32 and rounds once, so the result is bitwise reproducible.  A slot whose
// id was out of range (slot_pos = -1) contributes nothing.
#include "common.h"
#include "kernels.h"

namespace moe {

// Grid: (token, block of 256 16-byte chunks).  Each thread owns one chunk of
// one token's output row; its K source rows are loaded 8 at a time before
// they are accumulated in k order, so their latencies overlap.  NT: the rows
// are read with the non-temporal hint (o larger than the last-level cache,
// where the GEMM that wrote it leaves no useful copy behind).
template <typename T, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ o,
                                                      const int32_t *__restrict__ slot_pos,
                                                      const float *__restrict__ gates,
                                                      T *__restrict__ y, int H, int K,
                                                      const int32_t *__restrict__ offsets,
                                                      int Er, int S, int64_t ntok)
{
    constexpr int VEC = 16 / (int)sizeof(T);
    const int64_t t = blockIdx.x;
    const int nch = H / VEC;
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= nch)
        return;
    float acc[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j)
        acc[j] = 0.f;
    for (int k0 = 0; k0 < K; k0 += 8) {
        int32_t pk[8];
        u32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pk[i] = k0 + i < K ? slot_pos[t * K + k0 + i] : -1;
            const int64_t row = pk[i] > 0 ? pk[i] : 0;
            const u32x4 *src = reinterpret_cast<const u32x4 *>(o + row * H + (int64_t)c * VEC);
            v[i] = NT ? __builtin_nontemporal_load(src) : *src;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (pk[i] < 0)
                continue;
            const float g = gates[t * K + k0 + i];
            const T *vv = reinterpret_cast<const T *>(&v[i]);
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                acc[j] += g * to_f32<T>(vv[j]);
        }
    }
    // the shared expert's chunks (issue page, section 6.1: merged at combine),
    // gate 1, after the routed terms
    if (S > 0) {
        const int64_t base = offsets[Er] + t;
        for (int sc = 0; sc < S; ++sc) {
            const u32x4 v =
                *reinterpret_cast<const u32x4 *>(o + (base + sc * ntok) * H + (int64_t)c * VEC);
            const T *vv = reinterpret_cast<const T *>(&v);
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                acc[j] += to_f32<T>(vv[j]);
        }
    }
    u32x4 out;
    T *oo = reinterpret_cast<T *>(&out);
#pragma unroll
    for (int j = 0; j < VEC; ++j)
        oo[j] = from_f32<T>(acc[j]);
    *reinterpret_cast<u32x4 *>(y + t * H + (int64_t)c * VEC) = out;
}

// Backward combine (issue page, section 2.2 "Combine(dX)"): one workgroup per
// token sums its K rows of dx_perm in k order (no gate: it is already inside
// dh) and finishes d_topk_weights[t, k] by summing that row's partial dots in a
// fixed order.  Deterministic; a dropped slot (slot_pos = -1) gives 0, and a
// saved context that failed the backward set-up's check gives all zeros
// (slot_pos is then not read).
__global__ __launch_bounds__(256) void combine_bwd_kernel(const bf16 *__restrict__ dxp,
                                                          const float *__restrict__ dgp,
                                                          int dgp_stride,
                                                          const int32_t *__restrict__ slot_pos,
                                                          const int32_t *__restrict__ status,
                                                          bf16 *__restrict__ dx,
                                                          float *__restrict__ d_topk, int H, int K,
                                                          const int32_t *__restrict__ offsets,
                                                          int Er, int S, int64_t ntok)
{
    // grid: (token, block of 256 16-byte chunks); the first chunk block of a
    // token also finishes its d_topk_weights
    const int64_t t = blockIdx.x;
    const int nch = H / 8;
    const int c = blockIdx.y * 256 + threadIdx.x;
    const bool bad = status[0] & (MOE_DEV_BAD_SAVED | MOE_DEV_BAD_WS);
    if (c < nch) {
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[j] = 0.f;
        if (!bad) {
            for (int k0 = 0; k0 < K; k0 += 8) {
                int32_t pk[8];
                u32x4 v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    pk[i] = k0 + i < K ? slot_pos[t * K + k0 + i] : -1;
                    const int64_t row = pk[i] > 0 ? pk[i] : 0;
                    v[i] = *reinterpret_cast<const u32x4 *>(dxp + row * H + (int64_t)c * 8);
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (pk[i] < 0)
                        continue;
                    const bf16 *vv = reinterpret_cast<const bf16 *>(&v[i]);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc[j] += static_cast<float>(vv[j]);
                }
            }
            // the shared expert's chunks, after the routed terms
            if (S > 0) {
                const int64_t base = offsets[Er] + t;
                for (int sc = 0; sc < S; ++sc) {
                    const u32x4 v = *reinterpret_cast<const u32x4 *>(
                        dxp + (base + sc * ntok) * H + (int64_t)c * 8);
                    const bf16 *vv = reinterpret_cast<const bf16 *>(&v);
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        acc[j] += static_cast<float>(vv[j]);
                }
            }
        }
        u32x4 out;
        bf16 *oo = reinterpret_cast<bf16 *>(&out);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            oo[j] = static_cast<bf16>(acc[j]);
        *reinterpret_cast<u32x4 *>(dx + t * H + (int64_t)c * 8) = out;
    }
    // d_topk: one lane per k
    if (blockIdx.y == 0 && threadIdx.x < K) {
        const int k = threadIdx.x;
        float d = 0.f;
        if (!bad) {
            const int32_t p = slot_pos[t * K + k];
            if (p >= 0)
                for (int j = 0; j < dgp_stride; ++j)
                    d += dgp[(int64_t)p * dgp_stride + j];
        }
        d_topk[t * K + k] = d;
    }
}

hipError_t launch_combine_bwd(const void *dxp, const float *dgp, int dgp_stride,
                              const int32_t *slot_pos, const int32_t *status, void *dx,
                              float *d_topk, int64_t T, int H, int K, const int32_t *offsets,
                              int Er, int S, hipStream_t stream)
{
    if (T <= 0)
        return hipSuccess;
    const unsigned cblocks = (unsigned)((H / 8 + 255) / 256);
    hipLaunchKernelGGL(combine_bwd_kernel, dim3((unsigned)T, cblocks), dim3(256), 0, stream,
                       static_cast<const bf16 *>(dxp), dgp, dgp_stride, slot_pos, status,
                       static_cast<bf16 *>(dx), d_topk, H, K, offsets, Er, S, T);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4 *__restrict__ p, int64_t n)
{
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        p[i] = z;
}

hipError_t launch_zero_fill(void *p, size_t bytes, hipStream_t stream)
{
    const int64_t n = (int64_t)(bytes / 16);
    if (n <= 0)
        return hipSuccess;
    const int64_t blocks = n / 256 + 1 < 4096 ? n / 256 + 1 : 4096;
    hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<u32x4 *>(p), n);
    return hipGetLastError();
}

hipError_t launch_combine(int dtype, const void *o, const int32_t *slot_pos, const float *gates,
                          void *y, int64_t T, int H, int K, const int32_t *offsets, int Er, int S,
                          hipStream_t stream)
{
    if (T <= 0)
        return hipSuccess;
    const int vec = dtype == 1 ? 8 : 4;
    const unsigned cblocks = (unsigned)((H / vec + 255) / 256);
    const dim3 grid((unsigned)T, cblocks);
    // o of more than 192 MB does not stay in the 256 MB last-level cache
    // behind the GEMM that wrote it: stream it (skewed shape, 939 MB: the
    // combine 216 -> 184 us); smaller o is re-read from that cache, where
    // the hint made it slower (134 MB: 31 -> 37 us)
    const bool nt = T * (K + S) * (int64_t)H * (dtype == 1 ? 2 : 4) > ((int64_t)192 << 20);
    if (dtype == 1) {
        auto k = nt ? combine_kernel<bf16, true> : combine_kernel<bf16, false>;
        hipLaunchKernelGGL(k, grid, dim3(256), 0, stream, static_cast<const bf16 *>(o), slot_pos,
                           gates, static_cast<bf16 *>(y), H, K, offsets, Er, S, T);
    } else {
        auto k = nt ? combine_kernel<float, true> : combine_kernel<float, false>;
        hipLaunchKernelGGL(k, grid, dim3(256), 0, stream, static_cast<const float *>(o), slot_pos,
                           gates, static_cast<float *>(y), H, K, offsets, Er, S, T);
    }
    return hipGetLastError();
}

} // namespace moe
