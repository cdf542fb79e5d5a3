// combine.hip — unpermute and top-k gate-weighted combine.
//
// y[t, :] = Σ_{k = 0..K-1} g[t, k] · o[slot_pos[t·K + k], :]
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

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ o,
                                                      const int32_t *__restrict__ slot_pos,
                                                      const float *__restrict__ gates,
                                                      T *__restrict__ y, int H, int K)
{
    constexpr int VEC = 16 / (int)sizeof(T);
    const int64_t t = blockIdx.x;
    const int nch = H / VEC;
    for (int c = threadIdx.x; c < nch; c += 256) {
        float acc[VEC];
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            acc[j] = 0.f;
        for (int k = 0; k < K; ++k) {
            const int32_t p = slot_pos[t * K + k];
            if (p < 0)
                continue;
            const float g = gates[t * K + k];
            const u32x4 v = *reinterpret_cast<const u32x4 *>(o + (int64_t)p * H + (int64_t)c * VEC);
            const T *vv = reinterpret_cast<const T *>(&v);
#pragma unroll
            for (int j = 0; j < VEC; ++j)
                acc[j] += g * to_f32<T>(vv[j]);
        }
        u32x4 out;
        T *oo = reinterpret_cast<T *>(&out);
#pragma unroll
        for (int j = 0; j < VEC; ++j)
            oo[j] = from_f32<T>(acc[j]);
        *reinterpret_cast<u32x4 *>(y + t * H + (int64_t)c * VEC) = out;
    }
}

hipError_t launch_combine(int dtype, const void *o, const int32_t *slot_pos, const float *gates,
                          void *y, int64_t T, int H, int K, hipStream_t stream)
{
    if (T <= 0)
        return hipSuccess;
    if (dtype == 1)
        hipLaunchKernelGGL(combine_kernel<bf16>, dim3((unsigned)T), dim3(256), 0, stream,
                           static_cast<const bf16 *>(o), slot_pos, gates, static_cast<bf16 *>(y), H,
                           K);
    else
        hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)T), dim3(256), 0, stream,
                           static_cast<const float *>(o), slot_pos, gates, static_cast<float *>(y),
                           H, K);
    return hipGetLastError();
}

} // namespace moe
