// common.h — device types and helpers shared by the gfx950 kernels of the
// MoE expert-FFN library.  Internal header; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

using bf16 = __bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Matrix-core step for one element type.  Both operand fragments carry KPL
// consecutive k values per lane; a 16x16 output block accumulates in fp32.
//   A fragment: lane l holds row (l % 16), k = (l / 16) * KPL + [0, KPL)
//   B fragment: lane l holds column (l % 16), same k range
//   C block:    lane l holds column (l % 16), rows (l / 16) * 4 + [0, 4)
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
    static constexpr int KPL = 8;    // bf16 per lane per instruction
    static constexpr int KSTEP = 32; // k covered by one instruction
    using Frag = bf16x8;
    __device__ static inline f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<float> {
    static constexpr int KPL = 1;
    static constexpr int KSTEP = 4;
    using Frag = float;
    __device__ static inline f32x4 mma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <typename T> __device__ inline float to_f32(T v);
template <> __device__ inline float to_f32<float>(float v) { return v; }
template <> __device__ inline float to_f32<bf16>(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ inline T from_f32(float v);
template <> __device__ inline float from_f32<float>(float v) { return v; }
template <> __device__ inline bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

// silu(a) = a * sigmoid(a) = a / (1 + e^-a), with the hardware exp and
// reciprocal (about 1 ulp each).  Saturates correctly: a -> -inf gives -0
// (e^-a = inf, 1/inf = 0), a -> +inf gives a.
__device__ inline float silu_f(float a)
{
    return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// 16-byte vector of T
template <typename T> struct Vec16 {
    static constexpr int N = 16 / sizeof(T);
};

__device__ inline uint64_t lanemask_lt() {
    const unsigned lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

} // namespace moe
