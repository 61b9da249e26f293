// Device helpers shared by the gfx950 kernels of libpdn.so (not a public header).
#pragma once
#include <hip/hip_runtime.h>
#include <cmath>
#include <stdint.h>

#include "pdn.h"

namespace pdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Per-token decay is clamped below at this natural log in the prefill: the
// chunk algorithm splits exp(G_r - G_s) around a reference inside a 16-token
// block, and the clamp keeps both factors inside the fp32/bf16 range.  (The
// scalar-decay kernel forms a chunk that decays more strongly element by
// element instead, and floors log decays only at kLogAlphaFloor: e^-80 is
// below what an fp32 state resolves.)
constexpr float kLogAlphaMin = -10.0f;
constexpr float kLogAlphaFloor = -80.0f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    bf16 h = static_cast<bf16>(x);  // round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

// Load element i of a q/k/v tensor stored as fp32 or bf16.
template <bool BF16>
__device__ __forceinline__ float load_in(const void* p, long i) {
    if constexpr (BF16)
        return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    else
        return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace pdn
