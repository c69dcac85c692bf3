// Device helpers shared by the gfx950 kernels: element loads/stores for the two
// input dtypes and cross-lane reductions.  Wavefronts are 64 lanes wide.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

typedef __bf16 bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Floor applied to every per-token, per-channel log-decay (channel-wise forms)
// when it is loaded.  Those kernels take exponents relative to 16-token block
// boundaries; 16 tokens at the floor sum to -85, and e^85 stays inside fp32.
// Below the floor the factors would overflow; a gate that is clamped gets a
// zero gradient.  (-85/16 is exact in bf16.)
constexpr float kLogDecayFloor = -85.0f / 16.0f;

// Input element types: fp32 or bf16 (stored as raw 16-bit patterns).
struct F32 {
    typedef float T;
    static constexpr int bytes = 4;
};
struct BF16 {
    typedef uint16_t T;
    static constexpr int bytes = 2;
};
// fp32 inputs whose chunk products run as three bf16 terms of split operands
// (hi + lo, about 16 significant bits) on the bf16 matrix cores; for callers
// whose tolerance is that of bf16 data (DeltaTTT-pre with bf16 inputs).
struct F32S {
    typedef float T;
    static constexpr int bytes = 4;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    bf16_t h = static_cast<bf16_t>(x);
    return __builtin_bit_cast(uint16_t, h);
}

template <typename E>
__device__ __forceinline__ float load_elem(const void* base, int64_t i);
template <>
__device__ __forceinline__ float load_elem<F32>(const void* base, int64_t i) {
    return static_cast<const float*>(base)[i];
}
template <>
__device__ __forceinline__ float load_elem<BF16>(const void* base, int64_t i) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
}

// Four consecutive elements from i (a multiple of 4 in a 16-byte-aligned tensor):
// one 16-byte (fp32) or 8-byte (bf16) load.
template <typename E>
__device__ __forceinline__ float4 load4(const void* base, int64_t i);
template <>
__device__ __forceinline__ float4 load4<F32>(const void* base, int64_t i) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
}
template <>
__device__ __forceinline__ float4 load4<BF16>(const void* base, int64_t i) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

template <typename E>
__device__ __forceinline__ void store_elem(void* base, int64_t i, float x);
template <>
__device__ __forceinline__ void store_elem<F32>(void* base, int64_t i, float x) {
    static_cast<float*>(base)[i] = x;
}
template <>
__device__ __forceinline__ void store_elem<BF16>(void* base, int64_t i, float x) {
    static_cast<uint16_t*>(base)[i] = f32_to_bf16_bits(x);
}

// Sum over the 32 lanes of a half-wave (xor butterfly); every lane gets the sum.
__device__ __forceinline__ float half_wave_sum(float x) {
#pragma unroll
    for (int s = 16; s >= 1; s >>= 1) x += __shfl_xor(x, s, 32);
    return x;
}

}  // namespace dr
