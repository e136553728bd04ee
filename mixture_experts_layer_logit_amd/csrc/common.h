// Device helpers shared by the gfx950 kernels of the MoE-layer forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Element types as stored in memory.  bf16 is kept as its raw 16-bit pattern.
struct f32_t {
    typedef float storage;
    static constexpr int kBytes = 4;
};
struct bf16_t {
    typedef uint16_t storage;
    static constexpr int kBytes = 2;
};
// OCP FP8 E4M3 codes (sign, 4 exponent bits with bias 7, 3 mantissa bits).
struct fp8_t {
    typedef uint8_t storage;
    static constexpr int kBytes = 1;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Unpack 16 bytes into 8 fp32 values.
__device__ __forceinline__ void unpack8(const uint4& v, float* out, bf16_t)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(w[i] << 16);
        out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Load 8 consecutive elements (16 B for bf16, 32 B for fp32) as fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float* out)
{
    uint4 v = *reinterpret_cast<const uint4*>(p);
    unpack8(v, out, bf16_t{});
}
__device__ __forceinline__ void load8(const float* p, float* out)
{
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Store 8 fp32 values as 8 elements.
__device__ __forceinline__ void store8(uint16_t* p, const float* v)
{
    uint4 o;
    o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
    o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
    o.z = f32_to_bf16_bits(v[4]) | (f32_to_bf16_bits(v[5]) << 16);
    o.w = f32_to_bf16_bits(v[6]) | (f32_to_bf16_bits(v[7]) << 16);
    *reinterpret_cast<uint4*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float* v)
{
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace moe
