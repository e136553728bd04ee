// Per-row FP8 (OCP E4M3) quantisation (gfx950).
//
// FP8 experts (Skywork-MoE model card: an FP8 checkpoint; news item
// "4090推理": FP8-quantised inference; Megatron-Core page, "关键特性": FP8
// among the coming features).  Every row gets the smallest power-of-two
// scale s with max|row| <= 448 s, and each value v becomes the E4M3 code
// nearest to v / s (ties to even).  The scale is a power of two, so v / s is
// exact and every code is decided exactly; gfx950's packed conversion
// (v_cvt_pk_fp8_f32, OCP E4M3, round to nearest even) does the rounding, and
// |v / s| <= 448 (the largest E4M3 value) by the choice of s, so it never
// overflows.
//
// bf16 rows up to 16384 values: one block per row, read once into registers.
// Longer rows and fp32 rows: one wavefront per row, two passes (max|v|, then
// codes).  Codes are written 8 bytes per 8 values.
#include "common.h"

namespace moe {

// Exponent e of the row scale 2^e: the smallest integer with
// amax <= 448 * 2^e (0 for amax == 0).  With amax = m * 2^x, m in [0.5, 1):
// 448 = 0.875 * 2^9, so e = x - 9 when m <= 0.875, else x - 8.
__device__ __forceinline__ int fp8_scale_exp(float amax)
{
    if (!(amax > 0.0f))
        return 0;
    int x;
    const float m = frexpf(amax, &x);
    return m <= 0.875f ? x - 9 : x - 8;
}

// E4M3 codes of 8 values scaled by 2^-e (|f / 2^e| <= 448), little-endian
// bytes in value order.
__device__ __forceinline__ uint2 e4m3_encode8(const float* f, int e)
{
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[0], -e), ldexpf(f[1], -e), 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[2], -e), ldexpf(f[3], -e), lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[4], -e), ldexpf(f[5], -e), 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[6], -e), ldexpf(f[7], -e), hi, true);
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

template <typename ET>
__global__ __launch_bounds__(256) void moe_quantize_fp8_kernel(const typename ET::storage* __restrict__ src,
                                                               long long R, int K, uint8_t* __restrict__ codes,
                                                               float* __restrict__ scales)
{
    const int lane = lane_id();
    const long long r = (long long)blockIdx.x * 4 + threadIdx.x / kWave;
    if (r >= R)
        return;
    const typename ET::storage* row = src + (size_t)r * K;
    const int nvec = K / 8;  // 8 values per step (16 B of bf16, 32 B of fp32)
    float amax = 0.0f;
    for (int c = lane; c < nvec; c += kWave) {
        float f[8];
        load8(row + (size_t)c * 8, f);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            amax = fmaxf(amax, fabsf(f[i]));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, o));
    const int e = fp8_scale_exp(amax);
    uint8_t* out = codes + (size_t)r * K;
    for (int c = lane; c < nvec; c += kWave) {
        float f[8];
        load8(row + (size_t)c * 8, f);
        *reinterpret_cast<uint2*>(out + (size_t)c * 8) = e4m3_encode8(f, e);
    }
    if (lane == 0)
        scales[r] = ldexpf(1.0f, e);
}

// bf16 rows of at most 256 * 8 * V values, one block of 256 threads per
// row: the row is read once into registers (V 16-byte vectors per thread),
// the block finds max|v| (wavefront shuffles, then the 4 wavefronts through
// LDS) and writes the codes from the registers, so the row crosses HBM once.
// The loads are non-temporal (the row is not read again) and unconditional
// (index clamped; vectors past the row are zeroed after the load).
template <int V>
__global__ __launch_bounds__(256) void moe_quantize_fp8_bf16_kernel(const uint16_t* __restrict__ src, int K,
                                                                    uint8_t* __restrict__ codes,
                                                                    float* __restrict__ scales)
{
    __shared__ float s_max[4];
    const long long r = blockIdx.x;
    const uint4* row = reinterpret_cast<const uint4*>(src + (size_t)r * K);
    const int nvec = K / 8;
    uint4 buf[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int c = threadIdx.x + 256 * i;
        typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
        const u32x4v q = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(row + min(c, nvec - 1)));
        buf[i] = c < nvec ? make_uint4(q.x, q.y, q.z, q.w) : make_uint4(0u, 0u, 0u, 0u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        float f[8];
        unpack8(buf[i], f, bf16_t{});
#pragma unroll
        for (int q = 0; q < 8; ++q)
            amax = fmaxf(amax, fabsf(f[q]));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        amax = fmaxf(amax, __shfl_xor(amax, o));
    if (lane_id() == 0)
        s_max[threadIdx.x / kWave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const int e = fp8_scale_exp(amax);
    uint8_t* out = codes + (size_t)r * K;
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int c = threadIdx.x + 256 * i;
        if (c < nvec) {
            float f[8];
            unpack8(buf[i], f, bf16_t{});
            *reinterpret_cast<uint2*>(out + (size_t)c * 8) = e4m3_encode8(f, e);
        }
    }
    if (threadIdx.x == 0)
        scales[r] = ldexpf(1.0f, e);
}

}  // namespace moe

// src: R rows of K values (dtype 0 fp32, 1 bf16), K a multiple of 8.
extern "C" hipError_t moe_launch_quantize_fp8(int dtype, const void* src, long long R, int K, uint8_t* codes,
                                              float* scales, hipStream_t stream)
{
    using namespace moe;
    if (R <= 0)
        return hipSuccess;
    const dim3 grid((unsigned)((R + 3) / 4)), block(256);
    const int per_thread = (K / 8 + 255) / 256;  // 16-byte bf16 vectors per thread, one block per row
    const uint16_t* sb = (const uint16_t*)src;
    const dim3 rows((unsigned)R);
    if (dtype == 0)
        moe_quantize_fp8_kernel<f32_t><<<grid, block, 0, stream>>>((const float*)src, R, K, codes, scales);
    else if (per_thread <= 2)
        moe_quantize_fp8_bf16_kernel<2><<<rows, block, 0, stream>>>(sb, K, codes, scales);
    else if (per_thread <= 4)
        moe_quantize_fp8_bf16_kernel<4><<<rows, block, 0, stream>>>(sb, K, codes, scales);
    else if (per_thread <= 8)
        moe_quantize_fp8_bf16_kernel<8><<<rows, block, 0, stream>>>(sb, K, codes, scales);
    else
        moe_quantize_fp8_kernel<bf16_t><<<grid, block, 0, stream>>>(sb, R, K, codes, scales);
    return hipGetLastError();
}
