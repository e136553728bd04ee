// Gate-weighted combine back to token order (gfx950).
//
// The gate weights the chosen experts' outputs (industry overview page,
// "MoE的內涵"); a dropped choice contributes nothing and the residual outside
// the layer carries the token (Megatron-Core page, "MoE负载均衡的挑战与应对").
//
// A wavefront owns a slice of one token's row (two 16-byte vectors per lane,
// so a 4096-wide bf16 row takes four wavefronts).  For j = 0..k-1 in order,
// if slot[t,j] >= 0 it reads that slice of y_perm[slot] and accumulates
// topk_w[t,j] * row in fp32 (fma, fixed order, so results are reproducible
// and do not depend on the slicing), then writes its slice of y[t] once
// (non-temporal stores).  The loads of two choices are issued before either
// is added.  y_perm rows are read once, with non-temporal loads: they do not
// displace dirty lines that would then be written back during the combine
// (with a freshly written 1 GiB buffer in the caches a launch took 35 us
// with plain loads, 22 us with these).  Short slices keep the registers low enough for eight wavefronts
// per SIMD, and the many small wavefronts overlap their load, add and store
// phases across the chip.
// Slots at or past the row count (T*k) are treated as dropped.  With y_add
// (the shared expert's output, industry overview page, "MoE未來重點研究方向"
// item 4: DeepSeekMoE's shared experts) the sum starts from y_add[t]: every
// token gets it with weight one (its row is read once too, non-temporally).
#include "common.h"

namespace moe {

// 16-byte vectors per lane in one wavefront's slice of a row, and choices
// whose loads are issued together
constexpr int kCombineVec = 2;
constexpr int kCombineGroup = 2;

template <typename ET>
__global__ __launch_bounds__(256) void moe_combine_kernel(const typename ET::storage* __restrict__ y_perm,
                                                          const int32_t* __restrict__ slot,
                                                          const float* __restrict__ topk_w,
                                                          const typename ET::storage* __restrict__ y_add, int T,
                                                          int d, int k, int max_rows, int nparts,
                                                          typename ET::storage* __restrict__ y)
{
    constexpr int kVec = kCombineVec, kG = kCombineGroup;
    const int lane = lane_id();
    const int unit = blockIdx.x * 4 + threadIdx.x / kWave;
    const int t = unit / nparts;
    const int part = unit - t * nparts;
    if (t >= T)
        return;
    constexpr int kPer = 16 / ET::kBytes;
    const int nvec = d / kPer;
    const int v0 = part * kWave * kVec;
    float acc[kVec][kPer];
#pragma unroll
    for (int u = 0; u < kVec; ++u)
#pragma unroll
        for (int q = 0; q < kPer; ++q)
            acc[u][q] = 0.0f;
    if (y_add) {
        const uint4* src = reinterpret_cast<const uint4*>(y_add + (size_t)t * d);
        uint4 ra[kVec];
#pragma unroll
        for (int u = 0; u < kVec; ++u) {
            const int v = v0 + u * kWave + lane;
            if (v < nvec) {
                typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
                const u32x4v q = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(src + v));
                ra[u] = make_uint4(q.x, q.y, q.z, q.w);
            }
        }
#pragma unroll
        for (int u = 0; u < kVec; ++u) {
            const int v = v0 + u * kWave + lane;
            if (v < nvec) {
                if constexpr (ET::kBytes == 2) {
                    unpack8(ra[u], acc[u], bf16_t{});
                } else {
                    acc[u][0] = __uint_as_float(ra[u].x);
                    acc[u][1] = __uint_as_float(ra[u].y);
                    acc[u][2] = __uint_as_float(ra[u].z);
                    acc[u][3] = __uint_as_float(ra[u].w);
                }
            }
        }
    }
    for (int j0 = 0; j0 < k; j0 += kG) {
        int rows[kG];
        float w[kG];
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            const int j = j0 + h;
            rows[h] = (j < k) ? slot[(size_t)t * k + j] : -1;
            if (rows[h] >= max_rows)
                rows[h] = -1;  // out-of-range slots count as dropped
            w[h] = (j < k) ? topk_w[(size_t)t * k + j] : 0.0f;
        }
        uint4 raw[kG][kVec];
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            if (rows[h] < 0)
                continue;
            const uint4* src = reinterpret_cast<const uint4*>(y_perm + (size_t)rows[h] * d);
#pragma unroll
            for (int u = 0; u < kVec; ++u) {
                const int v = v0 + u * kWave + lane;
                if (v < nvec) {
                    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
                    const u32x4v q = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(src + v));
                    raw[h][u] = make_uint4(q.x, q.y, q.z, q.w);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            if (rows[h] < 0)
                continue;
#pragma unroll
            for (int u = 0; u < kVec; ++u) {
                const int v = v0 + u * kWave + lane;
                if (v < nvec) {
                    float f[kPer];
                    if constexpr (ET::kBytes == 2) {
                        unpack8(raw[h][u], f, bf16_t{});
                    } else {
                        f[0] = __uint_as_float(raw[h][u].x);
                        f[1] = __uint_as_float(raw[h][u].y);
                        f[2] = __uint_as_float(raw[h][u].z);
                        f[3] = __uint_as_float(raw[h][u].w);
                    }
#pragma unroll
                    for (int q = 0; q < kPer; ++q)
                        acc[u][q] = fmaf(w[h], f[q], acc[u][q]);
                }
            }
        }
    }
    uint4* dst = reinterpret_cast<uint4*>(y + (size_t)t * d);
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
        const int v = v0 + u * kWave + lane;
        if (v < nvec) {
            uint4 o;
            if constexpr (ET::kBytes == 2) {
                o.x = f32_to_bf16_bits(acc[u][0]) | (f32_to_bf16_bits(acc[u][1]) << 16);
                o.y = f32_to_bf16_bits(acc[u][2]) | (f32_to_bf16_bits(acc[u][3]) << 16);
                o.z = f32_to_bf16_bits(acc[u][4]) | (f32_to_bf16_bits(acc[u][5]) << 16);
                o.w = f32_to_bf16_bits(acc[u][6]) | (f32_to_bf16_bits(acc[u][7]) << 16);
            } else {
                o.x = __float_as_uint(acc[u][0]);
                o.y = __float_as_uint(acc[u][1]);
                o.z = __float_as_uint(acc[u][2]);
                o.w = __float_as_uint(acc[u][3]);
            }
            // y is written once and not read back here: a non-temporal
            // store (measured 10% faster at the Mixtral shape)
            typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
            __builtin_nontemporal_store(u32x4v{o.x, o.y, o.z, o.w}, reinterpret_cast<u32x4v*>(dst + v));
        }
    }
}

}  // namespace moe

// y_add (nullable): added to every token's sum with weight one.
extern "C" hipError_t moe_launch_combine(int dtype, const void* y_perm, const int32_t* slot, const float* topk_w,
                                         const void* y_add, int T, int d, int k, int max_rows, void* y,
                                         hipStream_t stream)
{
    using namespace moe;
    const int per = dtype == 0 ? 4 : 8;  // elements per 16-byte vector
    const int nparts = (d / per + kWave * kCombineVec - 1) / (kWave * kCombineVec);
    const long units = (long)T * nparts;
    if (units == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((units + 3) / 4)), block(256);
    if (dtype == 0)
        moe_combine_kernel<f32_t><<<grid, block, 0, stream>>>((const float*)y_perm, slot, topk_w,
                                                              (const float*)y_add, T, d, k, max_rows, nparts,
                                                              (float*)y);
    else
        moe_combine_kernel<bf16_t><<<grid, block, 0, stream>>>((const uint16_t*)y_perm, slot, topk_w,
                                                               (const uint16_t*)y_add, T, d, k, max_rows, nparts,
                                                               (uint16_t*)y);
    return hipGetLastError();
}
