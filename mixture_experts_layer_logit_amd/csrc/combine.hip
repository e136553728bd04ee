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
// (non-temporal stores).  The token's slots and weights are wave-uniform
// (scalar loads), and every choice's row is read through a buffer resource
// over that row alone (empty for a dropped choice), so the loads of all k
// choices leave back to back with no branch between them; the adds follow.
// y_perm rows are read once, with non-temporal loads: they do not displace
// dirty lines that would then be written back during the combine (with a
// freshly written 1 GiB buffer in the caches a launch took 35 us with plain
// loads, 22 us with these).  Short slices keep the registers low enough for
// eight wavefronts per SIMD, and the many small wavefronts overlap their
// load, add and store phases across the chip.
// Slots at or past the row count (T*k) are treated as dropped.  With y_add
// (the shared expert's output, industry overview page, "MoE未來重點研究方向"
// item 4: DeepSeekMoE's shared experts) the sum starts from y_add[t]: every
// token gets it with weight one (its row is read once too, non-temporally).
#include <type_traits>

#include "common.h"

namespace moe {

// 16-byte vectors per lane in one wavefront's slice of a row
constexpr int kCombineVec = 2;

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over one row of `bytes` bytes (0: every load returns
// zero and every store is dropped, without a memory access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// KMAX: a compile-time bound on k.  The token, its slots and weights are
// wave-uniform (scalar loads); each choice's row is addressed through a
// buffer resource of that row alone, empty for a dropped choice, and a lane's
// vectors past the row's end fall outside it too, so every choice's loads are
// issued back to back with no branch or wait between them (loads past a
// resource read zero).  The sum then runs over the kept choices in order.
template <typename ET, int KMAX>
__global__ __launch_bounds__(256) void moe_combine_kernel(const typename ET::storage* __restrict__ y_perm,
                                                          const int32_t* __restrict__ slot,
                                                          const float* __restrict__ topk_w,
                                                          const typename ET::storage* __restrict__ y_add, int T,
                                                          int d, int k, int max_rows, int nparts,
                                                          typename ET::storage* __restrict__ y)
{
    constexpr int kVec = kCombineVec;
    constexpr int kPer = 16 / ET::kBytes;  // elements per 16-byte vector
    constexpr int kNT = 2;                 // buffer cache policy: non-temporal
    const int lane = lane_id();
    const int unit = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + threadIdx.x / kWave);
    const int t = unit / nparts;
    const int part = unit - t * nparts;
    if (t >= T)
        return;
    const uint32_t row_bytes = (uint32_t)d * ET::kBytes;
    // this lane's byte offsets in a row
    uint32_t off[kVec];
#pragma unroll
    for (int u = 0; u < kVec; ++u)
        off[u] = (uint32_t)((part * kWave * kVec + u * kWave + lane) * 16);
    float acc[kVec][kPer];
#pragma unroll
    for (int u = 0; u < kVec; ++u)
#pragma unroll
        for (int q = 0; q < kPer; ++q)
            acc[u][q] = 0.0f;
    auto unpack = [](const i32x4_t& r, float* f) {
        if constexpr (ET::kBytes == 2) {
            unpack8(make_uint4(r.x, r.y, r.z, r.w), f, bf16_t{});
        } else {
            f[0] = __int_as_float(r.x);
            f[1] = __int_as_float(r.y);
            f[2] = __int_as_float(r.z);
            f[3] = __int_as_float(r.w);
        }
    };
    int rows[KMAX];
    float w[KMAX];
    i32x4_t raw[KMAX][kVec];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        rows[j] = -1;
        w[j] = 0.0f;
        if (j < k) {
            rows[j] = slot[(size_t)t * k + j];
            w[j] = topk_w[(size_t)t * k + j];
            if (rows[j] >= max_rows)
                rows[j] = -1;  // out-of-range slots count as dropped
        }
        const bool kept = rows[j] >= 0;
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(y_perm + (size_t)(kept ? rows[j] : 0) * d, kept ? row_bytes : 0);
#pragma unroll
        for (int u = 0; u < kVec; ++u)
            raw[j][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off[u], 0, kNT);
    }
    if (y_add) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(y_add + (size_t)t * d, row_bytes);
#pragma unroll
        for (int u = 0; u < kVec; ++u)
            unpack(__builtin_amdgcn_raw_buffer_load_b128(rs, (int)off[u], 0, kNT), acc[u]);
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (rows[j] < 0)
            continue;
#pragma unroll
        for (int u = 0; u < kVec; ++u) {
            float f[kPer];
            unpack(raw[j][u], f);
#pragma unroll
            for (int q = 0; q < kPer; ++q)
                acc[u][q] = fmaf(w[j], f[q], acc[u][q]);
        }
    }
    // y is written once and not read back here: non-temporal stores; lanes
    // past the row's end fall outside its resource and store nothing
    const __amdgpu_buffer_rsrc_t ry = row_rsrc(y + (size_t)t * d, row_bytes);
#pragma unroll
    for (int u = 0; u < kVec; ++u) {
        i32x4_t o;
        if constexpr (ET::kBytes == 2) {
            o.x = (int)(f32_to_bf16_bits(acc[u][0]) | (f32_to_bf16_bits(acc[u][1]) << 16));
            o.y = (int)(f32_to_bf16_bits(acc[u][2]) | (f32_to_bf16_bits(acc[u][3]) << 16));
            o.z = (int)(f32_to_bf16_bits(acc[u][4]) | (f32_to_bf16_bits(acc[u][5]) << 16));
            o.w = (int)(f32_to_bf16_bits(acc[u][6]) | (f32_to_bf16_bits(acc[u][7]) << 16));
        } else {
            o.x = __float_as_int(acc[u][0]);
            o.y = __float_as_int(acc[u][1]);
            o.z = __float_as_int(acc[u][2]);
            o.w = __float_as_int(acc[u][3]);
        }
        __builtin_amdgcn_raw_buffer_store_b128(o, ry, (int)off[u], 0, kNT);
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
    auto go = [&](auto et, auto kmax) {
        typedef decltype(et) ET;
        typedef typename ET::storage St;
        moe_combine_kernel<ET, decltype(kmax)::value><<<grid, block, 0, stream>>>(
            (const St*)y_perm, slot, topk_w, (const St*)y_add, T, d, k, max_rows, nparts, (St*)y);
    };
    auto by_k = [&](auto et) {
        if (k <= 2)
            go(et, std::integral_constant<int, 2>{});
        else if (k <= 4)
            go(et, std::integral_constant<int, 4>{});
        else
            go(et, std::integral_constant<int, 8>{});
    };
    if (dtype == 0)
        by_k(f32_t{});
    else
        by_k(bf16_t{});
    return hipGetLastError();
}
