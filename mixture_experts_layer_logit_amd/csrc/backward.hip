// Backward of the MoE layer: the memory-bound pieces (gfx950).
//
// The layer's gradient (all throughput figures on the pages are for training:
// Skywork news item "训练Infra", FastMoE page "特色三", Megatron-Core page
// "训练效果与性能实测").  The expert GEMMs of the backward run on the grouped
// GEMM kernel; this file holds what surrounds them:
//   combine backward   d_yp[slot[t,j]] = w[t,j] dy[t];  d_w[t,j] = <dy[t], y_perm[slot[t,j]]>
//   segment offsets    each expert's rows padded to a multiple of 64, for the
//                      weight gradients' K ranges
//   transposes         the weights (so the input-gradient GEMMs keep K
//                      contiguous), and the permuted rows of d_yp, h, du, x
//                      into [columns][padded rows] (so the weight-gradient
//                      GEMMs reduce over rows with K contiguous)
//   un-permute         dx[t] = sum_j dx_perm[slot[t,j]] + sum_e dz[t,e] Wg[e]
//   gate gradients     dWg[e] = sum_t dz[t,e] x[t],  dbg[e] = sum_t dz[t,e]
// Every sum runs in a fixed order (no atomics), so results are the same on
// every run.
#include "common.h"

namespace moe {

__device__ __forceinline__ float wave_sum_f(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

template <typename ET>
__device__ __forceinline__ void load_vec(const typename ET::storage* p, float* f)  // 16 bytes
{
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    if constexpr (ET::kBytes == 2) {
        unpack8(raw, f, bf16_t{});
    } else {
        f[0] = __uint_as_float(raw.x);
        f[1] = __uint_as_float(raw.y);
        f[2] = __uint_as_float(raw.z);
        f[3] = __uint_as_float(raw.w);
    }
}

template <typename ET>
__device__ __forceinline__ void store_vec(typename ET::storage* p, const float* f)  // 16 bytes
{
    uint4 o;
    if constexpr (ET::kBytes == 2) {
        o.x = f32_to_bf16_bits(f[0]) | (f32_to_bf16_bits(f[1]) << 16);
        o.y = f32_to_bf16_bits(f[2]) | (f32_to_bf16_bits(f[3]) << 16);
        o.z = f32_to_bf16_bits(f[4]) | (f32_to_bf16_bits(f[5]) << 16);
        o.w = f32_to_bf16_bits(f[6]) | (f32_to_bf16_bits(f[7]) << 16);
    } else {
        o.x = __float_as_uint(f[0]);
        o.y = __float_as_uint(f[1]);
        o.z = __float_as_uint(f[2]);
        o.w = __float_as_uint(f[3]);
    }
    *reinterpret_cast<uint4*>(p) = o;
}

template <typename ET>
__device__ __forceinline__ void unpack_vec(const uint4& raw, float* f)  // 16 bytes
{
    if constexpr (ET::kBytes == 2) {
        unpack8(raw, f, bf16_t{});
    } else {
        f[0] = __uint_as_float(raw.x);
        f[1] = __uint_as_float(raw.y);
        f[2] = __uint_as_float(raw.z);
        f[3] = __uint_as_float(raw.w);
    }
}

// 16 bytes of a stream read once (non-temporal: no allocation that would
// displace reused or dirty lines).
template <typename T>
__device__ __forceinline__ uint4 nt_load16(const T* p)
{
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v q = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
    return make_uint4(q.x, q.y, q.z, q.w);
}

// One wavefront per token.  Lane l owns 16-byte vectors l, l+64, ... of the
// row; a dot product is the lanes' partial sums (each in vector order) added
// by a fixed shuffle tree.  Slots at or past max_rows count as dropped.  Two
// vectors of dy and of every kept choice's y_perm row are loaded before any
// is used (kMaxK bounds k, so the registers follow the choice count).
template <typename ET, int kMaxK>
__global__ __launch_bounds__(256) void moe_combine_bwd_kernel(const typename ET::storage* __restrict__ dy,
                                                              const typename ET::storage* __restrict__ y_perm,
                                                              const int32_t* __restrict__ slot,
                                                              const float* __restrict__ topk_w, int T, int d, int k,
                                                              int max_rows, typename ET::storage* __restrict__ d_yp,
                                                              float* __restrict__ d_w)
{
    constexpr int kPer = 16 / ET::kBytes;
    constexpr int kU = 2;  // vectors per lane per pass
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T)
        return;
    const int nvec = d / kPer;
    int rows[kMaxK];
    float w[kMaxK], dot[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        rows[j] = (j < k) ? slot[(size_t)t * k + j] : -1;
        if (rows[j] >= max_rows)
            rows[j] = -1;
        w[j] = (j < k) ? topk_w[(size_t)t * k + j] : 0.0f;
        dot[j] = 0.0f;
    }
    const uint4* gsrc = reinterpret_cast<const uint4*>(dy + (size_t)t * d);
    for (int v0 = lane; v0 < nvec; v0 += kWave * kU) {
        uint4 graw[kU], yraw[kU][kMaxK];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int v = v0 + u * kWave;
            if (v < nvec)
                graw[u] = nt_load16(gsrc + v);
        }
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (rows[j] < 0)
                continue;
            const uint4* ysrc = reinterpret_cast<const uint4*>(y_perm + (size_t)rows[j] * d);
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                const int v = v0 + u * kWave;
                if (v < nvec)
                    yraw[u][j] = nt_load16(ysrc + v);
            }
        }
        // keep the uses below the loads (otherwise each load is waited on alone)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int v = v0 + u * kWave;
            if (v >= nvec)
                break;
            float g[kPer];
            unpack_vec<ET>(graw[u], g);
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (rows[j] < 0)
                    continue;
                float yv[kPer], o[kPer];
                unpack_vec<ET>(yraw[u][j], yv);
#pragma unroll
                for (int q = 0; q < kPer; ++q) {
                    dot[j] = fmaf(g[q], yv[q], dot[j]);
                    o[q] = w[j] * g[q];
                }
                store_vec<ET>(d_yp + (size_t)rows[j] * d + (size_t)v * kPer, o);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (j >= k)
            break;
        const float s = wave_sum_f(dot[j]);
        if (lane == 0)
            d_w[(size_t)t * k + j] = rows[j] >= 0 ? s : 0.0f;
    }
}

// Padded segment starts: kofs[e] = sum over e' < e of round_up(rows_e', align),
// rows_e from offsets clamped into [0, max_rows] and made non-decreasing.  One
// block of 1024 threads (E <= 1024).
__global__ __launch_bounds__(1024) void moe_kofs_kernel(const int32_t* __restrict__ offsets, int E, int max_rows,
                                                        int align, int32_t* __restrict__ kofs)
{
    __shared__ int32_t wsum[1024 / kWave];
    const int e = threadIdx.x;
    int padded = 0;
    if (e < E) {
        const int lo = min(max(offsets[e], 0), max_rows);
        const int hi = min(max(offsets[e + 1], lo), max_rows);
        padded = (hi - lo + align - 1) / align * align;
    }
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    int incl = padded;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int n = __shfl_up(incl, o);
        if (lane >= o)
            incl += n;
    }
    if (lane == kWave - 1)
        wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w)
        base += wsum[w];
    if (e < E)
        kofs[e] = base + incl - padded;
    if (e == E - 1)
        kofs[E] = base + incl;
}

// 64 x 64 tile transpose through LDS with 16-byte global accesses: row r of
// the tile is read from src_row(r) (nullptr: zeros), and row c of the
// transposed tile (column c of the input) is written to dst_row(c); both are
// 16-byte aligned pointers to 64 consecutive elements.  256 threads.  The
// tile pitch of 65 elements spreads both the row-wise LDS writes and the
// column-wise LDS reads over the banks.
template <typename ET, typename SrcRow, typename DstRow>
__device__ __forceinline__ void transpose_tile64(typename ET::storage (*tile)[65], SrcRow src_row, DstRow dst_row)
{
    typedef typename ET::storage T;
    constexpr int kPer = 16 / ET::kBytes;      // elements per 16-byte vector
    constexpr int kVecs = 64 / kPer;            // vectors per 64-element row
    constexpr int kRows = 256 / kVecs;          // rows per pass
    const int v = threadIdx.x % kVecs, r0 = threadIdx.x / kVecs;
#pragma unroll
    for (int p = 0; p < 64 / kRows; ++p) {
        const int r = r0 + p * kRows;
        const T* row = src_row(r);
        uint4 raw = make_uint4(0u, 0u, 0u, 0u);
        if (row)
            raw = *reinterpret_cast<const uint4*>(row + v * kPer);
        const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            tile[r][v * kPer + j] = e[j];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 64 / kRows; ++p) {
        const int c = r0 + p * kRows;
        uint4 raw;
        T* e = reinterpret_cast<T*>(&raw);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
            e[j] = tile[v * kPer + j][c];
        *reinterpret_cast<uint4*>(dst_row(c) + v * kPer) = raw;
    }
}

// Batched transpose: dst[b][c][r] = src[b][r][c] for R x C matrices, R and C
// multiples of 64.  Block: one 64 x 64 tile (blockIdx.x: column tile,
// blockIdx.y: row tile, blockIdx.z: matrix).
template <typename ET>
__global__ __launch_bounds__(256) void moe_transpose_kernel(const typename ET::storage* __restrict__ src, int R,
                                                            int C, typename ET::storage* __restrict__ dst)
{
    typedef typename ET::storage T;
    __shared__ T tile[64][65];
    const size_t b = blockIdx.z;
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const T* s = src + b * (size_t)R * C + (size_t)r0 * C + c0;
    T* o = dst + b * (size_t)R * C + (size_t)c0 * R + r0;
    transpose_tile64<ET>(
        tile, [&](int r) -> const T* { return s + (size_t)r * C; }, [&](int c) -> T* { return o + (size_t)c * R; });
}

// Permuted rows into [columns][padded rows]: dst[c][q] for padded position q
// of expert e (kofs[e] <= q < kofs[e+1]) is src[row][c] with row =
// offsets[e] + q - kofs[e] (through gather[row] when given) while that is
// inside the expert's rows, else 0.  C a multiple of 64; ld (dst row stride)
// a multiple of 64.  Block: 64 positions (blockIdx.x, the long axis) x 64
// columns (blockIdx.y).
template <typename ET>
__global__ __launch_bounds__(256) void moe_seg_transpose_kernel(const typename ET::storage* __restrict__ src,
                                                                const int32_t* __restrict__ gather,
                                                                int gather_rows, const int32_t* __restrict__ offsets,
                                                                const int32_t* __restrict__ kofs, int E,
                                                                int max_rows, int C, int ld,
                                                                typename ET::storage* __restrict__ dst)
{
    typedef typename ET::storage T;
    __shared__ T tile[64][65];
    __shared__ int32_t s_row[64];
    const int q0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
    if (threadIdx.x < 64) {
        const int q = q0 + threadIdx.x;
        int row = -1;
        if (q < kofs[E]) {
            int lo = 0, hi = E;  // largest e with kofs[e] <= q
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (kofs[mid] <= q)
                    lo = mid;
                else
                    hi = mid;
            }
            const int a = min(max(offsets[lo], 0), max_rows);
            const int b = min(max(offsets[lo + 1], a), max_rows);
            const int r = a + (q - kofs[lo]);
            if (r < b) {
                row = r;
                if (gather) {
                    row = gather[r];
                    if (row < 0 || row >= gather_rows)
                        row = -1;
                }
            }
        }
        s_row[threadIdx.x] = row;
    }
    __syncthreads();
    transpose_tile64<ET>(
        tile,
        [&](int r) -> const T* {
            const int row = s_row[r];
            return row >= 0 ? src + (size_t)row * C + c0 : nullptr;
        },
        [&](int c) -> T* { return dst + (size_t)(c0 + c) * ld + q0; });
}

// bf16 version of the segment transpose without LDS: one wavefront per
// 64 positions x 64 columns.  Lane l loads 8 columns (one 16-byte vector) of
// the rows of positions 8 (l % 8) + i, i = 0..7, at columns 8 (l / 8) + 0..7,
// transposes that 8 x 8 block in registers, and stores it as 8 columns x 8
// positions (16-byte vectors): the 8 lanes of equal l / 8 load 8 whole
// 128-byte row runs and store 8 whole 128-byte runs of destination rows.
// Block: 4 wavefronts over 4 column tiles (blockIdx.y covers 256 columns).
__global__ __launch_bounds__(256) void moe_seg_transpose_bf16_kernel(const uint16_t* __restrict__ src,
                                                                     const int32_t* __restrict__ gather,
                                                                     int gather_rows,
                                                                     const int32_t* __restrict__ offsets,
                                                                     const int32_t* __restrict__ kofs, int E,
                                                                     int max_rows, int C, int ld,
                                                                     uint16_t* __restrict__ dst)
{
    const int lane = lane_id();
    const int q0 = blockIdx.x * 64;
    const int c0 = (blockIdx.y * 4 + threadIdx.x / kWave) * 64;
    if (c0 >= C)
        return;
    // source row of position q0 + lane (-1: padding or an empty gather entry)
    int row = -1;
    {
        const int q = q0 + lane;
        if (q < kofs[E]) {
            int lo = 0, hi = E;  // largest e with kofs[e] <= q
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (kofs[mid] <= q)
                    lo = mid;
                else
                    hi = mid;
            }
            const int a = min(max(offsets[lo], 0), max_rows);
            const int b = min(max(offsets[lo + 1], a), max_rows);
            const int r = a + (q - kofs[lo]);
            if (r < b) {
                row = r;
                if (gather) {
                    row = gather[r];
                    if (row < 0 || row >= gather_rows)
                        row = -1;
                }
            }
        }
    }
    const int pg = lane % 8, cg = lane / 8;  // position group (8 positions), column group (8 columns)
    uint32_t w[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = __shfl(row, 8 * pg + i);
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (r >= 0)
            v = nt_load16(src + (size_t)r * C + c0 + 8 * cg);
        w[i][0] = v.x;
        w[i][1] = v.y;
        w[i][2] = v.z;
        w[i][3] = v.w;
    }
    // output column j: positions 8 pg + 0..7, two per 32-bit word
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const uint32_t a = w[2 * m][j / 2], b = w[2 * m + 1][j / 2];
            o[m] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        *reinterpret_cast<uint4*>(dst + (size_t)(c0 + 8 * cg + j) * ld + q0 + 8 * pg) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// dx[t] = sum over kept j (in order) of dx_perm[slot[t,j]], plus, with a
// gate, sum over e (in order) of dz[t,e] Wg[e].  A wavefront owns a slice of
// the rows of kUnpTok consecutive tokens (kUnpVec 16-byte vectors per lane):
// each gate row slice it loads serves all of its tokens, and the loads of two
// choices of every token, or of four experts' gate rows, are issued before
// they are added.
constexpr int kUnpVec = 1;
constexpr int kUnpTok = 2;

template <typename ET>
__global__ __launch_bounds__(256) void moe_unpermute_bwd_kernel(const typename ET::storage* __restrict__ dx_perm,
                                                                const int32_t* __restrict__ slot, int T, int d, int k,
                                                                int max_rows, const float* __restrict__ dz,
                                                                const typename ET::storage* __restrict__ Wg, int E,
                                                                int nparts, typename ET::storage* __restrict__ dx)
{
    constexpr int kPer = 16 / ET::kBytes;
    const int lane = lane_id();
    const int unit = blockIdx.x * 4 + threadIdx.x / kWave;
    const int tg = unit / nparts;
    const int part = unit - tg * nparts;
    const int t0 = tg * kUnpTok;
    if (t0 >= T)
        return;
    const int ntok = min(kUnpTok, T - t0);
    const int nvec = d / kPer;
    const int v0 = part * kWave * kUnpVec;
    float acc[kUnpTok][kUnpVec][kPer];
#pragma unroll
    for (int i = 0; i < kUnpTok; ++i)
#pragma unroll
        for (int u = 0; u < kUnpVec; ++u)
#pragma unroll
            for (int q = 0; q < kPer; ++q)
                acc[i][u][q] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += 2) {
        int rows[kUnpTok][2];
#pragma unroll
        for (int i = 0; i < kUnpTok; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int j = j0 + h;
                rows[i][h] = (i < ntok && j < k) ? slot[(size_t)(t0 + i) * k + j] : -1;
                if (rows[i][h] >= max_rows)
                    rows[i][h] = -1;
            }
        uint4 raw[kUnpTok][2][kUnpVec];
#pragma unroll
        for (int i = 0; i < kUnpTok; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (rows[i][h] < 0)
                    continue;
                const uint4* src = reinterpret_cast<const uint4*>(dx_perm + (size_t)rows[i][h] * d);
#pragma unroll
                for (int u = 0; u < kUnpVec; ++u) {
                    const int v = v0 + u * kWave + lane;
                    if (v < nvec)
                        raw[i][h][u] = nt_load16(src + v);
                }
            }
#pragma unroll
        for (int i = 0; i < kUnpTok; ++i)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (rows[i][h] < 0)
                    continue;
#pragma unroll
                for (int u = 0; u < kUnpVec; ++u) {
                    if (v0 + u * kWave + lane < nvec) {
                        float g[kPer];
                        unpack_vec<ET>(raw[i][h][u], g);
#pragma unroll
                        for (int q = 0; q < kPer; ++q)
                            acc[i][u][q] += g[q];
                    }
                }
            }
    }
    if (Wg) {
        for (int e0 = 0; e0 < E; e0 += 4) {
            uint4 raw[4][kUnpVec];
            float z[kUnpTok][4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if (e0 + h >= E)
                    continue;
#pragma unroll
                for (int i = 0; i < kUnpTok; ++i)
                    z[i][h] = i < ntok ? dz[(size_t)(t0 + i) * E + e0 + h] : 0.0f;
                const uint4* src = reinterpret_cast<const uint4*>(Wg + (size_t)(e0 + h) * d);
#pragma unroll
                for (int u = 0; u < kUnpVec; ++u) {
                    const int v = v0 + u * kWave + lane;
                    if (v < nvec)
                        raw[h][u] = src[v];
                }
            }
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                if (e0 + h >= E)
                    continue;
#pragma unroll
                for (int u = 0; u < kUnpVec; ++u) {
                    if (v0 + u * kWave + lane < nvec) {
                        float wv[kPer];
                        unpack_vec<ET>(raw[h][u], wv);
#pragma unroll
                        for (int i = 0; i < kUnpTok; ++i)
#pragma unroll
                            for (int q = 0; q < kPer; ++q)
                                acc[i][u][q] = fmaf(z[i][h], wv[q], acc[i][u][q]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kUnpTok; ++i) {
        if (i >= ntok)
            break;
#pragma unroll
        for (int u = 0; u < kUnpVec; ++u) {
            const int v = v0 + u * kWave + lane;
            if (v < nvec)
                store_vec<ET>(dx + (size_t)(t0 + i) * d + (size_t)v * kPer, acc[i][u]);
        }
    }
}

// Gate gradients, pass 1: block (token chunk of 64, column group of 256,
// expert group of 16): partial[chunk][e][c] = sum over the chunk's tokens (in
// order) of dz[t,e] x[t,c]; the column-group-0 blocks also write
// partial_b[chunk][e] = sum over the chunk's tokens of dz[t,e].  Pass 2 adds
// the chunks in order.  The chunk's dz values are staged in LDS (read as
// broadcasts) and each thread loads x for 16 tokens before using them, so
// the loads overlap instead of each token waiting for its own.
constexpr int kGateChunk = 64;

template <typename ET>
__global__ __launch_bounds__(256) void moe_gate_wgrad_kernel(const float* __restrict__ dz,
                                                             const typename ET::storage* __restrict__ x, int T, int d,
                                                             int E, float* __restrict__ partial,
                                                             float* __restrict__ partial_b)
{
    __shared__ float4 sdz[kGateChunk][4];  // [token of the chunk][experts e0..e0+15], zero past E
    const int t0 = blockIdx.x * kGateChunk, nt = min(T, t0 + kGateChunk) - t0;
    const int e0 = blockIdx.z * 16;
    for (int i = threadIdx.x; i < kGateChunk * 16; i += 256) {
        const int tt = i >> 4, ee = i & 15;
        reinterpret_cast<float*>(sdz)[i] = (tt < nt && e0 + ee < E) ? dz[(size_t)(t0 + tt) * E + e0 + ee] : 0.0f;
    }
    __syncthreads();
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c < d) {
        float acc[16];
#pragma unroll
        for (int ee = 0; ee < 16; ++ee)
            acc[ee] = 0.0f;
        auto token = [&](int tt, float xt) {
            float z[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 q = sdz[tt][g];
                z[4 * g] = q.x;
                z[4 * g + 1] = q.y;
                z[4 * g + 2] = q.z;
                z[4 * g + 3] = q.w;
            }
#pragma unroll
            for (int ee = 0; ee < 16; ++ee)
                acc[ee] = fmaf(z[ee], xt, acc[ee]);
        };
        auto load_x = [&](int tt) -> float {
            const size_t at = (size_t)(t0 + tt) * d + c;
            if constexpr (ET::kBytes == 2)
                return __uint_as_float((uint32_t)x[at] << 16);
            else
                return x[at];
        };
        // whole batches of 16 tokens: the loads carry no branch, so all 16
        // are in flight before the first is used; then the chunk's tail
        int tb = 0;
        for (; tb + 16 <= nt; tb += 16) {
            float xv[16];
#pragma unroll
            for (int u = 0; u < 16; ++u)
                xv[u] = load_x(tb + u);
            // keep the scheduler from interleaving the uses with the loads
            // (it otherwise reuses one register per load and waits on each)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 16; ++u)
                token(tb + u, xv[u]);
        }
        for (; tb < nt; ++tb)
            token(tb, load_x(tb));
#pragma unroll
        for (int ee = 0; ee < 16; ++ee)
            if (e0 + ee < E)
                partial[((size_t)blockIdx.x * E + e0 + ee) * d + c] = acc[ee];
    }
    if (blockIdx.y == 0 && threadIdx.x < 16 && e0 + (int)threadIdx.x < E) {
        const float* col = reinterpret_cast<const float*>(sdz) + threadIdx.x;
        float sb = 0.0f;
        for (int tt = 0; tt < nt; ++tt)
            sb += col[16 * tt];
        partial_b[(size_t)blockIdx.x * E + e0 + threadIdx.x] = sb;
    }
}

// Pass 2: element i < E*d of dWg, then the E entries of dbg, each the sum of
// its nchunks partials in chunk order (eight loads issued before they are
// added).
__global__ __launch_bounds__(64) void moe_gate_wgrad_reduce_kernel(const float* __restrict__ partial,
                                                                   const float* __restrict__ partial_b, int nchunks,
                                                                   int E, int d, float* __restrict__ dWg,
                                                                   float* __restrict__ dbg)
{
    const size_t i = (size_t)blockIdx.x * 64 + threadIdx.x;
    const size_t n = (size_t)E * d;
    if (i >= n + E)
        return;
    const float* src = i < n ? partial + i : partial_b + (i - n);
    const size_t stride = i < n ? n : (size_t)E;
    float s = 0.0f;
    int ch = 0;
    for (; ch + 8 <= nchunks; ch += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = src[(size_t)(ch + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            s += v[u];
    }
    for (; ch < nchunks; ++ch)
        s += src[(size_t)ch * stride];
    if (i < n)
        dWg[i] = s;
    else
        dbg[i - n] = s;
}

// n floats set to 0 (a kernel, so that a captured graph holds no memset node).
__global__ __launch_bounds__(256) void moe_zero_kernel(float* __restrict__ p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = 0.0f;
}

}  // namespace moe

extern "C" hipError_t moe_launch_zero(float* p, size_t n, hipStream_t stream)
{
    if (n == 0)
        return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    moe::moe_zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(p, n);
    return hipGetLastError();
}

extern "C" hipError_t moe_launch_combine_bwd(int dtype, const void* dy, const void* y_perm, const int32_t* slot,
                                             const float* topk_w, int T, int d, int k, int max_rows, void* d_yp,
                                             float* d_w, hipStream_t stream)
{
    using namespace moe;
    const dim3 grid((T + 3) / 4), block(256);
    if (dtype == 0 && k <= 2)
        moe_combine_bwd_kernel<f32_t, 2><<<grid, block, 0, stream>>>((const float*)dy, (const float*)y_perm, slot,
                                                                     topk_w, T, d, k, max_rows, (float*)d_yp, d_w);
    else if (dtype == 0)
        moe_combine_bwd_kernel<f32_t, 8><<<grid, block, 0, stream>>>((const float*)dy, (const float*)y_perm, slot,
                                                                     topk_w, T, d, k, max_rows, (float*)d_yp, d_w);
    else if (k <= 2)
        moe_combine_bwd_kernel<bf16_t, 2><<<grid, block, 0, stream>>>((const uint16_t*)dy, (const uint16_t*)y_perm,
                                                                      slot, topk_w, T, d, k, max_rows,
                                                                      (uint16_t*)d_yp, d_w);
    else
        moe_combine_bwd_kernel<bf16_t, 8><<<grid, block, 0, stream>>>((const uint16_t*)dy, (const uint16_t*)y_perm,
                                                                      slot, topk_w, T, d, k, max_rows,
                                                                      (uint16_t*)d_yp, d_w);
    return hipGetLastError();
}

extern "C" hipError_t moe_launch_kofs(const int32_t* offsets, int E, int max_rows, int align, int32_t* kofs,
                                      hipStream_t stream)
{
    moe::moe_kofs_kernel<<<1, 1024, 0, stream>>>(offsets, E, max_rows, align, kofs);
    return hipGetLastError();
}

// B matrices of R x C (multiples of 64) -> C x R.
extern "C" hipError_t moe_launch_transpose(int dtype, const void* src, int B, int R, int C, void* dst,
                                           hipStream_t stream)
{
    using namespace moe;
    const dim3 grid(C / 64, R / 64, B), block(256);
    if (dtype == 0)
        moe_transpose_kernel<f32_t><<<grid, block, 0, stream>>>((const float*)src, R, C, (float*)dst);
    else
        moe_transpose_kernel<bf16_t><<<grid, block, 0, stream>>>((const uint16_t*)src, R, C, (uint16_t*)dst);
    return hipGetLastError();
}

// dst [C][ld] from permuted rows of src ([*][C]); ld >= kofs[E], multiple of 64.
extern "C" hipError_t moe_launch_seg_transpose(int dtype, const void* src, const int32_t* gather, int gather_rows,
                                               const int32_t* offsets, const int32_t* kofs, int E, int max_rows,
                                               int C, int ld, void* dst, hipStream_t stream)
{
    using namespace moe;
    if (dtype == 0) {
        const dim3 grid(ld / 64, C / 64), block(256);
        moe_seg_transpose_kernel<f32_t><<<grid, block, 0, stream>>>((const float*)src, gather, gather_rows, offsets,
                                                                    kofs, E, max_rows, C, ld, (float*)dst);
    } else {
        const dim3 grid(ld / 64, (C / 64 + 3) / 4), block(256);
        moe_seg_transpose_bf16_kernel<<<grid, block, 0, stream>>>((const uint16_t*)src, gather, gather_rows, offsets,
                                                                   kofs, E, max_rows, C, ld, (uint16_t*)dst);
    }
    return hipGetLastError();
}

extern "C" hipError_t moe_launch_unpermute_bwd(int dtype, const void* dx_perm, const int32_t* slot, int T, int d,
                                               int k, int max_rows, const float* dz, const void* Wg, int E, void* dx,
                                               hipStream_t stream)
{
    using namespace moe;
    const int per = dtype == 0 ? 4 : 8;  // elements per 16-byte vector
    const int nparts = (d / per + kWave * kUnpVec - 1) / (kWave * kUnpVec);
    const long units = (long)((T + kUnpTok - 1) / kUnpTok) * nparts;
    if (units == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((units + 3) / 4)), block(256);
    if (dtype == 0)
        moe_unpermute_bwd_kernel<f32_t><<<grid, block, 0, stream>>>((const float*)dx_perm, slot, T, d, k, max_rows, dz,
                                                                    (const float*)Wg, E, nparts, (float*)dx);
    else
        moe_unpermute_bwd_kernel<bf16_t><<<grid, block, 0, stream>>>((const uint16_t*)dx_perm, slot, T, d, k,
                                                                     max_rows, dz, (const uint16_t*)Wg, E, nparts,
                                                                     (uint16_t*)dx);
    return hipGetLastError();
}

extern "C" size_t moe_gate_wgrad_partial_bytes(int T, int d, int E)
{
    size_t nch = (size_t)(T + moe::kGateChunk - 1) / moe::kGateChunk;
    if (nch == 0)
        nch = 1;
    return nch * (size_t)E * (d + 1) * sizeof(float);  // [nch][E][d], then [nch][E]
}

extern "C" hipError_t moe_launch_gate_wgrad(int dtype, const float* dz, const void* x, int T, int d, int E,
                                            float* partial, float* dWg, float* dbg, hipStream_t stream)
{
    using namespace moe;
    const int nch = (T + kGateChunk - 1) / kGateChunk;
    float* partial_b = partial + (size_t)nch * E * d;
    const dim3 grid(nch, (d + 255) / 256, (E + 15) / 16), block(256);
    if (dtype == 0)
        moe_gate_wgrad_kernel<f32_t><<<grid, block, 0, stream>>>(dz, (const float*)x, T, d, E, partial, partial_b);
    else
        moe_gate_wgrad_kernel<bf16_t><<<grid, block, 0, stream>>>(dz, (const uint16_t*)x, T, d, E, partial,
                                                                  partial_b);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const size_t n = (size_t)E * d + E;
    moe_gate_wgrad_reduce_kernel<<<dim3((unsigned)((n + 63) / 64)), dim3(64), 0, stream>>>(partial, partial_b, nch, E,
                                                                                           d, dWg, dbg);
    return hipGetLastError();
}
