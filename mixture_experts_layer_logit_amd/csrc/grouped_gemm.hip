// Grouped GEMM over variable-size expert segments (gfx950, MFMA).
//
// The expert FFN of the MoE layer: every expert is a two-layer MLP (FastMoE
// announcement page, "特色三": ReLU experts; many experts on one GPU), run as
// one grouped GEMM over all experts' row segments (Megatron-Core page,
// "关键特性": GroupedGEMM merges the per-expert GEMMs into one kernel).  SwiGLU
// takes the gate and up projections fused in one weight, gate rows first
// (Megatron-Core page, "从HuggingFace到Megatron的权重转换要点").
//
//   up:    C[r, n] = act( sum_k A[r, k] * W[e, n, k] )   A = x_perm, W = W1
//   down:  C[r, n] =      sum_k A[r, k] * W[e, n, k]     A = h,      W = W2
// for every expert e and row r in [offsets[e], offsets[e+1]).  Both operands
// have K contiguous ("X W^T"), fp32 accumulation, output stored in the input
// type.  SwiGLU: C[r, f] = silu(u_f) * u_{F+f}, silu(g) = g / (1 + exp(-g)).
//
// Design (gfx950):
//  * Persistent grid, one block per CU slot.  Each block walks a flattened
//    list of tiles; the per-expert tile counts come from the device offsets
//    (no host round trip), scanned in LDS at kernel start.  Tile order is
//    (expert, n-tile, m-tile) with m fastest, so the tiles sharing a weight
//    panel are consecutive; each round of the persistent loop hands every XCD
//    a contiguous range of that order (blocks are dealt to the 8 XCDs
//    round-robin), so panel re-reads hit that XCD's L2.
//  * Block tile BM x BN, K in 128-byte slices (64 bf16 / 32 fp32), staged
//    global -> registers -> LDS, double-buffered with one barrier per slice.
//    16-byte chunks of each LDS row are XOR-swizzled by (row & 7), so the
//    MFMA operand reads (32 rows, same chunk) hit distinct banks.
//  * MFMA 32x32x16 bf16 (fp32: 32x32x2, four per 16-byte chunk).  The weight
//    tile is the MFMA "A" operand and the activation tile the "B" operand, so
//    each lane's accumulator holds 4 consecutive output columns of one row,
//    stored as one 8-byte (bf16) / 16-byte (fp32) write.
//  * SwiGLU: a wave's N range holds its gate columns then the matching up
//    columns, so gate and up values of one output meet in the same lane.
//  * Rows past a segment's end read a clamped (valid) row and are not stored.
#include "common.h"

namespace moe {

enum { EPI_NONE = 0, EPI_RELU = 1, EPI_SWIGLU = 2 };

constexpr int kGemmMaxE = 1024;
constexpr int kRowBytes = 128;  // bytes of each row in one K slice

template <typename ET, int BM_, int BN_, int WM_, int WN_>
struct GemmShape {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int kBK = kRowBytes / ET::kBytes;
    static constexpr int kPer = 16 / ET::kBytes;  // elements per 16-byte chunk
    static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
    static constexpr int kFM = kWaveM / 32, kFN = kWaveN / 32;
    static constexpr int kLdsA = BM * kRowBytes, kLdsB = BN * kRowBytes;
    static constexpr int kStage = kLdsA + kLdsB;
    static constexpr int kChunksA = BM * 8 / kThreads;
    static constexpr int kChunksB = BN * 8 / kThreads;
    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BM * 8 % kThreads == 0 && BN * 8 % kThreads == 0, "tile load must split evenly");
};

__device__ __forceinline__ uint32_t swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

// Exclusive scan of per-expert tile counts into s_pref[0..E] (s_pref[E] = total).
template <int kThreads>
__device__ void tile_prefix(const int32_t* __restrict__ offsets, int E, int BM, int ntn, int32_t* s_pref,
                            int32_t* s_wsum)
{
    constexpr int kPerThread = (kGemmMaxE + kThreads - 1) / kThreads;
    const int tid = threadIdx.x;
    int vals[kPerThread];
    int local = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int e = tid * kPerThread + i;
        int v = 0;
        if (e < E) {
            const int rows = offsets[e + 1] - offsets[e];
            v = ((rows + BM - 1) / BM) * ntn;
        }
        vals[i] = v;
        local += v;
    }
    const int lane = lane_id(), wave = tid / kWave;
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int n = __shfl_up(incl, o);
        if (lane >= o)
            incl += n;
    }
    if (lane == kWave - 1)
        s_wsum[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w)
        base += s_wsum[w];
    int run = base + incl - local;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        const int e = tid * kPerThread + i;
        if (e < E)
            s_pref[e] = run;
        run += vals[i];
    }
    if (tid == kThreads - 1)
        s_pref[E] = run;
    __syncthreads();
}

template <typename ET, typename S, int EPI>
__global__ __launch_bounds__(S::kThreads) void moe_grouped_gemm_kernel(
    const typename ET::storage* __restrict__ A, const typename ET::storage* __restrict__ W,
    typename ET::storage* __restrict__ C, const int32_t* __restrict__ offsets, int E, int K, int Nw, int Nout,
    int F)
{
    typedef typename ET::storage T;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * S::kStage];
    __shared__ int32_t s_pref[kGemmMaxE + 1];
    __shared__ int32_t s_wsum[S::kThreads / kWave];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int wm = wave / S::WN, wn = wave % S::WN;

    // columns of output per tile; SwiGLU tiles hold gate and up halves
    const int tile_cols = (EPI == EPI_SWIGLU) ? S::BN / 2 : S::BN;
    const int ncols = (EPI == EPI_SWIGLU) ? F : Nout;
    const int ntn = (ncols + tile_cols - 1) / tile_cols;
    tile_prefix<S::kThreads>(offsets, E, S::BM, ntn, s_pref, s_wsum);
    const int total = s_pref[E];
    const int G = gridDim.x;
    const int nk = K / S::kBK;

    for (int base = 0; base < total; base += G) {
        // XCD-aware order: blocks b, b+8, b+16, ... share an XCD.
        const int b = blockIdx.x;
        const int tile = (G % 8 == 0) ? base + (b % 8) * (G / 8) + b / 8 : base + b;
        if (tile >= total)
            continue;
        int lo = 0, hi = E;  // largest e with s_pref[e] <= tile
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_pref[mid] <= tile)
                lo = mid;
            else
                hi = mid;
        }
        const int e = lo;
        const int seg0 = offsets[e];
        const int seg_rows = offsets[e + 1] - seg0;
        const int mt_e = (seg_rows + S::BM - 1) / S::BM;
        const int local = tile - s_pref[e];
        const int nt = local / mt_e;
        const int mt = local % mt_e;
        const int row0 = seg0 + mt * S::BM;
        const int rows = min(S::BM, seg_rows - mt * S::BM);
        const int n0 = nt * tile_cols;

        // global source offsets of this thread's chunks
        size_t a_off[S::kChunksA];
        size_t b_off[S::kChunksB];
        uint32_t a_lds[S::kChunksA], b_lds[S::kChunksB];
#pragma unroll
        for (int i = 0; i < S::kChunksA; ++i) {
            const int q = tid + S::kThreads * i;
            const int r = q >> 3, c = q & 7;
            const int gr = row0 + min(r, rows - 1);
            a_off[i] = (size_t)gr * K + c * S::kPer;
            a_lds[i] = swz(r, c);
        }
        const size_t w_base = (size_t)e * Nw * K;
#pragma unroll
        for (int i = 0; i < S::kChunksB; ++i) {
            const int q = tid + S::kThreads * i;
            const int r = q >> 3, c = q & 7;
            int wrow;
            if (EPI == EPI_SWIGLU) {
                const int wblk = r / S::kWaveN, rr = r % S::kWaveN;
                const int half = rr / (S::kWaveN / 2);
                const int hc = min(n0 + wblk * (S::kWaveN / 2) + rr % (S::kWaveN / 2), F - 1);
                wrow = half ? F + hc : hc;
            } else {
                wrow = min(n0 + r, Nw - 1);
            }
            b_off[i] = w_base + (size_t)wrow * K + c * S::kPer;
            b_lds[i] = S::kLdsA + swz(r, c);
        }

        f32x16 acc[S::kFM][S::kFN];
#pragma unroll
        for (int i = 0; i < S::kFM; ++i)
#pragma unroll
            for (int j = 0; j < S::kFN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[i][j][v] = 0.0f;

        uint4 ra[S::kChunksA], rb[S::kChunksB];
        // prologue: slice 0 -> buffer 0
#pragma unroll
        for (int i = 0; i < S::kChunksA; ++i)
            ra[i] = *reinterpret_cast<const uint4*>(A + a_off[i]);
#pragma unroll
        for (int i = 0; i < S::kChunksB; ++i)
            rb[i] = *reinterpret_cast<const uint4*>(W + b_off[i]);
        __syncthreads();  // previous tile's readers of buffer 0 are done
#pragma unroll
        for (int i = 0; i < S::kChunksA; ++i)
            *reinterpret_cast<uint4*>(lds + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < S::kChunksB; ++i)
            *reinterpret_cast<uint4*>(lds + b_lds[i]) = rb[i];
        __syncthreads();

        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) {
                const size_t koff = (size_t)(kt + 1) * S::kBK;
#pragma unroll
                for (int i = 0; i < S::kChunksA; ++i)
                    ra[i] = *reinterpret_cast<const uint4*>(A + a_off[i] + koff);
#pragma unroll
                for (int i = 0; i < S::kChunksB; ++i)
                    rb[i] = *reinterpret_cast<const uint4*>(W + b_off[i] + koff);
            }
            const uint8_t* bufA = lds + cur * S::kStage;
            const uint8_t* bufB = bufA + S::kLdsA;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int c = 2 * kk + (lane >> 5);
                uint4 fa[S::kFN], fb[S::kFM];
#pragma unroll
                for (int j = 0; j < S::kFN; ++j)
                    fa[j] = *reinterpret_cast<const uint4*>(bufB + swz(wn * S::kWaveN + j * 32 + (lane & 31), c));
#pragma unroll
                for (int i = 0; i < S::kFM; ++i)
                    fb[i] = *reinterpret_cast<const uint4*>(bufA + swz(wm * S::kWaveM + i * 32 + (lane & 31), c));
#pragma unroll
                for (int i = 0; i < S::kFM; ++i)
#pragma unroll
                    for (int j = 0; j < S::kFN; ++j) {
                        if constexpr (ET::kBytes == 2) {
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                __builtin_bit_cast(bf16x8, fa[j]), __builtin_bit_cast(bf16x8, fb[i]), acc[i][j], 0,
                                0, 0);
                        } else {
                            const f32x4 va = __builtin_bit_cast(f32x4, fa[j]);
                            const f32x4 vb = __builtin_bit_cast(f32x4, fb[i]);
#pragma unroll
                            for (int s = 0; s < 4; ++s)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[s], vb[s], acc[i][j], 0, 0, 0);
                        }
                    }
            }
            if (kt + 1 < nk) {
                uint8_t* nxt = lds + (cur ^ 1) * S::kStage;
#pragma unroll
                for (int i = 0; i < S::kChunksA; ++i)
                    *reinterpret_cast<uint4*>(nxt + a_lds[i]) = ra[i];
#pragma unroll
                for (int i = 0; i < S::kChunksB; ++i)
                    *reinterpret_cast<uint4*>(nxt + b_lds[i]) = rb[i];
            }
            __syncthreads();
        }

        // epilogue: lane holds rows m = .. + (lane & 31), 4 consecutive columns per group
#pragma unroll
        for (int i = 0; i < S::kFM; ++i) {
            const int m = wm * S::kWaveM + i * 32 + (lane & 31);
            if (m >= rows)
                continue;
            T* crow = C + (size_t)(row0 + m) * Nout;
            constexpr int kJ = (EPI == EPI_SWIGLU) ? S::kFN / 2 : S::kFN;
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = j * 32 + 8 * g + 4 * (lane >> 5);
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float u = acc[i][j][4 * g + q];
                        if (EPI == EPI_RELU)
                            u = fmaxf(u, 0.0f);
                        if (EPI == EPI_SWIGLU) {
                            const float up = acc[i][j + S::kFN / 2][4 * g + q];
                            u = u / (1.0f + __expf(-u)) * up;
                        }
                        v[q] = u;
                    }
                    const int n = n0 + ((EPI == EPI_SWIGLU) ? wn * (S::kWaveN / 2) : wn * S::kWaveN) + nl;
                    if (n < ncols) {
                        if constexpr (ET::kBytes == 2) {
                            uint2 o;
                            o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                            o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                            *reinterpret_cast<uint2*>(crow + n) = o;
                        } else {
                            *reinterpret_cast<float4*>(crow + n) = make_float4(v[0], v[1], v[2], v[3]);
                        }
                    }
                }
            }
        }
    }
}

}  // namespace moe

namespace {
using namespace moe;

template <typename ET, typename S, int EPI>
hipError_t launch_one(const void* A, const void* W, void* C, const int32_t* offsets, int E, int K, int Nw, int Nout,
                      int F, int max_rows, int ncu, hipStream_t stream)
{
    typedef typename ET::storage T;
    const int tile_cols = (EPI == EPI_SWIGLU) ? S::BN / 2 : S::BN;
    const int ncols = (EPI == EPI_SWIGLU) ? F : Nout;
    const long long ntn = (ncols + tile_cols - 1) / tile_cols;
    // upper bound on m-tiles: floor(P/BM) full tiles plus one partial per expert
    const long long mt_max = max_rows / S::BM + (long long)(E < max_rows ? E : max_rows);
    long long tiles_max = mt_max * ntn;
    long long grid = ncu;  // one block per CU (LDS-limited)
    if (tiles_max < grid)
        grid = (tiles_max + 7) / 8 * 8;
    if (grid < 1)
        grid = 1;
    moe_grouped_gemm_kernel<ET, S, EPI><<<dim3((unsigned)grid), dim3(S::kThreads), 0, stream>>>(
        (const T*)A, (const T*)W, (T*)C, offsets, E, K, Nw, Nout, F);
    return hipGetLastError();
}

template <typename ET, typename S>
hipError_t launch_epi(int epi, const void* A, const void* W, void* C, const int32_t* offsets, int E, int K, int Nw,
                      int Nout, int F, int max_rows, int ncu, hipStream_t stream)
{
    if (epi == EPI_RELU)
        return launch_one<ET, S, EPI_RELU>(A, W, C, offsets, E, K, Nw, Nout, F, max_rows, ncu, stream);
    if (epi == EPI_SWIGLU)
        return launch_one<ET, S, EPI_SWIGLU>(A, W, C, offsets, E, K, Nw, Nout, F, max_rows, ncu, stream);
    return launch_one<ET, S, EPI_NONE>(A, W, C, offsets, E, K, Nw, Nout, F, max_rows, ncu, stream);
}
}  // namespace

// epi: 0 none, 1 ReLU, 2 SwiGLU.  Nw = weight rows per expert, Nout = output
// row stride (= output columns).  max_rows bounds offsets[E].
extern "C" hipError_t moe_launch_grouped_gemm(int dtype, int epi, const void* A, const void* W, void* C,
                                              const int32_t* offsets, int E, int K, int Nw, int Nout, int F,
                                              int max_rows, int ncu, hipStream_t stream)
{
    if (dtype == 0)
        return launch_epi<f32_t, GemmShape<f32_t, 128, 128, 2, 2>>(epi, A, W, C, offsets, E, K, Nw, Nout, F,
                                                                   max_rows, ncu, stream);
    return launch_epi<bf16_t, GemmShape<bf16_t, 256, 256, 2, 2>>(epi, A, W, C, offsets, E, K, Nw, Nout, F, max_rows,
                                                                 ncu, stream);
}
