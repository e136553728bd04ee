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
//  * Block tile BM x BN, K in 128-byte slices (64 bf16 / 32 fp32), loaded
//    straight from memory into LDS (buffer_load ... lds: no staging
//    registers), double-buffered with one barrier per slice.  Each wave load
//    fills a contiguous 1 KB LDS block (8 rows); the 16-byte chunks of an LDS
//    row are XOR-swizzled by (row & 7) -- applied on the source side, by
//    choosing which chunk each lane fetches -- so the MFMA operand reads
//    (32 rows, same chunk) hit distinct banks.
//  * Buffer resources give 32-bit offsets from scalar bases: one over the
//    tile's activation rows, whose end is the segment end (rows past it read
//    zero), one over the expert's weight matrix.
//  * MFMA 32x32x16 bf16 (fp32: 32x32x2, four per 16-byte chunk).  The weight
//    tile is the MFMA "A" operand and the activation tile the "B" operand, so
//    each lane's accumulator holds 4 consecutive output columns of one row,
//    stored as one 8-byte (bf16) / 16-byte (fp32) write.
//  * SwiGLU: a wave's N range holds its gate columns then the matching up
//    columns, so gate and up values of one output meet in the same lane.
//  * Rows past a segment's end are computed on zeros and not stored.
#include "common.h"

namespace moe {

enum { EPI_NONE = 0, EPI_RELU = 1, EPI_SWIGLU = 2 };

constexpr int kGemmMaxE = 1024;
#ifndef MOE_XCD_REMAP
#define MOE_XCD_REMAP 1
#endif

// Tile geometry.  BM x BN output tile per block, WM x WN waves; each K slice
// is RB bytes of every tile row (64 or 128), staged through S LDS buffers;
// OCC = blocks per CU the kernel is built for; GM = m-tiles grouped together
// in the tile order.
template <typename ET, int BM_, int BN_, int WM_, int WN_, int RB_, int S_, int OCC_, int GM_>
struct GemmShape {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, RB = RB_, S = S_, OCC = OCC_, GM = GM_;
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int kWaves = WM * WN;
    static constexpr int kBK = RB / ET::kBytes;          // K elements per slice
    static constexpr int kPer = 16 / ET::kBytes;         // elements per 16-byte chunk
    static constexpr int kNch = RB / 16;                 // 16-byte chunks per row
    static constexpr int kRowsPerBlk = 1024 / RB;        // rows per 1 KB DMA block
    static constexpr int kSwzShift = (RB == 128) ? 1 : 2; // log2(256 / RB): rows per 256-byte bank cycle
    static constexpr int kKSteps = RB / 32;              // MFMA k-steps per slice
    static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
    static constexpr int kFM = kWaveM / 32, kFN = kWaveN / 32;
    static constexpr int kLdsA = BM * RB, kLdsB = BN * RB;
    static constexpr int kStage = kLdsA + kLdsB;
    static constexpr int kBlkA = BM / kRowsPerBlk / kWaves;  // DMA blocks per wave per slice
    static constexpr int kBlkB = BN / kRowsPerBlk / kWaves;
    static constexpr int kLoads = kBlkA + kBlkB;
    static_assert(RB == 64 || RB == 128, "slice rows are 64 or 128 bytes");
    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BM % (kRowsPerBlk * kWaves) == 0 && BN % (kRowsPerBlk * kWaves) == 0,
                  "DMA blocks must split evenly across waves");
    static_assert(S >= 2 && S <= 4, "2 to 4 stages");
    static_assert((S - 2) * kLoads <= 63, "vmcnt range");
};

// LDS byte offset of 16-byte chunk `c` of tile row `row` for RB-byte rows.
// gfx950's LDS has 64 banks (256 bytes per clock) and serves 16 lanes of a
// 16-byte read per clock.  256/RB consecutive rows fill the 64 banks once, so
// rows 256/RB apart share banks; XOR-ing the chunk index with
// (row / (256/RB)) mod (chunks per row) gives the rows of any 16-row group
// that share banks distinct chunk slots, so reading one chunk of 16
// consecutive rows touches all 64 banks once.
template <typename S>
__device__ __forceinline__ uint32_t swz(int row, int c)
{
    return row * S::RB + ((c ^ ((row >> S::kSwzShift) & (S::kNch - 1))) << 4);
}

// Rows of expert e, with the offsets clamped into [0, max_rows] and made
// non-decreasing, so that no offsets array can send a tile out of bounds.
__device__ __forceinline__ void seg_bounds(const int32_t* __restrict__ offsets, int e, int max_rows, int& lo,
                                           int& rows)
{
    lo = min(max(offsets[e], 0), max_rows);
    const int hi = min(max(offsets[e + 1], lo), max_rows);
    rows = hi - lo;
}

// Exclusive scan of per-expert tile counts into s_pref[0..E] (s_pref[E] = total).
template <int kThreads>
__device__ void tile_prefix(const int32_t* __restrict__ offsets, int E, int max_rows, int BM, int ntn,
                            int32_t* s_pref, int32_t* s_wsum)
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
            int lo, rows;
            seg_bounds(offsets, e, max_rows, lo, rows);
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

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));  // stride 0: raw buffer
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);                 // num_records, in bytes
    r[3] = 0x00020000;                                                 // gfx9 raw-buffer descriptor word 3
    return r;
}

// 16 bytes per lane from buffer `rsrc` at voff + soff straight into LDS at
// lds + 16 * lane (buffer_load_dwordx4 ... lds; M0 holds the LDS base).
// Issued from asm so that the compiler does not track the LDS writes: they
// are ordered by the kernel's own vmcnt waits and barriers (the compiler
// would otherwise make every LDS read wait for all loads in flight).  The
// instruction has no destination register; its address operands are read at
// issue.
__device__ __forceinline__ void dma16(const i32x4& rsrc, const uint8_t* lds, uint32_t voff, uint32_t soff)
{
    // scalar operands: wave-uniform by construction; readfirstlane makes the
    // compiler place them in SGPRs (and keeps the offset off the immediate field)
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
    uint32_t so = __builtin_amdgcn_readfirstlane(soff);
    __asm__("" : "+s"(so));
    __asm__ volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "s"(m0), "v"(voff), "s"(rsrc), "s"(so)
                     : "memory");
}

// Workgroup barrier for the K loop.  __syncthreads() (and any workgroup
// fence that covers LDS) waits for every outstanding load, DMA loads into LDS
// included, which would drain the load pipeline at each K slice.  Here the
// ordering is explicit instead: before the barrier each wave waits (vmcnt)
// for its own loads of the slice about to be read and (lgkmcnt) for its own
// LDS reads of the slice about to be overwritten; the asm statement's memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt((0x3f & 0xf) | ((0x3f >> 4) << 14) | (0x7 << 4) | (0 << 8));  // lgkmcnt(0)
    __asm__ volatile("s_barrier" ::: "memory");
}

// s_waitcnt with vmcnt(n) and no wait on the other counters (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

template <typename ET, typename S, int EPI>
__global__ __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(S::OCC, S::OCC)))
void moe_grouped_gemm_kernel(const typename ET::storage* __restrict__ A, const typename ET::storage* __restrict__ W,
                             typename ET::storage* __restrict__ C, const int32_t* __restrict__ offsets, int E,
                             int K, int Nw, int Nout, int F, int max_rows)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses device-only types; the host pass needs the stub only
    typedef typename ET::storage T;
    constexpr int kWaves = S::kWaves;
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[S::kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[S::kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[S::S > 2 ? S::kStage : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[S::S > 3 ? S::kStage : 16];
    __shared__ int32_t s_pref[kGemmMaxE + 1];
    __shared__ int32_t s_wsum[kWaves];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid / kWave;
    const int wm = wave / S::WN, wn = wave % S::WN;
    const uint32_t rowK = (uint32_t)K * ET::kBytes;  // bytes of one row
    // lane's place inside a 1 KB DMA block of rows [R0, R0 + 1024/RB): row
    // R0 + lane / kNch, physical chunk lane % kNch, which holds the logical
    // chunk of swz().  The swizzle term depends on the block only through the
    // parity of its index for 128-byte rows; a wave's blocks are
    // wave + kWaves*i, whose parity is the wave's (kWaves is even).
    static_assert(kWaves % 2 == 0, "block parity must be fixed per wave");
    const int lrow = lane / S::kNch, lphys = lane % S::kNch;
    const int blk_row0 = (S::RB == 128) ? 8 * (wave & 1) : 0;  // R0 mod (2 * 256 / RB) that matters
    const int lchunk = lphys ^ (((blk_row0 + lrow) >> S::kSwzShift) & (S::kNch - 1));
    const uint32_t lane_off = (uint32_t)lrow * rowK + (uint32_t)(lchunk << 4);

    const int tile_cols = (EPI == EPI_SWIGLU) ? S::BN / 2 : S::BN;
    const int ncols = (EPI == EPI_SWIGLU) ? F : Nout;
    const int ntn = (ncols + tile_cols - 1) / tile_cols;
    tile_prefix<S::kThreads>(offsets, E, max_rows, S::BM, ntn, s_pref, s_wsum);
    const int total = s_pref[E];
    const int G = gridDim.x;
    const int nk = K / S::kBK;

    for (int base = 0; base < total; base += G) {
        // XCD-aware order: blocks b, b+8, b+16, ... share an XCD.
        const int b = blockIdx.x;
        const int tile = (MOE_XCD_REMAP && G % 8 == 0) ? base + (b % 8) * (G / 8) + b / 8 : base + b;
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
        int seg0, seg_rows;
        seg_bounds(offsets, e, max_rows, seg0, seg_rows);
        const int mt_e = (seg_rows + S::BM - 1) / S::BM;
        // (m-group, n-tile, m-tile within group) order: groups of GM m-tiles
        // sweep all n-tiles together, so GM activation tiles and a run of
        // weight panels are live on an XCD at once
        const int local = tile - s_pref[e];
        const int g = local / (S::GM * ntn);
        const int within = local - g * S::GM * ntn;
        const int gs = min(S::GM, mt_e - g * S::GM);
        const int nt = within / gs;
        const int mt = g * S::GM + within % gs;
        const int row0 = seg0 + mt * S::BM;
        const int rows = min(S::BM, seg_rows - mt * S::BM);
        const int n0 = nt * tile_cols;

        // activation rows [row0, row0 + rows): rows past the segment read 0
        const i32x4 rsA = make_rsrc(A + (size_t)row0 * K, (uint32_t)rows * rowK);
        // this expert's weight matrix: rows past Nw read 0
        const i32x4 rsW = make_rsrc(W + (size_t)e * Nw * K, (uint32_t)Nw * rowK);
        uint32_t voffA[S::kBlkA], voffB[S::kBlkB];
#pragma unroll
        for (int i = 0; i < S::kBlkA; ++i)
            voffA[i] = (uint32_t)(S::kRowsPerBlk * (wave + kWaves * i)) * rowK + lane_off;
#pragma unroll
        for (int i = 0; i < S::kBlkB; ++i) {
            const int r = S::kRowsPerBlk * (wave + kWaves * i);  // first LDS row of the block
            int wrow;
            if (EPI == EPI_SWIGLU) {
                const int wblk = r / S::kWaveN, rr = r % S::kWaveN;
                const int half = rr / (S::kWaveN / 2);
                const int hc = n0 + wblk * (S::kWaveN / 2) + rr % (S::kWaveN / 2);
                wrow = half ? F + hc : (hc < F ? hc : Nw);  // gate rows past F read 0
            } else {
                wrow = n0 + r;
            }
            voffB[i] = (uint32_t)wrow * rowK + lane_off;
        }

        auto issue = [&](int kt, uint8_t* dst) {
            const uint32_t soff = (uint32_t)kt * S::RB;
#pragma unroll
            for (int i = 0; i < S::kBlkA; ++i)
                dma16(rsA, dst + (wave + kWaves * i) * 1024, voffA[i], soff);
#pragma unroll
            for (int i = 0; i < S::kBlkB; ++i)
                dma16(rsW, dst + S::kLdsA + (wave + kWaves * i) * 1024, voffB[i], soff);
        };

        f32x16 acc[S::kFM][S::kFN];
#pragma unroll
        for (int i = 0; i < S::kFM; ++i)
#pragma unroll
            for (int j = 0; j < S::kFN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc[i][j][v] = 0.0f;

        // Wait until at most n slices of this wave's loads are in flight.
        auto wait_slices = [&](int n) {
            if (S::S >= 4 && n >= 2)
                wait_vmcnt<(S::S >= 4 ? 2 : 0) * S::kLoads>();
            else if (S::S >= 3 && n >= 1)
                wait_vmcnt<(S::S >= 3 ? 1 : 0) * S::kLoads>();
            else
                wait_vmcnt<0>();
        };

        // One K slice kt held in `cur`: wait for it (later slices may stay in
        // flight), meet the other waves (they have finished slice kt-1, so its
        // buffer `nxt` is free), start loading slice kt+S-1 into `nxt`, then
        // multiply.  Buffers are distinct LDS arrays known at compile time, so
        // reads of `cur` never wait for the loads into `nxt`.
        auto slice = [&](int kt, const uint8_t* cur, uint8_t* nxt) {
            wait_slices(min(S::S - 2, nk - 1 - kt));
            lds_barrier();
            if (kt + S::S - 1 < nk)
                issue(kt + S::S - 1, nxt);
            const uint8_t* bufA = cur;
            const uint8_t* bufB = cur + S::kLdsA;
#pragma unroll
            for (int kk = 0; kk < S::kKSteps; ++kk) {
                const int c = 2 * kk + (lane >> 5);
                uint4 fa[S::kFN], fb[S::kFM];
#pragma unroll
                for (int j = 0; j < S::kFN; ++j)
                    fa[j] = *reinterpret_cast<const uint4*>(bufB +
                                                            swz<S>(wn * S::kWaveN + j * 32 + (lane & 31), c));
#pragma unroll
                for (int i = 0; i < S::kFM; ++i)
                    fb[i] = *reinterpret_cast<const uint4*>(bufA +
                                                            swz<S>(wm * S::kWaveM + i * 32 + (lane & 31), c));
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
                            for (int q = 0; q < 4; ++q)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[q], vb[q], acc[i][j], 0, 0, 0);
                        }
                    }
            }
        };

        wait_vmcnt<0>();  // the previous tile's stores are out of the vmcnt count
        __syncthreads();  // every wave is done with the previous tile's buffers
#pragma unroll
        for (int s0 = 0; s0 < S::S - 1; ++s0) {
            if (s0 < nk)
                issue(s0, s0 == 0 ? lds0 : s0 == 1 ? lds1 : lds2);
        }
        int kt = 0;
        if constexpr (S::S == 2) {
            for (; kt + 2 <= nk; kt += 2) {
                slice(kt, lds0, lds1);
                slice(kt + 1, lds1, lds0);
            }
            if (kt < nk)
                slice(kt, lds0, lds1);
        } else if constexpr (S::S == 3) {
            for (; kt + 3 <= nk; kt += 3) {
                slice(kt, lds0, lds2);
                slice(kt + 1, lds1, lds0);
                slice(kt + 2, lds2, lds1);
            }
            if (kt < nk)
                slice(kt, lds0, lds2);
            if (kt + 1 < nk)
                slice(kt + 1, lds1, lds0);
        } else {
            for (; kt + 4 <= nk; kt += 4) {
                slice(kt, lds0, lds3);
                slice(kt + 1, lds1, lds0);
                slice(kt + 2, lds2, lds1);
                slice(kt + 3, lds3, lds2);
            }
            if (kt < nk)
                slice(kt, lds0, lds3);
            if (kt + 1 < nk)
                slice(kt + 1, lds1, lds0);
            if (kt + 2 < nk)
                slice(kt + 2, lds2, lds1);
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
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int nl = j * 32 + 8 * g4 + 4 * (lane >> 5);
                    float v[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float u = acc[i][j][4 * g4 + q];
                        if (EPI == EPI_RELU)
                            u = fmaxf(u, 0.0f);
                        if (EPI == EPI_SWIGLU) {
                            const float up = acc[i][j + S::kFN / 2][4 * g4 + q];
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
#endif
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
    long long grid = (long long)ncu * S::OCC;  // persistent: as many blocks as are resident at once
    if (tiles_max < grid)
        grid = (tiles_max + 7) / 8 * 8;
    if (grid < 1)
        grid = 1;
    moe_grouped_gemm_kernel<ET, S, EPI><<<dim3((unsigned)grid), dim3(S::kThreads), 0, stream>>>(
        (const T*)A, (const T*)W, (T*)C, offsets, E, K, Nw, Nout, F, max_rows);
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

// bf16 tile configurations (BM, BN, WM, WN, slice bytes, stages, blocks per
// CU, m-tile group), picked from the mean rows per expert, which the host
// knows without reading the device-side offsets:
//   large   >= 512 rows per expert: 256 x 256 tiles, 8 waves (2 per SIMD, 128 x
//           64 each), the densest tile that fits the register file; 2 x 64 KB
//           of LDS stages
//   medium  128..511 rows: 128 x 128 tiles, 4 waves, 2 blocks per CU
//   small   < 128 rows: 64 x 256 tiles, 4 waves (short
//           segments, so tall tiles would mostly compute padding)
#ifndef MOE_LARGE_TILE
#define MOE_LARGE_TILE 256, 256, 2, 4, 128, 2, 1, 8
#endif
#ifndef MOE_MEDIUM_TILE
#define MOE_MEDIUM_TILE 128, 128, 2, 2, 128, 2, 2, 4
#endif
#ifndef MOE_SMALL_TILE
#define MOE_SMALL_TILE 64, 256, 1, 4, 128, 2, 1, 4
#endif

// epi: 0 none, 1 ReLU, 2 SwiGLU.  Nw = weight rows per expert, Nout = output
// row stride (= output columns).  max_rows bounds offsets[E]; mean_rows is the
// expected rows per expert (selects the tile configuration).
extern "C" hipError_t moe_launch_grouped_gemm(int dtype, int epi, const void* A, const void* W, void* C,
                                              const int32_t* offsets, int E, int K, int Nw, int Nout, int F,
                                              int max_rows, int mean_rows, int ncu, hipStream_t stream)
{
    if (dtype == 0)
        return launch_epi<f32_t, GemmShape<f32_t, 128, 128, 2, 2, 128, 2, 1, 4>>(epi, A, W, C, offsets, E, K, Nw,
                                                                                 Nout, F, max_rows, ncu, stream);
    if (mean_rows >= 512)
        return launch_epi<bf16_t, GemmShape<bf16_t, MOE_LARGE_TILE>>(epi, A, W, C, offsets, E, K, Nw, Nout, F,
                                                                      max_rows, ncu, stream);
    if (mean_rows >= 128)
        return launch_epi<bf16_t, GemmShape<bf16_t, MOE_MEDIUM_TILE>>(epi, A, W, C, offsets, E, K, Nw, Nout, F,
                                                                       max_rows, ncu, stream);
    return launch_epi<bf16_t, GemmShape<bf16_t, MOE_SMALL_TILE>>(epi, A, W, C, offsets, E, K, Nw, Nout, F,
                                                                  max_rows, ncu, stream);
}
