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
// for every expert e and row r in [offsets[e], offsets[e+1]) (or, without
// offsets, one weight matrix over all rows: the shared expert).  Both operands
// have K contiguous ("X W^T"), fp32 accumulation, output stored in the input
// type.  SwiGLU: C[r, f] = silu(u_f) * u_{F+f}, silu(g) = g / (1 + exp(-g)).
// With a gather index, A row r is read from row gather[r] of A (the up
// projection reads the token rows of x directly, so the permuted copy x_perm
// need not be written and read back).
//
// FP8 experts: A and W hold OCP E4M3 codes, each A row and each W row with a
// power-of-two scale; the MFMA multiplies the codes (32x32x64 f8f6f4, twice
// the bf16 rate) and the epilogue applies a_scale[row] * w_scale[e][col]
// before the activation; the output is bf16.
//
// Design (gfx950):
//  * Persistent grid, one block per resident slot.  The per-expert tile
//    counts come from the device offsets (no host round trip), scanned in
//    LDS at kernel start.  Tile order is (expert, group of GM m-tiles,
//    n-tile, m-tile); each round of the persistent loop hands every XCD a
//    contiguous run of that order (blocks are dealt to the 8 XCDs
//    round-robin), so the XCD's concurrent tiles share GM activation tiles
//    and a run of weight panels in its L2.
//  * Tail split: the tiles left after the last full round of the grid are
//    split along K into up to 4 parts that fill that round; their fp32
//    partial tiles go to a workspace and a second kernel adds the parts in a
//    fixed order and applies the epilogue (deterministic, no atomics).
//  * Block tile BM x BN, K in 128-byte slices (64 bf16 / 32 fp32), loaded
//    straight from memory into LDS (buffer_load ... lds: no staging
//    registers) through a ring of S LDS stages, one barrier per slice.  Each wave load
//    fills a contiguous 1 KB LDS block (8 rows); the 16-byte chunks of an LDS
//    row are XOR-swizzled (see swz) by choosing which chunk each lane fetches,
//    so the MFMA operand reads hit every LDS bank once.
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
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace moe {

// Epilogues: none; forward activations (ReLU, SwiGLU); backward of the
// activation applied to the incoming gradient dh (the tile computes dh and the
// epilogue turns it into du with the saved pre-activation u).
enum { EPI_NONE = 0, EPI_RELU = 1, EPI_SWIGLU = 2, EPI_DRELU = 3, EPI_DSWIGLU = 4 };

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kGemmMaxE = 1024;
constexpr int kMaxSplit = 4;         // K parts of a tail tile
constexpr int kSplitSlots = 256;     // partial tiles the workspace holds
constexpr int kMinSplitSlices = 8;   // split only tiles with at least this many K slices

// Tile geometry.  BM x BN output tile per block, WM x WN waves; each K slice
// is RB bytes of every tile row, staged through S LDS buffers; OCC = blocks
// per CU the kernel is built for; GM = m-tiles grouped together in the tile
// order.
template <typename ET, int BM_, int BN_, int WM_, int WN_, int RB_, int S_, int OCC_, int GM_>
struct GemmShape {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, RB = RB_, S = S_, OCC = OCC_, GM = GM_;
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int kWaves = WM * WN;
    // waves each SIMD holds with OCC blocks resident (the compiler's
    // register budget): 4 SIMDs per CU
    static constexpr int kWavesPerSimd = OCC * kWaves / 4;
    static constexpr int kBK = RB / ET::kBytes;           // K elements per slice
    static constexpr int kNch = RB / 16;                  // 16-byte chunks per row
    static constexpr int kRowsPerBlk = 1024 / RB;         // rows per 1 KB DMA block
    static constexpr int kSwzShift = (RB == 128) ? 1 : 2;  // log2(256 / RB)
    // bytes of a row one MFMA k-step consumes: 32 (bf16 32x32x16, fp32 4 x
    // 32x32x2), 64 (fp8 32x32x64); a lane holds kChunks 16-byte chunks of it
    static constexpr int kStepBytes = ET::kBytes == 1 ? 64 : 32;
    static constexpr int kChunks = kStepBytes / 32;
    static constexpr int kKSteps = RB / kStepBytes;       // MFMA k-steps per slice
    // one lane's share of an operand block for one k-step (kept as one
    // register tuple, the MFMA's operand)
    typedef typename std::conditional<ET::kBytes == 1, i32x8, i32x4>::type frag_t;
    static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
    static constexpr int kFM = kWaveM / 32, kFN = kWaveN / 32;
    static constexpr int kLdsA = BM * RB, kLdsB = BN * RB;
    static constexpr int kStage = kLdsA + kLdsB;
    static constexpr int kBlkA = BM / kRowsPerBlk / kWaves;  // DMA blocks per wave per slice
    static constexpr int kBlkB = BN / kRowsPerBlk / kWaves;
    static constexpr int kLoads = kBlkA + kBlkB;
    static constexpr int kTileFloats = BM * BN;          // one partial tile
    static_assert(RB == 64 || RB == 128, "slice rows are 64 or 128 bytes");
    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BM % (kRowsPerBlk * kWaves) == 0 && BN % (kRowsPerBlk * kWaves) == 0,
                  "DMA blocks must split evenly across waves");
    static_assert(S >= 2 && S <= 4, "2 to 4 stages");
    static_assert((S - 1) * kLoads <= 63, "vmcnt range");
    static_assert(kWaves % 2 == 0, "block parity must be fixed per wave");
    static_assert(kWavesPerSimd >= 1 && (OCC * kWaves) % 4 == 0, "whole waves per SIMD");
};

// LDS byte offset of 16-byte chunk `c` of tile row `row` for RB-byte rows.
// gfx950's LDS has 64 banks (256 bytes per clock) and serves 16 lanes of a
// 16-byte read per clock.  256/RB consecutive rows fill the 64 banks once, so
// rows 256/RB apart share banks; XOR-ing the chunk index with
// (row / (256/RB)) mod (chunks per row) gives the rows of any 16-row group
// that share banks distinct chunk slots, so reading one chunk of 16
// consecutive rows touches all 64 banks once.
// Swizzle term of row `row` of a transposed (WT) weight slice: the 32-byte
// column block b is stored at b ^ wt_f(row).  One transpose read touches
// rows k0 + {0..3, 8..11} (or + 4) in two adjacent blocks; wt_f takes the 8
// distinct values 0..7 there, so the 16 row segments fall 2 per 8-bank group
// (the minimum for 512 bytes on 64 banks).
__device__ __forceinline__ int wt_f(int row)
{
    return ((row & 3) << 1) | ((row >> 3) & 1);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b16 at an LDS location reached through a generic pointer
// into a __shared__ array.
__device__ __forceinline__ v4i16 ds_read_tr16(const uint8_t* p)
{
    typedef __attribute__((address_space(3))) v4i16* lds_v4_t;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_t)(__attribute__((address_space(3))) void*)p);
}

template <typename S>
__device__ __forceinline__ uint32_t swz(int row, int c)
{
    return row * S::RB + ((c ^ ((row >> S::kSwzShift) & (S::kNch - 1))) << 4);
}

// Rows of expert e, with the offsets clamped into [0, max_rows] and made
// non-decreasing, so that no offsets array can send a tile out of bounds.
// offsets == NULL: one segment of all max_rows rows (a dense layer, E = 1).
__device__ __forceinline__ void seg_bounds(const int32_t* __restrict__ offsets, int e, int max_rows, int& lo,
                                           int& rows)
{
    if (offsets == nullptr) {
        lo = 0;
        rows = max_rows;
        return;
    }
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

// One output tile: expert, first row and row count, first output column.
struct TileDec {
    int e, row0, rows, n0;
};

template <typename S>
__device__ __forceinline__ TileDec decode_tile(int tile, const int32_t* s_pref, const int32_t* __restrict__ offsets,
                                               int E, int max_rows, int ntn, int tile_cols)
{
    int lo = 0, hi = E;  // largest e with s_pref[e] <= tile
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= tile)
            lo = mid;
        else
            hi = mid;
    }
    TileDec t;
    t.e = lo;
    int seg0, seg_rows;
    seg_bounds(offsets, t.e, max_rows, seg0, seg_rows);
    const int mt_e = (seg_rows + S::BM - 1) / S::BM;
    // (m-group, n-tile, m-tile within group) order inside the expert
    const int local = tile - s_pref[t.e];
    const int g = local / (S::GM * ntn);
    const int within = local - g * S::GM * ntn;
    const int gs = min(S::GM, mt_e - g * S::GM);
    const int nt = within / gs;
    const int mt = g * S::GM + within % gs;
    t.row0 = seg0 + mt * S::BM;
    t.rows = min(S::BM, seg_rows - mt * S::BM);
    t.n0 = nt * tile_cols;
    return t;
}

// K parts of each tail tile: the tiles after the last full round of G blocks
// are split so that the last round is filled (at most kSplitSlots partials,
// each part at least kMinSplitSlices / 2 slices long).
__device__ __forceinline__ int split_parts(int total, int G, int nk, bool enabled)
{
    const int tail = total % G;
    if (!enabled || tail == 0 || nk < kMinSplitSlices)
        return 1;
    const int slots = min(G, kSplitSlots);
    return max(1, min(min(kMaxSplit, slots / tail), nk / (kMinSplitSlices / 2)));
}

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

// Byte address of a shared-memory object in the LDS address space.
__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// 16 bytes per lane from buffer `rsrc` at voff + soff straight into LDS at
// byte address lds + 16 * lane (buffer_load_dwordx4 ... lds; M0 holds the
// LDS base).
// Issued from asm so that the compiler does not track the LDS writes: they
// are ordered by the kernel's own vmcnt waits and barriers (the compiler
// would otherwise make LDS reads wait for all loads in flight).  The
// instruction has no destination register; its address operands are read at
// issue.
__device__ __forceinline__ void dma16(const i32x4& rsrc, uint32_t lds, uint32_t voff, uint32_t soff)
{
    // scalar operands: wave-uniform by construction; readfirstlane makes the
    // compiler place them in SGPRs (and keeps the offset off the immediate field)
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
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

// Accumulators of one wave: kFM x kFN 32x32 blocks.
template <typename S>
struct Acc {
    f32x16 v[S::kFM][S::kFN];
};

// One k-step's MFMA operands of a wave: 16 bytes per lane of each of its
// kFN weight blocks (a) and kFM activation blocks (b).
template <typename S>
struct Frag {
    typename S::frag_t a[S::kFN], b[S::kFM];
};

// Epilogue arguments.  a, w: per-row scales of an FP8 GEMM (null: none),
// a[source row of A] and w[e * Nw + weight row].  aux_out (nullable): the
// forward's pre-activation u is stored there as well ([rows][aux_ld], the
// gate columns then the up columns for SwiGLU).  aux_in: the saved u that
// the activation-backward epilogues read ([rows][aux_ld]).
struct EpiArgs {
    const float* a;
    const float* w;
    const void* aux_in;
    void* aux_out;
    int aux_ld;
};

// 4 consecutive elements of a row: loaded as stored (raw4, unpack4), or
// stored from fp32 (store4).
template <typename OT>
using raw4_t = typename std::conditional<OT::kBytes == 2, uint2, float4>::type;
template <typename OT>
__device__ __forceinline__ raw4_t<OT> load_raw4(const typename OT::storage* p)
{
    return *reinterpret_cast<const raw4_t<OT>*>(p);
}
template <typename OT>
__device__ __forceinline__ void unpack4(const raw4_t<OT>& w, float* v)
{
    if constexpr (OT::kBytes == 2) {
        v[0] = __uint_as_float(w.x << 16);
        v[1] = __uint_as_float(w.x & 0xffff0000u);
        v[2] = __uint_as_float(w.y << 16);
        v[3] = __uint_as_float(w.y & 0xffff0000u);
    } else {
        v[0] = w.x;
        v[1] = w.y;
        v[2] = w.z;
        v[3] = w.w;
    }
}
template <typename OT>
__device__ __forceinline__ void store4(typename OT::storage* p, const float* v)
{
    if constexpr (OT::kBytes == 2) {
        uint2 o;
        o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
        o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
        *reinterpret_cast<uint2*>(p) = o;
    } else {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// Epilogue: activation and store of a tile from the wave's accumulators.
// Lane holds row m = .. + (lane & 31), 4 consecutive columns per group.
// `wave` is the wave slot of the tile whose accumulators these are; OT the
// stored element type.  With scales, u = acc * a_scale(row) * w_scale(col)
// enters the epilogue (a_scale of row r is a[gather[r]] with a gather index).
// Backward epilogues (acc = dh at column f < F, u the saved pre-activation):
//   EPI_DRELU:   du[f] = u[f] > 0 ? dh : 0
//   EPI_DSWIGLU: g = u[f], v = u[F+f], s = 1/(1+e^-g):
//                du[f] = dh v s (1 + g (1 - s)),  du[F+f] = dh g s
// ONLY_I >= 0: store row fragment ONLY_I alone (the others are not read).
template <typename OT, typename S, int EPI, int ONLY_I = -1>
__device__ __forceinline__ void store_tile(const Acc<S>& acc, typename OT::storage* __restrict__ C, const TileDec& t,
                                           int Nout, int ncols, int wave, EpiArgs ep, const int32_t* gather, int Nw,
                                           int F)
{
    typedef typename OT::storage T;
    // lane-derived addresses stay here, not hoisted before the tile loop
    int lane = lane_id();
    __asm__ volatile("" : "+v"(lane));
    const int wm = wave / S::WN, wn = wave % S::WN;
#pragma unroll
    for (int i = 0; i < S::kFM; ++i) {
        if (ONLY_I >= 0 && i != ONLY_I)
            continue;
        const int m = wm * S::kWaveM + i * 32 + (lane & 31);
        if (m >= t.rows)
            continue;
        T* crow = C + (size_t)(t.row0 + m) * Nout;
        const T* urow = ep.aux_in ? (const T*)ep.aux_in + (size_t)(t.row0 + m) * ep.aux_ld : nullptr;
        T* prow = ep.aux_out ? (T*)ep.aux_out + (size_t)(t.row0 + m) * ep.aux_ld : nullptr;
        float as = 1.0f;
        if (ep.a)
            as = ep.a[gather ? gather[t.row0 + m] : t.row0 + m];
        const float* wsc = ep.w ? ep.w + (size_t)t.e * Nw : nullptr;
        // SwiGLU: the wave's kWaveN columns are its gate columns, then the
        // matching up columns.  With two or more 32-column blocks per wave
        // the up value of gate block j sits in block j + kFN / 2 at the same
        // place; with one block (kWaveN = 32) gate and up share the block,
        // the up value 16 columns (two 8-column groups) further on.
        constexpr bool kOneBlock = S::kFN == 1;
        constexpr int kJ = (EPI == EPI_SWIGLU) ? (kOneBlock ? 1 : S::kFN / 2) : S::kFN;
        constexpr int kG4 = (EPI == EPI_SWIGLU && kOneBlock) ? 2 : 4;  // gate groups of a block
        constexpr int kUpJ = kOneBlock ? 0 : S::kFN / 2, kUpG4 = kOneBlock ? 2 : 0;
        // Backward epilogues: this row fragment's saved u, all loaded before
        // any of its stores.  Stores and loads retire in issue order, so a
        // load issued after a store would wait for that store as well.
        constexpr bool kBwd = (EPI == EPI_DRELU || EPI == EPI_DSWIGLU);
        raw4_t<OT> ug[kBwd ? kJ : 1][4], uv[EPI == EPI_DSWIGLU ? kJ : 1][4];
        if constexpr (kBwd) {
#pragma unroll
            for (int j = 0; j < kJ; ++j)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int n = t.n0 + wn * S::kWaveN + j * 32 + 8 * g4 + 4 * (lane >> 5);
                    ug[j][g4] = raw4_t<OT>{};
                    if (n < ncols)
                        ug[j][g4] = load_raw4<OT>(urow + n);
                    if constexpr (EPI == EPI_DSWIGLU) {
                        uv[j][g4] = raw4_t<OT>{};
                        if (n < ncols)
                            uv[j][g4] = load_raw4<OT>(urow + F + n);
                    }
                }
        }
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
#pragma unroll
            for (int g4 = 0; g4 < kG4; ++g4) {
                const int nl = j * 32 + 8 * g4 + 4 * (lane >> 5);
                const int n = t.n0 + ((EPI == EPI_SWIGLU) ? wn * (S::kWaveN / 2) : wn * S::kWaveN) + nl;
                if (n >= ncols)
                    continue;
                float v[4], v2[4], pre[4], pre2[4], uin[4], uin2[4];
                if constexpr (kBwd)
                    unpack4<OT>(ug[j][g4], uin);
                if constexpr (EPI == EPI_DSWIGLU)
                    unpack4<OT>(uv[j][g4], uin2);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float u = acc.v[i][j][4 * g4 + q];
                    float up = (EPI == EPI_SWIGLU) ? acc.v[i][j + kUpJ][4 * (g4 + kUpG4) + q] : 0.0f;
                    if (wsc) {
                        u *= as * wsc[n + q];
                        if (EPI == EPI_SWIGLU)
                            up *= as * wsc[F + n + q];
                    }
                    pre[q] = u;
                    pre2[q] = up;
                    v2[q] = 0.0f;
                    if (EPI == EPI_RELU)
                        u = fmaxf(u, 0.0f);
                    if (EPI == EPI_SWIGLU)
                        u = u / (1.0f + __expf(-u)) * up;
                    if (EPI == EPI_DRELU)
                        u = uin[q] > 0.0f ? u : 0.0f;
                    if (EPI == EPI_DSWIGLU) {
                        const float g = uin[q], gv = uin2[q];
                        const float sg = 1.0f / (1.0f + __expf(-g));
                        v2[q] = u * g * sg;
                        u = u * gv * sg * (1.0f + g * (1.0f - sg));
                    }
                    v[q] = u;
                }
                store4<OT>(crow + n, v);
                if (EPI == EPI_DSWIGLU)
                    store4<OT>(crow + F + n, v2);
                if ((EPI == EPI_RELU || EPI == EPI_SWIGLU) && prow) {
                    store4<OT>(prow + n, pre);
                    if (EPI == EPI_SWIGLU)
                        store4<OT>(prow + F + n, pre2);
                }
            }
        }
    }
}

// Activation-backward epilogue through LDS (bf16 outputs).  The direct
// epilogue reads u and writes du 8 bytes per lane with the 32 lanes of a
// wave half on 32 different rows, so every wave instruction touches 32
// cache lines.  Here each row fragment i of every wave (kRowsPass rows) is
// first staged as fp32 dh [row][column] in a stage buffer (16-byte chunks
// XOR-swizzled by row, as in the plain epilogue below), then processed in
// the row domain: a thread takes 8 consecutive columns of one row (16-byte
// loads of u and stores of du, a wave covering whole row runs).  The
// arithmetic is that of store_tile, element by element.  The fragment's u
// loads are issued before its staging, so their latency overlaps it.
template <typename OT, typename S, int EPI>
__device__ __forceinline__ void store_tile_lds_bwd(const Acc<S>& acc, typename OT::storage* __restrict__ C,
                                                   const TileDec& t, int Nout, int ncols, int wave, EpiArgs ep, int F,
                                                   uint8_t* buf0, uint8_t* buf1)
{
    static_assert(OT::kBytes == 2, "bf16 outputs");
    static_assert(EPI == EPI_DRELU || EPI == EPI_DSWIGLU, "activation-backward epilogues");
    typedef typename OT::storage T;
    constexpr int kRowsPass = S::WM * 32;
    constexpr int kRowBytes = S::BN * 4;  // fp32 staging
    constexpr int kChunks = kRowBytes / 16;
    constexpr int kGroups = S::BN / 8;    // 8-column groups of a row
    constexpr int kPerThread = kRowsPass * kGroups / S::kThreads;
    static_assert(kRowsPass * kRowBytes <= S::kStage, "one fp32 row fragment of the tile fits a stage buffer");
    static_assert(kRowsPass * kGroups % S::kThreads == 0, "whole groups per thread");
    constexpr bool kPair = EPI == EPI_DSWIGLU;
    int tid = threadIdx.x;
    __asm__ volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int wm = wave / S::WN, wn = wave % S::WN;
    const int r = wm * 32 + (lane & 31);  // this lane's staging row within a pass
    const T* U = (const T*)ep.aux_in;
    lds_barrier();
#pragma unroll
    for (int i = 0; i < S::kFM; ++i) {
        uint8_t* buf = (i & 1) ? buf1 : buf0;
        uint4 ug[kPerThread], uv[kPair ? kPerThread : 1];
#pragma unroll
        for (int it = 0; it < kPerThread; ++it) {
            const int c = tid + it * S::kThreads;
            const int rr = c / kGroups, q = c % kGroups;
            const int m = (rr / 32) * S::kWaveM + i * 32 + (rr % 32);
            const int n = t.n0 + 8 * q;
            ug[it] = uint4{0, 0, 0, 0};
            if constexpr (kPair)
                uv[it] = uint4{0, 0, 0, 0};
            if (m < t.rows && n < ncols) {
                const T* urow = U + (size_t)(t.row0 + m) * ep.aux_ld;
                ug[it] = *reinterpret_cast<const uint4*>(urow + n);
                if constexpr (kPair)
                    uv[it] = *reinterpret_cast<const uint4*>(urow + F + n);
            }
        }
#pragma unroll
        for (int j = 0; j < S::kFN; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int byte = (wn * S::kWaveN + j * 32 + 8 * g4 + 4 * (lane >> 5)) * 4;
                *reinterpret_cast<float4*>(buf + r * kRowBytes + (((byte >> 4) ^ (r % kChunks)) << 4)) =
                    make_float4(acc.v[i][j][4 * g4], acc.v[i][j][4 * g4 + 1], acc.v[i][j][4 * g4 + 2],
                                acc.v[i][j][4 * g4 + 3]);
            }
        lds_barrier();
#pragma unroll
        for (int it = 0; it < kPerThread; ++it) {
            const int c = tid + it * S::kThreads;
            const int rr = c / kGroups, q = c % kGroups;
            const int m = (rr / 32) * S::kWaveM + i * 32 + (rr % 32);
            const int n = t.n0 + 8 * q;
            if (m >= t.rows || n >= ncols)
                continue;
            const float4 d0 = *reinterpret_cast<const float4*>(buf + rr * kRowBytes + (((2 * q) ^ (rr % kChunks)) << 4));
            const float4 d1 =
                *reinterpret_cast<const float4*>(buf + rr * kRowBytes + (((2 * q + 1) ^ (rr % kChunks)) << 4));
            const float dh[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            float g[8], gv[8], out[8], out2[8];
            unpack4<OT>(uint2{ug[it].x, ug[it].y}, g);
            unpack4<OT>(uint2{ug[it].z, ug[it].w}, g + 4);
            if constexpr (kPair) {
                unpack4<OT>(uint2{uv[it].x, uv[it].y}, gv);
                unpack4<OT>(uint2{uv[it].z, uv[it].w}, gv + 4);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float u = dh[e];
                if constexpr (kPair) {
                    const float sg = 1.0f / (1.0f + __expf(-g[e]));
                    out2[e] = u * g[e] * sg;
                    u = u * gv[e] * sg * (1.0f + g[e] * (1.0f - sg));
                } else {
                    u = g[e] > 0.0f ? u : 0.0f;
                }
                out[e] = u;
            }
            T* crow = C + (size_t)(t.row0 + m) * Nout;
            uint4 o;
            o.x = f32_to_bf16_bits(out[0]) | (f32_to_bf16_bits(out[1]) << 16);
            o.y = f32_to_bf16_bits(out[2]) | (f32_to_bf16_bits(out[3]) << 16);
            o.z = f32_to_bf16_bits(out[4]) | (f32_to_bf16_bits(out[5]) << 16);
            o.w = f32_to_bf16_bits(out[6]) | (f32_to_bf16_bits(out[7]) << 16);
            *reinterpret_cast<uint4*>(crow + n) = o;
            if constexpr (kPair) {
                o.x = f32_to_bf16_bits(out2[0]) | (f32_to_bf16_bits(out2[1]) << 16);
                o.y = f32_to_bf16_bits(out2[2]) | (f32_to_bf16_bits(out2[3]) << 16);
                o.z = f32_to_bf16_bits(out2[4]) | (f32_to_bf16_bits(out2[5]) << 16);
                o.w = f32_to_bf16_bits(out2[6]) | (f32_to_bf16_bits(out2[7]) << 16);
                *reinterpret_cast<uint4*>(crow + F + n) = o;
            }
        }
    }
}

// Forward epilogue through LDS (bf16 outputs): the staging of
// store_tile_lds_bwd, then per thread 8 consecutive output columns of one
// row.  None: the value itself; ReLU: h = max(u, 0) over the tile's BN
// columns.  SwiGLU: a wave's accumulator columns are kWaveN/2 gate columns
// then the matching up columns, so h column c of the tile (BN/2 of them)
// takes its gate value from staged column (c / half) * kWaveN + c % half and
// its up value half further.  With scales (FP8 operands) u = acc *
// (a_scale(row) * w_scale(column)) first, as in store_tile.  aux_out
// (nullable): the pre-activation u is stored as well, at column n (gate or
// ReLU) and F + n (up).
template <typename OT, typename S, int EPI>
__device__ __forceinline__ void store_tile_lds_fwd(const Acc<S>& acc, typename OT::storage* __restrict__ C,
                                                   const TileDec& t, int Nout, int ncols, int wave, EpiArgs ep,
                                                   const int32_t* gather, int Nw, int F, uint8_t* buf0, uint8_t* buf1)
{
    static_assert(OT::kBytes == 2, "bf16 outputs");
    static_assert(EPI == EPI_NONE || EPI == EPI_RELU || EPI == EPI_SWIGLU, "forward epilogues");
    typedef typename OT::storage T;
    constexpr bool kGlu = EPI == EPI_SWIGLU;
    constexpr int kHalf = S::kWaveN / 2;
    constexpr int kRowsPass = S::WM * 32;
    constexpr int kRowBytes = S::BN * 4;  // fp32 staging
    constexpr int kChunks = kRowBytes / 16;
    constexpr int kOutCols = kGlu ? S::BN / 2 : S::BN;
    constexpr int kGroups = kOutCols / 8;  // 8-column groups of an output row
    constexpr int kPerThread = kRowsPass * kGroups / S::kThreads;
    static_assert(kRowsPass * kRowBytes <= S::kStage, "one fp32 row fragment of the tile fits a stage buffer");
    static_assert(kRowsPass * kGroups % S::kThreads == 0, "whole groups per thread");
    static_assert(!kGlu || kHalf % 8 == 0, "a group stays within one wave's gate columns");
    int tid = threadIdx.x;
    __asm__ volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int wm = wave / S::WN, wn = wave % S::WN;
    const int r = wm * 32 + (lane & 31);
    T* P = (T*)ep.aux_out;
    auto staged = [&](uint8_t* buf, int rr, int col) {  // 4 fp32 values at staged column col (a multiple of 4)
        return *reinterpret_cast<const float4*>(buf + rr * kRowBytes + ((((col * 4) >> 4) ^ (rr % kChunks)) << 4));
    };
    auto pack8 = [](const float* v) {
        uint4 o;
        o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
        o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
        o.z = f32_to_bf16_bits(v[4]) | (f32_to_bf16_bits(v[5]) << 16);
        o.w = f32_to_bf16_bits(v[6]) | (f32_to_bf16_bits(v[7]) << 16);
        return o;
    };
    lds_barrier();
#pragma unroll
    for (int i = 0; i < S::kFM; ++i) {
        uint8_t* buf = (i & 1) ? buf1 : buf0;
#pragma unroll
        for (int j = 0; j < S::kFN; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int byte = (wn * S::kWaveN + j * 32 + 8 * g4 + 4 * (lane >> 5)) * 4;
                *reinterpret_cast<float4*>(buf + r * kRowBytes + (((byte >> 4) ^ (r % kChunks)) << 4)) =
                    make_float4(acc.v[i][j][4 * g4], acc.v[i][j][4 * g4 + 1], acc.v[i][j][4 * g4 + 2],
                                acc.v[i][j][4 * g4 + 3]);
            }
        lds_barrier();
#pragma unroll
        for (int it = 0; it < kPerThread; ++it) {
            const int c = tid + it * S::kThreads;
            const int rr = c / kGroups, q = c % kGroups;
            const int m = (rr / 32) * S::kWaveM + i * 32 + (rr % 32);
            const int oc = 8 * q;  // output column within the tile
            const int n = t.n0 + oc;
            if (m >= t.rows || n >= ncols)
                continue;
            const int sc0 = kGlu ? (oc / kHalf) * S::kWaveN + oc % kHalf : oc;  // staged column of the first value
            const float4 a0 = staged(buf, rr, sc0), a1 = staged(buf, rr, sc0 + 4);
            float u[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            float up[8], h[8];
            if constexpr (kGlu) {
                const float4 b0 = staged(buf, rr, sc0 + kHalf), b1 = staged(buf, rr, sc0 + kHalf + 4);
                const float v[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    up[e] = v[e];
            }
            if (ep.w) {
                const float as = ep.a ? ep.a[gather ? gather[t.row0 + m] : t.row0 + m] : 1.0f;
                const float* wsc = ep.w + (size_t)t.e * Nw;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    u[e] *= as * wsc[n + e];
                    if constexpr (kGlu)
                        up[e] *= as * wsc[F + n + e];
                }
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (kGlu)
                    h[e] = u[e] / (1.0f + __expf(-u[e])) * up[e];
                else if constexpr (EPI == EPI_RELU)
                    h[e] = fmaxf(u[e], 0.0f);
                else
                    h[e] = u[e];
            }
            *reinterpret_cast<uint4*>(C + (size_t)(t.row0 + m) * Nout + n) = pack8(h);
            if (P) {
                T* prow = P + (size_t)(t.row0 + m) * ep.aux_ld;
                *reinterpret_cast<uint4*>(prow + n) = pack8(u);
                if constexpr (kGlu)
                    *reinterpret_cast<uint4*>(prow + F + n) = pack8(up);
            }
        }
    }
}

// Plain epilogue (no activation, no scales) through LDS.  Direct stores
// from the accumulators write 4 consecutive values of 32 different rows per
// instruction, pieces HBM takes at well under half its write bandwidth; so
// each row fragment i of every wave (tile rows wm*kWaveM + i*32 + 0..31, WM
// bands of 32 rows) is first written to a stage buffer as [band row][column],
// 16-byte chunks XOR-swizzled by row (writes of a fragment and reads of a
// row both take the minimum LDS cycles), then stored by the whole block with
// one 16-byte chunk per lane, a wavefront covering a contiguous row run.
// Fragments alternate between the two stage buffers, one barrier each.  The
// caller's K loop must be finished (the first barrier here also covers its
// last LDS reads).
// NT: non-temporal global stores (outputs no later kernel here reads soon:
// the weight gradients).
template <typename OT, typename S, bool NT = false>
__device__ __forceinline__ void store_tile_lds(const Acc<S>& acc, typename OT::storage* __restrict__ C,
                                               const TileDec& t, int Nout, int ncols, int wave, uint8_t* buf0,
                                               uint8_t* buf1)
{
    constexpr int kRowsPass = S::WM * 32;
    constexpr int kRowBytes = S::BN * OT::kBytes;
    constexpr int kChunks = kRowBytes / 16;
    static_assert(kRowsPass * kRowBytes <= S::kStage, "one row fragment of the tile fits a stage buffer");
    // The addresses below depend on the thread index only; an opaque copy of
    // it keeps the compiler from computing them once before the tile loop
    // and holding them in registers through every K loop.
    int tid = threadIdx.x;
    __asm__ volatile("" : "+v"(tid));
    const int lane = tid & (kWave - 1);
    const int wm = wave / S::WN, wn = wave % S::WN;
    const int r = wm * 32 + (lane & 31);  // this lane's row within a pass
    lds_barrier();
#pragma unroll
    for (int i = 0; i < S::kFM; ++i) {
        uint8_t* buf = (i & 1) ? buf1 : buf0;
#pragma unroll
        for (int j = 0; j < S::kFN; ++j)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int col = wn * S::kWaveN + j * 32 + 8 * g4 + 4 * (lane >> 5);
                const int byte = col * OT::kBytes;
                uint8_t* dst = buf + r * kRowBytes + (((byte >> 4) ^ (r % kChunks)) << 4) + (byte & 15);
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    v[q] = acc.v[i][j][4 * g4 + q];
                if constexpr (OT::kBytes == 2) {
                    uint2 o;
                    o.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
                    o.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
                    *reinterpret_cast<uint2*>(dst) = o;
                } else {
                    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                }
            }
        lds_barrier();
        static_assert(kRowsPass * kChunks % S::kThreads == 0, "whole chunks per thread");
#pragma unroll
        for (int it = 0; it < kRowsPass * kChunks / S::kThreads; ++it) {
            const int c = tid + it * S::kThreads;
            const int rr = c / kChunks, q = c % kChunks;
            const int m = (rr / 32) * S::kWaveM + i * 32 + (rr % 32);
            const int col = q * (16 / OT::kBytes);
            if (m < t.rows && t.n0 + col < ncols) {
                const uint4 v = *reinterpret_cast<const uint4*>(buf + rr * kRowBytes + ((q ^ (rr % kChunks)) << 4));
                uint4* dst = reinterpret_cast<uint4*>(C + (size_t)(t.row0 + m) * Nout + t.n0 + col);
                if constexpr (NT) {
                    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
                    __builtin_nontemporal_store(u32x4v{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4v*>(dst));
                } else {
                    *dst = v;
                }
            }
        }
    }
}

// Partial tiles hold the accumulators in thread order: float4 number
// ((wave*kFM + i)*kFN + j)*4 + g of every lane, lane-minor, so both kernels
// read and write them with coalesced 16-byte accesses.
template <typename S>
__device__ __forceinline__ size_t partial_index(int wave, int i, int j, int g, int lane)
{
    return ((((size_t)(wave * S::kFM + i) * S::kFN + j) * 4 + g) * kWave + lane) * 4;
}

// WT (weights stored transposed, bf16): W[e] is [K][Nw], Nw contiguous, as the
// backward's input-gradient GEMMs find W2 [d][F] and W1 [n1][d].  A K slice
// of the weight tile is then kBK rows of BN consecutive columns; the DMA lays
// it out [k][n] (16-byte chunks of 32-byte column blocks XOR-swizzled by the
// row), and each MFMA weight fragment (8 consecutive k of one column) is two
// ds_read_b64_tr_b16: within a group of 16 lanes that instruction hands lane
// i value i % 4 of the 64-bit chunk at lane 4j + i / 4's address as its j-th
// value, so lanes pointing at rows k0..k0+3, columns c0 + 4 (s % 4) give lane
// i the column c0 + i at k0..k0+3.
//
// KG (K-grouped, the weight gradients): one dense output per expert,
// C[e] = A W^T over expert e's K range [offsets[e], offsets[e+1]) (device
// array, multiples of the K slice): A [max_rows][K], W [Nw][K] row-major with
// row stride K, C [E][max_rows][Nout] (Nout == Nw).  No row segments, no
// gather, no split.
template <typename ET, typename OT, typename S, int EPI, bool KG = false, bool WT = false>
__global__ __launch_bounds__(S::kThreads) __attribute__((amdgpu_waves_per_eu(S::kWavesPerSimd, S::kWavesPerSimd)))
void moe_grouped_gemm_kernel(const typename ET::storage* __restrict__ A, const int32_t* __restrict__ gather,
                             int gather_rows, const typename ET::storage* __restrict__ W,
                             typename OT::storage* __restrict__ C, const int32_t* __restrict__ offsets, int E,
                             int K, int Nw, int Nout, int F, int max_rows, float* __restrict__ partial, EpiArgs sc)
{
#if defined(__HIP_DEVICE_COMPILE__)  // the body uses device-only types; the host pass needs the stub only
    constexpr int kWaves = S::kWaves;
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[S::kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[S::kStage];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[S::S > 2 ? S::kStage : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[S::S > 3 ? S::kStage : 16];
    __shared__ int32_t s_pref[kGemmMaxE + 1];
    __shared__ int32_t s_wsum[kWaves];

    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // uniform: keeps DMA bases scalar
    const int wm = wave / S::WN, wn = wave % S::WN;
    const uint32_t rowK = (uint32_t)K * ET::kBytes;  // bytes of one row
    // LDS byte addresses of the stages
    const uint32_t stage_addr[4] = {lds_addr(lds0), lds_addr(lds1), lds_addr(lds2), lds_addr(lds3)};
    // per-lane LDS read offsets of each k-step's first 32-row block; blocks
    // 32 rows apart keep the same swizzle term, so the others sit at fixed
    // offsets from these
    uint32_t rdA[S::kKSteps][S::kChunks], rdB[S::kKSteps][S::kChunks];
#pragma unroll
    for (int kk = 0; kk < S::kKSteps; ++kk)
#pragma unroll
        for (int h = 0; h < S::kChunks; ++h) {
            const int c = S::kChunks * (2 * kk + (lane >> 5)) + h;  // logical 16-byte chunk of the row
            rdA[kk][h] = swz<S>(wm * S::kWaveM + (lane & 31), c);
            rdB[kk][h] = S::kLdsA + swz<S>(wn * S::kWaveN + (lane & 31), c);
        }
    // lane's place inside a 1 KB DMA block of rows [R0, R0 + 1024/RB): row
    // R0 + lane / kNch, physical chunk lane % kNch, which holds the logical
    // chunk of swz().  The swizzle term depends on the block only through the
    // parity of its index for 128-byte rows; a wave's blocks are
    // wave + kWaves*i, whose parity is the wave's (kWaves is even).
    const int lrow = lane / S::kNch, lphys = lane % S::kNch;
    const int blk_row0 = (S::RB == 128) ? 8 * (wave & 1) : 0;
    const int lchunk = lphys ^ (((blk_row0 + lrow) >> S::kSwzShift) & (S::kNch - 1));
    const uint32_t lane_chunk = (uint32_t)(lchunk << 4);
    // WT: weight tile rows are k, kWtPitch bytes of columns each.  Lane s of
    // lane group g (16 lanes) reads rows 16 kk + 8 (g >> 1) + (s >> 2) (+4 for
    // a fragment's second half), columns wn*kWaveN + 32 j + 16 (g & 1) +
    // 4 (s & 3).  The swizzle term wt_f(row) depends only on row bits 0, 1
    // and 3, which are (s >> 2) and (g >> 1) here, so it is one value per lane.
    static_assert(!WT || (ET::kBytes == 2 && S::kChunks == 1), "WT is a bf16 layout");
    constexpr uint32_t kWtPitch = S::BN * 2;
    uint32_t rdBT[S::kFN];
    if constexpr (WT) {
        const int g = lane >> 4, sl = lane & 15;
        const int row = 8 * (g >> 1) + (sl >> 2);
        const int f = wt_f(row);
#pragma unroll
        for (int j = 0; j < S::kFN; ++j) {
            const int blk = (wn * S::kWaveN + 32 * j) / 16 + (g & 1);
            rdBT[j] = S::kLdsA + row * kWtPitch + ((blk ^ f) << 5) + 8 * (sl & 3);
        }
    }

    const int tile_cols = (EPI == EPI_SWIGLU) ? S::BN / 2 : S::BN;
    const int ncols = (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU) ? F : Nout;
    const int ntn = (ncols + tile_cols - 1) / tile_cols;
    const int mtk = (max_rows + S::BM - 1) / S::BM;  // K-grouped mode: m-tiles per expert
    int total;
    if constexpr (KG) {
        total = E * mtk * ntn;
    } else {
        tile_prefix<S::kThreads>(offsets, E, max_rows, S::BM, ntn, s_pref, s_wsum);
        total = s_pref[E];
    }
    const int G = gridDim.x;
    const int nk = K / S::kBK;
    const int parts = KG ? 1 : split_parts(total, G, nk, partial != nullptr);
    const int full = total - total % G;
    const int tail = total - full;
    const int items = full + tail * parts;

    for (int base = 0; base < items; base += G) {
        // XCD-aware order: blocks b, b+8, b+16, ... share an XCD.
        const int b = blockIdx.x;
        const int item = (G % 8 == 0) ? base + (b % 8) * (G / 8) + b / 8 : base + b;
        if (item >= items)
            continue;
        int tile = item, k0 = 0, k1 = nk, slot = -1;
        if (item >= full && parts > 1) {
            const int j = item - full, part = j / tail;
            tile = full + j % tail;
            k0 = part * nk / parts;
            k1 = (part + 1) * nk / parts;
            slot = (j % tail) * parts + part;
        }
        TileDec t;
        typename OT::storage* Cb = C;
        if constexpr (KG) {
            // (expert, group of GM m-tiles, n-tile, m-tile) order, as decode_tile
            t.e = tile / (mtk * ntn);
            const int local = tile - t.e * mtk * ntn;
            const int g = local / (S::GM * ntn);
            const int within = local - g * S::GM * ntn;
            const int gs = min(S::GM, mtk - g * S::GM);
            const int mt = g * S::GM + within % gs;
            t.row0 = mt * S::BM;
            t.rows = min(S::BM, max_rows - t.row0);
            t.n0 = (within / gs) * tile_cols;
            const int ka = min(max(offsets[t.e], 0), K);
            const int kb = min(max(offsets[t.e + 1], ka), K);
            k0 = ka / S::kBK;
            k1 = kb / S::kBK;
            Cb = C + (size_t)t.e * max_rows * Nout;
        } else {
            t = decode_tile<S>(tile, s_pref, offsets, E, max_rows, ntn, tile_cols);
        }

        // activation rows: the tile's rows of A (rows past the segment read
        // 0), or rows gather[row] of A
        i32x4 rsA;
        uint32_t voffA[S::kBlkA];
        if (gather) {
            rsA = make_rsrc(A, (uint32_t)gather_rows * rowK);
#pragma unroll
            for (int i = 0; i < S::kBlkA; ++i) {
                const int r = S::kRowsPerBlk * (wave + kWaves * i) + lrow;
                const int src = (r < t.rows) ? gather[t.row0 + r] : -1;
                voffA[i] = (src >= 0 && src < gather_rows) ? (uint32_t)src * rowK + lane_chunk : 0xf0000000u;
            }
        } else {
            rsA = make_rsrc(A + (size_t)t.row0 * K, (uint32_t)t.rows * rowK);
#pragma unroll
            for (int i = 0; i < S::kBlkA; ++i)
                voffA[i] = (uint32_t)(S::kRowsPerBlk * (wave + kWaves * i) + lrow) * rowK + lane_chunk;
        }
        // this expert's weight matrix (K-grouped: the one W): rows past Nw read 0
        const i32x4 rsW = make_rsrc(KG ? W : W + (size_t)t.e * Nw * K, (uint32_t)Nw * rowK);
        uint32_t voffB[S::kBlkB];
#pragma unroll
        for (int i = 0; i < S::kBlkB; ++i) {
            const int r = S::kRowsPerBlk * (wave + kWaves * i);  // first LDS row of the block
            int wrow;
            if (EPI == EPI_SWIGLU) {
                const int wblk = r / S::kWaveN, rr = r % S::kWaveN;
                const int half = rr / (S::kWaveN / 2);
                const int hc = t.n0 + wblk * (S::kWaveN / 2) + rr % (S::kWaveN / 2);
                wrow = half ? F + hc : (hc < F ? hc : Nw);  // gate rows past F read 0
            } else {
                wrow = t.n0 + r;
            }
            voffB[i] = (uint32_t)(wrow + lrow) * rowK + lane_chunk;
            if constexpr (WT) {
                // 1 KB block = 1024 / kWtPitch rows of the [k][n] slice; the
                // lane's physical chunk holds the logical one of wt_f(row)
                constexpr int kRowsB = 1024 / kWtPitch, kChB = kWtPitch / 16;
                const int blk = wave + kWaves * i;
                const int row = kRowsB * blk + lane / kChB, pc = lane % kChB;
                const int lb = (pc >> 1) ^ wt_f(row);
                voffB[i] = (uint32_t)row * (uint32_t)Nw * 2u + (uint32_t)(t.n0 + 16 * lb + 8 * (pc & 1)) * 2u;
            }
        }

        // part: 0 the activation rows of the slice, 1 the weight rows, 2 both
        auto issue = [&](int kt, int stage, int part = 2) {
            const uint32_t soff = (uint32_t)kt * S::RB;
            // WT: the slice is kBK rows further down W[e]
            const uint32_t soffB = WT ? (uint32_t)kt * S::kBK * (uint32_t)Nw * 2u : soff;
            const uint32_t dst = stage_addr[stage] + wave * 1024;
            if (part != 1) {
#pragma unroll
                for (int i = 0; i < S::kBlkA; ++i)
                    dma16(rsA, dst + kWaves * i * 1024, voffA[i], soff);
            }
            if (part != 0) {
#pragma unroll
                for (int i = 0; i < S::kBlkB; ++i)
                    dma16(rsW, dst + S::kLdsA + kWaves * i * 1024, voffB[i], soffB);
            }
        };

        Acc<S> acc;
#pragma unroll
        for (int i = 0; i < S::kFM; ++i)
#pragma unroll
            for (int j = 0; j < S::kFN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    acc.v[i][j][v] = 0.0f;

        // Wait until at most n (< S) slices of this wave's loads are in flight.
        auto wait_slices = [&](int n) {
            if (S::S >= 4 && n >= 3)
                wait_vmcnt<(S::S >= 4 ? 3 : 0) * S::kLoads>();
            else if (S::S >= 3 && n >= 2)
                wait_vmcnt<(S::S >= 3 ? 2 : 0) * S::kLoads>();
            else if (n >= 1)
                wait_vmcnt<S::kLoads>();
            else
                wait_vmcnt<0>();
        };

        // MFMA operand fragments of one k-step, double-buffered in registers
        // so that a k-step's LDS reads can be issued before the previous
        // k-step's MFMAs.
        // LC (a std::integral_constant) is the number of this wave's row
        // fragments that hold rows of the segment: all kFM except in an
        // expert's last, partly filled m-tile, where fragments wholly past
        // the segment's end are neither read nor multiplied (their rows are
        // never stored).  Each count has its own copy of the K loop below, so
        // the full-tile loop keeps its schedule.
        Frag<S> fr0, fr1;
        auto read_frags = [&](const uint8_t* buf, int kk, Frag<S>& f, auto LC) {
            constexpr int L = decltype(LC)::value;
            auto rd = [&](uint32_t off) { return *reinterpret_cast<const i32x4*>(buf + off); };
            if constexpr (L > 0) {
#pragma unroll
            for (int j = 0; j < S::kFN; ++j) {
                if constexpr (WT) {
                    const uint8_t* p = buf + rdBT[j] + 16 * kk * kWtPitch;
                    const i32x2 lo = __builtin_bit_cast(i32x2, ds_read_tr16(p));
                    const i32x2 hi = __builtin_bit_cast(i32x2, ds_read_tr16(p + 4 * kWtPitch));
                    f.a[j] = i32x4{lo[0], lo[1], hi[0], hi[1]};
                } else if constexpr (S::kChunks == 2) {
                    f.a[j].lo = rd(rdB[kk][0] + j * 32 * S::RB);
                    f.a[j].hi = rd(rdB[kk][1] + j * 32 * S::RB);
                } else {
                    f.a[j] = rd(rdB[kk][0] + j * 32 * S::RB);
                }
            }
            }
#pragma unroll
            for (int i = 0; i < L; ++i) {
                if constexpr (S::kChunks == 2) {
                    f.b[i].lo = rd(rdA[kk][0] + i * 32 * S::RB);
                    f.b[i].hi = rd(rdA[kk][1] + i * 32 * S::RB);
                } else {
                    f.b[i] = rd(rdA[kk][0] + i * 32 * S::RB);
                }
            }
        };
        auto mfmas = [&](const Frag<S>& f, auto LC) {
            constexpr int L = decltype(LC)::value;
#pragma unroll
            for (int i = 0; i < L; ++i)
#pragma unroll
                for (int j = 0; j < S::kFN; ++j) {
                    if constexpr (ET::kBytes == 1) {
                        // E4M3 x E4M3, unit block scales (E8M0 127 = 2^0)
                        acc.v[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[j], f.b[i], acc.v[i][j],
                                                                                      0, 0, 0, 127, 0, 127);
                    } else if constexpr (ET::kBytes == 2) {
                        acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, f.a[j]), __builtin_bit_cast(bf16x8, f.b[i]), acc.v[i][j],
                            0, 0, 0);
                    } else {
                        const f32x4 va = __builtin_bit_cast(f32x4, f.a[j]);
                        const f32x4 vb = __builtin_bit_cast(f32x4, f.b[i]);
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[q], vb[q], acc.v[i][j], 0, 0, 0);
                    }
                }
        };
        // One K slice kt held in `cur` (stage cur_stage), whose first k-step
        // fragments are already in fr0.  Each k-step reads the next one's
        // fragments, then runs its MFMAs.  Before the last k-step's MFMAs the
        // slice boundary is crossed: wait for this wave's loads of slice
        // kt+1, meet the other waves (after which slice kt+1 is in LDS
        // everywhere and every wave's reads of `cur` are done), start loading
        // slice kt+S into `cur`, and read slice kt+1's first fragments from
        // `nxt`, so that the barrier and that LDS latency are hidden behind
        // the last k-step's MFMAs.  Buffers are distinct LDS arrays known at
        // compile time.
        static_assert(S::kKSteps == 2 || S::kKSteps == 4, "2 or 4 k-steps per slice");
        auto slice = [&](int kt, const uint8_t* cur, int cur_stage, const uint8_t* nxt, auto LC) {
            constexpr int L = decltype(LC)::value;
            if constexpr (S::kChunks == 2) {
                // FP8: a k-step's fragments are 32 bytes per operand block,
                // too wide to double-buffer beside 128 accumulators; they are
                // refilled in place once the k-step's MFMAs are issued
                // (scheduling fences keep the compiler from hoisting later
                // k-steps' reads above the MFMAs, which would need a second
                // register set for the fragments)
                static_assert(S::kKSteps == 2, "FP8 slices are 128 bytes: 2 k-steps");
                static_assert(S::kFN == 2, "FP8 k-step order assumes two weight blocks");
                // One k-step: MFMAs in (weight block j, row fragment i) order;
                // each operand is refilled with the next k-step's data as soon
                // as its last MFMA of this k-step is issued (a[0] after the
                // j = 0 group, b[i] after MFMA (i, 1), a[1] at the end), so
                // every refill has at least three MFMAs to land before the
                // next k-step uses it.
                auto kstep = [&](const uint8_t* src, int kk) {
                    auto rd = [&](uint32_t off) { return *reinterpret_cast<const i32x4*>(src + off); };
                    auto mf = [&](int i, int j) {
                        acc.v[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr0.a[j], fr0.b[i], acc.v[i][j],
                                                                                      0, 0, 0, 127, 0, 127);
                    };
#pragma unroll
                    for (int i = 0; i < L; ++i)
                        mf(i, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (L > 0) {
                        fr0.a[0].lo = rd(rdB[kk][0]);
                        fr0.a[0].hi = rd(rdB[kk][1]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < L; ++i) {
                        mf(i, 1);
                        __builtin_amdgcn_sched_barrier(0);
                        fr0.b[i].lo = rd(rdA[kk][0] + i * 32 * S::RB);
                        fr0.b[i].hi = rd(rdA[kk][1] + i * 32 * S::RB);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    if constexpr (L > 0) {
                        fr0.a[1].lo = rd(rdB[kk][0] + 32 * S::RB);
                        fr0.a[1].hi = rd(rdB[kk][1] + 32 * S::RB);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                };
                kstep(cur, 1);
                const bool more = kt + 1 < k1;
                if (more) {
                    wait_slices(min(S::S - 2, k1 - 2 - kt));
                    lds_barrier();
                    if (kt + S::S < k1)
                        issue(kt + S::S, cur_stage);
                }
                kstep(nxt, 0);  // after the last slice this reads stale, in-bounds data nobody uses
                return;
            }
            // 256x256 tiles: each k-step's 8 MFMAs alternate with the next
            // k-step's LDS reads (MFMA, read, MFMA, read, ...), so reads
            // spread over the MFMA stream instead of leaving in bursts whose
            // results the next MFMAs wait for (3-4% on these tiles; the
            // smaller tiles of the short-K shapes are faster as scheduled).
            constexpr bool kInterleave = S::kFM == 4 && S::kFN == 2;
            constexpr int kMfmas = L * S::kFN;
            constexpr int kReads = (L > 0 ? (WT ? 2 * S::kFN : S::kFN) : 0) + L;
            auto interleave = [&]() {
                if constexpr (kInterleave) {
#pragma unroll
                    for (int q = 0; q < (kMfmas < kReads ? kMfmas : kReads); ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                    }
                    if constexpr (kMfmas > kReads)
                        __builtin_amdgcn_sched_group_barrier(0x008, kMfmas - kReads, 0);
                    if constexpr (kReads > kMfmas)
                        __builtin_amdgcn_sched_group_barrier(0x100, kReads - kMfmas, 0);
                }
            };
            read_frags(cur, 1, fr1, LC);
            mfmas(fr0, LC);
            interleave();
            if constexpr (S::kKSteps == 4) {
                read_frags(cur, 2, fr0, LC);
                mfmas(fr1, LC);
                interleave();
                read_frags(cur, 3, fr1, LC);
                mfmas(fr0, LC);
                interleave();
            }
            // Two-stage rings request the slice's activation rows at the
            // barrier and its weight rows after this k-step's MFMAs: issued
            // together, the 8 waves' DMA filled the address unit's queues
            // right after every barrier (SQ_VMEM_TA_*_FIFO_FULL) and held up
            // the MFMAs behind them.  Split, on one box each: the Mixtral
            // up-projection 1.70-1.72 -> 1.68-1.70 ms, its training forward
            // 2.72 -> 2.66 ms and backward 6.50 -> 6.39 ms.  The next
            // barrier's wait covers both parts.
            constexpr bool kSplit = S::S == 2;
            if (kt + 1 < k1) {
                wait_slices(min(S::S - 2, k1 - 2 - kt));
                lds_barrier();
                if (kt + S::S < k1)
                    issue(kt + S::S, cur_stage, kSplit ? 0 : 2);
            }
            // After the last slice this reads stale data nobody uses (an
            // in-bounds LDS read; the next tile's __syncthreads waits for it
            // before any DMA reuses the buffer).  Reading unconditionally
            // keeps the fragment registers free of a merge of old and new
            // values, which would cost register copies.
            read_frags(nxt, 0, fr0, LC);
            mfmas(fr1, LC);
            interleave();
            if constexpr (kSplit) {
                if (kt + S::S < k1)
                    issue(kt + S::S, cur_stage, 1);
            }
        };
        static_assert(S::kKSteps % 2 == 0, "k-steps per slice must be even");

        auto kloop = [&](auto LC) {
        wait_vmcnt<0>();  // the previous tile's stores are out of the vmcnt count
        __syncthreads();  // every wave is done with the previous tile's buffers
        // fill the ring: slices k0 .. k0+S-1, then wait for the first
#pragma unroll
        for (int s0 = 0; s0 < S::S; ++s0) {
            if (k0 + s0 < k1)
                issue(k0 + s0, s0);
        }
        wait_slices(min(S::S - 1, k1 - 1 - k0));
        lds_barrier();
        read_frags(lds0, 0, fr0, LC);
        // slice k0 + n uses buffer n mod S
        int kt = k0;
        if constexpr (S::kChunks == 2) {
            // FP8: one slice per iteration (the unrolled form below gives the
            // accumulators of the wide FP8 MFMA several merge points, which
            // the register allocator resolves with copies and spills)
            static_assert(S::S == 2, "FP8 tiles use 2 LDS stages");
            for (; kt < k1; ++kt) {
                const bool odd = (kt - k0) & 1;
                slice(kt, odd ? lds1 : lds0, odd ? 1 : 0, odd ? lds0 : lds1, LC);
            }
        } else if constexpr (S::S == 2) {
            for (; kt + 2 <= k1; kt += 2) {
                slice(kt, lds0, 0, lds1, LC);
                slice(kt + 1, lds1, 1, lds0, LC);
            }
            if (kt < k1)
                slice(kt, lds0, 0, lds1, LC);
        } else if constexpr (S::S == 3) {
            for (; kt + 3 <= k1; kt += 3) {
                slice(kt, lds0, 0, lds1, LC);
                slice(kt + 1, lds1, 1, lds2, LC);
                slice(kt + 2, lds2, 2, lds0, LC);
            }
            if (kt < k1)
                slice(kt, lds0, 0, lds1, LC);
            if (kt + 1 < k1)
                slice(kt + 1, lds1, 1, lds2, LC);
        } else {
            for (; kt + 4 <= k1; kt += 4) {
                slice(kt, lds0, 0, lds1, LC);
                slice(kt + 1, lds1, 1, lds2, LC);
                slice(kt + 2, lds2, 2, lds3, LC);
                slice(kt + 3, lds3, 3, lds0, LC);
            }
            if (kt < k1)
                slice(kt, lds0, 0, lds1, LC);
            if (kt + 1 < k1)
                slice(kt + 1, lds1, 1, lds2, LC);
            if (kt + 2 < k1)
                slice(kt + 2, lds2, 2, lds3, LC);
        }

        };
        // live row fragments of this wave (see read_frags); the 256-row
        // tiles, whose expert segments end in partly filled m-tiles, take a
        // loop per count
        if constexpr (S::kFM == 4 && !KG) {
            const int live = min(max((t.rows - wm * S::kWaveM + 31) / 32, 0), S::kFM);
            if (live >= 4)
                kloop(std::integral_constant<int, 4>{});
            else if (live == 3)
                kloop(std::integral_constant<int, 3>{});
            else if (live == 2)
                kloop(std::integral_constant<int, 2>{});
            else if (live == 1)
                kloop(std::integral_constant<int, 1>{});
            else
                kloop(std::integral_constant<int, 0>{});
        } else {
            kloop(std::integral_constant<int, S::kFM>{});
        }
        if (slot < 0) {
            if constexpr (EPI == EPI_NONE && ET::kBytes != 1)  // unscaled plain output
                store_tile_lds<OT, S, KG>(acc, Cb, t, Nout, ncols, wave, lds0, lds1);
            else if constexpr ((EPI == EPI_DRELU || EPI == EPI_DSWIGLU) && OT::kBytes == 2)
                store_tile_lds_bwd<OT, S, EPI>(acc, Cb, t, Nout, ncols, wave, sc, F, lds0, lds1);
            else if constexpr (EPI != EPI_DRELU && EPI != EPI_DSWIGLU && OT::kBytes == 2)  // activation or scales
                store_tile_lds_fwd<OT, S, EPI>(acc, Cb, t, Nout, ncols, wave, sc, gather, Nw, F, lds0, lds1);
            else
                store_tile<OT, S, EPI>(acc, Cb, t, Nout, ncols, wave, sc, gather, Nw, F);
        } else {
            float* dst = partial + (size_t)slot * S::kTileFloats;
#pragma unroll
            for (int i = 0; i < S::kFM; ++i)
#pragma unroll
                for (int j = 0; j < S::kFN; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        *reinterpret_cast<float4*>(dst + partial_index<S>(wave, i, j, g, lane)) =
                            make_float4(acc.v[i][j][4 * g], acc.v[i][j][4 * g + 1], acc.v[i][j][4 * g + 2],
                                        acc.v[i][j][4 * g + 3]);
        }
    }
#endif
}

// Second pass of the tail split: one wavefront per (split tile, wave slot,
// row fragment) adds that fragment's K parts in part order and stores it
// through the same epilogue (kFM times the work items of one per wave slot,
// so the reduction is not latency-bound on a few wavefronts per CU).
template <typename OT, typename S, int EPI, int I>
__device__ __forceinline__ void tail_fragment(const float* __restrict__ partial, int j, int parts, int wave, int lane,
                                              typename OT::storage* __restrict__ C, const TileDec& t, int Nout,
                                              int ncols, EpiArgs sc, const int32_t* gather, int Nw, int F)
{
    Acc<S> acc;
#pragma unroll
    for (int jj = 0; jj < S::kFN; ++jj)
#pragma unroll
        for (int v = 0; v < 16; ++v)
            acc.v[I][jj][v] = 0.0f;
    for (int part = 0; part < parts; ++part) {
        const float* src = partial + (size_t)(j * parts + part) * S::kTileFloats;
#pragma unroll
        for (int jj = 0; jj < S::kFN; ++jj)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 p = *reinterpret_cast<const float4*>(src + partial_index<S>(wave, I, jj, g, lane));
                acc.v[I][jj][4 * g] += p.x;
                acc.v[I][jj][4 * g + 1] += p.y;
                acc.v[I][jj][4 * g + 2] += p.z;
                acc.v[I][jj][4 * g + 3] += p.w;
            }
    }
    store_tile<OT, S, EPI, I>(acc, C, t, Nout, ncols, wave, sc, gather, Nw, F);
}

template <typename OT, typename S, int EPI>
__global__ __launch_bounds__(256) void moe_grouped_gemm_tail_kernel(
    typename OT::storage* __restrict__ C, const int32_t* __restrict__ offsets, int E, int K, int Nw, int Nout, int F,
    int max_rows, int G, const float* __restrict__ partial, EpiArgs sc, const int32_t* __restrict__ gather)
{
    __shared__ int32_t s_pref[kGemmMaxE + 1];
    __shared__ int32_t s_wsum[256 / kWave];
    const int tile_cols = (EPI == EPI_SWIGLU) ? S::BN / 2 : S::BN;
    const int ncols = (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU) ? F : Nout;
    const int ntn = (ncols + tile_cols - 1) / tile_cols;
    tile_prefix<256>(offsets, E, max_rows, S::BM, ntn, s_pref, s_wsum);
    const int total = s_pref[E];
    const int nk = K / S::kBK;
    const int parts = split_parts(total, G, nk, true);
    if (parts <= 1)
        return;
    const int full = total - total % G;
    const int tail = total - full;
    const int lane = lane_id();
    static_assert(S::kFM <= 4, "row fragments per wave slot");
    const int nwork = tail * S::kWaves * S::kFM;
    for (int wk = blockIdx.x * 4 + threadIdx.x / kWave; wk < nwork; wk += gridDim.x * 4) {
        const int fi = wk % S::kFM, ws = wk / S::kFM;
        const int j = ws / S::kWaves, wave = ws % S::kWaves;
        const TileDec t = decode_tile<S>(full + j, s_pref, offsets, E, max_rows, ntn, tile_cols);
        if (fi == 0)
            tail_fragment<OT, S, EPI, 0>(partial, j, parts, wave, lane, C, t, Nout, ncols, sc, gather, Nw, F);
        else if (fi == 1)
            tail_fragment<OT, S, EPI, (S::kFM > 1 ? 1 : 0)>(partial, j, parts, wave, lane, C, t, Nout, ncols, sc,
                                                              gather, Nw, F);
        else if (fi == 2)
            tail_fragment<OT, S, EPI, (S::kFM > 2 ? 2 : 0)>(partial, j, parts, wave, lane, C, t, Nout, ncols, sc,
                                                              gather, Nw, F);
        else
            tail_fragment<OT, S, EPI, (S::kFM > 3 ? 3 : 0)>(partial, j, parts, wave, lane, C, t, Nout, ncols, sc,
                                                              gather, Nw, F);
    }
}

}  // namespace moe

namespace {
using namespace moe;

struct GemmArgs {
    const void* A;
    const int32_t* gather;
    int gather_rows;
    const void* W;
    void* C;
    const int32_t* offsets;
    int E, K, Nw, Nout, F, max_rows, ncu;
    float* partial;
    EpiArgs sc;
    hipStream_t stream;
};

// The tail split costs a second launch and the fp32 partial tiles; it pays
// only where a tile's K range is long.  Measured with and without it: the
// 512- and 1024-long K ranges of the 64-expert 512/1024 layer ran 2.2 us
// faster per GEMM without it (about 36 and 28 us); the 14336-long one of the
// Mixtral-shaped down-projection 0.22 ms faster with it.
constexpr int kMinSplitK = 2048;

template <typename ET, typename OT, typename S, int EPI, bool WT = false>
hipError_t launch_one(const GemmArgs& args)
{
    GemmArgs g = args;
    if (g.K < kMinSplitK)
        g.partial = nullptr;
    typedef typename ET::storage T;
    typedef typename OT::storage TO;
    const int tile_cols = (EPI == EPI_SWIGLU) ? S::BN / 2 : S::BN;
    const int ncols = (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU) ? g.F : g.Nout;
    const long long ntn = (ncols + tile_cols - 1) / tile_cols;
    // upper bound on m-tiles: floor(P/BM) full tiles plus one partial per expert
    const long long mt_max = g.max_rows / S::BM + (long long)(g.E < g.max_rows ? g.E : g.max_rows);
    const long long tiles_max = mt_max * ntn;
    long long grid = (long long)g.ncu * S::OCC;  // persistent: as many blocks as are resident at once
    // without the split a grid beyond the tile count only idles; with it the
    // spare blocks take K parts of the tiles
    if (tiles_max < grid && g.partial == nullptr)
        grid = (tiles_max + 7) / 8 * 8;
    if (grid < 1)
        grid = 1;
    moe_grouped_gemm_kernel<ET, OT, S, EPI, false, WT><<<dim3((unsigned)grid), dim3(S::kThreads), 0, g.stream>>>(
        (const T*)g.A, g.gather, g.gather_rows, (const T*)g.W, (TO*)g.C, g.offsets, g.E, g.K, g.Nw, g.Nout, g.F,
        g.max_rows, g.partial, g.sc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || g.partial == nullptr)
        return err;
    // at most kSplitSlots / 2 split tiles (each has >= 2 parts) x kWaves wave slots x kFM row
    // fragments, 4 per block
    moe_grouped_gemm_tail_kernel<OT, S, EPI>
        <<<dim3(kSplitSlots / 2 * S::kWaves * S::kFM / 4), dim3(256), 0, g.stream>>>(
        (TO*)g.C, g.offsets, g.E, g.K, g.Nw, g.Nout, g.F, g.max_rows, (int)grid, g.partial, g.sc, g.gather);
    return hipGetLastError();
}

template <typename ET, typename OT, typename S>
hipError_t launch_epi(int epi, const GemmArgs& g)
{
    if (epi == EPI_RELU)
        return launch_one<ET, OT, S, EPI_RELU>(g);
    if (epi == EPI_SWIGLU)
        return launch_one<ET, OT, S, EPI_SWIGLU>(g);
    if constexpr (ET::kBytes != 1) {  // the backward epilogues exist for bf16 and fp32
        if (epi == EPI_DRELU)
            return launch_one<ET, OT, S, EPI_DRELU>(g);
        if (epi == EPI_DSWIGLU)
            return launch_one<ET, OT, S, EPI_DSWIGLU>(g);
    }
    return launch_one<ET, OT, S, EPI_NONE>(g);
}

// Transposed-weight launches (bf16): the plain and activation-backward
// epilogues of the input-gradient GEMMs.
template <typename S>
hipError_t launch_wt(int epi, const GemmArgs& g)
{
    if (epi == EPI_DRELU)
        return launch_one<bf16_t, bf16_t, S, EPI_DRELU, true>(g);
    if (epi == EPI_DSWIGLU)
        return launch_one<bf16_t, bf16_t, S, EPI_DSWIGLU, true>(g);
    return launch_one<bf16_t, bf16_t, S, EPI_NONE, true>(g);
}
}  // namespace

// Tile configurations (BM, BN, WM, WN, slice bytes, stages, blocks per CU,
// m-tile group), picked from the mean rows per expert, which the host knows
// without reading the device-side offsets:
//   large   >= 512 rows per expert (bf16 forward: >= 256 rows where K >=
//           kLargeTileMinK): 256 x 256 tiles, 8 waves (2 per SIMD, 128 x 64
//           each), the densest tile that fits the register file; 2 x 64 KB
//           of LDS stages
//   medium  128..511 rows: 128 x 128 tiles, 8 waves (64 x 32 each), 2 blocks
//           per CU, so 4 waves share each SIMD (against 4 waves of 64 x 64,
//           same box, per layer: the 64-expert 512/1024 layer 0.1213-0.1216 ->
//           0.1192-0.1194 ms, the 2048-token Mixtral-family case 0.0402-0.0405
//           -> 0.0382-0.0383 ms; outputs bit-identical)
//   small   < 128 rows: 64 x 256 tiles, 8 waves (64 x 32 each, 2 per SIMD;
//           short segments, so tall tiles would mostly compute padding); 3 LDS
//           stages of 40 KB, which keep two slices in flight per CU on these
//           weight-streaming shapes (512 experts of 1024 x 512: up 138 -> 129
//           us, down 156 -> 147 us against 2 stages).  Against 4 waves of 64 x
//           64, same box, per layer: the 2048-token 512-expert case 0.0663-
//           0.0681 -> 0.0600-0.0619 ms, the 512-expert 16384-token layer
//           0.3401-0.3463 -> 0.3336-0.3387 ms; outputs bit-identical
// The same shapes serve bf16 and FP8 (a 128-byte slice is 64 bf16 or 128 FP8
// values of K); the FP8 small tile keeps 2 stages and the FP8 medium tile 4
// waves of 64 x 64, which its K loop needs (two weight blocks per wave).
#ifndef MOE_LARGE_TILE
#define MOE_LARGE_TILE 256, 256, 2, 4, 128, 2, 1, 8
#endif
#ifndef MOE_MEDIUM_TILE
#define MOE_MEDIUM_TILE 128, 128, 2, 4, 128, 2, 2, 4
#endif
#define MOE_MEDIUM_TILE_FP8 128, 128, 2, 2, 128, 2, 2, 4
#ifndef MOE_SMALL_TILE
#define MOE_SMALL_TILE 64, 256, 1, 8, 128, 3, 1, 4
#endif
#define MOE_SMALL_TILE_FP8 64, 256, 1, 4, 128, 2, 1, 4
#define MOE_F32_TILE 128, 128, 2, 2, 128, 2, 1, 4

// The bf16 forward takes the large tile from 256 mean rows on where K is at
// least this long: the 64-expert 512/1024 layer's down-projection (K = 1024,
// 256 rows per expert) ran 38.9 us on 256 x 256 tiles against 43.5 us on
// 128 x 128, while its up-projection (K = 512) ran 52.8 against 44.9 us.
constexpr int kLargeTileMinK = 1024;

// ... and only where that gives at least a quarter of the CUs a tile
// (estimated from the mean rows per expert): the 16-expert 256/1024 layer of
// 2048 tokens has about 16 tiles of 256 x 256 for its down-projection and ran
// 0.0526-0.0553 ms per layer on the 8-wave 128 x 128 tile against 0.0642-
// 0.0661 ms, while the 8192-token 64-expert layer (about 128 estimated, 194
// actual) keeps the large tile (0.1168-0.1200 against 0.1198-0.1239 ms).
static bool large_tile_fills(const GemmArgs& g, int epi, int mean_rows)
{
    const int ncols = epi == EPI_SWIGLU ? g.F : g.Nout;
    const int tile_cols = epi == EPI_SWIGLU ? 128 : 256;
    const long long est = (long long)g.E * std::max(1, mean_rows / 256) * ((ncols + tile_cols - 1) / tile_cols);
    return 4 * est >= g.ncu;
}

// Workspace bytes the tail split needs for a problem with this mean rows per
// expert (the partial tiles of the largest configuration the launcher may
// pick for it).  dtype: 0 fp32, 1 bf16, 2 FP8.
extern "C" size_t moe_grouped_gemm_partial_bytes(int dtype, int mean_rows)
{
    size_t tile_floats;
    if (dtype == 0)
        tile_floats = GemmShape<f32_t, MOE_F32_TILE>::kTileFloats;
    else if (mean_rows >= 256)
        tile_floats = GemmShape<bf16_t, MOE_LARGE_TILE>::kTileFloats;
    else if (mean_rows >= 128)
        tile_floats = GemmShape<bf16_t, MOE_MEDIUM_TILE>::kTileFloats;
    else
        tile_floats = GemmShape<bf16_t, MOE_SMALL_TILE>::kTileFloats;
    return (size_t)kSplitSlots * tile_floats * sizeof(float);
}

// epi: 0 none, 1 ReLU, 2 SwiGLU, 3 ReLU backward, 4 SwiGLU backward.  Nw =
// weight rows per expert, Nout = output row stride (= output columns).
// max_rows bounds offsets[E]; mean_rows is the expected rows per expert
// (selects the tile configuration).  gather (nullable) maps each permuted row
// to its row of A (gather_rows rows).  partial (nullable) is the tail-split
// workspace of moe_grouped_gemm_partial_bytes bytes; NULL disables the split.
// aux_out (nullable; epi 1, 2): the pre-activation u is stored there too;
// aux_in (epi 3, 4): the saved u; both [rows][aux_ld].
extern "C" hipError_t moe_launch_grouped_gemm(int dtype, int epi, const void* A, const int32_t* gather,
                                              int gather_rows, const void* W, void* C, const int32_t* offsets, int E,
                                              int K, int Nw, int Nout, int F, int max_rows, int mean_rows, int ncu,
                                              float* partial, const void* aux_in, void* aux_out, int aux_ld,
                                              hipStream_t stream)
{
    const GemmArgs g = {A, gather, gather_rows, W, C, offsets, E, K, Nw, Nout, F, max_rows, ncu, partial,
                        EpiArgs{nullptr, nullptr, aux_in, aux_out, aux_ld}, stream};
    if (dtype == 0)
        return launch_epi<f32_t, f32_t, GemmShape<f32_t, MOE_F32_TILE>>(epi, g);
    if (mean_rows >= 512 || (mean_rows >= 256 && K >= kLargeTileMinK && large_tile_fills(g, epi, mean_rows)))
        return launch_epi<bf16_t, bf16_t, GemmShape<bf16_t, MOE_LARGE_TILE>>(epi, g);
    if (mean_rows >= 128)
        return launch_epi<bf16_t, bf16_t, GemmShape<bf16_t, MOE_MEDIUM_TILE>>(epi, g);
    return launch_epi<bf16_t, bf16_t, GemmShape<bf16_t, MOE_SMALL_TILE>>(epi, g);
}

// bf16 grouped GEMM with the weights stored transposed: W [E][K][Nw] (Nw
// contiguous), so C = A W[e] per segment.  epi: 0 none, 3 ReLU backward, 4
// SwiGLU backward (aux_in / aux_ld as moe_launch_grouped_gemm).  No gather.
// Nw a multiple of 64; other arguments as moe_launch_grouped_gemm.
extern "C" hipError_t moe_launch_grouped_gemm_wt(int epi, const void* A, const void* W, void* C,
                                                 const int32_t* offsets, int E, int K, int Nw, int Nout, int F,
                                                 int max_rows, int mean_rows, int ncu, float* partial,
                                                 const void* aux_in, int aux_ld, hipStream_t stream)
{
    const GemmArgs g = {A, nullptr, 0, W, C, offsets, E, K, Nw, Nout, F, max_rows, ncu, partial,
                        EpiArgs{nullptr, nullptr, aux_in, nullptr, aux_ld}, stream};
    if (mean_rows >= 512)
        return launch_wt<GemmShape<bf16_t, MOE_LARGE_TILE>>(epi, g);
    if (mean_rows >= 128)
        return launch_wt<GemmShape<bf16_t, MOE_MEDIUM_TILE>>(epi, g);
    return launch_wt<GemmShape<bf16_t, MOE_SMALL_TILE>>(epi, g);
}

// FP8 grouped GEMM: A [rows][K] and W [E][Nw][K] hold E4M3 codes, a_scale
// the scale of each A row (indexed by the source row when gathering),
// w_scale [E][Nw] the scale of each weight row; C is bf16.  K must be a
// multiple of 128.  Other arguments as moe_launch_grouped_gemm.
extern "C" hipError_t moe_launch_grouped_gemm_fp8(int epi, const void* A, const int32_t* gather, int gather_rows,
                                                  const void* W, void* C, const int32_t* offsets, int E, int K,
                                                  int Nw, int Nout, int F, int max_rows, int mean_rows, int ncu,
                                                  float* partial, const float* a_scale, const float* w_scale,
                                                  hipStream_t stream)
{
    const GemmArgs g = {A, gather, gather_rows, W, C, offsets, E, K, Nw, Nout, F, max_rows, ncu, partial,
                        EpiArgs{a_scale, w_scale, nullptr, nullptr, 0}, stream};
    if (mean_rows >= 512)
        return launch_epi<fp8_t, bf16_t, GemmShape<fp8_t, MOE_LARGE_TILE>>(epi, g);
    if (mean_rows >= 128)
        return launch_epi<fp8_t, bf16_t, GemmShape<fp8_t, MOE_MEDIUM_TILE_FP8>>(epi, g);
    return launch_epi<fp8_t, bf16_t, GemmShape<fp8_t, MOE_SMALL_TILE_FP8>>(epi, g);
}

// Weight gradients, K-grouped: C[e] (fp32 [M][N]) = A[:, K_e] W[:, K_e]^T for
// every expert e, K_e = [kofs[e], kofs[e+1]) columns of A [M][lda] and
// W [N][lda] (bf16 or fp32 per dtype), kofs multiples of 64 (bf16) or 32
// (fp32) and <= lda, lda a multiple of 64.  Columns past an expert's rows must
// hold zeros (padding).
extern "C" hipError_t moe_launch_grouped_gemm_kgrp(int dtype, const void* A, const void* W, float* C,
                                                   const int32_t* kofs, int E, int lda, int M, int N, int ncu,
                                                   hipStream_t stream)
{
    auto go = [&](auto et, auto shape) -> hipError_t {
        typedef decltype(et) ET;
        typedef decltype(shape) S;
        typedef typename ET::storage T;
        const long long total = (long long)E * ((M + S::BM - 1) / S::BM) * ((N + S::BN - 1) / S::BN);
        long long grid = (long long)ncu * S::OCC;
        if (total < grid)
            grid = (total + 7) / 8 * 8;
        if (grid < 1)
            grid = 1;
        moe_grouped_gemm_kernel<ET, f32_t, S, EPI_NONE, true><<<dim3((unsigned)grid), dim3(S::kThreads), 0, stream>>>(
            (const T*)A, nullptr, 0, (const T*)W, C, kofs, E, lda, N, N, N, M, nullptr,
            EpiArgs{nullptr, nullptr, nullptr, nullptr, 0});
        return hipGetLastError();
    };
    if (dtype == 0)
        return go(f32_t{}, GemmShape<f32_t, MOE_F32_TILE>{});
    return go(bf16_t{}, GemmShape<bf16_t, MOE_LARGE_TILE>{});
}
