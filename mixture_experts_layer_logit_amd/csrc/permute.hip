// Counting-sort permutation of token rows by expert (gfx950).
//
// Megatron-Core page, "关键特性": token permutation kernel; "MoE负载均衡的挑战与应对":
// capacity with dropping, or dropless variable-size expert inputs.
//
// The T*k assignments are ordered by (expert, token).  The rank of assignment
// (t,j) on its expert e is the number of earlier tokens that chose e; ranks
// below the capacity C are kept at row offsets[e] + rank.  No atomic decides
// a rank, so the permutation is the same on every run:
//
//   count   chunks of 256 tokens build per-chunk expert histograms
//           (LDS atomics only count; counts do not depend on their order)
//   scan    one block: per-expert prefix over chunks (-> each chunk's base
//           rank), counts, capacity clip, exclusive scan over experts
//   scatter chunk by chunk again: rank = chunk base + earlier wavefronts'
//           counts + rank inside the wavefront, the last from ballots that
//           find the lanes holding the same expert; writes slot, src_token.
//           When nchunks*E is small it does the scan's work itself and the
//           scan is not launched
//   gather  one wavefront per token reads x[t] once (16-byte loads) and
//           writes it to each of the token's kept rows of x_perm
#include "common.h"

namespace moe {

constexpr int kChunk = 256;  // tokens per chunk (one thread per token)
constexpr int kMaxE = 1024;

__global__ __launch_bounds__(kChunk) void moe_count_kernel(const int32_t* __restrict__ topk_idx, int T, int E,
                                                           int k, int32_t* __restrict__ chunk_cnt)
{
    __shared__ int32_t hist[kMaxE];
    for (int e = threadIdx.x; e < E; e += kChunk)
        hist[e] = 0;
    __syncthreads();
    const int t = blockIdx.x * kChunk + threadIdx.x;
    if (t < T) {
        // the token's k choices loaded together, then counted
        int ch[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            ch[j] = j < k ? topk_idx[(size_t)t * k + j] : -1;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (ch[j] >= 0 && ch[j] < E)
                atomicAdd(&hist[ch[j]], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kChunk)
        chunk_cnt[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block of 1024 threads; thread e owns expert e.  chunk_cnt is turned
// into each chunk's base rank in place.
__global__ __launch_bounds__(1024) void moe_scan_kernel(int32_t* __restrict__ chunk_cnt, int nchunks, int E,
                                                        long long C, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ offsets)
{
    __shared__ int32_t wsum[1024 / kWave];
    const int e = threadIdx.x;
    int running = 0;
    if (e < E) {
        int c = 0;
        for (; c + 4 <= nchunks; c += 4) {
            const int v0 = chunk_cnt[(size_t)(c + 0) * E + e];
            const int v1 = chunk_cnt[(size_t)(c + 1) * E + e];
            const int v2 = chunk_cnt[(size_t)(c + 2) * E + e];
            const int v3 = chunk_cnt[(size_t)(c + 3) * E + e];
            chunk_cnt[(size_t)(c + 0) * E + e] = running;
            chunk_cnt[(size_t)(c + 1) * E + e] = running + v0;
            chunk_cnt[(size_t)(c + 2) * E + e] = running + v0 + v1;
            chunk_cnt[(size_t)(c + 3) * E + e] = running + v0 + v1 + v2;
            running += v0 + v1 + v2 + v3;
        }
        for (; c < nchunks; ++c) {
            const int v = chunk_cnt[(size_t)c * E + e];
            chunk_cnt[(size_t)c * E + e] = running;
            running += v;
        }
        counts[e] = running;
    }
    int kept = (e < E) ? running : 0;
    if (C >= 0 && kept > C)
        kept = (int)C;
    // exclusive scan of kept over the 1024 threads
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    int incl = kept;
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
        offsets[e] = base + incl - kept;
    if (e == E - 1)
        offsets[E] = base + incl;
}

// The scatter, as above.  With kFused the scan is done here too: chunk_cnt
// still holds the per-chunk counts, and every block sums them for its own
// base ranks (the chunks before it) and the experts' totals, clips them to
// the capacity and scans them into offsets (block 0 writes counts and
// offsets out).  That costs each block nchunks*E reads, so it is used when
// that product is at most kFuseScanMax, and saves the scan's launch.
constexpr long long kFuseScanMax = 64 * 1024;
constexpr int kScanBatch = 32;

template <bool kFused>
__global__ __launch_bounds__(kChunk) void moe_scatter_kernel(const int32_t* __restrict__ topk_idx, int T, int E,
                                                             int k, long long C,
                                                             const int32_t* __restrict__ chunk_cnt, int nchunks,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ slot,
                                                             int32_t* __restrict__ src_token)
{
    constexpr int kWaves = kChunk / kWave;
    __shared__ int32_t wave_cnt[kWaves][kMaxE];
    __shared__ int32_t s_base[kMaxE];  // this chunk's base rank per expert
    __shared__ int32_t s_off[kMaxE];   // the experts' first rows
    __shared__ int32_t wsum[kWaves];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    for (int i = threadIdx.x; i < kWaves * E; i += kChunk)
        wave_cnt[i / E][i % E] = 0;
    if constexpr (kFused) {
        for (int e = threadIdx.x; e < E; e += kChunk) {
            int b = 0, tot = 0;  // integer sums: the order does not matter
            // 32 chunk counts in flight at a time: the sums are bound by
            // the latency of these loads, not by their bytes
            for (int c0 = 0; c0 < nchunks; c0 += kScanBatch) {
                int v[kScanBatch];
#pragma unroll
                for (int q = 0; q < kScanBatch; ++q)
                    v[q] = chunk_cnt[(size_t)min(c0 + q, nchunks - 1) * E + e];
#pragma unroll
                for (int q = 0; q < kScanBatch; ++q) {
                    const int c = c0 + q;
                    b += c < (int)blockIdx.x ? v[q] : 0;
                    tot += c < nchunks ? v[q] : 0;
                }
            }
            s_base[e] = b;
            s_off[e] = (C >= 0 && tot > C) ? (int)C : tot;  // kept, scanned below
            if (blockIdx.x == 0)
                counts[e] = tot;
        }
        __syncthreads();
        // exclusive scan of the kept counts: thread i holds experts 4i..4i+3
        int v[4], loc = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * (int)threadIdx.x + q;
            v[q] = e < E ? s_off[e] : 0;
            loc += v[q];
        }
        int incl = loc;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int n = __shfl_up(incl, o);
            if (lane >= o)
                incl += n;
        }
        if (lane == kWave - 1)
            wsum[wave] = incl;
        __syncthreads();
        int run = incl - loc, total = 0;
        for (int w = 0; w < kWaves; ++w) {
            run += w < wave ? wsum[w] : 0;
            total += wsum[w];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = 4 * (int)threadIdx.x + q;
            if (e < E) {
                s_off[e] = run;
                if (blockIdx.x == 0)
                    offsets[e] = run;
                run += v[q];
            }
        }
        if (blockIdx.x == 0 && threadIdx.x == 0)
            offsets[E] = total;
    } else {
        for (int e = threadIdx.x; e < E; e += kChunk) {
            s_base[e] = chunk_cnt[(size_t)blockIdx.x * E + e];
            s_off[e] = offsets[e];
        }
    }
    __syncthreads();
    const int t = blockIdx.x * kChunk + threadIdx.x;
    const bool live = t < T;
    int my[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        my[j] = (j < k && live) ? topk_idx[(size_t)t * k + j] : -1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        my[j] = (my[j] >= 0 && my[j] < E) ? my[j] : -1;
        if (my[j] >= 0)
            atomicAdd(&wave_cnt[wave][my[j]], 1);
    }
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E)
        ++nbits;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j >= k)
            break;
        const int e = my[j];
        // lanes below this one whose choice in some column equals e
        int r = 0;
#pragma unroll
        for (int j2 = 0; j2 < 8; ++j2) {
            if (j2 >= k)
                break;
            const int col = my[j2];
            uint64_t peers = __ballot(col >= 0);
            for (int b = 0; b < nbits; ++b) {
                const uint64_t ones = __ballot(col >= 0 && ((col >> b) & 1));
                peers &= (((e >> b) & 1) ? ones : ~ones);
            }
            r += __popcll(peers & below);
        }
        if (e < 0)
            continue;
        for (int w = 0; w < wave; ++w)
            r += wave_cnt[w][e];
        const long long rank = (long long)s_base[e] + r;
        if (C < 0 || rank < C) {
            const int row = s_off[e] + (int)rank;
            slot[(size_t)t * k + j] = row;
            src_token[row] = t;
        } else {
            slot[(size_t)t * k + j] = -1;
        }
    }
    if (live) {
        for (int j = 0; j < k; ++j)
            if (my[j] < 0)
                slot[(size_t)t * k + j] = -1;
    }
}

// Small problems (T <= kSmallT tokens, E <= kSmallE experts): count, scan and
// scatter in one block of 1024 threads, saving two launches.  Counts come
// from LDS atomics over every assignment; then the tokens are walked in
// chunks of 1024 (one per thread) with a running per-expert base: a
// choice's rank is that base plus the counts of the earlier wavefronts of
// the chunk plus its rank inside the wavefront (ballots, as in the scatter
// kernel).  Same ranks, same rows, one launch.  Each chunk costs about 5 us
// on the one CU, so beyond one chunk the three-kernel path is faster
// (measured: 27 against 15 us at 4096 tokens, 8.7 against 12 us at 256).
constexpr int kSmallThreads = 1024;
constexpr int kSmallT = 1024;
constexpr int kSmallE = 256;

__global__ __launch_bounds__(kSmallThreads) void moe_permute_small_kernel(const int32_t* __restrict__ topk_idx, int T,
                                                                         int E, int k, long long C,
                                                                         int32_t* __restrict__ counts,
                                                                         int32_t* __restrict__ offsets,
                                                                         int32_t* __restrict__ slot,
                                                                         int32_t* __restrict__ src_token)
{
    constexpr int kWaves = kSmallThreads / kWave;
    __shared__ int32_t s_cnt[kSmallE];
    __shared__ int32_t s_off[kSmallE];
    __shared__ int32_t s_run[kSmallE];
    __shared__ int32_t wave_cnt[kWaves][kSmallE];
    __shared__ int32_t wsum[kWaves];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    if (tid < E)
        s_cnt[tid] = 0;
    __syncthreads();
    for (int a = tid; a < T * k; a += kSmallThreads) {
        const int e = topk_idx[a];
        if (e >= 0 && e < E)
            atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    // counts, capacity clip, exclusive scan over experts
    int kept = 0;
    if (tid < E) {
        counts[tid] = s_cnt[tid];
        kept = s_cnt[tid];
        if (C >= 0 && kept > C)
            kept = (int)C;
        s_run[tid] = 0;
    }
    int incl = kept;
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
    if (tid < E) {
        s_off[tid] = base + incl - kept;
        offsets[tid] = base + incl - kept;
    }
    if (tid == E - 1)
        offsets[E] = base + incl;
    int nbits = 0;
    while ((1 << nbits) < E)
        ++nbits;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int t0 = 0; t0 < T; t0 += kSmallThreads) {
        for (int i = tid; i < kWaves * E; i += kSmallThreads)
            wave_cnt[i / E][i % E] = 0;
        __syncthreads();
        const int t = t0 + tid;
        const bool live = t < T;
        int my[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            my[j] = -1;
            if (j < k && live) {
                const int e = topk_idx[(size_t)t * k + j];
                my[j] = (e >= 0 && e < E) ? e : -1;
            }
            if (my[j] >= 0)
                atomicAdd(&wave_cnt[wave][my[j]], 1);
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j >= k)
                break;
            const int e = my[j];
            int r = 0;
#pragma unroll
            for (int j2 = 0; j2 < 8; ++j2) {
                if (j2 >= k)
                    break;
                const int col = my[j2];
                uint64_t peers = __ballot(col >= 0);
                for (int b = 0; b < nbits; ++b) {
                    const uint64_t ones = __ballot(col >= 0 && ((col >> b) & 1));
                    peers &= (((e >> b) & 1) ? ones : ~ones);
                }
                r += __popcll(peers & below);
            }
            if (e < 0)
                continue;
            for (int w = 0; w < wave; ++w)
                r += wave_cnt[w][e];
            const long long rank = (long long)s_run[e] + r;
            if (C < 0 || rank < C) {
                const int row = s_off[e] + (int)rank;
                slot[(size_t)t * k + j] = row;
                src_token[row] = t;
            } else {
                slot[(size_t)t * k + j] = -1;
            }
        }
        if (live) {
            for (int j = 0; j < k; ++j)
                if (my[j] < 0)
                    slot[(size_t)t * k + j] = -1;
        }
        __syncthreads();
        if (tid < E) {
            int add = 0;
            for (int w = 0; w < kWaves; ++w)
                add += wave_cnt[w][tid];
            s_run[tid] += add;
        }
        // the next chunk clears wave_cnt only after this barrier
        __syncthreads();
    }
}

// One wavefront per token; the row is read once and written to each kept
// slot.  The token and its slots are wave-uniform (scalar loads, no
// divergent branches); x is read and x_perm written with non-temporal
// accesses (each byte is touched once here).
template <typename ET>
__global__ __launch_bounds__(256) void moe_gather_kernel(const typename ET::storage* __restrict__ x,
                                                         const int32_t* __restrict__ slot, int T, int d, int k,
                                                         typename ET::storage* __restrict__ x_perm)
{
    typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
    const int lane = lane_id();
    const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + threadIdx.x / kWave);
    if (t >= T)
        return;
    constexpr int kPer = 16 / ET::kBytes;           // elements per 16-byte vector
    const int nvec = d / kPer;                       // 16-byte vectors per row
    int rows[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        rows[j] = (j < k) ? slot[(size_t)t * k + j] : -1;
    const u32x4v* src = reinterpret_cast<const u32x4v*>(x + (size_t)t * d);
    for (int v0 = 0; v0 < nvec; v0 += kWave * 8) {
        u32x4v buf[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int v = v0 + u * kWave + lane;
            if (v < nvec)
                buf[u] = __builtin_nontemporal_load(src + v);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (rows[j] < 0)
                continue;
            u32x4v* dst = reinterpret_cast<u32x4v*>(x_perm + (size_t)rows[j] * d);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int v = v0 + u * kWave + lane;
                if (v < nvec)
                    __builtin_nontemporal_store(buf[u], dst + v);
            }
        }
    }
}

}  // namespace moe

// x_perm == NULL skips the row copy (a caller that reads the rows of x
// through src_token itself).
extern "C" hipError_t moe_launch_permute(int dtype, const int32_t* topk_idx, const void* x, int T, int d, int E,
                                         int k, long long C, int32_t* counts, int32_t* offsets, int32_t* slot,
                                         int32_t* src_token, void* x_perm, int32_t* chunk_cnt,
                                         hipStream_t stream)
{
    using namespace moe;
    if (T <= kSmallT && E <= kSmallE) {
        moe_permute_small_kernel<<<1, kSmallThreads, 0, stream>>>(topk_idx, T, E, k, C, counts, offsets, slot,
                                                                   src_token);
    } else {
        const int nchunks = (T + kChunk - 1) / kChunk;
        moe_count_kernel<<<nchunks, kChunk, 0, stream>>>(topk_idx, T, E, k, chunk_cnt);
        if ((long long)nchunks * E <= kFuseScanMax) {
            moe_scatter_kernel<true><<<nchunks, kChunk, 0, stream>>>(topk_idx, T, E, k, C, chunk_cnt, nchunks,
                                                                     offsets, counts, slot, src_token);
        } else {
            moe_scan_kernel<<<1, 1024, 0, stream>>>(chunk_cnt, nchunks, E, C, counts, offsets);
            moe_scatter_kernel<false><<<nchunks, kChunk, 0, stream>>>(topk_idx, T, E, k, C, chunk_cnt, nchunks,
                                                                      offsets, counts, slot, src_token);
        }
    }
    if (x_perm == nullptr)
        return hipGetLastError();
    const dim3 grid((T + 3) / 4);
    if (dtype == 0)
        moe_gather_kernel<f32_t><<<grid, 256, 0, stream>>>((const float*)x, slot, T, d, k, (float*)x_perm);
    else
        moe_gather_kernel<bf16_t><<<grid, 256, 0, stream>>>((const uint16_t*)x, slot, T, d, k,
                                                            (uint16_t*)x_perm);
    return hipGetLastError();
}
