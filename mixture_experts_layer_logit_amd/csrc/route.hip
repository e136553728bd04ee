// Gate GEMM and wavefront-per-token router (gfx950); for up to 64 experts
// both in one kernel, routing each token with a group of lanes.
//
// Gate: one fully connected layer scores every token against every expert
// (FastMoE announcement page, "特色二").  Router: optional Skywork gating-logit
// normalisation (Skywork-MoE news item, "技术创新 1"; Skywork slides, slide 6),
// softmax over all experts, top-k on the fp32 logit (Megatron-Core page,
// "关键特性"; FastMoE page, Fig. 4: the top-2 gate takes the two best scores).
#include "common.h"

#include <type_traits>

namespace moe {

// ---------------------------------------------------------------- gate GEMM
// logits[t,e] = (float)( sum_i x[t,i] * Wg[e,i] + bg[e] ) with every product
// and sum in fp64.  bf16 x bf16 and fp32 x fp32 products are exact in fp64,
// so the only roundings are the fp64 additions; the result is the correctly
// rounded fp32 value of a sum accurate to ~1e-16 relative, independent of the
// tiling.  Routing decisions therefore do not depend on how this kernel (or
// any other correct gate) orders its sums.
//
// Work split: the fp64 matrix cores (v_mfma_f64_16x16x4f64: D[i][j] +=
// sum over 4 k of A[i][k] B[k][j], products exact, fp64 accumulation).  A
// block owns 16 tokens x 16 experts; its kGateSplit wavefronts split the
// model dimension into 32-element blocks (wavefront w takes blocks w, w +
// kGateSplit, ...).  Lane l (operand row l % 16, k group g = l / 16) loads 8
// consecutive elements of its token's x row and of its expert's Wg row (16
// bytes of bf16, 32 of fp32) at 8 g within the block and feeds them as the
// k = g column of 8 successive MFMAs: both operands take the block's k
// values in the same permuted order, so the 8 MFMAs add every product of the
// block.  The wavefronts' 16 x 16 partial sums then meet in LDS and are added
// in wavefront order with the bias (fp64), and rounded once to fp32.  Output
// layout of the MFMA (probed in bounds on the GPU): value r of lane l is
// D[4 r + l / 16][l % 16].  Rows past T or E are computed from clamped rows
// and not stored.
constexpr int kGateSplit = 8;
constexpr int kGateTile = 16;
constexpr int kGateDepth = 4;

// 8 consecutive values of a row as loaded (16 bytes of bf16, 32 of fp32).
template <typename ET>
struct GateChunk;
template <>
struct GateChunk<bf16_t> {
    uint4 v;
    __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void unpack(float* f) const { unpack8(v, f, bf16_t{}); }
};
template <>
struct GateChunk<f32_t> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p)
    {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void unpack(float* f) const
    {
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
};

template <typename ET>
__global__ __launch_bounds__(kGateSplit * kWave) void moe_gate_logits_kernel(
    const typename ET::storage* __restrict__ x, const typename ET::storage* __restrict__ Wg,
    const float* __restrict__ bg, float* __restrict__ logits, int T, int d, int E)
{
    typedef double f64x4 __attribute__((ext_vector_type(4)));
    __shared__ double s_part[kGateSplit][kGateTile * kGateTile];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int t0 = blockIdx.x * kGateTile, e0 = blockIdx.y * kGateTile;
    const int i = lane % kGateTile, g = lane / kGateTile;
    const typename ET::storage* xr = x + (size_t)min(t0 + i, T - 1) * d + 8 * g;
    const typename ET::storage* wr = Wg + (size_t)min(e0 + i, E - 1) * d + 8 * g;
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
    // this wavefront's blocks: wave, wave + kGateSplit, ...; their raw 16- or
    // 32-byte chunks go through a ring of kGateDepth register slots, refilled
    // kGateDepth blocks ahead, so several loads are in flight per wavefront
    const int nb = (d / 32 - wave + kGateSplit - 1) / kGateSplit;
    typedef GateChunk<ET> Chunk;
    Chunk xq[kGateDepth], wq[kGateDepth];
#pragma unroll
    for (int q = 0; q < kGateDepth; ++q)
        if (q < nb) {
            xq[q].load(xr + (size_t)(wave + q * kGateSplit) * 32);
            wq[q].load(wr + (size_t)(wave + q * kGateSplit) * 32);
        }
    for (int it = 0; it < nb; it += kGateDepth) {
#pragma unroll
        for (int q = 0; q < kGateDepth; ++q) {
            if (it + q < nb) {
                float xf[8], wf[8];
                xq[q].unpack(xf);
                wq[q].unpack(wf);
                if (it + q + kGateDepth < nb) {
                    const size_t off = (size_t)(wave + (it + q + kGateDepth) * kGateSplit) * 32;
                    xq[q].load(xr + off);
                    wq[q].load(wr + off);
                }
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xf[s], (double)wf[s], acc, 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
        s_part[wave][(4 * r + g) * kGateTile + i] = acc[r];
    __syncthreads();
    if (threadIdx.x < kGateTile * kGateTile) {
        const int t = t0 + threadIdx.x / kGateTile, e = e0 + threadIdx.x % kGateTile;
        double sum = s_part[0][threadIdx.x];
#pragma unroll
        for (int w = 1; w < kGateSplit; ++w)
            sum += s_part[w][threadIdx.x];
        if (t < T && e < E) {
            if (bg)
                sum += (double)bg[e];
            logits[(size_t)t * E + e] = (float)sum;
        }
    }
}

// ---------------------------------------------------------------- router
// One group of G = 16, 32 or 64 lanes per token.  Expert e lives in group
// lane e % G, register e / G.
//
// Selection key: the raw fp32 logit mapped to an order-preserving 32-bit
// integer (-0 folded onto +0), in the high half of a 64-bit key whose low
// half is (0xffffffff - e); the group-wide maximum is then the largest
// logit with ties going to the lowest expert index.  k rounds of max-reduce
// give the k experts in descending order.  The standardise-and-scale
// normalisation and the softmax are strictly increasing maps for lambda > 0
// and sigma > 0 (and constant otherwise), so selecting on the logit is the
// same as selecting on the probability, without depending on how either side
// rounds exp or the reductions.
//
// Probabilities are formed in fp64 (mean, population variance, softmax: the
// denominator's terms from the fp32 exp, see token_probs) and only the k
// selected ones are stored, rounded to fp32.
__device__ __forceinline__ uint32_t ordered_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) == 0)
        u = 0;  // -0 == +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Reductions over aligned groups of G lanes (G = 16, 32 or 64: the
// wavefront).  Within each row of 16 lanes four DPP steps pair lane i with
// i ^ 1, i ^ 2, 7 - i (within 8) and 15 - i: every step combines two partial
// results that are bitwise equal on both lanes of a pair (the operations are
// commutative), so after them every lane of a row holds the same row result,
// with no trip through the LDS crossbar.  Rows are then combined by one
// shuffle (G = 32) or, for the whole wavefront, by reading the four row
// results as wave-uniform values and combining them in one fixed order.
constexpr int kDppXor1 = 0xb1;        // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}
template <int G, typename T, typename Op>
__device__ __forceinline__ T group_reduce(T v, Op op)
{
    static_assert(sizeof(T) == 8, "64-bit values");
    static_assert(G == 16 || G == 32 || G == 64, "groups of whole rows");
    auto step = [&](auto ctrl) {
        constexpr int C = decltype(ctrl)::value;
        v = op(v, __builtin_bit_cast(T, dpp_u64<C>(__builtin_bit_cast(uint64_t, v))));
    };
    step(std::integral_constant<int, kDppXor1>{});
    step(std::integral_constant<int, kDppXor2>{});
    step(std::integral_constant<int, kDppHalfMirror>{});
    step(std::integral_constant<int, kDppMirror>{});
    if constexpr (G == 32) {
        v = op(v, __shfl_xor(v, 16));
    } else if constexpr (G == 64) {
        const uint64_t u = __builtin_bit_cast(uint64_t, v);
        const T r0 = __builtin_bit_cast(T, readlane_u64(u, 0)), r1 = __builtin_bit_cast(T, readlane_u64(u, 16));
        const T r2 = __builtin_bit_cast(T, readlane_u64(u, 32)), r3 = __builtin_bit_cast(T, readlane_u64(u, 48));
        v = op(op(r0, r1), op(r2, r3));
    }
    return v;
}
template <int G>
__device__ __forceinline__ double group_sum(double v)
{
    return group_reduce<G>(v, [](double a, double b) { return a + b; });
}
template <int G>
__device__ __forceinline__ double group_max(double v)
{
    return group_reduce<G>(v, [](double a, double b) { return fmax(a, b); });
}
template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v)
{
    return group_reduce<G>(v, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ double wave_sum(double v) { return group_sum<kWave>(v); }
__device__ __forceinline__ double wave_max(double v) { return group_max<kWave>(v); }

// Gate probabilities of one token held by a group of G lanes (by default
// the wavefront): z[i] is the logit of expert lane + G i, lane being the
// index within the group (0 past E).  Scores s in fp64 are the logit, or
// lambda * (z - mu) / sigma (population sigma over the E experts; sigma == 0
// gives s = 0); p_e = ex[i] / denom with ex = exp(s - max s), s and m = max s
// returned as well.
// FAST (the forward router, which stores only the k selected weights): the
// terms of the denominator are exp(s - m) of the fp32-rounded argument in
// fp32 (one hardware exp each instead of a software fp64 exp), summed in
// fp64.  Every term lies in (0, 1] with a relative error of a few fp32 units
// (the argument's rounding adds at most |s - m| 2^-24, which matters only
// where the term itself is tiny), so the sum is within about 2^-21 relative
// of the fp64 one; the selected numerators are recomputed in fp64
// (select_topk), so a weight differs from the all-fp64 value by at most a
// few fp32 units.
// Score of one logit: z itself, or lambda * (z - mu) / sigma when
// normalised (sigma == 0 gives 0).
__device__ __forceinline__ double logit_score(float z, int normalize, float lambda, double mu, double sigma)
{
    if (!normalize)
        return (double)z;
    return sigma == 0.0 ? 0.0 : (double)lambda * ((double)z - mu) / sigma;
}

template <int VPL, int G = kWave, bool FAST = false>
__device__ __forceinline__ void token_probs(const float (&z)[VPL], int lane, int E, int normalize, float lambda,
                                            double (&ex)[VPL], double& denom, double& m, double& mu, double& sigma)
{
    mu = 0.0;
    sigma = 0.0;
    if (normalize) {
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            part += (lane + G * i < E) ? (double)z[i] : 0.0;
        mu = group_sum<G>(part) / E;
        part = 0.0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const double c = (double)z[i] - mu;
            part += (lane + G * i < E) ? c * c : 0.0;
        }
        sigma = sqrt(group_sum<G>(part) / E);
    }
    double s[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        s[i] = logit_score(z[i], normalize, lambda, mu, sigma);
    m = -INFINITY;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (lane + G * i < E)
            m = fmax(m, s[i]);
    m = group_max<G>(m);
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        if constexpr (FAST)
            ex[i] = (lane + G * i < E) ? (double)__expf((float)(s[i] - m)) : 0.0;
        else
            ex[i] = (lane + G * i < E) ? exp(s[i] - m) : 0.0;
        part += ex[i];
    }
    denom = group_sum<G>(part);
}
template <int VPL, int G = kWave>
__device__ __forceinline__ void token_probs(const float (&z)[VPL], int lane, int E, int normalize, float lambda,
                                            double (&ex)[VPL], double& denom)
{
    double m, mu, sigma;
    token_probs<VPL, G, false>(z, lane, E, normalize, lambda, ex, denom, m, mu, sigma);
}

// Selection key of expert e with logit z: the order-preserving 32-bit image
// of the fp32 logit above (0xffffffff - e), so that the largest key is the
// largest logit with ties going to the lowest expert index.  Real keys are
// never 0, which marks an empty or taken slot.
__device__ __forceinline__ uint64_t select_key(float z, int e)
{
    return ((uint64_t)ordered_key(z) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e);
}
// The logit a key was made from (-0 comes back as +0, which scores alike).
__device__ __forceinline__ float key_logit(uint64_t key)
{
    const uint32_t o = (uint32_t)(key >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// The k selections of one token held by a group of G lanes: k rounds of a
// group-wide maximum of the keys; every lane clears the winning key where
// it holds it and forms the winner's weight exp(s - m) / denom in fp64 from
// the logit inside the key (the same score as in the denominator), so the
// weight is group-uniform and needs no exchange.  Lane 0 of the group
// stores.
template <int VPL, int G = kWave>
__device__ __forceinline__ void select_topk(uint64_t (&key)[VPL], int normalize, float lambda, double mu,
                                            double sigma, double m, double denom, int lane, int t, int k,
                                            int32_t* __restrict__ topk_idx, float* __restrict__ topk_w)
{
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            best = key[i] > best ? key[i] : best;
        best = group_max_u64<G>(best);
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            key[i] = key[i] == best ? 0 : key[i];
        const int e = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffu));
        const double pe = exp(logit_score(key_logit(best), normalize, lambda, mu, sigma) - m) / denom;
        if (lane == 0) {
            topk_idx[(size_t)t * k + j] = e;
            topk_w[(size_t)t * k + j] = (float)pe;
        }
    }
}

// One group of G lanes per token (256 / G tokens per block): expert e in
// group lane e % G, register e / G.
template <int VPL, int G>
__global__ __launch_bounds__(256) void moe_router_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                         int normalize, float lambda,
                                                         int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w)
{
    const int li = threadIdx.x % G;
    const int t = blockIdx.x * (256 / G) + threadIdx.x / G;
    if (t >= T)
        return;  // whole groups leave together
    const float* zt = logits + (size_t)t * E;
    float z[VPL];
    uint64_t key[VPL];
    // every load from a clamped index, the padding zeroed afterwards: a load
    // under the index test is waited on before the next one is issued
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        z[i] = zt[min(li + G * i, E - 1)];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = li + G * i;
        z[i] = e < E ? z[i] : 0.0f;
        key[i] = e < E ? select_key(z[i], e) : 0;
    }
    double ex[VPL], denom, m, mu, sigma;
    token_probs<VPL, G, true>(z, li, E, normalize, lambda, ex, denom, m, mu, sigma);
    select_topk<VPL, G>(key, normalize, lambda, mu, sigma, m, denom, li, t, k, topk_idx, topk_w);
}

// ---------------------------------------------------------------- gate + router
// For E <= 64 one block computes all E logits of its 16 tokens and routes
// them, which saves the router's launch and its re-read of the logits.
// The gate part is the gate kernel above with NT 16-expert column tiles
// that share each x chunk: every logit is still the fp64 sum of exact
// products, each wavefront adding its own k blocks, the wavefronts'
// partials added in wavefront order with the bias, rounded once to fp32.
// The logits go to memory and to LDS; then each token is routed by a group
// of G = threads / 16 lanes, expert e in group lane e % G, register e / G,
// with the router kernel's arithmetic (selection on the fp32 logit, fp64
// probabilities).
template <typename ET, int NT, int SPLIT>
__global__ __launch_bounds__(SPLIT * kWave) void moe_gate_route_kernel(
    const typename ET::storage* __restrict__ x, const typename ET::storage* __restrict__ Wg,
    const float* __restrict__ bg, float* __restrict__ logits, int T, int d, int E, int k, int normalize,
    float lambda, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w)
{
    typedef double f64x4 __attribute__((ext_vector_type(4)));
    constexpr int kCols = kGateTile * NT;             // experts covered
    constexpr int G = SPLIT * kWave / kGateTile;      // routing lanes per token
    constexpr int VPL = (kCols + G - 1) / G;
    static_assert(G <= kWave && kWave % G == 0, "routing groups lie inside a wavefront");
    __shared__ double s_part[SPLIT][kGateTile * kCols];
    __shared__ float s_z[kGateTile][kCols];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    const int t0 = blockIdx.x * kGateTile;
    const int i = lane % kGateTile, g = lane / kGateTile;
    const typename ET::storage* xr = x + (size_t)min(t0 + i, T - 1) * d + 8 * g;
    const typename ET::storage* wr[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n)
        wr[n] = Wg + (size_t)min(kGateTile * n + i, E - 1) * d + 8 * g;
    f64x4 acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n)
        acc[n] = f64x4{0.0, 0.0, 0.0, 0.0};
    const int nb = (d / 32 - wave + SPLIT - 1) / SPLIT;
    typedef GateChunk<ET> Chunk;
    Chunk xq[kGateDepth], wq[kGateDepth][NT];
#pragma unroll
    for (int q = 0; q < kGateDepth; ++q)
        if (q < nb) {
            const size_t off = (size_t)(wave + q * SPLIT) * 32;
            xq[q].load(xr + off);
#pragma unroll
            for (int n = 0; n < NT; ++n)
                wq[q][n].load(wr[n] + off);
        }
    for (int it = 0; it < nb; it += kGateDepth) {
#pragma unroll
        for (int q = 0; q < kGateDepth; ++q) {
            if (it + q < nb) {
                float xf[8], wf[NT][8];
                xq[q].unpack(xf);
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    wq[q][n].unpack(wf[n]);
                if (it + q + kGateDepth < nb) {
                    const size_t off = (size_t)(wave + (it + q + kGateDepth) * SPLIT) * 32;
                    xq[q].load(xr + off);
#pragma unroll
                    for (int n = 0; n < NT; ++n)
                        wq[q][n].load(wr[n] + off);
                }
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const double xd = (double)xf[s];
#pragma unroll
                    for (int n = 0; n < NT; ++n)
                        acc[n] = __builtin_amdgcn_mfma_f64_16x16x4f64(xd, (double)wf[n][s], acc[n], 0, 0, 0);
                }
            }
        }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            s_part[wave][(4 * r + g) * kCols + kGateTile * n + i] = acc[n][r];
    __syncthreads();
    for (int q = threadIdx.x; q < kGateTile * kCols; q += SPLIT * kWave) {
        const int tok = q / kCols, e = q % kCols;
        double sum = s_part[0][q];
#pragma unroll
        for (int w = 1; w < SPLIT; ++w)
            sum += s_part[w][q];
        if (bg && e < E)
            sum += (double)bg[e];
        const float z = (float)sum;
        s_z[tok][e] = z;
        if (t0 + tok < T && e < E)
            logits[(size_t)(t0 + tok) * E + e] = z;
    }
    __syncthreads();
    const int tok = threadIdx.x / G, li = threadIdx.x % G;
    const int t = t0 + tok;
    if (t >= T)
        return;  // whole groups leave together
    float z[VPL];
    uint64_t key[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v)
        z[v] = s_z[tok][min(li + G * v, kCols - 1)];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
        const int e = li + G * v;
        z[v] = e < E ? z[v] : 0.0f;
        key[v] = e < E ? select_key(z[v], e) : 0;
    }
    double ex[VPL], denom, m, mu, sigma;
    token_probs<VPL, G, true>(z, li, E, normalize, lambda, ex, denom, m, mu, sigma);
    select_topk<VPL, G>(key, normalize, lambda, mu, sigma, m, denom, li, t, k, topk_idx, topk_w);
}

// ---------------------------------------------------------------- router backward
// Logit gradient of one token from the gate-weight gradients d_w[t,j] (the
// combine's <dy, y_perm row>): dp[e] = d_w of the kept choice on e (0 for
// other experts and dropped choices; top-k passes no gradient),
// ds = p (dp - <p, dp>) through the softmax, and with the normalisation
// s = lambda zh, zh = (z - mu) / sigma:
//   dz = (lambda / sigma) (ds - mean(ds) - zh mean(ds zh)),  0 when sigma == 0.
// Balancing losses (the router statistics' definitions) with coefficients
// aux_coef and z_coef: aux = E sum_e f_e P_e with f_e = counts_e / (T k)
// constant adds aux_coef E f_e / T to dp before the softmax backward; the
// Z-loss (1/T) sum_t lse(z_t)^2 on the raw logits adds
// z_coef (2/T) lse(z_t) softmax(z_t) to dz.
// fp64 throughout (the router's arithmetic), stored fp32.  One wavefront per
// token.
template <int VPL>
__global__ __launch_bounds__(256) void moe_router_bwd_kernel(const float* __restrict__ logits,
                                                             const int32_t* __restrict__ topk_idx,
                                                             const int32_t* __restrict__ slot,
                                                             const float* __restrict__ d_w, int T, int E, int k,
                                                             int normalize, float lambda, float aux_coef,
                                                             float z_coef, const int32_t* __restrict__ counts,
                                                             float* __restrict__ dz)
{
    const int lane = lane_id();
    const int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T)
        return;
    const float* zt = logits + (size_t)t * E;
    float z[VPL];
    // unconditional loads (index clamped, padding zeroed after): all VPL
    // are in flight together
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        z[i] = zt[min(lane + kWave * i, E - 1)];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (lane + kWave * i >= E)
            z[i] = 0.0f;
    double ex[VPL], denom;
    token_probs<VPL>(z, lane, E, normalize, lambda, ex, denom);
    double p[VPL], dp[VPL];
    const double aux_scale = (double)aux_coef * (double)E / ((double)T * (double)k) / (double)T;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        p[i] = ex[i] / denom;
        const int32_t ce = counts[min(e, E - 1)];
        dp[i] = (aux_coef != 0.0f && e < E) ? aux_scale * (double)ce : 0.0;
    }
    for (int j = 0; j < k; ++j) {
        const size_t a = (size_t)t * k + j;
        const int e = topk_idx[a];
        if (slot[a] < 0 || e < 0 || e >= E)
            continue;
        const double g = (double)d_w[a];
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane + kWave * i == e)
                dp[i] += g;
    }
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        part += p[i] * dp[i];
    const double pdp = wave_sum(part);
    double ds[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        ds[i] = (lane + kWave * i < E) ? p[i] * (dp[i] - pdp) : 0.0;
    if (normalize) {
        part = 0.0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            part += (lane + kWave * i < E) ? (double)z[i] : 0.0;
        const double mu = wave_sum(part) / E;
        part = 0.0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            const double c = (double)z[i] - mu;
            part += (lane + kWave * i < E) ? c * c : 0.0;
        }
        const double sigma = sqrt(wave_sum(part) / E);
        if (sigma == 0.0) {
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                ds[i] = 0.0;
        } else {
            double zh[VPL], p1 = 0.0, p2 = 0.0;
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                zh[i] = ((double)z[i] - mu) / sigma;
                p1 += ds[i];
                p2 += (lane + kWave * i < E) ? ds[i] * zh[i] : 0.0;
            }
            const double m1 = wave_sum(p1) / E, m2 = wave_sum(p2) / E;
#pragma unroll
            for (int i = 0; i < VPL; ++i)
                ds[i] = (double)lambda / sigma * (ds[i] - m1 - zh[i] * m2);
        }
    }
    if (z_coef != 0.0f) {  // Z-loss on the raw logits
        double m = -INFINITY;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane + kWave * i < E)
                m = fmax(m, (double)z[i]);
        m = wave_max(m);
        double q[VPL], part = 0.0;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            q[i] = (lane + kWave * i < E) ? exp((double)z[i] - m) : 0.0;
            part += q[i];
        }
        const double sum = wave_sum(part);
        const double c = (double)z_coef * 2.0 / (double)T * (m + log(sum)) / sum;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            ds[i] += c * q[i];
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int e = lane + kWave * i;
        if (e < E)
            dz[(size_t)t * E + e] = (float)ds[i];
    }
}

// ---------------------------------------------------------------- router by-products
// Sums over tokens for the balancing statistics (Megatron-Core page, "MoE负载
// 均衡的挑战与应对" and "关键特性": auxiliary loss, Z-Loss; Skywork news item,
// "技术创新 2", and slides, slide 7: the drop-rate-driven coefficient).
//
// Pass 1: block b takes tokens b*4 + wave, stepping by 4 * gridDim.x; each
// wavefront adds its tokens' gate probabilities (fp64, the same arithmetic as
// the router) per expert and (logsumexp z)^2 of the raw logits; the block's
// 4 wavefronts are added in wave order and stored as partial[b][0..E-1] and
// partial[b][E].  Passes 2 and 3 add the blocks and then the experts in fixed
// orders.  The grid depends only on T, so the sums are the same on every run.
constexpr int kStatsBlocks = 256;

template <int VPL>
__global__ __launch_bounds__(256) void moe_router_stats_kernel(const float* __restrict__ logits, int T, int E,
                                                               int normalize, float lambda,
                                                               double* __restrict__ partial)
{
    __shared__ double s_acc[4][VPL * kWave + 1];
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    double psum[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        psum[i] = 0.0;
    double zsum = 0.0;
    for (int t = blockIdx.x * 4 + wave; t < T; t += 4 * gridDim.x) {
        const float* zt = logits + (size_t)t * E;
        float z[VPL];
        // unconditional loads (index clamped, padding zeroed after)
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            z[i] = zt[min(lane + kWave * i, E - 1)];
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane + kWave * i >= E)
                z[i] = 0.0f;
        double ex[VPL], denom;
        token_probs<VPL>(z, lane, E, normalize, lambda, ex, denom);
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            psum[i] += ex[i] / denom;
        // logsumexp of the raw logits
        double m = -INFINITY;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (lane + kWave * i < E)
                m = fmax(m, (double)z[i]);
        m = wave_max(m);
        double part = 0.0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            part += (lane + kWave * i < E) ? exp((double)z[i] - m) : 0.0;
        const double lse = m + log(wave_sum(part));
        zsum += lse * lse;
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        s_acc[wave][lane + kWave * i] = psum[i];
    if (lane == 0)
        s_acc[wave][VPL * kWave] = zsum;
    __syncthreads();
    double* dst = partial + (size_t)blockIdx.x * (E + 1);
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        dst[e] = ((s_acc[0][e] + s_acc[1][e]) + s_acc[2][e]) + s_acc[3][e];
    if (threadIdx.x == 0)
        dst[E] = ((s_acc[0][VPL * kWave] + s_acc[1][VPL * kWave]) + s_acc[2][VPL * kWave]) + s_acc[3][VPL * kWave];
}

// Pass 2, one wavefront per item e in [0, E] (E is the Z-loss sum): lanes
// add partial[b][e] for b = lane, lane + 64, ... in order, then a fixed
// reduction tree (group_reduce) adds the lanes.  Writes mean_prob[e] =
// sum / T and frac[e] = counts[e] / (T k) and keeps terms[e] = frac[e] *
// mean_prob[e]
// (terms[E] = Z-loss sum) for pass 3.
__global__ __launch_bounds__(256) void moe_router_stats_reduce_kernel(const double* __restrict__ partial,
                                                                       int nblocks, int T, int E, int k,
                                                                       const int32_t* __restrict__ counts,
                                                                       float* __restrict__ frac,
                                                                       float* __restrict__ mean_prob,
                                                                       double* __restrict__ terms)
{
    const int e = blockIdx.x * 4 + threadIdx.x / kWave;
    if (e > E)
        return;
    const int lane = lane_id();
    double s = 0.0;
    for (int b = lane; b < nblocks; b += kWave)
        s += partial[(size_t)b * (E + 1) + e];
    s = wave_sum(s);
    if (lane == 0) {
        if (e < E) {
            const double mp = s / (double)T;
            const double f = (double)counts[e] / ((double)T * (double)k);
            mean_prob[e] = (float)mp;
            frac[e] = (float)f;
            terms[e] = f * mp;
        } else {
            terms[E] = s;
        }
    }
}

// Pass 3, one block of 1024 threads (thread e owns expert e):
//   scalars = {E * sum_e terms[e], terms[E] / T, (T k - offsets[E]) / (T k)}
// with the sum over experts a fixed tree (the wavefront reduction, then the 16
// wavefronts in order).
__global__ __launch_bounds__(1024) void moe_router_stats_final_kernel(const double* __restrict__ terms, int T,
                                                                      int E, int k,
                                                                      const int32_t* __restrict__ offsets,
                                                                      float* __restrict__ scalars)
{
    __shared__ double s_w[1024 / kWave];
    const int e = threadIdx.x;
    double term = e < E ? terms[e] : 0.0;
    term = wave_sum(term);
    if (lane_id() == 0)
        s_w[threadIdx.x / kWave] = term;
    __syncthreads();
    if (threadIdx.x == 0) {
        double aux = 0.0;
        for (int w = 0; w < 1024 / kWave; ++w)
            aux += s_w[w];
        const double n = (double)T * (double)k;
        const int kept = min(max(offsets[E], 0), T * k);
        scalars[0] = (float)((double)E * aux);
        scalars[1] = (float)(terms[E] / (double)T);
        scalars[2] = (float)((n - (double)kept) / n);
    }
}

}  // namespace moe

// ---------------------------------------------------------------- launchers
extern "C" hipError_t moe_launch_gate(int dtype, const void* x, const void* Wg, const float* bg, float* logits,
                                      int T, int d, int E, hipStream_t stream)
{
    using namespace moe;
    const dim3 grid((T + kGateTile - 1) / kGateTile, (E + kGateTile - 1) / kGateTile), block(kGateSplit * kWave);
    if (dtype == 0)
        moe_gate_logits_kernel<f32_t><<<grid, block, 0, stream>>>((const float*)x, (const float*)Wg, bg, logits, T, d, E);
    else
        moe_gate_logits_kernel<bf16_t>
            <<<grid, block, 0, stream>>>((const uint16_t*)x, (const uint16_t*)Wg, bg, logits, T, d, E);
    return hipGetLastError();
}

// Gate and router in one launch; E <= 64 (hipErrorInvalidValue otherwise).
extern "C" hipError_t moe_launch_gate_route(int dtype, const void* x, const void* Wg, const float* bg, float* logits,
                                            int T, int d, int E, int k, int normalize, float lambda,
                                            int32_t* topk_idx, float* topk_w, hipStream_t stream)
{
    using namespace moe;
    const int nt = (E + kGateTile - 1) / kGateTile;
    if (nt < 1 || nt > 4)
        return hipErrorInvalidValue;
    const dim3 grid((T + kGateTile - 1) / kGateTile);
    // up to 32 experts: 8 wavefronts split the model dimension (as in the
    // gate kernel); beyond, 4 wavefronts keep the partial tiles at 32 KB
    auto go = [&](auto et, auto ntc, auto splitc) {
        typedef decltype(et) ET;
        constexpr int NT = decltype(ntc)::value, SPLIT = decltype(splitc)::value;
        moe_gate_route_kernel<ET, NT, SPLIT><<<grid, SPLIT * kWave, 0, stream>>>(
            (const typename ET::storage*)x, (const typename ET::storage*)Wg, bg, logits, T, d, E, k, normalize,
            lambda, topk_idx, topk_w);
    };
    auto by_nt = [&](auto et) {
        if (nt == 1)
            go(et, std::integral_constant<int, 1>{}, std::integral_constant<int, 8>{});
        else if (nt == 2)
            go(et, std::integral_constant<int, 2>{}, std::integral_constant<int, 8>{});
        else if (nt == 3)
            go(et, std::integral_constant<int, 3>{}, std::integral_constant<int, 4>{});
        else
            go(et, std::integral_constant<int, 4>{}, std::integral_constant<int, 4>{});
    };
    if (dtype == 0)
        by_nt(f32_t{});
    else
        by_nt(bf16_t{});
    return hipGetLastError();
}

extern "C" hipError_t moe_launch_router(const float* logits, int T, int E, int k, int normalize, float lambda,
                                        int32_t* topk_idx, float* topk_w, hipStream_t stream)
{
    using namespace moe;
    // groups of 16 lanes up to 256 experts, then 32 and 64 lanes: at most 16
    // experts per lane (32 per lane at 512 experts took 238 registers and
    // ran slower at two wavefronts per SIMD)
    auto go = [&](auto vplc, auto gc) {
        constexpr int VPL = decltype(vplc)::value, G = decltype(gc)::value;
        const dim3 grid((T + 256 / G - 1) / (256 / G)), block(256);
        moe_router_kernel<VPL, G><<<grid, block, 0, stream>>>(logits, T, E, k, normalize, lambda, topk_idx, topk_w);
    };
    if (E <= 16)
        go(std::integral_constant<int, 1>{}, std::integral_constant<int, 16>{});
    else if (E <= 32)
        go(std::integral_constant<int, 2>{}, std::integral_constant<int, 16>{});
    else if (E <= 64)
        go(std::integral_constant<int, 4>{}, std::integral_constant<int, 16>{});
    else if (E <= 128)
        go(std::integral_constant<int, 8>{}, std::integral_constant<int, 16>{});
    else if (E <= 256)
        go(std::integral_constant<int, 16>{}, std::integral_constant<int, 16>{});
    else if (E <= 512)
        go(std::integral_constant<int, 16>{}, std::integral_constant<int, 32>{});
    else
        go(std::integral_constant<int, 16>{}, std::integral_constant<int, 64>{});
    return hipGetLastError();
}

// Workspace of the statistics, in bytes: the first pass's block partials,
// then the E + 1 per-item sums of the second.
extern "C" size_t moe_router_stats_partial_bytes(int T, int E)
{
    const int nb = T < 4 * moe::kStatsBlocks ? (T + 3) / 4 : moe::kStatsBlocks;
    return (size_t)((nb > 0 ? nb : 1) + 1) * (E + 1) * sizeof(double);
}

extern "C" hipError_t moe_launch_router_stats(const float* logits, int T, int E, int k, int normalize, float lambda,
                                              const int32_t* counts, const int32_t* offsets, double* partial,
                                              float* frac, float* mean_prob, float* scalars, hipStream_t stream)
{
    using namespace moe;
    const int nb = T < 4 * kStatsBlocks ? (T + 3) / 4 : kStatsBlocks;
    const int vpl = (E + kWave - 1) / kWave;
    const dim3 grid(nb), block(256);
    if (vpl <= 1)
        moe_router_stats_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, normalize, lambda, partial);
    else if (vpl <= 2)
        moe_router_stats_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, normalize, lambda, partial);
    else if (vpl <= 4)
        moe_router_stats_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, normalize, lambda, partial);
    else if (vpl <= 8)
        moe_router_stats_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, normalize, lambda, partial);
    else
        moe_router_stats_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, normalize, lambda, partial);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    double* terms = partial + (size_t)nb * (E + 1);
    moe_router_stats_reduce_kernel<<<dim3((E + 1 + 3) / 4), dim3(256), 0, stream>>>(partial, nb, T, E, k, counts,
                                                                                   frac, mean_prob, terms);
    err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    moe_router_stats_final_kernel<<<1, 1024, 0, stream>>>(terms, T, E, k, offsets, scalars);
    return hipGetLastError();
}

extern "C" hipError_t moe_launch_router_bwd(const float* logits, const int32_t* topk_idx, const int32_t* slot,
                                            const float* d_w, int T, int E, int k, int normalize, float lambda,
                                            float aux_coef, float z_coef, const int32_t* counts, float* dz,
                                            hipStream_t stream)
{
    using namespace moe;
    const dim3 grid((T + 3) / 4), block(256);
    const int vpl = (E + kWave - 1) / kWave;
    auto go = [&](auto v) {
        moe_router_bwd_kernel<decltype(v)::value><<<grid, block, 0, stream>>>(
            logits, topk_idx, slot, d_w, T, E, k, normalize, lambda, aux_coef, z_coef, counts, dz);
    };
    if (vpl <= 1)
        go(std::integral_constant<int, 1>{});
    else if (vpl <= 2)
        go(std::integral_constant<int, 2>{});
    else if (vpl <= 4)
        go(std::integral_constant<int, 4>{});
    else if (vpl <= 8)
        go(std::integral_constant<int, 8>{});
    else
        go(std::integral_constant<int, 16>{});
    return hipGetLastError();
}
