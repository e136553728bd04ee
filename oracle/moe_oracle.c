/*
 * moe_oracle.c -- plain CPU oracle of the sparsely-gated MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP implementation.
 *
 * What is computed, and where it is defined:
 *   - gate:       a single fully connected layer gives one logit per expert
 *                 (FastMoE announcement page, "特色二": the gate shipped is a
 *                 one-layer FC network; "§1 MoE 设计", Fig. 1: a gating
 *                 network picks k of n experts for every input).
 *   - normalise:  Skywork-MoE gating-logit normalisation: per token, the
 *                 logits are standardised over the experts, scaled by lambda,
 *                 then passed to the softmax (Skywork-MoE news item,
 *                 "技术创新 1. Gating Logits 归一化操作"; Skywork-MoE slides,
 *                 slide 6 "Gating Logit Normalization", lambda = 1 best).  The
 *                 page lost the formula; the reading used here (population
 *                 standard deviation, no epsilon, sigma == 0 gives all zeros)
 *                 is the plainest one consistent with "sharper" probabilities.
 *   - softmax:    over all E experts, no renormalisation of the k kept weights
 *                 (the gate both selects experts and weights their mix:
 *                 industry-overview page, section "MoE的內涵、優勢").
 *   - top-k:      the k experts with the highest scores ("top-2 gate", FastMoE
 *                 page Fig. 4 caption; Megatron-Core page "关键特性": Top-K
 *                 router).  Compared on the fp32 logit, descending, equal
 *                 keys to the lower expert index; -0 equals +0.
 *   - capacity:   C = ceil(cf * T * k / E); assignments beyond C on an expert
 *                 are dropped and contribute zero (the residual connection
 *                 outside the layer carries the token) -- Megatron-Core page,
 *                 "MoE负载均衡的挑战与应对" and its Q&A on load imbalance.
 *                 cf <= 0 means dropless (same section: variable-length
 *                 inputs with no dropping, as in MegaBlocks / Mixtral).
 *                 Per expert the earliest tokens are kept.
 *   - experts:    a two-layer MLP, ReLU (FastMoE page "特色三": 512->1024->512
 *                 ReLU experts) or SwiGLU with the gate projection rows
 *                 before the up projection rows (Megatron-Core page,
 *                 "从HuggingFace到Megatron的权重转换要点": gate_proj and
 *                 up_proj fused into one weight, order matters).  No biases.
 *   - combine:    y_t = sum over the token's kept choices j, in selection
 *                 order, of w[t,j] * expert_j(x_t).
 *   - FP8 experts: expert weights stored as OCP FP8 E4M3 codes (Skywork-MoE
 *                 model card links an FP8 checkpoint; news item "4090推理":
 *                 FP8-quantised inference on 8 RTX 4090s; Megatron-Core page,
 *                 "关键特性": FP8 training among the coming features).  The
 *                 pages fix no scheme; the plainest one used here: every row
 *                 of a weight matrix, every token row of x and every row of h
 *                 carries a power-of-two scale s, the smallest with
 *                 max|row| <= 448 s, and its codes are the E4M3 values
 *                 nearest to v / s (ties to even, saturating at 448).  The
 *                 products are of the dequantised values code * s.
 *   - backward:   the gradient of the layer (all throughput figures on the
 *                 pages are for training: Skywork news "训练Infra", FastMoE
 *                 page "特色三", Megatron-Core page "训练效果与性能实测").  The
 *                 chain rule through the combine, both expert layers, the
 *                 softmax, the normalisation and the gate; the top-k choice
 *                 and the capacity drops are piecewise constant and pass no
 *                 gradient (a dropped choice does not touch y at all).
 *   - router by-products: the quantities the load-balancing auxiliary loss,
 *                 its adaptive coefficient and the Z-loss are built from
 *                 (Megatron-Core page, "MoE负载均衡的挑战与应对": an auxiliary
 *                 loss pushes experts towards equal token counts, and
 *                 "关键特性": Z-Loss among the balancing methods; Skywork-MoE
 *                 news item, "技术创新 2. 自适应的Aux Loss", and slides, slide 7:
 *                 the coefficient follows the token drop rate).  The pages
 *                 give no formulas; the plainest readings are used: per
 *                 expert the share of the T*k assignments f_e and the mean
 *                 gate probability P_e, the loss E * sum_e f_e P_e (without
 *                 its coefficient), the Z-loss mean_t (log sum_e exp z)^2 on
 *                 the raw logits, and the drop rate = dropped / (T*k).
 *
 * Arithmetic: every floating-point sum and product is done in double; bf16
 * inputs are widened exactly (bf16 is the top half of an IEEE binary32).
 * The only fp32 values are the logits, which are the selection key.
 *
 * Parallelism: OpenMP over tokens (or rows); every output element is written
 * by exactly one thread and computed in a fixed order, so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_RELU 0
#define ORC_SWIGLU 1

/* Element i of an fp32 or bf16 array, widened to double exactly. */
static double elem(int dtype, const void* base, size_t i)
{
    if (dtype == ORC_F32)
        return (double)((const float*)base)[i];
    uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int orc_threads(void) { return omp_get_max_threads(); }

double orc_bf16_to_double(uint16_t bits) { return elem(ORC_BF16, &bits, 0); }

/* Gate: z[t,e] = sum_i x[t,i] * Wg[e,i] + bg[e], x [T,d], Wg [E,d] row-major.
 * z_exact (nullable) receives the double value, z32 (nullable) the value
 * rounded to fp32 (round to nearest even). */
void orc_gate_logits(int T, int d, int E, int dtype, const void* x, const void* Wg,
                     const float* bg, double* z_exact, float* z32)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int i = 0; i < d; ++i)
                s += elem(dtype, x, (size_t)t * d + i) * elem(dtype, Wg, (size_t)e * d + i);
            if (bg)
                s += (double)bg[e];
            if (z_exact)
                z_exact[(size_t)t * E + e] = s;
            if (z32)
                z32[(size_t)t * E + e] = (float)s;
        }
    }
}

/* Skywork gating-logit normalisation for one token:
 * mu = mean_e z, sigma = sqrt(mean_e (z - mu)^2), zt = lambda * (z - mu) / sigma;
 * sigma == 0 gives zt = 0 for every expert. */
void orc_normalize(int E, const float* z, double lambda, double* zt)
{
    double mu = 0.0;
    for (int e = 0; e < E; ++e)
        mu += (double)z[e];
    mu /= E;
    double var = 0.0;
    for (int e = 0; e < E; ++e)
        var += ((double)z[e] - mu) * ((double)z[e] - mu);
    var /= E;
    double sigma = sqrt(var);
    for (int e = 0; e < E; ++e)
        zt[e] = (sigma == 0.0) ? 0.0 : lambda * ((double)z[e] - mu) / sigma;
}

/* Softmax over E scores: p_e = exp(s_e - max s) / sum_e' exp(s_e' - max s). */
void orc_softmax(int E, const double* s, double* p)
{
    double m = s[0];
    for (int e = 1; e < E; ++e)
        if (s[e] > m)
            m = s[e];
    double sum = 0.0;
    for (int e = 0; e < E; ++e) {
        p[e] = exp(s[e] - m);
        sum += p[e];
    }
    for (int e = 0; e < E; ++e)
        p[e] /= sum;
}

/* Gate probabilities of one token: softmax of the (optionally normalised)
 * logits. */
void orc_gate_probs(int E, const float* z, int normalize, double lambda, double* p)
{
    double* s = (double*)malloc(sizeof(double) * (size_t)E);
    if (normalize) {
        orc_normalize(E, z, lambda, s);
    } else {
        for (int e = 0; e < E; ++e)
            s[e] = (double)z[e];
    }
    orc_softmax(E, s, p);
    free(s);
}

/* Top-k of one token: k rounds, each taking the not-yet-taken expert with the
 * largest fp32 logit.  Scanning e upward with a strict '>' leaves equal keys
 * to the lower index; C's '==' treats -0 and +0 as equal. */
void orc_topk(int E, int k, const float* z, int32_t* idx)
{
    char* taken = (char*)calloc((size_t)E, 1);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e])
                continue;
            if (best < 0 || z[e] > z[best])
                best = e;
        }
        idx[j] = best;
        taken[best] = 1;
    }
    free(taken);
}

/* Routing of all T tokens: idx [T,k] (selection order), w [T,k] = p at the
 * selected experts, p_all (nullable) [T,E] = every probability. */
void orc_route(int T, int E, int k, int normalize, double lambda, const float* z,
               int32_t* idx, double* w, double* p_all)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double* p = (double*)malloc(sizeof(double) * (size_t)E);
        const float* zt = z + (size_t)t * E;
        orc_gate_probs(E, zt, normalize, lambda, p);
        orc_topk(E, k, zt, idx + (size_t)t * k);
        for (int j = 0; j < k; ++j)
            w[(size_t)t * k + j] = p[idx[(size_t)t * k + j]];
        if (p_all)
            memcpy(p_all + (size_t)t * E, p, sizeof(double) * (size_t)E);
        free(p);
    }
}

/* Expert capacity C = ceil(cf * T * k / E) (in double), or -1 (no limit) for
 * cf <= 0. */
long long orc_capacity(int T, int E, int k, double cf)
{
    if (!(cf > 0.0))
        return -1;
    return (long long)ceil(cf * T * k / E);
}

/* Counting, capacity clip and permutation of the T*k assignments.
 * The rank of assignment (t,j) on expert e = idx[t,j] is the number of earlier
 * tokens that chose e; it is kept when rank < C.  Kept assignments of expert
 * e occupy rows offsets[e] + rank, offsets = exclusive scan of the kept
 * counts.  slot[t,j] = row, or -1 when dropped; src_token[row] = t.
 * Returns P = offsets[E], the number of kept rows. */
int orc_dispatch(int T, int E, int k, long long C, const int32_t* idx, int32_t* counts,
                 int32_t* offsets, int32_t* slot, int32_t* src_token)
{
    int32_t* rank = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * k);
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = idx[(size_t)t * k + j];
            rank[(size_t)t * k + j] = counts[e];
            counts[e] += 1;
        }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) {
        long long kept = counts[e];
        if (C >= 0 && kept > C)
            kept = C;
        offsets[e + 1] = offsets[e] + (int32_t)kept;
    }
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            size_t a = (size_t)t * k + j;
            int e = idx[a];
            int r = rank[a];
            if (C < 0 || r < C) {
                slot[a] = offsets[e] + r;
                src_token[offsets[e] + r] = t;
            } else {
                slot[a] = -1;
            }
        }
    free(rank);
    return offsets[E];
}

/* One token through expert e.  W1 is [E][n1][d] with n1 = F (ReLU) or 2F
 * (SwiGLU: rows 0..F-1 are the gate projection, rows F..2F-1 the up
 * projection); W2 is [E][d][F].  xin [d], out [d], h (nullable) [F]. */
void orc_expert_ffn(int d, int F, int act, int dtype, const void* W1, const void* W2, int e,
                    const double* xin, double* out, double* h)
{
    const size_t n1 = (act == ORC_SWIGLU) ? 2 * (size_t)F : (size_t)F;
    const size_t w1e = (size_t)e * n1 * d;
    const size_t w2e = (size_t)e * d * F;
    double* hh = h ? h : (double*)malloc(sizeof(double) * (size_t)F);
    for (int f = 0; f < F; ++f) {
        double u = 0.0;
        for (int i = 0; i < d; ++i)
            u += elem(dtype, W1, w1e + (size_t)f * d + i) * xin[i];
        if (act == ORC_RELU) {
            hh[f] = u > 0.0 ? u : 0.0;
        } else {
            double v = 0.0;
            for (int i = 0; i < d; ++i)
                v += elem(dtype, W1, w1e + ((size_t)F + f) * d + i) * xin[i];
            double silu = u / (1.0 + exp(-u));
            hh[f] = silu * v;
        }
    }
    for (int o = 0; o < d; ++o) {
        double s = 0.0;
        for (int f = 0; f < F; ++f)
            s += elem(dtype, W2, w2e + (size_t)o * F + f) * hh[f];
        out[o] = s;
    }
    if (!h)
        free(hh);
}

/* Layer output for ntok tokens (tokens == NULL means tokens 0..ntok-1):
 * y[n] = sum over j with slot[t,j] >= 0 of w[t,j] * expert_{idx[t,j]}(x_t).
 * A token whose every choice was dropped gets y = 0. */
void orc_forward_tokens(int d, int k, int F, int act, int dtype, const void* x, const void* W1,
                        const void* W2, const int32_t* idx, const double* w, const int32_t* slot,
                        int ntok, const int32_t* tokens, double* y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int n = 0; n < ntok; ++n) {
        int t = tokens ? tokens[n] : n;
        double* xt = (double*)malloc(sizeof(double) * (size_t)d);
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
        double* yn = y + (size_t)n * d;
        for (int i = 0; i < d; ++i) {
            xt[i] = elem(dtype, x, (size_t)t * d + i);
            yn[i] = 0.0;
        }
        for (int j = 0; j < k; ++j) {
            size_t a = (size_t)t * k + j;
            if (slot[a] < 0)
                continue;
            orc_expert_ffn(d, F, act, dtype, W1, W2, idx[a], xt, o, NULL);
            for (int i = 0; i < d; ++i)
                yn[i] += w[a] * o[i];
        }
        free(xt);
        free(o);
    }
}

/* Expert FFN of permuted rows: row r belongs to the expert e with
 * offsets[e] <= r < offsets[e+1]; out[n] = expert_e(xp[r]) for r = rows[n]
 * (rows == NULL means rows 0..nrows-1); h (nullable) [nrows, F]. */
void orc_ffn_rows(int E, int d, int F, int act, int dtype, const int32_t* offsets, const void* xp,
                  const void* W1, const void* W2, int nrows, const int32_t* rows, double* out,
                  double* h)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int n = 0; n < nrows; ++n) {
        int r = rows ? rows[n] : n;
        int e = 0;
        while (e < E && !(offsets[e] <= r && r < offsets[e + 1]))
            ++e;
        double* xr = (double*)malloc(sizeof(double) * (size_t)d);
        for (int i = 0; i < d; ++i)
            xr[i] = elem(dtype, xp, (size_t)r * d + i);
        if (e < E) {
            orc_expert_ffn(d, F, act, dtype, W1, W2, e, xr, out + (size_t)n * d,
                           h ? h + (size_t)n * F : NULL);
        } else {
            for (int i = 0; i < d; ++i)
                out[(size_t)n * d + i] = 0.0;
        }
        free(xr);
    }
}

/* Weighted combine of expert outputs in permuted order:
 * y[t] = sum over j with slot[t,j] >= 0 of w[t,j] * yp[slot[t,j]]. */
void orc_combine(int T, int d, int k, int dtype, const void* yp, const int32_t* slot,
                 const double* w, double* y)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double* yt = y + (size_t)t * d;
        for (int i = 0; i < d; ++i)
            yt[i] = 0.0;
        for (int j = 0; j < k; ++j) {
            size_t a = (size_t)t * k + j;
            if (slot[a] < 0)
                continue;
            for (int i = 0; i < d; ++i)
                yt[i] += w[a] * elem(dtype, yp, (size_t)slot[a] * d + i);
        }
    }
}

/* Second expert layer alone on given hidden rows: out[n] = W2[e] h[r] for
 * r = rows[n] (rows == NULL means 0..nrows-1), e the expert whose segment
 * [offsets[e], offsets[e+1]) holds r.  h [*, F] dtype, out [nrows, d]. */
void orc_down_rows(int E, int d, int F, int dtype, const int32_t* offsets, const void* h, const void* W2,
                   int nrows, const int32_t* rows, double* out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int n = 0; n < nrows; ++n) {
        int r = rows ? rows[n] : n;
        int e = 0;
        while (e < E && !(offsets[e] <= r && r < offsets[e + 1]))
            ++e;
        for (int o = 0; o < d; ++o) {
            double s = 0.0;
            if (e < E)
                for (int f = 0; f < F; ++f)
                    s += elem(dtype, W2, (size_t)e * d * F + (size_t)o * F + f) * elem(dtype, h, (size_t)r * F + f);
            out[(size_t)n * d + o] = s;
        }
    }
}

/* Router by-products of a routed batch.  z [T,E] fp32 logits (the ones the
 * routing used), counts [E] assignments per expert before the capacity clip,
 * kept = number of assignments kept after it.  Outputs (double):
 *   frac[e]      = counts[e] / (T k)
 *   mean_prob[e] = (1/T) sum_t p[t,e], p the gate probabilities (after the
 *                  optional normalisation), tokens summed in order
 *   out3[0]      = E * sum_e frac[e] * mean_prob[e]   (auxiliary loss)
 *   out3[1]      = (1/T) sum_t (log sum_e exp z[t,e])^2   (Z-loss)
 *   out3[2]      = (T k - kept) / (T k)   (drop rate) */
void orc_router_stats(int T, int E, int k, int normalize, double lambda, const float* z,
                      const int32_t* counts, long long kept, double* frac, double* mean_prob, double* out3)
{
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    for (int e = 0; e < E; ++e)
        mean_prob[e] = 0.0;
    double zsum = 0.0;
    for (int t = 0; t < T; ++t) {
        const float* zt = z + (size_t)t * E;
        orc_gate_probs(E, zt, normalize, lambda, p);
        for (int e = 0; e < E; ++e)
            mean_prob[e] += p[e];
        double m = (double)zt[0];
        for (int e = 1; e < E; ++e)
            if ((double)zt[e] > m)
                m = (double)zt[e];
        double se = 0.0;
        for (int e = 0; e < E; ++e)
            se += exp((double)zt[e] - m);
        double lse = m + log(se);
        zsum += lse * lse;
    }
    const double n = (double)T * (double)k;
    double aux = 0.0;
    for (int e = 0; e < E; ++e) {
        mean_prob[e] /= (double)T;
        frac[e] = (double)counts[e] / n;
        aux += frac[e] * mean_prob[e];
    }
    out3[0] = (double)E * aux;
    out3[1] = zsum / (double)T;
    out3[2] = (n - (double)kept) / n;
    free(p);
}

/* ---------------------------------------------------------------- FP8 (E4M3) */

/* Value of an OCP FP8 E4M3FN code: sign, 4 exponent bits (bias 7), 3
 * mantissa bits; exponent 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN. */
double orc_e4m3_decode(uint8_t c)
{
    const int sgn = c >> 7, ex = (c >> 3) & 15, m = c & 7;
    if (ex == 15 && m == 7)
        return NAN;
    const double mag = ex == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, ex - 7);
    return sgn ? -mag : mag;
}

/* Nearest E4M3 code to a finite v, ties to the even code; magnitudes at or
 * above 448 (the largest finite value) give +-448. */
uint8_t orc_e4m3_encode(double v)
{
    const uint8_t sgn = signbit(v) ? 0x80 : 0x00;
    const double a = fabs(v);
    if (a >= 448.0)
        return sgn | 0x7E;
    if (a < ldexp(1.0, -6)) {                       /* subnormal range, step 2^-9 */
        const double q = nearbyint(ldexp(a, 9));    /* 0..8; 8 is the smallest normal */
        return sgn | (uint8_t)q;
    }
    int e;
    const double fr = frexp(a, &e);                 /* a = fr * 2^e, fr in [0.5, 1) */
    int ex = e - 1;                                 /* a = (2 fr) * 2^ex, 2 fr in [1, 2) */
    double q = nearbyint(fr * 16.0);                /* 8..16: 1 + mantissa/8 in eighths */
    if (q == 16.0) {
        q = 8.0;
        ex += 1;
    }
    return sgn | (uint8_t)(((ex + 7) << 3) | ((int)q - 8));
}

/* Exponent e of the power-of-two row scale: the smallest integer with
 * amax <= 448 * 2^e (0 for amax == 0).  448 = 0.875 * 2^9, so with
 * amax = m * 2^x, m in [0.5, 1): e = x - 9 if m <= 0.875, else x - 8. */
int orc_fp8_scale_exp(double amax)
{
    if (!(amax > 0.0))
        return 0;
    int x;
    const double m = frexp(amax, &x);
    return m <= 0.875 ? x - 9 : x - 8;
}

/* Quantise R rows of K values (fp32 / bf16, or double when dtype == 2):
 * codes[r][i] = encode(v[r][i] / s_r), scales[r] = s_r = 2^e. */
void orc_quant_rows_fp8(long long R, int K, int dtype, const void* src, uint8_t* codes, float* scales)
{
#pragma omp parallel for schedule(static)
    for (long long r = 0; r < R; ++r) {
        double amax = 0.0;
        for (int i = 0; i < K; ++i) {
            const size_t at = (size_t)r * K + i;
            const double v = dtype == 2 ? ((const double*)src)[at] : elem(dtype, src, at);
            if (fabs(v) > amax)
                amax = fabs(v);
        }
        const int e = orc_fp8_scale_exp(amax);
        for (int i = 0; i < K; ++i) {
            const size_t at = (size_t)r * K + i;
            const double v = dtype == 2 ? ((const double*)src)[at] : elem(dtype, src, at);
            codes[at] = orc_e4m3_encode(ldexp(v, -e));
        }
        scales[r] = (float)ldexp(1.0, e);
    }
}

/* One quantised input row (codes xq [d], scale xs) through FP8 expert e.
 * W1q [E][n1][d] codes with w1s [E][n1] row scales, W2q [E][d][F] with
 * w2s [E][d].  h (nullable, [F]) receives the activation output before it is
 * quantised; out [d] = W2^ * quant(h), ^ meaning dequantised. */
void orc_expert_ffn_fp8(int d, int F, int act, const uint8_t* W1q, const float* w1s, const uint8_t* W2q,
                        const float* w2s, int e, const uint8_t* xq, double xs, double* out, double* h)
{
    const size_t n1 = (act == ORC_SWIGLU) ? 2 * (size_t)F : (size_t)F;
    double* hh = h ? h : (double*)malloc(sizeof(double) * (size_t)F);
    double* xin = (double*)malloc(sizeof(double) * (size_t)d);
    uint8_t* hq = (uint8_t*)malloc((size_t)F);
    for (int i = 0; i < d; ++i)
        xin[i] = orc_e4m3_decode(xq[i]) * xs;
    for (int f = 0; f < F; ++f) {
        const size_t row_g = (size_t)e * n1 + f;
        double u = 0.0;
        for (int i = 0; i < d; ++i)
            u += orc_e4m3_decode(W1q[row_g * d + i]) * (double)w1s[row_g] * xin[i];
        if (act == ORC_RELU) {
            hh[f] = u > 0.0 ? u : 0.0;
        } else {
            const size_t row_u = (size_t)e * n1 + F + f;
            double v = 0.0;
            for (int i = 0; i < d; ++i)
                v += orc_e4m3_decode(W1q[row_u * d + i]) * (double)w1s[row_u] * xin[i];
            hh[f] = u / (1.0 + exp(-u)) * v;
        }
    }
    float hs;
    orc_quant_rows_fp8(1, F, 2, hh, hq, &hs);
    for (int o = 0; o < d; ++o) {
        const size_t row = (size_t)e * d + o;
        double s = 0.0;
        for (int f = 0; f < F; ++f)
            s += orc_e4m3_decode(W2q[row * F + f]) * (double)w2s[row] * orc_e4m3_decode(hq[f]) * (double)hs;
        out[o] = s;
    }
    free(hq);
    free(xin);
    if (!h)
        free(hh);
}

/* FP8 expert FFN of permuted rows (codes xq [*][d], row scales xs): as
 * orc_ffn_rows.  h (nullable) [nrows][F] gets the activation before it is
 * quantised. */
void orc_ffn_rows_fp8(int E, int d, int F, int act, const int32_t* offsets, const uint8_t* xq, const float* xs,
                      const uint8_t* W1q, const float* w1s, const uint8_t* W2q, const float* w2s, int nrows,
                      const int32_t* rows, double* out, double* h)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int n = 0; n < nrows; ++n) {
        int r = rows ? rows[n] : n;
        int e = 0;
        while (e < E && !(offsets[e] <= r && r < offsets[e + 1]))
            ++e;
        if (e < E) {
            orc_expert_ffn_fp8(d, F, act, W1q, w1s, W2q, w2s, e, xq + (size_t)r * d, (double)xs[r],
                               out + (size_t)n * d, h ? h + (size_t)n * F : NULL);
        } else {
            for (int o = 0; o < d; ++o)
                out[(size_t)n * d + o] = 0.0;
            if (h)
                for (int f = 0; f < F; ++f)
                    h[(size_t)n * F + f] = 0.0;
        }
    }
}

/* Second FP8 layer alone on given quantised hidden rows (codes hq [*][F],
 * row scales hs): out[n] = W2^[e] * hq^[r] for r = rows[n]. */
void orc_down_rows_fp8(int E, int d, int F, const int32_t* offsets, const uint8_t* hq, const float* hs,
                       const uint8_t* W2q, const float* w2s, int nrows, const int32_t* rows, double* out)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int n = 0; n < nrows; ++n) {
        int r = rows ? rows[n] : n;
        int e = 0;
        while (e < E && !(offsets[e] <= r && r < offsets[e + 1]))
            ++e;
        for (int o = 0; o < d; ++o) {
            double s = 0.0;
            if (e < E) {
                const size_t row = (size_t)e * d + o;
                for (int f = 0; f < F; ++f)
                    s += orc_e4m3_decode(W2q[row * F + f]) * (double)w2s[row] *
                         orc_e4m3_decode(hq[(size_t)r * F + f]) * (double)hs[r];
            }
            out[(size_t)n * d + o] = s;
        }
    }
}

/* FP8 layer output for ntok tokens: x_t (fp32 / bf16) is quantised per
 * token, each kept choice runs orc_expert_ffn_fp8, and the outputs are mixed
 * with the gate weights as in orc_forward_tokens. */
void orc_forward_tokens_fp8(int d, int k, int F, int act, int dtype, const void* x, const uint8_t* W1q,
                            const float* w1s, const uint8_t* W2q, const float* w2s, const int32_t* idx,
                            const double* w, const int32_t* slot, int ntok, const int32_t* tokens, double* y)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int n = 0; n < ntok; ++n) {
        int t = tokens ? tokens[n] : n;
        uint8_t* xq = (uint8_t*)malloc((size_t)d);
        float xs;
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
        double* yn = y + (size_t)n * d;
        if (dtype == ORC_F32)
            orc_quant_rows_fp8(1, d, dtype, (const float*)x + (size_t)t * d, xq, &xs);
        else
            orc_quant_rows_fp8(1, d, dtype, (const uint16_t*)x + (size_t)t * d, xq, &xs);
        for (int i = 0; i < d; ++i)
            yn[i] = 0.0;
        for (int j = 0; j < k; ++j) {
            size_t a = (size_t)t * k + j;
            if (slot[a] < 0)
                continue;
            orc_expert_ffn_fp8(d, F, act, W1q, w1s, W2q, w2s, idx[a], xq, (double)xs, o, NULL);
            for (int i = 0; i < d; ++i)
                yn[i] += w[a] * o[i];
        }
        free(o);
        free(xq);
    }
}

/* ---------------------------------------------------------------- backward */

/* Gradient of the layer output y with respect to its inputs and weights,
 * given dy = dL/dy [T][d] (dtype) and the forward's routing: z32 [T][E] the
 * fp32 logits the routing used, idx [T][k], slot [T][k] (-1 = dropped).
 * Per token t and kept choice j (expert e, weight w = p[t,e]):
 *   u = W1[e] x_t, h = act(u), o = W2[e] h, y_t += w o
 *   dw_j = <dy_t, o>;  do = w dy_t
 *   dW2[e] += do h^T;  dh = W2[e]^T do
 *   ReLU: du = dh [u > 0];  SwiGLU (g = u[:F], v = u[F:], h = silu(g) v):
 *     dg = dh v silu'(g), dv = dh silu(g), silu'(g) = s (1 + g (1 - s)), s = 1/(1+e^-g)
 *   dW1[e] += du x_t^T;  dx_t += W1[e]^T du
 * Router: dp[e] = dw_j for the kept choice j on expert e (0 otherwise);
 *   ds = p (dp - <p, dp>)   (softmax);
 *   dz = ds, or with the normalisation s = lambda zh, zh = (z - mu)/sigma:
 *   dz = (lambda/sigma) (ds - mean(ds) - zh mean(ds zh)); sigma == 0 gives 0.
 * Gate: dWg[e] += dz[e] x_t, dbg[e] += dz[e], dx_t += sum_e dz[e] Wg[e].
 * Balancing losses (orc_router_stats' definitions), added to the loss with
 * coefficients aux_coef and z_coef:
 *   aux = E sum_e f_e P_e, f_e = counts_e / (T k) over all choices (constant),
 *     P_e = (1/T) sum_t p[t,e]  =>  dp[t,e] += aux_coef E f_e / T, before
 *     the softmax and normalisation backward;
 *   Z-loss = (1/T) sum_t lse(z_t)^2 on the raw logits  =>
 *     dz[t,e] += z_coef (2/T) lse(z_t) softmax(z_t)[e].
 * Outputs (double): dx [T][d], dWg [E][d], dbg [E], dW1 [E][n1][d], dW2 [E][d][F];
 * Wg == NULL means the logits were given (no gate): dWg, dbg and the gate term
 * of dx are skipped.  dz (nullable) [T][E] receives the logit gradient. */
void orc_backward(int T, int d, int E, int k, int F, int act, int dtype, int normalize, double lambda,
                  double aux_coef, double z_coef, const void* x, const void* Wg, const void* W1, const void* W2, const float* z32,
                  const int32_t* idx, const int32_t* slot, const void* dy, double* dx, double* dWg, double* dbg,
                  double* dW1, double* dW2, double* dz_out)
{
    const size_t n1 = (act == ORC_SWIGLU) ? 2 * (size_t)F : (size_t)F;
    memset(dWg, 0, sizeof(double) * (size_t)E * d);
    memset(dbg, 0, sizeof(double) * (size_t)E);
    memset(dW1, 0, sizeof(double) * (size_t)E * n1 * d);
    memset(dW2, 0, sizeof(double) * (size_t)E * d * F);
    double* xt = (double*)malloc(sizeof(double) * (size_t)d);
    double* dyt = (double*)malloc(sizeof(double) * (size_t)d);
    double* u = (double*)malloc(sizeof(double) * n1);
    double* h = (double*)malloc(sizeof(double) * (size_t)F);
    double* o = (double*)malloc(sizeof(double) * (size_t)d);
    double* dh = (double*)malloc(sizeof(double) * (size_t)F);
    double* du = (double*)malloc(sizeof(double) * n1);
    double* p = (double*)malloc(sizeof(double) * (size_t)E);
    double* dp = (double*)malloc(sizeof(double) * (size_t)E);
    double* dzt = (double*)malloc(sizeof(double) * (size_t)E);
    double* aux_dp = (double*)malloc(sizeof(double) * (size_t)E);  /* aux_coef E f_e / T */
    for (int e = 0; e < E; ++e)
        aux_dp[e] = 0.0;
    for (size_t a = 0; a < (size_t)T * k; ++a)
        if (idx[a] >= 0 && idx[a] < E)
            aux_dp[idx[a]] += 1.0;
    for (int e = 0; e < E; ++e)
        aux_dp[e] = aux_coef * (double)E * (aux_dp[e] / ((double)T * k)) / (double)T;
    for (int t = 0; t < T; ++t) {
        double* dxt = dx + (size_t)t * d;
        for (int i = 0; i < d; ++i) {
            xt[i] = elem(dtype, x, (size_t)t * d + i);
            dyt[i] = elem(dtype, dy, (size_t)t * d + i);
            dxt[i] = 0.0;
        }
        orc_gate_probs(E, z32 + (size_t)t * E, normalize, lambda, p);
        for (int e = 0; e < E; ++e)
            dp[e] = aux_dp[e];
        for (int j = 0; j < k; ++j) {
            const size_t a = (size_t)t * k + j;
            if (slot[a] < 0)
                continue;
            const int e = idx[a];
            const double w = p[e];
            const size_t w1e = (size_t)e * n1 * d, w2e = (size_t)e * d * F;
            for (size_t n = 0; n < n1; ++n) {
                double s = 0.0;
                for (int i = 0; i < d; ++i)
                    s += elem(dtype, W1, w1e + n * d + i) * xt[i];
                u[n] = s;
            }
            for (int f = 0; f < F; ++f) {
                if (act == ORC_RELU) {
                    h[f] = u[f] > 0.0 ? u[f] : 0.0;
                } else {
                    const double g = u[f], v = u[F + f];
                    h[f] = g / (1.0 + exp(-g)) * v;
                }
            }
            double dw = 0.0;
            for (int i = 0; i < d; ++i) {
                double s = 0.0;
                for (int f = 0; f < F; ++f)
                    s += elem(dtype, W2, w2e + (size_t)i * F + f) * h[f];
                o[i] = s;
                dw += dyt[i] * s;
            }
            dp[e] += dw;
            /* do = w dy: dW2 and dh */
            for (int f = 0; f < F; ++f)
                dh[f] = 0.0;
            for (int i = 0; i < d; ++i) {
                const double doi = w * dyt[i];
                for (int f = 0; f < F; ++f) {
                    dW2[w2e + (size_t)i * F + f] += doi * h[f];
                    dh[f] += elem(dtype, W2, w2e + (size_t)i * F + f) * doi;
                }
            }
            for (int f = 0; f < F; ++f) {
                if (act == ORC_RELU) {
                    du[f] = u[f] > 0.0 ? dh[f] : 0.0;
                } else {
                    const double g = u[f], v = u[F + f];
                    const double sg = 1.0 / (1.0 + exp(-g));
                    const double silu = g * sg;
                    du[f] = dh[f] * v * sg * (1.0 + g * (1.0 - sg));
                    du[F + f] = dh[f] * silu;
                }
            }
            for (size_t n = 0; n < n1; ++n)
                for (int i = 0; i < d; ++i) {
                    dW1[w1e + n * d + i] += du[n] * xt[i];
                    dxt[i] += elem(dtype, W1, w1e + n * d + i) * du[n];
                }
        }
        /* softmax, then the normalisation */
        double pdp = 0.0;
        for (int e = 0; e < E; ++e)
            pdp += p[e] * dp[e];
        for (int e = 0; e < E; ++e)
            dzt[e] = p[e] * (dp[e] - pdp);
        if (normalize) {
            const float* zt = z32 + (size_t)t * E;
            double mu = 0.0;
            for (int e = 0; e < E; ++e)
                mu += (double)zt[e];
            mu /= E;
            double var = 0.0;
            for (int e = 0; e < E; ++e)
                var += ((double)zt[e] - mu) * ((double)zt[e] - mu);
            const double sigma = sqrt(var / E);
            if (sigma == 0.0) {
                for (int e = 0; e < E; ++e)
                    dzt[e] = 0.0;
            } else {
                double m1 = 0.0, m2 = 0.0;
                for (int e = 0; e < E; ++e) {
                    const double zh = ((double)zt[e] - mu) / sigma;
                    m1 += dzt[e];
                    m2 += dzt[e] * zh;
                }
                m1 /= E;
                m2 /= E;
                for (int e = 0; e < E; ++e) {
                    const double zh = ((double)zt[e] - mu) / sigma;
                    dzt[e] = lambda / sigma * (dzt[e] - m1 - zh * m2);
                }
            }
        }
        if (z_coef != 0.0) {  /* Z-loss on the raw logits */
            const float* zt = z32 + (size_t)t * E;
            double m = -INFINITY;
            for (int e = 0; e < E; ++e)
                m = fmax(m, (double)zt[e]);
            double sum = 0.0;
            for (int e = 0; e < E; ++e)
                sum += exp((double)zt[e] - m);
            const double lse = m + log(sum);
            for (int e = 0; e < E; ++e)
                dzt[e] += z_coef * 2.0 / (double)T * lse * exp((double)zt[e] - m) / sum;
        }
        if (dz_out)
            for (int e = 0; e < E; ++e)
                dz_out[(size_t)t * E + e] = dzt[e];
        if (Wg) {
            for (int e = 0; e < E; ++e) {
                dbg[e] += dzt[e];
                for (int i = 0; i < d; ++i) {
                    dWg[(size_t)e * d + i] += dzt[e] * xt[i];
                    dxt[i] += dzt[e] * elem(dtype, Wg, (size_t)e * d + i);
                }
            }
        }
    }
    free(xt); free(dyt); free(u); free(h); free(o); free(dh); free(du); free(p); free(dp); free(dzt); free(aux_dp);
}
