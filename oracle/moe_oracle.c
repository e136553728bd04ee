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
